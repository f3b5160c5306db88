"""Attention over the paged FP8 / BF16 cache: decode and prefill references.

TEST INFRASTRUCTURE ONLY (see the package docstring).

All arithmetic is float64 on dequantised values (scale * decode(code)).

Decode ([BLOG] "Performance benchmarks / Single-request benchmark": the
attention kernel reads the FP8 cache natively and rescales the online softmax
as it goes).  Split-KV with an online softmax and a log-sum-exp merge is an
exact rearrangement of softmax attention, so the decode oracle is the plain
definition:  o = sum_j softmax(s)_j * V_j  with  s_j = sm_scale * q . K_j.

Prefill ([BLOG] "Introduction": both matmuls, QK and Score*V, run in e4m3;
"Kernel and vLLM improvements / Two-level accumulation": partial P*V sums are
flushed into true FP32 registers).  Two references:

* ``prefill_exact``: softmax attention on the dequantised Q, K, V with an
  unquantised P.  This is what the method approximates; reported, not gated.
* ``prefill_mirror``: the same, except that the probabilities that enter the
  P*V product are quantised to e4m3 exactly where the method quantises them:
  per KV tile of ``kv_tile`` keys at absolute, tile-aligned positions, visited
  in ascending order, with p = exp(s - m_t) against the running maximum m_t
  reached after that tile.  The softmax denominator uses the unquantised p.

Masking: a query at absolute position ``pos`` sees key ``j`` iff j <= pos and,
when window > 0, pos - j < window (the window counts the query's own token).
Chunked prefill: a sequence of length L whose last T tokens are the queries
has its queries at positions L - T .. L - 1.
"""

import numpy as np

from .e4m3 import encode, decode
from .quant import BLOCK_SIZE, dequantize, quantize_rows


# ----------------------------------------------------------------------------
# paged cache access
# ----------------------------------------------------------------------------

def gather_kv(cache, block_table_row, lo, hi, head, cache_dtype, k_scale, v_scale):
    """Dequantised K and V (float64 [hi-lo][D]) of tokens lo..hi-1 of one
    sequence and one KV head, read through the block table."""
    t = np.arange(lo, hi, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[t // BLOCK_SIZE]
    rows = t % BLOCK_SIZE
    kc = cache[blocks, head, 0, rows, :]
    vc = cache[blocks, head, 1, rows, :]
    fp8 = cache_dtype in ("e4m3", "e5m2")
    ks = k_scale[head] if fp8 else None
    vs = v_scale[head] if fp8 else None
    return dequantize(kc, ks, cache_dtype), dequantize(vc, vs, cache_dtype)


def visible_range(pos, window):
    """[lo, hi) of keys visible from a query at absolute position ``pos``."""
    lo = max(0, pos - window + 1) if window > 0 else 0
    return lo, pos + 1


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def decode_attention(q, cache, block_table, seq_lens, k_scale, v_scale,
                     sm_scale, window, cache_dtype, num_kv_heads):
    """One decode step: out[b, h_q, :] for queries q[B][H_q][D] (bf16 values).

    Query head h_q reads KV head h_q // G with G = H_q / H_kv.  The query is
    the last token of the sequence (position L - 1), whose K/V is already in
    the cache.  L = 0 gives a zero row.

    Parity: pinned by the uniform-score closed form (mean of V), L = 1, a
    literal triple loop on tiny inputs, and a split + log-sum-exp
    reformulation (tests/test_oracle_attention.py).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    sm = np.float64(np.float32(sm_scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        lo, hi = visible_range(L - 1, window)
        for h in range(num_kv_heads):
            K, V = gather_kv(cache, block_table[b], lo, hi, h, cache_dtype,
                             k_scale, v_scale)
            qh = q[b, h * G:(h + 1) * G, :]          # [G][D]
            s = sm * (qh @ K.T)                      # [G][n]
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[b, h * G:(h + 1) * G, :] = (p @ V) / p.sum(axis=1, keepdims=True)
    return out


def lse_combine(o_parts, m_parts, l_parts):
    """Merge split partials: o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s.

    o_parts [S][D] are unnormalised partial outputs, m_parts [S] the split
    maxima (natural-log domain) and l_parts [S] the partial denominators.
    An empty split carries m = -inf and weight 0; all splits empty -> zeros.
    """
    m = np.asarray(m_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(l_parts, dtype=np.float64)
    if not np.any(np.isfinite(m)):
        return np.zeros(o.shape[1:], dtype=np.float64)
    M = m[np.isfinite(m)].max()
    w = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, M) - M), 0.0)
    return (w[:, None] * o).sum(axis=0) / (w * l).sum()


def decode_attention_split(q, cache, block_table, seq_lens, k_scale, v_scale,
                           sm_scale, window, cache_dtype, num_kv_heads, rng,
                           max_splits=8):
    """Second formulation of decode: cut each context at random points, form
    (unnormalised o_s, m_s, l_s) per piece and merge with ``lse_combine``.
    Used only to pin ``decode_attention`` and the merge formula."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // num_kv_heads
    sm = np.float64(np.float32(sm_scale))
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        lo, hi = visible_range(L - 1, window)
        n_cut = int(rng.integers(0, max_splits))
        cuts = np.sort(rng.integers(lo, hi + 1, size=n_cut))
        bounds = np.concatenate([[lo], cuts, [hi]])
        for h in range(num_kv_heads):
            K, V = gather_kv(cache, block_table[b], lo, hi, h, cache_dtype,
                             k_scale, v_scale)
            for g in range(G):
                qv = q[b, h * G + g]
                parts_o, parts_m, parts_l = [], [], []
                for a, e in zip(bounds[:-1], bounds[1:]):
                    if e <= a:     # empty split
                        parts_o.append(np.zeros(D))
                        parts_m.append(-np.inf)
                        parts_l.append(0.0)
                        continue
                    s = sm * (K[a - lo:e - lo] @ qv)
                    m = s.max()
                    p = np.exp(s - m)
                    parts_o.append(p @ V[a - lo:e - lo])
                    parts_m.append(m)
                    parts_l.append(p.sum())
                out[b, h * G + g] = lse_combine(parts_o, parts_m, parts_l)
    return out


# ----------------------------------------------------------------------------
# prefill
# ----------------------------------------------------------------------------

def quantize_query(q, q_scale):
    """Dequantised FP8 query: q_scale * decode(e4m3(fl32(q / q_scale))).
    One per-tensor query scale ([EXPLAINER] "FP8 combines value and scale":
    per-tensor scaling keeps one scale each for Q, K and V)."""
    codes = quantize_rows(q, np.float32(q_scale))
    return np.float64(np.float32(q_scale)) * decode(codes)


def _prefill_rows_pair(q, cu_q_lens, cache, block_table, seq_lens, q_scale, k_scale,
                       v_scale, sm_scale, window, rows, row_fn, cache_dtype="e4m3"):
    """Like _prefill_rows for a row function returning a [2][D] array."""
    out = _prefill_rows(q, cu_q_lens, cache, block_table, seq_lens, q_scale, k_scale,
                        v_scale, sm_scale, window, rows, row_fn, width=2,
                        cache_dtype=cache_dtype)
    return out[:, :, 0, :].copy(), out[:, :, 1, :].copy()


def _prefill_rows(q, cu_q_lens, cache, block_table, seq_lens, q_scale, k_scale,
                  v_scale, sm_scale, window, rows, row_fn, width=None, cache_dtype="e4m3"):
    q = np.asarray(q, dtype=np.float64)
    Ttot, Hq, D = q.shape
    Hkv = cache.shape[1]
    G = Hq // Hkv
    sm = np.float64(np.float32(sm_scale))
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    if rows is None:
        rows = np.arange(Ttot)
    rows = np.asarray(rows, dtype=np.int64)
    qhat = quantize_query(q[rows], q_scale)            # [R][Hq][D]
    shape = (len(rows), Hq, D) if width is None else (len(rows), Hq, width, D)
    out = np.zeros(shape, dtype=np.float64)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    for b in np.unique(seq_of):
        sel = np.nonzero(seq_of == b)[0]
        L = int(seq_lens[b])
        T = int(cu[b + 1] - cu[b])
        P = L - T
        pos = P + (rows[sel] - cu[b])                  # absolute positions
        lo_all = min(visible_range(int(p), window)[0] for p in pos)
        hi_all = int(pos.max()) + 1
        for h in range(Hkv):
            K, V = gather_kv(cache, block_table[b], lo_all, hi_all, h, cache_dtype,
                             k_scale, v_scale)
            keys = np.arange(lo_all, hi_all)
            for g in range(G):
                hq = h * G + g
                S = sm * (qhat[sel, hq, :] @ K.T)      # [R][n]
                for r, p in enumerate(pos):
                    lo, hi = visible_range(int(p), window)
                    vis = (keys >= lo) & (keys < hi)
                    out[sel[r], hq] = row_fn(S[r, vis], keys[vis], V[vis])
    return out


def _exact_row(s, keys, V):
    p = np.exp(s - s.max())
    return (p @ V) / p.sum()


def prefill_exact(q, cu_q_lens, cache, block_table, seq_lens, q_scale, k_scale,
                  v_scale, sm_scale, window, rows=None, cache_dtype="e4m3"):
    """Softmax attention with FP8-quantised Q, K, V and an unquantised P.

    ``rows`` selects packed query rows (default: all); returns [R][H_q][D].
    ``cache_dtype`` is the FP8 format of the cache ('e4m3' or 'e5m2'); the
    query is always e4m3.  Not the parity target of the GPU kernel (FP8 P is
    part of the method)."""
    return _prefill_rows(q, cu_q_lens, cache, block_table, seq_lens, q_scale,
                         k_scale, v_scale, sm_scale, window, rows, _exact_row,
                         cache_dtype=cache_dtype)


def mirror_row(s, keys, V, kv_tile, quantize_p=True, flip_tol=0.0, return_slack=False):
    """One query row of the tile-mirrored reference, closed form.

    s     scores (float64) of the visible keys, in ascending key order
    keys  absolute key positions;  V  dequantised values [n][D]
    Tiles are [t*kv_tile, (t+1)*kv_tile).  With tmax_t the maximum of the
    scores in tile t and m_t = max(tmax_0..tmax_t) (running maximum):
        p_j  = exp(s_j - m_t)            j in tile t
        pq_j = decode(e4m3(p_j))         (unit scale; p_j in [0, 1])
        O    = sum_t e^{m_t - m_last} sum_{j in t} pq_j V_j
        l    = sum_t e^{m_t - m_last} sum_{j in t} p_j
        o    = O / l
    """
    tile = keys // kv_tile
    tiles, first = np.unique(tile, return_index=True)
    tmax = np.maximum.reduceat(s, first)
    m_run = np.maximum.accumulate(tmax)
    idx = np.searchsorted(tiles, tile)
    m_j = m_run[idx]
    p = np.exp(s - m_j)
    pq = decode(encode(p)) if quantize_p else p
    w_tile = np.exp(m_j - m_run[-1])
    l = (p * w_tile).sum()
    o = ((pq * w_tile) @ V) / l
    if not return_slack:
        return o
    # Flip allowance: a kernel computes p in float32, so a p that lies within
    # a relative flip_tol of an e4m3 rounding midpoint may legitimately round
    # to the neighbouring code.  slack bounds, per output element, how far
    # such alternative roundings can move o.
    slack = np.zeros(V.shape[1])
    if quantize_p and flip_tol > 0:
        alt_lo = decode(encode(p * (1.0 - flip_tol)))
        alt_hi = decode(encode(p * (1.0 + flip_tol)))
        dq = np.maximum(np.abs(alt_lo - pq), np.abs(alt_hi - pq))
        if np.any(dq > 0):
            slack = ((dq * w_tile) @ np.abs(V)) / l
    return o, slack


def prefill_mirror(q, cu_q_lens, cache, block_table, seq_lens, q_scale, k_scale,
                   v_scale, sm_scale, window, kv_tile, rows=None, quantize_p=True,
                   flip_tol=None, cache_dtype="e4m3"):
    """Tile-mirrored FP8-P reference (the parity target of the prefill kernel).

    ``kv_tile`` is the key-tile width the kernel visits (its value is part of
    the numeric contract because the running maximum at which each p is
    quantised depends on it).  ``quantize_p=False`` turns this into the exact
    reference (online-softmax identity), which the tests check.

    Parity: pinned by the literal tile recurrence below, by the uniform-score
    closed form (p = 1 quantises exactly, o = mean V), by kv_tile >= n reducing
    to quantising exp(s - max s), and by a hand-written tiny example.
    """
    if flip_tol is None:
        fn = lambda s, keys, V: mirror_row(s, keys, V, kv_tile, quantize_p)  # noqa: E731
        return _prefill_rows(q, cu_q_lens, cache, block_table, seq_lens, q_scale,
                             k_scale, v_scale, sm_scale, window, rows, fn,
                             cache_dtype=cache_dtype)
    # With flip_tol: returns (out, slack), slack stacked after out along a
    # new leading axis of length 2 in the per-row function, split here.
    fn = lambda s, keys, V: np.stack(mirror_row(s, keys, V, kv_tile, quantize_p,  # noqa: E731
                                                flip_tol, True))
    both = _prefill_rows_pair(q, cu_q_lens, cache, block_table, seq_lens, q_scale,
                              k_scale, v_scale, sm_scale, window, rows, fn,
                              cache_dtype=cache_dtype)
    return both[0], both[1]


def recurrence_row(s, keys, V, kv_tile, quantize_p=True):
    """The same row computed tile by tile, as a flash-attention loop with the
    two-level structure: a zeroed per-tile accumulator acc = sum pq_j V_j,
    then O = alpha * O + acc with alpha = exp(m_old - m_new).  Slow; used to
    pin ``mirror_row`` on small inputs."""
    D = V.shape[1]
    m = -np.inf
    l = 0.0
    O = np.zeros(D)
    t_first = keys[0] // kv_tile
    t_last = keys[-1] // kv_tile
    for t in range(t_first, t_last + 1):
        in_t = [i for i in range(len(keys)) if keys[i] // kv_tile == t]
        if not in_t:
            continue
        m_new = max(m, max(s[i] for i in in_t))
        alpha = 0.0 if m == -np.inf else np.exp(m - m_new)
        acc = np.zeros(D)
        lsum = 0.0
        for i in in_t:
            p = np.exp(s[i] - m_new)
            pq = float(decode(encode(np.array([p])))[0]) if quantize_p else p
            acc += pq * V[i]
            lsum += p
        O = alpha * O + acc
        l = alpha * l + lsum
        m = m_new
    return O / l
