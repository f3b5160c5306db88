"""Host model of the prefill kernel's tile and page arithmetic (CPU only).

The prefill kernel stages 128-key tiles of K and V through LDS and fetches
block-table entries two tiles ahead.  This module restates that index
arithmetic in Python for every workgroup of a launch and checks, for the
shapes the GPU tests use, that

* every block-table entry the kernel reads belongs to a page holding a key
  that some query of the chunk can see (pages lo/16 .. (L-1)/16, lo the
  first query's window start), so entries outside the window are never
  dereferenced, and
* every staged key row that no row of the workgroup can see (before the
  window start or past the sequence end) has its V row zeroed, and its
  score masked, before it meets the P.V product.

The model follows the kernel source (csrc/prefill.hip): grid
(ceil(max_q_len/BM), H_q, B) with BM = 64 or 128 query rows per workgroup,
blocks dispatched longest-first, key range [lo_key, hi_key] per workgroup,
tiles t_lo .. t_hi, block ids of tiles t_lo and t_lo+1 before the loop
(clamped below to the window's first page) and of tile t+2 inside step t
(clamped at the end only), staged copies of tile t+1 inside step t (at its
start with two tile buffers, at its end with one; either way one tile past
t_hi is staged and never read), V rows zeroed before the window start in the
prologue and past the end in the tail tile.  It also checks that the block
id a lane holds is the one its wave's copy of the same index needs, for the
workgroup shapes the launcher picks.
"""

import pytest

KV_TILE = 128
BLOCK = 16
BLOCK_MS = (64, 128)   # query rows per workgroup (head_dim 256 and 64: 64)


def workgroups(q_len, seq_len, window, max_q_len, block_m=128):
    """(q0, lo_key, hi_key, t_lo, t_hi) of every workgroup that does work."""
    out = []
    nx = (max_q_len + block_m - 1) // block_m
    P0 = seq_len - q_len
    for x in range(nx):
        q0 = (nx - 1 - x) * block_m
        if q0 >= q_len:
            continue
        rmax = min(q0 + block_m, q_len) - 1
        lo_key = max(0, P0 + q0 - window + 1) if window > 0 else 0
        hi_key = P0 + rmax
        out.append((q0, lo_key, hi_key, lo_key // KV_TILE, hi_key // KV_TILE))
    return out


def entries_read(seq_len, lo_key, t_lo, t_hi):
    """Indices into the sequence's block-table row the workgroup reads."""
    ppt = KV_TILE // BLOCK
    n_pages = (seq_len + BLOCK - 1) // BLOCK
    pg_lo = lo_key // BLOCK

    def page_blk(page):                            # the end clamp
        return page if page < n_pages else n_pages - 1

    idx = set()
    for i in range(2 * ppt):                       # tiles t_lo, t_lo + 1 (prologue)
        idx.add(page_blk(max((t_lo + i // ppt) * ppt + i % ppt, pg_lo)))
    t = t_lo
    while t <= t_hi:                               # loop unrolled by two
        for tt in (t, t + 1):
            if tt > t_hi:
                break
            for i in range(ppt):                   # block ids of tile tt+2
                page = (tt + 2) * ppt + i
                # the loop applies no lower clamp: its pages lie above the
                # window start by construction
                assert page >= pg_lo, (page, pg_lo)
                idx.add(page_blk(page))
        t += 2
    return idx


def zeroed_or_visible(seq_len, lo_key, hi_key, t):
    """For tile t: every key row either is visible to some row of the
    workgroup or has its V row zeroed by the kernel's staging step."""
    bad = []
    for r in range(KV_TILE):
        key = t * KV_TILE + r
        # the tail tile zeroes rows past the end; the prologue zeroes the
        # rows of tile t_lo before the window start
        zeroed = ((t + 1) * KV_TILE > seq_len and r >= seq_len - t * KV_TILE) or \
            (t == lo_key // KV_TILE and r < lo_key - t * KV_TILE)
        visible = lo_key <= key <= hi_key and key < seq_len
        if not (zeroed or visible):
            # a key above hi_key but below seq_len is a real, written key
            # that causal masking hides: finite data, p = 0
            if key < lo_key or key >= seq_len:
                bad.append(key)
    return bad


# the shapes of the prefill GPU tests (q_lens, seq_lens, window)
SHAPES = [
    ([200], [200], 0), ([130, 100, 17], [130, 400, 260], 0),
    ([130, 100, 17], [130, 400, 260], 100), ([130, 75], [130, 333], 0),
    ([70], [150], 0), ([1024], [1024], 0), ([8192], [8192], 0),
    ([32768], [32768], 0), ([32768], [131072], 0), ([130, 100, 17], [130, 1000, 260], 0),
]
for w in (100, 128, 513):
    SHAPES.append(([200, 130, 17], [1000, 700, 260], w))
    SHAPES.append(([300], [2000], w))
    SHAPES.append(([1], [513], w))
    SHAPES.append(([129, 128], [129, 4096], w))
    SHAPES.append(([300, 129], [2000, 4096], w))


@pytest.mark.parametrize("block_m", BLOCK_MS)
@pytest.mark.parametrize("q_lens,seq_lens,window", SHAPES)
def test_block_table_reads_stay_in_window(q_lens, seq_lens, window, block_m):
    max_q = max(q_lens)
    for T, L in zip(q_lens, seq_lens):
        lo_seq = max(0, L - T - window + 1) if window > 0 else 0
        n_pages = (L + BLOCK - 1) // BLOCK
        for q0, lo_key, hi_key, t_lo, t_hi in workgroups(T, L, window, max_q, block_m):
            idx = entries_read(L, lo_key, t_lo, t_hi)
            assert min(idx) >= lo_seq // BLOCK, (T, L, window, q0, sorted(idx)[:4])
            assert max(idx) <= n_pages - 1, (T, L, window, q0)


@pytest.mark.parametrize("block_m", BLOCK_MS)
@pytest.mark.parametrize("q_lens,seq_lens,window", SHAPES)
def test_invisible_staged_rows_are_zeroed(q_lens, seq_lens, window, block_m):
    max_q = max(q_lens)
    for T, L in zip(q_lens, seq_lens):
        for q0, lo_key, hi_key, t_lo, t_hi in workgroups(T, L, window, max_q, block_m):
            for t in range(t_lo, t_hi + 1):
                assert zeroed_or_visible(L, lo_key, hi_key, t) == [], (T, L, window, q0, t)


def test_model_sees_the_old_clamp_fail():
    # the earlier form (pages past the end read entry 0, no lower clamp, no
    # zeroing before the window start) reads entries outside the window for a
    # windowed chunk deep in its sequence: the model tells the two apart
    T, L, window = 300, 2000, 100
    lo_seq = L - T - window + 1
    old = set()
    for q0, lo_key, hi_key, t_lo, t_hi in workgroups(T, L, window, T):
        ppt = KV_TILE // BLOCK
        n_pages = (L + BLOCK - 1) // BLOCK
        for i in range(2 * ppt):
            page = (t_lo + i // ppt) * ppt + i % ppt
            old.add(page if page < n_pages else 0)
    assert min(old) < lo_seq // BLOCK


# (head_dim, query blocks per wave, waves per workgroup) of every prefill
# instantiation: prefill_mb and prefill_nwv, two-level/one-level then
# flush every N tiles
LAUNCH_SHAPES = [(256, 1, 4), (128, 2, 4), (64, 1, 4), (256, 1, 8), (128, 1, 8)]


@pytest.mark.parametrize("D,MB,NWV", LAUNCH_SHAPES)
def test_lane_block_ids_match_the_copies(D, MB, NWV):
    # copy u of wave w stages rows (idx % CPT) * RPI .. of the K (idx < CPT)
    # or V tile, idx = u * NWV + w; lane j holds the id of page
    # ((j % NCOPY) * NWV + w) % CPT * RPI / 16 and copy u broadcasts lane u's
    tile = KV_TILE * D
    rpi = 1024 // D
    cpt = tile // 1024
    ncopy = 2 * cpt // NWV
    assert 16 * MB * NWV in BLOCK_MS and ncopy >= 1 and BLOCK % rpi == 0
    staged = set()
    for w in range(NWV):
        lane_page = [((j % ncopy) * NWV + w) % cpt * rpi // BLOCK for j in range(64)]
        for u in range(ncopy):
            idx = u * NWV + w
            assert idx < 2 * cpt
            row0 = (idx % cpt) * rpi
            assert lane_page[u] == row0 // BLOCK, (D, NWV, w, u)
            staged |= {(idx // cpt, row0 + r) for r in range(rpi)}
    # the copies of all waves cover every row of the K and V tiles once
    assert staged == {(kv, r) for kv in (0, 1) for r in range(KV_TILE)}
