/*
 * fa8attn: attention over an FP8-e4m3 paged KV cache with per-KV-head scales,
 * for AMD CDNA4 (gfx950 / MI355X).  C ABI of libfa8attn.so.
 *
 * Pages the operations follow (cited by title and section):
 *   [BLOG]      "State of FP8 KV-Cache and Attention Quantization in vLLM"
 *               (vLLM Blog, 2026-04-22).
 *   [EXPLAINER] "KV Cache量子化とは？FP8でLLMの同時実行数を増やす前に測ること"
 *               (vasteelab.pages.dev, 2026-10-07).
 * The e4m3 bits follow the OCP OFP8 E4M3 definition (bias 7, max 448, no
 * infinity, S.1111.111 = NaN), which the pages name but do not spell out.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller (normally
 *   the storage of a torch tensor).  The library allocates nothing; scratch
 *   space for decode is a caller-sized workspace (fa8_decode_attention_noalloc
 *   uses a fixed array of the library's own instead, described there).
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL = the null stream).  No call synchronises with the host or copies
 *   between host and device, so every call can be captured in a HIP graph.
 * - Paged cache layout, one allocation per layer:
 *       cache[num_blocks][num_kv_heads][2][16][head_dim]
 *   index 2 is 0 = K, 1 = V; 16 tokens per block (page).  A token with slot
 *   id t lives in block t / 16, row t % 16.  Element type: one byte per
 *   element for the FP8 caches (an e4m3 code for FA8_E4M3, an e5m2 code for
 *   FA8_E5M2), two (bf16 bits) for FA8_BF16.  The
 *   K rows and the V rows of one (block, head) are each 16*head_dim elements
 *   of contiguous memory.
 * - Scales: k_scale[num_kv_heads], v_scale[num_kv_heads] fp32 in device
 *   memory, one per KV head ([BLOG] "Kernel and vLLM improvements /
 *   Per-Head Scales").  A per-tensor scale is the case of equal entries.
 *   Dequantised value = scale * decode(code).  Scales must be finite and
 *   positive (not checked on the device).
 * - Errors: host-side checks return FA8_EINVAL (bad argument) or
 *   FA8_EUNSUPPORTED (valid but not built, e.g. head_dim 96, or a batch or
 *   head count above 65535 for decode and prefill) before anything is
 *   launched; a failed launch returns FA8_EHIP.  fa8_last_error() gives a
 *   message for the calling thread.  Indices that only the device sees
 *   (slot ids, block ids, sequence lengths) are preconditions: out-of-range
 *   values are undefined behaviour.
 */
#ifndef FA8ATTN_H
#define FA8ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA8_OK = 0,
  FA8_EINVAL = 1,
  FA8_EUNSUPPORTED = 2,
  FA8_EHIP = 3
} fa8_status;

/*
 * FA8_E5M2 is the OCP OFP8 E5M2 encoding (bias 15, max finite 57344,
 * S.11111.00 = inf, other exponent-31 codes NaN), the second FP8 cache format
 * [GPUSTACK] "KV キャッシュの量子化" names.  Both FP8 caches follow one
 * contract: round-to-nearest-even, saturation at the largest finite value
 * (so an e5m2 cache never holds an infinity), NaN -> 0x7F|sign.
 */
typedef enum { FA8_F32 = 0, FA8_BF16 = 1, FA8_E4M3 = 2, FA8_E5M2 = 3 } fa8_dtype;

#define FA8_BLOCK_SIZE 16

/*
 * Quantise and scatter new K/V rows into the paged cache.
 * [BLOG] "Kernel and vLLM improvements / Per-Head Scales" (the cache-write
 * kernel takes one scale per KV head); [EXPLAINER] "FP8 combines value and
 * scale" (values are divided by their scale before quantisation).
 *
 *   k, v          [n_tokens][num_kv_heads][head_dim], in_dtype FA8_F32 or
 *                 FA8_BF16, row-major, contiguous.
 *   slot_mapping  int64 [n_tokens]; a negative slot skips the row (padding).
 *                 Slots must be < num_blocks*16 and pairwise distinct.
 *   cache         see the layout above; cache_dtype FA8_E4M3, FA8_E5M2 or
 *                 FA8_BF16.
 * FA8_E4M3: code = e4m3(fl32(x / scale[h])) with the fp32 quotient
 *   correctly rounded, then round-to-nearest-even, saturation at +-448
 *   (also for +-inf), NaN -> 0x7F|sign, sign of zero kept.
 * FA8_E5M2: the same with e5m2 codes, saturation at +-57344.
 * FA8_BF16: the bf16 rounding (nearest-even) of x; scales are not read and
 *   may be NULL (layers kept in BF16, [BLOG] "Skipping layers").
 * n_tokens == 0 is a no-op.
 */
fa8_status fa8_cache_write(const void* k, const void* v, int32_t in_dtype,
                           int64_t n_tokens, int32_t num_kv_heads,
                           int32_t head_dim, const int64_t* slot_mapping,
                           const float* k_scale, const float* v_scale,
                           void* cache, int32_t cache_dtype, int64_t num_blocks,
                           void* stream);

/*
 * Per-KV-head scales computed on the device from the rows about to be
 * cached (dynamic scales).  [GPUSTACK] "キャリブレーション" (dynamic
 * quantization measures the value range at run time); [EXPLAINER]
 * "default scaleのまま本番へ出さない" (a scale must fit the data: too small
 * clips, too large wastes code points); [BLOG] "Kernel and vLLM improvements
 * / Per-Head Scales" (one scale per KV head).
 *
 *   k, v          [n_tokens][num_kv_heads][head_dim], in_dtype FA8_F32 or
 *                 FA8_BF16, row-major, contiguous (the same rows
 *                 fa8_cache_write takes).
 *   cache_dtype   the FP8 format the scales are for: each head's largest
 *                 magnitude maps onto the format's largest finite value,
 *                 F = 448 for FA8_E4M3, 57344 for FA8_E5M2.
 *   k_scale, v_scale  fp32 [num_kv_heads], written:
 *       scale[h] = max(fl32(absmax_h / F), 2^-126)
 *   with absmax_h the largest |x| over all finite entries of head h (NaN
 *   and +-inf are skipped; no rows or all zeros give the floor 2^-126) and
 *   the fp32 quotient correctly rounded.  The result is exact: it does not
 *   depend on the order in which the device combines partial maxima.
 * Between the call's launches k_scale/v_scale hold intermediate bit
 * patterns; they are final once the stream reaches the end of the call.
 * k_scale and v_scale must not overlap k or v.  n_tokens == 0 writes the
 * floor.  num_kv_heads is at most 4096.
 */
fa8_status fa8_absmax_scales(const void* k, const void* v, int32_t in_dtype,
                             int64_t n_tokens, int32_t num_kv_heads, int32_t head_dim,
                             int32_t cache_dtype, float* k_scale, float* v_scale,
                             void* stream);

/*
 * Split-KV decode: number of context splits the library picks for a batch
 * (host-only heuristic; depends on the device's CU count).  `window` as in
 * fa8_decode_attention.  Always >= 1.
 */
int32_t fa8_decode_num_splits(int32_t batch, int32_t num_kv_heads,
                              int32_t max_seq_len, int32_t window);

/*
 * Bytes of device workspace fa8_decode_attention needs for `num_splits`
 * splits: int32 arrival counters, each on its own 256-byte line (2 per
 * sequence and query head for up to 64 splits; beyond, NG + 2 with
 * NG = ceil(splits / 16) split groups), then per (sequence, query head,
 * split) one unnormalised partial output row (head_dim fp32) plus its running
 * maximum and denominator (2 fp32).
 */
size_t fa8_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                  int32_t head_dim, int32_t num_splits);

/*
 * One decode step of grouped-query attention over the paged cache.
 * [BLOG] "Performance benchmarks / Single-request benchmark" (the kernel
 * reads the FP8 cache natively, rescaling its online softmax as it goes);
 * [EXPLAINER] "Memory reduction is not speed" (quantised values are
 * dequantised inside the attention kernel, not in a separate pass).
 *
 *   q            bf16 [batch][num_q_heads][head_dim]; query head hq reads
 *                KV head hq / (num_q_heads / num_kv_heads).
 *   block_table  int32 [batch][max_blocks_per_seq] physical block ids.
 *                Only the entries of pages that hold a visible key are used:
 *                pages lo/16 .. (seq_lens[b]-1)/16 with lo the first key of
 *                the window (0 without one).  With a window, no other entry
 *                is read; without one, entries past the sequence end (within
 *                the row) may be read early but are never used.  Unused
 *                entries may hold anything (a freed page, -1), and the cache
 *                rows of invisible keys (also the rows of a visible page
 *                before lo or past the end) may hold any bytes, NaN codes
 *                included: they never reach the output.
 *   seq_lens     int32 [batch]; the query is token seq_lens[b]-1, whose K/V
 *                must already be in the cache.  0 gives a zero output row.
 *   max_seq_len  host upper bound of seq_lens (sizes the grid only).
 *   k_scale/v_scale  per-KV-head scales (read for the FP8 caches only).
 *   sm_scale     softmax scale (usually 1/sqrt(head_dim)).
 *   window       > 0: attend to the last `window` keys (the query's own
 *                token included); <= 0: the whole context.
 *   num_splits   context splits, 0..256; 0 = fa8_decode_num_splits(...).
 *                Beyond 64 splits up to 64 merging workgroups of a
 *                (sequence, KV head) wait, with a bounded poll, for its
 *                other splits: FA8_EUNSUPPORTED on a device with 64 or
 *                fewer compute units (fa8_decode_num_splits never picks
 *                more splits than there are compute units).
 *   out          fp32 [batch][num_q_heads][head_dim]
 *                out = sum_j softmax(sm_scale * q.K_j) * V_j.
 *   workspace    >= fa8_decode_workspace_bytes(batch, num_q_heads,
 *                head_dim, splits) bytes, 16-byte aligned.  It must be
 *                zero-filled before its first use; every call leaves its
 *                arrival counters at zero again, so a workspace can be reused
 *                without clearing.  Calls that share a workspace must be
 *                ordered on one stream.
 * Supported: head_dim in {64, 128, 256}; num_q_heads / num_kv_heads in
 * {1, 2, 4, 8, 16}; cache_dtype FA8_E4M3, FA8_E5M2 or FA8_BF16.
 */
fa8_status fa8_decode_attention(const void* q, int32_t batch,
                                int32_t num_q_heads, const void* cache,
                                int32_t cache_dtype, int64_t num_blocks,
                                int32_t num_kv_heads, int32_t head_dim,
                                const int32_t* block_table,
                                int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                const float* k_scale, const float* v_scale,
                                float sm_scale, int32_t window,
                                int32_t num_splits, float* out,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same operation, arguments, results and errors as
 * fa8_decode_attention, without the workspace: the split partials and
 * arrival counters live in a fixed scratch array inside the library,
 * FA8_DECODE_SCRATCH_BYTES on each GPU the library runs on, held until the
 * process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine).
 * Limits (FA8_EINVAL beyond them, before anything is launched), with S the
 * split count (num_splits, or fa8_decode_num_splits(...) when 0):
 *   batch * num_q_heads * C <= FA8_DECODE_SCRATCH_COUNTERS, where
 *     C = 2 for S <= 64, else ceil(S / 16) + 2, and
 *   fa8_decode_workspace_bytes(batch, num_q_heads, head_dim, S) minus the
 *     counters' bytes (256 per counter) <= FA8_DECODE_SCRATCH_BYTES - 256 *
 *     FA8_DECODE_SCRATCH_COUNTERS
 *   (e.g. 32 query heads, head_dim 128, batch 8 and up to 100 splits fit).
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * partials: calls that overlap on one GPU (two streams, two threads without
 * ordering) race and give wrong results, so order them on one stream.  The
 * counters must be zero at the start of a call; every call leaves them
 * zero, and the first call on a device that is not being captured clears
 * them first with a small kernel on `stream` (a captured call records that
 * clear in its graph until an eager call has done it).
 */
#define FA8_DECODE_SCRATCH_BYTES (16u << 20)
#define FA8_DECODE_SCRATCH_COUNTERS 4096
fa8_status fa8_decode_attention_noalloc(const void* q, int32_t batch,
                                        int32_t num_q_heads, const void* cache,
                                        int32_t cache_dtype, int64_t num_blocks,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        const int32_t* block_table,
                                        int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, int32_t max_seq_len,
                                        const float* k_scale, const float* v_scale,
                                        float sm_scale, int32_t window,
                                        int32_t num_splits, float* out, void* stream);

/*
 * Fused decode step: write the current token's K/V into the cache and attend
 * over the context including it, in one launch.  [BLOG] "Kernel 与 vLLM 改进"
 * and "单请求 Benchmark": quantising the new token is a fixed per-step cost
 * (the ITL intercept); here it rides on the decode launch instead of a
 * separate cache-write launch.
 *
 * Same arguments and results as fa8_decode_attention, plus:
 *   k_new, v_new  [batch][num_kv_heads][head_dim] rows of the current token
 *                 (position seq_lens[b]-1 of each sequence), in_dtype FA8_F32
 *                 or FA8_BF16.
 *   cache         written: the row at slot
 *                 block_table[b][(seq_lens[b]-1)/16]*16 + (seq_lens[b]-1)%16
 *                 of each sequence with seq_lens[b] > 0 receives exactly the
 *                 bytes fa8_cache_write would store for that row.
 * The decode output equals running fa8_cache_write on those rows followed
 * by fa8_decode_attention.
 */
fa8_status fa8_decode_attention_append(const void* q, const void* k_new, const void* v_new,
                                       int32_t in_dtype, int32_t batch, int32_t num_q_heads,
                                       void* cache, int32_t cache_dtype, int64_t num_blocks,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       const float* k_scale, const float* v_scale,
                                       float sm_scale, int32_t window, int32_t num_splits,
                                       float* out, void* workspace, size_t workspace_bytes,
                                       void* stream);

/*
 * Width (keys) of the KV tiles fa8_prefill_attention visits, in ascending,
 * tile-aligned order from key 0.  It is part of the numeric contract: the
 * probabilities are quantised to e4m3 against the running maximum reached
 * after each tile.  Returns 0 for an unsupported head_dim.
 */
int32_t fa8_prefill_kv_tile(int32_t head_dim);

/*
 * Causal FP8 prefill over the paged cache with two-level accumulation.
 * [BLOG] "Introduction" (QK and Score*V both run in e4m3); "Kernel and vLLM
 * improvements / Two-level accumulation" (partial P*V sums are flushed into
 * true FP32 registers); "Query Quantization Fusion" (Q is quantised with a
 * per-tensor scale right before attention).
 *
 *   q          bf16 [total_q][num_q_heads][head_dim], sequences packed;
 *              sequence b owns rows cu_q_lens[b] .. cu_q_lens[b+1]-1.
 *   cu_q_lens  int32 [batch+1], cu_q_lens[0] = 0.
 *   max_q_len  host upper bound of the per-sequence query counts.
 *   seq_lens   int32 [batch]: context length INCLUDING this chunk; the
 *              chunk's queries sit at positions seq_len - q_len .. seq_len-1
 *              and their K/V must already be in the cache.
 *   block_table  int32 [batch][max_blocks_per_seq].  Only the entries of
 *              pages lo/16 .. (seq_len-1)/16 are read, lo being the first
 *              key the chunk's first query sees (its position - window + 1,
 *              at least 0; 0 without a window).  Entries outside that range
 *              may hold anything (a freed page, -1), and cache rows no query
 *              sees (before a window start, past the end) may hold any
 *              bytes, NaN codes included: they never reach the output.
 *   q_scale    fp32 [1] device: q8 = e4m3(fl32(q / q_scale)) (the query is
 *              e4m3 whatever the cache's FP8 format).
 *   cache_dtype  FA8_E4M3 or FA8_E5M2: the format of K and V codes.  P is
 *              always e4m3; the P*V matrix product takes e5m2 V directly.
 *   window     as in decode, counted from each query's own position.
 *   accum_mode 1 = two-level (MFMA sums each KV tile into a zeroed fp32
 *              register tile, then O = alpha*O + tile in fp32; default);
 *              0 = one-level (MFMA accumulates into the rescaled O);
 *              N in 2..65536 = flush every N tiles ([BLOG] "大 Head
 *              Dimension 的限制": a level-1 accumulator spans N tiles, with
 *              its own alpha rescaling, before O = alpha'*O + acc).  All
 *              modes compute the same quantity; they differ in rounding.
 *   out        fp32 [total_q][num_q_heads][head_dim].
 * Per row and KV tile t (width fa8_prefill_kv_tile): running max m_t,
 * p = exp(s - m_t) in fp32, P*V uses e4m3(p), the denominator the fp32 p.
 * Supported: head_dim in {64, 128, 256}; cache_dtype FA8_E4M3 or FA8_E5M2.
 */
fa8_status fa8_prefill_attention(const void* q, const int32_t* cu_q_lens,
                                 int32_t batch, int32_t num_q_heads,
                                 int32_t max_q_len, const void* cache,
                                 int32_t cache_dtype,
                                 int64_t num_blocks, int32_t num_kv_heads,
                                 int32_t head_dim, const int32_t* block_table,
                                 int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, const float* q_scale,
                                 const float* k_scale, const float* v_scale,
                                 float sm_scale, int32_t window,
                                 int32_t accum_mode, float* out, void* stream);

/*
 * Bandwidth yardsticks (not part of attention).  Decode is a streaming
 * reader of the cache, so its HBM rate is also reported against what a plain
 * streaming read achieves on the same device; the copy is a kernel of known
 * traffic (reads `bytes`, writes `bytes`) for calibrating hardware byte
 * counters.
 *
 *   fa8_stream_read  reads src[0 .. bytes) once with 16-byte loads; `sink`
 *                    (device, 4 bytes) is written only for one improbable
 *                    xor of the data, so the loads cannot be dropped.
 *   fa8_stream_copy  dst[0 .. bytes) = src[0 .. bytes); the ranges must not
 *                    overlap.
 * bytes must be a multiple of 16 (FA8_EINVAL otherwise); pointers 16-byte
 * aligned device memory; asynchronous on `stream`.
 */
fa8_status fa8_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);
fa8_status fa8_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Static English name of a status code. */
const char* fa8_status_string(int32_t status);

/* Message of the last failed call on this thread ("" if none). */
const char* fa8_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA8ATTN_H */
