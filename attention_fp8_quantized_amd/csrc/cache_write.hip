// Cache write: quantise new K/V rows with their per-KV-head scale and scatter
// them into 16-token pages (e4m3 or e5m2 codes, or bf16 values).
//
// [BLOG] "Kernel and vLLM improvements / Per-Head Scales": the cache-write
// kernel takes an array of scales, one per KV head.  [EXPLAINER] "FP8
// combines value and scale": the value is divided by its scale before it is
// quantised.  Rounding is nearest-even with saturation at the format's largest
// finite value (448 for e4m3, 57344 for e5m2).
//
// One thread produces one 16-byte chunk of one cached row: 16 FP8 codes or
// 8 bf16 values.  Threads of a block walk (token, head, chunk) with the chunk
// fastest, so input reads are contiguous; blockIdx.y picks K (0) or V (1).
// The work is a single HBM-bound pass.  The fp32 quotient x / scale must be
// correctly rounded: this file is built without fast-math and with
// -fhip-fp32-correctly-rounded-divide-sqrt.

#include "fa8_device.hpp"
#include "fa8_internal.hpp"

namespace fa8 {

// kIdx: the integer type of the chunk index (uint32_t whenever the chunk
// count fits, so the index splits into (token, head, chunk) with 32-bit
// divisions instead of 64-bit ones).
template <bool kInBf16, int kFmt, typename kIdx>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const void* __restrict__ k, const void* __restrict__ v, int64_t n_tokens,
    int num_kv_heads, int head_dim, const int64_t* __restrict__ slot_mapping,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    uint8_t* __restrict__ cache) {
  constexpr bool kFp8Cache = kFmt != kFmtBf16;
  constexpr int kElemBytes = kFp8Cache ? 1 : 2;
  constexpr int kPerThread = 16 / kElemBytes;  // elements per 16-byte chunk
  const int chunks_per_row = head_dim / kPerThread;
  const int64_t total = n_tokens * num_kv_heads * chunks_per_row;
  const int which = blockIdx.y;  // 0 = K, 1 = V
  const void* src = which ? v : k;
  const float* scale = which ? v_scale : k_scale;

  const kIdx cpr = (kIdx)chunks_per_row, nkv = (kIdx)num_kv_heads;
  for (kIdx t = (kIdx)blockIdx.x * blockDim.x + threadIdx.x; t < (kIdx)total;
       t += (kIdx)gridDim.x * blockDim.x) {
    const int c = (int)(t % cpr);
    const kIdx rest = t / cpr;
    const int h = (int)(rest % nkv);
    const int64_t n = (int64_t)(rest / nkv);
    const int64_t slot = slot_mapping[n];
    if (slot < 0) continue;  // padding row

    const uint4 chunk = encode_chunk<kInBf16, kFmt>(
        src, (n * num_kv_heads + h) * head_dim + c * kPerThread, kFp8Cache ? scale[h] : 1.0f);

    const int64_t blk = slot / kBlockSize;
    const int row = (int)(slot % kBlockSize);
    const int64_t off =
        ((((blk * num_kv_heads + h) * 2 + which) * kBlockSize + row) * head_dim +
         (int64_t)c * kPerThread) * kElemBytes;
    *reinterpret_cast<uint4*>(cache + off) = chunk;
  }
}

hipError_t launch_cache_write(const void* k, const void* v, bool in_bf16,
                              int64_t n_tokens, int num_kv_heads, int head_dim,
                              const int64_t* slot_mapping, const float* k_scale,
                              const float* v_scale, void* cache, int fmt,
                              hipStream_t stream) {
  const int per = fmt != kFmtBf16 ? 16 : 8;
  const int64_t total = n_tokens * num_kv_heads * (head_dim / per);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65535) blocks = 65535;  // grid-stride loop covers the rest
  dim3 grid((unsigned)blocks, 2);
  uint8_t* c = reinterpret_cast<uint8_t*>(cache);
  // the grid-stride index stays below total + gridDim.x * blockDim.x
  const bool idx32 = total + (int64_t)blocks * threads < ((int64_t)1 << 32);
#define FA8_CW(BF, FMT)                                                                       \
  do {                                                                                        \
    if (idx32)                                                                                \
      hipLaunchKernelGGL((cache_write_kernel<BF, FMT, uint32_t>), grid, threads, 0, stream, k, \
                         v, n_tokens, num_kv_heads, head_dim, slot_mapping, k_scale, v_scale, c); \
    else                                                                                      \
      hipLaunchKernelGGL((cache_write_kernel<BF, FMT, uint64_t>), grid, threads, 0, stream, k, \
                         v, n_tokens, num_kv_heads, head_dim, slot_mapping, k_scale, v_scale, c); \
  } while (0)
  switch (fmt) {
    case kFmtE4m3: if (in_bf16) FA8_CW(true, kFmtE4m3); else FA8_CW(false, kFmtE4m3); break;
    case kFmtE5m2: if (in_bf16) FA8_CW(true, kFmtE5m2); else FA8_CW(false, kFmtE5m2); break;
    case kFmtBf16: if (in_bf16) FA8_CW(true, kFmtBf16); else FA8_CW(false, kFmtBf16); break;
    default: return hipErrorInvalidValue;
  }
#undef FA8_CW
  return hipGetLastError();
}

}  // namespace fa8
