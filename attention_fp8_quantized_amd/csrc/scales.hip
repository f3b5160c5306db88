// Per-KV-head scales computed on the device from the data:
//   scale_h = max(fl32(absmax_h / 448), 2^-126),
//   absmax_h = largest finite |x| of head h over every row and channel.
//
// [GPUSTACK] "キャリブレーション": dynamic quantization computes each
// tensor's range at run time.  [EXPLAINER] "default scaleのまま本番へ出さない":
// a scale that does not fit the data either clips values or wastes code
// points.  [BLOG] "Kernel and vLLM improvements / Per-Head Scales": one scale
// per KV head.  The range is mapped onto the largest finite e4m3 value.
//
// Three launches on the caller's stream, all writing only the two scale
// arrays:
//   1. zero the arrays (they hold the absmax bit patterns meanwhile);
//   2. a streaming pass over k and v: every thread keeps the running maximum
//      of the absolute values of one 16-byte column of the rows it visits
//      (a column never straddles two heads), folds it into a per-head
//      maximum in LDS, and the workgroup folds that into the arrays with one
//      global unsigned max per head.  For non-negative floats the order of
//      the bit patterns as unsigned integers is the order of the values, so
//      the maxima are taken on bits; non-finite magnitudes count as 0;
//   3. one thread per head turns the maximum into the scale.
// The result does not depend on the order of the atomics (max is exact).

#include "fa8_device.hpp"
#include "fa8_internal.hpp"

namespace fa8 {

constexpr int kScaleThreads = 256;

__device__ __forceinline__ uint32_t finite_abs_bits(uint32_t bits) {
  const uint32_t a = bits & 0x7FFFFFFFu;
  return a < 0x7F800000u ? a : 0u;
}

__global__ void absmax_zero_kernel(uint32_t* __restrict__ k_bits, uint32_t* __restrict__ v_bits,
                                   int num_kv_heads) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < num_kv_heads) {
    k_bits[i] = 0u;
    v_bits[i] = 0u;
  }
}

// Running maximum of the finite |x| in one 16-byte chunk.
template <bool kBf16>
__device__ __forceinline__ uint32_t chunk_absmax(uint4 w, uint32_t m) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (kBf16) {
      m = max(m, finite_abs_bits(ws[j] << 16));
      m = max(m, finite_abs_bits(ws[j] & 0xFFFF0000u));
    } else {
      m = max(m, finite_abs_bits(ws[j]));
    }
  }
  return m;
}

// grid (workgroups, 2): blockIdx.y = 0 reads k, 1 reads v.  Rows are the
// tokens, each num_kv_heads*head_dim elements = `cols` 16-byte chunks.  With
// cols <= 256 a workgroup covers `rpi` = 256/cols rows per step (thread t:
// row t/cols, column t%cols); otherwise one row per step and every thread
// walks the columns t, t+256, ...
template <bool kBf16>
__global__ __launch_bounds__(kScaleThreads) void absmax_reduce_kernel(
    const void* __restrict__ k, const void* __restrict__ v, int64_t n_tokens,
    int num_kv_heads, int head_dim, uint32_t* __restrict__ k_bits,
    uint32_t* __restrict__ v_bits) {
  extern __shared__ uint32_t s_max[];  // [num_kv_heads]
  const int which = blockIdx.y;
  const uint4* __restrict__ src = reinterpret_cast<const uint4*>(which ? v : k);
  uint32_t* __restrict__ bits = which ? v_bits : k_bits;

  constexpr int kPerChunk = kBf16 ? 8 : 4;
  const int cols = num_kv_heads * head_dim / kPerChunk;
  const int chunks_per_head = head_dim / kPerChunk;
  const int t = threadIdx.x;
  for (int h = t; h < num_kv_heads; h += kScaleThreads) s_max[h] = 0u;
  __syncthreads();

  const int rpi = cols <= kScaleThreads ? kScaleThreads / cols : 1;
  const int r_off = cols <= kScaleThreads ? t / cols : 0;
  const int64_t row_step = (int64_t)gridDim.x * rpi;
  if (r_off < rpi) {
    for (int c = cols <= kScaleThreads ? t % cols : t; c < cols; c += kScaleThreads) {
      uint32_t m = 0u;
      int64_t r = (int64_t)blockIdx.x * rpi + r_off;
      // four rows in flight per step
      for (; r + 3 * row_step < n_tokens; r += 4 * row_step) {
        uint4 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = src[(r + u * row_step) * cols + c];
#pragma unroll
        for (int u = 0; u < 4; ++u) m = chunk_absmax<kBf16>(w[u], m);
      }
      for (; r < n_tokens; r += row_step) m = chunk_absmax<kBf16>(src[r * cols + c], m);
      if (m != 0u) atomicMax(&s_max[c / chunks_per_head], m);
    }
  }
  __syncthreads();
  for (int h = t; h < num_kv_heads; h += kScaleThreads) {
    const uint32_t m = s_max[h];
    if (m != 0u) atomicMax(&bits[h], m);
  }
}

__global__ void absmax_finalize_kernel(uint32_t* __restrict__ k_bits,
                                       uint32_t* __restrict__ v_bits, int num_kv_heads,
                                       float fmt_max) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= 2 * num_kv_heads) return;
  uint32_t* p = i < num_kv_heads ? k_bits + i : v_bits + (i - num_kv_heads);
  // correctly rounded fp32 division (no fast-math in this library's build)
  const float s = __uint_as_float(*p) / fmt_max;
  *p = __float_as_uint(fmaxf(s, 0x1p-126f));
}

int absmax_reduce_grid(int64_t n_tokens, int num_kv_heads, int head_dim, bool in_bf16,
                       int cus) {
  const int cols = num_kv_heads * head_dim / (in_bf16 ? 8 : 4);
  const int64_t rpi = cols <= kScaleThreads ? kScaleThreads / cols : 1;
  const int64_t steps = (n_tokens + rpi - 1) / rpi;
  // each workgroup at least 4 steps (the loads in flight), at most 4 per CU
  int64_t wgs = (steps + 3) / 4;
  const int64_t cap = 4L * cus;
  if (wgs > cap) wgs = cap;
  if (wgs < 1) wgs = 1;
  return (int)wgs;
}

hipError_t launch_absmax_scales(const void* k, const void* v, bool in_bf16, int64_t n_tokens,
                                int num_kv_heads, int head_dim, float* k_scale,
                                float* v_scale, float fmt_max, int cus,
                                hipStream_t stream) {
  uint32_t* kb = reinterpret_cast<uint32_t*>(k_scale);
  uint32_t* vb = reinterpret_cast<uint32_t*>(v_scale);
  const int small = (num_kv_heads + 255) / 256;
  hipLaunchKernelGGL(absmax_zero_kernel, dim3(small), dim3(256), 0, stream, kb, vb,
                     num_kv_heads);
  if (n_tokens > 0) {
    const dim3 grid(absmax_reduce_grid(n_tokens, num_kv_heads, head_dim, in_bf16, cus), 2);
    const size_t lds = (size_t)num_kv_heads * sizeof(uint32_t);
    if (in_bf16)
      hipLaunchKernelGGL((absmax_reduce_kernel<true>), grid, dim3(kScaleThreads), lds, stream,
                         k, v, n_tokens, num_kv_heads, head_dim, kb, vb);
    else
      hipLaunchKernelGGL((absmax_reduce_kernel<false>), grid, dim3(kScaleThreads), lds, stream,
                         k, v, n_tokens, num_kv_heads, head_dim, kb, vb);
  }
  hipLaunchKernelGGL(absmax_finalize_kernel, dim3((2 * num_kv_heads + 255) / 256), dim3(256),
                     0, stream, kb, vb, num_kv_heads, fmt_max);
  return hipGetLastError();
}

}  // namespace fa8
