// Split-KV decode over the paged FP8 / BF16 cache, with the cross-split
// log-sum-exp combine fused into the same launch.
//
// [BLOG] "Performance benchmarks / Single-request benchmark": decode time is
// the per-token KV read, the FP8 cache is read natively and the online
// softmax is rescaled as the kernel goes.  [EXPLAINER] "Memory reduction is
// not speed": dequantisation happens inside the attention kernel, in
// registers, not as a separate pass back to high precision.
//
// Work decomposition (one workgroup per (split, KV head [x head group], seq)):
//   * the context pages of a sequence are cut into `num_splits` contiguous
//     page ranges; the NW waves of a workgroup take the pages of its range
//     round-robin, one 16-token page at a time;
//   * a page-head is 16 rows of D elements, i.e. 16*D*elem bytes of
//     contiguous memory for K and again for V.  Each lane loads 16-byte
//     chunks: LPT = D*elem/16 lanes cover one row, so one wave-wide load
//     covers TPW = 64/LPT rows (a contiguous 1 KiB) and every global load is
//     fully coalesced.  The next page is loaded while the current one is
//     processed (register double buffer);
//   * lanes of one row hold the same d-range of q for the GW query heads
//     that share the KV head (GQA).  Partial q.k dots use v_dot2_f32_bf16 on
//     bf16 pairs: e4m3 codes convert exactly to bf16 with one instruction per
//     pair, bf16 cache rows are used as they are.  The LPT partials are summed
//     with DPP lane permutes;
//   * each group of LPT lanes (a "row slot") keeps its own online-softmax
//     state (running max m and sum l in the log2 domain, fp32 output slice);
//     slots are merged with shuffles at the end, waves through LDS, and the
//     workgroup writes one unnormalised partial (o, m, l) per query head;
//   * the last workgroup of a (sequence, head group) to finish merges the
//     splits:  out = v_scale * sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Scales are folded: k_scale into the score multiplier, v_scale into the
// combine.  Empty splits carry m = -inf and weight 0; an all-empty row is 0.

#include "fa8_device.hpp"
#include "fa8_internal.hpp"

namespace fa8 {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxSplits = kDecodeMaxSplits;

// Merge the S split partials of GW query heads (run by one workgroup):
//   out = v_scale * sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Threads are laid out as (split row sr, 4-element column d4) so that many
// splits are read at once with 16-byte loads; one pass covers RPP splits.
template <int D, int GW, int NW>
__device__ __forceinline__ void combine_splits(const DecodeParams& p, int b, int h, int hq0) {
  constexpr int NT = 64 * NW;
  constexpr int TPR = D / 4;          // threads per split row
  constexpr int RPP = NT / TPR;       // split rows per pass
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[NT];
  __shared__ float4 s_acc[RPP][TPR];
  const int S = p.num_splits;
  const int t = threadIdx.x;
  const int sr = t / TPR;
  const int d4 = t % TPR;
  const float vsc = p.fp8 ? p.v_scale[h] : 1.0f;
  for (int g = 0; g < GW; ++g) {
    const size_t base = ((size_t)b * p.num_q_heads + hq0 + g) * S;
    // M = max_s m_s
    float M = kNegInf;
    for (int s = t; s < S; s += NT) M = fmaxf(M, p.ws_m[base + s]);
    s_red[t] = M;
    __syncthreads();
    for (int w = NT / 2; w > 0; w /= 2) {
      if (t < w) s_red[t] = fmaxf(s_red[t], s_red[t + w]);
      __syncthreads();
    }
    M = s_red[0];
    __syncthreads();
    // split weights 2^(m_s - M) and the denominator
    float den = 0.f;
    for (int s = t; s < S; s += NT) {
      const float ms = p.ws_m[base + s];
      const float f = (ms > kNegInf) ? fast_exp2(ms - M) : 0.f;
      s_w[s] = f;
      den += f * p.ws_l[base + s];
    }
    s_red[t] = den;
    __syncthreads();
    for (int w = NT / 2; w > 0; w /= 2) {
      if (t < w) s_red[t] += s_red[t + w];
      __syncthreads();
    }
    den = s_red[0];
    // numerator
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4* o4 = reinterpret_cast<const float4*>(p.ws_o + base * D);
    for (int s = sr; s < S; s += RPP) {
      const float f = s_w[s];
      const float4 v = o4[(size_t)s * TPR + d4];
      acc.x += f * v.x;
      acc.y += f * v.y;
      acc.z += f * v.z;
      acc.w += f * v.w;
    }
    s_acc[sr][d4] = acc;
    __syncthreads();
    if (t < TPR) {
      float4 r = s_acc[0][t];
      for (int q = 1; q < RPP; ++q) {
        r.x += s_acc[q][t].x;
        r.y += s_acc[q][t].y;
        r.z += s_acc[q][t].z;
        r.w += s_acc[q][t].w;
      }
      float4 res = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M > kNegInf) {
        const float sc = vsc / den;
        res = make_float4(r.x * sc, r.y * sc, r.z * sc, r.w * sc);
      }
      reinterpret_cast<float4*>(p.out + ((size_t)b * p.num_q_heads + hq0 + g) * D)[t] = res;
    }
    __syncthreads();
  }
}

template <int D, int GW, bool kFp8, int NW>
__global__ __launch_bounds__(64 * NW) void decode_split_kernel(DecodeParams p) {
  constexpr int ES = kFp8 ? 1 : 2;          // bytes per cached element
  constexpr int EPC = 16 / ES;              // elements per 16-byte lane chunk
  constexpr int LPT = D / EPC;              // lanes per token row
  constexpr int TPW = 64 / LPT;             // rows per wave-wide load
  constexpr int RPL = kBlockSize / TPW;     // rows per lane per page half
  constexpr int ROW_BYTES = D * ES;
  constexpr int HALF_BYTES = kBlockSize * ROW_BYTES;
  static_assert(LPT * TPW == 64 && RPL * TPW == kBlockSize, "tiling");

  const int split = blockIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int groups = G / GW;
  const int h = blockIdx.y / groups;
  const int hq0 = h * G + (blockIdx.y % groups) * GW;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slot = lane / LPT;
  const int c = lane % LPT;

  const int L = p.seq_lens[b];
  const int lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int page_lo = lo / kBlockSize;
  const int page_hi = (L + kBlockSize - 1) / kBlockSize;
  const int pg0 = page_lo + split * p.pages_per_split;
  const int pg1 = min(pg0 + p.pages_per_split, page_hi);

  // q slice (bf16 pairs) for d = c*EPC .. c*EPC+EPC-1 of each query head
  uint32_t qw[GW][EPC / 2];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    const uint4* src = reinterpret_cast<const uint4*>(
        p.q + ((size_t)b * p.num_q_heads + hq0 + g) * D + c * EPC);
#pragma unroll
    for (int i = 0; i < EPC / 8; ++i) {
      const uint4 w = src[i];
      qw[g][4 * i + 0] = w.x;
      qw[g][4 * i + 1] = w.y;
      qw[g][4 * i + 2] = w.z;
      qw[g][4 * i + 3] = w.w;
    }
  }
  const float qk_scale = p.sm_scale * kLog2e * (kFp8 ? p.k_scale[h] : 1.0f);

  float m[GW], l[GW], o[GW][EPC];
#pragma unroll
  for (int g = 0; g < GW; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[g][e] = 0.f;
  }

  const uint8_t* head_base = p.cache + (size_t)h * 2 * HALF_BYTES;
  const size_t blk_stride = (size_t)p.num_kv_heads * 2 * HALF_BYTES;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
  const int lane_off = slot * ROW_BYTES + c * 16;

  uint4 kr[RPL], vr[RPL];
  auto load_page = [&](int pg, uint4(&kd)[RPL], uint4(&vd)[RPL]) {
    const uint8_t* kb = head_base + (size_t)bt[pg] * blk_stride + lane_off;
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      kd[r] = *reinterpret_cast<const uint4*>(kb + r * TPW * ROW_BYTES);
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      vd[r] = *reinterpret_cast<const uint4*>(kb + HALF_BYTES + r * TPW * ROW_BYTES);
  };

  int pg = pg0 + wave;
  if (pg < pg1) load_page(pg, kr, vr);
  for (; pg < pg1; pg += NW) {
    uint4 kn[RPL], vn[RPL];
    const int pn = pg + NW;
    if (pn < pg1) load_page(pn, kn, vn);

    // ---- scores s = (q . k) * sm_scale * k_scale * log2(e) ----------------
    float s[RPL][GW];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const int tok = pg * kBlockSize + slot + r * TPW;
      const bool valid = tok >= lo && tok < L;
      const uint32_t kw[4] = {kr[r].x, kr[r].y, kr[r].z, kr[r].w};
      float part[GW];
#pragma unroll
      for (int g = 0; g < GW; ++g) part[g] = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (kFp8) {
          const bf16x2 k01 = e4m3x2_to_bf16<false>(kw[w]);
          const bf16x2 k23 = e4m3x2_to_bf16<true>(kw[w]);
#pragma unroll
          for (int g = 0; g < GW; ++g) {
            part[g] = dot2_bf16(as_bf16x2(qw[g][2 * w]), k01, part[g]);
            part[g] = dot2_bf16(as_bf16x2(qw[g][2 * w + 1]), k23, part[g]);
          }
        } else {
#pragma unroll
          for (int g = 0; g < GW; ++g)
            part[g] = dot2_bf16(as_bf16x2(qw[g][w]), as_bf16x2(kw[w]), part[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float full = group_sum<LPT>(part[g]);
        s[r][g] = valid ? full * qk_scale : kNegInf;
      }
    }

    // ---- online softmax: raise the running max, rescale when it moves ----
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      float mx = s[0][g];
#pragma unroll
      for (int r = 1; r < RPL; ++r) mx = fmaxf(mx, s[r][g]);
      if (mx > m[g]) {
        const float alpha = fast_exp2(m[g] - mx);  // 0 when m was -inf
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[g][e] *= alpha;
        m[g] = mx;
      }
    }

    // ---- P.V in fp32 -------------------------------------------------------
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float vf[EPC];
      const uint32_t vw[4] = {vr[r].x, vr[r].y, vr[r].z, vr[r].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (kFp8) {
          const f32x2 a = e4m3x2_to_f32<false>(vw[w]);
          const f32x2 bb = e4m3x2_to_f32<true>(vw[w]);
          vf[4 * w + 0] = a.x;
          vf[4 * w + 1] = a.y;
          vf[4 * w + 2] = bb.x;
          vf[4 * w + 3] = bb.y;
        } else {
          vf[2 * w + 0] = bf16_lo(vw[w]);
          vf[2 * w + 1] = bf16_hi(vw[w]);
        }
      }
#pragma unroll
      for (int g = 0; g < GW; ++g) {
        const float pr = s[r][g] > kNegInf ? fast_exp2(s[r][g] - m[g]) : 0.f;
        l[g] += pr;
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[g][e] = fmaf(pr, vf[e], o[g][e]);
      }
    }

#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      kr[r] = kn[r];
      vr[r] = vn[r];
    }
  }

  // ---- merge the TPW row slots of the wave (lanes with equal c) -------------
#pragma unroll
  for (int x = LPT; x < 64; x *= 2) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
      const float om = __shfl_xor(m[g], x);
      const float ol = __shfl_xor(l[g], x);
      const float M = fmaxf(m[g], om);
      const float a = m[g] > kNegInf ? fast_exp2(m[g] - M) : 0.f;
      const float bw = om > kNegInf ? fast_exp2(om - M) : 0.f;
      l[g] = a * l[g] + bw * ol;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float oo = __shfl_xor(o[g][e], x);
        o[g][e] = a * o[g][e] + bw * oo;
      }
      m[g] = M;
    }
  }

  // ---- merge the NW waves through LDS and write the split's partial --------
  __shared__ float s_o[NW][GW][D];
  __shared__ float s_m[NW][GW];
  __shared__ float s_l[NW][GW];
  __shared__ int s_last;
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < GW; ++g) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) s_o[wave][g][c * EPC + e] = o[g][e];
      if (c == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  const int S = p.num_splits;
  for (int idx = threadIdx.x; idx < GW * D; idx += 64 * NW) {
    const int g = idx / D;
    const int d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_m[w][g];
      const float f = mw > kNegInf ? fast_exp2(mw - M) : 0.f;
      num += f * s_o[w][g][d];
      den += f * s_l[w][g];
    }
    const size_t row = ((size_t)b * p.num_q_heads + hq0 + g) * S + split;
    p.ws_o[row * D + d] = num;
    if (d == 0) {
      p.ws_m[row] = M;
      p.ws_l[row] = den;
    }
  }

  // ---- the last workgroup of this (sequence, head group) merges the splits -
  // Release the partials device-wide and count arrivals; the workgroup that
  // arrives last acquires them, writes the output and re-arms the counter so
  // the workspace is ready for the next call.  No workgroup ever waits.
  __threadfence();
  __syncthreads();
  int* counter = p.ws_count + (size_t)b * gridDim.y + blockIdx.y;
  if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1) == S - 1);
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  combine_splits<D, GW, NW>(p, b, h, hq0);
  if (threadIdx.x == 0) *counter = 0;
}

static size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

static size_t decode_workspace_counter_bytes(int batch, int num_q_heads) {
  // one arrival counter per (sequence, query head) bounds the number of
  // (sequence, KV head, head group) workgroup sets
  return align16((size_t)batch * num_q_heads * 4);
}

size_t decode_workspace_bytes(int batch, int num_q_heads, int head_dim, int splits) {
  const size_t rows = (size_t)batch * num_q_heads * splits;
  return decode_workspace_counter_bytes(batch, num_q_heads) + align16(rows * head_dim * 4) +
         2 * align16(rows * 4);
}

void decode_workspace_carve(void* ws, int batch, int num_q_heads, int head_dim, int splits,
                            int** count, float** o, float** m, float** l) {
  const size_t rows = (size_t)batch * num_q_heads * splits;
  char* base = reinterpret_cast<char*>(ws);
  *count = reinterpret_cast<int*>(base);
  base += decode_workspace_counter_bytes(batch, num_q_heads);
  *o = reinterpret_cast<float*>(base);
  *m = reinterpret_cast<float*>(base + align16(rows * head_dim * 4));
  *l = reinterpret_cast<float*>(base + align16(rows * head_dim * 4) + align16(rows * 4));
}

template <int D, bool kFp8>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  constexpr int NW = 4;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int GW = G > 8 ? 8 : G;
  dim3 grid(p.num_splits, p.num_kv_heads * (G / GW), p.batch);
  dim3 block(64 * NW);
  switch (GW) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<D, 1, kFp8, NW>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<D, 2, kFp8, NW>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<D, 4, kFp8, NW>), grid, block, 0, stream, p); break;
    case 8: hipLaunchKernelGGL((decode_split_kernel<D, 8, kFp8, NW>), grid, block, 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, bool fp8_cache, hipStream_t stream) {
  switch (p.head_dim) {
    case 64: return fp8_cache ? launch_decode_d<64, true>(p, stream) : launch_decode_d<64, false>(p, stream);
    case 128: return fp8_cache ? launch_decode_d<128, true>(p, stream) : launch_decode_d<128, false>(p, stream);
    case 256: return fp8_cache ? launch_decode_d<256, true>(p, stream) : launch_decode_d<256, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa8
