// Split-KV decode over the paged FP8 / BF16 cache, with the cross-split
// log-sum-exp combine fused into the same launch.
//
// [BLOG] "Performance benchmarks / Single-request benchmark": decode time is
// the per-token KV read, the FP8 cache is read natively and the online
// softmax is rescaled as the kernel goes.  [EXPLAINER] "Memory reduction is
// not speed": dequantisation happens inside the attention kernel, in
// registers, not as a separate pass back to high precision.
//
// Work decomposition: one workgroup of NW waves per (split, KV head [x head
// group], sequence).
//   * The visible pages of a sequence are cut into `num_splits` contiguous
//     ranges; the waves of a workgroup take the pages of its range
//     round-robin.  Each wave reads its block ids once (one lane per page)
//     and keeps two pages in flight in a 3-deep register ring while it
//     processes the third, so the block-table lookup never sits on the
//     load path.
//   * A page-head is 16 rows of D elements: 16*D*elem contiguous bytes for K
//     and again for V.  A lane loads CB-byte chunks (16 bytes; 8 for e4m3
//     with D = 64): LPT = D*elem/CB consecutive lanes cover a row, one
//     wave-wide load covers TPW = 64/LPT consecutive rows, so every load
//     instruction reads one contiguous span.  Each lane ends up with RPL
//     rows of the page (same columns).
//   * q . k: lanes of a row hold the same column range of q for the GW query
//     heads that share the KV head (GQA).  e4m3 codes convert exactly to bf16
//     pairs (one instruction per pair) and feed v_dot2_f32_bf16 with the bf16
//     query (also exact); bf16 cache rows feed it directly.  The LPT partial
//     sums are added across lanes with DPP.
//   * online softmax in the log2 domain; each row slot (LPT lanes) keeps its
//     own running max m, sum l and fp32 output columns, so nothing is
//     exchanged between slots inside the loop.  Full pages take a branch
//     without masking; the pages at the window start / sequence end mask.
//   * p . v: e4m3 -- two rows of the same lane form a token pair; their codes
//     are interleaved with v_perm_b32, converted to f16 pairs (exact) and
//     multiplied with the pair of probabilities rounded to f16 by
//     v_dot2_f32_f16 (fp32 accumulation).  bf16 -- rows convert to fp32 and
//     use fp32 FMAs.
//   * slots merge with shuffles, waves through LDS; each workgroup writes one
//     unnormalised partial (o, m, l) per query head.  The workgroup that
//     finishes last for its (sequence, head group) merges the splits:
//        out = v_scale * sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Scales are folded: k_scale into the score multiplier, v_scale into the
// combine.  Empty splits carry m = -inf and weight 0; an all-empty row is 0.

#include <type_traits>

#include "fa8_device.hpp"
#include "fa8_internal.hpp"

#ifndef FA8_DECODE_F16_PV
#define FA8_DECODE_F16_PV 1    // e4m3 p.v: f16 probability pairs + v_dot2_f32_f16
#endif

namespace fa8 {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxSplits = kDecodeMaxSplits;
// lazy-rescale threshold (log2 units): probabilities stay below 2^8, far
// inside f16 range, and fp32 sums lose nothing
constexpr float kLazy = 8.0f;

template <int N>
struct Chunk {
  uint32_t w[N];
};

template <int N>
__device__ __forceinline__ Chunk<N> load_chunk(const uint8_t* p) {
  Chunk<N> c;
  if constexpr (N == 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    c.w[0] = v.x; c.w[1] = v.y; c.w[2] = v.z; c.w[3] = v.w;
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    c.w[0] = v.x; c.w[1] = v.y;
  }
  return c;
}

// Workspace traffic between workgroups uses agent-scope atomic loads and
// stores: they are coherent across the chip's separate L2 caches without a
// full-cache fence (a __threadfence() writes back / invalidates a whole L2).
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the S split partials of GW query heads (run by the last workgroup):
//   out = v_scale * sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// The maxima, the denominators and the first CH partial rows of every output
// element are requested together, so the merge costs one memory round trip
// whenever S <= CH * R.
template <int D, int GW, int NW>
__device__ __forceinline__ void combine_splits(const DecodeParams& p, int b, int h, int hq0) {
  constexpr int NT = 64 * NW;
  constexpr int COLS = GW * D;                    // output elements
  constexpr int R = NT >= COLS ? NT / COLS : 1;   // threads per output element
  constexpr int CH = 16;                          // partial rows per thread per pass
  __shared__ float s_m[GW][kMaxSplits];
  __shared__ float s_l[GW][kMaxSplits];
  __shared__ float s_mx[GW];
  __shared__ float s_den[GW];
  const int S = p.num_splits;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const size_t base = ((size_t)b * p.num_q_heads + hq0) * S;   // row of (g=0, s=0)
  // this thread's first output element (the loop below covers the rest)
  const int col0 = t / R;
  const int r = t % R;
  float ov[CH];
  if (col0 < COLS) {
    const float* o = p.ws_o + (base + (size_t)(col0 / D) * S) * D + col0 % D;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int sp = r + i * R;
      ov[i] = sp < S ? ld_agent(o + (size_t)sp * D) : 0.f;
    }
  }
  for (int i = t; i < GW * S; i += NT) {
    s_m[i / S][i % S] = ld_agent(p.ws_m + base + i);
    s_l[i / S][i % S] = ld_agent(p.ws_l + base + i);
  }
  __syncthreads();
  // per head: M, weights 2^(m_s - M) (in place of m) and the denominator
  for (int g = wave; g < GW; g += NW) {
    float M = kNegInf;
    for (int sp = lane; sp < S; sp += 64) M = fmaxf(M, s_m[g][sp]);
#pragma unroll
    for (int x = 1; x < 64; x *= 2) M = fmaxf(M, __shfl_xor(M, x));
    float den = 0.f;
    for (int sp = lane; sp < S; sp += 64) {
      const float ms = s_m[g][sp];
      const float f = (M > kNegInf && ms > kNegInf) ? fast_exp2(ms - M) : 0.f;
      s_m[g][sp] = f;
      den += f * s_l[g][sp];
    }
#pragma unroll
    for (int x = 1; x < 64; x *= 2) den += __shfl_xor(den, x);
    if (lane == 0) {
      s_mx[g] = M;
      s_den[g] = den;
    }
  }
  __syncthreads();
  const float vsc = p.fp8 ? p.v_scale[h] : 1.0f;
  for (int col = col0; col < COLS; col += NT / R) {
    const int g = col / D;
    const int d = col % D;
    const float* o = p.ws_o + (base + (size_t)g * S) * D + d;
    float acc = 0.f;
    if (col == col0) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int sp = r + i * R;
        if (sp < S) acc += s_m[g][sp] * ov[i];
      }
    } else {
      for (int sp = r; sp < min(S, CH * R); sp += R) acc += s_m[g][sp] * ld_agent(o + (size_t)sp * D);
    }
    for (int sp = r + CH * R; sp < S; sp += R) acc += s_m[g][sp] * ld_agent(o + (size_t)sp * D);
#pragma unroll
    for (int x = 1; x < R; x *= 2) acc += __shfl_xor(acc, x);
    if (r == 0) {
      const float res = s_mx[g] > kNegInf ? acc * (vsc / s_den[g]) : 0.f;
      p.out[((size_t)b * p.num_q_heads + hq0 + g) * D + d] = res;
    }
  }
}

// Values of the lane `x` lanes away (x = 8: DPP rotate within a 16-lane row;
// 16 / 32: permlane swaps), returned as the pair (value from the lower
// partner, value from the upper partner) so that a symmetric merge needs no
// select.  For x = 8 the pair is (own, partner).
template <int X>
__device__ __forceinline__ void lane_pair(float v, float& a, float& b) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  if constexpr (X == 8) {
    a = v;
    b = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, (int)u, 0x128, 0xF, 0xF, false));
  } else if constexpr (X == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
  } else {
    static_assert(X == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = __builtin_bit_cast(float, (uint32_t)r[0]);
    b = __builtin_bit_cast(float, (uint32_t)r[1]);
  }
}

#ifdef FA8_DECODE_WAVES_PER_EU
#define FA8_DECODE_OCCUPANCY __attribute__((amdgpu_waves_per_eu(FA8_DECODE_WAVES_PER_EU)))
#else
#define FA8_DECODE_OCCUPANCY
#endif

template <int D, int GWW, int HG, bool kFp8, int NW, int PD>
__global__ __launch_bounds__(64 * NW) FA8_DECODE_OCCUPANCY void decode_split_kernel(DecodeParams p) {
  constexpr int ES = kFp8 ? 1 : 2;                     // bytes per element
  constexpr int CB = (kFp8 && D == 64) ? 8 : 16;       // bytes per lane chunk
  constexpr int CW = CB / 4;                           // dwords per chunk
  constexpr int EPC = CB / ES;                         // elements per chunk
  constexpr int LPT = D / EPC;                         // lanes per row
  constexpr int TPW = 64 / LPT;                        // rows per wave-load
  constexpr int RPL = kBlockSize / TPW;                // rows per lane per page
  constexpr int ROW_BYTES = D * ES;
  constexpr int HALF_BYTES = kBlockSize * ROW_BYTES;
  constexpr int GW = GWW * HG;                         // query heads per workgroup
  constexpr int NPW = NW / HG;                         // waves sharing one head group
  static_assert(LPT * TPW == 64 && RPL * TPW == kBlockSize, "tiling");
  static_assert(!kFp8 || RPL % 2 == 0, "e4m3 p.v pairs rows of a lane");
  static_assert(NW % HG == 0 && PD >= 2 && PD <= 8, "launch shape");
  using C = Chunk<CW>;
  constexpr bool kF16PV = FA8_DECODE_F16_PV != 0;

  const int split = blockIdx.x;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int groups = G / GW;
  const int h = blockIdx.y / groups;
  const int hq0 = h * G + (blockIdx.y % groups) * GW;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave % HG;        // which GWW query heads this wave serves
  const int pw = wave / HG;        // which pages of the split it reads
  const int slot = lane / LPT;
  const int c = lane % LPT;

  const int L = p.seq_lens[b];
  const int lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int page_lo = lo / kBlockSize;
  const int page_hi = (L + kBlockSize - 1) / kBlockSize;
  const int pg0 = page_lo + split * p.pages_per_split;
  const int pg1 = min(pg0 + p.pages_per_split, page_hi);

  // q columns c*EPC .. c*EPC+EPC-1 of this wave's query heads, as bf16 pairs
  const int hqw = hq0 + hg * GWW;
  uint32_t qw[GWW][EPC / 2];
#pragma unroll
  for (int g = 0; g < GWW; ++g) {
    const uint4* src = reinterpret_cast<const uint4*>(
        p.q + ((size_t)b * p.num_q_heads + hqw + g) * D + c * EPC);
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

  float m[GWW], l[GWW], o[GWW][EPC];
#pragma unroll
  for (int g = 0; g < GWW; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) o[g][e] = 0.f;
  }

  const uint8_t* head_base = p.cache + (size_t)h * 2 * HALF_BYTES + slot * ROW_BYTES + c * CB;
  const size_t blk_stride = (size_t)p.num_kv_heads * 2 * HALF_BYTES;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;

  struct Page {
    C k[RPL], v[RPL];
  };
  auto issue = [&](Page& pg, int blk) {
    const uint8_t* kb = head_base + (size_t)blk * blk_stride;
#pragma unroll
    for (int r = 0; r < RPL; ++r) pg.k[r] = load_chunk<CW>(kb + r * TPW * ROW_BYTES);
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      pg.v[r] = load_chunk<CW>(kb + HALF_BYTES + r * TPW * ROW_BYTES);
  };

  // One page, straight-line: the pages at the window start and sequence end
  // differ only in the validity mask (a select), so there is a single path.
  auto run_page = [&](const Page& pg, int page) {
    // ---- scores s = (q . k) * sm_scale * k_scale * log2(e) ------------------
    float s[RPL][GWW];
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float part[GWW];
#pragma unroll
      for (int w = 0; w < CW; ++w) {
        if constexpr (kFp8) {
          const bf16x2 k01 = e4m3x2_to_bf16<false>(pg.k[r].w[w]);
          const bf16x2 k23 = e4m3x2_to_bf16<true>(pg.k[r].w[w]);
#pragma unroll
          for (int g = 0; g < GWW; ++g) {
            part[g] = dot2_bf16(as_bf16x2(qw[g][2 * w]), k01, w == 0 ? 0.f : part[g]);
            part[g] = dot2_bf16(as_bf16x2(qw[g][2 * w + 1]), k23, part[g]);
          }
        } else {
#pragma unroll
          for (int g = 0; g < GWW; ++g)
            part[g] = dot2_bf16(as_bf16x2(qw[g][w]), as_bf16x2(pg.k[r].w[w]),
                                w == 0 ? 0.f : part[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GWW; ++g) s[r][g] = group_sum<LPT>(part[g]) * qk_scale;
    }
    // only the pages at the window start / sequence end hold invisible rows
    if (page * kBlockSize < lo || page * kBlockSize + kBlockSize > L) {
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        const int tok = page * kBlockSize + slot + r * TPW;
        const bool valid = tok >= lo && tok < L;
#pragma unroll
        for (int g = 0; g < GWW; ++g) s[r][g] = valid ? s[r][g] : kNegInf;
      }
    }
    // ---- reference maximum ---------------------------------------------------
    // m is the slot's reference point, not necessarily its exact maximum: it
    // moves (and the state is rescaled) only when a score exceeds it by more
    // than kLazy (log2 units), so p = 2^(s - m) stays below 2^kLazy and the
    // rescale is rare.  The result is the same softmax (any reference works).
    float mref[GWW];
#pragma unroll
    for (int g = 0; g < GWW; ++g) {
      float mx = s[0][g];
#pragma unroll
      for (int r = 1; r < RPL; ++r) mx = fmaxf(mx, s[r][g]);
      if (mx > m[g] + kLazy) {
        const float alpha = fast_exp2(m[g] - mx);  // 0 while m is -inf
        l[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[g][e] *= alpha;
        m[g] = mx;
      }
      // while nothing is visible yet (m = -inf) every s is -inf: use 0 as the
      // reference so that exp2(s - ref) = 0 instead of NaN
      mref[g] = m[g] > kNegInf ? m[g] : 0.f;
    }
    // ---- probabilities ---------------------------------------------------------
    float pr[RPL][GWW];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
#pragma unroll
      for (int g = 0; g < GWW; ++g) {
        pr[r][g] = fast_exp2(s[r][g] - mref[g]);
        l[g] += pr[r][g];
      }
    // ---- p . v -------------------------------------------------------------
    if constexpr (kFp8 && kF16PV) {
#pragma unroll
      for (int r = 0; r < RPL; r += 2) {
        f16x2 vp[EPC];
#pragma unroll
        for (int w = 0; w < CW; ++w) {
          // bytes [a0 b0 a1 b1] and [a2 b2 a3 b3] of rows r (a) and r+1 (b)
          const uint32_t lo2 = __builtin_amdgcn_perm(pg.v[r + 1].w[w], pg.v[r].w[w], 0x05010400u);
          const uint32_t hi2 = __builtin_amdgcn_perm(pg.v[r + 1].w[w], pg.v[r].w[w], 0x07030602u);
          vp[4 * w + 0] = e4m3x2_to_f16<false>(lo2);
          vp[4 * w + 1] = e4m3x2_to_f16<true>(lo2);
          vp[4 * w + 2] = e4m3x2_to_f16<false>(hi2);
          vp[4 * w + 3] = e4m3x2_to_f16<true>(hi2);
        }
#pragma unroll
        for (int g = 0; g < GWW; ++g) {
          const f16x2 pp = {(_Float16)pr[r][g], (_Float16)pr[r + 1][g]};
#pragma unroll
          for (int e = 0; e < EPC; ++e) o[g][e] = dot2_f16(vp[e], pp, o[g][e]);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        float vf[EPC];
#pragma unroll
        for (int w = 0; w < CW; ++w) {
          if constexpr (kFp8) {
            const f32x2 x01 = e4m3x2_to_f32<false>(pg.v[r].w[w]);
            const f32x2 x23 = e4m3x2_to_f32<true>(pg.v[r].w[w]);
            vf[4 * w + 0] = x01.x;
            vf[4 * w + 1] = x01.y;
            vf[4 * w + 2] = x23.x;
            vf[4 * w + 3] = x23.y;
          } else {
            vf[2 * w + 0] = bf16_lo(pg.v[r].w[w]);
            vf[2 * w + 1] = bf16_hi(pg.v[r].w[w]);
          }
        }
#pragma unroll
        for (int g = 0; g < GWW; ++g)
#pragma unroll
          for (int e = 0; e < EPC; ++e) o[g][e] = fmaf(pr[r][g], vf[e], o[g][e]);
      }
    }
  };

  // This wave's pages: pg0 + pw + NPW*j.  Block ids are fetched 64 at a
  // time, one per lane, and broadcast with readlane; PD-1 pages are in
  // flight while one is processed.
  const int first = pg0 + pw;
  const int npw = first < pg1 ? (pg1 - first + NPW - 1) / NPW : 0;
  for (int jb = 0; jb < npw; jb += 64) {
    const int n = min(64, npw - jb);
    const int page_base = first + NPW * jb;
    const int my_blk = lane < n ? bt[page_base + NPW * lane] : 0;
    // Steady PD-deep ring: PD-1 pages are in flight while one is processed.
    // Every buffer is consumed and re-issued in every round, and prefetches
    // past the end repeat the last page (an L2 hit), so every path keeps the
    // same loads in flight and the compiler waits for exactly the page it is
    // about to use.
    auto blk_of = [&](int j) { return __builtin_amdgcn_readlane(my_blk, min(j, n - 1)); };
    Page ring[PD];
#pragma unroll
    for (int k = 0; k < PD; ++k) issue(ring[k], blk_of(k));
    int j = 0;
    for (; j + PD <= n; j += PD) {
#pragma unroll
      for (int k = 0; k < PD; ++k) {
        run_page(ring[k], page_base + NPW * (j + k));
        __builtin_amdgcn_sched_barrier(0);   // keep the reissue after the use
        issue(ring[k], blk_of(j + k + PD));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int k = 0; k < PD - 1; ++k)
      if (j + k < n) run_page(ring[k], page_base + NPW * (j + k));
  }

  // ---- merge the TPW row slots of the wave (lanes with equal c) -------------
  // Slots sit LPT, 2*LPT, ... lanes apart; each step merges a lane's state
  // with its partner's (a symmetric merge, so both partners end up equal).
  auto merge_step = [&](auto xtag) {
    constexpr int X = decltype(xtag)::value;
#pragma unroll
    for (int g = 0; g < GWW; ++g) {
      float ma, mb, la, lb;
      lane_pair<X>(m[g], ma, mb);
      lane_pair<X>(l[g], la, lb);
      const float M = fmaxf(ma, mb);
      const float fa = ma > kNegInf ? fast_exp2(ma - M) : 0.f;
      const float fb = mb > kNegInf ? fast_exp2(mb - M) : 0.f;
      l[g] = fa * la + fb * lb;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float oa, ob;
        lane_pair<X>(o[g][e], oa, ob);
        o[g][e] = fa * oa + fb * ob;
      }
      m[g] = M;
    }
  };
  if constexpr (LPT <= 8) merge_step(std::integral_constant<int, 8>{});
  if constexpr (LPT <= 16) merge_step(std::integral_constant<int, 16>{});
  if constexpr (LPT <= 32) merge_step(std::integral_constant<int, 32>{});

  // ---- merge the waves of each head group through LDS (one round) ----------
  __shared__ float s_o[NW][GWW][D];
  __shared__ float s_m[NW][GWW];
  __shared__ float s_l[NW][GWW];
  __shared__ int s_last;
  const int S = p.num_splits;
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < GWW; ++g) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) s_o[wave][g][c * EPC + e] = o[g][e];
      if (c == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  // element t: head group hgi, local head g, column d; all stores are issued
  // back to back and waited for once below
  for (int t = threadIdx.x; t < HG * GWW * D; t += 64 * NW) {
    const int hgi = t / (GWW * D);
    const int g = (t / D) % GWW;
    const int d = t % D;
    float M = kNegInf;
#pragma unroll
    for (int w = hgi; w < NW; w += HG) M = fmaxf(M, s_m[w][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = hgi; w < NW; w += HG) {
      const float f = s_m[w][g] > kNegInf ? fast_exp2(s_m[w][g] - M) : 0.f;
      num += f * s_o[w][g][d];
      den += f * s_l[w][g];
    }
    const size_t row = ((size_t)b * p.num_q_heads + hq0 + hgi * GWW + g) * S + split;
    st_agent(p.ws_o + row * D + d, num);
    if (d == 0) {
      st_agent(p.ws_m + row, M);
      st_agent(p.ws_l + row, den);
    }
  }

  // ---- the last workgroup of this (sequence, head group) merges the splits -
  // Each thread waits until its partial stores are performed (they are
  // coherent agent-scope stores), the workgroup then counts its arrival; the
  // one that arrives last reads the partials with coherent loads, writes the
  // output and re-arms the counter for the next call.  No workgroup waits.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int* counter = p.ws_count + (size_t)b * gridDim.y + blockIdx.y;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
  __syncthreads();
  if (!s_last) return;
  combine_splits<D, GW, NW>(p, b, h, hq0);
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

#ifndef FA8_DECODE_PIPE
#define FA8_DECODE_PIPE 2      // e4m3 cache: pages held per wave (in flight + processed)
#endif
#ifndef FA8_DECODE_PIPE_BF16
#define FA8_DECODE_PIPE_BF16 2 // bf16 cache (pages are twice as large)
#endif
#ifndef FA8_DECODE_MAX_GWW
#define FA8_DECODE_MAX_GWW 4   // query heads per wave for head_dim 64 / 128
#endif

// Launch shape per (D, cache type): query heads per wave (GWW), waves per
// workgroup (NW).  Heads of one KV head beyond GWW go to other waves of the
// same workgroup (head groups), which read the same pages (L2 hits).
template <int D, bool kFp8, int GWW, int HG>
static void launch_shape(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  constexpr int NW = kDecodeWaves;
  constexpr int PD = kFp8 ? FA8_DECODE_PIPE : FA8_DECODE_PIPE_BF16;
  hipLaunchKernelGGL((decode_split_kernel<D, GWW, HG, kFp8, NW, PD>), grid,
                     dim3(64 * NW), 0, stream, p);
}

template <int D, bool kFp8>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  // at most 4 query heads per wave (2 for head_dim 256) keeps registers
  // below the spill point; at most 8 heads per workgroup
  constexpr int kMaxGWW = D == 256 ? 2 : FA8_DECODE_MAX_GWW;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int GW = G > 8 ? 8 : G;
  dim3 grid(p.num_splits, p.num_kv_heads * (G / GW), p.batch);
  switch (GW) {
    case 1: launch_shape<D, kFp8, 1, 1>(p, grid, stream); break;
    case 2: launch_shape<D, kFp8, 2, 1>(p, grid, stream); break;
    case 4: launch_shape<D, kFp8, (4 > kMaxGWW ? kMaxGWW : 4), (4 > kMaxGWW ? 4 / kMaxGWW : 1)>(p, grid, stream); break;
    case 8: launch_shape<D, kFp8, kMaxGWW, 8 / kMaxGWW>(p, grid, stream); break;
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
