// Split-KV decode over the paged FP8 (e4m3 or e5m2) / BF16 cache, with the
// cross-split log-sum-exp merge fused into the same launch.
//
// [BLOG] "性能 Benchmark / 单请求 Benchmark" (single-request benchmark):
// decode time is the per-token read of the cache, which the FP8 cache halves;
// the kernel keeps an online-softmax state that it rescales as it goes.
// [EXPLAINER] "FP8は値とscaleを組み合わせる": a stored value is a code and a
// scale; the codes are widened in registers, the scales are folded into the
// score multiplier (k_scale) and the final merge (v_scale).
//
// Work decomposition: one workgroup of NW waves per (split, KV head,
// sequence).  The visible pages of a sequence are cut into `num_splits`
// contiguous ranges; the waves of a workgroup take the pages of their range
// round-robin, one page (16 keys) at a time, keeping PD pages in flight in a
// register ring.  The G query heads that share the KV head are handled
// together: per page the work is a (16 keys x D) by (D x G) product and its
// (G x 16) by (16 x D) counterpart, done on the matrix cores:
//
//   * loads: lane (r, g) (r = lane % 16, g = lane / 16) reads 16-byte pieces
//     of key row r at byte offsets 64*hh + 16*g, so each load instruction
//     covers the first / next 64 bytes of all 16 rows of the page;
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: K codes are widened to bf16
//     (exact), the bf16 query is the other operand (exact; columns >= G are
//     zero).  The head dim is split into 32-wide chunks whose 8 elements per
//     lane group are the ones lane group g loaded; the query chunks follow
//     the same assignment.  The result leaves lane (n, g) with the scores of
//     keys 4g..4g+3 for query head n;
//   * softmax in the log2 domain: page maximum per head across the 4 lane
//     groups (permlane swaps), lazily moved reference maximum, p = 2^(s - m);
//   * P . V on v_mfma_f32_16x16x16 (f16 for the FP8 caches: p split into an
//     f16 high and low part, V widened to f16 exactly; bf16 for the bf16
//     cache with p split into a bf16 high and low part; two products each):
//     lane (n, g) already holds P for
//     head n and keys 4g..4g+3, the A operand.  V is written to a small
//     per-wave LDS slice and read back transposed (ds_read_b64_tr_b8 / _b16)
//     as the B operand (keys 4g..4g+3 of one column per lane).  The output
//     tile leaves lane (n, g) with O[head 4g+i][16c + n].
// The waves' states merge through LDS; each workgroup writes one
// unnormalised partial (o, m, l) per query head, and the workgroup that
// arrives last for its (sequence, KV head) merges the splits (with many
// splits, the last arrivals share the merge, one slice of columns each):
//   out = v_scale * sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// Empty splits carry m = -inf and weight 0; an all-empty row is 0.

#include "fa8_device.hpp"
#include "fa8_internal.hpp"

namespace fa8 {

constexpr float kNegInf = -__builtin_huge_valf();
// lazy-rescale threshold (log2 units): probabilities stay below 2^8, far
// inside f16 range, and fp32 sums lose nothing
constexpr float kLazy = 8.0f;

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2* lds_i32x2_ptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// Workspace traffic between workgroups uses agent-scope atomic loads and
// stores: they are coherent across the chip's separate L2 caches without a
// full-cache fence (a __threadfence() writes back / invalidates a whole L2).
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reductions over the 64 lanes of a wave: DPP within each row of 16 lanes
// (pairs, quads, half-rows, rows), then permlane swaps across the rows.
__device__ __forceinline__ float cross_rows_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                       __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float cross_rows_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                       __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
  v = fmaxf(v, dpp<0x140>(v));   // row_mirror
  return cross_rows_max(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  return cross_rows_sum(group_sum<16>(v));
}

// Workspace accesses of 4, 8 or 16 bytes with the cache policy the compiler
// gives agent-scope atomic loads and stores (sc1): coherent across the L2
// caches like ld_agent / st_agent, but up to four floats per memory request.
// A merger's partials stream through one CU, whose request rate can bound it.
constexpr int kScopeAgent = 16;                 // cache-policy bits: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, (int)bytes, 0x00020000);
}
// V consecutive floats (V = 1, 2 or 4) in the low lanes of an f32x4
template <int V>
__device__ __forceinline__ f32x4 ld_agentv(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  if constexpr (V == 4) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kScopeAgent));
  } else if constexpr (V == 2) {
    const f32x2 x = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, kScopeAgent));
    return f32x4{x[0], x[1], 0.f, 0.f};
  } else {
    return f32x4{__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, kScopeAgent)),
                 0.f, 0.f, 0.f};
  }
}
template <int V>
__device__ __forceinline__ void st_agentv(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, f32x4 v) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (V == 4) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kScopeAgent);
  } else if constexpr (V == 2) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{v[0], v[1]}), r, byte_off, 0,
                                          kScopeAgent);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v[0]), r, byte_off, 0, kScopeAgent);
  }
}
// Floats per workspace access: the widest that still gives every thread of
// a workgroup of nt threads its own group of columns (cols outputs), so that
// the merges keep all threads busy and issue the fewest requests.
constexpr int ws_vec(int cols, int nt) { return cols >= 4 * nt ? 4 : cols >= 2 * nt ? 2 : 1; }

// Merge the n (<= kDecodeSingleLevel) unnormalised partials (o, m, l) of
// each of GW query heads into the output, run by one workgroup.  Head g's
// partial rows are rows 0 .. n-1 of a block of n rows starting at (head g) * n:
//   M = max_i m_i,  w_i = 2^(m_i - M),
//   out[g][d] = v_scale * sum_i w_i o_i[d] / sum_i w_i l_i  (0 when every
//   partial is empty).
// Each thread owns V consecutive columns (one load of V floats per partial
// row); R adjacent lanes share them and take every R-th row.  All partial
// loads of a batch are issued before any is used, and the first batch is in
// flight while the maxima are reduced.
template <int D, int GW, int NW>
__device__ __forceinline__ void merge_rows(const float* o_in, const float* m_in,
                                           const float* l_in, int n, float* o_dst, float vsc) {
  constexpr int NT = 64 * NW;
  constexpr int V = ws_vec(GW * D, NT);               // columns per load
  constexpr int CG = GW * D / V;                      // V-column groups of the output
  constexpr int R = NT >= CG ? NT / CG : 1;           // threads per group
  constexpr int EPT = CG > NT ? CG / NT : 1;          // groups per thread
  // partial rows per thread per batch: 32 four-byte or 16 wider loads in
  // flight for one group, 8 rows for several
  constexpr int JB = EPT > 1 ? 8 : V == 1 ? 32 : 16;
  constexpr int kMaxRows = kDecodeSingleLevel;
  static_assert(R * CG == NT || EPT * NT == CG, "merge tiling");
  static_assert(R <= 64, "a group's threads are lanes of one wave");
  __shared__ float s_w[GW][kMaxRows];
  __shared__ float s_l[GW][kMaxRows];
  __shared__ float s_mx[GW];
  __shared__ float s_den[GW];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int col0 = t / R;
  const int r = t % R;
  const __amdgpu_buffer_rsrc_t src = ws_rsrc(o_in, (uint32_t)(GW * n * D * 4));

  f32x4 v[EPT][JB];
  auto issue = [&](int j0) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int col = col0 + e * (NT / R);
      const uint32_t base = (uint32_t)((col / (D / V)) * n) * D + (col % (D / V)) * V;
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int i = min(j0 + r + j * R, n - 1);   // rows past n repeat row n-1, weight 0
        v[e][j] = ld_agentv<V>(src, (base + (uint32_t)i * D) * 4);
      }
    }
  };
  // the (head, row) maxima and denominators (at most MLT per thread) are
  // requested before the first batch of partial rows, so that only they are
  // waited for here
  constexpr int MLT = (GW * kMaxRows + NT - 1) / NT;
  float mv[MLT], lv[MLT];
#pragma unroll
  for (int k = 0; k < MLT; ++k) {
    const int i = t + k * NT;
    mv[k] = kNegInf;
    lv[k] = 0.f;
    if (i < GW * n) {
      mv[k] = ld_agent(m_in + i);   // head i / n, row i % n
      lv[k] = ld_agent(l_in + i);
    }
  }
  issue(0);
#pragma unroll
  for (int k = 0; k < MLT; ++k) {
    const int i = t + k * NT;
    if (i < GW * n) {
      s_w[i / n][i % n] = mv[k];
      s_l[i / n][i % n] = lv[k];
    }
  }
  __syncthreads();
  // one wave per head: M, weights 2^(m_i - M) (in place of m) and the
  // denominator, with in-register wave reductions
  for (int g = wave; g < GW; g += NW) {
    const float mk = lane < n ? s_w[g][lane] : kNegInf;
    const float M = wave_max(mk);
    const float f = (M > kNegInf && mk > kNegInf) ? fast_exp2(mk - M) : 0.f;
    const float den = wave_sum(lane < n ? f * s_l[g][lane] : 0.f);
    if (lane < n) s_w[g][lane] = f;
    if (lane == 0) {
      s_mx[g] = M;
      s_den[g] = den;
    }
  }
  __syncthreads();
  f32x4 acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < n; j0 += JB * R) {
    if (j0 > 0) issue(j0);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const int g = (col0 + e * (NT / R)) / (D / V);
#pragma unroll
      for (int j = 0; j < JB; ++j) {
        const int i = j0 + r + j * R;
        if (i < n) {
          const float w = s_w[g][i];
#pragma unroll
          for (int c = 0; c < V; ++c) acc[e][c] += w * v[e][j][c];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    f32x4 a = acc[e];
#pragma unroll
    for (int c = 0; c < V; ++c) a[c] = group_sum<R>(a[c]);   // the R threads are adjacent lanes
    const int col = col0 + e * (NT / R);
    const int g = col / (D / V);
    const int d = (col % (D / V)) * V;
    if (r == 0) {
      const float f = vsc / s_den[g];
#pragma unroll
      for (int c = 0; c < V; ++c) o_dst[(size_t)g * D + d + c] = s_mx[g] > kNegInf ? a[c] * f : 0.f;
    }
  }
}


// Polls of the set counter by a slice merger waiting for the last split
// group (each poll is an agent-scope load plus a short sleep; the bound is
// far beyond any real wait, so that the kernel ends even if a split never
// came).
constexpr int kMergeWaitPolls = 1 << 20;

// Output columns per slice merger (a power of two from 16 to 256; capped at
// head_dim).  Measured on MI355X, single-KV-head head_dim-256 layer with 8
// query heads and 256 splits, 128k / 32k context: 16 columns 23.64 / 15.85
// us, 32: 22.60 / 14.66, 64: 22.08 / 14.05, 128: 21.77 / 13.80 (16
// mergers, one per split group), 256: 23.50 / 15.68.
constexpr int kSliceCols = 128;

// Merge all n (<= kDecodeMaxSplits) partial rows of one query head over the
// SW output columns c0 .. c0+SW-1, run by one workgroup of NW waves:
//   M = max_i m_i,  w_i = 2^(m_i - M),
//   out[c] = v_scale * sum_i w_i o_i[c] / sum_i w_i l_i  (0 when every
//   partial is empty).
// The head's partial rows are rows 0 .. n-1 of o_head ([n][D]).  Lane l of a
// wave owns the four columns 4 (l % CG) .. +3 (CG = SW / 4) of one
// row, the wave's lanes covering 64 / CG consecutive rows, so that one load
// instruction covers whole row slices (the loads bypass the caches: rows
// scattered over the lanes would fetch each line several times).  The
// maxima and denominators are loaded first and all partial loads are issued
// before the weights are waited for; the row sums meet through lane shuffles
// and an LDS array.
template <int D, int NW, int SW>
__device__ __forceinline__ void merge_slice(const float* o_head, const float* m_head,
                                            const float* l_head, int n, int c0,
                                            float* out_head, float vsc) {
  constexpr int NT = 64 * NW;
  constexpr int CG = SW / 4;                          // four-column groups of the slice
  constexpr int RW = 64 / CG;                         // rows per wave per pass
  constexpr int RP = RW * NW;                         // rows per pass of all waves
  constexpr int JR = (kDecodeMaxSplits + RP - 1) / RP; // passes (rows per lane) at most
  constexpr int MK = kDecodeMaxSplits / 64;           // rows per lane of the weight wave
  static_assert(CG >= 4 && CG <= 64 && (CG & (CG - 1)) == 0, "slice width");
  __shared__ float s_w[kDecodeMaxSplits];
  __shared__ float s_lw[kDecodeMaxSplits];
  __shared__ f32x4 s_part[NW][CG];
  __shared__ float s_mx, s_den;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int cg = lane % CG;                           // four-column group
  const int rp = RW * wave + lane / CG;               // first row of the lane
  const __amdgpu_buffer_rsrc_t src = ws_rsrc(o_head, (uint32_t)(n * D * 4));
  // the maxima and denominators are requested first, so that only they are
  // waited for before the weights; the partial rows stream in meanwhile
  constexpr int ML = (kDecodeMaxSplits + NT - 1) / NT;
  float mv[ML], lv[ML];
#pragma unroll
  for (int k = 0; k < ML; ++k) {
    const int i = t + k * NT;
    if (i < n) {
      mv[k] = ld_agent(m_head + i);
      lv[k] = ld_agent(l_head + i);
    }
  }
  // rows past n-1 lie beyond the buffer resource's range (n rows): those
  // loads return zeros without a memory access, and no branch splits the
  // batch, so the wait below covers only the maxima and denominators
  f32x4 v[JR];
#pragma unroll
  for (int j = 0; j < JR; ++j)
    v[j] = ld_agentv<4>(src, (uint32_t)((rp + j * RP) * D + c0 + 4 * cg) * 4);
#pragma unroll
  for (int k = 0; k < ML; ++k) {
    const int i = t + k * NT;
    if (i < n) {
      s_w[i] = mv[k];
      s_lw[i] = lv[k];
    }
  }
  __syncthreads();
  if (t < 64) {   // one wave: the maximum, the weights and the denominator
    float mk[MK];
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < MK; ++k) {
      const int i = t + 64 * k;
      mk[k] = i < n ? s_w[i] : kNegInf;
      M = fmaxf(M, mk[k]);
    }
    M = wave_max(M);
    float den = 0.f;
#pragma unroll
    for (int k = 0; k < MK; ++k) {
      const int i = t + 64 * k;
      const float f = (M > kNegInf && mk[k] > kNegInf) ? fast_exp2(mk[k] - M) : 0.f;
      if (i < n) {
        s_w[i] = f;
        den += f * s_lw[i];
      }
    }
    den = wave_sum(den);
    if (t == 0) {
      s_mx = M;
      s_den = den;
    }
  }
  __syncthreads();
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < JR; ++j) {
    const int i = rp + j * RP;
    if (i < n) {
      const float w = s_w[i];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += w * v[j][c];
    }
  }
  // the RW lanes of this column group in the wave (l ^ CG, l ^ 2CG, ...)
#pragma unroll
  for (int x = CG; x < 64; x *= 2)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], x);
  if (lane < CG) s_part[wave][lane] = acc;
  __syncthreads();
  if (t < CG) {
    f32x4 a = s_part[0][t];
#pragma unroll
    for (int w = 1; w < NW; ++w)
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] += s_part[w][t][c];
    const float f = vsc / s_den;
#pragma unroll
    for (int c = 0; c < 4; ++c) out_head[c0 + 4 * t + c] = s_mx > kNegInf ? a[c] * f : 0.f;
  }
}

// 8 FP8 codes (two dwords) -> 8 bf16 (exact for e4m3 and e5m2)
template <int kFmt>
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = fp8x2_to_bf16<kFmt, false>(w0), b = fp8x2_to_bf16<kFmt, true>(w0);
  const bf16x2 c = fp8x2_to_bf16<kFmt, false>(w1), d = fp8x2_to_bf16<kFmt, true>(w1);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 w) { return __builtin_bit_cast(bf16x8, w); }

// Waves per SIMD the register budget is sized for, without spills: four at
// head_dim 64, three at 128 (two with 16 query heads per KV head, whose
// merge state needs more), two at 256.
template <int D, int G>
constexpr int decode_min_waves() {
  return D == 64 ? 4 : D == 128 ? (G == 16 ? 2 : 3) : 2;
}

template <int D, int G, int kFmt, int NW, int PD>
__global__ __launch_bounds__(64 * NW, (decode_min_waves<D, G>())) void decode_split_kernel(DecodeParams p) {
  constexpr bool kFp8 = kFmt != kFmtBf16;
  constexpr int ES = kFp8 ? 1 : 2;       // bytes per element
  constexpr int ROW = D * ES;            // bytes per cached row
  constexpr int HALF = kBlockSize * ROW; // K (or V) bytes of one page-head
  constexpr int NL = ROW / 64;           // 16-byte loads per lane per page-half
  constexpr int NQ = D / 32;             // 32-wide head-dim chunks (QK MFMAs per page)
  constexpr int NB = D / 16;             // 16-wide output column blocks
  constexpr int BPS = kFp8 ? 4 : 2;      // column blocks per 64-byte slice
  constexpr int RS = 64 + 16;            // LDS row stride of the V slice (bytes)
  static_assert(NL >= 1 && NB == NL * BPS, "tiling");
  static_assert(G >= 1 && G <= 16, "query heads per KV head");

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hq0 = h * G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;     // key row (loads, K operand) / head (Q, S, P) / column (V, O)
  const int g = lane >> 4;     // k-group of the MFMA operands

  // Without a window a split's page range starts at split * pages_per_split
  // whatever the sequence length, so the block ids of this wave's first 64
  // pages are requested together with the length instead of after it (one
  // dependent round trip less before the first page).  Entries past the
  // sequence end (inside the row) are read but never used.
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
  const bool early_ids = p.window <= 0 && p.max_blocks > 0;
  int early_blk = 0;
  if (early_ids)
    early_blk = bt[min(split * p.pages_per_split + wave + NW * lane, p.max_blocks - 1)];
  const int L = p.seq_lens[b];
  const int lo = p.window > 0 ? max(0, L - p.window) : 0;
  const int page_lo = lo / kBlockSize;
  const int page_hi = (L + kBlockSize - 1) / kBlockSize;
  const int pg0 = page_lo + split * p.pages_per_split;
  const int pg1 = min(pg0 + p.pages_per_split, page_hi);

  // ---- query operand: chunk q holds, for lane group g, head-dim elements
  //      FP8 cache: 64*(q/2) + 16*g + 8*(q%2) + i;  bf16 cache: 32*q + 8*g + i
  bf16x8 qop[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int d0 = kFp8 ? 64 * (q / 2) + 16 * g + 8 * (q % 2) : 32 * q + 8 * g;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < G) w = *reinterpret_cast<const uint4*>(p.q + ((size_t)b * p.num_q_heads + hq0 + n) * D + d0);
    qop[q] = as_bf16x8(w);
  }
  const float qk = p.sm_scale * kLog2e * (kFp8 ? p.k_scale[h] : 1.0f);

  float m = kNegInf;   // reference maximum of head n (equal in the 4 lane groups)
  float l = 0.f;       // sum of p over this lane's keys, head n
  f32x4 o[NB];         // O[head 4g+i][16c + n]
#pragma unroll
  for (int c = 0; c < NB; ++c) o[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // two LDS regions: the per-wave V slices of the page loop, and the wave
  // merge, which a wave fills as soon as its own loop ends (no barrier
  // between the last page of one wave and another wave's merge writes)
  constexpr int kSliceBytes = kBlockSize * RS;
  // query heads merged per LDS round: all of them within a 64 KB budget
  constexpr int kMergeHeads = (65536 / (NW * D * 4)) < G ? (65536 / (NW * D * 4)) : G;
  constexpr int kMergeBytes = NW * kMergeHeads * D * 4 + 2 * NW * 16 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t s_vsl[NW * kSliceBytes];
  __shared__ __attribute__((aligned(16))) uint8_t s_mrg[kMergeBytes];
  uint8_t* sv = s_vsl + wave * kSliceBytes;

  const uint8_t* head_base = p.cache + (size_t)h * 2 * HALF + n * ROW + 16 * g;
  const size_t blk_stride = (size_t)p.num_kv_heads * 2 * HALF;

  struct Page {
    uint4 k[NL], v[NL];
  };
  auto issue = [&](Page& pg, int blk) {
    const uint8_t* kb = head_base + (size_t)blk * blk_stride;
#pragma unroll
    for (int hh = 0; hh < NL; ++hh) pg.k[hh] = *reinterpret_cast<const uint4*>(kb + 64 * hh);
#pragma unroll
    for (int hh = 0; hh < NL; ++hh) pg.v[hh] = *reinterpret_cast<const uint4*>(kb + HALF + 64 * hh);
  };

  // Fused append: the wave that will read the page holding token L-1 encodes
  // that token's K and V row from the inputs (the same rounding as
  // cache_write), stores it into the cache and into an LDS slot of its own,
  // and swaps it in for the row the page load returns.  Every lane of that
  // wave takes AE = D/32 consecutive elements of the K row (lanes 0-31) or
  // the V row (lanes 32-63).  The inputs are loaded here; they are encoded
  // only after the wave's first page loads are issued, so the owner wave
  // starts streaming as early as the others.
  const bool append = p.k_new != nullptr && L > 0;
  const int new_page = (L - 1) / kBlockSize;
  const int new_row = (L - 1) % kBlockSize;
  __shared__ __attribute__((aligned(16))) uint8_t s_new[2 * ROW];
  const bool owner = append && new_page >= pg0 && new_page < pg1 && (new_page - pg0) % NW == wave;
  constexpr int AE = D / 32;
  const int a_kv = lane >> 5;             // 0: K row, 1: V row
  const int a_e0 = (lane & 31) * AE;      // first element of this lane's piece
  float a_x[AE];
  int a_blk = 0;
  if (owner) {
    a_blk = bt[new_page];
    const size_t e = ((size_t)b * p.num_kv_heads + h) * D + a_e0;
    const void* src = a_kv ? p.v_new : p.k_new;
    if (p.new_bf16) {
      const uint16_t* s16 = reinterpret_cast<const uint16_t*>(src) + e;
      uint32_t w[AE / 2];
      if constexpr (AE == 2) {
        w[0] = *reinterpret_cast<const uint32_t*>(s16);
      } else if constexpr (AE == 4) {
        const uint2 t = *reinterpret_cast<const uint2*>(s16);
        w[0] = t.x; w[1] = t.y;
      } else {
        const uint4 t = *reinterpret_cast<const uint4*>(s16);
        w[0] = t.x; w[1] = t.y; w[2] = t.z; w[3] = t.w;
      }
#pragma unroll
      for (int i = 0; i < AE / 2; ++i) {
        a_x[2 * i] = bf16_lo(w[i]);
        a_x[2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
      const float* s32 = reinterpret_cast<const float*>(src) + e;
#pragma unroll
      for (int i = 0; i < AE; i += 2) {
        const float2 t = *reinterpret_cast<const float2*>(s32 + i);
        a_x[i] = t.x;
        a_x[i + 1] = t.y;
      }
    }
  }
  // encode this lane's piece, store it to the cache row and to the LDS slot
  auto append_row = [&]() {
    constexpr int PB = AE * ES;           // bytes of the piece: 2 .. 16
    const float sc = kFp8 ? (a_kv ? p.v_scale[h] : p.k_scale[h]) : 1.0f;
    uint32_t w[PB >= 4 ? PB / 4 : 1] = {};
#pragma unroll
    for (int i = 0; i < AE; ++i) {
      if constexpr (kFp8) {
        w[i / 4] |= fp8_encode<kFmt>(a_x[i] / sc) << (8 * (i % 4));
      } else {
        w[i / 2] |= bf16_bits(a_x[i]) << (16 * (i % 2));
      }
    }
    uint8_t* dst = const_cast<uint8_t*>(p.cache) + (size_t)a_blk * blk_stride +
                   (size_t)h * 2 * HALF + a_kv * HALF + new_row * ROW + a_e0 * ES;
    uint8_t* lds = s_new + a_kv * ROW + a_e0 * ES;
    if constexpr (PB == 2) {
      *reinterpret_cast<uint16_t*>(dst) = (uint16_t)w[0];
      *reinterpret_cast<uint16_t*>(lds) = (uint16_t)w[0];
    } else if constexpr (PB == 4) {
      *reinterpret_cast<uint32_t*>(dst) = w[0];
      *reinterpret_cast<uint32_t*>(lds) = w[0];
    } else if constexpr (PB == 8) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
      *reinterpret_cast<uint2*>(lds) = make_uint2(w[0], w[1]);
    } else {
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
      *reinterpret_cast<uint4*>(lds) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  auto patch_new_row = [&](Page& pg) {
    if (n != new_row) return;
#pragma unroll
    for (int hh = 0; hh < NL; ++hh) {
      pg.k[hh] = *reinterpret_cast<const uint4*>(s_new + 64 * hh + 16 * g);
      pg.v[hh] = *reinterpret_cast<const uint4*>(s_new + ROW + 64 * hh + 16 * g);
    }
  };

  auto run_page = [&](const Page& pg_in, int page) {
    Page pg = pg_in;
    if (owner && page == new_page) patch_new_row(pg);
    // ---- S^T = K . Q^T ------------------------------------------------------
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      bf16x8 a;
      if constexpr (kFp8) {
        const uint4 w = pg.k[q / 2];
        a = (q % 2 == 0) ? fp8x8_to_bf16<kFmt>(w.x, w.y) : fp8x8_to_bf16<kFmt>(w.z, w.w);
      } else {
        a = as_bf16x8(pg.k[q]);
      }
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qop[q], s, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] *= qk;
    // only the pages at the window start / sequence end hold invisible keys
    // (their V rows are zeroed as operands too: the rows past the sequence end
    // hold whatever the page held before, and 0 * NaN would be NaN)
    uint32_t vmask_lo = ~0u, vmask_hi = ~0u;   // byte (FP8) or half-word (bf16) masks
    if (page * kBlockSize < lo || page * kBlockSize + kBlockSize > L) {
      uint32_t bits = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = page * kBlockSize + 4 * g + i;
        const bool valid = key >= lo && key < L;
        s[i] = valid ? s[i] : kNegInf;
        bits |= valid ? 1u << i : 0u;
      }
      if constexpr (kFp8) {
        vmask_lo = (bits & 1 ? 0xFFu : 0u) | (bits & 2 ? 0xFF00u : 0u) |
                   (bits & 4 ? 0xFF0000u : 0u) | (bits & 8 ? 0xFF000000u : 0u);
      } else {
        vmask_lo = (bits & 1 ? 0xFFFFu : 0u) | (bits & 2 ? 0xFFFF0000u : 0u);
        vmask_hi = (bits & 4 ? 0xFFFFu : 0u) | (bits & 8 ? 0xFFFF0000u : 0u);
      }
    }
    // ---- reference maximum -------------------------------------------------
    // m moves (and the state is rescaled) only when a score exceeds it by more
    // than kLazy, so p = 2^(s - m) < 2^kLazy and rescales are rare; any
    // reference gives the same softmax.
    const float mx = cross_rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
    const bool up = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float m_new = up ? mx : m;
      const float alpha = m_new == m ? 1.0f : fast_exp2(m - m_new);   // 0 while m = -inf
      l *= alpha;
      // output rows are heads 4g+i: their factors live in lanes 4g+i
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i);
#pragma unroll
      for (int c = 0; c < NB; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[c][i] *= ar[i];
      m = m_new;
    }
    // while nothing is visible yet (m = -inf) every s is -inf: reference 0
    const float mref = m > kNegInf ? m : 0.f;
    float pr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = fast_exp2(s[i] - mref);
      l += pr[i];
    }
    // ---- P . V ---------------------------------------------------------------
    // V slice hh: bytes [64 hh, 64 hh + 64) of the 16 rows, row-major in LDS
    if constexpr (kFp8) {
      // p = hi + lo, both f16 (together 22 significant bits; V is exact in
      // f16, so each product pair carries p to about 2^-22)
      const f16x4 pa = {(_Float16)pr[0], (_Float16)pr[1], (_Float16)pr[2], (_Float16)pr[3]};
      const f16x4 pl = {(_Float16)(pr[0] - (float)pa[0]), (_Float16)(pr[1] - (float)pa[1]),
                        (_Float16)(pr[2] - (float)pa[2]), (_Float16)(pr[3] - (float)pa[3])};
#pragma unroll
      for (int hh = 0; hh < NL; ++hh) {
        *reinterpret_cast<uint4*>(sv + n * RS + 16 * g) = pg.v[hh];
#pragma unroll
        for (int cb = 0; cb < BPS; ++cb) {
          // lanes 2j, 2j+1 of the group address the two 8-byte halves of
          // row 4g + (j & 3) (rows repeat: the low 4 bytes are used); lane n
          // receives column 16 cb + n of rows 4g .. 4g+3
          const int j = n >> 1;
          const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_i32x2_ptr)(sv + (4 * g + (j & 3)) * RS + 16 * cb + 8 * (n & 1)));
          const uint32_t codes = (uint32_t)t[0] & vmask_lo;
          const f16x2 v01 = fp8x2_to_f16<kFmt, false>(codes);
          const f16x2 v23 = fp8x2_to_f16<kFmt, true>(codes);
          const f16x4 vb = {v01[0], v01[1], v23[0], v23[1]};
          f32x4 acc = o[hh * BPS + cb];
          acc = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, vb, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x16f16(pl, vb, acc, 0, 0, 0);
          o[hh * BPS + cb] = acc;
        }
      }
    } else {
      // p = hi + lo, both bf16 (together 16 significant bits)
      s16x4 ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t hb = bf16_bits(pr[i]);
        ph[i] = (short)hb;
        pl[i] = (short)bf16_bits(pr[i] - __uint_as_float(hb << 16));
      }
#pragma unroll
      for (int hh = 0; hh < NL; ++hh) {
        *reinterpret_cast<uint4*>(sv + n * RS + 16 * g) = pg.v[hh];
#pragma unroll
        for (int cb = 0; cb < BPS; ++cb) {
          // lane j of the group addresses elements 16 cb + 4 (j & 3) .. +3 of
          // row 4g + (j >> 2); lane 4a + b receives element b of the pieces
          // of lanes a, a+4, a+8, a+12: column 16 cb + n of rows 4g .. 4g+3
          const s16x4 vr = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4_ptr)(sv + (4 * g + (n >> 2)) * RS + 2 * (16 * cb + 4 * (n & 3))));
          const i32x2 vw = __builtin_bit_cast(i32x2, vr);
          const s16x4 vb = __builtin_bit_cast(
              s16x4, i32x2{(int)((uint32_t)vw[0] & vmask_lo), (int)((uint32_t)vw[1] & vmask_hi)});
          f32x4 acc = o[hh * BPS + cb];
          acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vb, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pl, vb, acc, 0, 0, 0);
          o[hh * BPS + cb] = acc;
        }
      }
    }
  };

  // This wave's pages: pg0 + wave + NW*j.  Block ids are fetched 64 at a
  // time, one per lane, and broadcast with readlane.  PD-deep ring: every
  // buffer is consumed and re-issued in every steady round (prefetch indices
  // past the batch end clamp to its last page), so the compiler waits for
  // exactly the page about to be used; the last round issues nothing.
  const int first = pg0 + wave;
  const int npw = first < pg1 ? (pg1 - first + NW - 1) / NW : 0;
  for (int jb = 0; jb < npw; jb += 64) {
    const int cnt = min(64, npw - jb);
    const int page_base = first + NW * jb;
    const int my_blk = (jb == 0 && early_ids) ? early_blk
                                              : lane < cnt ? bt[page_base + NW * lane] : 0;
    auto blk_of = [&](int j) { return __builtin_amdgcn_readlane(my_blk, min(j, cnt - 1)); };
    Page ring[PD];
#pragma unroll
    for (int k = 0; k < PD; ++k) issue(ring[k], blk_of(k));
    if (jb == 0 && owner) append_row();   // before any page is used
    // steady rounds (straight-line: use each buffer, re-issue it), then the
    // last round without re-issues: a load past the batch would hold its
    // registers busy after the loop for data nobody reads
    int j = 0;
    for (; j + PD < cnt; j += PD) {
#pragma unroll
      for (int k = 0; k < PD; ++k) {
        run_page(ring[k], page_base + NW * (j + k));
        __builtin_amdgcn_sched_barrier(0);   // keep the reissue after the use
        issue(ring[k], blk_of(j + k + PD));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int k = 0; k < PD; ++k)
      if (j + k < cnt) run_page(ring[k], page_base + NW * (j + k));
  }

  // ---- merge the waves through LDS, kMergeHeads query heads per round -------
  l = cross_rows_sum(l);     // all keys of this wave, head n
  float* s_o = reinterpret_cast<float*>(s_mrg);                  // [NW][kMergeHeads][D]
  float* s_m = s_o + NW * kMergeHeads * D;                       // [NW][16]
  float* s_l = s_m + NW * 16;                                    // [NW][16]
  const int S = p.num_splits;
  const float vsc = p.fp8 ? p.v_scale[h] : 1.0f;
  __shared__ int s_last;
  if (lane < 16) {
    s_m[wave * 16 + lane] = m;
    s_l[wave * 16 + lane] = l;
  }
#pragma unroll
  for (int r0 = 0; r0 < G; r0 += kMergeHeads) {
    // this wave's rows r0 .. r0 + kMergeHeads - 1
#pragma unroll
    for (int c = 0; c < NB; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g + i - r0;
        if (hd >= 0 && hd < kMergeHeads && 4 * g + i < G)
          s_o[(wave * kMergeHeads + hd) * D + 16 * c + n] = o[c][i];
      }
    __syncthreads();
    // VW consecutive columns per thread, one partial store each
    constexpr int VW = ws_vec(kMergeHeads * D, 64 * NW);
    for (int t = threadIdx.x; t < kMergeHeads * D / VW; t += 64 * NW) {
      const int hd = t / (D / VW);
      const int d = (t % (D / VW)) * VW;
      const int hq = r0 + hd;
      if (hq < G) {
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w * 16 + hq]);
        f32x4 num = f32x4{0.f, 0.f, 0.f, 0.f};
        float den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float mw = s_m[w * 16 + hq];
          const float f = mw > kNegInf ? fast_exp2(mw - M) : 0.f;
#pragma unroll
          for (int c = 0; c < VW; ++c) num[c] += f * s_o[(w * kMergeHeads + hd) * D + d + c];
          den += f * s_l[w * 16 + hq];
        }
        if (S == 1) {
          // a single split: this workgroup's state is the whole answer (the
          // same expression as the split merge's output with one partial)
          const float f = vsc / den;
#pragma unroll
          for (int c = 0; c < VW; ++c)
            p.out[((size_t)b * p.num_q_heads + hq0 + hq) * D + d + c] = M > kNegInf ? num[c] * f : 0.f;
        } else {
          // this set's partial rows: [G heads][S splits][D] from head hq0
          const int row = hq * S + split;
          st_agentv<VW>(ws_rsrc(p.ws_o + ((size_t)b * p.num_q_heads + hq0) * S * D, (uint32_t)(G * S * D * 4)),
                    (uint32_t)(row * D + d) * 4, num);
          if (d == 0) {
            const size_t mrow = ((size_t)b * p.num_q_heads + hq0 + hq) * S + split;
            st_agent(p.ws_m + mrow, M);
            st_agent(p.ws_l + mrow, den);
          }
        }
      }
    }
    if (r0 + kMergeHeads < G) __syncthreads();
  }
  if (S == 1) return;   // no partials, no arrival count, no merge

  // ---- the last workgroups of this (sequence, head group) merge the splits --
  // Each thread waits until its partial stores are performed (they are
  // coherent agent-scope stores), then the workgroup counts its arrival.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int NG = p.num_groups;
  const size_t set = (size_t)b * gridDim.y + blockIdx.y;
  const size_t head0 = (size_t)b * p.num_q_heads + hq0;   // first query head of the set
  if (NG == 1) {
    // up to kDecodeSingleLevel splits: the last arrival merges them all into
    // the output and re-arms the counter for the next call
    int* counter = p.ws_count + set * kCounterStride;
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
    __syncthreads();
    if (!s_last) return;
    merge_rows<D, G, NW>(p.ws_o + head0 * S * D, p.ws_m + head0 * S, p.ws_l + head0 * S, S,
                         p.out + head0 * D, vsc);
    if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  // More splits: arrivals count per group of kDecodeFan splits, each group
  // counter on a line of its own (the arrivals of a launch would serialise
  // at the memory's atomic unit on a single line).  The last arrival of a
  // group re-arms its group counter and counts the group on the set counter.
  // The last mpg arrivals of every group merge, one slice of SW output
  // columns of one query head at a time, over all S partials, instead of one
  // workgroup reading every partial.  A merger that did not see the set
  // counter reach NG itself waits for it.  The wait ends: workgroups are
  // dispatched in grid order, so every split of an earlier set has started
  // and will finish, the splits of this set that have not arrived are running
  // or start on the CUs that other workgroups leave, and at most nm (<= 64)
  // workgroups of a set wait at a time; the poll count is bounded all the
  // same.  The last merger to finish re-arms the set counter and the done
  // counter for the next call; it does so only after every merger has seen
  // the full count.
  constexpr int SW = kSliceCols < D ? kSliceCols : D;   // columns per slice
  constexpr int NSL = G * D / SW;                 // output slices of the set
  const int grp = split / kDecodeFan;
  const int gn = min(kDecodeFan, S - grp * kDecodeFan);      // splits of this group
  const int gn_last = S - (NG - 1) * kDecodeFan;
  const int mpg = min((NSL + NG - 1) / NG, kDecodeFan);      // mergers per full group
  const int nm = (NG - 1) * mpg + min(gn_last, mpg);          // mergers in all
  int* gcount = p.ws_count + (set * NG + grp) * kCounterStride;
  int* scount = p.ws_count2 + (set * 2) * kCounterStride;
  int* done = p.ws_count2 + (set * 2 + 1) * kCounterStride;
  __shared__ int s_all;
  if (threadIdx.x == 0) {
    const int ticket = __hip_atomic_fetch_add(gcount, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int all = 0;
    if (ticket == gn - 1) {
      __hip_atomic_store(gcount, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      all = __hip_atomic_fetch_add(scount, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == NG - 1;
    }
    s_last = ticket;
    s_all = all;
  }
  __syncthreads();
  const int k = s_last - (gn - min(gn, mpg));     // merger index within the group
  if (k < 0) return;
  if (threadIdx.x == 0 && !s_all) {
    for (int it = 0; it < kMergeWaitPolls; ++it) {
      if (__hip_atomic_load(scount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= NG) break;
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  for (int sl = grp * mpg + k; sl < NSL; sl += nm) {
    const int g = sl / (D / SW);
    merge_slice<D, NW, SW>(p.ws_o + (head0 + g) * S * D, p.ws_m + (head0 + g) * S,
                           p.ws_l + (head0 + g) * S, S, (sl % (D / SW)) * SW,
                           p.out + (head0 + g) * D, vsc);
    __syncthreads();   // the slice's LDS is reused by the next one
  }
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nm - 1) {
    __hip_atomic_store(scount, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

static size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Counter sets are bounded by B * Hq (one per sequence, KV head and head
// group).  Each counter has a line of its own (kCounterStride ints): the
// arrivals of many workgroups at neighbouring counters of one line serialise
// at the memory's atomic unit (measured on MI355X: 32k Llama-shaped layer
// 20.40 -> 19.75 us with the counters apart; giving each split's m and l a
// line too measured 0.2-0.4 us slower, the merger then fetches more lines).
size_t decode_counter_bytes(int batch, int num_q_heads, int splits) {
  const size_t heads = (size_t)batch * num_q_heads;
  const int ng = decode_num_groups(splits);
  return heads * (ng + (ng > 1 ? 2 : 1)) * kCounterStride * 4;
}

size_t decode_partial_bytes(int batch, int num_q_heads, int head_dim, int splits) {
  const size_t heads = (size_t)batch * num_q_heads;
  return align16(heads * splits * head_dim * 4) + 2 * align16(heads * splits * 4);
}

size_t decode_workspace_bytes(int batch, int num_q_heads, int head_dim, int splits) {
  return decode_counter_bytes(batch, num_q_heads, splits) +
         decode_partial_bytes(batch, num_q_heads, head_dim, splits);
}

void decode_workspace_carve_split(int* counters, void* partials, int batch, int num_q_heads,
                                  int head_dim, int splits, DecodeParams& p) {
  const size_t heads = (size_t)batch * num_q_heads;
  const int ng = decode_num_groups(splits);
  p.ws_count = counters;
  p.ws_count2 = counters + heads * ng * kCounterStride;
  char* at = reinterpret_cast<char*>(partials);
  p.ws_o = reinterpret_cast<float*>(at);
  at += align16(heads * splits * head_dim * 4);
  p.ws_m = reinterpret_cast<float*>(at);
  at += align16(heads * splits * 4);
  p.ws_l = reinterpret_cast<float*>(at);
}

void decode_workspace_carve(void* ws, int batch, int num_q_heads, int head_dim, int splits,
                            DecodeParams& p) {
  decode_workspace_carve_split(reinterpret_cast<int*>(ws),
                               reinterpret_cast<char*>(ws) +
                                   decode_counter_bytes(batch, num_q_heads, splits),
                               batch, num_q_heads, head_dim, splits, p);
}

// Pages in flight per wave, by head_dim.  With one workgroup per CU a
// two-deep ring asks for a large share of a layer at once (half of a 67 MB
// head_dim-256 layer) and the first pages queue behind it; one page per wave
// measured faster on MI355X: head_dim 256, 128k single-KV-head layer
// 24.45 -> 23.19 us, 32k 16.26 -> 14.90 us; head_dim 128 (Llama-shaped),
// 32k 19.80 -> 19.36 us, 128k 55.08 -> 53.45 us, 8 x 20k 64.45 -> 62.80 us
// (8k 11.15 -> 11.28 us).  A deeper ring at head_dim 64 (3 or 4 pages)
// measured 5-6% slower.
template <int D>
constexpr int decode_pipe() {
  return D == 64 ? 2 : 1;
}

template <int D, int G, int kFmt>
static void launch_shape(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  constexpr int NW = kDecodeWaves;
  hipLaunchKernelGGL((decode_split_kernel<D, G, kFmt, NW, decode_pipe<D>()>), grid, dim3(64 * NW),
                     0, stream, p);
}

template <int D, int kFmt>
static hipError_t launch_decode_d(const DecodeParams& p, hipStream_t stream) {
  const int G = p.num_q_heads / p.num_kv_heads;
  const dim3 grid(p.num_splits, p.num_kv_heads, p.batch);
  switch (G) {
    case 1: launch_shape<D, 1, kFmt>(p, grid, stream); break;
    case 2: launch_shape<D, 2, kFmt>(p, grid, stream); break;
    case 4: launch_shape<D, 4, kFmt>(p, grid, stream); break;
    case 8: launch_shape<D, 8, kFmt>(p, grid, stream); break;
    case 16: launch_shape<D, 16, kFmt>(p, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int kFmt>
static hipError_t launch_decode_f(const DecodeParams& p, hipStream_t stream) {
  switch (p.head_dim) {
    case 64: return launch_decode_d<64, kFmt>(p, stream);
    case 128: return launch_decode_d<128, kFmt>(p, stream);
    case 256: return launch_decode_d<256, kFmt>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeParams& p, int fmt, hipStream_t stream) {
  switch (fmt) {
    case kFmtE4m3: return launch_decode_f<kFmtE4m3>(p, stream);
    case kFmtE5m2: return launch_decode_f<kFmtE5m2>(p, stream);
    case kFmtBf16: return launch_decode_f<kFmtBf16>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa8
