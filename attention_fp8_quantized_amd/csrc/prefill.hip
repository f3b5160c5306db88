// Causal FP8 prefill over the paged cache with two-level accumulation.
//
// [BLOG] "Introduction": both matmuls of attention, QK and Score*V, run in
// e4m3.  "Kernel and vLLM improvements / Two-level accumulation": the P*V
// partial sums of a tile are flushed into true fp32 registers, so the error
// does not grow with the contraction length (the context).  "Query
// Quantization Fusion": the query is quantised with a per-tensor scale right
// before attention -- here in the kernel's prologue.
//
// The cache holds e4m3 or e5m2 codes ([GPUSTACK] "KV キャッシュの量子化"
// names both FP8 cache formats); the query and P are always e4m3.
//
// Work decomposition: one workgroup per (query block, query head,
// sequence): at head_dim 256 and 64, 64 query rows in 4 waves of 16 rows
// (several workgroups per CU, one tile buffer each); at head_dim 128, 128
// rows in 4 waves of two 16-row blocks; flushing every N tiles, 128 rows in
// 8 waves of 16 (see prefill_mb and prefill_nwv).  Keys are visited in tiles
// of 128 at absolute, 128-aligned positions, in ascending order (this order
// and width are part of the numeric contract, see fa8_prefill_kv_tile).
//
// Per KV tile:
//   * the tile's K and V rows (8 pages of FP8 codes) are copied straight
//     into LDS (buffer loads with an LDS destination, 16 bytes per lane):
//     with two buffers the next tile's copies are in flight during the
//     current tile; with one, they start when every wave is done with it;
//     the block ids two tiles ahead are fetched meanwhile;
//   * S^T = K . Q^T on v_mfma_f32_16x16x32_bf16: the A operand is 8 K codes
//     of one key row per lane, widened to bf16 after the LDS read (exact:
//     bf16 holds every e4m3 and e5m2 value), the B operand the e4m3 query
//     (decoded to bf16, exact; held in registers for the whole kernel).  The
//     products are exactly the FP8 x FP8 products; the bf16 MFMA sums
//     them in fp32.  (The FP8 MFMA of this chip sums its 128 products with
//     about 13 bits below the largest one; the scores decide how each p
//     rounds to e4m3, so they are formed with fp32 sums.)  The result leaves
//     each lane with one query and 32 keys of the tile -- exactly the layout
//     the P operand of P.V needs;
//   * scores are scaled by q_scale*k_scale*sm_scale*log2(e), masked (causal,
//     window), the running row maximum m_t is updated, p = 2^(s - m_t) in
//     fp32; l = alpha*l + sum p (fp32, unquantised);
//   * P is rounded to e4m3 (round-to-nearest-even, the hardware packed
//     convert; unit scale, p in [0, 1]);
//   * V^T operand: ds_read_b64_tr_b8 gathers, for 16 lanes, one byte column
//     of 8 key rows; the key order matches the P operand slot by slot;
//   * P~ . V~ on the FP8 MFMA v_mfma_f32_16x16x128_f8f6f4 (K = the tile's
//     128 keys).  Level 1: acc = P~ . V~ into a zeroed fp32 accumulator;
//     level 2: O = alpha*O + acc in VALU fp32 (every tile).  The level-1
//     accumulator is one 16-column block at a time (4 registers), so the
//     flush costs no register file.  accum_mode = 0 instead lets the MFMA
//     accumulate into alpha*O (one level).  accum_mode = N >= 2 flushes every
//     N tiles ([BLOG] "大 Head Dimension 的限制" names this as the remedy on
//     its hardware): a full-width level-1 accumulator acc[D] keeps
//     acc = alpha*acc + P~.V~ on the MFMA for N tiles, then
//     O = (product of those alphas)*O + acc; a separate instantiation, so the
//     extra registers never burden modes 0 and 1.
// Epilogue: out = O * v_scale / l.

#include <type_traits>

#include "fa8_device.hpp"
#include "fa8_internal.hpp"

namespace fa8 {

constexpr int kTileN = 128;      // keys per KV tile
constexpr float kNegInfP = -__builtin_huge_valf();

int prefill_kv_tile(int) { return kTileN; }

// P~ (e4m3, A operand: cbsz = 0) times V~ (the cache's FP8 format, B
// operand: blgp = 0 for e4m3, 1 for e5m2), unit block scales (E8M0 127 = 2^0)
template <int kFmt>
__device__ __forceinline__ f32x4 mfma_pv(i32x8 a, i32x8 b, f32x4 c) {
  constexpr int kBlgp = kFmt == kFmtE5m2 ? 1 : 0;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, kBlgp, 0, 127, 0, 127);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2* lds_i32x2_ptr;

// 8 bytes per lane, transposed within each 16-lane group: lanes 2j and 2j+1
// give the addresses of the two 8-byte halves of row j (j = 0..7); lane i of
// the group receives byte column i of those 8 rows.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* lds_addr) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_ptr)(lds_addr));
}

// Lanes n, n+16, n+32, n+48 hold the same query: combine across them.
__device__ __forceinline__ float group4_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                       __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                       __builtin_bit_cast(uint32_t, v), false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// LDS layout of a staged tile: rows of D bytes, no padding; the 16-byte
// chunk c of row r sits at chunk position c ^ sw(r).  sw spreads the rows an
// operand read touches over the 64 banks: the K operand reads 16 consecutive
// rows, the transposed V reads rows 4g..4g+3 and 16+4g..16+4g+3.
template <int D>
__device__ __forceinline__ int swz(int r) {
  constexpr int CPR = D / 16;              // chunks per row
  constexpr int RPB = 256 / D;             // rows per 256-byte bank period
  return ((r / RPB) % CPR) ^ (((r >> 4) & 1) * (CPR / 2));
}

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// s_waitcnt immediate: wait until at most n vector-memory operations are
// outstanding (lgkm and exp counters not waited on); n up to 63
constexpr int vmcnt_imm(int n) { return 0x3F70 | (n & 15) | ((n >> 4) << 14); }
// s_waitcnt immediate: wait until every LDS operation of this wave is done
// (vector-memory and exp counters not waited on)
constexpr int kLgkm0 = 0xC07F;

// MB = query blocks of 16 rows per wave, NWV = waves per workgroup (16 MB
// NWV = 64 or 128 query rows).  With MB = 2 each widened K operand and each
// V^T operand feeds two MFMAs.  At head_dim 128 a wave then fits in 256
// registers, so two workgroups of four waves share a CU (two waves per
// SIMD, as with MB = 1); at head_dim 256 it needs a whole SIMD.  Four-wave
// workgroups run two per CU (four at head_dim 64).  The register budget is
// two waves per SIMD (256 registers per lane), four at head_dim 64 (128).
template <int D, int kFmt, bool kDeferred, int MB, int NWV>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2, D == 64 ? 4 : 2)))
void prefill_kernel(PrefillParams p) {
  constexpr int BM = 16 * MB * NWV;        // query rows per workgroup
  // 64-row workgroups (two per CU at head_dim 256, four at 64) stage each
  // tile into a single buffer once the tile before it is done; the other
  // workgroups of the CU compute meanwhile, and their barriers are not the
  // ones this workgroup waits at
  constexpr bool kSB = BM == 64;
  constexpr int KQ = D / 32;               // 32-wide chunks of the head dim (bf16 MFMA K)
  constexpr int DB = D / 16;               // 16-wide output column blocks
  constexpr int TILE = kTileN * D;         // bytes of one staged K (or V) tile
  constexpr int PPT = kTileN / kBlockSize; // pages per tile
  constexpr int RPI = 1024 / D;            // rows per wave-wide 16-byte-per-lane copy
  constexpr int CPT = TILE / 1024;         // copies per staged K (or V) tile
  constexpr int NCOPY = 2 * CPT / NWV;     // copies per wave per tile
  static_assert(MB == 1 || MB == 2, "query blocks per wave");
  static_assert(!kDeferred || MB == 1, "flush every N tiles: one query block per wave");
  static_assert(NCOPY >= 1 && kBlockSize % RPI == 0 && NCOPY + 1 <= 63, "staging tiling");
  static_assert(BM == 64 || BM == 128, "rows per workgroup");
  // tile buffers (K then V), filled by direct global->LDS copies: two, one
  // filled while the other is computed on, or (kSB) one
  __shared__ __attribute__((aligned(16))) uint8_t s_buf0[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint8_t s_buf1[kSB ? 16 : 2 * TILE];
  // Block ids of the staged pages live in registers, except in the
  // flush-every-N instantiation at head_dim 256: it spills, and the extra
  // live register raised its spill from 124 to 156 bytes per lane (32k
  // chunk with N = 2: 6.17 against 5.70 ms), so it keeps them in an LDS ring
  // of tiles t .. t+3.
  constexpr bool kIdRing = kDeferred && D == 256;
  __shared__ int s_bt[kIdRing ? 4 : 1][PPT];

  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int G = p.num_q_heads / p.num_kv_heads;
  const int h = hq / G;
  const int qs = p.cu_q_lens[b];
  const int T = p.cu_q_lens[b + 1] - qs;
  // longest causal blocks first: block x of the grid takes query block
  // (gridDim.x - 1 - x)
  const int q0 = (gridDim.x - 1 - blockIdx.x) * BM;
  if (q0 >= T) return;
  const int L = p.seq_lens[b];
  const int P0 = L - T;                    // position of the chunk's first query
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;                 // lane group (k-slot group of the MFMA)
  const int n = lane & 15;                 // query (S^T, P) or column (V, O) of the lane
  const int rbase = q0 + wave * 16 * MB;   // first query row of this wave
  int row[MB], pos[MB];                    // this lane's query row of block mb (S^T layout)
  bool row_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    row[mb] = rbase + 16 * mb + n;
    row_ok[mb] = row[mb] < T;
    pos[mb] = P0 + row[mb];
  }

  // ---- prologue: quantise this lane's slice of Q (B operand of S^T) ------
  // q8 = e4m3(fl32(q / q_scale)); the operand holds decode(q8) as bf16
  // (exact); q_scale enters the score multiplier.  Lane (g, n) holds query n
  // of each block; MFMA chunk kq takes the head-dim columns
  // 64*(kq/2) + 16*g + 8*(kq%2) .. +7 (a permutation of the contraction
  // index, the same for K), so that the K operands of chunks 2m and 2m+1
  // are one 16-byte run of a key row.
  const float qsc = p.q_scale[0];
  bf16x8 qb[MB][KQ];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int kq = 0; kq < KQ; ++kq) {
      uint4 w4 = make_uint4(0, 0, 0, 0);
      if (row_ok[mb])
        w4 = *reinterpret_cast<const uint4*>(
            p.q + ((size_t)(qs + row[mb]) * p.num_q_heads + hq) * D + 64 * (kq / 2) +
            16 * g + 8 * (kq % 2));
      const uint32_t ws[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int h2 = 0; h2 < 4; ++h2) {
        const uint32_t c2 = e4m3_encode(bf16_lo(ws[h2]) / qsc) |
                            (e4m3_encode(bf16_hi(ws[h2]) / qsc) << 8);
        const bf16x2 d2 = e4m3x2_to_bf16<false>(c2);
        qb[mb][kq][2 * h2] = d2[0];
        qb[mb][kq][2 * h2 + 1] = d2[1];
      }
      __builtin_amdgcn_sched_barrier(0);   // one chunk at a time (register pressure)
    }
  // log2-domain score multiplier
  const float qk = qsc * p.k_scale[h] * p.sm_scale * kLog2e;

  // ---- key range of this workgroup ---------------------------------------
  const int rmax = min(q0 + BM, T) - 1;
  const int lo_key = p.window > 0 ? max(0, P0 + q0 - p.window + 1) : 0;
  const int hi_key = P0 + rmax;
  const int t_lo = lo_key / kTileN;
  const int t_hi = hi_key / kTileN;
  const int n_pages = (L + kBlockSize - 1) / kBlockSize;
  const int32_t* bt = p.block_table + (size_t)b * p.max_blocks;
  const size_t head_off = (size_t)h * 2 * kBlockSize * D;
  const size_t blk_stride = (size_t)p.num_kv_heads * 2 * kBlockSize * D;

  // ---- state ----------------------------------------------------------------
  float m_run[MB], l_run[MB];    // running max (log2 domain) and denominator per block
  f32x4 o[MB][DB];               // O[query 4g+i of block mb][16db + n]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    m_run[mb] = kNegInfP;
    l_run[mb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[mb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // flush every N tiles (MB = 1 only): the full-width level-1 accumulator,
  // the product of the alphas since the last flush (rows 4g+i), tiles since
  // the last flush
  f32x4 acc_n[kDeferred ? DB : 1];
  float acum[4] = {1.f, 1.f, 1.f, 1.f};
  int since = 0;
  if constexpr (kDeferred) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc_n[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto flush_n = [&]() {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[0][db][i] = acum[i] * o[0][db][i] + acc_n[db][i];
      acc_n[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acum[i] = 1.f;
  };

  // Block id of page `page` of the sequence.  Only the entries of pages
  // lo_key/16 .. n_pages-1 are ever read (lo_key is the first key any row of
  // this block can see), so entries outside the window (a freed page, -1)
  // are never dereferenced.  A staged tile that reaches below the window or
  // past the end copies the nearest visible page instead; those rows are
  // masked in the scores and their V rows zeroed after the copy.  Inside the
  // tile loop the pages fetched (tile t+2 >= t_lo+2) all lie above the
  // window start, so only the end needs the clamp there.
  auto page_blk = [&](int page) { return bt[page < n_pages ? page : n_pages - 1]; };
  // Copy u of this wave (0..NCOPY-1) fills rows row0 .. row0+RPI-1 of the K
  // (first TILE bytes) or V tile, one 16-byte chunk per lane.  The row of a
  // lane within its page, and so its swizzle, depends on u at most through
  // u's parity: the two per-lane source offsets are computed once, and each
  // copy adds the (uniform) page address.  Lane j of a wave holds the block
  // id of the page its copy j % NCOPY reads: the ids are loaded a tile ahead
  // of their copies into registers and broadcast with readlane.  (With the
  // LDS ring, thread j < PPT loads page j's id and stores it in the ring.)
  const int cpage = kIdRing ? (int)(threadIdx.x % PPT)
                            : (((lane % NCOPY) * NWV + wave) % CPT) * RPI / kBlockSize;
  int lane_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int idx = (par % NCOPY) * NWV + wave;
    const int r = (idx % CPT) * RPI + lane / (D / 16);            // tile row of the lane
    lane_off[par] = (r % kBlockSize) * D + ((lane % (D / 16)) ^ swz<D>(r)) * 16;
  }
  // The copies are buffer loads with an LDS destination over one page's K
  // or V rows: unlike the global (FLAT-encoded) form, which may also reach
  // LDS through the flat aperture, they leave the compiler's LDS counter in
  // order, so an operand read waits for its own data only instead of for
  // every LDS read in flight.
  auto stage = [&](uint8_t* buf, int ids, int slot) {
    // opaque per call, so that the compiler keeps 32-bit lane offsets and
    // uniform page addresses instead of hoisting a 64-bit address per copy
    int voff0 = lane_off[0], voff1 = lane_off[1];
    asm volatile("" : "+v"(voff0), "+v"(voff1));
#pragma unroll
    for (int u = 0; u < NCOPY; ++u) {
      const int idx = u * NWV + wave;                    // 0 .. 2*CPT-1
      const int kv = idx / CPT;
      const int row0 = (idx % CPT) * RPI;                // first row (within the tile)
      const int blk = kIdRing ? __builtin_amdgcn_readfirstlane(s_bt[slot][row0 / kBlockSize])
                              : __builtin_amdgcn_readlane(ids, u);
      const uint8_t* page = p.cache + (size_t)blk * blk_stride + head_off +
                            (size_t)kv * kBlockSize * D;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint8_t*>(page), 0, kBlockSize * D, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(buf + kv * TILE + row0 * D), 16,
                                               (u & 1) ? voff1 : voff0, 0, 0, 0);
    }
  };

  // block ids of the first two tiles (pages below the window start read the
  // first visible page's entry instead)
  const int ids_first = page_blk(max(t_lo * PPT + cpage, lo_key / kBlockSize));
  int ids_n1 = page_blk(max((t_lo + 1) * PPT + cpage, lo_key / kBlockSize));   // tile t+1
  if constexpr (kIdRing) {
    if (threadIdx.x < PPT) {
      s_bt[t_lo & 3][threadIdx.x] = ids_first;
      s_bt[(t_lo + 1) & 3][threadIdx.x] = ids_n1;
    }
    __syncthreads();
  }
  stage(s_buf0, ids_first, t_lo & 3);
  // A window that starts inside the first tile: its V rows before the first
  // visible key hold another page's rows or a stale page's bytes (NaN codes,
  // say), and P = 0 times NaN would be NaN.  Wait for this tile's copies and
  // zero those rows; the first tile's barrier publishes them.
  if (lo_key > t_lo * kTileN) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const int rows_lo = lo_key - t_lo * kTileN;
#pragma unroll
    for (int u = 0; u < NCOPY; ++u) {
      const int idx = u * NWV + wave;
      const int row0 = (idx % CPT) * RPI;
      if (idx / CPT == 1 && row0 + lane / (D / 16) < rows_lo)
        *reinterpret_cast<uint4*>(s_buf0 + TILE + row0 * D + lane * 16) = make_uint4(0, 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(kLgkm0);
  }

  // One tile.  kOdd selects the buffer roles at compile time (the tile loop is
  // unrolled by two), so the compiler sees that the copies in flight target
  // the other buffer than the one being read.
  auto tile_step = [&](auto odd_tag, int t) {
    constexpr bool kOdd = decltype(odd_tag)::value;
    uint8_t* cur = (kOdd && !kSB) ? s_buf1 : s_buf0;
    uint8_t* nxt = (kOdd || kSB) ? s_buf0 : s_buf1;
    const uint8_t* s_k = cur;
    const uint8_t* s_v = cur + TILE;
    // block ids of tile t+2 (every lane loads one, so that the number of
    // loads in flight is the same in every lane)
    const int ids_n2 = page_blk((t + 2) * PPT + cpage);
    // the next tile's copies (after the last tile: a tile past the end, all
    // zero rows, never read), then wait for this tile's copies: everything
    // but the id load and the NCOPY copies just issued
    if constexpr (!kSB) {
      stage(nxt, ids_n1, (t + 1) & 3);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NCOPY + 1));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(1));   // all but the id load
    }
    // rows past the sequence end (the tail tile only): they hold another
    // page's rows or whatever a stale page held, and P = 0 times NaN would
    // be NaN, so every lane overwrites the V chunks it copied there with
    // zeros before the barrier publishes them (rows before a window start:
    // the prologue)
    if ((t + 1) * kTileN > L) {
      const int rows_left = L - t * kTileN;
#pragma unroll
      for (int u = 0; u < NCOPY; ++u) {
        const int idx = u * NWV + wave;
        const int row0 = (idx % CPT) * RPI;
        if (idx / CPT == 1 && row0 + lane / (D / 16) >= rows_left)
          *reinterpret_cast<uint4*>(cur + TILE + row0 * D + lane * 16) = make_uint4(0, 0, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(kLgkm0);   // the zeros land before the barrier
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // The scores run at raised wave priority: while one wave of a SIMD issues
    // its QK^T products (and the K widening that feeds them), the other
    // wave's softmax and P.V fill the gaps, instead of the two competing
    // for issue slots as equals.  Measured on MI355X: 32k head_dim-256
    // chunk 4.51 -> 4.28 ms, head_dim 128 2.87 -> 2.73 ms; raising it
    // through the softmax as well is slower (4.43 ms).
    __builtin_amdgcn_s_setprio(1);
    // ---- S^T = K . Q^T : 8 blocks of 16 keys -----------------------------------
    // the A operand: 8 K codes of key 16 kb + n, columns 32 kq + 8 g,
    // widened to bf16 (exact) once and used for every query block
    f32x4 s[MB][8];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) s[mb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // software pipeline over the 8 key blocks: the operand reads of block
    // kb+1 (one 16-byte read per pair of chunks) are issued after block kb's
    // first product, so the LDS round trip hides behind the rest
    auto k_reads = [&](uint4 (&ka)[KQ / 2], int kb) {
      const int kr = 16 * kb + n;
      const uint8_t* krow = s_k + kr * D;
      const int ksw = swz<D>(kr);
#pragma unroll
      for (int m = 0; m < KQ / 2; ++m)
        ka[m] = *reinterpret_cast<const uint4*>(krow + (((4 * m + g) ^ ksw) * 16));
    };
    uint4 ka[2][KQ / 2];
    k_reads(ka[0], 0);
    __builtin_amdgcn_sched_group_barrier(0x100, KQ / 2, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      if (kb + 1 < 8) k_reads(ka[(kb + 1) & 1], kb + 1);
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        const uint4 pair = ka[kb & 1][kq / 2];
        const uint2 a = (kq % 2) ? make_uint2(pair.z, pair.w) : make_uint2(pair.x, pair.y);
        const bf16x2 a0 = fp8x2_to_bf16<kFmt, false>(a.x), a1 = fp8x2_to_bf16<kFmt, true>(a.x);
        const bf16x2 a2 = fp8x2_to_bf16<kFmt, false>(a.y), a3 = fp8x2_to_bf16<kFmt, true>(a.y);
        const bf16x8 av = {a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          s[mb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb[mb][kq], s[mb][kb], 0, 0, 0);
      }
      // instruction order: (4 converts, MB products) per chunk of this block,
      // with the next block's reads after the first chunk (the wait before
      // the first chunk then covers only this block's reads)
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) {
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MB, 0);
        if (kq == 0 && kb + 1 < 8) __builtin_amdgcn_sched_group_barrier(0x100, KQ / 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    __builtin_amdgcn_s_setprio(0);
    // tiles wholly visible to every row of the block skip the mask
    const int k_first = t * kTileN, k_last = k_first + kTileN - 1;
    const bool full = k_last <= P0 + q0 && q0 + BM <= T &&
                      (p.window <= 0 || P0 + rmax - k_first < p.window);
    i32x8 pa[MB];
    float alpha_o[MB][4];    // alpha of the four queries (4g + i) whose O rows this lane holds
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      float tmax = kNegInfP;
      if (full) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[mb][kb][i] *= qk;
            tmax = fmaxf(tmax, s[mb][kb][i]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k_first + 16 * kb + 4 * g + i;
            const bool vis = row_ok[mb] && key <= pos[mb] &&
                             (p.window <= 0 || pos[mb] - key < p.window);
            const float v = vis ? s[mb][kb][i] * qk : kNegInfP;
            s[mb][kb][i] = v;
            tmax = fmaxf(tmax, v);
          }
      }
      tmax = group4_max(tmax);
      const float m_new = fmaxf(m_run[mb], tmax);
      const float ref = m_new > kNegInfP ? m_new : 0.f;
      const float alpha = m_run[mb] > kNegInfP ? fast_exp2(m_run[mb] - m_new) : 0.f;

      // ---- probabilities: fp32 sum, e4m3 operand -----------------------------
      float psum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[i] = fast_exp2(s[mb][kb][i] - ref);
          psum += pv[i];
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);  // RNE
        w = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], w, true);
        pa[mb][kb] = w;
      }
      psum = group4_sum(psum);
      l_run[mb] = alpha * l_run[mb] + psum;
      m_run[mb] = m_new;
#pragma unroll
      for (int i = 0; i < 4; ++i) alpha_o[mb][i] = __shfl(alpha, 4 * g + i);
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- P~ . V~ per 16-column block -------------------------------------------
    // row j = n/2 of read r is key kappa(g, 8r + j); lanes 2j, 2j+1 give the
    // two 8-byte halves of the block's 16 columns
    const int j = n >> 1;
    const uint8_t* vrow[4];
    int vsw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kr = 32 * r + 16 * (j >> 2) + 4 * g + (j & 3);
      vrow[r] = s_v + kr * D + (n & 1) * 8;
      vsw[r] = swz<D>(kr);
    }
    auto load_vb = [&](int db) {
      i32x8 vb;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const i32x2 v2 = lds_read_tr8(vrow[r] + ((db ^ vsw[r]) * 16));
        vb[2 * r] = v2[0];
        vb[2 * r + 1] = v2[1];
      }
      return vb;
    };
    // software pipeline: the next block's V^T reads are in flight while this
    // block's products run.  The accumulation mode is tested once per tile.
    if constexpr (kDeferred) {
      i32x8 vb_next = load_vb(0);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i32x8 vb = vb_next;
        if (db + 1 < DB) vb_next = load_vb(db + 1);
        f32x4 c;
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = alpha_o[0][i] * acc_n[db][i];
        acc_n[db] = mfma_pv<kFmt>(pa[0], vb, c);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acum[i] *= alpha_o[0][i];
      if (++since == p.accum_mode) {   // uniform: every lane visits the same tiles
        flush_n();
        since = 0;
      }
    } else if (p.accum_mode == 1) {
      // level 1: this tile's P.V of a 16-column block into a zeroed
      // accumulator; level 2: the fp32 flush O = alpha*O + acc, one block
      // behind, so that the flush's wait for its product overlaps the next
      // block's product (measured on MI355X, 32k chunk: head_dim 256 3.95 ->
      // 3.90 ms, 128 2.39 -> 2.34 ms, 64 1.72 -> 1.69 ms)
      i32x8 vb_next = load_vb(0);
      f32x4 acc_prev[MB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i32x8 vb = vb_next;
        if (db + 1 < DB) vb_next = load_vb(db + 1);
        f32x4 acc[MB];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb] = mfma_pv<kFmt>(pa[mb], vb, f32x4{0.f, 0.f, 0.f, 0.f});
        if (db > 0) {
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) o[mb][db - 1][i] = alpha_o[mb][i] * o[mb][db - 1][i] + acc_prev[mb][i];
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc_prev[mb] = acc[mb];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[mb][DB - 1][i] = alpha_o[mb][i] * o[mb][DB - 1][i] + acc_prev[mb][i];
    } else {
      i32x8 vb_next = load_vb(0);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i32x8 vb = vb_next;
        if (db + 1 < DB) vb_next = load_vb(db + 1);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          f32x4 c;
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] = alpha_o[mb][i] * o[mb][db][i];
          o[mb][db] = mfma_pv<kFmt>(pa[mb], vb, c);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const int ids_n1_cur = ids_n1;
    ids_n1 = ids_n2;
    // every wave is done with this buffer (the next copies into it start
    // after this barrier).  The fence covers LDS only, so the copies in
    // flight into the other buffer stay in flight across the barrier (a
    // full workgroup fence waits for every vector-memory operation).  With
    // the LDS ring the barrier also publishes the block ids of tile t+2.
    if constexpr (kIdRing) {
      if (threadIdx.x < PPT) s_bt[(t + 2) & 3][threadIdx.x] = ids_n2;
      __syncthreads();
    } else {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    if constexpr (kSB) stage(nxt, ids_n1_cur, (t + 1) & 3);
  };

  for (int t = t_lo; t <= t_hi; t += 2) {
    tile_step(std::false_type{}, t);
    if (t + 1 <= t_hi) tile_step(std::true_type{}, t + 1);
  }
  // the last tile's copies (a tile past the end) land before the waves end
  // and the workgroup's LDS is released (s_endpgm would also wait for them)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  if constexpr (kDeferred) flush_n();   // the tiles since the last flush

  // ---- epilogue: out = O * v_scale / l ---------------------------------------
  const float vsc = p.v_scale[h];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float li = __shfl(l_run[mb], 4 * g + i);
      const int orow = rbase + 16 * mb + 4 * g + i;
      if (orow < T) {
        const float sc = li > 0.f ? vsc / li : 0.f;
        float* dst = p.out + ((size_t)(qs + orow) * p.num_q_heads + hq) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) dst[16 * db + n] = o[mb][db][i] * sc;
      }
    }
}

// Query blocks per wave by head_dim, measured on MI355X (32k causal chunk,
// 8 query heads on one KV head, two-level / one-level accumulation): at 128
// two blocks take 2.50 / 2.42-2.44 ms against 2.73 / 2.59 ms for one; at 64
// one block is faster (1.80-1.84 / 1.73 ms against 1.86 / 1.77 ms); at 256
// two blocks need a whole SIMD per wave and spill (8.3 ms against 4.3 ms).
// Flush every N tiles keeps one block per wave (its second accumulator
// already fills the registers).
template <int D, bool kDeferred>
constexpr int prefill_mb() {
  return (!kDeferred && D == 128) ? 2 : 1;
}

// Waves per workgroup.  Four-wave workgroups of one block per wave (64
// rows, single tile buffer) at head_dim 256 and 64, measured on MI355X
// against eight-wave double-buffered ones (32k chunk, 8 query heads on one
// KV head): head_dim 256 4.01-4.07 / 3.84-3.99 ms against 4.20 / 4.10 ms
// (two-level / one-level), head_dim 64 1.70-1.73 / 1.64 ms against
// 1.77-1.81 / 1.69 ms (every 4 tiles 1.73 against 1.93 ms).  The head_dim
// 256 flush-every-N instantiation spills more in that form (196 against 112
// bytes per lane, 7.9 against 5.5 ms with N = 2) and keeps eight waves.
template <int D, bool kDeferred>
constexpr int prefill_nwv() {
  return ((D == 256 && !kDeferred) || D == 64) ? 4 : 8 / prefill_mb<D, kDeferred>();
}

template <int D, int kFmt, bool kDeferred>
static void launch_prefill_d(const PrefillParams& p, dim3 grid, hipStream_t stream) {
  constexpr int MB = prefill_mb<D, kDeferred>();
  constexpr int NWV = prefill_nwv<D, kDeferred>();
  grid.x = (p.max_q_len + 16 * MB * NWV - 1) / (16 * MB * NWV);
  hipLaunchKernelGGL((prefill_kernel<D, kFmt, kDeferred, MB, NWV>), grid, dim3(64 * NWV), 0, stream, p);
}

template <int kFmt, bool kDeferred>
static hipError_t launch_prefill_f(const PrefillParams& p, dim3 grid, hipStream_t stream) {
  switch (p.head_dim) {
    case 64: launch_prefill_d<64, kFmt, kDeferred>(p, grid, stream); break;
    case 128: launch_prefill_d<128, kFmt, kDeferred>(p, grid, stream); break;
    case 256: launch_prefill_d<256, kFmt, kDeferred>(p, grid, stream); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid(1, p.num_q_heads, p.batch);   // x: query blocks, set per instantiation
  const bool deferred = p.accum_mode >= 2;
  switch (p.fmt) {
    case kFmtE4m3:
      return deferred ? launch_prefill_f<kFmtE4m3, true>(p, grid, stream)
                      : launch_prefill_f<kFmtE4m3, false>(p, grid, stream);
    case kFmtE5m2:
      return deferred ? launch_prefill_f<kFmtE5m2, true>(p, grid, stream)
                      : launch_prefill_f<kFmtE5m2, false>(p, grid, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace fa8
