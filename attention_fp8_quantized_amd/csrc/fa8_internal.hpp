// Host-side launch entry points of the fa8attn kernels (internal; the public
// C ABI is include/fa8attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa8 {

// Element formats of the paged cache (template arguments of the kernels).
constexpr int kFmtBf16 = 0;   // bf16 values, 2 bytes
constexpr int kFmtE4m3 = 1;   // OCP E4M3 codes, 1 byte
constexpr int kFmtE5m2 = 2;   // OCP E5M2 codes, 1 byte

hipError_t launch_cache_write(const void* k, const void* v, bool in_bf16,
                              int64_t n_tokens, int num_kv_heads, int head_dim,
                              const int64_t* slot_mapping, const float* k_scale,
                              const float* v_scale, void* cache, int fmt,
                              hipStream_t stream);

// Per-KV-head absmax scales of k and v: three launches (zero, reduce,
// finalize) that write only k_scale and v_scale.
hipError_t launch_absmax_scales(const void* k, const void* v, bool in_bf16, int64_t n_tokens,
                                int num_kv_heads, int head_dim, float* k_scale,
                                float* v_scale, float fmt_max, int cus, hipStream_t stream);

struct DecodeParams {
  const uint16_t* q;          // bf16 [B][Hq][D]
  const uint8_t* cache;       // [nb][Hkv][2][16][D] elements
  const int32_t* block_table; // [B][max_blocks]
  const int32_t* seq_lens;    // [B]
  const float* k_scale;       // [Hkv]
  const float* v_scale;       // [Hkv]
  int* ws_count;              // group arrival counters [B][Hq][NG], zero between calls
  int* ws_count2;             // NG > 1: set and merger counters [B][Hq][2], zero between calls
  float* ws_o;                // [B][Hq][S][D]
  float* ws_m;                // [B][Hq][S]  (log2 domain)
  float* ws_l;                // [B][Hq][S]
  float* out;                 // [B][Hq][D]
  const void* k_new;          // fused append: [B][Hkv][D] row of token seq_len-1 (or null)
  const void* v_new;
  int new_bf16;               // fused append input: bf16 (1) or fp32 (0)
  int batch, num_q_heads, num_kv_heads, head_dim, max_blocks;
  int num_splits, pages_per_split, window, fp8;
  int num_groups, group_size; // split groups of the arrival count (1 group: single merger)
  float sm_scale;
};

// Splits are merged by the last workgroup to arrive when there are at most
// kDecodeSingleLevel of them; beyond that, arrivals are counted per group of
// kDecodeFan splits and the merge is spread over the last arrivals of every
// group, one slice of output columns each (decode.hip).
constexpr int kDecodeMaxSplits = 256;
constexpr int kDecodeSingleLevel = 64;
constexpr int kDecodeFan = 16;
inline int decode_num_groups(int splits) {
  return splits <= kDecodeSingleLevel ? 1 : (splits + kDecodeFan - 1) / kDecodeFan;
}

// Decode workspace layout for `splits` splits: int32 arrival counters
// [B][Hq][NG] and then [B][Hq] (NG = 1) or [B][Hq][2] (NG > 1: the set and
// merger counters), each kCounterStride ints apart (zero before the first
// call; every call leaves them zero), then fp32 o_part [B][Hq][S][D], m and
// l [B][Hq][S].  Every array starts 16-byte aligned when the workspace does.
constexpr int kCounterStride = 64;   // ints per counter (256 bytes: one line each)
constexpr int kDecodeWaves = 8;      // waves per decode workgroup
size_t decode_workspace_bytes(int batch, int num_q_heads, int head_dim, int splits);
void decode_workspace_carve(void* ws, int batch, int num_q_heads, int head_dim, int splits,
                            DecodeParams& p);
// The same layout in two pieces: the counters (decode_counter_bytes, zero
// between calls) and the partials (decode_partial_bytes, no initial value).
size_t decode_counter_bytes(int batch, int num_q_heads, int splits);
size_t decode_partial_bytes(int batch, int num_q_heads, int head_dim, int splits);
void decode_workspace_carve_split(int* counters, void* partials, int batch, int num_q_heads,
                                  int head_dim, int splits, DecodeParams& p);

// fmt: kFmtE4m3, kFmtE5m2 or kFmtBf16 (fa8_device.hpp)
hipError_t launch_decode(const DecodeParams& p, int fmt, hipStream_t stream);

struct PrefillParams {
  const uint16_t* q;          // bf16 [Tq][Hq][D]
  const int32_t* cu_q_lens;   // [B+1]
  const uint8_t* cache;       // FP8 codes [nb][Hkv][2][16][D]
  const int32_t* block_table; // [B][max_blocks]
  const int32_t* seq_lens;    // [B] (context incl. the chunk)
  const float* q_scale;       // [1]
  const float* k_scale;       // [Hkv]
  const float* v_scale;       // [Hkv]
  float* out;                 // [Tq][Hq][D]
  int batch, num_q_heads, num_kv_heads, head_dim, max_blocks, max_q_len;
  int window, accum_mode;
  int fmt;                    // cache format: kFmtE4m3 or kFmtE5m2
  float sm_scale;
};

int prefill_kv_tile(int head_dim);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

// bandwidth yardsticks (stream_bench.hip)
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, int cus,
                              hipStream_t stream);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, int cus,
                              hipStream_t stream);

}  // namespace fa8
