// C ABI of libfa8attn.so (declared in include/fa8attn.h): argument checks,
// split heuristic, workspace sizing, error strings, then the launches.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/fa8attn.h"
#include "fa8_internal.hpp"

namespace {

thread_local std::string g_last_error;

fa8_status fail(fa8_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fa8_status fail(fa8_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

fa8_status ok() {
  g_last_error.clear();
  return FA8_OK;
}

fa8_status hip_fail(hipError_t e, const char* what) {
  return fail(FA8_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool head_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
bool fp8_cache(int32_t dt) { return dt == FA8_E4M3 || dt == FA8_E5M2; }

// fa8_dtype of a cache -> kernel template format (caller checked the value)
int kernel_fmt(int32_t dt) {
  return dt == FA8_E4M3 ? fa8::kFmtE4m3 : dt == FA8_E5M2 ? fa8::kFmtE5m2 : fa8::kFmtBf16;
}
bool group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

// The decode and prefill grids put heads on y and sequences on z, whose
// extent a launch limits to 65535 workgroups.
constexpr int kMaxGridYZ = 65535;

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  static thread_local int cached_dev = -1, cached_cus = 0;
  if (dev == cached_dev) return cached_cus;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  cached_dev = dev;
  cached_cus = cus;
  return cus;
}

// Pages one decode workgroup may have to visit for the longest sequence.
int decode_pages_max(int max_seq_len, int window) {
  if (max_seq_len <= 0) return 0;
  const int visible = window > 0 ? std::min(window, max_seq_len) : max_seq_len;
  // a window that does not start on a page boundary spans one extra page
  return (visible + FA8_BLOCK_SIZE - 1) / FA8_BLOCK_SIZE + (window > 0 ? 1 : 0);
}

}  // namespace

// ---- scratch of the allocation-free decode entry point ----------------------
// Split partials and arrival counters of fa8_decode_attention_noalloc live in
// this array instead of a caller's workspace: the first
// FA8_DECODE_SCRATCH_COUNTERS counters (each on its own 256-byte line, as in
// a workspace) are the arrival counters (zero between calls: cleared once
// per device, then re-armed by every call), the rest holds the partials.  Each GPU the library runs on has its own copy, held
// until the process ends.  Host code never uses the name itself (it is a
// host-side stand-in, not a device address): kernels and fills get the
// per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[FA8_DECODE_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchCounterBytes = (size_t)FA8_DECODE_SCRATCH_COUNTERS * 4 * fa8::kCounterStride;
constexpr int kMaxDevices = 64;

struct ScratchSlot {
  void* ptr = nullptr;   // device address of `scratch` on this device
  bool cleared = false;  // counters cleared by a call that ran eagerly
};
ScratchSlot g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// Device address of this device's scratch; on a call that is not being
// captured into a graph and finds the counters not yet cleared, the counter
// region is cleared first on `stream` (a kernel, not a memset, so that a
// captured call records an ordinary kernel node; a captured call clears on
// every replay until an eager call has cleared them).
fa8_status scratch_for_call(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "decode_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FA8_EUNSUPPORTED, "decode_noalloc: device ordinal %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchSlot& slot = g_scratch[dev];
  if (!slot.ptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e, "decode_noalloc: hipGetSymbolAddress");
    slot.ptr = ptr;
  }
  if (!slot.cleared) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_fail(e, "decode_noalloc: hipStreamIsCapturing");
    hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t*>(slot.ptr), (int)(kScratchCounterBytes / 4));
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "decode_noalloc: counter clear launch");
    if (cap == hipStreamCaptureStatusNone) slot.cleared = true;
  }
  *out = slot.ptr;
  return FA8_OK;
}

}  // namespace

extern "C" {

const char* fa8_status_string(int32_t status) {
  switch (status) {
    case FA8_OK: return "ok";
    case FA8_EINVAL: return "invalid argument";
    case FA8_EUNSUPPORTED: return "unsupported configuration";
    case FA8_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fa8_last_error(void) { return g_last_error.c_str(); }

fa8_status fa8_cache_write(const void* k, const void* v, int32_t in_dtype,
                           int64_t n_tokens, int32_t num_kv_heads, int32_t head_dim,
                           const int64_t* slot_mapping, const float* k_scale,
                           const float* v_scale, void* cache, int32_t cache_dtype,
                           int64_t num_blocks, void* stream) {
  if (n_tokens < 0) return fail(FA8_EINVAL, "cache_write: n_tokens < 0");
  if (in_dtype != FA8_F32 && in_dtype != FA8_BF16)
    return fail(FA8_EINVAL, "cache_write: in_dtype must be FA8_F32 or FA8_BF16");
  if (!fp8_cache(cache_dtype) && cache_dtype != FA8_BF16)
    return fail(FA8_EINVAL, "cache_write: cache_dtype must be FA8_E4M3, FA8_E5M2 or FA8_BF16");
  if (num_kv_heads <= 0) return fail(FA8_EINVAL, "cache_write: num_kv_heads must be > 0");
  if (!head_dim_ok(head_dim))
    return fail(FA8_EUNSUPPORTED, "cache_write: head_dim %d not in {64,128,256}", head_dim);
  if (num_blocks < 0) return fail(FA8_EINVAL, "cache_write: num_blocks < 0");
  if (n_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !cache)
    return fail(FA8_EINVAL, "cache_write: null k, v, slot_mapping or cache");
  if (fp8_cache(cache_dtype) && (!k_scale || !v_scale))
    return fail(FA8_EINVAL, "cache_write: an FP8 cache needs k_scale and v_scale");
  const hipError_t e = fa8::launch_cache_write(
      k, v, in_dtype == FA8_BF16, n_tokens, num_kv_heads, head_dim, slot_mapping,
      k_scale, v_scale, cache, kernel_fmt(cache_dtype),
      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache_write launch");
  return ok();
}

fa8_status fa8_absmax_scales(const void* k, const void* v, int32_t in_dtype,
                             int64_t n_tokens, int32_t num_kv_heads, int32_t head_dim,
                             int32_t cache_dtype, float* k_scale, float* v_scale,
                             void* stream) {
  if (n_tokens < 0) return fail(FA8_EINVAL, "absmax_scales: n_tokens < 0");
  if (in_dtype != FA8_F32 && in_dtype != FA8_BF16)
    return fail(FA8_EINVAL, "absmax_scales: in_dtype must be FA8_F32 or FA8_BF16");
  if (!fp8_cache(cache_dtype))
    return fail(FA8_EINVAL, "absmax_scales: cache_dtype must be FA8_E4M3 or FA8_E5M2");
  if (num_kv_heads <= 0 || num_kv_heads > 4096)
    return fail(FA8_EINVAL, "absmax_scales: num_kv_heads must be in 1..4096");
  if (!head_dim_ok(head_dim))
    return fail(FA8_EUNSUPPORTED, "absmax_scales: head_dim %d not in {64,128,256}", head_dim);
  if (!k_scale || !v_scale) return fail(FA8_EINVAL, "absmax_scales: null k_scale or v_scale");
  if (n_tokens > 0 && (!k || !v)) return fail(FA8_EINVAL, "absmax_scales: null k or v");
  const hipError_t e = fa8::launch_absmax_scales(
      k, v, in_dtype == FA8_BF16, n_tokens, num_kv_heads, head_dim, k_scale, v_scale,
      cache_dtype == FA8_E4M3 ? 448.0f : 57344.0f,
      device_cu_count(), reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "absmax_scales launch");
  return ok();
}

int32_t fa8_decode_num_splits(int32_t batch, int32_t num_kv_heads, int32_t max_seq_len,
                              int32_t window) {
  const int pages = decode_pages_max(max_seq_len, window);
  if (batch <= 0 || num_kv_heads <= 0 || pages <= 0) return 1;
  // One workgroup per CU (a decode workgroup fills a CU's register file):
  // as many splits as fit the CUs beside the other (sequence, KV head) sets
  // without a second round of workgroups, and at least one page per wave in
  // every split.  Each split pays a fixed chain (block ids, first pages, its
  // share of the merge).  Measured on MI355X with the arrival counters on
  // separate lines: 32k Llama-shaped layer 19.9-20.0 us with 32 splits
  // against 20.3 us with 28 (7/8 of the CUs); single-KV-head head_dim-256
  // 128k layer 24.4 us with 256 splits against 24.6-25.4 us with 224.
  const int cus = device_cu_count();
  const long sets = (long)batch * num_kv_heads;
  long splits = cus / sets;
  const long min_pages = fa8::kDecodeWaves;
  const long by_pages = pages / min_pages;
  if (splits > by_pages) splits = by_pages;
  if (splits < 1) splits = 1;
  if (splits > fa8::kDecodeMaxSplits) splits = fa8::kDecodeMaxSplits;
  return (int32_t)splits;
}

size_t fa8_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_splits) {
  if (batch <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  return fa8::decode_workspace_bytes(batch, num_q_heads, head_dim, num_splits);
}

static fa8_status decode_impl(const void* q, int32_t batch, int32_t num_q_heads,
                              const void* cache, int32_t cache_dtype, int64_t num_blocks,
                              int32_t num_kv_heads, int32_t head_dim,
                              const int32_t* block_table, int32_t max_blocks_per_seq,
                              const int32_t* seq_lens, int32_t max_seq_len,
                              const float* k_scale, const float* v_scale, float sm_scale,
                              int32_t window, int32_t num_splits, float* out,
                              void* workspace, size_t workspace_bytes, void* stream,
                              const void* k_new, const void* v_new, int32_t new_dtype,
                              bool use_scratch = false) {
  if (batch < 0) return fail(FA8_EINVAL, "decode: batch < 0");
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(FA8_EINVAL, "decode: head counts must be > 0");
  if (num_q_heads % num_kv_heads != 0)
    return fail(FA8_EINVAL, "decode: num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (!group_ok(num_q_heads / num_kv_heads))
    return fail(FA8_EUNSUPPORTED, "decode: query heads per KV head %d not in {1,2,4,8,16}",
                num_q_heads / num_kv_heads);
  if (!head_dim_ok(head_dim))
    return fail(FA8_EUNSUPPORTED, "decode: head_dim %d not in {64,128,256}", head_dim);
  if (!fp8_cache(cache_dtype) && cache_dtype != FA8_BF16)
    return fail(FA8_EINVAL, "decode: cache_dtype must be FA8_E4M3, FA8_E5M2 or FA8_BF16");
  if (max_seq_len < 0 || max_blocks_per_seq < 0 || num_blocks < 0)
    return fail(FA8_EINVAL, "decode: negative size");
  if ((int64_t)max_blocks_per_seq * FA8_BLOCK_SIZE < max_seq_len)
    return fail(FA8_EINVAL, "decode: max_blocks_per_seq*16 < max_seq_len");
  if (!(std::isfinite(sm_scale)))
    return fail(FA8_EINVAL, "decode: sm_scale must be finite");
  if (num_splits < 0 || num_splits > fa8::kDecodeMaxSplits)
    return fail(FA8_EINVAL, "decode: num_splits must be in 0..%d", fa8::kDecodeMaxSplits);
  if (batch > kMaxGridYZ || num_kv_heads > kMaxGridYZ)
    return fail(FA8_EUNSUPPORTED, "decode: batch and num_kv_heads must be <= %d", kMaxGridYZ);
  if (batch == 0) return ok();
  if (!q || !cache || !block_table || !seq_lens || !out || (!use_scratch && !workspace))
    return fail(FA8_EINVAL, "decode: null pointer argument");
  if (fp8_cache(cache_dtype) && (!k_scale || !v_scale))
    return fail(FA8_EINVAL, "decode: an FP8 cache needs k_scale and v_scale");
  if (!use_scratch && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(FA8_EINVAL, "decode: workspace must be 16-byte aligned");

  const int S = num_splits > 0 ? num_splits
                               : fa8_decode_num_splits(batch, num_kv_heads, max_seq_len, window);
  // Beyond kDecodeSingleLevel splits up to that many mergers of a set wait
  // for the set's other splits, which must still find a CU to start on.
  if (fa8::decode_num_groups(S) > 1 && device_cu_count() <= fa8::kDecodeSingleLevel)
    return fail(FA8_EUNSUPPORTED, "decode: %d splits need more than %d compute units, the device has %d",
                S, fa8::kDecodeSingleLevel, device_cu_count());
  fa8::DecodeParams p{};
  if (use_scratch) {
    const size_t cb = fa8::decode_counter_bytes(batch, num_q_heads, S);
    const size_t pb = fa8::decode_partial_bytes(batch, num_q_heads, head_dim, S);
    if (cb > kScratchCounterBytes || pb > FA8_DECODE_SCRATCH_BYTES - kScratchCounterBytes)
      return fail(FA8_EINVAL,
                  "decode_noalloc: %d splits need %zu counter bytes and %zu partial bytes; "
                  "the scratch holds at most %zu and %zu",
                  S, cb, pb, kScratchCounterBytes,
                  (size_t)FA8_DECODE_SCRATCH_BYTES - kScratchCounterBytes);
    void* base = nullptr;
    const fa8_status st = scratch_for_call(reinterpret_cast<hipStream_t>(stream), &base);
    if (st != FA8_OK) return st;
    fa8::decode_workspace_carve_split(reinterpret_cast<int*>(base),
                                      reinterpret_cast<char*>(base) + kScratchCounterBytes,
                                      batch, num_q_heads, head_dim, S, p);
  } else {
    const size_t need = fa8::decode_workspace_bytes(batch, num_q_heads, head_dim, S);
    if (workspace_bytes < need)
      return fail(FA8_EINVAL, "decode: workspace has %zu bytes, %zu needed for %d splits",
                  workspace_bytes, need, S);
    fa8::decode_workspace_carve(workspace, batch, num_q_heads, head_dim, S, p);
  }

  p.q = reinterpret_cast<const uint16_t*>(q);
  p.cache = reinterpret_cast<const uint8_t*>(cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.out = out;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.max_blocks = max_blocks_per_seq;
  p.num_splits = S;
  p.num_groups = fa8::decode_num_groups(S);
  p.group_size = p.num_groups == 1 ? S : fa8::kDecodeFan;
  const int pages = decode_pages_max(max_seq_len, window);
  p.pages_per_split = pages > 0 ? (pages + S - 1) / S : 1;
  p.window = window > 0 ? window : 0;
  p.fp8 = fp8_cache(cache_dtype) ? 1 : 0;
  p.sm_scale = sm_scale;
  p.k_new = k_new;
  p.v_new = v_new;
  p.new_bf16 = new_dtype == FA8_BF16 ? 1 : 0;
  const hipError_t e =
      fa8::launch_decode(p, kernel_fmt(cache_dtype), reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

fa8_status fa8_decode_attention(const void* q, int32_t batch, int32_t num_q_heads,
                                const void* cache, int32_t cache_dtype, int64_t num_blocks,
                                int32_t num_kv_heads, int32_t head_dim,
                                const int32_t* block_table, int32_t max_blocks_per_seq,
                                const int32_t* seq_lens, int32_t max_seq_len,
                                const float* k_scale, const float* v_scale, float sm_scale,
                                int32_t window, int32_t num_splits, float* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(q, batch, num_q_heads, cache, cache_dtype, num_blocks, num_kv_heads,
                     head_dim, block_table, max_blocks_per_seq, seq_lens, max_seq_len, k_scale,
                     v_scale, sm_scale, window, num_splits, out, workspace, workspace_bytes,
                     stream, nullptr, nullptr, FA8_F32);
}

fa8_status fa8_decode_attention_noalloc(const void* q, int32_t batch, int32_t num_q_heads,
                                        const void* cache, int32_t cache_dtype,
                                        int64_t num_blocks, int32_t num_kv_heads,
                                        int32_t head_dim, const int32_t* block_table,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                        int32_t max_seq_len, const float* k_scale,
                                        const float* v_scale, float sm_scale, int32_t window,
                                        int32_t num_splits, float* out, void* stream) {
  return decode_impl(q, batch, num_q_heads, cache, cache_dtype, num_blocks, num_kv_heads,
                     head_dim, block_table, max_blocks_per_seq, seq_lens, max_seq_len, k_scale,
                     v_scale, sm_scale, window, num_splits, out, nullptr, 0, stream, nullptr,
                     nullptr, FA8_F32, true);
}

fa8_status fa8_decode_attention_append(const void* q, const void* k_new, const void* v_new,
                                       int32_t in_dtype, int32_t batch, int32_t num_q_heads,
                                       void* cache, int32_t cache_dtype, int64_t num_blocks,
                                       int32_t num_kv_heads, int32_t head_dim,
                                       const int32_t* block_table, int32_t max_blocks_per_seq,
                                       const int32_t* seq_lens, int32_t max_seq_len,
                                       const float* k_scale, const float* v_scale,
                                       float sm_scale, int32_t window, int32_t num_splits,
                                       float* out, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  if (in_dtype != FA8_F32 && in_dtype != FA8_BF16)
    return fail(FA8_EINVAL, "decode_append: in_dtype must be FA8_F32 or FA8_BF16");
  if (batch > 0 && (!k_new || !v_new))
    return fail(FA8_EINVAL, "decode_append: null k_new or v_new");
  return decode_impl(q, batch, num_q_heads, cache, cache_dtype, num_blocks, num_kv_heads,
                     head_dim, block_table, max_blocks_per_seq, seq_lens, max_seq_len, k_scale,
                     v_scale, sm_scale, window, num_splits, out, workspace, workspace_bytes,
                     stream, k_new, v_new, in_dtype);
}

int32_t fa8_prefill_kv_tile(int32_t head_dim) {
  if (!head_dim_ok(head_dim)) return 0;
  return fa8::prefill_kv_tile(head_dim);
}

fa8_status fa8_prefill_attention(const void* q, const int32_t* cu_q_lens, int32_t batch,
                                 int32_t num_q_heads, int32_t max_q_len, const void* cache,
                                 int32_t cache_dtype, int64_t num_blocks,
                                 int32_t num_kv_heads, int32_t head_dim,
                                 const int32_t* block_table, int32_t max_blocks_per_seq,
                                 const int32_t* seq_lens, const float* q_scale,
                                 const float* k_scale, const float* v_scale, float sm_scale,
                                 int32_t window, int32_t accum_mode, float* out,
                                 void* stream) {
  if (batch < 0 || max_q_len < 0 || num_blocks < 0 || max_blocks_per_seq < 0)
    return fail(FA8_EINVAL, "prefill: negative size");
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(FA8_EINVAL, "prefill: head counts must be > 0");
  if (num_q_heads % num_kv_heads != 0)
    return fail(FA8_EINVAL, "prefill: num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (batch > kMaxGridYZ || num_q_heads > kMaxGridYZ)
    return fail(FA8_EUNSUPPORTED, "prefill: batch and num_q_heads must be <= %d", kMaxGridYZ);
  if (!head_dim_ok(head_dim))
    return fail(FA8_EUNSUPPORTED, "prefill: head_dim %d not in {64,128,256}", head_dim);
  if (!fp8_cache(cache_dtype))
    return fail(FA8_EINVAL, "prefill: cache_dtype must be FA8_E4M3 or FA8_E5M2");
  if (accum_mode < 0 || accum_mode > 65536)
    return fail(FA8_EINVAL, "prefill: accum_mode must be in 0..65536");
  if (!(std::isfinite(sm_scale)))
    return fail(FA8_EINVAL, "prefill: sm_scale must be finite");
  if (batch == 0 || max_q_len == 0) return ok();
  if (!q || !cu_q_lens || !cache || !block_table || !seq_lens || !q_scale || !k_scale ||
      !v_scale || !out)
    return fail(FA8_EINVAL, "prefill: null pointer argument");

  fa8::PrefillParams p{};
  p.q = reinterpret_cast<const uint16_t*>(q);
  p.cu_q_lens = cu_q_lens;
  p.cache = reinterpret_cast<const uint8_t*>(cache);
  p.block_table = block_table;
  p.seq_lens = seq_lens;
  p.q_scale = q_scale;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.out = out;
  p.batch = batch;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.max_blocks = max_blocks_per_seq;
  p.max_q_len = max_q_len;
  p.window = window > 0 ? window : 0;
  p.accum_mode = accum_mode;
  p.fmt = kernel_fmt(cache_dtype);
  p.sm_scale = sm_scale;
  const hipError_t e = fa8::launch_prefill(p, reinterpret_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(FA8_EUNSUPPORTED, "prefill: configuration not built");
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

fa8_status fa8_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes % 16 != 0) return fail(FA8_EINVAL, "stream_read: bytes must be a multiple of 16");
  if (bytes == 0) return ok();
  if (!src || !sink) return fail(FA8_EINVAL, "stream_read: null pointer argument");
  const hipError_t e = fa8::launch_stream_read(src, bytes, sink, device_cu_count(),
                                               reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream_read launch");
  return ok();
}

fa8_status fa8_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes % 16 != 0) return fail(FA8_EINVAL, "stream_copy: bytes must be a multiple of 16");
  if (bytes == 0) return ok();
  if (!src || !dst) return fail(FA8_EINVAL, "stream_copy: null pointer argument");
  const hipError_t e = fa8::launch_stream_copy(dst, src, bytes, device_cu_count(),
                                               reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream_copy launch");
  return ok();
}

}  // extern "C"
