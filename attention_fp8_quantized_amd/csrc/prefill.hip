// FP8 prefill (placeholder until the MFMA kernel lands).
#include "fa8_device.hpp"
#include "fa8_internal.hpp"

namespace fa8 {

int prefill_kv_tile(int head_dim) { return head_dim == 256 ? 64 : 64; }

hipError_t launch_prefill(const PrefillParams&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa8
