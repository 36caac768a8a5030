// streamed_linear_fwd_noalloc: the fused NF4 forward with its scratch (the
// packed activation and the fp32 partials of a split contraction) in a
// file-scope device array instead of a caller workspace, for callers that
// cannot allocate device memory.
//
// The array is one per GPU (every device the library is loaded on holds it
// until the process ends). Host code never passes the array's name to a
// kernel: its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what the
// kernels receive. Every call on a GPU shares the array and leaves it holding
// the last call's partials; nothing in it has to start at zero (the packed
// activation and every partial are written before they are read). Calls that
// overlap on one GPU (different streams, or host threads) race on it.
#include <mutex>

#include "common.h"

namespace {

constexpr size_t kScratchBytes = NF4S_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch is handed out in 256-byte units");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nf4s::set_error(NF4S_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return nf4s::set_error(NF4S_EHIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return nf4s::set_error(NF4S_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return NF4S_OK;
}

}  // namespace

extern "C" int streamed_linear_fwd_noalloc(const void* shard_dev, const nf4s_tensor_desc* d,
                                           const uint16_t* x, int64_t M, uint16_t* y,
                                           const float* lora_u, const float* lora_B, int r,
                                           float scale, void* stream) {
  if (!d) return nf4s::set_error(NF4S_EINVAL, "descriptor is NULL");
  size_t need = 0;
  int rc = nf4s_workspace_bytes(NF4S_OP_LINEAR_FWD, M, d->n_out, d->k_in, &need);
  if (rc) return rc;
  if (need > kScratchBytes)
    return nf4s::set_error(NF4S_EWORKSPACE,
                           "M=%lld, %lld x %lld needs %zu bytes of scratch; the library holds %zu "
                           "(call streamed_linear_fwd with a workspace)",
                           (long long)M, (long long)d->n_out, (long long)d->k_in, need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_on_current_device(&ws))) return rc;
  return streamed_linear_fwd(shard_dev, d, x, M, y, lora_u, lora_B, r, scale, ws, kScratchBytes, stream);
}
