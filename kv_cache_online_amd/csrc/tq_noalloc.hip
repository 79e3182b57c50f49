// Decode attention for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// the same kernels as tq_decode_attention, with the workspace taken from a
// fixed array inside the library instead of from the caller.
//
// The array lives in device memory from the time the library's code is loaded
// on a device until the process ends, one copy per device.  Its address is
// looked up once per device (hipGetSymbolAddress, with that device current) and
// kept; host code never passes the array's own name to a kernel, since on the
// host that name is not a device address.  Every call on a device shares that
// device's array and leaves its last contents there: calls that overlap on one
// device (different streams, different threads) race.  The decode reads only
// what it has written into its workspace in the same call, so nothing needs
// clearing between calls.

#include <hip/hip_runtime.h>

#include <atomic>

#include "tq_common.h"

namespace {

static __device__ __align__(256) unsigned char scratch[TQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];

// Device address of this device's scratch array, looked up on the first call on
// the device and kept (a lookup that fails is retried on the next call).
void *scratch_address(int dev) {
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  void *q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" int tq_decode_attention_noalloc(const tq_config *cfg, const void *q, tq_dtype dt, int32_t batch,
                                           const int64_t *seq_start, const int32_t *seq_len, int32_t max_len,
                                           const tq_cache *kc, const tq_cache *vc, float sm_scale, float *out,
                                           uint32_t *status, hipStream_t stream) {
  if (!cfg || batch < 0 || max_len < 0) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  const size_t need = tq_decode_workspace_bytes(cfg, batch, max_len);
  if (need == 0) return TQ_ERR_INVALID_ARG;
  if (need > TQ_NOALLOC_SCRATCH_BYTES) return TQ_ERR_WORKSPACE;  // beyond the fixed scratch
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_LAUNCH;
  void *ws = scratch_address(dev);
  if (!ws) return TQ_ERR_LAUNCH;
  return tq_decode_attention(cfg, q, dt, batch, seq_start, seq_len, max_len, kc, vc, sm_scale, out, status, ws,
                             TQ_NOALLOC_SCRATCH_BYTES, stream);
}
