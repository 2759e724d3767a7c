// moe_decode_layer_noalloc: single-token decode for callers that cannot
// allocate (code under HIP graph capture, tight serving loops).  The
// decode's scratch (router logits and the k experts' SwiGLU outputs) lives in
// the file-scope device array `scratch` below instead of a caller buffer:
// each GPU the library runs on holds its own copy until the process ends.
// Its device address is looked up once per device, with that device current,
// and that address -- never the array's host-side name -- is what the kernels
// are given.
#include <hip/hip_runtime.h>

#include <atomic>

#include "rl_common.h"
#include "rl_kernels.h"
#include "rl_moe.h"

namespace {

constexpr int64_t kScratchBytes = RL_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (nullptr on failure).
// Concurrent first calls on one device look up and store the same address.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
    (void)hipGetLastError();   // the failed lookup must not surface at the caller's next call
    return nullptr;
  }
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" int moe_decode_layer_noalloc(const rl_moe_desc* d, int32_t layer, const float* x,
                                        const float* router_w, const float* router_bias,
                                        const int32_t* residency, const void* slot_pool,
                                        const rl_route_out* route, float* y, void* stream) {
  // every check runs before the first device call; the scratch argument of
  // the common checks is a stand-in that is aligned and not NULL
  const int rc = rl::decode_layer_check(d, layer, x, router_w, residency, slot_pool, route,
                                        reinterpret_cast<const void*>(uintptr_t(256)), y);
  if (rc) return rc;
  const int64_t need = rl_decode_scratch_bytes(d);
  if (need < 0) return int(need);
  if (need > kScratchBytes) return RL_E_SCRATCH;
  void* s = device_scratch();
  if (!s) return RL_E_DEVICE;
  return moe_decode_layer(d, layer, x, router_w, router_bias, residency, slot_pool, route, s,
                          kScratchBytes, y, stream);
}
