// Decode attention for callers that cannot allocate device memory (code under HIP graph capture,
// serving loops and harnesses that forbid hipMalloc): the split partials live in a workspace of
// static device memory that the library holds, one copy per GPU for the life of the process.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

namespace {

constexpr int MAX_DEVICES = 64;

// The workspace.  Its name is a host-side stand-in in host code, never a device address: every use on
// the host goes through the per-device address hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[KVQ_STATIC_WS_BYTES];

std::mutex g_mu;
void* g_addr[MAX_DEVICES];  // device address of `scratch` on each device (nullptr: not taken yet)

// Address of `scratch` on the current device, taken once per device with that device current.
kvq_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return kvq::set_error(KVQ_EDEVICE, "hipGetDevice failed");
  if (dev < 0 || dev >= MAX_DEVICES) return kvq::set_error(KVQ_EDEVICE, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return kvq::set_error(KVQ_EDEVICE, "hipGetSymbolAddress of the static workspace failed");
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return KVQ_OK;
}

}  // namespace

namespace kvq {

kvq_status static_ws_prepare() {
  void* p = nullptr;
  return scratch_address(&p);
}

}  // namespace kvq

extern "C" kvq_status kvq_decode_attn_nomalloc(kvq_cache* c, int32_t layer, const void* q, float* out, float scale,
                                               void* stream) {
  void* ws = nullptr;
  kvq_status st = scratch_address(&ws);
  if (st != KVQ_OK) return st;
  return kvq::decode_attn_ws(c, layer, q, out, scale, ws, KVQ_STATIC_WS_BYTES, stream);
}
