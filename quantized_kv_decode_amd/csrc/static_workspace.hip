// Fixed per-GPU workspace of loopkv_decode_attention_static, the decode entry point for callers
// that cannot allocate device memory: the split merge counters and split partials of a call live
// in this array instead of the plan's arena. Each GPU the library runs on holds its own copy
// until the process ends. Host code never passes the array's name to a kernel or a copy (on the
// host it is only a stand-in for the symbol); it uses the device address looked up here.
#include <mutex>

#include "loopkv_internal.h"

namespace loopkv {
namespace {

static __device__ __align__(256) uint8_t scratch[kStaticWsBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};   // device address of `scratch` per device, once looked up

}  // namespace

void* static_workspace(int device, hipStream_t stream) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_addr[device]) return g_addr[device];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  // the counters must start at zero; every decode leaves them at zero again
  if (hipMemsetAsync(ptr, 0, kStaticWsCounterBytes, stream) != hipSuccess) return nullptr;
  if (hipStreamSynchronize(stream) != hipSuccess) return nullptr;
  g_addr[device] = ptr;
  return ptr;
}

}  // namespace loopkv
