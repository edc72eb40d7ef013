// Layer forward that allocates nothing: its workspace is a static device
// array of the library instead of a caller buffer.  For callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
#include <mutex>
#include <vector>

#include "common.h"

namespace moe {

// The workspace of moe_layer_forward_noalloc: every GPU the library runs on
// holds its own copy until the process ends.  No kernel needs any of it to
// start at zero (each writes the scratch it later reads), so it is never
// cleared.  In host code this name is only a host-side stand-in: kernels get
// the device address from scratch_address().
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_layer_forward_noalloc(const moe_layer_args* a, hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, "null args");
  const size_t need = moe_workspace_bytes(a);
  if (need > MOE_STATIC_SCRATCH_BYTES) {
    set_error("moe_layer_forward_noalloc: the layer needs " + std::to_string(need) +
              " bytes of workspace, more than the static scratch of " +
              std::to_string((size_t)MOE_STATIC_SCRATCH_BYTES) +
              " bytes; use moe_layer_forward with a caller workspace");
    return MOE_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  MOE_CHECK_HIP(scratch_address(&ws));
  return moe_layer_forward(a, ws, MOE_STATIC_SCRATCH_BYTES, stream);
}
