// Host side of libmoe: error state, device properties, capacity, the
// whole-layer entry point and its workspace.
#include <string.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "common.h"

namespace moe {

namespace {
thread_local std::string g_last_error;
thread_local bool g_check_only = false;
}

bool check_only() { return g_check_only; }
CheckOnly::CheckOnly() { g_check_only = true; }
CheckOnly::~CheckOnly() { g_check_only = false; }

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }

DeviceInfo device_info() {
  static std::mutex mu;
  static std::vector<DeviceInfo> cache;
  static std::vector<bool> have;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) {
    cache.resize(dev + 1);
    have.resize(dev + 1, false);
  }
  if (!have[dev]) {
    DeviceInfo info{256, 160 * 1024};
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      info.cus = v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0)
      info.lds_bytes = v;
    cache[dev] = info;
    have[dev] = true;
  }
  return cache[dev];
}

hipError_t set_dynamic_lds(const void* kernel, int bytes) {
  // the largest size set so far per (device, kernel): a kernel whose LDS
  // depends on its arguments (the router's on E) is raised when a call
  // needs more than any before it
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find({dev, kernel});
  if (it != done.end() && it->second >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done[{dev, kernel}] = bytes;
  return e;
}

moe_status expert_ffn_impl(const moe_ffn_args* a, void* ws, size_t ws_bytes, hipStream_t stream,
                           hipEvent_t mid_event);

}  // namespace moe

using namespace moe;

extern "C" const char* moe_last_error(void) { return g_last_error.c_str(); }

// ceil(cf * T * k / E) exactly: cf = m * 2^ex with an integer mantissa m, so
// the quotient is a ratio of integers evaluated in 128-bit arithmetic.
extern "C" int32_t moe_capacity(int64_t T, int32_t k, int32_t E, double cf) {
  if (!(cf > 0.0) || E <= 0 || T < 0 || k <= 0) return INT32_MAX;
  int ex = 0;
  const double fr = frexp(cf, &ex);                // cf = fr * 2^ex, fr in [0.5, 1)
  const int64_t m = (int64_t)ldexp(fr, 53);        // exact 53-bit integer
  ex -= 53;                                        // cf = m * 2^ex
  unsigned __int128 num = (unsigned __int128)m * (unsigned __int128)T * (unsigned __int128)k;
  unsigned __int128 den = (unsigned __int128)E;
  if (ex >= 0) {
    if (ex > 60) return INT32_MAX;
    const unsigned __int128 big = num << ex;
    if ((big >> ex) != num) return INT32_MAX;
    num = big;
  } else {
    if (-ex > 100) {
      // cf is tiny: ceil of a positive value below 1 (T*k > 0) is 1
      return (T > 0) ? 1 : 0;
    }
    den <<= -ex;
  }
  unsigned __int128 q = num / den;
  if (num % den) q += 1;
  if (q > (unsigned __int128)INT32_MAX) return INT32_MAX;
  return (int32_t)q;
}

extern "C" size_t moe_workspace_bytes(const moe_layer_args* a) {
  if (!a) return 0;
  size_t w = moe_route_workspace_bytes(&a->route);
  const size_t d = moe_dispatch_workspace_bytes(&a->dispatch);
  const size_t f = moe_ffn_workspace_bytes(&a->ffn);
  if (d > w) w = d;
  if (f > w) w = f;
  return w;
}

extern "C" moe_status moe_layer_forward(const moe_layer_args* a, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, "null args");
  const size_t need = moe_workspace_bytes(a);
  if (ws_bytes < need || (need && !ws)) {
    set_error("moe_layer_forward: workspace too small");
    return MOE_ERR_WORKSPACE;
  }
  // every block's arguments and the wiring between them, before any launch
  {
    const CheckOnly guard;
    moe_status st = moe_route(&a->route, ws, ws_bytes, stream);
    if (st == MOE_OK) st = moe_dispatch(&a->dispatch, ws, ws_bytes, stream);
    if (st == MOE_OK) st = expert_ffn_impl(&a->ffn, ws, ws_bytes, stream, nullptr);
    if (st == MOE_OK) st = moe_combine(&a->combine, stream);
    if (st != MOE_OK) return st;
  }
  clear_error();
  const moe_route_args& r = a->route;
  const moe_dispatch_args& ds = a->dispatch;
  const moe_ffn_args& f = a->ffn;
  const moe_combine_args& c = a->combine;
  MOE_CHECK_ARG(r.T == ds.T && r.T == c.T, "route, dispatch and combine need the same T");
  MOE_CHECK_ARG(r.k == ds.k && r.k == c.k, "route, dispatch and combine need the same k");
  MOE_CHECK_ARG(r.E == ds.E && r.E == f.E, "route, dispatch and ffn need the same E");
  MOE_CHECK_ARG(ds.d == f.d && ds.d == c.d && (r.x == nullptr || r.d == ds.d),
                "all stages need the same d");
  MOE_CHECK_ARG(r.act_dtype == ds.act_dtype && r.act_dtype == f.act_dtype &&
                    r.act_dtype == c.act_dtype,
                "all stages need the same act_dtype");
  MOE_CHECK_ARG(ds.ids == r.ids && c.ids == r.ids && c.weights == r.weights && c.slot == ds.slot,
                "ids, weights and slot must be the buffers route and dispatch write");
  MOE_CHECK_ARG(c.e_begin == f.e_begin && c.e_end == f.e_end,
                "ffn and combine need the same executed experts");
  MOE_CHECK_ARG(f.e_begin == f.e_end || (f.x_send == ds.x_send && f.expert_off == ds.expert_off &&
                                         c.y_send == f.y_send),
                "x_send, expert_off and y_send must be wired between the stages");
  const bool dense = f.x_dense != nullptr && f.T_dense > 0;
  MOE_CHECK_ARG(!dense || (f.x_dense == ds.x && f.T_dense == r.T && c.shared_out == f.y_dense),
                "the shared expert runs over the layer's x and feeds combine's shared_out");
  hipEvent_t* ev = a->events;
  if (ev && ev[0]) MOE_CHECK_HIP(hipEventRecord(ev[0], stream));
  moe_status st = moe_route(&a->route, ws, ws_bytes, stream);
  if (st != MOE_OK) return st;
  if (ev && ev[1]) MOE_CHECK_HIP(hipEventRecord(ev[1], stream));
  st = moe_dispatch(&a->dispatch, ws, ws_bytes, stream);
  if (st != MOE_OK) return st;
  if (ev && ev[2]) MOE_CHECK_HIP(hipEventRecord(ev[2], stream));
  st = expert_ffn_impl(&a->ffn, ws, ws_bytes, stream, ev ? ev[3] : nullptr);
  if (st != MOE_OK) return st;
  if (ev && ev[4]) MOE_CHECK_HIP(hipEventRecord(ev[4], stream));
  st = moe_combine(&a->combine, stream);
  if (st != MOE_OK) return st;
  if (ev && ev[5]) MOE_CHECK_HIP(hipEventRecord(ev[5], stream));
  return MOE_OK;
}
