// Internal helpers shared by the HIP sources of libmoe (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------- errors
// Thread-local message of the last non-OK status (moe_last_error()).
void set_error(const std::string& msg);
void clear_error();

#define MOE_CHECK_ARG(cond, ...)                                   \
  do {                                                             \
    if (!(cond)) {                                                 \
      ::moe::set_error(std::string(__func__) + ": " + (__VA_ARGS__)); \
      return MOE_ERR_INVALID;                                      \
    }                                                              \
  } while (0)

#define MOE_CHECK_HIP(expr)                                                   \
  do {                                                                        \
    hipError_t e_ = (expr);                                                   \
    if (e_ != hipSuccess) {                                                   \
      ::moe::set_error(std::string(__func__) + ": " + #expr + ": " +         \
                       hipGetErrorString(e_));                               \
      return MOE_ERR_HIP;                                                     \
    }                                                                         \
  } while (0)

// Launch check: catches configuration errors reported at launch time.
#define MOE_CHECK_LAUNCH() MOE_CHECK_HIP(hipGetLastError())

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Check-only mode of the calling thread: while a CheckOnly object lives,
// every entry point validates its arguments and returns MOE_OK (or the
// error) without launching or recording anything.  moe_layer_forward uses it
// to check all four stages before the first launch.
bool check_only();
struct CheckOnly {
  CheckOnly();
  ~CheckOnly();
};

// Device properties of the current device (cached per device).
struct DeviceInfo {
  int cus;
  int lds_bytes;
};
DeviceInfo device_info();

// Allows `kernel` `bytes` of dynamic LDS on the current device; the attribute
// is set again only when a call asks for more than before on that device,
// and the call is thread-safe.
hipError_t set_dynamic_lds(const void* kernel, int bytes);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- numbers
using bf16_t = uint16_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16 bytes in registers

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even; NaN stays NaN (quiet bit forced).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16 with the hardware conversion (round to nearest
// even, like f32_to_bf16 for finite values).
__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
  const bf16x2_hw v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// OCP e4m3fn byte -> fp32, exact.  Placing the 7 exponent+mantissa bits at
// bit 20 makes an fp32 with exponent field e and mantissa m<<20, i.e.
// 2^(e-127)(1+m/8) (or m*2^-129 for e == 0); scaling by 2^120 gives the
// e4m3 value 2^(e-7)(1+m/8) (or the subnormal m*2^-9).  fp32 denormals are
// kept (HIP default), so the e == 0 case is exact too.
__device__ __forceinline__ float e4m3_to_f32(uint32_t q) {
  float mag = __uint_as_float((q & 0x7fu) << 20) * 0x1p120f;
  return __uint_as_float(__float_as_uint(mag) | ((q & 0x80u) << 24));
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would drain register
// prefetches issued just before it; here only the LDS counter is drained.
// The "memory" clobber keeps the compiler from moving memory accesses across.
#define MOE_BARRIER_LDS() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
