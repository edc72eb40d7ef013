// Combine: un-permute, router-weighted sum and residual (gfx950).
//
// Each token's expert outputs come back to where the token started; each is
// scaled by the token's router weight for that expert and the results are
// added (Ultralytics glossary "Expert Parallelism", "How Tokens Move Between
// GPUs", step 4).  A token that lost its expert slots to the capacity limit
// leaves the layer as its residual input, untouched ("Load Balancing and
// Capacity", paragraph after the bullets; ai360xpert "Load Balancing and
// Dropped Tokens").
//
// One wave per token, 128-bit loads and stores over the row.  The sum is
// accumulated in fp32 starting from x (and the shared-expert output), adding
// only kept, executed assignments, then rounded once; a token with nothing
// to add is therefore written back as exactly x.  HBM-bound: per token it
// reads x, the shared output and up to k expert rows, and writes y.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// The layer output is written once and not read back here: nontemporal
// stores (measured: Switch combine 44 -> 41 us, DeepSeek-V3 share 75 -> 70 us).
__device__ __forceinline__ void store_y(uint4* dst, const uint4& v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(dst));
}

template <typename T>
struct Row16;

template <>
struct Row16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void to_f32(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 from_f32(const float* f) {
    return uint4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};

template <>
struct Row16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void to_f32(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static uint4 from_f32(const float* f) {
    return uint4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                 pack_bf16x2(f[6], f[7])};
  }
};

template <typename ET, int UNROLL, int WPT>
__global__ void __launch_bounds__(kThreads) combine_kernel(
    const uint4* __restrict__ x, const uint4* __restrict__ shared_out,
    const uint4* __restrict__ y_send, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ slot, const float* __restrict__ weights, uint4* __restrict__ y,
    int64_t T, int k, int e_begin, int e_end, int row16) {
  constexpr int N = Row16<ET>::N;
  const int lane = lane_id();
  // WPT waves share one token's row (decode-sized batches); the row's 16-byte
  // pieces are dealt round-robin over their 64*WPT lanes.
  const int64_t slots = (int64_t)gridDim.x * (kThreads / 64);
  const int64_t wid = (int64_t)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int sub = (int)(wid % WPT);
  for (int64_t t = wid / WPT; t < T; t += slots / WPT) {
    int sj[MOE_MAX_TOPK];  // -1: nothing to add for choice j
    float wj[MOE_MAX_TOPK];
    bool any = false;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      sj[j] = -1;
      wj[j] = 0.f;
      if (j < k) {
        const int s = slot[t * k + j];
        const int e = ids[t * k + j];
        if (s >= 0 && e >= e_begin && e < e_end) {
          sj[j] = s;
          wj[j] = weights[t * k + j];
          any = true;
        }
      }
    }
    const uint4* xr = x + t * row16;
    const uint4* sr = shared_out ? shared_out + t * row16 : nullptr;
    uint4* yr = y + t * row16;
    constexpr int STRIDE = 64 * WPT;
    for (int c0 = sub * 64 + lane; c0 < row16; c0 += STRIDE * UNROLL) {
      uint4 xv[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int c = c0 + u * STRIDE;
        xv[u] = (c < row16) ? xr[c] : uint4{0, 0, 0, 0};
      }
      if (!any && !sr) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int c = c0 + u * STRIDE;
          if (c < row16) store_y(yr + c, xv[u]);
        }
        continue;
      }
      float acc[UNROLL][N];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) Row16<ET>::to_f32(xv[u], acc[u]);
      if (sr) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int c = c0 + u * STRIDE;
          if (c < row16) {
            float f[N];
            Row16<ET>::to_f32(sr[c], f);
#pragma unroll
            for (int i = 0; i < N; ++i) acc[u][i] += f[i];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (sj[j] < 0) continue;
        const uint4* er = y_send + (int64_t)sj[j] * row16;
        const float w = wj[j];
        uint4 ev[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int c = c0 + u * STRIDE;
          ev[u] = (c < row16) ? er[c] : uint4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          float f[N];
          Row16<ET>::to_f32(ev[u], f);
#pragma unroll
          for (int i = 0; i < N; ++i) acc[u][i] = fmaf(w, f[i], acc[u][i]);
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int c = c0 + u * STRIDE;
        if (c < row16) store_y(yr + c, Row16<ET>::from_f32(acc[u]));
      }
    }
  }
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine(const moe_combine_args* a, hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, "null args");
  MOE_CHECK_ARG(a->T >= 0, "T < 0");
  MOE_CHECK_ARG(a->k >= 1 && a->k <= MOE_MAX_TOPK, "k out of range [1, 8]");
  MOE_CHECK_ARG(a->e_begin <= a->e_end, "e_begin > e_end");
  MOE_CHECK_ARG(a->act_dtype == MOE_F32 || a->act_dtype == MOE_BF16, "bad act_dtype");
  const int es = a->act_dtype == MOE_F32 ? 4 : 2;
  MOE_CHECK_ARG(a->d >= 1 && ((int64_t)a->d * es) % 16 == 0, "row must be a multiple of 16 bytes");
  if (a->T == 0) return MOE_OK;
  MOE_CHECK_ARG(a->x && a->y && a->ids && a->slot && a->weights, "null data pointer");
  MOE_CHECK_ARG(a->y_send || a->e_begin == a->e_end, "y_send is required");
  MOE_CHECK_ARG(aligned16(a->x) && aligned16(a->y) && (!a->y_send || aligned16(a->y_send)) &&
                    (!a->shared_out || aligned16(a->shared_out)),
                "rows not 16-byte aligned");
  MOE_CHECK_ARG(a->x != a->y, "y may not alias x");
  if (check_only()) return MOE_OK;
  const int row16 = (int)((int64_t)a->d * es / 16);
  // decode-sized batches: a workgroup per token so every load is in flight at once
  const bool wide = a->T < 4 * (int64_t)device_info().cus;
  const int64_t want = wide ? a->T : (a->T + 3) / 4;
  const int64_t cap = (int64_t)device_info().cus * 16;
  const int grid = (int)(want < cap ? want : cap);
  if (a->act_dtype == MOE_F32) {
    if (wide)
      combine_kernel<float, 2, 4><<<grid, kThreads, 0, stream>>>(
          (const uint4*)a->x, (const uint4*)a->shared_out, (const uint4*)a->y_send, a->ids, a->slot,
          a->weights, (uint4*)a->y, a->T, a->k, a->e_begin, a->e_end, row16);
    else
      combine_kernel<float, 4, 1><<<grid, kThreads, 0, stream>>>(
          (const uint4*)a->x, (const uint4*)a->shared_out, (const uint4*)a->y_send, a->ids, a->slot,
          a->weights, (uint4*)a->y, a->T, a->k, a->e_begin, a->e_end, row16);
  } else {
    if (wide)
      combine_kernel<bf16_t, 2, 4><<<grid, kThreads, 0, stream>>>(
          (const uint4*)a->x, (const uint4*)a->shared_out, (const uint4*)a->y_send, a->ids, a->slot,
          a->weights, (uint4*)a->y, a->T, a->k, a->e_begin, a->e_end, row16);
    else
      combine_kernel<bf16_t, 4, 1><<<grid, kThreads, 0, stream>>>(
          (const uint4*)a->x, (const uint4*)a->shared_out, (const uint4*)a->y_send, a->ids, a->slot,
          a->weights, (uint4*)a->y, a->T, a->k, a->e_begin, a->e_end, row16);
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
