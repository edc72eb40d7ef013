// Route: router logits, scores and top-k (gfx950).
//
// Ultralytics glossary "Expert Parallelism", "How Tokens Move Between GPUs",
// step 1: a linear layer produces one score per (token, expert) pair and
// each token goes to its k highest-scoring experts.  The score function, weight renormalisation and
// tie order are not on the pages: softmax or sigmoid, optional
// renormalisation over the selected experts, ties to the lower expert index.
// The selection-only bias follows "Load Balancing and Capacity" (bias-based
// balancing bullet): it enters the selection key and nothing else.
//
// Kernels
//   route_mfma_kernel  : bf16, E <= 32, many tokens.  Logits on the matrix
//                        cores (x by DMA through per-wave LDS rings), top-k
//                        and weights fused.  Measured on the prefill workload
//                        (E = 8, d = 4096): 31 us cache-cold, against 70 us for the
//                        VALU kernel below, whose FMAs and bf16 widening
//                        limited it well below the HBM rate.
//   route_small_kernel : E <= 8 and W_r fits in LDS (fp32, or few tokens).
//                        One pass over x with W_r staged in LDS, fp32 VALU
//                        dot products, wave butterfly reduction, top-k and
//                        weights fused.
//   logits_valu_kernel : any E, W_r read through L2; writes fp32 logits.
//   topk_kernel        : one wave per token over fp32 logits in memory,
//                        E <= 256; wavefront-shuffle arg-max k times.
// Large E (E % 64 == 0, bf16) computes the logits with the bf16 MFMA GEMM of
// the expert FFN (router intensity 2E/s_a is 64-256 flop/B there, above the
// VALU ridge), then runs topk_kernel.
#include <algorithm>

#include "common.h"
#include "gemm.h"
#include "gemm_common.h"

namespace moe {
namespace {

constexpr int kWave = 64;

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ bool key_better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Order-preserving image of a selection key: a larger key gives a larger
// image (-0 counts as +0; NaN sorts below every number).
__device__ __forceinline__ uint32_t key_image(float f) {
  if (f != f) return 1u;
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One DPP move of both halves of a 64-bit value; rows outside ROW_MASK keep v.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = (int)(uint32_t)v, hi = (int)(uint32_t)(v >> 32);
  const uint32_t nlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false);
  const uint32_t nhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false);
  return ((uint64_t)nhi << 32) | nlo;
}

// Maximum over the 64 lanes, returned to every lane: within each quad
// (quad_perm 1032, 2301), each row (half-row and row mirrors), then across
// rows (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows 2 and 3),
// which leaves the maximum in lane 63.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xb1, 0xf>(v);   v = o > v ? o : v;
  o = dpp_u64<0x4e, 0xf>(v);   v = o > v ? o : v;
  o = dpp_u64<0x141, 0xf>(v);  v = o > v ? o : v;
  o = dpp_u64<0x140, 0xf>(v);  v = o > v ? o : v;
  o = dpp_u64<0x142, 0xa>(v);  v = o > v ? o : v;
  o = dpp_u64<0x143, 0xc>(v);  v = o > v ? o : v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Top-k selection rounds reduce packed (key, index) values with DPP row
// moves (measured against three shuffles per butterfly step: DeepSeek-V3
// share route 76 -> 68 us, Switch 38 -> 35.5 us).

// fp32 of sigmoid evaluated in double: the selection key precision.
__device__ __forceinline__ float sigmoid_f32_via_f64(float x) {
  return (float)(1.0 / (1.0 + exp(-(double)x)));
}

template <typename T>
struct Vec16;  // 16 bytes of T, widened to floats

template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void widen(u32x4 v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
  }
  __device__ __forceinline__ static void load(const void* p, float* out) {
    widen(*reinterpret_cast<const u32x4*>(p), out);
  }
};

template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(u32x4 v, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v[i] << 16);
      out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
  __device__ __forceinline__ static void load(const void* p, float* out) {
    widen(*reinterpret_cast<const u32x4*>(p), out);
  }
};

// Scores, top-k and weights of one token from its E (<= 8) final logits.
template <int EMAX>
__device__ void finish_token_small(const float* L, int E, int k, int score, int renorm,
                                   const float* __restrict__ b_select, int64_t t,
                                   int32_t* __restrict__ ids, float* __restrict__ weights) {
  float key[EMAX];
  float sc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (e < E) {
      if (score == MOE_SIGMOID) {
        sc[e] = sigmoid_f32_via_f64(L[e]);
        key[e] = b_select ? sc[e] + b_select[e] : sc[e];
      } else {
        key[e] = L[e];
      }
    } else {
      key[e] = -INFINITY;
    }
  }
  bool taken[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) taken[e] = false;
  int sel[MOE_MAX_TOPK];
  for (int j = 0; j < k; ++j) {
    int best = -1;
    float bk = 0.f;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e < E && !taken[e] && (best < 0 || key_better(key[e], e, bk, best))) {
        best = e;
        bk = key[e];
      }
    }
#pragma unroll
    for (int e = 0; e < EMAX; ++e) taken[e] = taken[e] || (e == best);
    sel[j] = best;
  }
  // weights
  float wsel[MOE_MAX_TOPK];
  float denom = 0.f;
  if (score == MOE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) m = fmaxf(m, L[e]);
    float all = 0.f;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (e < E) all += __expf(L[e] - m);
    for (int j = 0; j < k; ++j) {
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e == sel[j]) v = L[e];
      wsel[j] = __expf(v - m);
      denom += wsel[j];
    }
    if (!renorm) denom = all;
  } else {
    for (int j = 0; j < k; ++j) {
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (e == sel[j]) v = sc[e];
      wsel[j] = v;
      denom += v;
    }
    if (!renorm) denom = 1.f;
  }
  const float inv = 1.f / denom;
  for (int j = 0; j < k; ++j) {
    ids[t * k + j] = sel[j];
    weights[t * k + j] = wsel[j] * inv;
  }
}

// ---------------------------------------------------------------- E <= 8 fused
constexpr int kRsTpw = 4;  // tokens per wave in flight
// Block = 4 waves; each wave owns TPW tokens at a time.  Lane l covers the
// 16-byte chunks l, l+64, ... of a row (coalesced 128-bit loads of x).
template <typename T, int TPW, bool WR_LDS>
__global__ void __launch_bounds__(256) route_small_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ b_router,
    const float* __restrict__ b_select, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ weights, int64_t T_tok, int d, int E, int k, int score, int renorm) {
  constexpr int EMAX = 8;
  constexpr int VN = Vec16<T>::N;  // elements per 16 B
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const T* sw = wr;  // [E][d]: LDS copy when staged, else read through L2
  if constexpr (WR_LDS) {
    T* dst = reinterpret_cast<T*>(smem_raw);
    const int n16 = E * d / VN;
    const uint4* g = reinterpret_cast<const uint4*>(wr);
    uint4* s = reinterpret_cast<uint4*>(dst);
    for (int i = threadIdx.x; i < n16; i += blockDim.x) s[i] = g[i];
    __syncthreads();
    sw = dst;
  }
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int nchunk = d / VN;  // 16-byte chunks per row
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t t0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave) * TPW; t0 < T_tok;
       t0 += waves_total * TPW) {
    float acc[TPW][EMAX];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int e = 0; e < EMAX; ++e) acc[i][e] = 0.f;
    // x chunks are fetched one step ahead (clamped index, so the loads are
    // unconditional): the next chunk is in flight while this one is used.
    u32x4 nxt[TPW];
    auto fetch = [&](int c_) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int64_t t = min(t0 + i, T_tok - 1);
        nxt[i] = *reinterpret_cast<const u32x4*>(x + t * d + (int64_t)c_ * VN);
      }
    };
    fetch(min(lane, nchunk - 1));
    for (int c = lane; c < nchunk; c += kWave) {
      float xv[TPW][VN];
#pragma unroll
      for (int i = 0; i < TPW; ++i) Vec16<T>::widen(nxt[i], xv[i]);
      fetch(min(c + kWave, nchunk - 1));
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (e < E) {
          float wv[VN];
          Vec16<T>::load(sw + (int64_t)e * d + c * VN, wv);
#pragma unroll
          for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int v = 0; v < VN; ++v) acc[i][e] = fmaf(xv[i][v], wv[v], acc[i][e]);
        }
      }
    }
    // butterfly: every lane ends with the full sums
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[i][e] += __shfl_xor(acc[i][e], off, kWave);
    if (lane < TPW) {
      const int64_t t = t0 + lane;
      if (t < T_tok) {
        float L[EMAX];
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
          float v = 0.f;
#pragma unroll
          for (int i = 0; i < TPW; ++i)
            if (i == lane) v = acc[i][e];
          L[e] = (e < E) ? v + (b_router ? b_router[e] : 0.f) : 0.f;
        }
        if (logits_out) {
          for (int e = 0; e < E; ++e) logits_out[t * E + e] = L[e];
        }
        finish_token_small<EMAX>(L, E, k, score, renorm, b_select, t, ids, weights);
      }
    }
  }
}

// ---------------------------------------------------------------- decode-sized T
// One workgroup per token: the 4 waves split the row, so every lane has only
// a couple of 16-byte pieces of x (and of each W_r row, read through L2) to
// fetch and all of them are in flight at once; the partial logits are
// reduced across lanes by shuffles and across waves through LDS.
template <typename T>
__global__ void __launch_bounds__(256) route_decode_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ b_router,
    const float* __restrict__ b_select, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ weights, int64_t T_tok, int d, int E, int k, int score, int renorm) {
  constexpr int EMAX = 8;
  constexpr int VN = Vec16<T>::N;
  __shared__ float part[4][EMAX];
  const int64_t t = blockIdx.x;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int nchunk = d / VN;
  float acc[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) acc[e] = 0.f;
  // All loads of a chunk are issued before any is used and none sits behind a
  // branch (experts past E re-read row E-1; their sums are never used), so
  // they are in flight together instead of one L2 round trip each.
#pragma unroll 2
  for (int c = threadIdx.x; c < nchunk; c += 256) {
    const u32x4 xr = *reinterpret_cast<const u32x4*>(x + t * d + (int64_t)c * VN);
    u32x4 wraw[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      wraw[e] = *reinterpret_cast<const u32x4*>(wr + (int64_t)min(e, E - 1) * d + (int64_t)c * VN);
    float xv[VN];
    Vec16<T>::widen(xr, xv);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      float wv[VN];
      Vec16<T>::widen(wraw[e], wv);
#pragma unroll
      for (int v = 0; v < VN; ++v) acc[e] = fmaf(xv[v], wv[v], acc[e]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) part[wave][e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float L[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      L[e] = (e < E) ? (part[0][e] + part[1][e]) + (part[2][e] + part[3][e]) +
                           (b_router ? b_router[e] : 0.f)
                     : 0.f;
    if (logits_out) {
      for (int e = 0; e < E; ++e) logits_out[t * E + e] = L[e];
    }
    finish_token_small<EMAX>(L, E, k, score, renorm, b_select, t, ids, weights);
  }
}

// ---------------------------------------------------------------- generic logits
// logits[t, e] = x[t] . wr[e] for e in an 8-expert slice (blockIdx.y), no bias.
template <typename T, int TPW>
__global__ void __launch_bounds__(256) logits_valu_kernel(const T* __restrict__ x,
                                                         const T* __restrict__ wr,
                                                         float* __restrict__ logits,
                                                         int64_t T_tok, int d, int E) {
  constexpr int ES = 8;
  constexpr int VN = Vec16<T>::N;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int e0 = blockIdx.y * ES;
  const int nchunk = d / VN;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t t0 = ((int64_t)blockIdx.x * (blockDim.x / kWave) + wave) * TPW; t0 < T_tok;
       t0 += waves_total * TPW) {
    float acc[TPW][ES];
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int e = 0; e < ES; ++e) acc[i][e] = 0.f;
    for (int c = lane; c < nchunk; c += kWave) {
      // every load of the chunk in flight at once: tokens past T and experts
      // past E re-read the last row (their sums are never stored)
      u32x4 xr[TPW], wraw[ES];
#pragma unroll
      for (int i = 0; i < TPW; ++i)
        xr[i] = *reinterpret_cast<const u32x4*>(x + min(t0 + i, T_tok - 1) * d + (int64_t)c * VN);
#pragma unroll
      for (int e = 0; e < ES; ++e)
        wraw[e] = *reinterpret_cast<const u32x4*>(wr + (int64_t)min(e0 + e, E - 1) * d +
                                                  (int64_t)c * VN);
      float xv[TPW][VN];
#pragma unroll
      for (int i = 0; i < TPW; ++i) Vec16<T>::widen(xr[i], xv[i]);
#pragma unroll
      for (int e = 0; e < ES; ++e) {
        float wv[VN];
        Vec16<T>::widen(wraw[e], wv);
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
          for (int v = 0; v < VN; ++v) acc[i][e] = fmaf(xv[i][v], wv[v], acc[i][e]);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
      for (int i = 0; i < TPW; ++i)
#pragma unroll
        for (int e = 0; e < ES; ++e) acc[i][e] += __shfl_xor(acc[i][e], off, kWave);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int64_t t = t0 + i;
        if (t < T_tok) {
#pragma unroll
          for (int e = 0; e < ES; ++e)
            if (e0 + e < E) logits[t * E + e0 + e] = acc[i][e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- top-k
// One wave per token.  Lane l owns experts l, l+64, l+128, l+192.
// `add_bias` adds b_router to the logits read (raw GEMM output) and, if
// logits_out is set, writes the final logits back.
// Group-limited selection (ng > 0, tg < ng): group scores are the largest
// key per group, gathered into lane g; tg rounds of wave arg-max pick the
// groups; keys outside them become -inf.
__device__ __forceinline__ void group_limit(float (&key)[MOE_MAX_EXPERTS / kWave], int E, int ng,
                                            int tg) {
  constexpr int PER = MOE_MAX_EXPERTS / kWave;
  const int lane = lane_id();
  const int gs = E / ng;
  float gmax = -INFINITY;  // lane g < ng: score of group g
  if (gs < kWave) {
    // groups are aligned runs of gs lanes inside a slot: segmented max
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float v = key[i];
      for (int o = 1; o < gs; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
      const int gbase = (kWave * i) / gs;           // first group of slot i
      const int src = (lane - gbase) * gs;           // leader lane of group `lane`
      const bool mine = lane >= gbase && lane < gbase + kWave / gs && kWave * i < E;
      const float got = __shfl(v, mine ? src : 0, kWave);
      if (mine) gmax = got;
    }
  } else {
    // a group spans gs / 64 whole slots
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      float v = key[i];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
      if (kWave * i < E && lane == (kWave * i) / gs) gmax = fmaxf(gmax, v);
    }
  }
  // pick tg groups: (score desc, group asc)
  bool taken = lane >= ng;
  bool chosen = false;
  for (int r = 0; r < tg; ++r) {
    float bk = taken ? -INFINITY : gmax;
    int bi = taken ? 0x7fffffff : lane;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ok = __shfl_xor(bk, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (key_better(ok, oi, bk, bi)) {
        bk = ok;
        bi = oi;
      }
    }
    if (lane == bi) {
      taken = true;
      chosen = true;
    }
  }
  const uint64_t sel = ballot(chosen);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + kWave * i;
    if (e < E && !((sel >> (e / gs)) & 1ull)) key[i] = -INFINITY;
  }
}

// logits_in holds KS slices [KS][T][E] of partial sums, added in slice order.
// PERN: experts per lane actually present (ceil(E / 64)).  All KS * PERN
// loads of a token are issued together, unconditionally (experts past E
// re-read expert E-1 and are ignored), so they overlap instead of each
// waiting for the previous one.
template <int PERN, int KS>
__global__ void __launch_bounds__(256) topk_kernel(
    const float* __restrict__ logits_in, const float* __restrict__ b_router,
    const float* __restrict__ b_select, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ weights, int64_t T_tok, int E, int k, int score, int renorm, int ng,
    int tg) {
  constexpr int PER = MOE_MAX_EXPERTS / kWave;  // 4
  static_assert(PERN >= 1 && PERN <= PER, "experts per lane");
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t waves_total = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + wave; t < T_tok;
       t += waves_total) {
    float L[PER], key[PER], sc[PER];
    bool taken[PER];
    float part[PERN][KS];
#pragma unroll
    for (int i = 0; i < PERN; ++i) {
      const int ec = min(lane + i * kWave, E - 1);
#pragma unroll
      for (int z = 0; z < KS; ++z) part[i][z] = logits_in[(int64_t)z * T_tok * E + t * E + ec];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + i * kWave;
      taken[i] = e >= E;
      L[i] = -INFINITY;
      key[i] = -INFINITY;
      sc[i] = 0.f;
      if (i < PERN && e < E) {
        float l = part[i < PERN ? i : 0][0];
#pragma unroll
        for (int z = 1; z < KS; ++z) l += part[i < PERN ? i : 0][z];
        L[i] = l + (b_router ? b_router[e] : 0.f);
        if (logits_out) logits_out[t * E + e] = L[i];
        if (score == MOE_SIGMOID) {
          sc[i] = sigmoid_f32_via_f64(L[i]);
          key[i] = b_select ? sc[i] + b_select[e] : sc[i];
        } else {
          key[i] = L[i];
        }
      }
    }
    if (ng > 0 && tg < ng) group_limit(key, E, ng, tg);
    int sel_e = -1;      // lane j < k keeps the j-th selection
    float sel_v = 0.f;   // its logit (softmax) or sigmoid score
    float first_logit = 0.f;
    // (key, index) packed so that one unsigned max picks the larger key and,
    // on equal keys, the lower expert index; 0 marks a taken expert
    uint64_t pk[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = lane + i * kWave;
      pk[i] = taken[i] ? 0ull
                       : ((uint64_t)key_image(key[i]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
    }
    for (int j = 0; j < k; ++j) {
      uint64_t mine = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) mine = pk[i] > mine ? pk[i] : mine;
      const uint64_t win = wave_max_u64(mine);
      const int bi = (int)(0xffffffffu - (uint32_t)win);  // wave-uniform
      const int owner = bi & (kWave - 1), slot = bi / kWave;
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == slot) {
          v = (score == MOE_SIGMOID) ? sc[i] : L[i];
          if (lane == owner) pk[i] = 0;
        }
      const float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), owner));
      if (lane == j) {
        sel_e = bi;
        sel_v = bv;
      }
      if (j == 0) first_logit = bv;
    }
    // weights
    float num = 0.f;
    float denom;
    if (score == MOE_SOFTMAX) {
      // the top key is the largest logit: use it as the softmax shift
      num = (lane < k) ? __expf(sel_v - first_logit) : 0.f;
      if (renorm) {
        denom = num;
      } else {
        denom = 0.f;
#pragma unroll
        for (int i = 0; i < PER; ++i)
          if (lane + i * kWave < E) denom += __expf(L[i] - first_logit);
      }
    } else {
      num = (lane < k) ? sel_v : 0.f;
      denom = num;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) denom += __shfl_xor(denom, off, kWave);
    if (score == MOE_SIGMOID && !renorm) denom = 1.f;
    if (lane < k) {
      ids[t * k + lane] = sel_e;
      weights[t * k + lane] = num / denom;
    }
  }
}

// Maximum (and sum) over the 16 lanes of each row, returned to all 16: the
// first four steps of wave_max_u64.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<0xb1, 0xf>(v);   v = o > v ? o : v;
  o = dpp_u64<0x4e, 0xf>(v);   v = o > v ? o : v;
  o = dpp_u64<0x141, 0xf>(v);  v = o > v ? o : v;
  o = dpp_u64<0x140, 0xf>(v);  v = o > v ? o : v;
  return v;
}
template <int CTRL>
__device__ __forceinline__ float dpp_row_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum_f32(float v) {
  v += dpp_row_f32<0xb1>(v);
  v += dpp_row_f32<0x4e>(v);
  v += dpp_row_f32<0x141>(v);
  v += dpp_row_f32<0x140>(v);
  return v;
}

// Top-k for E <= 64 without group limits: four tokens per wave, one per
// 16-lane row, each lane holding experts sub + 16 i (i < 4); the arg-max of
// a round stays inside the row (DPP row moves, no cross-row step), and the
// chosen expert's value comes from its lane with one bpermute.  Same
// selection order, keys and weights as topk_kernel.
// Selection and weights of the token of one 16-lane row (topk_rows_kernel,
// route_mfma_kernel): lane `sub` holds the final logits L[i] of experts
// sub + 16 i (i < 4; entries past E are ignored).
__device__ __forceinline__ void rows_select(const float (&L)[4], int sub, int row0, int64_t t,
                                            int E, int k, int score, int renorm,
                                            const float* __restrict__ b_select,
                                            int32_t* __restrict__ ids,
                                            float* __restrict__ weights) {
  constexpr int PER = 4, RL = 16;
  float sc[PER];
  uint64_t pk[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = sub + i * RL;
    float key;
    if (score == MOE_SIGMOID) {
      sc[i] = sigmoid_f32_via_f64(L[i]);
      key = (b_select && e < E) ? sc[i] + b_select[e] : sc[i];
    } else {
      sc[i] = 0.f;
      key = L[i];
    }
    pk[i] = e < E ? ((uint64_t)key_image(key) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e) : 0ull;
  }
  int sel_e = -1;
  float sel_v = 0.f, first_logit = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t mine = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) mine = pk[i] > mine ? pk[i] : mine;
    const uint64_t win = row_max_u64(mine);
    const int bi = (int)(0xffffffffu - (uint32_t)win);  // uniform within the row
    const int owner = bi & (RL - 1), slot = bi / RL;
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (i == slot) {
        v = (score == MOE_SIGMOID) ? sc[i] : L[i];
        if (sub == owner) pk[i] = 0;
      }
    const float bv = __shfl(v, row0 + owner, kWave);
    if (sub == j) {
      sel_e = bi;
      sel_v = bv;
    }
    if (j == 0) first_logit = bv;
  }
  float num, denom;
  if (score == MOE_SOFTMAX) {
    num = (sub < k) ? __expf(sel_v - first_logit) : 0.f;
    if (renorm) {
      denom = num;
    } else {
      denom = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (sub + i * RL < E) denom += __expf(L[i] - first_logit);
    }
  } else {
    num = (sub < k) ? sel_v : 0.f;
    denom = num;
  }
  denom = row_sum_f32(denom);
  if (score == MOE_SIGMOID && !renorm) denom = 1.f;
  if (sub < k) {
    ids[t * k + sub] = sel_e;
    weights[t * k + sub] = num / denom;
  }
}

template <int KS>
__global__ void __launch_bounds__(256) topk_rows_kernel(
    const float* __restrict__ logits_in, const float* __restrict__ b_router,
    const float* __restrict__ b_select, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ weights, int64_t T_tok, int E, int k, int score, int renorm) {
  constexpr int PER = 4, RL = 16;  // experts per lane, lanes per row
  const int lane = lane_id();
  const int sub = lane & (RL - 1), row0 = lane & ~(RL - 1);
  const int64_t rows_total = (int64_t)gridDim.x * (blockDim.x / RL);
  // the 16 lanes of a row share t, so a row runs or leaves the loop whole
  // and the row moves only ever read active lanes
  for (int64_t t = (int64_t)blockIdx.x * (blockDim.x / RL) + threadIdx.x / RL; t < T_tok;
       t += rows_total) {
    float part[PER][KS];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int ec = min(sub + i * RL, E - 1);
#pragma unroll
      for (int z = 0; z < KS; ++z) part[i][z] = logits_in[(int64_t)z * T_tok * E + t * E + ec];
    }
    float L[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = sub + i * RL;
      float l = part[i][0];
#pragma unroll
      for (int z = 1; z < KS; ++z) l += part[i][z];
      L[i] = l + ((b_router && e < E) ? b_router[e] : 0.f);
      if (logits_out && e < E) logits_out[t * E + e] = L[i];
    }
    rows_select(L, sub, row0, t, E, k, score, renorm, b_select, ids, weights);
  }
}

// ---------------------------------------------------------------- E <= 32, bf16, many tokens
// Logits on the matrix cores, top-k fused.  A workgroup of four waves takes
// 32 tokens at a time; each wave runs v_mfma_f32_32x32x16_bf16 over a
// quarter of d, with the tokens as M and the experts as N (one 32-wide
// tile; columns past E are computed from row E - 1 of W_r and dropped).  x reaches the wave through its own
// LDS ring by DMA (buffer_load ... lds, 8 token rows x 128 bytes per
// instruction: a cold read of the prefill input in this shape ran 8% faster
// than in 16 rows x 64 bytes; the 16-byte chunks of row r are placed at
// chunk c ^ h(r) so the fragment reads are conflict-free); only the wave
// itself reads its ring, so an s_waitcnt suffices, no barrier.  W_r (a few
// hundred KB at most, L2-resident) is read straight into B fragments.  x
// blocks of 64 k and their W_r fragments are loaded three blocks ahead; the
// next tile's first blocks are in flight while the current tile's partial
// logits are summed through LDS (16 tokens at a time) and each token is
// selected by one 16-lane row as in topk_rows_kernel.  The biases are
// staged behind the first loads, not ahead of them.
constexpr int kRmWaves = 4;
constexpr int kRmRing = 4;           // x blocks per wave ring (three ahead)
constexpr int kRmBlock = 32 * 128;   // bytes of one block: 32 rows x 64 k
constexpr int kRmBlockK = kRmBlock / 64;

__host__ __device__ constexpr size_t rm_lds_bytes(int E) {
  return (size_t)kRmWaves * kRmRing * kRmBlock + (size_t)(kRmWaves * 16 + 2) * E * sizeof(float);
}

// chunk slot of logical 16-byte chunk c of block row r is c ^ rm_swz(r):
// any 8 consecutive rows, and the even (odd) rows of any 16, hit distinct
// bank groups
__device__ __forceinline__ int rm_swz(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

template <int NT>
__global__ void __launch_bounds__(64 * kRmWaves, 2) route_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ b_router,
    const float* __restrict__ b_select, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ weights, int64_t T_tok, int d, int E, int k, int score, int renorm) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  unsigned char* ring = smem_raw + wave * kRmRing * kRmBlock;
  float* part = reinterpret_cast<float*>(smem_raw + kRmWaves * kRmRing * kRmBlock);  // [w][16][E]
  float* s_brouter = part + kRmWaves * 16 * E;
  float* s_bselect = s_brouter + E;
  // the biases (E <= 64 < blockDim) are loaded now, written to LDS once the
  // first x blocks are in flight, and read after the epilogue's barrier
  const int eb = min((int)threadIdx.x, E - 1);
  const float br_v = b_router ? b_router[eb] : 0.f;
  const float bs_v = b_select ? b_select[eb] : 0.f;
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the first x blocks
  const int h = lane >> 5;
  const int sub = lane & 15, row0 = lane & ~15;
  const int nbw = d / kRmBlockK / kRmWaves;  // 64-k blocks of this wave's quarter of d
  const int kb0 = wave * nbw;
  const int64_t tiles = (T_tok + 31) / 32;
  // DMA lane role: row dr of the 8 of an instruction; the chunk it loads
  // depends on the instruction's rows through the swizzle
  const int dr = lane >> 3;
  // B fragment rows: expert nt * 32 + (lane & 31), clamped to E - 1; a
  // column past E only ever feeds its own logits column, which is never read
  const bf16_t* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) wrow[nt] = wr + (int64_t)min(nt * 32 + (lane & 31), E - 1) * d;
  constexpr int kSteps = kRmBlockK / 16;  // MFMA k-steps per block
  constexpr int kDma = kRmBlock / 1024;    // DMA instructions per block
  constexpr int kVm = kDma + kSteps * NT;  // vector-memory instructions per fetch
  u32x4 wb[kRmRing][NT][kSteps];           // W_r fragments of the ring's blocks
  // block blk (< nbw) of tile tl into ring slot `slot`: four DMA instructions
  // (rows 8i .. 8i + 7; tokens past T re-read the last row) and the W_r
  // fragments.  Exactly kVm vector-memory instructions.
  auto fetch = [&](int slot, int64_t tl, int blk) {
    const int kk = (kb0 + blk) * kRmBlockK;  // first k of the block
    // the tile's 32 rows as a raw buffer (a buffer_load ... lds, unlike
    // global_load_lds, leaves the compiler's waits for the W_r registers
    // exact instead of waiting for every DMA in flight)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + tl * 32 * d), 0, 32 * 2 * d, 0x00020000);
    const int rlast = (int)min(T_tok - 1 - tl * 32, (int64_t)31);  // last row of the tile
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
      const int r = 8 * i + dr;
      const int dc = (lane & 7) ^ rm_swz(r);  // lane's LDS slot is lane & 7
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (void __attribute__((address_space(3)))*)(ring + slot * kRmBlock + i * 1024), 16,
          min(r, rlast) * 2 * d + (kk + dc * 8) * 2, 0, 0, 0);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int s = 0; s < kSteps; ++s)
        wb[slot][nt][s] = *reinterpret_cast<const u32x4*>(wrow[nt] + kk + 8 * (2 * s + h));
  };
  int64_t tile = blockIdx.x;
#pragma unroll
  for (int u = 0; u < kRmRing - 1; ++u) fetch(u, min(tile, tiles - 1), u);
  if (threadIdx.x < E) {
    s_brouter[threadIdx.x] = br_v;
    s_bselect[threadIdx.x] = bs_v;
  }
  for (; tile < tiles; tile += gridDim.x) {
    const int64_t next = min(tile + (int64_t)gridDim.x, tiles - 1);
    f32x16 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
    // block kb + u sits in slot u (nbw is a multiple of kRmRing); with it in
    // use, slot (u - 1) mod kRmRing is refilled with block kb + u + kRmRing - 1
    // or, past the quarter, with the next tile's block of that index - nbw
    for (int kb = 0; kb < nbw; kb += kRmRing) {
#pragma unroll
      for (int u = 0; u < kRmRing; ++u) {
        const int nb_ = kb + u + kRmRing - 1;
        const bool here = nb_ < nbw;
        fetch((u + kRmRing - 1) % kRmRing, here ? tile : next, here ? nb_ : nb_ - nbw);
        // slot u's DMA and fragments have landed: only the kRmRing - 1 later
        // fetches may be outstanding
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kRmRing - 1) * kVm) : "memory");
        __builtin_amdgcn_sched_barrier(0);
        const unsigned char* st = ring + u * kRmBlock;
        // all of the block's A fragments are read before its first MFMA (left
        // alone the compiler waited out each read's latency before each MFMA);
        // k-step s takes chunks 2s (lanes 0-31) and 2s + 1 (lanes 32-63)
        u32x4 af[kSteps];
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
          const int r = lane & 31, c = 2 * s + h;
          af[s] = *reinterpret_cast<const u32x4*>(st + r * 128 + ((c ^ rm_swz(r)) * 16));
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, af[s]), __builtin_bit_cast(bf16x8_t, wb[u][nt][s]),
                acc[nt], 0, 0, 0);
          }
        }
        // the next refill overwrites the slot read here: keep it behind
        // these MFMAs, which waited for the reads
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // value v of a lane: token 8 (v / 4) + 4 h + v % 4, expert nt * 32 + lane % 32
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int e = nt * 32 + (lane & 31);
#pragma unroll
        for (int v = 8 * half; v < 8 * half + 8; ++v) {
          const int r = 8 * (v / 4) + 4 * h + (v % 4) - 16 * half;
          if (e < E) part[(wave * 16 + r) * E + e] = acc[nt][v];
        }
      }
      // LDS-only barriers here: __syncthreads would also wait for the next
      // tile's loads in flight
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // wave w selects tokens 4w .. 4w + 3 of the 16, one per 16-lane row
      const int r = 4 * wave + (lane >> 4);
      const int64_t t = tile * 32 + 16 * half + r;
      if (t < T_tok) {
        float L[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = min(sub + 16 * i, E - 1);
          float l = 0.f;
#pragma unroll
          for (int w = 0; w < kRmWaves; ++w) l += part[(w * 16 + r) * E + e];
          L[i] = l + s_brouter[e];
          if (logits_out && sub + 16 * i < E) logits_out[t * E + e] = L[i];
        }
        rows_select(L, sub, row0, t, E, k, score, renorm, b_select ? s_bselect : nullptr, ids,
                    weights);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the ring's last refills
}

int grid_for(int64_t units, int per_block);


template <int PERN>
bool launch_topk_p(const float* in, int ks, const moe_route_args* a, const float* b_router,
                   float* logits_out, int ng, hipStream_t stream) {
  const dim3 grid(grid_for(a->T, 4)), tb(256);
  const int tg = a->topk_groups;
  switch (ks) {
#define MOE_TOPK_CASE(K_)                                                                    \
  case K_:                                                                                 \
    topk_kernel<PERN, K_><<<grid, tb, 0, stream>>>(in, b_router, a->b_select, logits_out,  \
                                                   a->ids, a->weights, a->T, a->E, a->k,   \
                                                   a->score, a->renorm, ng, tg);           \
    break;
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(16)
#undef MOE_TOPK_CASE
    default:
      return false;
  }
  return true;
}

// Scores and top-k from ks slices of logits; false (nothing launched) unless
// ks is a power of two <= 16.
bool launch_topk(const float* in, int ks, const moe_route_args* a, const float* b_router,
                 float* logits_out, int ng, hipStream_t stream) {
  if (a->E <= 64 && (ng == 0 || a->topk_groups >= ng)) {
    const dim3 grid(grid_for(a->T, 16)), tb(256);
    switch (ks) {
#define MOE_TOPK_ROWS_CASE(K_)                                                                 \
  case K_:                                                                                   \
    topk_rows_kernel<K_><<<grid, tb, 0, stream>>>(in, b_router, a->b_select, logits_out, a->ids, \
                                                  a->weights, a->T, a->E, a->k, a->score,   \
                                                  a->renorm);                               \
    return true;
      MOE_TOPK_ROWS_CASE(1)
      MOE_TOPK_ROWS_CASE(2)
      MOE_TOPK_ROWS_CASE(4)
      MOE_TOPK_ROWS_CASE(8)
      MOE_TOPK_ROWS_CASE(16)
#undef MOE_TOPK_ROWS_CASE
      default:
        return false;
    }
  }
  const int pern = (a->E + kWave - 1) / kWave;
  if (pern <= 1) return launch_topk_p<1>(in, ks, a, b_router, logits_out, ng, stream);
  if (pern <= 2) return launch_topk_p<2>(in, ks, a, b_router, logits_out, ng, stream);
  return launch_topk_p<4>(in, ks, a, b_router, logits_out, ng, stream);
}

int grid_for(int64_t units, int per_block) {
  const int64_t want = (units + per_block - 1) / per_block;
  const int64_t cap = (int64_t)device_info().cus * 8;
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

bool grouped(const moe_route_args* a) { return a->n_groups > 0 && a->topk_groups < a->n_groups; }

bool small_route_fits(const moe_route_args* a) {
  const size_t es = a->act_dtype == MOE_F32 ? 4 : 2;
  return !grouped(a) && a->E <= 8 && (size_t)a->E * a->d * es <= 64 * 1024;
}


// bf16, E <= 32 without group limits, many tokens: route_mfma_kernel
bool mfma_rows_route(const moe_route_args* a) {
  // each wave's quarter of d is a whole number of ring rounds of 64-k blocks.
  // E <= 32 only: with two 32-wide expert tiles the ring's W_r fragments
  // (128 registers) no longer fit two workgroups per CU without spilling
  return a->act_dtype == MOE_BF16 && a->E <= 32 && !grouped(a) &&
         a->d % (kRmBlockK * kRmWaves * kRmRing) == 0 && a->T > 1024;
}

bool mfma_route(const moe_route_args* a) {
  return a->act_dtype == MOE_BF16 && a->E % 64 == 0 && a->d % 128 == 0 && !small_route_fits(a) &&
         !mfma_rows_route(a);
}

}  // namespace
}  // namespace moe

using namespace moe;

// Split-K slices of the router logits (1 unless the MFMA path splits K).
static int route_ksplit(const moe_route_args* a) {
  return mfma_route(a) ? dense_logits_ksplit(a->T, a->d, a->E) : 1;
}

extern "C" size_t moe_route_workspace_bytes(const moe_route_args* a) {
  if (!a || a->x == nullptr || small_route_fits(a) || mfma_rows_route(a)) return 0;
  return align_up((size_t)route_ksplit(a) * a->T * a->E * sizeof(float), 256);
}

extern "C" moe_status moe_route(const moe_route_args* a, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, "null args");
  MOE_CHECK_ARG(a->T >= 0, "T < 0");
  MOE_CHECK_ARG(a->E >= 1 && a->E <= MOE_MAX_EXPERTS, "E out of range [1, 256]");
  MOE_CHECK_ARG(a->k >= 1 && a->k <= MOE_MAX_TOPK && a->k <= a->E, "k out of range [1, min(8, E)]");
  MOE_CHECK_ARG(a->score == MOE_SOFTMAX || a->score == MOE_SIGMOID, "bad score");
  MOE_CHECK_ARG(a->b_select == nullptr || a->score == MOE_SIGMOID,
                "b_select needs sigmoid scores");
  MOE_CHECK_ARG(a->act_dtype == MOE_F32 || a->act_dtype == MOE_BF16, "bad act_dtype");
  MOE_CHECK_ARG(a->ids && a->weights, "ids/weights are required");
  if (a->n_groups > 0) {
    MOE_CHECK_ARG(a->n_groups <= 64 && a->E % a->n_groups == 0, "n_groups must divide E, <= 64");
    const int gs = a->E / a->n_groups;
    MOE_CHECK_ARG((gs < 64 && (gs & (gs - 1)) == 0) || gs % 64 == 0,
                  "E/n_groups must be a power of two below 64 or a multiple of 64");
    MOE_CHECK_ARG(a->topk_groups >= 0, "topk_groups < 0");
    MOE_CHECK_ARG(!grouped(a) || (int64_t)a->k <= (int64_t)a->topk_groups * gs,
                  "k exceeds the experts of topk_groups groups");
    MOE_CHECK_ARG(!grouped(a) || a->topk_groups >= 1, "topk_groups must be >= 1");
  }
  MOE_CHECK_ARG(aligned16(a->ids) && aligned16(a->weights), "ids/weights not 16-byte aligned");
  if (a->T == 0) return MOE_OK;
  const int tb = 256;
  if (a->x == nullptr) {
    MOE_CHECK_ARG(a->logits != nullptr, "x == NULL needs input logits");
    MOE_CHECK_ARG(a->b_router == nullptr, "x == NULL: logits are final, b_router must be NULL");
    if (check_only()) return MOE_OK;
    if (!launch_topk(a->logits, 1, a, nullptr, nullptr, grouped(a) ? a->n_groups : 0, stream)) {
      set_error("moe_route: unsupported split of the router logits");
      return MOE_ERR_INVALID;
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  MOE_CHECK_ARG(a->w_router != nullptr, "w_router is required");
  MOE_CHECK_ARG(a->d >= 1, "d < 1");
  const int vn = a->act_dtype == MOE_F32 ? 4 : 8;
  MOE_CHECK_ARG(a->d % vn == 0, "d must be a multiple of 16 bytes");
  MOE_CHECK_ARG(aligned16(a->x) && aligned16(a->w_router), "x/w_router not 16-byte aligned");
  if (mfma_rows_route(a)) {
    if (check_only()) return MOE_OK;
    const size_t lds = rm_lds_bytes(a->E);
    const int per_cu = 2 * lds <= 160 * 1024 ? 2 : 1;
    const int grid = (int)std::min<int64_t>((a->T + 31) / 32, (int64_t)device_info().cus * per_cu);
    MOE_CHECK_HIP(set_dynamic_lds((const void*)route_mfma_kernel<1>, (int)lds));
    route_mfma_kernel<1><<<grid, 64 * kRmWaves, lds, stream>>>(
        (const bf16_t*)a->x, (const bf16_t*)a->w_router, a->b_router, a->b_select, a->logits,
        a->ids, a->weights, a->T, a->d, a->E, a->k, a->score, a->renorm);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  if (small_route_fits(a)) {
    if (check_only()) return MOE_OK;
    // Many tokens: stage W_r in LDS once per workgroup and loop over tokens.
    // Few tokens (decode): one workgroup per token, W_r read through L2.
    const bool stage = a->T > 1024;
    const size_t lds = stage ? (size_t)a->E * a->d * (a->act_dtype == MOE_F32 ? 4 : 2) : 0;
    if (stage) {
      constexpr int TPW = kRsTpw;
      const int grid = (int)std::min<int64_t>((a->T + 4 * TPW - 1) / (4 * TPW),
                                              (int64_t)device_info().cus * 2);
      if (a->act_dtype == MOE_F32) {
        route_small_kernel<float, TPW, true><<<grid, tb, lds, stream>>>(
            (const float*)a->x, (const float*)a->w_router, a->b_router, a->b_select, a->logits,
            a->ids, a->weights, a->T, a->d, a->E, a->k, a->score, a->renorm);
      } else {
        route_small_kernel<bf16_t, TPW, true><<<grid, tb, lds, stream>>>(
            (const bf16_t*)a->x, (const bf16_t*)a->w_router, a->b_router, a->b_select, a->logits,
            a->ids, a->weights, a->T, a->d, a->E, a->k, a->score, a->renorm);
      }
    } else {
      const int grid = (int)a->T;
      if (a->act_dtype == MOE_F32) {
        route_decode_kernel<float><<<grid, tb, 0, stream>>>(
            (const float*)a->x, (const float*)a->w_router, a->b_router, a->b_select, a->logits,
            a->ids, a->weights, a->T, a->d, a->E, a->k, a->score, a->renorm);
      } else {
        route_decode_kernel<bf16_t><<<grid, tb, 0, stream>>>(
            (const bf16_t*)a->x, (const bf16_t*)a->w_router, a->b_router, a->b_select, a->logits,
            a->ids, a->weights, a->T, a->d, a->E, a->k, a->score, a->renorm);
      }
    }
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  const size_t need = moe_route_workspace_bytes(a);
  if (ws_bytes < need || (need && ws == nullptr)) {
    set_error("moe_route: workspace too small");
    return MOE_ERR_WORKSPACE;
  }
  if (check_only()) return MOE_OK;
  float* raw = static_cast<float*>(ws);
  const int ks = route_ksplit(a);
  if (mfma_route(a)) {
    const moe_status st = dense_logits_gemm(a->x, a->w_router, raw, a->T, a->d, a->E, stream);
    if (st != MOE_OK) return st;
  } else {
    constexpr int TPW = 4;
    dim3 grid(grid_for(a->T, 4 * TPW), (a->E + 7) / 8);
    if (a->act_dtype == MOE_F32) {
      logits_valu_kernel<float, TPW><<<grid, tb, 0, stream>>>(
          (const float*)a->x, (const float*)a->w_router, raw, a->T, a->d, a->E);
    } else {
      logits_valu_kernel<bf16_t, TPW><<<grid, tb, 0, stream>>>(
          (const bf16_t*)a->x, (const bf16_t*)a->w_router, raw, a->T, a->d, a->E);
    }
    MOE_CHECK_LAUNCH();
  }
  if (!launch_topk(raw, ks, a, a->b_router, a->logits, grouped(a) ? a->n_groups : 0, stream)) {
    set_error("moe_route: unsupported split of the router logits");
    return MOE_ERR_INVALID;
  }
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
