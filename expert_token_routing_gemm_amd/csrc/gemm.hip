// Grouped expert GEMM on gfx950 MFMA, with a device-side per-expert tile
// scheduler, and the expert-FFN entry point.
//
// Local expert compute: once the rows of an expert are gathered, experts
// run independently (Ultralytics glossary "Expert Parallelism", "How Tokens
// Move Between GPUs", step 3; mbrenndoerfer "Expert Parallelism > Summary").
// The FFN form (ReLU, GELU, SwiGLU) is not on the pages; the workload
// definitions fix it.
//
// Structure
//  * One persistent kernel per GEMM.  Groups are the executed experts (rows
//    [off[e], off[e+1]) of the send buffer, read from device memory) plus an
//    optional dense group (the shared expert).  At start every workgroup
//    turns the row counts into a tile prefix in LDS; tile t -> (group, m, n)
//    by binary search, so no host synchronisation is needed.
//  * blockIdx is remapped so that consecutive tiles run on the same XCD
//    (workgroups are dealt round-robin over the 8 XCDs, each with its own
//    L2), and tiles of a group are ordered in strips of GM m-tiles so that
//    concurrently running tiles share A and B panels.
//  * A and B tiles are staged through LDS (rows of 128 bytes + 16 bytes pad,
//    so the 16 lanes reading one MFMA fragment hit distinct banks), double
//    buffered, with 128-bit global loads.  Each lane reads 16-byte fragments:
//    v_mfma_f32_16x16x32_bf16 for bf16, and four v_mfma_f32_16x16x4_f32 for
//    fp32 (k is permuted consistently on A and B inside each 16-k step).
//  * fp8 e4m3 weights are read as bytes (half the HBM traffic), dequantised
//    exactly to fp32, multiplied by their 128x128 block scale and rounded
//    once to bf16 on the way into LDS; the MFMA runs in bf16 with fp32
//    accumulation.
//  * Decode-sized groups use the weight-streaming kernel of stream_gemm.hip.
//  * SwiGLU: a wave's B rows are w1 rows and the w3 rows of the same output
//    columns, so silu(z1) * z3 is formed in registers.
#include <math.h>

#include <type_traits>

#include "gemm.h"
#include "gemm_common.h"

// Padding (bytes) after each LDS tile row of the LDS-staged kernel.
constexpr int kLdsPad = 16;

namespace moe {
namespace {

constexpr int kThreads = kGemmThreads;
constexpr int kGM = 4;  // m-tiles per strip

// Exclusive scan of up to 2*kThreads values held two per thread.
__device__ void scan_pairs(int v0, int v1, int* out0, int* out1, int* total, int* sh) {
  const int lane = lane_id();
  const int w = threadIdx.x / 64;
  int s = v0 + v1;
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh[w] = incl;
  __syncthreads();
  int add = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    if (i < w) add += sh[i];
    tot += sh[i];
  }
  const int excl = incl - s + add;
  *out0 = excl;
  *out1 = excl + v0;
  *total = tot;
}

template <typename AT, typename CT, int BSRC, int EPI, int BM, int BN, int WAVES_M, int WAVES_N,
          int MINB, int RB>
__global__ void __launch_bounds__(kThreads, MINB) grouped_gemm_kernel(GroupedParams p) {
  // RB: bytes of a tile row per K-stage (128 or 64); LDS rows are padded by
  // 16 bytes so the 16 lanes reading one MFMA fragment hit distinct banks.
  constexpr int kRowBytes = RB;
  constexpr int kLdsRow = RB + kLdsPad;
  constexpr int CPR = RB / 16;               // 16-byte chunks per row
  constexpr int RPP = kThreads / CPR;        // rows covered by one pass of the block
  constexpr int STEPS = RB / 64;             // MFMA k-steps per stage
  static_assert(WAVES_M * WAVES_N == kThreads / 64, "4 waves");
  constexpr int WTM = BM / WAVES_M;  // rows per wave
  constexpr int WTN = BN / WAVES_N;  // B rows per wave
  constexpr bool M32 = sizeof(AT) == 2;       // bf16 -> 32x32x16 MFMA
  constexpr int QS = M32 ? 32 : 16;           // subtile edge
  constexpr int QM = WTM / QS;
  constexpr int QN = WTN / QS;
  using Acc = typename std::conditional<M32, f32x16, f32x4>::type;
  static_assert(EPI != EPI_SWIGLU || QN % 2 == 0, "SwiGLU pairs subtiles");
  constexpr int BK = kRowBytes / (int)sizeof(AT);  // elements per K-stage
  constexpr int A_CH = BM / RPP;                     // 16-byte chunks per thread
  constexpr int B_CH = BN / RPP;
  static_assert(A_CH >= 1 && B_CH >= 1, "tile too small");

  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* lds_a = smem;                              // [2][BM][kLdsRow]
  unsigned char* lds_b = smem + 2 * BM * kLdsRow;           // [2][BN][kLdsRow]
  int* s_tstart = reinterpret_cast<int*>(smem + 2 * (BM + BN) * kLdsRow);  // [kMaxGroups+1]
  int* s_rows = s_tstart + (kMaxGroups + 1);                               // [kMaxGroups]
  int* s_r0 = s_rows + kMaxGroups;                                         // [kMaxGroups]
  int* s_scan = s_r0 + kMaxGroups;                                         // [4]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / 64;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int ngroups = p.n_routed + (p.t_dense > 0 ? 1 : 0);
  const int nt = p.N / BN;

  // ---- tile table
  {
    int t2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = 2 * tid + h;
      int rows = 0, r0 = 0;
      if (g < p.n_routed) {
        r0 = p.off[p.e_begin + g];
        rows = p.off[p.e_begin + g + 1] - r0;
      } else if (g < ngroups) {
        rows = (int)p.t_dense;
      }
      if (g < kMaxGroups) {
        s_rows[g] = rows;
        s_r0[g] = r0;
      }
      t2[h] = (g < ngroups) ? ((rows + BM - 1) / BM) * nt : 0;
    }
    int e0, e1, tot;
    scan_pairs(t2[0], t2[1], &e0, &e1, &tot, s_scan);
    if (2 * tid < kMaxGroups + 1) s_tstart[2 * tid] = e0;
    if (2 * tid + 1 < kMaxGroups + 1) s_tstart[2 * tid + 1] = e1;
    if (tid == 0) s_tstart[ngroups] = tot;  // (same value as the scan gives)
  }
  __syncthreads();
  const int total = s_tstart[ngroups];
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int first = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int a_sub = (p.a_shift && p.n_routed > 0) ? p.off[p.e_begin] : 0;
  const int c_sub = (p.c_shift && p.n_routed > 0) ? p.off[p.e_begin] : 0;

  for (int tile = first; tile < total; tile += G) {
    // ---- decode tile -> (group, m tile, n tile)
    int lo = 0, hi = ngroups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tstart[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int local = tile - s_tstart[g];
    const int rows = s_rows[g];
    const int mt = (rows + BM - 1) / BM;
    const int strip = local / (kGM * nt);
    const int rem = local - strip * kGM * nt;
    const int gm = min(kGM, mt - strip * kGM);
    const int m_t = strip * kGM + rem % gm;
    const int n_t = rem / gm;
    const bool dense = g >= p.n_routed;
    const int m0 = m_t * BM;

    const AT* A;
    CT* C;
    const unsigned char* B1;
    const unsigned char* B3;
    const float* S1;
    const float* S3;
    {
      const int bes = BSRC == B_FP8 ? 1 : (int)sizeof(AT);
      if (!dense) {
        A = reinterpret_cast<const AT*>(p.a_routed) + (int64_t)(s_r0[g] - a_sub) * p.K;
        C = reinterpret_cast<CT*>(p.c_routed) + (int64_t)(s_r0[g] - c_sub) * p.ldc;
        B1 = reinterpret_cast<const unsigned char*>(p.b1) + (int64_t)g * p.b_stride * bes;
        B3 = p.b3 ? reinterpret_cast<const unsigned char*>(p.b3) + (int64_t)g * p.b_stride * bes
                  : nullptr;
        S1 = p.s1 ? p.s1 + (int64_t)g * p.ns * p.ks : nullptr;
        S3 = p.s3 ? p.s3 + (int64_t)g * p.ns * p.ks : nullptr;
      } else {
        A = reinterpret_cast<const AT*>(p.a_dense);
        C = reinterpret_cast<CT*>(p.c_dense);
        B1 = reinterpret_cast<const unsigned char*>(p.bd1);
        B3 = reinterpret_cast<const unsigned char*>(p.bd3);
        S1 = p.sd1;
        S3 = p.sd3;
      }
    }

    // ---- per-thread load descriptors
    // Chunk i of a stage covers tile row r0 + RPP*i (r0 = tid / CPR) and the
    // 16-byte column tid % CPR.  Only r0 varies across threads, so per-chunk
    // row offsets are uniform and the compiler keeps one address per matrix.
    const int r0t = tid / CPR;
    const int c16 = tid % CPR;
    const unsigned char* a_base = reinterpret_cast<const unsigned char*>(A) + c16 * 16;
    const int64_t a_stride = (int64_t)p.K * sizeof(AT);
    constexpr int bes = BSRC == B_FP8 ? 1 : (int)sizeof(AT);
    const int64_t b_stride = (int64_t)p.K * bes;
    // B row of chunk i (SwiGLU: the wave's w1 rows, then the matching w3 rows)
    auto b_row = [&](int i) -> int {
      const int r = RPP * i + r0t;
      if (EPI == EPI_SWIGLU) {
        const int w_ = r / WTN, rr = r % WTN;
        return n_t * (BN / 2) + w_ * (WTN / 2) + rr % (WTN / 2);
      }
      return n_t * BN + r;
    };
    auto b_which = [&](int i) -> int {
      return (EPI == EPI_SWIGLU) ? ((RPP * i + r0t) % WTN) / (WTN / 2) : 0;
    };
    const unsigned char* b1_base = B1 + c16 * (BSRC == B_FP8 ? 8 : 16);
    const unsigned char* b3_base = (EPI == EPI_SWIGLU ? B3 : B1) + c16 * (BSRC == B_FP8 ? 8 : 16);
    // bf16: v_mfma_f32_32x32x16_bf16 on 32x32 subtiles (the full-rate bf16
    // MFMA on gfx950); fp32: v_mfma_f32_16x16x4_f32 on 16x16 subtiles.
    Acc acc[QM][QN];
#pragma unroll
    for (int i = 0; i < QM; ++i)
#pragma unroll
      for (int j = 0; j < QN; ++j) acc[i][j] = Acc{};

    // Two register sets of global loads: while stage kt is computed from
    // LDS, stage kt+1 (in registers) is waiting to be written to the other
    // LDS buffer and stage kt+2 is being fetched.  The barrier orders LDS
    // only, so the fetch of kt+2 stays in flight across it.  Chunk indices
    // are clamped instead of skipping loads (no branches around loads).
    // fp8 weights stay as bytes in registers and are dequantised when they
    // are written to LDS.
    u32x4 ra[2][A_CH];
    u32x4 rb[2][B_CH];
    uint2 rq[2][B_CH];
    float rs[2][B_CH];
    const int KT = p.K / BK;

#define MOE_GEMM_LOAD_STAGE(SET_, KT_)                                                  \
    {                                                                                   \
      const int64_t kb = (int64_t)(KT_) * kRowBytes;                                    \
      _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                \
        const int row_ = m0 + r0t + RPP * i;                                             \
        ra[SET_][i] = *reinterpret_cast<const u32x4*>(                                  \
            a_base + (int64_t)min(row_, rows - 1) * a_stride + kb);                     \
      }                                                                                 \
      _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                \
        const unsigned char* bb_ = (b_which(i) ? b3_base : b1_base) +                   \
                                   (int64_t)b_row(i) * b_stride;                        \
        if constexpr (BSRC == B_FP8) {                                                  \
          rq[SET_][i] = *reinterpret_cast<const uint2*>(bb_ + (int64_t)(KT_) * BK);     \
          const float* sb_ = b_which(i) ? S3 : S1;                                      \
          rs[SET_][i] = sb_[(int64_t)(b_row(i) / 128) * p.ks + ((KT_) * BK) / 128];     \
        } else {                                                                        \
          rb[SET_][i] = *reinterpret_cast<const u32x4*>(bb_ + kb);                      \
        }                                                                               \
      }                                                                                 \
    }
#define MOE_GEMM_STORE_STAGE(SET_, BUF_)                                                \
    {                                                                                   \
      unsigned char* la_ = lds_a + (BUF_) * BM * kLdsRow;                               \
      unsigned char* lb_ = lds_b + (BUF_) * BN * kLdsRow;                               \
      _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                \
        const int row_ = m0 + r0t + RPP * i;                                             \
        *reinterpret_cast<u32x4*>(la_ + (r0t + RPP * i) * kLdsRow + c16 * 16) =          \
            ra[SET_][i] & (row_ < rows ? 0xffffffffu : 0u);                             \
      }                                                                                 \
      _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                \
        u32x4 v_;                                                                       \
        if constexpr (BSRC == B_FP8) {                                                  \
          const uint2 q = rq[SET_][i];                                                  \
          const float sc = rs[SET_][i];                                                 \
          v_.x = pack_bf16x2(e4m3_to_f32(q.x & 0xffu) * sc, e4m3_to_f32((q.x >> 8) & 0xffu) * sc);   \
          v_.y = pack_bf16x2(e4m3_to_f32((q.x >> 16) & 0xffu) * sc, e4m3_to_f32(q.x >> 24) * sc);    \
          v_.z = pack_bf16x2(e4m3_to_f32(q.y & 0xffu) * sc, e4m3_to_f32((q.y >> 8) & 0xffu) * sc);   \
          v_.w = pack_bf16x2(e4m3_to_f32((q.y >> 16) & 0xffu) * sc, e4m3_to_f32(q.y >> 24) * sc);    \
        } else {                                                                        \
          v_ = rb[SET_][i];                                                             \
        }                                                                               \
        *reinterpret_cast<u32x4*>(lb_ + (r0t + RPP * i) * kLdsRow + c16 * 16) = v_;       \
      }                                                                                 \
    }
#define MOE_GEMM_COMPUTE(BUF_)                                                          \
    {                                                                                   \
      const unsigned char* la = lds_a + (BUF_) * BM * kLdsRow;                          \
      const unsigned char* lb = lds_b + (BUF_) * BN * kLdsRow;                          \
      if constexpr (M32) {                                                              \
        /* lane: row lane%32 of a 32-row subtile, 8 k at byte 32*step + 16*(lane/32) */ \
        _Pragma("unroll") for (int step = 0; step < RB / 32; ++step) {                  \
          const int kofs = step * 32 + (lane >> 5) * 16;                                \
          u32x4 bfr[QN];                                                                \
          _Pragma("unroll") for (int j = 0; j < QN; ++j)                                \
            bfr[j] = *reinterpret_cast<const u32x4*>(                                   \
                lb + (wn * WTN + j * 32 + (lane & 31)) * kLdsRow + kofs);               \
          _Pragma("unroll") for (int i = 0; i < QM; ++i) {                              \
            const u32x4 af = *reinterpret_cast<const u32x4*>(                           \
                la + (wm * WTM + i * 32 + (lane & 31)) * kLdsRow + kofs);               \
            _Pragma("unroll") for (int j = 0; j < QN; ++j)                              \
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                      \
                  __builtin_bit_cast(bf16x8_t, af), __builtin_bit_cast(bf16x8_t, bfr[j]), \
                  acc[i][j], 0, 0, 0);                                                  \
          }                                                                             \
        }                                                                               \
      } else {                                                                          \
        _Pragma("unroll") for (int step = 0; step < STEPS; ++step) {                    \
          const int chunk = (lane >> 4) + 4 * step;                                     \
          u32x4 bfr[QN];                                                                \
          _Pragma("unroll") for (int j = 0; j < QN; ++j)                                \
            bfr[j] = *reinterpret_cast<const u32x4*>(                                   \
                lb + (wn * WTN + j * 16 + (lane & 15)) * kLdsRow + chunk * 16);         \
          _Pragma("unroll") for (int i = 0; i < QM; ++i) {                              \
            const u32x4 af = *reinterpret_cast<const u32x4*>(                           \
                la + (wm * WTM + i * 16 + (lane & 15)) * kLdsRow + chunk * 16);         \
            _Pragma("unroll") for (int j = 0; j < QN; ++j) {                            \
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(                         \
                  __uint_as_float(af.x), __uint_as_float(bfr[j].x), acc[i][j], 0, 0, 0); \
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(                         \
                  __uint_as_float(af.y), __uint_as_float(bfr[j].y), acc[i][j], 0, 0, 0); \
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(                         \
                  __uint_as_float(af.z), __uint_as_float(bfr[j].z), acc[i][j], 0, 0, 0); \
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(                         \
                  __uint_as_float(af.w), __uint_as_float(bfr[j].w), acc[i][j], 0, 0, 0); \
            }                                                                           \
          }                                                                             \
        }                                                                               \
      }                                                                                 \
    }

    MOE_BARRIER_LDS();  // previous tile's LDS reads are complete
    MOE_GEMM_LOAD_STAGE(0, 0);
    MOE_GEMM_LOAD_STAGE(1, min(1, KT - 1));
    MOE_GEMM_STORE_STAGE(0, 0);
    MOE_BARRIER_LDS();

    for (int kt = 0; kt < KT; kt += 2) {
      // even stage: LDS buffer 0, registers of stage kt+1 in set 1
      MOE_GEMM_LOAD_STAGE(0, min(kt + 2, KT - 1));
      MOE_GEMM_COMPUTE(0);
      MOE_GEMM_STORE_STAGE(1, 1);
      MOE_BARRIER_LDS();
      if (kt + 1 >= KT) break;
      // odd stage: LDS buffer 1, registers of stage kt+2 in set 0
      MOE_GEMM_LOAD_STAGE(1, min(kt + 3, KT - 1));
      MOE_GEMM_COMPUTE(1);
      MOE_GEMM_STORE_STAGE(0, 0);
      MOE_BARRIER_LDS();
    }
#undef MOE_GEMM_LOAD_STAGE
#undef MOE_GEMM_STORE_STAGE
#undef MOE_GEMM_COMPUTE

    // ---- epilogue.  32x32 subtile: value v of a lane is row
    // 8*(v/4) + 4*(lane/32) + v%4, column lane%32.  16x16 subtile: value r is
    // row 4*(lane/16) + r, column lane%16.
    constexpr int NV = M32 ? 16 : 4;
#pragma unroll
    for (int i = 0; i < QM; ++i) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int rsub = M32 ? 8 * (v / 4) + 4 * (lane >> 5) + (v % 4) : 4 * (lane >> 4) + v;
        const int csub = M32 ? (lane & 31) : (lane & 15);
        const int row = m0 + wm * WTM + i * QS + rsub;
        if (row >= rows) continue;
        CT* crow = C + (int64_t)row * p.ldc;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < QN / 2; ++j) {
            const int col = n_t * (BN / 2) + wn * (WTN / 2) + j * QS + csub;
            store_out<CT>(crow + col, act_silu(acc[i][j][v]) * acc[i][j + QN / 2][v]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < QN; ++j) {
            const int col = n_t * BN + wn * WTN + j * QS + csub;
            float x = acc[i][j][v];
            if (EPI == EPI_RELU) x = fmaxf(x, 0.f);
            if (EPI == EPI_GELU) x = act_gelu(x);
            store_out<CT>(crow + col, x);
          }
        }
      }
    }
  }
}


// ---------------------------------------------------------------- launch

// Tile of the LDS-staged grouped GEMM for many-row groups (bf16 MFMA):
// BM x BN with 2 x 2 waves, MINB workgroups per CU.
constexpr int kBigBm = 128;
constexpr int kBigBn = 128;
constexpr int kBigMinb = 2;

template <int BM, int BN, int RB>
constexpr size_t lds_bytes() {
  return 2 * (BM + BN) * (RB + kLdsPad) + (3 * kMaxGroups + 1 + 4) * sizeof(int);
}

struct LaunchCfg {
  int grid;
};

constexpr int kBigRb = 64;
template <typename AT, typename CT, int BSRC, int EPI, int BM, int BN, int WM, int WN, int MINB>
moe_status launch(const GroupedParams& p, int64_t max_routed_rows, hipStream_t stream) {
  constexpr int RB = kBigRb;
  auto kern = grouped_gemm_kernel<AT, CT, BSRC, EPI, BM, BN, WM, WN, MINB, RB>;
  constexpr size_t lds = lds_bytes<BM, BN, RB>();
  MOE_CHECK_HIP(set_dynamic_lds((const void*)kern, (int)lds));
  const int nt = p.N / BN;
  const int ngroups = p.n_routed + (p.t_dense > 0 ? 1 : 0);
  const int64_t m_tiles_ub = (max_routed_rows + BM - 1) / BM + p.n_routed +
                             (p.t_dense > 0 ? (p.t_dense + BM - 1) / BM : 0);
  const int64_t tiles_ub = m_tiles_ub * nt;
  if (ngroups == 0 || tiles_ub == 0) return MOE_OK;
  int per_cu = (int)(160 * 1024 / lds);
  if (per_cu < 1) per_cu = 1;
  if (per_cu > MINB) per_cu = MINB;
  int64_t grid = (int64_t)device_info().cus * per_cu;
  if (grid > tiles_ub) grid = tiles_ub;
  if (grid >= 8) grid = grid / 8 * 8;
  kern<<<(int)grid, kThreads, lds, stream>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <typename AT, int BSRC, int BM, int BN, int WM, int WN, int MINB>
moe_status launch_gemm1(int act, const GroupedParams& p, int64_t rows, hipStream_t s) {
  switch (act) {
    case MOE_RELU:
      return launch<AT, AT, BSRC, EPI_RELU, BM, BN, WM, WN, MINB>(p, rows, s);
    case MOE_GELU:
      return launch<AT, AT, BSRC, EPI_GELU, BM, BN, WM, WN, MINB>(p, rows, s);
    default:
      return launch<AT, AT, BSRC, EPI_SWIGLU, BM, BN, WM, WN, MINB>(p, rows, s);
  }
}

// Launch plan of the expert FFN: kernel family, split-K factors and the
// workspace layout [act rows x h][fp32 split-K partials].
struct FfnPlan {
  bool small_m;
  int ks1, ks2;
  size_t act_bytes;
  size_t partial_bytes;
};

FfnPlan plan_ffn(const moe_ffn_args* a) {
  FfnPlan pl{};
  const int n_routed = a->e_end - a->e_begin;
  const bool dense = a->x_dense != nullptr && a->T_dense > 0;
  const int ngroups = n_routed + (dense ? 1 : 0);
  const bool swiglu = a->act == MOE_SWIGLU;
  const size_t es = a->act_dtype == MOE_F32 ? 4 : 2;
  const int64_t prow_total = a->max_rows + (dense ? a->T_dense : 0);
  // Decode-sized groups (a few rows per expert) stream weights.
  pl.small_m = a->act_dtype == MOE_BF16 &&
               a->max_rows <= (int64_t)64 * (n_routed > 0 ? n_routed : 1) &&
               (!dense || a->T_dense <= 64);
  pl.ks1 = pl.ks2 = 1;
  if (pl.small_m && ngroups > 0) {
    pl.ks1 = stream_ksplit(ngroups, a->h, a->d, stream_ck_for(swiglu, a->d));
    pl.ks2 = stream_ksplit(ngroups, a->d, a->h, stream_ck_for(false, a->h));
  }
  pl.act_bytes = align_up((size_t)prow_total * a->h * es, 256);
  const size_t p1 = pl.ks1 > 1 ? (size_t)pl.ks1 * prow_total * (swiglu ? 2 : 1) * a->h * 4 : 0;
  const size_t p2 = pl.ks2 > 1 ? (size_t)pl.ks2 * prow_total * a->d * 4 : 0;
  pl.partial_bytes = align_up(p1 > p2 ? p1 : p2, 256);
  return pl;
}

// fp32 activations: square tile edge and workgroups per CU of the LDS-staged
// kernel.  64x64 tiles, four workgroups per CU (measured on the tiny fp32
// workload, 8192 rows x 512 x 512 per GEMM: 74 -> 56 us per GEMM against
// 128x128 tiles; 64x64 with two per CU: 62 us).
constexpr int kF32Tile = 64;
constexpr int kF32Minb = 4;
template <typename AT, int BSRC>
moe_status run_ffn(const moe_ffn_args* a, const FfnPlan& pl, void* ws, hipStream_t stream,
                   hipEvent_t mid_event) {
  const int d = a->d, h = a->h;
  const int n_routed = a->e_end - a->e_begin;
  const bool swiglu = a->act == MOE_SWIGLU;
  const int64_t rows = a->max_rows;
  AT* act_routed = static_cast<AT*>(ws);
  AT* act_dense = act_routed + rows * (int64_t)h;
  float* partial = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + pl.act_bytes);
  const bool small_m = pl.small_m;

  GroupedParams p1{};
  p1.a_routed = a->x_send;
  p1.a_dense = a->x_dense;
  p1.c_routed = act_routed;
  p1.c_dense = act_dense;
  p1.b1 = a->w1;
  p1.b3 = swiglu ? a->w3 : nullptr;
  p1.bd1 = a->ws1;
  p1.bd3 = swiglu ? a->ws3 : nullptr;
  p1.s1 = a->s1;
  p1.s3 = a->s3;
  p1.sd1 = a->ss1;
  p1.sd3 = a->ss3;
  p1.off = a->expert_off;
  p1.e_begin = a->e_begin;
  p1.n_routed = n_routed;
  p1.a_shift = 0;
  p1.c_shift = 1;
  p1.t_dense = a->x_dense ? a->T_dense : 0;
  p1.K = d;
  p1.N = swiglu ? 2 * h : h;
  p1.ldc = h;
  p1.b_stride = (int64_t)h * d;
  p1.ks = d / 128;
  p1.ns = h / 128;
  p1.b_tiled = a->w_layout == MOE_W_TILED16 ? 1 : 0;
  p1.partial = partial;
  p1.ksplit = pl.ks1;
  p1.max_rows = rows;
  p1.prow_total = rows + p1.t_dense;

  GroupedParams p2 = p1;
  p2.a_routed = act_routed;
  p2.a_dense = act_dense;
  p2.c_routed = a->y_send;
  p2.c_dense = a->y_dense;
  p2.b1 = a->w2;
  p2.b3 = nullptr;
  p2.bd1 = a->ws2;
  p2.bd3 = nullptr;
  p2.s1 = a->s2;
  p2.s3 = nullptr;
  p2.sd1 = a->ss2;
  p2.sd3 = nullptr;
  p2.a_shift = 1;
  p2.c_shift = 0;
  p2.K = h;
  p2.N = d;
  p2.ldc = d;
  p2.b_stride = (int64_t)d * h;
  p2.ks = h / 128;
  p2.ns = d / 128;
  p2.ksplit = pl.ks2;

  const bool streaming = small_m && sizeof(AT) == 2;
  if (!streaming && p1.b_tiled &&
      (sizeof(AT) == 4 || !dma_gemm_supported(p1, BSRC) ||
       !dma_gemm_supported(p2, BSRC))) {
    set_error("moe_expert_ffn: tiled weights need bf16 activations and, off the streaming path, "
              "h and d multiples of 256 (fp8 weights: at most 16384)");
    return MOE_ERR_UNSUPPORTED;
  }
  if (check_only()) return MOE_OK;
  moe_status st;
  if (streaming) {
    st = launch_stream_gemm1_any(BSRC, a->act, p1, stream);
    if (st != MOE_OK) return st;
    if (mid_event) MOE_CHECK_HIP(hipEventRecord(mid_event, stream));
    st = launch_stream_gemm2_any(BSRC, p2, stream);
  } else if (sizeof(AT) == 4) {
    p1.ksplit = p2.ksplit = 1;
    constexpr int FT = sizeof(AT) == 4 ? kF32Tile : 128;
    constexpr int FB = FT == 128 ? 2 : kF32Minb;
    st = launch_gemm1<AT, BSRC, FT, FT, 2, 2, FB>(a->act, p1, rows, stream);
    if (st != MOE_OK) return st;
    if (mid_event) MOE_CHECK_HIP(hipEventRecord(mid_event, stream));
    st = launch<AT, AT, BSRC, EPI_NONE, FT, FT, 2, 2, FB>(p2, rows, stream);
  } else if (dma_gemm_supported(p1, BSRC) && dma_gemm_supported(p2, BSRC)) {
    p1.ksplit = p2.ksplit = 1;
    const int epi1 = a->act == MOE_RELU ? EPI_RELU : (a->act == MOE_GELU ? EPI_GELU : EPI_SWIGLU);
    st = launch_dma_gemm(BSRC, epi1, p1, rows, stream);
    if (st != MOE_OK) return st;
    if (mid_event) MOE_CHECK_HIP(hipEventRecord(mid_event, stream));
    st = launch_dma_gemm(BSRC, EPI_NONE, p2, rows, stream);
  } else {
    p1.ksplit = p2.ksplit = 1;
    st = launch_gemm1<AT, BSRC, kBigBm, kBigBn, 2, 2, kBigMinb>(a->act, p1, rows, stream);
    if (st != MOE_OK) return st;
    if (mid_event) MOE_CHECK_HIP(hipEventRecord(mid_event, stream));
    st = launch<AT, AT, BSRC, EPI_NONE, kBigBm, kBigBn, 2, 2, kBigMinb>(p2, rows, stream);
  }
  return st;
}

}  // namespace

// K slices of the router logits GEMM on the LDS-DMA kernel (E a multiple
// of 256: whole 256-wide tiles; 256-row tiles): enough (tile, slice) work
// items for kLogitsWgPerCu per CU, at most kLogitsMaxKs.  Each slice writes
// and re-reads T x E fp32 partials, so more slices are not free.  On the
// DeepSeek-V3 share (T = 8192, E = 256, cache-cold) 8 slices of 256-row
// tiles (one item per CU, two waves per SIMD) route in 74 us; 128-row tiles
// of 4 waves took 79-80 us with 4 slices (one item per CU) whether their
// ring held 3, 5 or 6 stages, and 81 us with 8 slices (two per CU).
constexpr int kLogitsWgPerCu = 1;
constexpr int kLogitsMaxKs = 16;
int dense_logits_ksplit(int64_t T, int d, int E) {
  if (E % 256 != 0 || d % BKE_DMA != 0) return 1;
  const int64_t m_tiles = (T + 255) / 256;
  const int64_t target = kLogitsWgPerCu * (int64_t)device_info().cus;
  int ks = 1;
  while (ks < kLogitsMaxKs && m_tiles * ks < target && (d / BKE_DMA) % (2 * ks) == 0) ks *= 2;
  return ks;
}

moe_status dense_logits_gemm(const void* x, const void* w_router, float* out, int64_t T, int d,
                             int E, hipStream_t stream) {
  if (E % 256 == 0 && d % BKE_DMA == 0) {
    GroupedParams p{};
    p.a_dense = x;
    p.bd1 = w_router;
    p.n_routed = 0;
    p.t_dense = T;
    p.K = d;
    p.N = E;
    p.ldc = E;
    p.partial = out;
    p.ksplit = dense_logits_ksplit(T, d, E);
    p.prow_total = T;
    p.max_rows = 0;
    return launch_dma_partial(p, stream);
  }
  GroupedParams p{};
  p.a_dense = x;
  p.c_dense = out;
  p.bd1 = w_router;
  p.n_routed = 0;
  p.t_dense = T;
  p.K = d;
  p.N = E;
  p.ldc = E;
  p.ksplit = 1;
  return launch<bf16_t, float, B_SAME, EPI_NONE, 128, 64, 2, 2, 2>(p, 0, stream);
}

// Internal: FFN with an optional event recorded between the two GEMMs.
moe_status expert_ffn_impl(const moe_ffn_args* a, void* ws, size_t ws_bytes, hipStream_t stream,
                           hipEvent_t mid_event);

}  // namespace moe

using namespace moe;

extern "C" size_t moe_ffn_workspace_bytes(const moe_ffn_args* a) {
  if (!a) return 0;
  const FfnPlan pl = plan_ffn(a);
  return pl.act_bytes + pl.partial_bytes;
}

moe_status moe::expert_ffn_impl(const moe_ffn_args* a, void* ws, size_t ws_bytes,
                                hipStream_t stream, hipEvent_t mid_event) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, "null args");
  MOE_CHECK_ARG(a->d >= 128 && a->d % 128 == 0, "d must be a positive multiple of 128");
  MOE_CHECK_ARG(a->h >= 128 && a->h % 128 == 0, "h must be a positive multiple of 128");
  MOE_CHECK_ARG(a->E >= 1 && a->E <= MOE_MAX_EXPERTS, "E out of range [1, 256]");
  MOE_CHECK_ARG(0 <= a->e_begin && a->e_begin <= a->e_end && a->e_end <= a->E,
                "need 0 <= e_begin <= e_end <= E");
  MOE_CHECK_ARG(a->act == MOE_RELU || a->act == MOE_GELU || a->act == MOE_SWIGLU, "bad act");
  MOE_CHECK_ARG(a->w_layout == MOE_W_ROWMAJOR || a->w_layout == MOE_W_TILED16, "bad w_layout");
  MOE_CHECK_ARG(a->max_rows >= 0 && a->T_dense >= 0, "negative row count");
  MOE_CHECK_ARG(a->max_rows + a->T_dense < (int64_t)1 << 31, "row count must fit in int32");
  const bool f32 = a->act_dtype == MOE_F32;
  MOE_CHECK_ARG(f32 || a->act_dtype == MOE_BF16, "bad act_dtype");
  if (f32) {
    MOE_CHECK_ARG(a->w_dtype == MOE_F32, "fp32 activations need fp32 weights");
  } else if (a->w_dtype != MOE_BF16 && a->w_dtype != MOE_FP8_E4M3) {
    set_error("moe_expert_ffn: bf16 activations need bf16 or fp8 weights");
    return MOE_ERR_UNSUPPORTED;
  }
  const bool fp8 = a->w_dtype == MOE_FP8_E4M3;
  const bool swiglu = a->act == MOE_SWIGLU;
  const int n_routed = a->e_end - a->e_begin;
  if (n_routed > 0) {
    MOE_CHECK_ARG(a->x_send && a->y_send && a->expert_off && a->w1 && a->w2,
                  "routed experts need x_send, y_send, expert_off, w1, w2");
    MOE_CHECK_ARG(!swiglu || a->w3, "SwiGLU needs w3");
    MOE_CHECK_ARG(!fp8 || (a->s1 && a->s2 && (!swiglu || a->s3)), "fp8 weights need scales");
    MOE_CHECK_ARG(aligned16(a->x_send) && aligned16(a->y_send) && aligned16(a->w1) &&
                      aligned16(a->w2) && (!swiglu || aligned16(a->w3)),
                  "routed pointers not 16-byte aligned");
  }
  if (a->T_dense > 0 && a->x_dense) {
    MOE_CHECK_ARG(a->y_dense && a->ws1 && a->ws2 && (!swiglu || a->ws3),
                  "shared expert needs y_dense, ws1, ws2 (, ws3)");
    MOE_CHECK_ARG(!fp8 || (a->ss1 && a->ss2 && (!swiglu || a->ss3)), "fp8 shared expert needs scales");
    MOE_CHECK_ARG(aligned16(a->x_dense) && aligned16(a->y_dense), "dense pointers not aligned");
  }
  const size_t need = moe_ffn_workspace_bytes(a);
  if (ws_bytes < need || (need && !ws)) {
    set_error("moe_expert_ffn: workspace too small");
    return MOE_ERR_WORKSPACE;
  }
  const int groups = n_routed + ((a->x_dense && a->T_dense > 0) ? 1 : 0);
  if (groups == 0 && check_only()) return MOE_OK;
  if (groups == 0) {
    if (mid_event) MOE_CHECK_HIP(hipEventRecord(mid_event, stream));
    return MOE_OK;
  }
  const FfnPlan pl = plan_ffn(a);
  if (f32) return run_ffn<float, B_SAME>(a, pl, ws, stream, mid_event);
  if (fp8) return run_ffn<bf16_t, B_FP8>(a, pl, ws, stream, mid_event);
  return run_ffn<bf16_t, B_SAME>(a, pl, ws, stream, mid_event);
}

extern "C" moe_status moe_expert_ffn(const moe_ffn_args* a, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
  return moe::expert_ffn_impl(a, ws, ws_bytes, stream, nullptr);
}
