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
//  * SwiGLU: a wave's B rows are w1 rows and the w3 rows of the same output
//    columns, so silu(z1) * z3 is formed in registers.
#include <math.h>

#include "gemm.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Epi { EPI_NONE = 0, EPI_RELU = 1, EPI_GELU = 2, EPI_SWIGLU = 3 };
enum BSrc { B_SAME = 0, B_FP8 = 1 };

constexpr int kThreads = 256;
constexpr int kMaxGroups = MOE_MAX_EXPERTS + 1;
constexpr int kRowBytes = 128;              // one K-stage of a tile row
constexpr int kLdsRow = kRowBytes + 16;     // padded LDS row
constexpr int kGM = 4;                      // m-tiles per strip

struct GroupedParams {
  const void* a_routed;
  const void* a_dense;
  void* c_routed;
  void* c_dense;
  const void* b1;   // routed weights [n_routed][rows][K]
  const void* b3;   // SwiGLU partner weights, or null
  const void* bd1;  // dense weights [rows][K]
  const void* bd3;
  const float* s1;  // fp8 scales, routed [n_routed][ns][ks]
  const float* s3;
  const float* sd1;
  const float* sd3;
  const int32_t* off;  // expert offsets [E+1]
  int e_begin;
  int n_routed;
  int a_shift;  // 1: A row = send row - off[e_begin]
  int c_shift;  // 1: C row = send row - off[e_begin]
  int64_t t_dense;
  int K;        // reduction length (elements)
  int N;        // B rows covered by the tile grid (SwiGLU: 2 x output columns)
  int ldc;      // output columns
  int64_t b_stride;  // elements between two experts' weight matrices
  int ks;       // K / 128
  int ns;       // output-dim / 128 (scale rows)
  // split-K (weight-streaming kernel only): ksplit > 1 writes fp32 partial
  // sums [ksplit][prow_total][nmat * out_cols] to `partial`; partial rows are
  // the group rows relative to off[e_begin], then the dense rows at max_rows.
  float* partial;
  int ksplit;
  int64_t prow_total;
  int64_t max_rows;
};

template <typename AT>
struct ATraits;
template <>
struct ATraits<float> {
  static constexpr int kElems16 = 4;
};
template <>
struct ATraits<bf16_t> {
  static constexpr int kElems16 = 8;
};

__device__ __forceinline__ float act_gelu(float v) {
  return 0.5f * v * (1.f + erff(v * 0.70710678118654752440f));
}
__device__ __forceinline__ float act_silu(float v) { return v / (1.f + __expf(-v)); }

template <typename CT>
__device__ __forceinline__ void store_out(CT* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t* p, float v) {
  *p = (bf16_t)f32_to_bf16(v);
}

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
          int MINB>
__global__ void __launch_bounds__(kThreads, MINB) grouped_gemm_kernel(GroupedParams p) {
  static_assert(WAVES_M * WAVES_N == kThreads / 64, "4 waves");
  constexpr int WTM = BM / WAVES_M;  // rows per wave
  constexpr int WTN = BN / WAVES_N;  // B rows per wave
  constexpr int TM = WTM / 16;
  constexpr int TN = WTN / 16;
  static_assert(EPI != EPI_SWIGLU || TN % 2 == 0, "SwiGLU pairs subtiles");
  constexpr int BK = kRowBytes / (int)sizeof(AT);  // elements per K-stage
  constexpr int A_CH = BM * 8 / kThreads;            // 16-byte chunks per thread
  constexpr int B_CH = BN * 8 / kThreads;
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
    // A chunk i: row = c >> 3, 16-byte column cc = c & 7 of the K-stage
    const unsigned char* a_src[A_CH];
    bool a_ok[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3;
      a_ok[i] = (m0 + r) < rows;
      a_src[i] = reinterpret_cast<const unsigned char*>(A + (int64_t)(a_ok[i] ? m0 + r : 0) * p.K) +
                 (c & 7) * 16;
    }
    const unsigned char* b_src[B_CH];
    const float* b_scale[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * kThreads;
      const int r = c >> 3;
      int which = 0, orow;
      if (EPI == EPI_SWIGLU) {
        const int w_ = r / WTN, rr = r % WTN;
        which = rr / (WTN / 2);
        orow = n_t * (BN / 2) + w_ * (WTN / 2) + rr % (WTN / 2);
      } else {
        orow = n_t * BN + r;
      }
      const unsigned char* base = which ? B3 : B1;
      if (BSRC == B_FP8) {
        b_src[i] = base + (int64_t)orow * p.K + (c & 7) * 8;
        const float* sb = which ? S3 : S1;
        b_scale[i] = sb + (int64_t)(orow / 128) * p.ks;
      } else {
        b_src[i] = base + (int64_t)orow * p.K * sizeof(AT) + (c & 7) * 16;
        b_scale[i] = nullptr;
      }
    }

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[A_CH];
    u32x4 rb[B_CH];
    const int KT = p.K / BK;

#define MOE_GEMM_LOAD_STAGE(KT_)                                                        \
    {                                                                                   \
      const int64_t kb = (int64_t)(KT_) * kRowBytes;                                    \
      _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                \
        const u32x4 v = *reinterpret_cast<const u32x4*>(a_src[i] + kb);                 \
        const uint32_t m = a_ok[i] ? 0xffffffffu : 0u;                                  \
        ra[i] = v & m;                                                                  \
      }                                                                                 \
      _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                \
        if constexpr (BSRC == B_FP8) {                                                  \
          const uint2 q = *reinterpret_cast<const uint2*>(b_src[i] + (int64_t)(KT_) * BK); \
          const float sc = b_scale[i][((KT_) * BK) / 128];                              \
          rb[i].x = pack_bf16x2(e4m3_to_f32(q.x & 0xffu) * sc,                          \
                                e4m3_to_f32((q.x >> 8) & 0xffu) * sc);                  \
          rb[i].y = pack_bf16x2(e4m3_to_f32((q.x >> 16) & 0xffu) * sc,                  \
                                e4m3_to_f32(q.x >> 24) * sc);                           \
          rb[i].z = pack_bf16x2(e4m3_to_f32(q.y & 0xffu) * sc,                          \
                                e4m3_to_f32((q.y >> 8) & 0xffu) * sc);                  \
          rb[i].w = pack_bf16x2(e4m3_to_f32((q.y >> 16) & 0xffu) * sc,                  \
                                e4m3_to_f32(q.y >> 24) * sc);                           \
        } else {                                                                        \
          rb[i] = *reinterpret_cast<const u32x4*>(b_src[i] + kb);                       \
        }                                                                               \
      }                                                                                 \
    }
#define MOE_GEMM_STORE_STAGE(BUF_)                                                      \
    {                                                                                   \
      unsigned char* la_ = lds_a + (BUF_) * BM * kLdsRow;                               \
      unsigned char* lb_ = lds_b + (BUF_) * BN * kLdsRow;                               \
      _Pragma("unroll") for (int i = 0; i < A_CH; ++i) {                                \
        const int c = tid + i * kThreads;                                               \
        *reinterpret_cast<u32x4*>(la_ + (c >> 3) * kLdsRow + (c & 7) * 16) = ra[i];      \
      }                                                                                 \
      _Pragma("unroll") for (int i = 0; i < B_CH; ++i) {                                \
        const int c = tid + i * kThreads;                                               \
        *reinterpret_cast<u32x4*>(lb_ + (c >> 3) * kLdsRow + (c & 7) * 16) = rb[i];      \
      }                                                                                 \
    }

    MOE_GEMM_LOAD_STAGE(0);
    __syncthreads();  // previous tile's LDS reads are complete
    MOE_GEMM_STORE_STAGE(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const bool more = kt + 1 < KT;
      if (more) MOE_GEMM_LOAD_STAGE(kt + 1);
      const unsigned char* la = lds_a + (kt & 1) * BM * kLdsRow;
      const unsigned char* lb = lds_b + (kt & 1) * BN * kLdsRow;
#pragma unroll
      for (int step = 0; step < 2; ++step) {
        const int chunk = (lane >> 4) + 4 * step;
        u32x4 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[i] = *reinterpret_cast<const u32x4*>(la + (wm * WTM + i * 16 + (lane & 15)) * kLdsRow +
                                                  chunk * 16);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          bfr[j] = *reinterpret_cast<const u32x4*>(lb + (wn * WTN + j * 16 + (lane & 15)) * kLdsRow +
                                                   chunk * 16);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (sizeof(AT) == 2) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bfr[j]),
                  acc[i][j], 0, 0, 0);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  __uint_as_float(af[i].x), __uint_as_float(bfr[j].x), acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  __uint_as_float(af[i].y), __uint_as_float(bfr[j].y), acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  __uint_as_float(af[i].z), __uint_as_float(bfr[j].z), acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(
                  __uint_as_float(af[i].w), __uint_as_float(bfr[j].w), acc[i][j], 0, 0, 0);
            }
          }
        }
      }
      if (more) MOE_GEMM_STORE_STAGE((kt + 1) & 1);
      __syncthreads();
    }
#undef MOE_GEMM_LOAD_STAGE
#undef MOE_GEMM_STORE_STAGE

    // ---- epilogue: lane holds rows 4*(lane/16) + r, column lane % 16 of each subtile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + r;
        if (row >= rows) continue;
        CT* crow = C + (int64_t)row * p.ldc;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < TN / 2; ++j) {
            const int col = n_t * (BN / 2) + wn * (WTN / 2) + j * 16 + (lane & 15);
            const float z1 = acc[i][j][r];
            const float z3 = acc[i][j + TN / 2][r];
            store_out<CT>(crow + col, act_silu(z1) * z3);
          }
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n_t * BN + wn * WTN + j * 16 + (lane & 15);
            float v = acc[i][j][r];
            if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
            if (EPI == EPI_GELU) v = act_gelu(v);
            store_out<CT>(crow + col, v);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- weight streaming
// Decode-sized groups (at most a few tens of rows per expert) are bound by
// streaming the expert weights from HBM once.  Each wave owns 16 output
// columns of one group (for SwiGLU the 16 w1 rows and the 16 matching w3
// rows) and walks the whole K extent: its B fragments go from global memory
// straight into registers (no LDS), double buffered one K-chunk ahead, with
// each lane reading CK/2 contiguous bytes of a weight row per chunk.  The
// group's rows (<= 64 per pass) are staged through LDS once per chunk and
// shared by the block's 4 waves.  Inside a chunk the lane groups q = lane/16
// own disjoint K ranges; the same K permutation is applied to the A
// fragments read from LDS, so every MFMA still sums over 32 distinct k.
// Tuning of the weight-streaming kernel: K chunk and minimum waves per SIMD
// for the SwiGLU pair and for single-matrix GEMMs, and whether row subtiles
// past a group's rows are skipped (branches) or computed on padding rows.
#ifndef MOE_SG_CK
#define MOE_SG_CK 64
#endif
#ifndef MOE_SG_MINW
#define MOE_SG_MINW 4
#endif
#ifndef MOE_SG_SKIP
#define MOE_SG_SKIP 1
#endif
#ifndef MOE_DN_CK
#define MOE_DN_CK 64
#endif
#ifndef MOE_DN_MINW
#define MOE_DN_MINW 4
#endif
#ifndef MOE_DN_SKIP
#define MOE_DN_SKIP 0
#endif

template <int BSRC, int EPI, int CK, int MINW>
__global__ void __launch_bounds__(kThreads, MINW) stream_gemm_kernel(GroupedParams p) {
  constexpr int NMAT = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int V = CK / 32;                 // 16-byte bf16 pieces per lane per matrix
  constexpr int RS = CK * 2 + 16;            // LDS row stride (bytes)
  constexpr int MROWS = 64;                  // rows per pass
  constexpr int A_PIECES = MROWS * CK * 2 / 16 / kThreads;  // 16-byte A pieces per thread
  constexpr int QB = CK / 4;                 // K elements per lane group per chunk
  constexpr bool SKIP = (EPI == EPI_SWIGLU) ? MOE_SG_SKIP : MOE_DN_SKIP;
  static_assert(A_PIECES >= 1, "chunk too small");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* lds_a = smem;  // [2][MROWS][RS]

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / 64;
  const int q = lane >> 4;
  const int g = blockIdx.y;
  const bool dense = g >= p.n_routed;
  int rows, r0 = 0;
  if (!dense) {
    r0 = p.off[p.e_begin + g];
    rows = p.off[p.e_begin + g + 1] - r0;
  } else {
    rows = (int)p.t_dense;
  }
  if (rows <= 0) return;
  const int a_sub = (p.a_shift && p.n_routed > 0) ? p.off[p.e_begin] : 0;
  const int c_sub = (p.c_shift && p.n_routed > 0) ? p.off[p.e_begin] : 0;
  const bf16_t* A = dense ? reinterpret_cast<const bf16_t*>(p.a_dense)
                          : reinterpret_cast<const bf16_t*>(p.a_routed) + (int64_t)(r0 - a_sub) * p.K;
  bf16_t* Cp = dense ? reinterpret_cast<bf16_t*>(p.c_dense)
                     : reinterpret_cast<bf16_t*>(p.c_routed) + (int64_t)(r0 - c_sub) * p.ldc;
  const int bes = BSRC == B_FP8 ? 1 : 2;
  const unsigned char* Bm[NMAT];
  const float* Sm[NMAT];
  {
    const unsigned char* b1 = dense ? reinterpret_cast<const unsigned char*>(p.bd1)
                                    : reinterpret_cast<const unsigned char*>(p.b1) + (int64_t)g * p.b_stride * bes;
    const float* s1 = dense ? p.sd1 : (p.s1 ? p.s1 + (int64_t)g * p.ns * p.ks : nullptr);
    Bm[0] = b1;
    Sm[0] = s1;
    if constexpr (NMAT == 2) {
      Bm[1] = dense ? reinterpret_cast<const unsigned char*>(p.bd3)
                    : reinterpret_cast<const unsigned char*>(p.b3) + (int64_t)g * p.b_stride * bes;
      Sm[1] = dense ? p.sd3 : (p.s3 ? p.s3 + (int64_t)g * p.ns * p.ks : nullptr);
    }
  }
  const int ocol0 = blockIdx.x * 64 + wave * 16;  // first output column of this wave
  const int brow = ocol0 + (lane & 15);            // the weight row this lane streams
  const int NC = p.K / CK / p.ksplit;       // chunks of this block's K slice
  const int cb = blockIdx.z * NC;           // first chunk of the slice

  // per-lane byte pointers into the weight rows (lane group q owns QB elements)
  const unsigned char* bptr[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) bptr[m] = Bm[m] + ((int64_t)brow * p.K + q * QB) * bes;

  u32x4 breg[2][NMAT][V];
  float bscale[2][NMAT];

#define MOE_STREAM_LOAD_B(BUF_, C_)                                                        \
  {                                                                                        \
    _Pragma("unroll") for (int m = 0; m < NMAT; ++m) {                                     \
      if constexpr (BSRC == B_FP8) {                                                       \
        const unsigned char* src_ = bptr[m] + (int64_t)(C_) * CK;                          \
        _Pragma("unroll") for (int v = 0; v < V / 2; ++v)                                  \
          breg[BUF_][m][v] = *reinterpret_cast<const u32x4*>(src_ + v * 16);               \
        bscale[BUF_][m] = Sm[m][(int64_t)(brow / 128) * p.ks + ((C_) * CK + q * QB) / 128]; \
      } else {                                                                             \
        const unsigned char* src_ = bptr[m] + (int64_t)(C_) * CK * 2;                      \
        _Pragma("unroll") for (int v = 0; v < V; ++v)                                      \
          breg[BUF_][m][v] = *reinterpret_cast<const u32x4*>(src_ + v * 16);               \
      }                                                                                    \
    }                                                                                      \
  }

  for (int m0 = 0; m0 < rows; m0 += MROWS) {
    const int mr = min(MROWS, rows - m0);
    const int mt = (mr + 15) / 16;
    // A staging: piece c = tid + i*256 of the chunk -> row c / PR, 16-byte
    // column c % PR.  Every thread loads and stores all its pieces (rows past
    // the group's end repeat its last row): no divergent branches, so the
    // compiler can count outstanding loads exactly and the weight prefetch
    // issued before the A store stays in flight.
    constexpr int PR = CK * 2 / 16;
    u32x4 areg[A_PIECES];
    const unsigned char* a_row[A_PIECES];
#pragma unroll
    for (int i = 0; i < A_PIECES; ++i) {
      const int c_ = tid + i * kThreads;
      const int rr_ = min(m0 + c_ / PR, rows - 1);
      a_row[i] = reinterpret_cast<const unsigned char*>(A + (int64_t)rr_ * p.K) + (c_ % PR) * 16;
    }
#define MOE_STREAM_LOAD_A(C_)                                                              \
    _Pragma("unroll") for (int i = 0; i < A_PIECES; ++i)                                   \
      areg[i] = *reinterpret_cast<const u32x4*>(a_row[i] + (int64_t)(C_) * CK * 2);
#define MOE_STREAM_STORE_A(BUF_)                                                           \
    _Pragma("unroll") for (int i = 0; i < A_PIECES; ++i) {                                 \
      const int c_ = tid + i * kThreads;                                                   \
      *reinterpret_cast<u32x4*>(lds_a + (BUF_) * MROWS * RS + (c_ / PR) * RS +             \
                                (c_ % PR) * 16) = areg[i];                                 \
    }

    f32x4 acc[NMAT][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    MOE_BARRIER_LDS();  // LDS of the previous pass is no longer read
    // Loads are never skipped (chunk indices are clamped instead): branches
    // around loads would make the compiler's wait-count tracking fall back
    // to draining every outstanding load.
    MOE_STREAM_LOAD_B(0, cb);
    MOE_STREAM_LOAD_B(1, cb + min(1, NC - 1));
    MOE_STREAM_LOAD_A(cb);
    MOE_STREAM_STORE_A(0);
    MOE_BARRIER_LDS();

#define MOE_STREAM_COMPUTE(BUF_)                                                           \
    {                                                                                      \
      const unsigned char* la_ = lds_a + (BUF_) * MROWS * RS;                              \
      _Pragma("unroll") for (int s = 0; s < V; ++s) {                                      \
        u32x4 bf[NMAT];                                                                    \
        _Pragma("unroll") for (int m = 0; m < NMAT; ++m) {                                 \
          if constexpr (BSRC == B_FP8) {                                                   \
            const u32x4 w8 = breg[BUF_][m][s / 2];                                         \
            const uint32_t lo = (s & 1) ? w8[2] : w8[0];                                   \
            const uint32_t hi = (s & 1) ? w8[3] : w8[1];                                   \
            const float sc = bscale[BUF_][m];                                              \
            bf[m][0] = pack_bf16x2(e4m3_to_f32(lo & 0xffu) * sc, e4m3_to_f32((lo >> 8) & 0xffu) * sc);   \
            bf[m][1] = pack_bf16x2(e4m3_to_f32((lo >> 16) & 0xffu) * sc, e4m3_to_f32(lo >> 24) * sc);    \
            bf[m][2] = pack_bf16x2(e4m3_to_f32(hi & 0xffu) * sc, e4m3_to_f32((hi >> 8) & 0xffu) * sc);   \
            bf[m][3] = pack_bf16x2(e4m3_to_f32((hi >> 16) & 0xffu) * sc, e4m3_to_f32(hi >> 24) * sc);    \
          } else {                                                                         \
            bf[m] = breg[BUF_][m][s];                                                      \
          }                                                                                \
        }                                                                                  \
        /* all 4 row subtiles, also past the group's rows: no branches here */             \
        _Pragma("unroll") for (int i = 0; i < 4; ++i) {                                    \
          if (SKIP && i >= mt) continue;                                                   \
          const u32x4 af = *reinterpret_cast<const u32x4*>(                                \
              la_ + (i * 16 + (lane & 15)) * RS + (q * QB + s * 8) * 2);                   \
          _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                 \
            acc[m][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                           \
                __builtin_bit_cast(bf16x8_t, af), __builtin_bit_cast(bf16x8_t, bf[m]),     \
                acc[m][i], 0, 0, 0);                                                       \
        }                                                                                  \
      }                                                                                    \
    }

    for (int c = 0; c < NC; c += 2) {
      // even chunk: buffers 0
      MOE_STREAM_LOAD_A(cb + min(c + 1, NC - 1));
      MOE_STREAM_COMPUTE(0);
      MOE_STREAM_LOAD_B(0, cb + min(c + 2, NC - 1));
      MOE_STREAM_STORE_A(1);
      MOE_BARRIER_LDS();
      if (c + 1 >= NC) break;
      // odd chunk: buffers 1
      MOE_STREAM_LOAD_A(cb + min(c + 2, NC - 1));
      MOE_STREAM_COMPUTE(1);
      MOE_STREAM_LOAD_B(1, cb + min(c + 3, NC - 1));
      MOE_STREAM_STORE_A(0);
      MOE_BARRIER_LDS();
    }
#undef MOE_STREAM_LOAD_A
#undef MOE_STREAM_STORE_A
#undef MOE_STREAM_COMPUTE

    // epilogue: lane holds rows 4*q + r of each 16-row subtile, column lane & 15
    const int out_cols = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
    const int64_t prow0 = dense ? p.max_rows : (int64_t)(r0 - (p.n_routed > 0 ? p.off[p.e_begin] : 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= mt) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + i * 16 + 4 * q + r;
        if (row >= rows) continue;
        const int col = ocol0 + (lane & 15);
        if (p.ksplit > 1) {
          float* dst = p.partial + ((int64_t)blockIdx.z * p.prow_total + prow0 + row) *
                                       (int64_t)(NMAT * out_cols) + col;
#pragma unroll
          for (int m = 0; m < NMAT; ++m) dst[m * out_cols] = acc[m][i][r];
          continue;
        }
        float v;
        if constexpr (EPI == EPI_SWIGLU) {
          v = act_silu(acc[0][i][r]) * acc[1][i][r];
        } else {
          v = acc[0][i][r];
          if (EPI == EPI_RELU) v = fmaxf(v, 0.f);
          if (EPI == EPI_GELU) v = act_gelu(v);
        }
        Cp[(int64_t)row * p.ldc + col] = (bf16_t)f32_to_bf16(v);
      }
    }
  }
#undef MOE_STREAM_LOAD_B
}

// Split-K reduction: sums the fp32 partials of each output element in slice
// order (deterministic), applies the activation and stores bf16.  Rows are
// the partial rows: executed groups' rows (count read from the offsets),
// then the dense rows.
template <int EPI>
__global__ void __launch_bounds__(kThreads) splitk_reduce_kernel(GroupedParams p, int64_t t_dense_rows) {
  constexpr int NMAT = (EPI == EPI_SWIGLU) ? 2 : 1;
  const int out_cols = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
  const int q4 = out_cols / 4;
  const int64_t i4 = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t prow = i4 / q4;
  const int col = (int)(i4 % q4) * 4;
  if (prow >= p.prow_total) return;
  const int base = p.n_routed > 0 ? p.off[p.e_begin] : 0;
  const int routed = p.n_routed > 0 ? p.off[p.e_begin + p.n_routed] - base : 0;
  bf16_t* dst;
  if (prow < p.max_rows) {
    if (prow >= routed) return;
    dst = reinterpret_cast<bf16_t*>(p.c_routed) + (prow + (p.c_shift ? 0 : base)) * p.ldc + col;
  } else {
    if (prow - p.max_rows >= t_dense_rows) return;
    dst = reinterpret_cast<bf16_t*>(p.c_dense) + (prow - p.max_rows) * p.ldc + col;
  }
  float4 s[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int z = 0; z < p.ksplit; ++z) {
    const float* src = p.partial + ((int64_t)z * p.prow_total + prow) * (int64_t)(NMAT * out_cols) + col;
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      const float4 v = *reinterpret_cast<const float4*>(src + m * out_cols);
      s[m].x += v.x;
      s[m].y += v.y;
      s[m].z += v.z;
      s[m].w += v.w;
    }
  }
  float o[4] = {s[0].x, s[0].y, s[0].z, s[0].w};
  if constexpr (EPI == EPI_SWIGLU) {
    const float g[4] = {s[NMAT - 1].x, s[NMAT - 1].y, s[NMAT - 1].z, s[NMAT - 1].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = act_silu(o[j]) * g[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (EPI == EPI_RELU) o[j] = fmaxf(o[j], 0.f);
      if (EPI == EPI_GELU) o[j] = act_gelu(o[j]);
    }
  }
  uint2 packed;
  packed.x = pack_bf16x2(o[0], o[1]);
  packed.y = pack_bf16x2(o[2], o[3]);
  *reinterpret_cast<uint2*>(dst) = packed;
}

// ---------------------------------------------------------------- launch

template <int BM, int BN>
constexpr size_t lds_bytes() {
  return 2 * (BM + BN) * kLdsRow + (3 * kMaxGroups + 1 + 4) * sizeof(int);
}

struct LaunchCfg {
  int grid;
};

template <typename AT, typename CT, int BSRC, int EPI, int BM, int BN, int WM, int WN, int MINB>
moe_status launch(const GroupedParams& p, int64_t max_routed_rows, hipStream_t stream) {
  auto kern = grouped_gemm_kernel<AT, CT, BSRC, EPI, BM, BN, WM, WN, MINB>;
  constexpr size_t lds = lds_bytes<BM, BN>();
  static bool attr_set = false;  // one dynamic-LDS opt-in per process
  if (!attr_set) {
    MOE_CHECK_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)lds));
    attr_set = true;
  }
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

template <int BSRC, int EPI, int CK>
moe_status launch_stream(const GroupedParams& p, hipStream_t stream) {
  auto kern = stream_gemm_kernel<BSRC, EPI, CK, (EPI == EPI_SWIGLU ? MOE_SG_MINW : MOE_DN_MINW)>;
  constexpr size_t lds = 2 * 64 * (CK * 2 + 16);
  static bool attr_set = false;
  if (!attr_set) {
    MOE_CHECK_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)lds));
    attr_set = true;
  }
  const int ngroups = p.n_routed + (p.t_dense > 0 ? 1 : 0);
  const int out_cols = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
  if (ngroups == 0) return MOE_OK;
  dim3 grid(out_cols / 64, ngroups, p.ksplit);
  kern<<<grid, kThreads, lds, stream>>>(p);
  MOE_CHECK_LAUNCH();
  if (p.ksplit > 1) {
    const int64_t n4 = p.prow_total * (out_cols / 4);
    splitk_reduce_kernel<EPI><<<(int)((n4 + kThreads - 1) / kThreads), kThreads, 0, stream>>>(
        p, p.t_dense);
    MOE_CHECK_LAUNCH();
  }
  return MOE_OK;
}

// K slices for the weight-streaming kernel: enough waves to keep about 12
// per CU streaming (the decode down-projection has few output columns and a
// long K), in powers of two that divide the chunk count.
#ifndef MOE_MAX_KSPLIT
#define MOE_MAX_KSPLIT 4
#endif
#ifndef MOE_KSPLIT_WAVES_PER_CU
#define MOE_KSPLIT_WAVES_PER_CU 12
#endif
int stream_ksplit(int ngroups, int out_cols, int K, int CK) {
  const int64_t waves = (int64_t)ngroups * (out_cols / 64) * 4;
  const int64_t target = (int64_t)device_info().cus * MOE_KSPLIT_WAVES_PER_CU;
  int ks = 1;
  while (ks < MOE_MAX_KSPLIT && waves * ks < target && (K / CK) % (2 * ks) == 0) ks *= 2;
  return ks;
}

int stream_ck_for(bool swiglu, int K) {
  const int ck = swiglu ? MOE_SG_CK : MOE_DN_CK;
  return K % ck == 0 ? ck : 128;
}

// The tuned K chunk when K allows it, else 128 (d and h are multiples of 128).
template <int BSRC, int EPI>
moe_status launch_stream_k(const GroupedParams& p, hipStream_t s) {
  constexpr int CK = EPI == EPI_SWIGLU ? MOE_SG_CK : MOE_DN_CK;
  if (p.K % CK == 0) return launch_stream<BSRC, EPI, CK>(p, s);
  return launch_stream<BSRC, EPI, 128>(p, s);
}

template <int BSRC>
moe_status launch_stream_gemm1(int act, const GroupedParams& p, hipStream_t s) {
  switch (act) {
    case MOE_RELU:
      return launch_stream_k<BSRC, EPI_RELU>(p, s);
    case MOE_GELU:
      return launch_stream_k<BSRC, EPI_GELU>(p, s);
    default:
      return launch_stream_k<BSRC, EPI_SWIGLU>(p, s);
  }
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

  moe_status st;
  if (small_m && sizeof(AT) == 2) {
    st = launch_stream_gemm1<BSRC>(a->act, p1, stream);
    if (st != MOE_OK) return st;
    if (mid_event) MOE_CHECK_HIP(hipEventRecord(mid_event, stream));
    st = launch_stream_k<BSRC, EPI_NONE>(p2, stream);
  } else {
    p1.ksplit = p2.ksplit = 1;
    st = launch_gemm1<AT, BSRC, 128, 128, 2, 2, 2>(a->act, p1, rows, stream);
    if (st != MOE_OK) return st;
    if (mid_event) MOE_CHECK_HIP(hipEventRecord(mid_event, stream));
    st = launch<AT, AT, BSRC, EPI_NONE, 128, 128, 2, 2, 2>(p2, rows, stream);
  }
  return st;
}

}  // namespace

moe_status dense_logits_gemm(const void* x, const void* w_router, float* out, int64_t T, int d,
                             int E, hipStream_t stream) {
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
