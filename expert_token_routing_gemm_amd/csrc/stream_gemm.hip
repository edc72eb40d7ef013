// Weight-streaming grouped GEMM for decode-sized expert groups (gfx950).
//
// Local expert compute: once the rows of an expert are gathered, experts
// run independently (Ultralytics glossary "Expert Parallelism", "How Tokens
// Move Between GPUs", step 3).  With a few tens of rows per expert the GEMMs
// are bound by reading every executed expert's weights from HBM once.
#include "gemm_common.h"

namespace moe {
namespace {

constexpr int kThreads = kGemmThreads;
// Waves per workgroup of the streaming kernel (they share one A staging).
// The SwiGLU GEMM may use another count that divides its output columns
// into whole rounds of resident workgroups (see stream_waves).
constexpr int kSgWaves = 8;
constexpr int kSgWavesAlt = 7;

// ---------------------------------------------------------------- weight streaming
// Decode-sized groups (at most a few tens of rows per expert) are bound by
// streaming the expert weights from HBM once.  Each wave owns 16 output
// columns of one group (for SwiGLU the 16 w1 rows and the 16 matching w3
// rows) and walks the whole K extent: its B fragments go from global memory
// straight into registers (no LDS), double buffered one K-chunk ahead, with
// each lane reading CK/2 contiguous bytes of a weight row per chunk.  The
// group's rows (<= 64 per pass) are staged through LDS once per chunk and
// shared by the block's waves.  Inside a chunk the lane groups q = lane/16
// own disjoint K ranges; the same K permutation is applied to the A
// fragments read from LDS, so every MFMA still sums over 32 distinct k.
// Tuning of the weight-streaming kernel: K chunk and minimum waves per SIMD
// for the SwiGLU pair and for single-matrix GEMMs, and whether row subtiles
// past a group's rows are skipped (branches) or computed on padding rows.
constexpr int kSgCk = 64;
constexpr int kSgMinw = 4;
constexpr bool kSgSkip = true;
constexpr int kDnCk = 64;
constexpr int kDnMinw = 4;
constexpr bool kDnSkip = false;
// Weights are read exactly once per launch.  On the tiled layout every load
// is a whole contiguous 1 KB piece, and nontemporal loads stream those
// faster from HBM; on row-major rows (64-byte pieces of 16 rows per load)
// they are slower, so they are used for tiles only.

template <bool TL>
__device__ __forceinline__ u32x4 load_stream(const unsigned char* ptr) {
  const u32x4* p = reinterpret_cast<const u32x4*>(ptr);
  if constexpr (TL) return __builtin_nontemporal_load(p);
  return *p;
}

// TL: weights in the 16-row tiled layout (each wave's loads of a chunk are
// whole contiguous 1 KB pieces; see moe_weight_tile) instead of row-major.
template <int BSRC, int EPI, int CK, int MINW, bool TL, int WAVES>
__global__ void __launch_bounds__(64 * WAVES, MINW) stream_gemm_kernel(GroupedParams p) {
  constexpr int kSgThreads = 64 * WAVES;
  constexpr int NMAT = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int V = CK / 32;                 // 16-byte bf16 pieces per lane per matrix
  constexpr int RS = CK * 2 + 16;            // LDS row stride (bytes)
  constexpr int MROWS = 64;                  // rows per pass
  constexpr int A_TOTAL = MROWS * CK * 2 / 16;  // 16-byte A pieces per chunk
  constexpr int A_PIECES = (A_TOTAL + kSgThreads - 1) / kSgThreads;  // per thread
  constexpr bool SKIP = (EPI == EPI_SWIGLU) ? kSgSkip : kDnSkip;
  static_assert(A_PIECES >= 1, "chunk too small");
  static_assert(BSRC != B_FP8 || CK <= 128, "one fp8 scale block per chunk");
  static_assert(BSRC != B_FP8 || CK >= 64, "fp8 chunks hold whole 16-byte loads per lane");
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
  const int ocol0 = blockIdx.x * (16 * WAVES) + wave * 16;  // first output column of this wave
  const int brow = ocol0 + (lane & 15);            // the weight row this lane streams
  const int NC = p.K / CK / p.ksplit;       // chunks of this block's K slice
  const int cb = blockIdx.z * NC;           // first chunk of the slice

  // per-lane byte pointers into the weight rows
  const unsigned char* bptr[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
    bptr[m] = TL ? Bm[m] + (int64_t)ocol0 * p.K * bes + lane * 16
                 : Bm[m] + (int64_t)brow * p.K * bes + q * 16;
  // bytes between a lane's loads in a chunk: each 16-byte load of the wave
  // covers 64 contiguous bytes of each of its 16 weight rows (row-major) or
  // one whole 1 KB tile piece (tiled)
  constexpr int VSTEP = TL ? 1024 : 64;
  const int64_t cstride = TL ? (int64_t)CK * bes * 16 : (int64_t)CK * bes;  // per chunk
  // K offset (elements, inside the chunk) of the 8 values lane group q feeds
  // to MFMA step s; the A fragments use the same map
  auto koff = [&](int s_) {
    if constexpr (BSRC == B_FP8) return (s_ >> 1) * 64 + q * 16 + (s_ & 1) * 8;
    return s_ * 32 + q * 8;
  };

  u32x4 breg[2][NMAT][V];
  float bscale[2][NMAT];

#define MOE_STREAM_LOAD_B(BUF_, C_)                                                        \
  {                                                                                        \
    _Pragma("unroll") for (int m = 0; m < NMAT; ++m) {                                     \
      if constexpr (BSRC == B_FP8) {                                                       \
        const unsigned char* src_ = bptr[m] + (int64_t)(C_) * cstride;                     \
        _Pragma("unroll") for (int v = 0; v < V / 2; ++v)                                  \
          breg[BUF_][m][v] = load_stream<TL>(src_ + v * VSTEP);                                \
        bscale[BUF_][m] = Sm[m][(int64_t)(brow / 128) * p.ks + ((C_) * CK) / 128];         \
      } else {                                                                             \
        const unsigned char* src_ = bptr[m] + (int64_t)(C_) * cstride;                     \
        _Pragma("unroll") for (int v = 0; v < V; ++v)                                      \
          breg[BUF_][m][v] = load_stream<TL>(src_ + v * VSTEP);                                \
      }                                                                                    \
    }                                                                                      \
  }

  for (int m0 = 0; m0 < rows; m0 += MROWS) {
    const int mr = min(MROWS, rows - m0);
    const int mt = (mr + 15) / 16;
    // A staging: piece c = min(tid + i * threads, A_TOTAL - 1) of the chunk
    // -> row c / PR, 16-byte column c % PR.  Every thread loads and stores
    // all its pieces (rows past the group's end repeat its last row; threads
    // past the last piece repeat it, storing the same bytes): no divergent
    // branches, so the compiler can count outstanding loads exactly and the
    // weight prefetch issued before the A store stays in flight.
    constexpr int PR = CK * 2 / 16;
    u32x4 areg[A_PIECES];
    const unsigned char* a_row[A_PIECES];
#pragma unroll
    for (int i = 0; i < A_PIECES; ++i) {
      const int c_ = min(tid + i * kSgThreads, A_TOTAL - 1);
      const int rr_ = min(m0 + c_ / PR, rows - 1);
      a_row[i] = reinterpret_cast<const unsigned char*>(A + (int64_t)rr_ * p.K) + (c_ % PR) * 16;
    }
#define MOE_STREAM_LOAD_A(C_)                                                              \
    _Pragma("unroll") for (int i = 0; i < A_PIECES; ++i)                                   \
      areg[i] = *reinterpret_cast<const u32x4*>(a_row[i] + (int64_t)(C_) * CK * 2);
#define MOE_STREAM_STORE_A(BUF_)                                                           \
    _Pragma("unroll") for (int i = 0; i < A_PIECES; ++i) {                                 \
      const int c_ = min(tid + i * kSgThreads, A_TOTAL - 1);                               \
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
    // Weights of the next chunk are in flight while a chunk is computed; the
    // group's rows of the next chunk are fetched during the compute and
    // stored to the other LDS buffer before the barrier.
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
              la_ + (i * 16 + (lane & 15)) * RS + koff(s) * 2);                             \
          _Pragma("unroll") for (int m = 0; m < NMAT; ++m)                                 \
            acc[m][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(                           \
                __builtin_bit_cast(bf16x8_t, af), __builtin_bit_cast(bf16x8_t, bf[m]),     \
                acc[m][i], 0, 0, 0);                                                       \
        }                                                                                  \
      }                                                                                    \
    }

    // Steady state: every weight load is a chunk still to be computed (an odd
    // chunk count re-reads its last chunk once); the last one or two chunks
    // are computed after the loop without further weight loads.
    int c = 0;
    for (; c + 2 < NC; c += 2) {
      MOE_STREAM_LOAD_A(cb + c + 1);
      MOE_STREAM_COMPUTE(0);
      MOE_STREAM_LOAD_B(0, cb + c + 2);
      MOE_STREAM_STORE_A(1);
      MOE_BARRIER_LDS();
      MOE_STREAM_LOAD_A(cb + c + 2);
      MOE_STREAM_COMPUTE(1);
      MOE_STREAM_LOAD_B(1, cb + min(c + 3, NC - 1));
      MOE_STREAM_STORE_A(0);
      MOE_BARRIER_LDS();
    }
    MOE_STREAM_LOAD_A(cb + min(c + 1, NC - 1));
    MOE_STREAM_COMPUTE(0);
    MOE_STREAM_STORE_A(1);
    MOE_BARRIER_LDS();
    if (c + 1 < NC) MOE_STREAM_COMPUTE(1);
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

// Waves per workgroup of the SwiGLU streaming GEMM.  Each wave streams
// 16 output columns over the whole K slice, so all workgroups carry the
// same bytes and a grid that ends in a partial round of resident
// workgroups leaves slots idle at its end.  The alternative count is taken
// when it divides the columns and fills its last round better.  Measured on
// the decode Mixtral layer (h = 14336, 8 experts): 896 workgroups of 8
// waves are 1.75 rounds of 2 per CU, 1024 of 7 waves exactly 2; GEMM 1
// takes 308 instead of 329 us (14-wave workgroups, 1 round: 318 us).
int stream_waves(int out_cols, int ngroups, int ksplit) {
  if (out_cols % (16 * kSgWavesAlt) != 0) return kSgWaves;
  const int64_t slots_per_cu = 4 * kSgMinw;  // resident waves per CU at the VGPR budget
  const int64_t cus = device_info().cus;
  auto frac_tail = [&](int w) {  // fraction of the last round's slots that are busy
    const int64_t per = cus * (slots_per_cu / w);
    const int64_t wg = (int64_t)out_cols / (16 * w) * ngroups * ksplit;
    const int64_t r = wg % per;
    return r == 0 ? 1.0 : (double)r / per;
  };
  return frac_tail(kSgWavesAlt) > frac_tail(kSgWaves) ? kSgWavesAlt : kSgWaves;
}

template <int BSRC, int EPI, int CK, int WAVES>
moe_status launch_stream_w(const GroupedParams& p, int ngroups, int out_cols, hipStream_t stream) {
  constexpr int MW = EPI == EPI_SWIGLU ? kSgMinw : kDnMinw;
  auto kern = p.b_tiled ? stream_gemm_kernel<BSRC, EPI, CK, MW, true, WAVES>
                        : stream_gemm_kernel<BSRC, EPI, CK, MW, false, WAVES>;
  constexpr size_t lds = 2 * 64 * (CK * 2 + 16);
  static_assert(lds <= 64 * 1024, "within the default LDS limit");
  dim3 grid(out_cols / (16 * WAVES), ngroups, p.ksplit);
  kern<<<grid, 64 * WAVES, lds, stream>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

template <int BSRC, int EPI, int CK>
moe_status launch_stream(const GroupedParams& p, hipStream_t stream) {
  const int ngroups = p.n_routed + (p.t_dense > 0 ? 1 : 0);
  const int out_cols = (EPI == EPI_SWIGLU) ? p.N / 2 : p.N;
  if (ngroups == 0) return MOE_OK;
  moe_status st;
  if (EPI == EPI_SWIGLU && stream_waves(out_cols, ngroups, p.ksplit) == kSgWavesAlt)
    st = launch_stream_w<BSRC, EPI, CK, kSgWavesAlt>(p, ngroups, out_cols, stream);
  else
    st = launch_stream_w<BSRC, EPI, CK, kSgWaves>(p, ngroups, out_cols, stream);
  if (st != MOE_OK) return st;
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
}  // namespace

constexpr int kMaxKsplit = 4;
constexpr int kKsplitWavesPerCu = 12;
int stream_ksplit(int ngroups, int out_cols, int K, int CK) {
  const int64_t waves = (int64_t)ngroups * (out_cols / 16);
  const int64_t target = (int64_t)device_info().cus * kKsplitWavesPerCu;
  int ks = 1;
  while (ks < kMaxKsplit && waves * ks < target && (K / CK) % (2 * ks) == 0) ks *= 2;
  return ks;
}

int stream_ck_for(bool swiglu, int K) {
  const int ck = swiglu ? kSgCk : kDnCk;
  return K % ck == 0 ? ck : 128;
}

// The tuned K chunk when K allows it, else 128 (d and h are multiples of 128).
namespace {

template <int BSRC, int EPI>
moe_status launch_stream_k(const GroupedParams& p, hipStream_t s) {
  constexpr int CK0 = EPI == EPI_SWIGLU ? kSgCk : kDnCk;
  constexpr int CK = (BSRC == B_FP8 && CK0 < 64) ? 64 : CK0;
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

}  // namespace

moe_status launch_stream_gemm1_any(int bsrc, int act, const GroupedParams& p, hipStream_t s) {
  return bsrc == B_FP8 ? launch_stream_gemm1<B_FP8>(act, p, s) : launch_stream_gemm1<B_SAME>(act, p, s);
}

moe_status launch_stream_gemm2_any(int bsrc, const GroupedParams& p, hipStream_t s) {
  return bsrc == B_FP8 ? launch_stream_k<B_FP8, EPI_NONE>(p, s) : launch_stream_k<B_SAME, EPI_NONE>(p, s);
}

}  // namespace moe
