// Grouped expert GEMM for many-row bf16 groups (prefill), gfx950.
//
// Local expert compute (Ultralytics glossary "Expert Parallelism", "How
// Tokens Move Between GPUs", step 3): each executed expert multiplies its
// gathered rows by its own weights, independently of the others.
//
// Design (MI355X-specific):
//  * 256x256 output tile per workgroup of 8 waves (2 per SIMD); each wave
//    owns 128x64 as 4x2 v_mfma_f32_32x32x16_bf16 subtiles (the full-rate bf16
//    MFMA on gfx950; 128 fp32 accumulators per lane).  bf16 GEMMs without an
//    activation use 4 waves of 128x128 (256 accumulators per lane in
//    AccVGPRs, one wave per SIMD), each stage's DMA split over its two
//    k-steps.  Groups averaging a few hundred rows (with no shared expert)
//    use 128x256 tiles of 4 waves, two workgroups per CU, or, without an
//    activation and with whole 512-column tiles, 128x512 tiles of 8 waves
//    (128x64 each), one workgroup per CU.
//  * Global -> LDS with global_load_lds_dwordx4 (no register staging) into
//    a ring of 32-k stages: 4 stages of 32 KB (24 KB with fp8 weights) for
//    256x256 tiles, 3 for 128x256 and 128x512.  Each wave waits for its own loads of a
//    stage (vmcnt), then a workgroup barrier makes them visible; the
//    compiler does not track these waits, they are issued explicitly.
//  * 256x256 main loop: one barrier per stage, between its two 16-k steps.
//    The MFMAs of one step run while the fragments of the next step are
//    read from LDS and the DMA of a later stage is issued, one read and one
//    load instruction after each MFMA in an order fixed with sched_barrier
//    fences.  Measured with timing-only variants: the barrier costs ~1%;
//    the LDS-DMA costs ~17% (its writes contend with the fragment reads:
//    the loop without global loads takes 5.35 instead of 6.4 ms on the
//    prefill GEMM 1), and neither deeper prefetch nor one barrier per two
//    stages helps.  4-wave 128x128 tiles (a third less LDS reading) win
//    only with the stage's DMA split over both k-steps and no activation
//    epilogue (prefill GEMM 2 3.24 -> 3.18 ms; GEMM 1 6.03 against 5.93 ms).
//  * 128x256 tiles (two workgroups per CU) run the same loop (Switch
//    workload GEMM 1 351 -> 336 us); there the short K (1024) leaves the
//    per-tile work (GELU epilogue, stores, pipeline refill) at ~45% of the
//    time: without any loads in the loop GEMM 1 still takes 250 us.  The
//    split-K router logits GEMM runs 256x256 tiles of 8 waves on this loop
//    (DeepSeek-V3 share route 79.5 -> 74 us against 128x256 tiles of 4 waves
//    with the older loop, one barrier at the top of each stage).
//  * Every wave instruction fills 1 KB of LDS.  Row-major 16-bit operands:
//    16 tile rows x 64 bytes, four consecutive lanes per row (full 64-byte
//    global segments); inside the block the 16-byte chunks of row r are
//    XOR-swizzled by h(r) = ((r >> 1) ^ (r >> 2)) & 3, so the MFMA fragment
//    reads (consecutive rows, same chunk) hit distinct banks.  Tiled bf16
//    weights: each stage of a 16-row tile is one contiguous 1 KB piece, which
//    lands chunk-major (chunk c of row r at (16c + r) * 16), conflict-free
//    without a swizzle.
//  * fp8 weights: 32 rows x 32 bytes per 1 KB block (row-major: two lanes per
//    row; tiled: two 512-byte chunk-major halves of 16 rows).  Each lane reads
//    the 16 values of both k-steps of a stage at once, dequantises them with
//    the block scale (hardware fp8 -> f32 conversion, scale, round to bf16)
//    and feeds the bf16 MFMA.  Lane half h covers k [16h, 16h + 16) of a
//    stage; the A fragments use the same k order.
//  * Persistent grid with the device-side tile table and XCD-aware order of
//    grouped_gemm_kernel, the tiles of a group taken in column blocks of 32
//    n-tiles walked in strips of 4 m-tiles; SwiGLU pairs the w1 and w3 rows
//    of the same output columns inside each wave.
#include <math.h>

#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace {

constexpr int BKE = 32;      // k elements per stage (64 bytes of bf16)
constexpr int NSTAGE = 4;    // LDS ring depth of the 256x256 tiles
constexpr int kMaxFp8K = 16384;  // fp8 weights: K per GEMM (the tile's scales sit in registers)
constexpr int kGM = 4;       // m-tiles per strip
constexpr int kCB = 32;      // n-tiles per column block

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// DMA instructions a k-step issues: none (ON false), all of the stage's, or,
// with the stage split over its two steps, the first or second half (HALF).
template <bool ON, bool HALF>
struct DmaTag {
  static constexpr bool value = ON;
  static constexpr bool half = HALF;
};

// Order in which one k-step's fragments are read: by first use in the
// i-major MFMA order (A subtile i, B subtile j), so the first MFMAs of the
// next step wait only for the first reads; B skipped when !WITH_B.
template <int QM, int QN, bool WITH_B>
struct ReadOrder {
  int n = 0;
  int kind[QM + QN] = {};  // 0: A, 1: B
  int idx[QM + QN] = {};
  constexpr ReadOrder() {
    bool sa[QM] = {}, sb[QN] = {};
    for (int m = 0; m < QM * QN; ++m) {
      const int i = m / QN, j = m % QN;
      if (!sa[i]) {
        sa[i] = true;
        kind[n] = 0;
        idx[n++] = i;
      }
      if (WITH_B && !sb[j]) {
        sb[j] = true;
        kind[n] = 1;
        idx[n++] = j;
      }
    }
  }
};

// Output elements are written once per launch.  The first GEMM's
// activations (read back only by the second GEMM, after the whole first one)
// go out nontemporally; the second GEMM's rows are read right after by the
// combine and stay cacheable.  Measured: prefill GEMM1 7.31 -> 7.26 ms, Switch
// GEMM1 420 -> 410 us.
template <bool NT>
__device__ __forceinline__ void store_c(bf16_t* p, float v) {
  // hardware round-to-nearest-even (software rounding had cost ~5
  // instructions per value: Switch GEMM 1 300 -> 287 us)
  const bf16_t b = (bf16_t)(bf16_pair(v, 0.f) & 0xffffu);
  if constexpr (NT) __builtin_nontemporal_store(b, p);
  else *p = b;
}

#define MOE_GPTR(p) ((const void __attribute__((address_space(1)))*)(p))
#define MOE_LPTR(p) ((void __attribute__((address_space(3)))*)(p))

// Waits until at most `stages` later stages of this wave's DMA (LPW
// instructions each, 0 <= stages <= 3) are in flight and its LDS reads have
// returned, then synchronises the workgroup.
template <int LPW>
__device__ __forceinline__ void wait_dma_and_barrier(int stages) {
  static_assert(3 * LPW <= 63, "vmcnt range");
  if (stages >= 3) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(3 * LPW) : "memory");
  } else if (stages == 2) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LPW) : "memory");
  } else if (stages == 1) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LPW) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

template <int NTHREADS>
__device__ void scan_pairs_dma(int v0, int v1, int* out0, int* out1, int* total, int* sh) {
  const int lane = lane_id();
  const int w = threadIdx.x / 64;
  const int s = v0 + v1;
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
  for (int i = 0; i < NTHREADS / 64; ++i) {
    if (i < w) add += sh[i];
    tot += sh[i];
  }
  const int excl = incl - s + add;
  *out0 = excl;
  *out1 = excl + v0;
  *total = tot;
}

// NS: LDS ring depth (loads run NS-1 stages ahead); MINW: waves per SIMD the
// register budget must allow (2 with 4-wave workgroups = two per CU).
// PART: split-K into p.ksplit slices, each writing fp32 partial sums
// [slice][row][col] (row = partial row as in GroupedParams) with no
// activation; the caller reduces the slices in a fixed order.
template <int BSRC, bool TL, int EPI, int BM, int BN, int WM_, int WN_, int NS, int MINW,
          bool PART>
__global__ void __launch_bounds__(64 * WM_ * WN_, MINW) dma_gemm_kernel(GroupedParams p) {
  constexpr bool F8 = BSRC == B_FP8;
  constexpr int NW = WM_ * WN_;                  // waves
  // 256x256 tiles of 8 waves, 128x256 tiles of 4 waves (two workgroups per
  // CU) and 128x512 tiles of 8 waves, all 128x64 per wave, and 256x256 tiles
  // of 4 waves (128x128 per wave): one barrier per stage, in the middle (see
  // below)
  static_assert((((NW == 8 && BM == 256) || (NW == 4 && BM == 128) || (NW == 4 && BM == 256)) &&
                 BN == 256) ||
                    (NW == 8 && BM == 128 && BN == 512),
                "tile shapes of the fenced schedule");
  // 256x256 tiles of 4 waves (one per SIMD): a stage's DMA is split over its
  // two k-steps, issued after the step's eight fragment reads (MFMAs 8-11)
  constexpr bool kSplit = NW == 4 && BM == 256;
  constexpr int kDmaAt = kSplit ? 8 : 0;  // MFMA after which a step's first DMA goes
  // stages of DMA issued before a tile's main loop
  constexpr int kPre = NS - 1;
  constexpr int kThreads = 64 * NW;
  constexpr int WTM = BM / WM_, WTN = BN / WN_;  // wave tile
  constexpr int QM = WTM / 32, QN = WTN / 32;    // 32x32 subtiles per wave
  constexpr int A_BYTES = BM * BKE * 2;
  constexpr int B_BYTES = BN * BKE * (F8 ? 1 : 2);
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_BLOCKS = A_BYTES / 1024, B_BLOCKS = B_BYTES / 1024;  // 1 KB blocks per stage
  constexpr int B_ROWS_PER_BLOCK = F8 ? 32 : 16;
  constexpr int kScRegs = F8 ? kMaxFp8K / 128 / 64 : 1;  // fp8 scale registers per B subtile
  constexpr int LPW = (A_BLOCKS + B_BLOCKS) / NW;  // DMA instructions per wave per stage
  static_assert((A_BLOCKS + B_BLOCKS) % NW == 0, "blocks split evenly over waves");
  static_assert(EPI != EPI_SWIGLU || QN % 2 == 0, "SwiGLU pairs subtiles");
  static_assert(2 * kThreads >= kMaxGroups + 1, "tile table needs two entries per thread");
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ring = smem;  // [NS][A | B]
  int* s_tstart = reinterpret_cast<int*>(smem + NS * STAGE_BYTES);
  int* s_rows = s_tstart + (kMaxGroups + 1);
  int* s_r0 = s_rows + kMaxGroups;
  int* s_scan = s_r0 + kMaxGroups;  // [8]: one partial sum per wave of the preamble's scan

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: LDS addresses in SGPRs
  const int wm = wave / WN_, wn = wave % WN_;
  const int ngroups = p.n_routed + (p.t_dense > 0 ? 1 : 0);
  const int nt = p.N / BN;

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
    scan_pairs_dma<kThreads>(t2[0], t2[1], &e0, &e1, &tot, s_scan);
    if (2 * tid < kMaxGroups + 1) s_tstart[2 * tid] = e0;
    if (2 * tid + 1 < kMaxGroups + 1) s_tstart[2 * tid + 1] = e1;
    if (tid == 0) s_tstart[ngroups] = tot;
  }
  __syncthreads();
  const int total = s_tstart[ngroups];
  const int G = gridDim.x;
  const int first = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const int a_sub = (p.a_shift && p.n_routed > 0) ? p.off[p.e_begin] : 0;
  const int c_sub = (p.c_shift && p.n_routed > 0) ? p.off[p.e_begin] : 0;
  const int64_t a_stride = (int64_t)p.K * 2;              // bytes per row of A
  const int64_t b_stride = (int64_t)p.K * (F8 ? 1 : 2);   // bytes per row of B
  const int64_t b_mat = p.b_stride * (F8 ? 1 : 2);        // bytes per expert matrix
  const int KS = PART ? p.ksplit : 1;
  const int KT = p.K / BKE / KS;  // stages of one K slice

  // Per-tile state.  The next tile's setup and first stages are issued
  // before the current tile's epilogue, so its loads overlap the epilogue's
  // activation math and stores.
  struct Ctx {
    int z, kbase, g, rows, m0, n_t;
    bool dense;
    bf16_t* C;
    const unsigned char* src[LPW];  // stage-0 global address of each DMA instruction
    int kstep[LPW];                 // its bytes per stage
    float sr[QN][kScRegs];          // fp8: scale of 128-k block 64r + lane, per B subtile
  };
  // DMA instruction i of this wave fills 1 KB block b = wave + NW*i of the
  // stage (A blocks first, then B blocks); LDS position l*16 <- lane l.
  const int dr = lane >> 2;                 // row-major 16-bit: row
  const int dchunk = (lane & 3) ^ swz(dr);  //   and logical chunk
  auto setup = [&](int work, Ctx& c) {
    c.z = work / total;  // K slice (consecutive work items share it)
    const int tile = work - c.z * total;
    c.kbase = c.z * KT;
    int lo = 0, hi = ngroups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tstart[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    c.g = lo;
    const int g = lo;
    const int local = tile - s_tstart[g];
    c.rows = s_rows[g];
    const int rows = c.rows;
    const int mt = (rows + BM - 1) / BM;
    // column blocks of kCB n-tiles, each walked strip by strip (kGM m-tiles
    // by its n-tiles, m fastest): an XCD's 32 consecutive tiles are 4 m x 8 n,
    // and a weight panel is used again one strip later rather than one
    // expert later (prefill GEMM 1 -2% against strips over all n-tiles)
    const int cb = local / (mt * kCB);
    const int nb_sz = min(kCB, nt - cb * kCB);
    const int idx = local - cb * mt * kCB;
    const int strip = idx / (kGM * nb_sz);
    const int rem = idx - strip * kGM * nb_sz;
    const int gm = min(kGM, mt - strip * kGM);
    const int m_t = strip * kGM + rem % gm;
    const int n_t = cb * kCB + rem / gm;
    c.n_t = n_t;
    const bool dense = g >= p.n_routed;
    c.dense = dense;
    const int m0 = m_t * BM;
    c.m0 = m0;

    const unsigned char *A, *B1, *B3;
    const float *S1 = nullptr, *S3 = nullptr;
    if (!dense) {
      A = reinterpret_cast<const unsigned char*>(p.a_routed) + (int64_t)(s_r0[g] - a_sub) * a_stride;
      c.C = reinterpret_cast<bf16_t*>(p.c_routed) + (int64_t)(s_r0[g] - c_sub) * p.ldc;
      B1 = reinterpret_cast<const unsigned char*>(p.b1) + (int64_t)g * b_mat;
      B3 = p.b3 ? reinterpret_cast<const unsigned char*>(p.b3) + (int64_t)g * b_mat : B1;
      if (F8) {
        S1 = p.s1 + (int64_t)g * p.ns * p.ks;
        S3 = p.s3 ? p.s3 + (int64_t)g * p.ns * p.ks : S1;
      }
    } else {
      A = reinterpret_cast<const unsigned char*>(p.a_dense);
      c.C = reinterpret_cast<bf16_t*>(p.c_dense);
      B1 = reinterpret_cast<const unsigned char*>(p.bd1);
      B3 = p.bd3 ? reinterpret_cast<const unsigned char*>(p.bd3) : B1;
      if (F8) {
        S1 = p.sd1;
        S3 = p.sd3 ? p.sd3 : S1;
      }
    }
    // weight row of B tile row tr (SwiGLU: each half of a wave column's rows
    // is w1 or w3 of the same output columns)
    auto b_row = [&](int tr, const unsigned char*& bm, const float*& sm) {
      bm = B1;
      sm = S1;
      if (EPI == EPI_SWIGLU) {
        const int col_wave = tr / WTN, rr = tr % WTN;
        if (rr >= WTN / 2) {
          bm = B3;
          sm = S3;
        }
        return n_t * (BN / 2) + col_wave * (WTN / 2) + rr % (WTN / 2);
      }
      return n_t * BN + tr;
    };

    // DMA instruction i of this wave fills 1 KB block b = wave + NW*i of the
    // stage (A blocks first, then B blocks); LDS position l*16 <- lane l.
    // c.src[i] is the stage-0 global address, c.kstep[i] the bytes per stage.
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int b = wave + NW * i;
      if (b < A_BLOCKS) {
        const int ar = min(m0 + 16 * b + dr, rows - 1);
        c.src[i] = A + (int64_t)ar * a_stride + dchunk * 16;
        c.kstep[i] = BKE * 2;
      } else {
        int r_in;  // row inside the block
        if (F8) r_in = TL ? 16 * (lane >> 5) + (lane & 15) : (lane >> 1);
        else r_in = TL ? (lane & 15) : dr;
        const int tr = B_ROWS_PER_BLOCK * (b - A_BLOCKS) + r_in;  // B tile row
        const unsigned char* bm;
        const float* sm;
        const int brow = b_row(tr, bm, sm);
        if (TL) {
          // 16-row tile: 1 KB pieces of 64 bytes per row, in lane order
          const int64_t tile_base = (int64_t)(brow >> 4) * 16 * b_stride;
          c.src[i] = bm + tile_base + (F8 ? (lane & 31) : lane) * 16;
          c.kstep[i] = F8 ? 512 : 1024;  // fp8: half kt%2 of piece kt/2
        } else {
          c.src[i] = bm + (int64_t)brow * b_stride + (F8 ? (lane & 1) : dchunk) * 16;
          c.kstep[i] = BKE * (F8 ? 1 : 2);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < LPW; ++i) c.src[i] += (int64_t)c.kbase * c.kstep[i];
    // fp8 scales: one per B subtile and 128-k block (the subtile's 32
    // weight rows lie in one 128-row block), all of the tile's K range
    // loaded here into registers (lane q of register r: block 64r + q); the
    // main loop picks one with readlane, so it issues no vector load of its
    // own, whose use would make the compiler wait for every LDS DMA in flight
    if constexpr (F8) {
      const int kblocks = KT / 4;
#pragma unroll
      for (int j = 0; j < QN; ++j) {
        const unsigned char* bm;
        const float* sm;
        const int brow = b_row(wn * WTN + j * 32, bm, sm);
        const float* srow = sm + (int64_t)(brow >> 7) * p.ks + c.kbase / 4;
#pragma unroll
        for (int r = 0; r < kScRegs; ++r) c.sr[j][r] = srow[min(64 * r + lane, kblocks - 1)];
      }
    }

  };
  auto issue = [&](const Ctx& c, int kt) {
    unsigned char* st = ring + (kt % NS) * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int b = wave + NW * i;
      __builtin_amdgcn_global_load_lds(MOE_GPTR(c.src[i] + (int64_t)kt * c.kstep[i]),
                                       MOE_LPTR(st + b * 1024), 16, 0, 0);
    }
  };

  const int W = total * KS;
  Ctx cur;
  if (first < W) {
    setup(first, cur);
    // every wave has finished reading the tile table's neighbours; ring free
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int s = 0; s < kPre; ++s)
      if (s < KT) issue(cur, s);
  }
  for (int work = first; work < W; work += G) {
    f32x16 acc[QM][QN];
#pragma unroll
    for (int i = 0; i < QM; ++i)
#pragma unroll
      for (int j = 0; j < QN; ++j) acc[i][j] = f32x16{};

    const int rows = cur.rows, m0 = cur.m0, n_t = cur.n_t, z = cur.z, kbase = cur.kbase, g = cur.g;
    const bool dense = cur.dense;
    bf16_t* const C = cur.C;

    const int h = lane >> 5;  // k half of this lane: [16h, 16h + 16) of a stage
    if constexpr (F8) {
      // the scales have landed before the loop (one wait per tile here,
      // instead of one in every stage)
#pragma unroll
      for (int j = 0; j < QN; ++j)
#pragma unroll
        for (int r = 0; r < kScRegs; ++r) asm volatile("" ::"v"(cur.sr[j][r]));
    }
    {
      // Two waves per SIMD (one workgroup of 8, or two of 4), 128x64 per
      // wave, one workgroup barrier per stage placed between the stage's two
      // 16-k steps.  The MFMAs of one step run while the fragments of the
      // next step are read from LDS, so no MFMA waits for an LDS read issued
      // just before it:
      //   step 0 of stage kt: MFMAs on X (step 0 of kt) | read Y = step 1 of
      //            kt | DMA of stage kt + NS - 1 into the slot of stage kt - 1
      //   barrier: every wave's DMA of stage kt + 1 has landed and its reads
      //            of stage kt have returned, so stage kt + 1 is visible and
      //            the slot of stage kt is free
      //   step 1 of stage kt: MFMAs on Y | read X = step 0 of kt + 1
      // Inside a step, MFMA q is followed by the q-th fragment read and the
      // q-th DMA instruction, each group fenced with sched_barrier: left to
      // itself the compiler bunches the reads and loads behind one MFMA and
      // the matrix core idles while they issue (measured: prefill GEMM 1
      // 7.2 -> 6.4 ms).
      // fp8 weights: a lane's 16 B fragment bytes hold both steps of a stage,
      // read with step 0 and converted to bf16 after the step-1 MFMAs.
      u32x4 aX[QM], aY[QM], bX[QN], bY[QN];
      uint32_t raw[QN][4];
      // A fragment of subtile i, k-step `step`, stage kt
      auto rd_a1 = [&](int kt, int step, int i) {
        const unsigned char* st = ring + (kt % NS) * STAGE_BYTES;
        const int c = 2 * h + step;  // A chunk: k [16h + 8 step, +8)
        const int R = wm * WTM + i * 32 + (lane & 31), r = R & 15;
        return *reinterpret_cast<const u32x4*>(st + (R >> 4) * 1024 + (r * 4 + (c ^ swz(r))) * 16);
      };
      // B fragment of subtile j; fp8: the raw bytes of both steps into raw[j]
      auto rd_b1 = [&](int kt, int step, int j, u32x4& bq) {
        const unsigned char* st = ring + (kt % NS) * STAGE_BYTES;
        const int R = wn * WTN + j * 32 + (lane & 31), r = R & 15;
        if constexpr (F8) {
          const int boff = TL ? ((R >> 4) & 1) * 512 + (16 * h + r) * 16 : (R & 31) * 32 + h * 16;
          const u32x4 w8 = *reinterpret_cast<const u32x4*>(st + A_BYTES + (R >> 5) * 1024 + boff);
#pragma unroll
          for (int q = 0; q < 4; ++q) raw[j][q] = w8[q];
        } else {
          const int c = 2 * h + step;
          const int boff = TL ? (16 * c + r) * 16 : (r * 4 + (c ^ swz(r))) * 16;
          bq = *reinterpret_cast<const u32x4*>(st + A_BYTES + (R >> 4) * 1024 + boff);
        }
      };
      // DMA instruction i of stage kt (as in issue())
      auto dma1 = [&](int kt, int i) {
        unsigned char* st = ring + (kt % NS) * STAGE_BYTES;
        __builtin_amdgcn_global_load_lds(MOE_GPTR(cur.src[i] + (int64_t)kt * cur.kstep[i]),
                                         MOE_LPTR(st + (wave + NW * i) * 1024), 16, 0, 0);
      };
      // fp8: raw bytes of stage kt -> bf16 B fragments of both steps
      auto cvt_b = [&](int kt) {
        if constexpr (F8) {
          const int q = kt >> 2;  // 128-k block of the stage within the slice
#pragma unroll
          for (int j = 0; j < QN; ++j) {
            float v = cur.sr[j][0];
#pragma unroll
            for (int r = 1; r < kScRegs; ++r)
              if (q >= 64 * r) v = cur.sr[j][r];
            const float sc =
                __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), q & 63));
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              u32x4 o;
#pragma unroll
              for (int wv = 0; wv < 2; ++wv) {
                const uint32_t word = raw[j][2 * s2 + wv];
                typedef float f2_t __attribute__((ext_vector_type(2)));
                const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
                const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
                o[2 * wv] = bf16_pair(lo.x * sc, lo.y * sc);
                o[2 * wv + 1] = bf16_pair(hi.x * sc, hi.y * sc);
              }
              if (s2 == 0) bX[j] = o;
              else bY[j] = o;
            }
          }
        }
      };
      // One 16-k step: the QM x QN MFMAs on (aq, bq); after MFMA q the q-th
      // read of the fragments (an, bn) of k-step step_rd of stage kt_rd and,
      // with DMA, the q-th load instruction of stage kt_dma.
      auto step = [&](const u32x4 (&aq)[QM], const u32x4 (&bq)[QN], u32x4 (&an)[QM],
                      u32x4 (&bn)[QN], int kt_rd, int step_rd, auto with_b, int kt_dma,
                      auto dma) {
        constexpr ReadOrder<QM, QN, decltype(with_b)::value> ord{};
        static_assert(ord.n <= QM * QN && kDmaAt + (kSplit ? LPW / 2 : LPW) <= QM * QN,
                      "one read and one load per MFMA");
#pragma unroll
        for (int q = 0; q < QM * QN; ++q) {
          const int i = q / QN, j = q % QN;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, aq[i]), __builtin_bit_cast(bf16x8_t, bq[j]), acc[i][j], 0,
              0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (q < ord.n) {
            if (ord.kind[q] == 0) an[ord.idx[q]] = rd_a1(kt_rd, step_rd, ord.idx[q]);
            else rd_b1(kt_rd, step_rd, ord.idx[q], bn[ord.idx[q]]);
          }
          if constexpr (decltype(dma)::value) {
            constexpr int d0 = kSplit && decltype(dma)::half ? LPW / 2 : 0;
            constexpr int nd = kSplit ? LPW / 2 : LPW;
            if (q >= kDmaAt && q - kDmaAt < nd) dma1(kt_dma, d0 + q - kDmaAt);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      // step 0 of stage kt (fp8: the B bytes of both steps came with step 0)
      auto step0 = [&](int kt, auto dma) {
        step(aX, bX, aY, bY, kt, 1, std::integral_constant<bool, !F8>{}, kt + NS - 1,
             DmaTag<decltype(dma)::value, false>{});
      };
      // step 1 of stage kt (with a split stage, the second half of the DMA of
      // stage kt + NS - 1: its slot was freed at the previous barrier); at the
      // last stage it reads a slot whose contents are not used
      auto step1 = [&](int kt, auto dma) {
        step(aY, bY, aX, bX, kt + 1, 0, std::true_type{}, kt + NS - 1,
             DmaTag<kSplit && decltype(dma)::value, true>{});
        if constexpr (F8) cvt_b(kt + 1);
      };
      wait_dma_and_barrier<LPW>(min(NS - 2, KT - 1));  // stage 0 visible
#pragma unroll
      for (int i = 0; i < QM; ++i) aX[i] = rd_a1(0, 0, i);
#pragma unroll
      for (int j = 0; j < QN; ++j) rd_b1(0, 0, j, bX[j]);
      if constexpr (F8) cvt_b(0);
      // every stage but the last NS - 1 loads stage kt + NS - 1, so NS - 2
      // later stages (NS - 2.5 with a split stage) are in flight at each of
      // these barriers
      int kt = 0;
      for (; kt < KT - NS + 1; ++kt) {
        step0(kt, std::true_type{});
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier"
                     ::"n"((NS - 2) * LPW - (kSplit ? LPW / 2 : 0)) : "memory");
        __builtin_amdgcn_sched_barrier(0);
        step1(kt, std::true_type{});
      }
      for (; kt < KT; ++kt) {
        step0(kt, std::false_type{});
        wait_dma_and_barrier<LPW>(min(NS - 2, KT - 2 - kt));
        __builtin_amdgcn_sched_barrier(0);
        step1(kt, std::false_type{});
      }
    }

    // every wave has finished reading the ring: start the next tile's loads
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const bool more = work + G < W;
    Ctx nxt;
    if (more) {
      setup(work + G, nxt);
#pragma unroll
      for (int s = 0; s < kPre; ++s)
        if (s < KT) issue(nxt, s);
    }
    // The epilogue's addresses are formed from copies that an empty asm
    // statement hides from the compiler: otherwise it computes the 64-bit row
    // addresses before the main loop and keeps them live through it.
    int e_rows = rows, e_m0 = m0, e_nt = n_t, e_z = z, e_g = g;
    bf16_t* e_C = C;
    asm volatile("" : "+v"(e_rows), "+v"(e_m0), "+v"(e_nt), "+v"(e_z), "+v"(e_g), "+v"(e_C));
    // epilogue: value v of a lane is row 8*(v/4) + 4*(lane/32) + v%4,
    // column lane%32 of its 32x32 subtile
    if constexpr (PART) {
      const int64_t prow0 =
          dense ? p.max_rows : (int64_t)(s_r0[e_g] - (p.n_routed > 0 ? p.off[p.e_begin] : 0));
#pragma unroll
      for (int i = 0; i < QM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = e_m0 + wm * WTM + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
          if (row >= e_rows) continue;
          float* prow = p.partial + ((int64_t)e_z * p.prow_total + prow0 + row) * p.ldc;
#pragma unroll
          for (int j = 0; j < QN; ++j) prow[e_nt * BN + wn * WTN + j * 32 + (lane & 31)] = acc[i][j][v];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < QM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = e_m0 + wm * WTM + i * 32 + 8 * (v / 4) + 4 * (lane >> 5) + (v % 4);
          if (row >= e_rows) continue;
          bf16_t* crow = e_C + (int64_t)row * p.ldc;
          if (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < QN / 2; ++j) {
              const int col = e_nt * (BN / 2) + wn * (WTN / 2) + j * 32 + (lane & 31);
              store_c<true>(crow + col, act_silu(acc[i][j][v]) * acc[i][j + QN / 2][v]);
            }
          } else {
#pragma unroll
            for (int j = 0; j < QN; ++j) {
              const int col = e_nt * BN + wn * WTN + j * 32 + (lane & 31);
              float x = acc[i][j][v];
              if (EPI == EPI_RELU) x = fmaxf(x, 0.f);
              if (EPI == EPI_GELU) x = act_gelu(x);
              store_c<EPI != EPI_NONE>(crow + col, x);
            }
          }
        }
      }
    }
    // the next tile's first stages (and these stores) have landed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (more) cur = nxt;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int BSRC, bool TL, int EPI, int BM, int BN, int WM_, int WN_, int NS = NSTAGE,
          int MINW = 1, bool PART = false>
moe_status launch_dma(const GroupedParams& p, int64_t max_routed_rows, hipStream_t stream) {
  auto kern = dma_gemm_kernel<BSRC, TL, EPI, BM, BN, WM_, WN_, NS, MINW, PART>;
  constexpr int per_cu = MINW * 4 / (WM_ * WN_) > 0 ? MINW * 4 / (WM_ * WN_) : 1;  // workgroups
  constexpr size_t lds = NS * (BM * 2 + BN * (BSRC == B_FP8 ? 1 : 2)) * BKE +
                         (3 * kMaxGroups + 1 + 8) * sizeof(int);
  static_assert(per_cu * lds <= 160 * 1024, "LDS of the resident workgroups");
  MOE_CHECK_HIP(set_dynamic_lds((const void*)kern, (int)lds));
  const int nt = p.N / BN;
  const int ngroups = p.n_routed + (p.t_dense > 0 ? 1 : 0);
  const int64_t m_tiles_ub = (max_routed_rows + BM - 1) / BM + p.n_routed +
                             (p.t_dense > 0 ? (p.t_dense + BM - 1) / BM : 0);
  const int64_t tiles_ub = m_tiles_ub * nt * (PART ? p.ksplit : 1);
  if (ngroups == 0 || tiles_ub == 0) return MOE_OK;
  int64_t grid = (int64_t)device_info().cus * per_cu;
  if (grid > tiles_ub) grid = tiles_ub;
  if (grid >= 8) grid = grid / 8 * 8;
  kern<<<(int)grid, 64 * WM_ * WN_, lds, stream>>>(p);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

// Tile shapes: 256x256 with 2x4 waves of 128x64 (one workgroup per CU) for
// large groups; 128x256 tiles of 4 waves, two workgroups per CU with a
// 3-stage ring each, for groups of a few hundred rows with no shared expert
// (less padding, and one workgroup's prologue and epilogue overlap the
// other's main loop).  Measured: Switch workload 1.00 -> 0.87 ms; the bf16
// prefill workload stays faster on 256x256 (11.8 vs 13.0 ms), and so does
// the DeepSeek-V3 share with fp8 weights (expert GEMM 1 662 -> 648 us).
// Groups average fewer than kSmallRows rows -> 128x256 tiles.
constexpr int64_t kSmallRows = 768;
template <int BSRC, bool TL, int EPI>
moe_status launch_dma_shape(const GroupedParams& p, int64_t max_routed_rows, hipStream_t s) {
  const int groups = p.n_routed > 0 ? p.n_routed : 1;
  const bool small_tiles = p.t_dense == 0 && max_routed_rows / groups < kSmallRows;
  // Without an activation epilogue, 128x512 tiles of 8 waves: a sixth fewer
  // bytes per flop through the LDS DMA, which bounds these tiles (Switch
  // GEMM 2 273 -> 253 us); with one, the two 128x256 workgroups of a CU
  // overlap one's epilogue with the other's main loop (Switch GEMM 1 286 us
  // against 290-295 us on 128x512 tiles).
  if (EPI == EPI_NONE && small_tiles && p.N % 512 == 0)
    return launch_dma<BSRC, TL, EPI, 128, 512, 1, 8, 3, 1>(p, max_routed_rows, s);
  if (small_tiles) return launch_dma<BSRC, TL, EPI, 128, 256, 1, 4, 3, 2>(p, max_routed_rows, s);
  // bf16 weights and no activation (the second expert GEMM): 4 waves of
  // 128x128, which read a third less from LDS and hold a higher clock
  // (prefill GEMM 2 3.24 -> 3.18 ms); with an activation epilogue, or fp8
  // weights, 8 waves are faster (prefill GEMM 1 5.93 against 6.03 ms,
  // DeepSeek-V3 GEMM 2 0.31 against 0.38 ms)
  if constexpr (EPI == EPI_NONE && BSRC == B_SAME)
    return launch_dma<BSRC, TL, EPI, 256, 256, 2, 2>(p, max_routed_rows, s);
  return launch_dma<BSRC, TL, EPI, 256, 256, 2, 4>(p, max_routed_rows, s);
}

template <int BSRC, bool TL>
moe_status launch_dma_epi(int epi, const GroupedParams& p, int64_t max_routed_rows,
                          hipStream_t stream) {
  switch (epi) {
    case EPI_RELU:
      return launch_dma_shape<BSRC, TL, EPI_RELU>(p, max_routed_rows, stream);
    case EPI_GELU:
      return launch_dma_shape<BSRC, TL, EPI_GELU>(p, max_routed_rows, stream);
    case EPI_SWIGLU:
      return launch_dma_shape<BSRC, TL, EPI_SWIGLU>(p, max_routed_rows, stream);
    default:
      return launch_dma_shape<BSRC, TL, EPI_NONE>(p, max_routed_rows, stream);
  }
}

}  // namespace

// Split-K fp32 partials for a single dense bf16 GEMM (the E >= 256 router
// logits): 256x256 tiles of 8 waves, the fenced schedule of the expert GEMMs.
moe_status launch_dma_partial(const GroupedParams& p, hipStream_t stream) {
  return launch_dma<B_SAME, false, EPI_NONE, 256, 256, 2, 4, 4, 1, true>(p, 0, stream);
}

// bf16 or fp8 weights (row-major or tiled); output columns in whole 256-wide
// tiles, K in whole 32-element stages (fp8: 128-element scale blocks, K at
// most kMaxFp8K).
bool dma_gemm_supported(const GroupedParams& p, int bsrc) {
  if (p.N % 256 != 0 || p.K % BKE != 0) return false;
  return bsrc == B_SAME || (bsrc == B_FP8 && p.K % 128 == 0 && p.K <= kMaxFp8K);
}

moe_status launch_dma_gemm(int bsrc, int epi, const GroupedParams& p, int64_t max_routed_rows,
                           hipStream_t stream) {
  if (bsrc == B_FP8)
    return p.b_tiled ? launch_dma_epi<B_FP8, true>(epi, p, max_routed_rows, stream)
                     : launch_dma_epi<B_FP8, false>(epi, p, max_routed_rows, stream);
  return p.b_tiled ? launch_dma_epi<B_SAME, true>(epi, p, max_routed_rows, stream)
                   : launch_dma_epi<B_SAME, false>(epi, p, max_routed_rows, stream);
}

}  // namespace moe
