// Shared definitions of the grouped expert GEMM kernels (gfx950).
#pragma once

#include <math.h>

#include "common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Epi { EPI_NONE = 0, EPI_RELU = 1, EPI_GELU = 2, EPI_SWIGLU = 3 };
enum BSrc { B_SAME = 0, B_FP8 = 1 };

constexpr int kGemmThreads = 256;
constexpr int BKE_DMA = 32;  // k elements per stage of the LDS-DMA kernel
constexpr int kMaxGroups = MOE_MAX_EXPERTS + 1;

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
  int b_tiled;  // 1: weights in the 16-row tiled layout (moe_weight_tile)
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

// GELU = 0.5 v (1 + erf(v / sqrt 2)).  erfc(z) = 1 - erf(z) for z >= 0 comes
// from Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26 (Hastings' rational approximation, absolute error <= 1.5e-7);
// 1 + erf(v / sqrt 2) is erfc(|z|) for v < 0 and 2 - erfc(|z|) otherwise, so
// negative inputs suffer no cancellation.  Over [-10, 10] the fp32 result is
// within 4.3e-7 of the exact GELU (fp32 rounding of the exact erf: 4.5e-7),
// at a fraction of the library erff's cost in the GEMM epilogue.
__device__ __forceinline__ inline float act_gelu(float v) {
  const float z = fabsf(v) * 0.70710678118654752440f;
  const float t = __builtin_amdgcn_rcpf(1.f + 0.3275911f * z);
  const float p =
      t * (0.254829592f +
           t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float q = p * __expf(-z * z);
  return 0.5f * v * (v < 0.f ? q : 2.f - q);
}
// SiLU with the hardware reciprocal (about 1 ulp) instead of an IEEE
// division, which took ~10 instructions per value in the SwiGLU epilogue
// (with the hardware bf16 rounding of the stores: prefill expert GEMM 1
// 6.24 -> 6.15 ms).
__device__ __forceinline__ float act_silu(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + __expf(-v));
}

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

// Launchers of the weight-streaming kernels (stream_gemm.hip).
int stream_ksplit(int ngroups, int out_cols, int K, int CK);
int stream_ck_for(bool swiglu, int K);
moe_status launch_stream_gemm1_any(int bsrc, int act, const GroupedParams& p, hipStream_t s);
moe_status launch_stream_gemm2_any(int bsrc, const GroupedParams& p, hipStream_t s);

// Launcher of the LDS-DMA grouped kernel for bf16 and fp8 weights (dma_gemm.hip).
bool dma_gemm_supported(const GroupedParams& p, int bsrc);
moe_status launch_dma_gemm(int bsrc, int epi, const GroupedParams& p, int64_t max_routed_rows,
                           hipStream_t stream);
moe_status launch_dma_partial(const GroupedParams& p, hipStream_t stream);

}  // namespace moe
