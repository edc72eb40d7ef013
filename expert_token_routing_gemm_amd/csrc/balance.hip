// Load balancing around the router (gfx950): the bias-balancing step and the
// auxiliary balancing loss value.
//
// Both serve the aim the pages state in Ultralytics "Expert Parallelism",
// "Load Balancing and Capacity": the most loaded GPU sets the time of the
// whole layer.  Bias balancing: the selection bias of overloaded experts goes down
// and of idle ones up after each step.  Auxiliary loss: an extra loss term
// rewards spreading tokens evenly (its form is not on the pages; the
// Switch-Transformer form alpha * E * sum_e f_e * P_e is used).
#include "common.h"

namespace moe {
namespace {

constexpr int kWave = 64;

__global__ void __launch_bounds__(256) bias_update_kernel(const int32_t* __restrict__ counts,
                                                         float* __restrict__ b, int E, int64_t tk,
                                                         float gamma) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int64_t c = (int64_t)counts[e] * E;
  const float s = c > tk ? 1.f : (c < tk ? -1.f : 0.f);
  b[e] = b[e] - gamma * s;
}

// Per-block sums of the router probabilities: block b owns a contiguous token
// range, wave w of it every 4th token of the range; lane l keeps experts
// l + 64 i.  Probabilities: softmax over the E logits, or the sigmoids
// normalised per token.  Waves are combined in a fixed order: the result does
// not depend on scheduling.
constexpr int kAuxThreads = 256;
constexpr int kAuxWaves = kAuxThreads / kWave;
constexpr int PER = MOE_MAX_EXPERTS / kWave;

__global__ void __launch_bounds__(kAuxThreads) aux_partial_kernel(const float* __restrict__ logits,
                                                                  int64_t T, int E, int score,
                                                                  int64_t per_block,
                                                                  float* __restrict__ partial) {
  __shared__ float red[kAuxWaves][MOE_MAX_EXPERTS];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int64_t t0 = (int64_t)blockIdx.x * per_block;
  const int64_t t1 = min(t0 + per_block, T);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  constexpr int G = 4;  // tokens per wave whose logits are loaded together
  for (int64_t tb = t0 + wave; tb < t1; tb += (int64_t)G * kAuxWaves) {
    float v[G][PER];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int64_t t = min(tb + (int64_t)u * kAuxWaves, T - 1);  // clamped: loads stay unconditional
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane + kWave * i;
        v[u][i] = e < E ? logits[t * E + e] : -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (tb + (int64_t)u * kAuxWaves >= t1) break;
      float m = -INFINITY;
      if (score == MOE_SOFTMAX) {
#pragma unroll
        for (int i = 0; i < PER; ++i) m = fmaxf(m, v[u][i]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
      }
      float q[PER];
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = lane + kWave * i;
        q[i] = 0.f;
        if (e < E) q[i] = (score == MOE_SOFTMAX) ? expf(v[u][i] - m) : 1.f / (1.f + expf(-v[u][i]));
        s += q[i];
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, kWave);
      const float inv = 1.f / s;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += q[i] * inv;
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) red[wave][lane + kWave * i] = acc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kAuxThreads) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kAuxWaves; ++w) sum += red[w][e];
    partial[(int64_t)blockIdx.x * E + e] = sum;
  }
}

// P_e = (sum of the block sums) / T; loss = alpha * E * sum_e counts_e /
// (T k) * P_e.  Thread (q, e) sums blocks q, q + 4, ... (8 loads in flight),
// the four quarter sums meet in LDS in q order, the loss in expert order; all
// in double.
constexpr int kFinalThreads = 4 * MOE_MAX_EXPERTS;

__global__ void __launch_bounds__(kFinalThreads) aux_final_kernel(
    const float* __restrict__ partial, int nblocks, const int32_t* __restrict__ counts, int64_t T,
    int E, int k, float alpha, float* __restrict__ prob_mean, float* __restrict__ loss) {
  __shared__ double quarter[4][MOE_MAX_EXPERTS];
  __shared__ double term[MOE_MAX_EXPERTS];
  const int e = threadIdx.x % MOE_MAX_EXPERTS;
  const int q = threadIdx.x / MOE_MAX_EXPERTS;
  if (e < E) {
    double sum = 0.0;
    int b = q;
    for (; b + 28 < nblocks; b += 32) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = partial[(int64_t)(b + 4 * u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += (double)v[u];
    }
    for (; b < nblocks; b += 4) sum += (double)partial[(int64_t)b * E + e];
    quarter[q][e] = sum;
  }
  __syncthreads();
  if (q == 0 && e < E) {
    const double tot = quarter[0][e] + quarter[1][e] + quarter[2][e] + quarter[3][e];
    const double P = T > 0 ? tot / (double)T : 0.0;
    prob_mean[e] = (float)P;
    term[e] = (double)counts[e] * P;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double acc = 0.0;
    for (int i = 0; i < E; ++i) acc += term[i];
    *loss = T > 0 ? (float)((double)alpha * E * acc / ((double)T * k)) : 0.f;
  }
}

int aux_blocks(int64_t T) {
  const int64_t want = (T + 63) / 64;
  const int64_t cap = 2 * (int64_t)device_info().cus;
  return (int)(want < 1 ? 1 : (want > cap ? cap : want));
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_bias_update(const int32_t* counts, float* b_select, int32_t E, int64_t T,
                                      int32_t k, float gamma, hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(E >= 1 && E <= MOE_MAX_EXPERTS, "E out of range [1, 256]");
  MOE_CHECK_ARG(T >= 0 && k >= 1, "bad T or k");
  MOE_CHECK_ARG(counts && b_select, "null pointer");
  bias_update_kernel<<<1, 256, 0, stream>>>(counts, b_select, E, T * (int64_t)k, gamma);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}

extern "C" size_t moe_aux_loss_workspace_bytes(int64_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return align_up((size_t)aux_blocks(T) * E * sizeof(float), 256);
}

extern "C" moe_status moe_aux_loss(const float* logits, const int32_t* counts, int64_t T,
                                   int32_t E, int32_t k, int32_t score, float alpha,
                                   float* prob_mean, float* loss, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(E >= 1 && E <= MOE_MAX_EXPERTS, "E out of range [1, 256]");
  MOE_CHECK_ARG(T >= 0 && k >= 1 && k <= E, "bad T or k");
  MOE_CHECK_ARG(score == MOE_SOFTMAX || score == MOE_SIGMOID, "bad score");
  MOE_CHECK_ARG(counts && prob_mean && loss, "null pointer");
  MOE_CHECK_ARG(T == 0 || logits != nullptr, "logits are required");
  const size_t need = moe_aux_loss_workspace_bytes(T, E);
  if (ws_bytes < need || ws == nullptr) {
    set_error("moe_aux_loss: workspace too small");
    return MOE_ERR_WORKSPACE;
  }
  float* partial = static_cast<float*>(ws);
  int nblocks = 0;
  if (T > 0) {
    nblocks = aux_blocks(T);
    const int64_t per_block = (T + nblocks - 1) / nblocks;
    aux_partial_kernel<<<nblocks, kAuxThreads, 0, stream>>>(logits, T, E, score, per_block, partial);
    MOE_CHECK_LAUNCH();
  }
  aux_final_kernel<<<1, kFinalThreads, 0, stream>>>(partial, nblocks, counts, T, E, k, alpha,
                                                    prob_mean, loss);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
