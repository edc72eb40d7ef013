// Internal interface of the grouped MFMA GEMM (gfx950).
#pragma once

#include "common.h"

namespace moe {

// Router logits for many experts on the bf16 MFMA tile code of the expert
// FFN: x[T, d] W_r[E, d]^T in fp32, E % 64 == 0, d % 128 == 0.  The result
// is dense_logits_ksplit(T, d, E) slices out[s][T][E] of partial sums over
// consecutive K ranges, to be added in slice order (1 slice: the logits).
int dense_logits_ksplit(int64_t T, int d, int E);
moe_status dense_logits_gemm(const void* x, const void* w_router, float* out, int64_t T, int d,
                             int E, hipStream_t stream);

}  // namespace moe
