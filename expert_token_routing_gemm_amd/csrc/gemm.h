// Internal interface of the grouped MFMA GEMM (gfx950).
#pragma once

#include "common.h"

namespace moe {

// Router logits for many experts: out[T, E] (fp32) = x[T, d] W_r[E, d]^T on
// the bf16 MFMA tile code of the expert FFN.  E % 64 == 0, d % 128 == 0.
moe_status dense_logits_gemm(const void* x, const void* w_router, float* out, int64_t T, int d,
                             int E, hipStream_t stream);

}  // namespace moe
