// One-time weight re-layout for the weight-streaming expert GEMM (gfx950).
//
// A wave feeding 16x16x32 matrix-core fragments holds, in lane 16q + r, 16
// bytes of weight row r at byte 64j + 16q of the row for its j-th load.  In
// the row-major layout one such load touches 16 rows, 64 bytes each; the
// tiled layout stores those 1 KB in lane order, so that every load of the
// streaming kernel is one contiguous, fully used 1 KB piece and a wave's 16
// rows stream as a single contiguous range.
#include "common.h"

namespace moe {
namespace {

// One thread per 16-byte destination piece: coalesced stores, 16-byte loads
// from 16 rows.
__global__ void __launch_bounds__(256) tile_kernel(const u32x4* __restrict__ w,
                                                  u32x4* __restrict__ out, int64_t n16,
                                                  int64_t row16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const int64_t tile16 = 16 * row16;  // 16-byte units per 16-row tile
  const int64_t t = i / tile16;       // global tile index (matrices are tile-aligned)
  const int64_t rem = i - t * tile16;
  const int64_t j = rem >> 6;         // 1 KB piece inside the tile
  const int l = (int)(rem & 63);      // lane order inside the piece
  const int r = l & 15, q = l >> 4;
  out[i] = w[(t * 16 + r) * row16 + j * 4 + q];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_weight_tile(const void* w, void* w_tiled, int64_t n_mats, int32_t rows,
                                      int64_t row_bytes, hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(n_mats >= 0 && rows >= 0 && row_bytes >= 0, "negative size");
  MOE_CHECK_ARG(rows % 16 == 0, "rows must be a multiple of 16");
  MOE_CHECK_ARG(row_bytes % 64 == 0, "row_bytes must be a multiple of 64");
  const int64_t n16 = n_mats * rows * (row_bytes / 16);
  if (n16 == 0) return MOE_OK;
  MOE_CHECK_ARG(w && w_tiled, "null pointer");
  MOE_CHECK_ARG(aligned16(w) && aligned16(w_tiled), "pointers not 16-byte aligned");
  const char* a = static_cast<const char*>(w);
  const char* b = static_cast<const char*>(w_tiled);
  MOE_CHECK_ARG(b + n16 * 16 <= a || a + n16 * 16 <= b, "w_tiled overlaps w");
  tile_kernel<<<(unsigned)((n16 + 255) / 256), 256, 0, stream>>>(
      static_cast<const u32x4*>(w), static_cast<u32x4*>(w_tiled), n16, row_bytes / 16);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
