// Dispatch: histogram, capacity drop, offsets, stable permutation and row
// pack into the rank-major / expert-major send buffer (gfx950).
//
// What is computed follows the Ultralytics glossary "Expert Parallelism":
// per-expert and per-rank assignment counts (the listing's bincount lines),
// ranks owning contiguous expert blocks (rank = e // (E/R) in the listing),
// and the capacity limit of "Load Balancing and Capacity" (an expert keeps at
// most C assignments; overflow skips the expert).  Token order inside every
// expert segment is preserved (mbrenndoerfer "Expert Parallelism > Summary",
// buffer-management bullet), which also fixes which assignments are dropped:
// the ones past the first C in token-major order.
//
// Large batches: two kernels, no ordering atomics (results are
// deterministic); small and tiny batches: see below.
//   hist_kernel      : block b owns a chunk of TB tokens (TB*k <= 256
//                      assignments); LDS-private histogram -> blk[b][e] (rows
//                      padded to a multiple of 4 experts with zeros).
//   rank_pack_kernel : every block first sums the column of each expert over
//                      all blocks (the total) and over the blocks before its
//                      own (its base), then kept = min(total, C) and the
//                      expert offsets by a wave-level scan; block 0 writes the
//                      counts, offsets and per-rank counts.  Each assignment's
//                      position is block base + earlier waves of the block +
//                      lanes of its wave holding the same expert (ballot /
//                      popcount), which is exactly the token-major position.
//                      Writes slot and src, then copies each token's row once
//                      from x into its kept slots with 128-bit loads and
//                      stores (x is read once).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Send-buffer rows are written once and not read again by this kernel's
// workgroups: nontemporal stores (measured: prefill dispatch 86 -> 76 us,
// DeepSeek-V3-share dispatch 220 -> 209 us).
__device__ __forceinline__ void store_row16(u32x4* dst, u32x4 v) {
  __builtin_nontemporal_store(v, dst);
}

__global__ void __launch_bounds__(kThreads) hist_kernel(const int32_t* __restrict__ ids,
                                                       int32_t* __restrict__ blk, int64_t n_assign,
                                                       int per_block, int E) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  const int E4 = (E + 3) & ~3;  // row stride of blk
  for (int e = threadIdx.x; e < E4; e += kThreads) cnt[e] = 0;
  __syncthreads();
  const int64_t g = (int64_t)blockIdx.x * per_block + threadIdx.x;
  if (threadIdx.x < per_block && g < n_assign) {
    const int e = ids[g];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);  // ids outside [0, E) are ignored
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E4; e += kThreads) blk[(int64_t)blockIdx.x * E4 + e] = cnt[e];
}

// Chunks of blocks the preamble of rank_pack_kernel splits the columns of
// blk into (at most): each thread sums one chunk of one 4-expert column
// with 16-byte loads, and every expert then adds up to this many partial
// sums.
constexpr int kPreChunks = 16;

template <int UNROLL>
__global__ void __launch_bounds__(kThreads) rank_pack_kernel(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ blk, int nblocks,
    const u32x4* __restrict__ x, int32_t* __restrict__ slot_out, int32_t* __restrict__ src_out,
    u32x4* __restrict__ x_send, int64_t T, int k, int E, int R, int C, int tokens_per_block,
    int row16, int32_t* __restrict__ counts, int32_t* __restrict__ kept_out,
    int32_t* __restrict__ off_out, int32_t* __restrict__ rank_counts,
    int32_t* __restrict__ rank_off) {
  __shared__ int wcnt[kWaves][MOE_MAX_EXPERTS];   // wave counts, then wave bases
  __shared__ int base[MOE_MAX_EXPERTS];           // this block's base per expert
  __shared__ int sl[kThreads];
  __shared__ int4 pre_part[kThreads];  // [chunk][4-expert column]
  __shared__ int4 tot_part[kThreads];
  __shared__ int s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int s_wsum[kWaves];
  const int lane = lane_id();
  const int w = threadIdx.x / 64;
  const int per_block = tokens_per_block * k;
  const int64_t n_assign = T * k;
  for (int i = threadIdx.x; i < kWaves * MOE_MAX_EXPERTS; i += kThreads) (&wcnt[0][0])[i] = 0;
  // this thread's assignment, loaded before the preamble's loads
  const int64_t g = (int64_t)blockIdx.x * per_block + threadIdx.x;
  const bool in_range = threadIdx.x < per_block && g < n_assign;
  const int e = in_range ? ids[g] : -1;
  const bool valid = in_range && e >= 0 && e < E;

  // Preamble: the totals of every expert over all blocks and its base
  // (the assignments of the blocks before this one).  Thread (p, q) sums
  // 4-expert column q over block chunk p with 16-byte loads, all issued
  // before any is used.
  {
    const int Q = (E + 3) >> 2;  // 4-expert columns of blk
    const int P = min(kThreads / Q, kPreChunks);
    const int q = threadIdx.x % Q, p = threadIdx.x / Q;
    if (p < P) {
      const int chunk = (nblocks + P - 1) / P;
      const int r0 = min(p * chunk, nblocks), r1 = min(r0 + chunk, nblocks);
      const int4* col = reinterpret_cast<const int4*>(blk) + q;
      int4 tot = {0, 0, 0, 0}, pre = {0, 0, 0, 0};
      const int b = (int)blockIdx.x;
      int r = r0;
      for (; r + 16 <= r1; r += 16) {
        int4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = col[(int64_t)(r + i) * Q];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          tot.x += v[i].x; tot.y += v[i].y; tot.z += v[i].z; tot.w += v[i].w;
          if (r + i < b) { pre.x += v[i].x; pre.y += v[i].y; pre.z += v[i].z; pre.w += v[i].w; }
        }
      }
      for (; r < r1; ++r) {
        const int4 v = col[(int64_t)r * Q];
        tot.x += v.x; tot.y += v.y; tot.z += v.z; tot.w += v.w;
        if (r < b) { pre.x += v.x; pre.y += v.y; pre.z += v.z; pre.w += v.w; }
      }
      pre_part[p * Q + q] = pre;
      tot_part[p * Q + q] = tot;
    }
    __syncthreads();
    // expert e = thread: total, base, kept; exclusive scan of kept over the
    // experts (a wave scan, then the sums of earlier waves)
    int tot = 0, pre = 0;
    if ((int)threadIdx.x < E) {
      const int xe = threadIdx.x;
      for (int pp = 0; pp < P; ++pp) {
        tot += reinterpret_cast<const int*>(&tot_part[pp * Q + (xe >> 2)])[xe & 3];
        pre += reinterpret_cast<const int*>(&pre_part[pp * Q + (xe >> 2)])[xe & 3];
      }
    }
    const int kp = (int)threadIdx.x < E ? min(tot, C) : 0;
    int ex = kp;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(ex, o, 64);
      if (lane >= o) ex += u;
    }
    if (lane == 63) s_wsum[w] = ex;
    __syncthreads();
    for (int i = 0; i < w; ++i) ex += s_wsum[i];
    if ((int)threadIdx.x < E) {
      const int xe = threadIdx.x;
      s_off[xe] = ex - kp;
      base[xe] = pre;
      if (xe == E - 1) s_off[E] = ex;
      if (blockIdx.x == 0) {
        counts[xe] = tot;
        kept_out[xe] = kp;
        off_out[xe] = ex - kp;
        if (xe == E - 1) off_out[E] = ex;
      }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
      const int per = E / R;
      for (int rr = threadIdx.x; rr < R; rr += kThreads) {
        rank_counts[rr] = s_off[(rr + 1) * per] - s_off[rr * per];
        rank_off[rr] = s_off[rr * per];
      }
      if (threadIdx.x == 0) rank_off[R] = s_off[E];
    }
  }

  // wave counts of this block
  if (valid) atomicAdd(&wcnt[w][e], 1);
  __syncthreads();
  // per-wave bases: block base + counts of the earlier waves
  for (int ee = threadIdx.x; ee < E; ee += kThreads) {
    int run = base[ee];
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const int c = wcnt[i][ee];
      wcnt[i][ee] = run;
      run += c;
    }
  }
  __syncthreads();
  // rank among the lanes of this wave with the same expert (token order)
  uint64_t todo = ballot(valid);
  int r = 0;
  while (todo) {
    const int leader = __ffsll((long long)todo) - 1;
    const int el = __shfl(e, leader, 64);
    const uint64_t m = ballot(valid && e == el);
    if (valid && e == el) r = popc64(m & lanemask_lt());
    todo &= ~m;
  }
  int s = -1;
  if (valid) {
    const int pos = wcnt[w][e] + r;
    if (pos < C) {
      s = s_off[e] + pos;
      src_out[s] = (int32_t)(g / k);
    }
  }
  if (in_range) slot_out[g] = s;
  sl[threadIdx.x] = s;
  __syncthreads();
  // row pack: each token's row is read once and written to its kept slots
  const int64_t t0 = (int64_t)blockIdx.x * tokens_per_block;
  for (int tt = w; tt < tokens_per_block; tt += kWaves) {
    const int64_t t = t0 + tt;
    if (t >= T) break;
    int sj[MOE_MAX_TOPK];
    bool any = false;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      sj[j] = j < k ? sl[tt * k + j] : -1;
      any |= sj[j] >= 0;
    }
    if (!any) continue;
    const u32x4* xr = x + t * row16;
    for (int c0 = lane; c0 < row16; c0 += 64 * UNROLL) {
      u32x4 v[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int c = c0 + u * 64;
        if (c < row16) v[u] = xr[c];
      }
#pragma unroll
      for (int j = 0; j < MOE_MAX_TOPK; ++j) {
        if (sj[j] < 0) continue;
        u32x4* dst = x_send + (int64_t)sj[j] * row16;
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
          const int c = c0 + u * 64;
          if (c < row16) store_row16(dst + c, v[u]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- small batches
// Decode-sized batches (T*k <= kSmallAssign): one workgroup does the
// histogram, the offsets and the ranks (rounds of 16 waves x 64 assignments in
// token-major order, a running per-expert position carried across rounds),
// and pack_kernel copies the rows with one wave per token.  Two launches
// instead of three, and no serial loop over many histogram blocks.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
// Largest assignment count for this path (measured: the tiny workload's 8192
// assignments take 19 us on the multi-block path against 27 us here).
constexpr int kSmallAssign = 4096;

__global__ void __launch_bounds__(kSmallThreads) plan_small_kernel(
    const int32_t* __restrict__ ids, int64_t n_assign, int k, int E, int R, int C,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ off,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_off,
    int32_t* __restrict__ slot_out, int32_t* __restrict__ src_out) {
  __shared__ int cnt[MOE_MAX_EXPERTS];
  __shared__ int run[MOE_MAX_EXPERTS];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int wc[kSmallWaves][MOE_MAX_EXPERTS];
  __shared__ int wsum[kSmallWaves];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / 64;
  for (int e = tid; e < MOE_MAX_EXPERTS; e += kSmallThreads) {
    cnt[e] = 0;
    run[e] = 0;
  }
  __syncthreads();
  for (int64_t g = tid; g < n_assign; g += kSmallThreads) {
    const int e = ids[g];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of kept over the experts (threads 0..255 = waves 0..3)
  int kp = 0, incl = 0;
  if (tid < MOE_MAX_EXPERTS) {
    kp = tid < E ? min(cnt[tid], C) : 0;
    incl = kp;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) wsum[w] = incl;
  }
  __syncthreads();
  if (tid < MOE_MAX_EXPERTS) {
    for (int i = 0; i < w; ++i) incl += wsum[i];
    if (tid < E) {
      counts[tid] = cnt[tid];
      kept[tid] = kp;
      off[tid] = incl - kp;
      offs[tid] = incl - kp;
    }
    if (tid == E - 1) {
      off[E] = incl;
      offs[E] = incl;
    }
  }
  __syncthreads();
  const int per = E / R;
  for (int r = tid; r < R; r += kSmallThreads) {
    rank_counts[r] = offs[(r + 1) * per] - offs[r * per];
    rank_off[r] = offs[r * per];
  }
  if (tid == 0) rank_off[R] = offs[E];
  // ranks, one round of kSmallThreads assignments at a time
  for (int64_t base = 0; base < n_assign; base += kSmallThreads) {
    for (int e = lane; e < MOE_MAX_EXPERTS; e += 64) wc[w][e] = 0;
    __syncthreads();
    const int64_t g = base + tid;
    const bool in_range = g < n_assign;
    const int e = in_range ? ids[g] : -1;
    const bool valid = in_range && e >= 0 && e < E;
    if (valid) atomicAdd(&wc[w][e], 1);
    __syncthreads();
    for (int ee = tid; ee < E; ee += kSmallThreads) {
      int r = run[ee];
#pragma unroll
      for (int i = 0; i < kSmallWaves; ++i) {
        const int c = wc[i][ee];
        wc[i][ee] = r;
        r += c;
      }
      run[ee] = r;
    }
    __syncthreads();
    uint64_t todo = ballot(valid);
    int rk = 0;
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int el = __shfl(e, leader, 64);
      const uint64_t m = ballot(valid && e == el);
      if (valid && e == el) rk = popc64(m & lanemask_lt());
      todo &= ~m;
    }
    if (in_range) {
      int s = -1;
      if (valid) {
        const int pos = wc[w][e] + rk;
        if (pos < C) {
          s = offs[e] + pos;
          src_out[s] = (int32_t)(g / k);
        }
      }
      slot_out[g] = s;
    }
    __syncthreads();
  }
}

// One workgroup per token (its 4 waves split the row): the row is read once
// and written to each kept slot, with every piece in flight at once.
template <int UNROLL>
__global__ void __launch_bounds__(kThreads) pack_kernel(const int32_t* __restrict__ slot,
                                                       const u32x4* __restrict__ x,
                                                       u32x4* __restrict__ x_send, int64_t T, int k,
                                                       int row16) {
  const int lane = threadIdx.x;  // 0..255 over the row
  const int64_t t = blockIdx.x;
  if (t >= T) return;
  int sj[MOE_MAX_TOPK];
  bool any = false;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    sj[j] = j < k ? slot[t * k + j] : -1;
    any |= sj[j] >= 0;
  }
  if (!any) return;
  const u32x4* xr = x + t * row16;
  for (int c0 = lane; c0 < row16; c0 += kThreads * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int c = c0 + u * kThreads;
      if (c < row16) v[u] = xr[c];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (sj[j] < 0) continue;
      u32x4* dst = x_send + (int64_t)sj[j] * row16;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int c = c0 + u * kThreads;
        if (c < row16) store_row16(dst + c, v[u]);
      }
    }
  }
}

// Tiny batches (T*k <= kTinyAssign, decode): one launch.  Every workgroup
// owns one token and recomputes the whole plan it needs from all the ids
// (at most kTinyAssign of them, read once into LDS): the per-expert
// histogram and offsets, and for each of its assignments the number of
// earlier assignments (token-major order) to the same expert, which is its
// position in that expert's segment.  Workgroup 0 also writes the counts
// and offsets.  The redundant plan costs a few microseconds of latency that
// overlaps the row copies; it saves the separate single-workgroup launch.
constexpr int kTinyAssign = 1024;

__global__ void __launch_bounds__(kThreads) plan_pack_tiny_kernel(
    const int32_t* __restrict__ ids, int64_t T, int k, int E, int R, int C,
    int32_t* __restrict__ counts, int32_t* __restrict__ kept, int32_t* __restrict__ off,
    int32_t* __restrict__ rank_counts, int32_t* __restrict__ rank_off,
    int32_t* __restrict__ slot_out, int32_t* __restrict__ src_out, const u32x4* __restrict__ x,
    u32x4* __restrict__ x_send, int row16) {
  __shared__ int s_ids[kTinyAssign];
  __shared__ int cnt[MOE_MAX_EXPERTS];
  __shared__ int offs[MOE_MAX_EXPERTS + 1];
  __shared__ int wsum[kWaves];
  __shared__ int part[kWaves][MOE_MAX_TOPK];
  __shared__ int s_slot[MOE_MAX_TOPK];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = tid / 64;
  const int64_t t = blockIdx.x;
  const int n = (int)(T * k);
  for (int e = tid; e < MOE_MAX_EXPERTS; e += kThreads) cnt[e] = 0;
  for (int g = tid; g < n; g += kThreads) s_ids[g] = ids[g];
  __syncthreads();
  for (int g = tid; g < n; g += kThreads) {
    const int e = s_ids[g];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of kept over the experts (one expert per thread)
  const int kp = tid < E ? min(cnt[tid], C) : 0;
  int incl = kp;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  for (int i = 0; i < w; ++i) incl += wsum[i];
  if (tid < E) offs[tid] = incl - kp;
  if (tid == E - 1) offs[E] = incl;
  if (t == 0 && tid < E) {
    counts[tid] = cnt[tid];
    kept[tid] = kp;
    off[tid] = incl - kp;
  }
  if (t == 0 && tid == E - 1) off[E] = incl;
  // earlier assignments to the same expert, for each of this token's k
  const int64_t first = t * k;
  int my_e[MOE_MAX_TOPK];
  int c[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    my_e[j] = j < k ? s_ids[first + j] : -1;
    c[j] = 0;
  }
  for (int g = tid; g < n; g += kThreads) {
    const int e = s_ids[g];
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) c[j] += (g < first + j && e == my_e[j]) ? 1 : 0;
  }
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) c[j] += __shfl_xor(c[j], o, 64);
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) part[w][j] = c[j];
  }
  __syncthreads();
  if (t == 0) {
    const int per = E / R;
    for (int r = tid; r < R; r += kThreads) {
      rank_counts[r] = offs[(r + 1) * per] - offs[r * per];
      rank_off[r] = offs[r * per];
    }
    if (tid == 0) rank_off[R] = offs[E];
  }
  if (tid < k) {
    const int e = my_e[tid];
    int pos = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) pos += part[i][tid];
    int sl = -1;
    if (e >= 0 && e < E && pos < C) {
      sl = offs[e] + pos;
      src_out[sl] = (int32_t)t;
    }
    slot_out[first + tid] = sl;
    s_slot[tid] = sl;
  }
  __syncthreads();
  // the row, read once, to each kept slot
  int sj[MOE_MAX_TOPK];
  bool any = false;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    sj[j] = j < k ? s_slot[j] : -1;
    any |= sj[j] >= 0;
  }
  if (!any) return;
  const u32x4* xr = x + t * row16;
  constexpr int UNROLL = 2;
  for (int c0 = tid; c0 < row16; c0 += kThreads * UNROLL) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int cc = c0 + u * kThreads;
      if (cc < row16) v[u] = xr[cc];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (sj[j] < 0) continue;
      u32x4* dst = x_send + (int64_t)sj[j] * row16;
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int cc = c0 + u * kThreads;
        if (cc < row16) store_row16(dst + cc, v[u]);
      }
    }
  }
}

struct Plan {
  int tokens_per_block;
  int nblocks;
};

// Histogram/pack blocks per CU the token range is cut into: fewer blocks
// shorten the single-workgroup scan over blocks x experts, more keep the pack
// busy.  Measured with one block per CU: DeepSeek-V3 share (top-8) dispatch
// 212 -> 204 us, Switch (top-1) 36 -> 50 us, top-2 workloads within 1 us;
// so one block per CU from top-4 up.
constexpr int kDispatchBlocksPerCu = 2;
constexpr int kDispatchBlocksPerCuWide = 1;
Plan plan_for(int64_t T, int k) {
  int tb = kThreads / k;  // TB*k <= 256
  const int64_t target_blocks =
      (k >= 4 ? kDispatchBlocksPerCuWide : kDispatchBlocksPerCu) *
      (int64_t)device_info().cus;
  const int64_t small = (T + target_blocks - 1) / target_blocks;
  if (small < tb) tb = (int)(small < 1 ? 1 : small);
  Plan p;
  p.tokens_per_block = tb;
  p.nblocks = (int)((T + tb - 1) / tb);
  return p;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int64_t moe_send_rows_max(int64_t T, int32_t k, int32_t E, int32_t capacity) {
  const int64_t a = T * (int64_t)k;
  const int64_t b = (int64_t)E * (int64_t)capacity;
  return a < b ? a : b;
}

extern "C" size_t moe_dispatch_workspace_bytes(const moe_dispatch_args* a) {
  if (!a || a->T <= 0 || a->k <= 0 || a->T * a->k <= kSmallAssign) return 0;
  const Plan p = plan_for(a->T, a->k);
  const int E4 = (a->E + 3) & ~3;  // block histogram rows padded to 4 experts
  return align_up((size_t)p.nblocks * E4 * sizeof(int32_t), 256);
}

extern "C" moe_status moe_dispatch(const moe_dispatch_args* a, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  clear_error();
  MOE_CHECK_ARG(a != nullptr, "null args");
  MOE_CHECK_ARG(a->T >= 0, "T < 0");
  MOE_CHECK_ARG(a->E >= 1 && a->E <= MOE_MAX_EXPERTS, "E out of range [1, 256]");
  MOE_CHECK_ARG(a->k >= 1 && a->k <= MOE_MAX_TOPK && a->k <= a->E, "k out of range [1, min(8, E)]");
  MOE_CHECK_ARG(a->R >= 1 && a->E % a->R == 0, "E must be a positive multiple of R");
  MOE_CHECK_ARG(a->capacity >= 0, "capacity < 0");
  MOE_CHECK_ARG(a->act_dtype == MOE_F32 || a->act_dtype == MOE_BF16, "bad act_dtype");
  const int es = a->act_dtype == MOE_F32 ? 4 : 2;
  MOE_CHECK_ARG(a->d >= 1 && ((int64_t)a->d * es) % 16 == 0, "row of x must be a multiple of 16 bytes");
  MOE_CHECK_ARG(a->T * (int64_t)a->k < (int64_t)1 << 31, "T*k must fit in int32");
  MOE_CHECK_ARG(a->counts && a->kept && a->expert_off && a->rank_counts && a->rank_off,
                "count/offset outputs are required");
  MOE_CHECK_ARG(a->ids && a->slot && a->src && a->x && a->x_send, "null data pointer");
  MOE_CHECK_ARG(aligned16(a->x) && aligned16(a->x_send), "x/x_send not 16-byte aligned");
  const int row16 = (int)((int64_t)a->d * es / 16);
  const Plan p = plan_for(a->T, a->k);
  const size_t need = moe_dispatch_workspace_bytes(a);
  if (need > 0 && (ws_bytes < need || ws == nullptr)) {
    set_error("moe_dispatch: workspace too small");
    return MOE_ERR_WORKSPACE;
  }
  if (check_only()) return MOE_OK;
  if (a->T > 0 && a->T * a->k <= kTinyAssign) {
    plan_pack_tiny_kernel<<<(int)a->T, kThreads, 0, stream>>>(
        a->ids, a->T, a->k, a->E, a->R, a->capacity, a->counts, a->kept, a->expert_off,
        a->rank_counts, a->rank_off, a->slot, a->src, (const u32x4*)a->x, (u32x4*)a->x_send, row16);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  if (a->T > 0 && a->T * a->k <= kSmallAssign) {
    plan_small_kernel<<<1, kSmallThreads, 0, stream>>>(
        a->ids, a->T * a->k, a->k, a->E, a->R, a->capacity, a->counts, a->kept, a->expert_off,
        a->rank_counts, a->rank_off, a->slot, a->src);
    MOE_CHECK_LAUNCH();
    pack_kernel<2><<<(int)a->T, kThreads, 0, stream>>>(
        a->slot, (const u32x4*)a->x, (u32x4*)a->x_send, a->T, a->k, row16);
    MOE_CHECK_LAUNCH();
    return MOE_OK;
  }
  int32_t* blk = static_cast<int32_t*>(ws);
  const int nblocks = a->T > 0 ? p.nblocks : 0;
  if (nblocks > 0) {
    hist_kernel<<<nblocks, kThreads, 0, stream>>>(a->ids, blk, a->T * a->k,
                                                  p.tokens_per_block * a->k, a->E);
    MOE_CHECK_LAUNCH();
  }
  // with no tokens one block still writes the zero counts and offsets
  rank_pack_kernel<4><<<nblocks > 0 ? nblocks : 1, kThreads, 0, stream>>>(
      a->ids, blk, nblocks, (const u32x4*)a->x, a->slot, a->src, (u32x4*)a->x_send, a->T, a->k,
      a->E, a->R, a->capacity, p.tokens_per_block, row16, a->counts, a->kept, a->expert_off,
      a->rank_counts, a->rank_off);
  MOE_CHECK_LAUNCH();
  return MOE_OK;
}
