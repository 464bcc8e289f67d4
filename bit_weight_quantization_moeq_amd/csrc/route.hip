// Deterministic bucketing of top-k assignments by expert (gfx950).
//
// The experts forward takes (hidden_states, top_k_index, top_k_weights) for
// every fused-expert architecture (unsloth-zoo issue #850, Suggested fix), so
// one generic routing stage groups the assignments a = t*K + k by expert:
// counts, exclusive offsets, perm (expert-major, ascending a within an
// expert) and its inverse slot.  No step depends on the order in which
// atomics or workgroups execute, so the output is bit-identical run to run.
//
//   1. rank:    per chunk of 256 assignments, each assignment's stable rank
//               among earlier assignments of the same expert in the chunk
//               (wave ballots, then a prefix over the chunk's 4 waves), and
//               the chunk's per-expert counts.
//   2. scan:    per expert, the exclusive prefix of its chunk counts over the
//               chunks and the expert's total.
//   3. scatter: per chunk, offsets from the totals (recomputed in LDS), then
//               perm[offsets[e] + chunk_base[c][e] + rank[a]] = a.
// The router front-end can produce step 1 itself (its workgroups are the
// chunks: 16 tokens x K assignments each) and then runs steps 2 and 3 here.
#include "moeq_internal.h"

namespace moeq {
namespace {

constexpr int kThreads = 256;
static_assert(kRouteChunk == kThreads, "one assignment per thread and chunk");

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive scan of one value per thread across the 256-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum /*[4]*/, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v, lane);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  *total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  return before + inc - v;
}

__global__ __launch_bounds__(kThreads) void route_rank_kernel(const int32_t* __restrict__ idx, int32_t n,
                                                             int32_t E, int32_t* __restrict__ chunk_counts,
                                                             int32_t* __restrict__ rank) {
  __shared__ int wcnt[4][MOEQ_MAX_EXPERTS];
  for (int i = threadIdx.x; i < 4 * E; i += kThreads) wcnt[i / E][i % E] = 0;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t a = blockIdx.x * kThreads + threadIdx.x;
  const int e = (a < n) ? idx[a] : -1;
  const bool valid = (e >= 0) && (e < E);

  // Stable rank inside the wave: resolve one distinct expert per iteration.
  int r = 0;
  uint64_t pending = __ballot(valid);
  while (pending) {
    const int leader = __builtin_ctzll(pending);
    const int el = __shfl(e, leader, 64);
    const uint64_t same = __ballot(valid && e == el);
    if (valid && e == el) r = __popcll(same & ((1ull << lane) - 1ull));
    if (lane == leader) wcnt[wave][el] = __popcll(same);
    pending &= ~same;
  }
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wcnt[w][e];
    rank[a] = before + r;
  }
  int32_t* out = chunk_counts + (int64_t)blockIdx.x * E;
  for (int x = threadIdx.x; x < E; x += kThreads) out[x] = wcnt[0][x] + wcnt[1][x] + wcnt[2][x] + wcnt[3][x];
}

// One workgroup per expert: exclusive prefix of chunk counts in chunk order.
__global__ __launch_bounds__(kThreads) void route_scan_kernel(const int32_t* __restrict__ chunk_counts,
                                                             int32_t nchunk, int32_t E,
                                                             int32_t* __restrict__ chunk_base,
                                                             int32_t* __restrict__ counts) {
  __shared__ int wsum[4];
  const int e = blockIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < nchunk; c0 += kThreads) {
    const int c = c0 + threadIdx.x;
    const int v = (c < nchunk) ? chunk_counts[(int64_t)c * E + e] : 0;
    int total;
    const int ex = block_exclusive_scan(v, wsum, &total);
    if (c < nchunk) chunk_base[(int64_t)c * E + e] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// One workgroup per chunk of `chunk` consecutive assignments.
__global__ __launch_bounds__(kThreads) void route_scatter_kernel(
    const int32_t* __restrict__ idx, int32_t n, int32_t E, int32_t tile_rows, int32_t chunk,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ rank, int32_t* __restrict__ offsets, int32_t* __restrict__ tile_start,
    int32_t* __restrict__ perm, int32_t* __restrict__ slot) {
  __shared__ int off[MOEQ_MAX_EXPERTS + 1];
  __shared__ int wsum[4];
  // offsets = exclusive prefix of counts; each thread owns 4 consecutive experts.
  {
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 4 * threadIdx.x + i;
      v[i] = (x < E) ? counts[x] : 0;
      s += v[i];
    }
    int total;
    int ex = block_exclusive_scan(s, wsum, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 4 * threadIdx.x + i;
      if (x < E) off[x] = ex;
      ex += v[i];
    }
    if (threadIdx.x == 0) off[E] = total;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int x = threadIdx.x; x <= E; x += kThreads) offsets[x] = off[x];
    // tiles per expert for the grouped GEMMs: ceil(count / tile_rows)
    int v[4], s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 4 * threadIdx.x + i;
      v[i] = (x < E) ? (counts[x] + tile_rows - 1) / tile_rows : 0;
      s += v[i];
    }
    int total;
    int ex = block_exclusive_scan(s, wsum, &total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 4 * threadIdx.x + i;
      if (x < E) tile_start[x] = ex;
      ex += v[i];
    }
    if (threadIdx.x == 0) tile_start[E] = total;
  }
  const int32_t* base = chunk_base + (int64_t)blockIdx.x * E;
  for (int i = threadIdx.x; i < chunk; i += kThreads) {
    const int32_t a = blockIdx.x * chunk + i;
    if (a >= n) break;
    const int e = idx[a];
    if (e >= 0 && e < E) {
      const int p = off[e] + base[e] + rank[a];
      perm[p] = a;
      slot[a] = p;
    } else {
      slot[a] = -1;
    }
  }
}

// tile_start = exclusive prefix of ceil(count_e / tile_rows) from offsets
// (for a forward handed routing buffers made elsewhere); one workgroup.
__global__ __launch_bounds__(kThreads) void tile_start_kernel(const int32_t* __restrict__ offsets, int32_t E,
                                                             int32_t tile_rows, int32_t* __restrict__ tile_start) {
  __shared__ int wsum[4];
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = 4 * threadIdx.x + i;
    v[i] = (x < E) ? (offsets[x + 1] - offsets[x] + tile_rows - 1) / tile_rows : 0;
    s += v[i];
  }
  int total;
  int ex = block_exclusive_scan(s, wsum, &total);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = 4 * threadIdx.x + i;
    if (x < E) tile_start[x] = ex;
    ex += v[i];
  }
  if (threadIdx.x == 0) tile_start[E] = total;
}

}  // namespace

int64_t route_chunks(int64_t n) { return (n + kRouteChunk - 1) / kRouteChunk; }

hipError_t launch_route_tail(const int32_t* idx, int32_t n, int32_t E, int32_t tile_rows, int32_t chunk,
                             const RouteBuffers& b, hipStream_t s) {
  const int nchunk = n > 0 ? (n + chunk - 1) / chunk : 0;
  route_scan_kernel<<<E, kThreads, 0, s>>>(b.chunk_counts, nchunk, E, b.chunk_base, b.counts);
  route_scatter_kernel<<<nchunk > 0 ? nchunk : 1, kThreads, 0, s>>>(
      idx, n, E, tile_rows, chunk, b.counts, b.chunk_base, b.rank, b.offsets, b.tile_start, b.perm, b.slot);
  return hipGetLastError();
}

hipError_t launch_route(const int32_t* idx, int32_t n, int32_t E, int32_t tile_rows,
                        const RouteBuffers& b, hipStream_t s) {
  const int nchunk = (int)route_chunks(n);
  if (nchunk > 0) {
    route_rank_kernel<<<nchunk, kThreads, 0, s>>>(idx, n, E, b.chunk_counts, b.rank);
  }
  return launch_route_tail(idx, n, E, tile_rows, kRouteChunk, b, s);
}

hipError_t launch_tile_start(const int32_t* offsets, int32_t E, int32_t tile_rows, int32_t* tile_start,
                             hipStream_t s) {
  tile_start_kernel<<<1, kThreads, 0, s>>>(offsets, E, tile_rows, tile_start);
  return hipGetLastError();
}

}  // namespace moeq
