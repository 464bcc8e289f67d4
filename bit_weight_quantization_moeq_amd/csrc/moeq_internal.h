// Internal declarations shared by the libmoeq HIP translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moeq.h"

namespace moeq {

// ---------------------------------------------------------------------------
// NF4 constants (frozen).  The pages name the NF4 format ("MoE Expert
// Quantization", Implementation details) without printing its levels; these
// are the QLoRA NormalFloat levels: standard-normal quantiles at evenly
// spaced probabilities from delta = ((1-1/30)+(1-1/32))/2 towards 1/2, 8 on
// the positive side and 7 on the negative side plus an exact zero, divided
// by the largest magnitude, formed in fp64 and rounded once to fp32.
// ---------------------------------------------------------------------------
constexpr uint32_t kNf4LevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

// Decision thresholds: t_i is the largest fp32 not above the exact midpoint
// (level_i + level_{i+1}) / 2.  With n = fp32(w / absmax), the nearest level
// (ties to the lower one) is #{i : n > t_i}.  For bf16 w and absmax a > 0 the
// kernels evaluate n > t_i without the division, as the exact test
// w >= a * t_i (the sign of fma(a, t_i, -w)); the two agree on every pair of
// bf16 values, which an exhaustive enumeration of all bf16 ratios confirms
// (no bf16 ratio falls between t_i and the rounding boundary above it).
constexpr uint32_t kNf4ThresholdBits[15] = {
    0xbf591cd9u, 0xbf1c5270u, 0xbeeb847du, 0xbeadea75u, 0xbe703ceau,
    0xbe0d38b9u, 0xbd3a7869u, 0x3d22fb01u, 0x3df6485fu, 0x3e5067dcu,
    0x3e9582d1u, 0x3ec753f5u, 0x3f006d01u, 0x3f248dacu, 0x3f5c89d8u};

constexpr int kNf4Block = 64;
constexpr int kNf4ZeroCode = 7;

// Double-quantized absmax: groups of 2^kDqGroupShift consecutive blocks of
// one expert share one fp32 group scale.
constexpr int kDqGroupShift = 8;
static_assert((1 << kDqGroupShift) == MOEQ_DQ_GROUP, "group size");
__host__ __device__ constexpr int64_t dq_groups(int64_t blocks_per_expert) {
  return (blocks_per_expert + MOEQ_DQ_GROUP - 1) >> kDqGroupShift;
}

// The NF4 decision in the kernels first picks a bucket of width 1/16 in n
// from an approximate ratio, then makes one exact threshold test.  Bucket j
// covers n in [(j-17)/16, (j-16)/16); every bucket holds at most one
// threshold and no threshold lies within 1e-3 of a bucket edge, so an
// approximate ratio that strays into a neighbouring bucket still yields the
// same code.  Entry: {threshold to test (2.0 when the bucket has none),
// number of thresholds below the bucket}.
constexpr int kNf4Buckets = 34;

// ---------------------------------------------------------------------------
// Launch helpers (host side), one per translation unit's kernels.
// ---------------------------------------------------------------------------
hipError_t launch_quantize_nf4(const uint16_t* w, uint8_t* q, float* absmax, int64_t nblocks,
                               hipStream_t s);
hipError_t launch_stream_reference(const uint16_t* w, uint8_t* q, float* absmax, int64_t nblocks, hipStream_t s);
hipError_t launch_quantize_int8(const uint16_t* w, int8_t* q, float* scale, int64_t nrows,
                                int32_t cols, hipStream_t s);
hipError_t launch_dequantize_nf4(const uint8_t* q, const float* absmax, uint16_t* out,
                                 int64_t nblocks, hipStream_t s);
hipError_t launch_dequantize_int8(const int8_t* q, const float* scale, uint16_t* out,
                                  int64_t nrows, int32_t cols, hipStream_t s);
// Double-quantized absmax: nb blocks per expert, E experts.
hipError_t launch_quantize_nf4_dq(const uint16_t* w, uint8_t* q, uint8_t* codes, float* gscale, int32_t E,
                                  int64_t nb, hipStream_t s);
hipError_t launch_compress_absmax(const float* absmax, uint8_t* codes, float* gscale, int32_t E, int64_t nb,
                                  hipStream_t s);
hipError_t launch_dequantize_nf4_dq(const uint8_t* q, const uint8_t* codes, const float* gscale, uint16_t* out,
                                    int32_t E, int64_t nb, hipStream_t s);

// Routing workspace carve-up (all int32).
struct RouteBuffers {
  int32_t* chunk_counts;  // [nchunk][E]
  int32_t* chunk_base;    // [nchunk][E]
  int32_t* rank;          // [n]
  int32_t* counts;        // [E]
  int32_t* offsets;       // [E+1]
  int32_t* tile_start;    // [E+1] (prefix sum of ceil(counts / tile_rows))
  int32_t* perm;          // [n]
  int32_t* slot;          // [n]
};
constexpr int kRouteChunk = 256;
int64_t route_chunks(int64_t n);
hipError_t launch_route(const int32_t* idx, int32_t n, int32_t E, int32_t tile_rows,
                        const RouteBuffers& b, hipStream_t s);
// Steps 2 and 3 of the routing stage (per-expert scan, scatter) over chunks of
// `chunk` assignments whose rank and chunk_counts are already in b.
hipError_t launch_route_tail(const int32_t* idx, int32_t n, int32_t E, int32_t tile_rows, int32_t chunk,
                             const RouteBuffers& b, hipStream_t s);
hipError_t launch_tile_start(const int32_t* offsets, int32_t E, int32_t tile_rows, int32_t* tile_start,
                             hipStream_t s);

struct ForwardArgs {
  const uint16_t* x;        // [T][H]
  const int32_t* idx;       // [T][K]
  const float* wts;         // [T][K]
  int32_t T, K, E, H, I;
  int32_t format;
  const void* gu_q;         // gate_up codes
  const float* gu_s;        // gate_up scales (double-quantized: group scales)
  const uint8_t* gu_c;      // gate_up absmax codes (double-quantized only)
  const void* dn_q;         // down codes
  const float* dn_s;        // down scales
  const uint8_t* dn_c;
  uint16_t* out;            // [T][H]
  RouteBuffers rb;
  uint16_t* h;              // [T*K][I] bf16, expert-sorted rows
  float* y;                 // [T*K][H]: bf16 expert-sorted rows (tiled path) or fp32 (few-assignment path)
  bool routed;              // rb.offsets / perm / slot already hold the routing of idx (only
                            // tile_start is derived here)
  float* gu_save = nullptr; // [T*K][2I] fp32, expert-sorted rows: g | u kept for the backward
                            // (non-null: the tiled path for every batch size)
};
// events: NULL or 5 events recorded at the stage boundaries.
hipError_t launch_experts_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t const* events);
// The few-assignment (decode) forward, n = T*K <= 512 (decode.hip); called by
// launch_experts_forward.
hipError_t launch_experts_decode(const ForwardArgs& a, hipStream_t s, hipEvent_t const* events);
// Slices of y the few-assignment forward's down launch writes (1, 2 or 4: K
// split across workgroups when few experts are touched); 1 off that path.
int decode_down_splits(int64_t n, int32_t E, int64_t H, int64_t I);

struct BackwardArgs {
  const uint16_t* x;        // [T][H]
  const int32_t* idx;       // [T][K]
  const float* wts;         // [T][K]
  const uint16_t* dout;     // [T][H]
  int32_t T, K, E, H, I;
  int32_t format;
  const void* gu_q;
  const float* gu_s;
  const uint8_t* gu_c;
  const void* dn_q;
  const float* dn_s;
  const uint8_t* dn_c;
  uint16_t* grad_x;         // [T][H]
  float* grad_w;            // [T][K]
  RouteBuffers rb;
  float* gw_part;           // [n][backward_col_tiles(I)] fp32, sorted rows: T1's shares of grad_w
  float* gu_save;           // [n][2I] fp32, sorted rows
  bool recompute = true;    // false: gu_save already holds the forward's g | u (no gate_up GEMM)
  float* dx;                // [n][H] fp32, sorted rows
  uint16_t* dgu;            // [n][2I] bf16, sorted rows
};
hipError_t launch_experts_backward(const BackwardArgs& a, hipStream_t s);

// rank / chunk_counts: nullptr, or the routing stage's rank and chunk counts
// for chunks of kRouterChunkTokens tokens (K <= kRouterRankMaxK).
constexpr int kRouterChunkTokens = 16;
constexpr int kRouterRankMaxK = 64;
hipError_t launch_router(const uint16_t* x, const uint16_t* gate, int32_t T, int32_t H, int32_t E, int32_t K,
                         int32_t renorm, int32_t* idx, float* wts, int32_t* rank, int32_t* chunk_counts,
                         hipStream_t s);
int32_t forward_tile_rows();
// column tiles of the backward's T1 over I columns (grad_w shares per row)
int32_t backward_col_tiles(int32_t I);

}  // namespace moeq
