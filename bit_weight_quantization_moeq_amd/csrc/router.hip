// Router front-end: logits = gate @ x_t (bf16 operands, fp32 MFMA
// accumulation), softmax over the E experts, top-K selection (largest logit
// first, equal logits to the lower expert index), weights = the selected
// probabilities or, renormalised, those divided by their sum.  The gate
// weight mlp.gate.weight stays bf16 next to the quantized experts
// ("MoE Expert Quantization", Axolotl docs, Expert LoRA targeting;
// bitsandbytes issue #1849, maintainer thread: router-only training over
// NF4 experts); its output is the (top_k_index, top_k_weights) pair of the
// experts interface (unsloth-zoo issue #850, Suggested fix).
//
// One workgroup (4 waves) per 16 tokens.  Wave w computes the logits of the
// expert blocks w, w + 4, ... (32 experts each) for the 16 tokens with
// v_mfma_f32_32x32x16_bf16 (gate rows as A, token rows as B; token columns
// 16..31 of the MFMA are zero), K running over H.  The logits meet in LDS;
// then each wave takes 4 tokens: max, sum of exponentials and K rounds of
// arg-max are wave reductions in a fixed butterfly order, so the result is
// deterministic.
#include "moeq_internal.h"

namespace moeq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTok = 16;  // tokens per workgroup

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// (value, index) order of the selection: larger value first, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int RBW>  // expert blocks of 32 per wave
__global__ __launch_bounds__(kThreads) void router_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ gate, int32_t T, int32_t H,
                                                         int32_t E, int32_t K, int32_t renorm, int32_t P,
                                                         int32_t* __restrict__ idx, float* __restrict__ wts) {
  extern __shared__ float slog[];  // [P][kTok][E]: partial logits of the P parts of H
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  // waves = (expert block groups) x (P parts of H): wave w takes part w % P
  // of H for the expert blocks w / P, w / P + 4 / P, ...
  const int part = wave % P, g0 = wave / P, gstep = kWaves / P;
  const int hlen = H / P, h0 = part * hlen;  // H % (64 P) == 0
  const int n64 = hlen / 64;                 // trips of 64 k

  // B operand: token row t0 + l32; A operands: gate rows e = 32 (g0 + gstep
  // j) + l32.  Rows past the tokens (l32 >= 16, or past T) or past the
  // experts read row 0 instead: their logits land in columns or rows never
  // stored.
  const bool tok_on = l32 < kTok && t0 + l32 < T;
  const uint16_t* xr = x + (tok_on ? (t0 + l32) : 0) * (int64_t)H + h0 + 8 * hh;
  const uint16_t* gr[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int e = 32 * (g0 + gstep * j) + l32;
    gr[j] = gate + (int64_t)(e < E ? e : 0) * H + h0 + 8 * hh;
  }
  f32x16 acc[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) acc[j] = (f32x16){};
  // two trips of 64 k in flight: the loads of trip i+1 issue before trip i's
  // MFMAs (register sets used in turn)
  struct Frags {
    bf16x8 b[4], a[4][RBW];
  };
  auto load = [&](Frags& f, int trip) {
    const int kc = trip < n64 ? 64 * trip : 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f.b[u] = ld8(xr + kc + 16 * u);
#pragma unroll
      for (int j = 0; j < RBW; ++j) f.a[u][j] = ld8(gr[j] + kc + 16 * u);
    }
  };
  auto mul = [&](const Frags& f) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < RBW; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[u][j], f.b[u], acc[j], 0, 0, 0);
  };
  Frags fa, fb;
  load(fa, 0);
  int i = 0;
  for (; i + 1 < n64; i += 2) {  // no branch between the two trips
    load(fb, i + 1);
    __builtin_amdgcn_sched_barrier(0);  // the next trip's loads issue before this trip's MFMAs
    mul(fa);
    __builtin_amdgcn_sched_barrier(0);
    load(fa, i + 2);
    __builtin_amdgcn_sched_barrier(0);
    mul(fb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i < n64) mul(fa);  // odd trip count: the last trip, already loaded
  // lane holds partial logits of experts 32 (g0 + gstep j) + 8 q + 4 hh + i for token l32
  if (l32 < kTok) {
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 32 * (g0 + gstep * j) + 8 * q + 4 * hh + i;
          if (e < E) slog[(part * kTok + l32) * E + e] = acc[j][4 * q + i];
        }
    }
  }
  __syncthreads();
  if (P > 1) {  // add the parts in part order into part 0
    for (int i = t; i < kTok * E; i += kThreads) {
      float v = slog[i];
      for (int p = 1; p < P; ++p) v += slog[p * kTok * E + i];
      slog[i] = v;
    }
    __syncthreads();
  }

  // softmax and top-K: wave w takes tokens w, w + 4, w + 8, w + 12
  constexpr int kPer = (MOEQ_MAX_EXPERTS + 63) / 64;  // logits per lane (at most)
  for (int tt = wave; tt < kTok; tt += kWaves) {
    const int64_t tok = t0 + tt;
    if (tok >= T) break;
    float v[kPer];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? slog[tt * E + e] : -INFINITY;
      m = fmaxf(m, v[j]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < kPer; ++j) sum += (lane + 64 * j < E) ? __expf(v[j] - m) : 0.0f;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
    const float inv = 1.0f / sum;
    // K rounds of arg-max (every lane ends a round holding the winner, whose
    // owner then takes it out of the race).  With renormalisation the sum of
    // the selected probabilities comes from a first pass over the same
    // selections, so the second pass can write the final weights.
    float sel_sum = 1.0f;
    for (int pass = renorm ? 0 : 1; pass < 2; ++pass) {
      float u[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) u[j] = v[j];
      float acc_p = 0.0f;
      const float scale = inv / sel_sum;
      for (int k = 0; k < K; ++k) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int e = lane + 64 * j;
          if (e < E && better(u[j], e, bv, bi)) {
            bv = u[j];
            bi = e;
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float ov = __shfl_xor(bv, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
          }
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (lane + 64 * j == bi) u[j] = -INFINITY;
        const float ex = __expf(bv - m);
        if (pass == 0) {
          acc_p += ex * inv;
        } else if (lane == 0) {
          idx[tok * K + k] = bi;
          wts[tok * K + k] = ex * scale;
        }
      }
      if (pass == 0) sel_sum = acc_p;
    }
  }
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* gate, int32_t T, int32_t H, int32_t E, int32_t K,
                         int32_t renorm, int32_t* idx, float* wts, hipStream_t s) {
  const int grid = (T + kTok - 1) / kTok;
  const int nrb = (E + 31) / 32;  // expert blocks of 32
  // few expert blocks: split H across the waves instead (P parts, H % 64P == 0)
  int P = nrb >= kWaves ? 1 : (nrb >= 2 ? 2 : 4);
  while (P > 1 && H % (64 * P) != 0) P /= 2;
  const int rbw = (nrb * P + kWaves - 1) / kWaves;  // expert blocks per wave
  const size_t lds = sizeof(float) * kTok * (size_t)E * P;
  if (rbw <= 1)
    router_kernel<1><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts);
  else if (rbw <= 2)
    router_kernel<2><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts);
  else if (rbw <= 4)
    router_kernel<4><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts);
  else
    router_kernel<8><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts);
  return hipGetLastError();
}

}  // namespace moeq
