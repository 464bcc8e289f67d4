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
// One workgroup (4 waves) per 16 tokens.  The waves split the expert blocks
// (32 experts each) and, when there are few, H as well; each computes its
// logits for the 16 tokens with v_mfma_f32_32x32x16_bf16 (gate rows as A,
// token rows as B; token columns 16..31 of the MFMA are unused), K running
// over H.  The logits meet in LDS; then each wave takes 4 tokens at once:
// max, sum of exponentials and K rounds of arg-max are DPP wave reductions
// in a fixed order, so the result is deterministic.
#include "moeq_internal.h"

namespace moeq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTok = 16;  // tokens per workgroup

__device__ __forceinline__ bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Wave reductions on DPP lane moves (quad permutes, half-row and row
// mirrors, then the row broadcasts that carry each row's result into the
// next rows), read from lane 63: a fixed order, so deterministic, and short
// dependent chains of VALU instructions.  `id` is the operation's identity,
// returned by lanes a move does not write.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x, uint32_t id) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v, 0u));        // quad_perm [1,0,3,2]
  v = max(v, dpp_u<0x4E>(v, 0u));        // quad_perm [2,3,0,1]
  v = max(v, dpp_u<0x141>(v, 0u));       // row_half_mirror
  v = max(v, dpp_u<0x140>(v, 0u));       // row_mirror: every lane holds its row's max
  v = max(v, dpp_u<0x142, 0xA>(v, 0u));  // row_bcast15 into rows 1 and 3
  v = max(v, dpp_u<0x143, 0xC>(v, 0u));  // row_bcast31 into rows 2 and 3
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  const uint32_t id = 0xffffffffu;
  v = min(v, dpp_u<0xB1>(v, id));
  v = min(v, dpp_u<0x4E>(v, id));
  v = min(v, dpp_u<0x141>(v, id));
  v = min(v, dpp_u<0x140>(v, id));
  v = min(v, dpp_u<0x142, 0xA>(v, id));
  v = min(v, dpp_u<0x143, 0xC>(v, id));
  return __builtin_amdgcn_readlane(v, 63);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_fsum(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ float wave_fsum(float v) {
  v += dpp_fsum<0xB1>(v);
  v += dpp_fsum<0x4E>(v);
  v += dpp_fsum<0x141>(v);
  v += dpp_fsum<0x140>(v);
  v += dpp_fsum<0x142, 0xA>(v);
  v += dpp_fsum<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// fp32 -> uint32 with the same order (-0 taken as +0 first); and back
__device__ __forceinline__ uint32_t ord(float f) {
  const uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Softmax over the E logits of each of the block's tokens and the K rounds of
// arg-max, from the logits in LDS; NPL logits per lane (E <= 64 NPL).
template <int NPL>
__device__ __forceinline__ void softmax_topk(const float* slog, int64_t t0, int32_t T, int32_t E, int32_t K,
                                             int32_t renorm, int wave, int lane, int32_t* __restrict__ idx,
                                             float* __restrict__ wts) {
  // softmax and top-K: wave w takes tokens w, w + 4, w + 8, w + 12, all four
  // at once (their cross-lane reductions are independent, so their shuffle
  // latencies overlap)
  constexpr int kTT = kTok / kWaves;                  // tokens per wave
  float v[kTT][NPL];
  float m[kTT], sum[kTT], inv[kTT];
#pragma unroll
  for (int q = 0; q < kTT; ++q) {
    const int tt = wave + kWaves * q;
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      v[q][j] = (e < E) ? slog[tt * E + e] : -INFINITY;
      lm = fmaxf(lm, v[q][j]);
    }
    m[q] = unord(wave_umax(ord(lm)));
  }
#pragma unroll
  for (int q = 0; q < kTT; ++q) {
    float ls = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) ls += (lane + 64 * j < E) ? __expf(v[q][j] - m[q]) : 0.0f;
    sum[q] = wave_fsum(ls);
    inv[q] = 1.0f / sum[q];
  }
  // K rounds of arg-max: the largest logit first (wave max of its ordered
  // bits), then the lowest index holding it (wave min), which its owner
  // takes out of the race.  With renormalisation the sum of the selected
  // probabilities comes from a first pass over the same selections, so the
  // second pass can write the final weights.
  float sel_sum[kTT];
#pragma unroll
  for (int q = 0; q < kTT; ++q) sel_sum[q] = 1.0f;
  for (int pass = renorm ? 0 : 1; pass < 2; ++pass) {
    float u[kTT][NPL], acc_p[kTT];
#pragma unroll
    for (int q = 0; q < kTT; ++q) {
      acc_p[q] = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) u[q][j] = v[q][j];
    }
    for (int k = 0; k < K; ++k) {
#pragma unroll
      for (int q = 0; q < kTT; ++q) {
        float lv = -INFINITY;
#pragma unroll
        for (int j = 0; j < NPL; ++j) lv = fmaxf(lv, u[q][j]);
        const uint32_t bm = wave_umax(ord(lv));
        uint32_t li = 0xffffffffu;  // this lane's lowest index holding the maximum
#pragma unroll
        for (int j = NPL - 1; j >= 0; --j) {
          const int e = lane + 64 * j;
          if (e < E && ord(u[q][j]) == bm) li = (uint32_t)e;
        }
        const int bi = (int)wave_umin(li);
#pragma unroll
        for (int j = 0; j < NPL; ++j)
          if (lane + 64 * j == bi) u[q][j] = -INFINITY;
        const float ex = __expf(unord(bm) - m[q]);
        const int64_t tok = t0 + wave + kWaves * q;
        if (pass == 0) {
          acc_p[q] += ex * inv[q];
        } else if (lane == 0 && tok < T) {
          idx[tok * K + k] = bi;
          wts[tok * K + k] = ex * (inv[q] / sel_sum[q]);
        }
      }
    }
    if (pass == 0) {
#pragma unroll
      for (int q = 0; q < kTT; ++q) sel_sum[q] = acc_p[q];
    }
  }
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

  switch ((E + 63) / 64) {
    case 1: softmax_topk<1>(slog, t0, T, E, K, renorm, wave, lane, idx, wts); break;
    case 2: softmax_topk<2>(slog, t0, T, E, K, renorm, wave, lane, idx, wts); break;
    case 3:
    case 4: softmax_topk<4>(slog, t0, T, E, K, renorm, wave, lane, idx, wts); break;
    case 5:
    case 6:
    case 7:
    case 8: softmax_topk<8>(slog, t0, T, E, K, renorm, wave, lane, idx, wts); break;
    default: softmax_topk<(MOEQ_MAX_EXPERTS + 63) / 64>(slog, t0, T, E, K, renorm, wave, lane, idx, wts); break;
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
