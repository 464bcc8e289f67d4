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
constexpr int kTok = kRouterChunkTokens;  // tokens per workgroup

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

// Softmax and top-K by radix select, for E <= 64 NPL with small NPL: the
// K-th largest order-preserving key (ord of the logit) is found bit by bit
// from the top, each bit one compare whose ballot, masked to the remaining
// candidates, gives a scalar count; keys above it are taken, and of the keys
// equal to it the lowest expert indices fill the rest.  The bits stop as soon
// as the remaining candidates are exactly as many as still needed (for
// distinct logits after about a dozen bits).  A taken expert's
// output slot is its rank among the taken (a larger logit first, equal
// logits by the lower index): the same selection and order as K rounds of
// arg-max.  Renormalised weights divide by the sum of the taken
// probabilities (one wave sum).  Wave w takes tokens w, w + 4, w + 8, w + 12,
// one after the other (four at once measured no faster: their candidate
// masks spill scalar registers).
template <int NPL>
__device__ __forceinline__ void softmax_topk_radix(const float* slog, int64_t t0, int32_t T, int32_t E, int32_t K,
                                                   int32_t renorm, int wave, int lane, int32_t* __restrict__ idx,
                                                   float* __restrict__ wts, int* sel) {
  constexpr int kTT = kTok / kWaves;  // tokens per wave, one after the other
  for (int q = 0; q < kTT; ++q) {
    const int tt = wave + kWaves * q;
    float v[NPL];
    uint32_t key[NPL];
    uint64_t cand[NPL], take[NPL];
    float lm = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      const bool valid = e < E;
      v[j] = valid ? slog[tt * E + e] : -INFINITY;
      key[j] = ord(v[j]);
      cand[j] = __ballot(valid);
      take[j] = 0;
      lm = fmaxf(lm, v[j]);
    }
    const float m = unord(wave_umax(ord(lm)));
    float ls = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) ls += (lane + 64 * j < E) ? __expf(v[j] - m) : 0.0f;
    const float inv = 1.0f / wave_fsum(ls);
    int need = K;
    for (int bit = 31; bit >= 0; --bit) {
      int cc = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) cc += __popcll(cand[j]);
      if (cc == need) break;  // every remaining candidate is among the K: take them all below
      uint64_t hi[NPL];
      int c1 = 0;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        hi[j] = cand[j] & __ballot((key[j] >> bit) & 1u);
        c1 += __popcll(hi[j]);
      }
      if (c1 >= need) {
#pragma unroll
        for (int j = 0; j < NPL; ++j) cand[j] = hi[j];
      } else {
        need -= c1;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          take[j] |= hi[j];
          cand[j] &= ~hi[j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      while (need > 0 && cand[j]) {
        const uint64_t low = cand[j] & (~cand[j] + 1);
        take[j] |= low;
        cand[j] ^= low;
        --need;
      }
    }
    int rank[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) rank[j] = 0;
#pragma unroll
    for (int jj = 0; jj < NPL; ++jj) {
      for (uint64_t b = take[jj]; b; b &= b - 1) {
        const int l = __builtin_ctzll(b);
        const uint32_t k2 = __builtin_amdgcn_readlane(key[jj], l);
        const int e2 = l + 64 * jj;
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const int e = lane + 64 * j;
          rank[j] += (k2 > key[j] || (k2 == key[j] && e2 < e)) ? 1 : 0;
        }
      }
    }
    float ex[NPL];
    float ps = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const bool mine = (take[j] >> lane) & 1u;
      ex[j] = mine ? __expf(v[j] - m) : 0.0f;
      ps += ex[j] * inv;
    }
    const float sel_sum = renorm ? wave_fsum(ps) : 1.0f;
    const int64_t tok = t0 + tt;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      if (((take[j] >> lane) & 1u) && tok < T) {
        const int e = lane + 64 * j;
        idx[tok * K + rank[j]] = e;
        wts[tok * K + rank[j]] = ex[j] * (inv / sel_sum);
        if (sel) sel[tt * K + rank[j]] = e;
      }
    }
  }
}

// Softmax over the E logits of each of the block's tokens and the K rounds of
// arg-max, from the logits in LDS; NPL logits per lane (E <= 64 NPL).
// sel (LDS, or nullptr): the selections again, sel[tt * K + k] for the
// block's token tt.
template <int NPL>
__device__ __forceinline__ void softmax_topk(const float* slog, int64_t t0, int32_t T, int32_t E, int32_t K,
                                             int32_t renorm, int wave, int lane, int32_t* __restrict__ idx,
                                             float* __restrict__ wts, int* sel) {
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
          if (sel) sel[(wave + kWaves * q) * K + k] = bi;
        }
      }
    }
    if (pass == 0) {
#pragma unroll
      for (int q = 0; q < kTT; ++q) sel_sum[q] = acc_p[q];
    }
  }
}

// The chunk of this workgroup's selections (its tokens' K assignments, in
// assignment order), ranked for the routing stage: rank[a] = the number of
// earlier assignments of the chunk with the same expert, chunk_counts[c][e] =
// the chunk's assignments of expert e.  The same quantities, in the same
// order, as the routing stage's own rank step computes from top_k_index.
// Resolves one distinct expert per wave ballot, 256 assignments at a time,
// with running per-expert counts in LDS.  wcnt: LDS [4][E] + run [E].
__device__ __forceinline__ void chunk_rank(const int* sel, int m, int32_t E, int* wcnt, int64_t a0,
                                           int32_t* __restrict__ rank, int32_t* __restrict__ counts_out) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int* run = wcnt + 4 * E;
  for (int i = t; i < 5 * E; i += kThreads) wcnt[i] = 0;
  __syncthreads();
  for (int g0 = 0; g0 < m; g0 += kThreads) {
    const int j = g0 + t;
    const bool valid = j < m;
    const int e = valid ? sel[j] : -1;
    int r = 0;
    uint64_t pending = __ballot(valid);
    while (pending) {
      const int leader = __builtin_ctzll(pending);
      const int el = __shfl(e, leader, 64);
      const uint64_t same = __ballot(valid && e == el);
      if (valid && e == el) r = __popcll(same & ((1ull << lane) - 1ull));
      if (lane == leader) wcnt[wave * E + el] = __popcll(same);
      pending &= ~same;
    }
    __syncthreads();
    if (valid) {
      int before = run[e];
      for (int w = 0; w < wave; ++w) before += wcnt[w * E + e];
      rank[a0 + j] = before + r;
    }
    __syncthreads();
    for (int x = t; x < E; x += kThreads) {
      run[x] += wcnt[x] + wcnt[E + x] + wcnt[2 * E + x] + wcnt[3 * E + x];
      wcnt[x] = wcnt[E + x] = wcnt[2 * E + x] = wcnt[3 * E + x] = 0;
    }
    __syncthreads();
  }
  for (int x = t; x < E; x += kThreads) counts_out[x] = run[x];
}

constexpr int kMaxSel = kTok * kRouterRankMaxK;  // assignments per workgroup when ranking

// The logits' way out, shared by both forms of the logits GEMM: lane holds,
// per expert block j of the wave, partial logits of experts
// 32 (g0 + gstep j) + 8 q + 4 hh + i for token l32 over part `part` of H.
// The parts meet in LDS (added in part order), then softmax and top-K, then
// (rank != nullptr) the routing stage's rank step over the block's chunk.
template <int RBW>
__device__ __forceinline__ void router_tail(const f32x16 (&acc)[RBW], float* slog, int* sel, int64_t t0, int32_t T,
                                            int32_t E, int32_t K, int32_t renorm, int32_t P, int part, int g0,
                                            int gstep, int wave, int lane, int32_t* __restrict__ idx,
                                            float* __restrict__ wts, int32_t* __restrict__ rank,
                                            int32_t* __restrict__ chunk_counts) {
  const int t = threadIdx.x, l32 = lane & 31, hh = lane >> 5;
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

  int* sl = rank ? sel : nullptr;
  switch ((E + 63) / 64) {
    case 1: softmax_topk_radix<1>(slog, t0, T, E, K, renorm, wave, lane, idx, wts, sl); break;
    case 2: softmax_topk_radix<2>(slog, t0, T, E, K, renorm, wave, lane, idx, wts, sl); break;
    case 3:
    case 4: softmax_topk<4>(slog, t0, T, E, K, renorm, wave, lane, idx, wts, sl); break;
    case 5:
    case 6:
    case 7:
    case 8: softmax_topk<8>(slog, t0, T, E, K, renorm, wave, lane, idx, wts, sl); break;
    default: softmax_topk<(MOEQ_MAX_EXPERTS + 63) / 64>(slog, t0, T, E, K, renorm, wave, lane, idx, wts, sl); break;
  }
  if (rank) {
    // the logits are no longer needed: their LDS holds the rank counters
    // (4 E + E ints <= kTok E floats)
    __syncthreads();
    const int ntok = (int)min<int64_t>(kTok, T - t0);
    chunk_rank(sel, ntok * K, E, reinterpret_cast<int*>(slog), t0 * K, rank, chunk_counts + (int64_t)blockIdx.x * E);
  }
}

// rank / chunk_counts: nullptr, or the routing stage's rank [T*K] and
// chunk_counts [ceil(T/16)][E] (chunks of 16 tokens x K assignments).
template <int RBW>  // expert blocks of 32 per wave
__global__ __launch_bounds__(kThreads) void router_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ gate, int32_t T, int32_t H,
                                                         int32_t E, int32_t K, int32_t renorm, int32_t P,
                                                         int32_t* __restrict__ idx, float* __restrict__ wts,
                                                         int32_t* __restrict__ rank,
                                                         int32_t* __restrict__ chunk_counts) {
  extern __shared__ float slog[];  // [P][kTok][E]: partial logits of the P parts of H
  __shared__ int sel[kMaxSel];
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
  router_tail<RBW>(acc, slog, sel, t0, T, E, K, renorm, P, part, g0, gstep, wave, lane, idx, wts, rank, chunk_counts);
}

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (global_load_lds_dwordx4, LDS base in M0), as inline assembly so that the
// compiler sees no LDS write to order against its own LDS reads: explicit
// waits before the barriers order the copies.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
               : "memory", "m0");
}

// The logits GEMM with its operands staged through LDS, for E <= 32 NRB with
// NRB expert blocks of 32 and P = 4 / NRB parts of H: wave w takes expert
// block w / P over part w % P.  Loaded straight into the MFMA layout, each
// 16-B lane load touches one cache line per row (32 per instruction); here
// every 64-k trip of the gate rows and the block's token rows is copied into
// LDS first, 8 whole 128-B row pieces per instruction, two trips ahead
// through three buffers, and the fragments are read from LDS.  Rows are stored with their 16-B chunks
// XOR-swizzled by (row / 2) % 8, so a fragment read (32 rows, one chunk)
// hits distinct banks.  The MFMAs, their operands and the logits' way out
// are those of router_kernel.
template <int NRB>
__global__ __launch_bounds__(kThreads) void router_staged_kernel(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ gate, int32_t T,
                                                                int32_t H, int32_t E, int32_t K, int32_t renorm,
                                                                int32_t* __restrict__ idx, float* __restrict__ wts,
                                                                int32_t* __restrict__ rank,
                                                                int32_t* __restrict__ chunk_counts) {
  constexpr int P = kWaves / NRB;                    // parts of H
  static_assert(NRB * P == kWaves, "one expert block and one part of H per wave");
  constexpr int kRows = 32 * NRB + kTok;             // staged rows per part: gate rows, then token rows
  constexpr int kPartBytes = kRows * 128;            // 64 k of each row
  constexpr int kBufBytes = P * kPartBytes;
  constexpr int kGroups = kRows / 8;                 // 8-row copies per part
  constexpr int kCopies = P * kGroups;               // per trip
  constexpr int kCopiesW = (kCopies + kWaves - 1) / kWaves;  // per wave (the last copy repeated to even out)
  extern __shared__ float slog[];  // [P][kTok][E]: partial logits of the P parts of H
  __shared__ int sel[kMaxSel];
  __shared__ __attribute__((aligned(16))) char ring[3 * kBufBytes];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int part = wave % P, g0 = wave / P;
  const int hlen = H / P;  // H % (64 P) == 0
  const int n64 = hlen / 64;
  auto swz = [](int r) { return (r >> 1) & 7; };

  // this wave's copies: copy d moves rows 8 (d % kGroups) .. +7 of part
  // d / kGroups; lane l takes row 8 (d % kGroups) + l / 8 and lands in its
  // LDS slot l % 8, which holds chunk (l % 8) ^ swz(row)
  const uint16_t* src[kCopiesW];
  uint32_t dst[kCopiesW];
#pragma unroll
  for (int c = 0; c < kCopiesW; ++c) {
    const int d = min(wave + kWaves * c, kCopies - 1);
    const int p = d / kGroups, g = d % kGroups, rr = 8 * g + (lane >> 3);
    const uint16_t* row;
    if (rr < 32 * NRB) {
      row = gate + (int64_t)(rr < E ? rr : 0) * H;  // rows past E: row 0 (its logits are never stored)
    } else {
      const int64_t tk = t0 + (rr - 32 * NRB);
      row = x + (tk < T ? tk : t0) * H;  // tokens past T: the block's first (never stored)
    }
    src[c] = row + p * hlen + 8 * ((lane & 7) ^ swz(rr));
    dst[c] = (uint32_t)(p * kPartBytes + g * 8 * 128);
  }
  uint32_t rlds = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)ring;
  asm volatile("" : "+s"(rlds));  // opaque, so it is not folded back into a pointer to the array
  auto stage = [&](int trip, int buf) {
#pragma unroll
    for (int c = 0; c < kCopiesW; ++c) lds_copy16(src[c] + 64 * trip, rlds + buf * kBufBytes + dst[c]);
  };

  f32x16 acc[1];
  acc[0] = (f32x16){};
  const int arow = 32 * g0 + l32, brow = 32 * NRB + (l32 & (kTok - 1));  // token columns 16..31 repeat 0..15
  stage(0, 0);
  if (n64 > 1) stage(1, 1);
  for (int i = 0; i < n64; ++i) {
    if (i + 2 < n64) {
      stage(i + 2, (i + 2) % 3);
      constexpr int kW = 2 * kCopiesW;
      __builtin_amdgcn_s_waitcnt((kW & 0xF) | ((kW >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    } else if (i + 1 < n64) {
      __builtin_amdgcn_s_waitcnt((kCopiesW & 0xF) | ((kCopiesW >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __builtin_amdgcn_s_barrier();  // every wave's copies of trip i have landed
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const char* base = ring + (i % 3) * kBufBytes + part * kPartBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 2 * u + hh;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(base + arow * 128 + 16 * (c ^ swz(arow)));
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(base + brow * 128 + 16 * (c ^ swz(brow)));
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[0], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt((0x3F & 0xF) | ((0x3F >> 4) << 14) | (0x7 << 4));  // this trip's LDS reads done
    __builtin_amdgcn_s_barrier();  // before trip i + 3 is copied over buffer i % 3
  }
  router_tail<1>(acc, slog, sel, t0, T, E, K, renorm, P, part, g0, kWaves, wave, lane, idx, wts, rank, chunk_counts);
}

}  // namespace

hipError_t launch_router(const uint16_t* x, const uint16_t* gate, int32_t T, int32_t H, int32_t E, int32_t K,
                         int32_t renorm, int32_t* idx, float* wts, int32_t* rank, int32_t* chunk_counts,
                         hipStream_t s) {
  const int grid = (T + kTok - 1) / kTok;
  const int nrb = (E + 31) / 32;  // expert blocks of 32
  // one, two or four expert blocks: operands staged through LDS (one block
  // and one part of H per wave)
  if ((nrb == 1 || nrb == 2 || nrb == 4) && H % (64 * (kWaves / nrb)) == 0) {
    const size_t lds_st = sizeof(float) * kTok * (size_t)E * (kWaves / nrb);
    if (nrb == 1)
      router_staged_kernel<1><<<grid, kThreads, lds_st, s>>>(x, gate, T, H, E, K, renorm, idx, wts, rank, chunk_counts);
    else if (nrb == 2)
      router_staged_kernel<2><<<grid, kThreads, lds_st, s>>>(x, gate, T, H, E, K, renorm, idx, wts, rank, chunk_counts);
    else
      router_staged_kernel<4><<<grid, kThreads, lds_st, s>>>(x, gate, T, H, E, K, renorm, idx, wts, rank, chunk_counts);
    return hipGetLastError();
  }
  // few expert blocks: split H across the waves instead (P parts, H % 64P == 0)
  int P = nrb >= kWaves ? 1 : (nrb >= 2 ? 2 : 4);
  while (P > 1 && H % (64 * P) != 0) P /= 2;
  const int rbw = (nrb * P + kWaves - 1) / kWaves;  // expert blocks per wave
  const size_t lds = sizeof(float) * kTok * (size_t)E * P;
  if (rbw <= 1)
    router_kernel<1><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts, rank, chunk_counts);
  else if (rbw <= 2)
    router_kernel<2><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts, rank, chunk_counts);
  else if (rbw <= 4)
    router_kernel<4><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts, rank, chunk_counts);
  else
    router_kernel<8><<<grid, kThreads, lds, s>>>(x, gate, T, H, E, K, renorm, P, idx, wts, rank, chunk_counts);
  return hipGetLastError();
}

}  // namespace moeq
