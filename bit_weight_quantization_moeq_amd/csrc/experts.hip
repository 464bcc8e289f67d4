// Routed experts forward straight from packed NF4 / int8 storage (gfx950).
//
// out[t] = sum_k w[t,k] * down[e] @ (silu(gate[e] x_t) * up[e] x_t), e = idx[t,k]
// (bitsandbytes issue #1849, Description: gate_up_proj [E, 2I, H],
// down_proj [E, H, I], act_fn between them; unsloth-zoo issue #850,
// Suggested fix: the (hidden_states, top_k_index, top_k_weights) interface).
//
// After the routing stage has sorted the assignments by expert:
//   G1  grouped GEMM over tiles (expert, 128 sorted assignments, 64 columns of
//       h): the gathered bf16 rows of x times the gate and up weight rows,
//       dequantized tile by tile into LDS as bf16, on v_mfma_f32_32x32x16_bf16
//       with fp32 accumulation; the epilogue pairs gate column j with up
//       column j and writes h = bf16(silu(g) * u) in sorted order.
//   G2  the same machinery over (expert, 128 sorted rows, 128 columns of the
//       output): h times the dequantized down rows, scaled by the routing
//       weight in fp32, written as fp32 y in sorted order.
//   C1  out[t] = bf16(sum over k = 0..K-1, in that order, of y[slot[t*K+k]]).
// No float atomics anywhere: every output element has one writer, so the
// forward is bit-identical run to run.
//
// The weights are the MFMA A operand (rows of the weight on the 32 M lanes)
// and the token rows the B operand, so each lane's accumulators hold four
// consecutive output columns of one token row, stored as 8- or 16-byte writes.
#include "moeq_internal.h"

namespace moeq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBM = 128;        // sorted assignment rows per tile
constexpr int kBK = 64;         // K step (= one NF4 block)
constexpr int kG1Cols = 64;     // h columns per G1 tile (64 gate + 64 up weight rows)
constexpr int kG2Cols = 128;    // output columns per G2 tile
constexpr int kWRows = 128;     // weight rows staged per K step (both kernels)
constexpr int kLds = kBK + 8;   // LDS row pitch in bf16 (144 B: conflict-free 16-B reads)

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// ---------------------------------------------------------------------------
// Weight staging: 128 weight rows x 64 k per step.  Thread t owns row t/2 and
// the k half t%2 (32 elements): it fetches the packed bytes into registers
// for the next step while the MFMAs of this step run, then dequantizes them
// into LDS as bf16 exactly as moeq_dequantize would:
// bf16_rne(fp32(level * absmax)) or bf16_rne(fp32(q * scale)).
// ---------------------------------------------------------------------------
template <int FMT>
struct WeightStage;

template <>
struct WeightStage<MOEQ_FMT_NF4> {
  uint4 codes;   // 32 codes (16 B)
  float scale;   // absmax of the row's 64-block
  bool valid;

  // row: weight row index within the expert tensor (rows x cols), k0: K offset
  __device__ __forceinline__ void fetch(const uint8_t* q, const float* s, int64_t row_global, int cols,
                                        int k0, int half, bool ok) {
    valid = ok;
    if (ok) {
      codes = *reinterpret_cast<const uint4*>(q + (row_global * cols + k0 + 32 * half) / 2);
      scale = s[row_global * (cols / kNf4Block) + k0 / kNf4Block];
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, const float* lv) const {
    uint4 out[4];
    if (valid) {
      const uint32_t w[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t byte = (w[i] >> (8 * m)) & 0xffu;
          o[m] = pack_bf16x2(lv[byte >> 4] * scale, lv[byte & 0xfu] * scale);
        }
        out[i] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(dst)[i] = out[i];
  }
};

template <>
struct WeightStage<MOEQ_FMT_INT8_ROWWISE> {
  uint4 q0, q1;  // 32 int8 codes
  float scale;
  bool valid;

  __device__ __forceinline__ void fetch(const uint8_t* q, const float* s, int64_t row_global, int cols,
                                        int k0, int half, bool ok) {
    valid = ok;
    if (ok) {
      const uint4* p = reinterpret_cast<const uint4*>(q + row_global * cols + k0 + 32 * half);
      q0 = p[0];
      q1 = p[1];
      scale = s[row_global];
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, const float*) const {
    uint4 out[4];
    if (valid) {
      const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t o[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t d = w[2 * i + m / 2];
          const int sh = 16 * (m & 1);
          const float f0 = (float)(int8_t)((d >> sh) & 0xffu) * scale;
          const float f1 = (float)(int8_t)((d >> (sh + 8)) & 0xffu) * scale;
          o[m] = pack_bf16x2(f0, f1);
        }
        out[i] = make_uint4(o[0], o[1], o[2], o[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(dst)[i] = out[i];
  }
};

// Token rows: 128 rows x 64 k of bf16 per step; thread t owns row t/2, half t%2.
struct RowStage {
  uint4 v[4];
  __device__ __forceinline__ void fetch(const uint16_t* rowp, int k0, int half) {
    if (rowp) {
      const uint4* p = reinterpret_cast<const uint4*>(rowp + k0 + 32 * half);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<uint4*>(dst)[i] = v[i];
  }
};

// Expert of grouped-GEMM tile `tile` (tile_start is the exclusive prefix of
// per-expert tile counts); -1 past the last tile.
__device__ __forceinline__ int tile_expert(const int32_t* tile_start, int E, int tile) {
  if (tile >= tile_start[E]) return -1;
  int lo = 0, hi = E - 1;  // largest e with tile_start[e] <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base) {
  return *reinterpret_cast<const bf16x8*>(base);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// G1: h[p][j] = bf16(silu(gate_j . x) * (up_j . x)) for the tile's rows p.
// Wave w: h columns 32*(w&1) .. +32 (gate and up), rows 64*(w>>1) .. +64.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(kThreads) void g1_kernel(const uint16_t* __restrict__ x, int32_t K, int32_t E,
                                                     int32_t H, int32_t I, const uint8_t* __restrict__ wq,
                                                     const float* __restrict__ ws,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ tile_start,
                                                     const int32_t* __restrict__ perm,
                                                     uint16_t* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[kWRows * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sX[kBM * kLds];
  __shared__ float lv[16];

  const int e = tile_expert(tile_start, E, blockIdx.x);
  if (e < 0) return;
  const int row0 = offsets[e] + (blockIdx.x - tile_start[e]) * kBM;
  const int nrows = min(kBM, offsets[e + 1] - row0);
  const int j0 = blockIdx.y * kG1Cols;

  if (threadIdx.x < 16) lv[threadIdx.x] = __uint_as_float(kNf4LevelBits[threadIdx.x]);

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // staging roles
  const int srow = t >> 1, half = t & 1;
  const int64_t wrow = (int64_t)e * 2 * I + (srow < kG1Cols ? j0 + srow : I + j0 + (srow - kG1Cols));
  const uint16_t* xrow = (srow < nrows) ? x + (int64_t)(perm[row0 + srow] / K) * H : nullptr;

  WeightStage<FMT> wst;
  RowStage xst;
  wst.fetch(wq, ws, wrow, H, 0, half, true);
  xst.fetch(xrow, 0, half);

  f32x16 acc[2][2];  // [gate/up][token block]
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[g][b] = (f32x16){};

  const int wj = wave & 1, wi = wave >> 1;
  const int l32 = lane & 31, khi = 8 * (lane >> 5);
  const uint16_t* aG = sW + (32 * wj + l32) * kLds + khi;
  const uint16_t* aU = sW + (kG1Cols + 32 * wj + l32) * kLds + khi;
  const uint16_t* b0 = sX + (64 * wi + l32) * kLds + khi;
  const uint16_t* b1 = sX + (64 * wi + 32 + l32) * kLds + khi;

  const int nks = H / kBK;
  for (int ks = 0; ks < nks; ++ks) {
    __syncthreads();
    wst.store(sW + srow * kLds + 32 * half, lv);
    xst.store(sX + srow * kLds + 32 * half);
    __syncthreads();
    if (ks + 1 < nks) {
      wst.fetch(wq, ws, wrow, H, (ks + 1) * kBK, half, true);
      xst.fetch(xrow, (ks + 1) * kBK, half);
    }
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const bf16x8 ag = lds_frag(aG + 16 * s), au = lds_frag(aU + 16 * s);
      const bf16x8 x0 = lds_frag(b0 + 16 * s), x1 = lds_frag(b1 + 16 * s);
      acc[0][0] = mfma(ag, x0, acc[0][0]);
      acc[0][1] = mfma(ag, x1, acc[0][1]);
      acc[1][0] = mfma(au, x0, acc[1][0]);
      acc[1][1] = mfma(au, x1, acc[1][1]);
    }
  }

  // epilogue: lane holds, per token block b and register quad q, the four
  // h columns 8q + 4*(lane/32) + 0..3 of token row l32.
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int r = 64 * wi + 32 * b + l32;
    if (r >= nrows) continue;
    uint16_t* hp = h + (int64_t)(row0 + r) * I + j0 + 32 * wj + 4 * (lane >> 5);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float g = acc[0][b][4 * q + i], u = acc[1][b][4 * q + i];
        v[i] = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
      }
      *reinterpret_cast<uint2*>(hp + 8 * q) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
  }
}

// ---------------------------------------------------------------------------
// G2: y[p][n] = w_p * (down_n . h_p) in fp32 for the tile's rows p.
// Wave w: output columns 64*(w&1) .. +64, rows 64*(w>>1) .. +64.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(kThreads) void g2_kernel(const uint16_t* __restrict__ h, const float* __restrict__ wts,
                                                     int32_t E, int32_t H, int32_t I,
                                                     const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ tile_start,
                                                     const int32_t* __restrict__ perm, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t sW[kWRows * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t sX[kBM * kLds];
  __shared__ float lv[16];
  __shared__ float sw[kBM];

  const int e = tile_expert(tile_start, E, blockIdx.x);
  if (e < 0) return;
  const int row0 = offsets[e] + (blockIdx.x - tile_start[e]) * kBM;
  const int nrows = min(kBM, offsets[e + 1] - row0);
  const int n0 = blockIdx.y * kG2Cols;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (t < 16) lv[t] = __uint_as_float(kNf4LevelBits[t]);
  if (t < kBM) sw[t] = (t < nrows) ? wts[perm[row0 + t]] : 0.0f;

  const int srow = t >> 1, half = t & 1;
  const bool wok = (n0 + srow) < H;
  const int64_t wrow = (int64_t)e * H + (wok ? n0 + srow : 0);
  const uint16_t* hrow = (srow < nrows) ? h + (int64_t)(row0 + srow) * I : nullptr;

  WeightStage<FMT> wst;
  RowStage hst;
  wst.fetch(wq, ws, wrow, I, 0, half, wok);
  hst.fetch(hrow, 0, half);

  f32x16 acc[2][2];  // [column block][token block]
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[g][b] = (f32x16){};

  const int wn = wave & 1, wi = wave >> 1;
  const int l32 = lane & 31, khi = 8 * (lane >> 5);
  const uint16_t* a0 = sW + (64 * wn + l32) * kLds + khi;
  const uint16_t* a1 = sW + (64 * wn + 32 + l32) * kLds + khi;
  const uint16_t* b0 = sX + (64 * wi + l32) * kLds + khi;
  const uint16_t* b1 = sX + (64 * wi + 32 + l32) * kLds + khi;

  const int nks = I / kBK;
  for (int ks = 0; ks < nks; ++ks) {
    __syncthreads();
    wst.store(sW + srow * kLds + 32 * half, lv);
    hst.store(sX + srow * kLds + 32 * half);
    __syncthreads();
    if (ks + 1 < nks) {
      wst.fetch(wq, ws, wrow, I, (ks + 1) * kBK, half, wok);
      hst.fetch(hrow, (ks + 1) * kBK, half);
    }
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const bf16x8 w0 = lds_frag(a0 + 16 * s), w1 = lds_frag(a1 + 16 * s);
      const bf16x8 x0 = lds_frag(b0 + 16 * s), x1 = lds_frag(b1 + 16 * s);
      acc[0][0] = mfma(w0, x0, acc[0][0]);
      acc[0][1] = mfma(w0, x1, acc[0][1]);
      acc[1][0] = mfma(w1, x0, acc[1][0]);
      acc[1][1] = mfma(w1, x1, acc[1][1]);
    }
  }

#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int r = 64 * wi + 32 * b + l32;
    if (r >= nrows) continue;
    const float wr = sw[r];
    float* yp = y + (int64_t)(row0 + r) * H;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 64 * wn + 32 * c + 8 * q + 4 * (lane >> 5);
        if (n < H) {
          *reinterpret_cast<float4*>(yp + n) =
              make_float4(acc[c][b][4 * q] * wr, acc[c][b][4 * q + 1] * wr, acc[c][b][4 * q + 2] * wr,
                          acc[c][b][4 * q + 3] * wr);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// C1: out[t] = bf16(y[slot[t*K]] + y[slot[t*K+1]] + ... ) in k order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ slot,
                                                          int32_t K, int32_t H, uint16_t* __restrict__ out) {
  const int64_t tok = blockIdx.x;
  const int32_t* sl = slot + tok * K;
  for (int n4 = threadIdx.x; n4 < H / 4; n4 += kThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k) {
      const int p = sl[k];
      if (p < 0) continue;
      const float4 v = *reinterpret_cast<const float4*>(y + (int64_t)p * H + 4 * n4);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<uint2*>(out + tok * H + 4 * n4) =
        make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

}  // namespace

int32_t forward_tile_rows() { return kBM; }

hipError_t launch_experts_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t const* ev) {
  const int32_t n = a.T * a.K;
  if (ev) hipEventRecord(ev[0], s);
  hipError_t err = launch_route(a.idx, n, a.E, kBM, a.rb, s);
  if (err != hipSuccess) return err;
  if (ev) hipEventRecord(ev[1], s);
  const int mtiles = (n + kBM - 1) / kBM + a.E;  // upper bound on sum_e ceil(count_e / kBM)
  const dim3 g1(mtiles, a.I / kG1Cols), g2(mtiles, (a.H + kG2Cols - 1) / kG2Cols);
  const uint8_t* guq = static_cast<const uint8_t*>(a.gu_q);
  const uint8_t* dnq = static_cast<const uint8_t*>(a.dn_q);
  if (a.format == MOEQ_FMT_NF4) {
    g1_kernel<MOEQ_FMT_NF4><<<g1, kThreads, 0, s>>>(a.x, a.K, a.E, a.H, a.I, guq, a.gu_s, a.rb.offsets,
                                                    a.rb.tile_start, a.rb.perm, a.h);
    if (ev) hipEventRecord(ev[2], s);
    g2_kernel<MOEQ_FMT_NF4><<<g2, kThreads, 0, s>>>(a.h, a.wts, a.E, a.H, a.I, dnq, a.dn_s, a.rb.offsets,
                                                    a.rb.tile_start, a.rb.perm, a.y);
  } else {
    g1_kernel<MOEQ_FMT_INT8_ROWWISE><<<g1, kThreads, 0, s>>>(a.x, a.K, a.E, a.H, a.I, guq, a.gu_s,
                                                             a.rb.offsets, a.rb.tile_start, a.rb.perm, a.h);
    if (ev) hipEventRecord(ev[2], s);
    g2_kernel<MOEQ_FMT_INT8_ROWWISE><<<g2, kThreads, 0, s>>>(a.h, a.wts, a.E, a.H, a.I, dnq, a.dn_s,
                                                             a.rb.offsets, a.rb.tile_start, a.rb.perm, a.y);
  }
  if (ev) hipEventRecord(ev[3], s);
  combine_kernel<<<a.T, kThreads, 0, s>>>(a.y, a.rb.slot, a.K, a.H, a.out);
  if (ev) hipEventRecord(ev[4], s);
  return hipGetLastError();
}

}  // namespace moeq
