// Routed experts forward straight from packed NF4 / int8 storage (gfx950).
//
// out[t] = sum_k w[t,k] * down[e] @ (silu(gate[e] x_t) * up[e] x_t), e = idx[t,k]
// (bitsandbytes issue #1849, Description: gate_up_proj [E, 2I, H],
// down_proj [E, H, I], act_fn between them; unsloth-zoo issue #850,
// Suggested fix: the (hidden_states, top_k_index, top_k_weights) interface).
//
// Two paths, chosen by the number of assignments n = T*K:
//
// Tiled path (n > 512), after the routing stage has sorted the assignments
// by expert:
//   G1  grouped GEMM over tiles (expert, up to 256 sorted assignments, 128
//       columns of h): gathered bf16 rows of x times the gate and up weight
//       rows, fp32 accumulation on v_mfma_f32_32x32x16_bf16; the epilogue
//       pairs gate column j with up column j and writes h = bf16(silu(g) * u).
//   G2  the same machinery over (expert, up to 256 sorted rows, 256 output
//       columns): h times the down rows, scaled by the routing weight in fp32
//       -> y, rounded to bf16 (the model's compute dtype).
//   C1  out[t] = bf16(fp32 sum over k = 0..K-1, in that order, of y[slot[t*K+k]]).
//
// Few-assignment path (n <= 512, decode; decode.hip): no routing kernels and
// no token tiles; each workgroup finds its expert and that expert's
// assignments from top_k_index itself, streams weight codes straight from
// HBM into registers and splits K across its waves when few experts are
// touched.  h and y rows are indexed by assignment.
//
// This file holds the tiled path (G1, G2; the combine and the shared
// machinery are in experts_core.h) and the backward through the packed
// experts, which reuses G1 and G2.
//
// No float atomics anywhere: every output element has one writer and every
// sum has a fixed order, so the forward is bit-identical run to run, and a
// token's output does not depend on the other tokens of the batch within a
// path.  The two paths add the K products in different orders.
//
// Data flow inside a tiled-GEMM workgroup (4 waves):
//   * The token rows of the tile (x rows gathered through perm, or h rows)
//     stream through 2 or 3 LDS buffers (3 for tiles of at most 192 rows),
//     copied by the LDS DMA of global_load_lds one or two K steps ahead and
//     shared by the 4 waves: they are the MFMA B operand.  Rows are
//     XOR-swizzled by 16-B chunk so the fragment reads are conflict-free.
//   * Each wave owns its own weight rows (G1: 32 gate + the matching 32 up
//     rows; G2: 64 down rows).  It loads their packed codes straight into
//     registers one K step ahead and dequantizes them in registers into the
//     MFMA A operand -- the weights never touch LDS.  The dequantized value is
//     exactly bf16_rne(fp32(level * absmax)) / bf16_rne(fp32(q * scale)), the
//     same bits moeq_dequantize writes.  With double-quantized absmax the
//     lane loads the block's 8-bit absmax code and its group's scale instead
//     and forms fp32(code * scale) when the step is consumed (bitsandbytes
//     issue #1849, Reproduction and maintainer thread: double quantization).
//   * K is permuted inside each K step (the GEMM does not care which k each
//     MFMA lane slot holds, as long as both operands agree): lane half h of
//     every MFMA covers one whole 64-wide NF4 block of its row, so one absmax
//     and one 16-entry bf16 table serve the lane for the whole K step.  NF4
//     codes become bf16 through v_perm_b32 byte lookups in that table, in
//     natural k order within each group of 8.
//   * Work items (expert, column tile, token tile) are laid out expert-major
//     and dealt to the 8 XCDs in contiguous ranges, so the tiles that share an
//     expert's weights and token rows run on the same L2; within an expert the
//     token tiles go in groups of four, column tile by column tile, so the
//     items in flight on one XCD share four token tiles and a few weight
//     column tiles instead of re-reading every token tile per column tile.
#include "experts_core.h"

namespace moeq {
namespace {

// ---------------------------------------------------------------------------
// G1: h[p][j] = bf16(silu(gate_j . x) * (up_j . x)) for the tile's rows p.
// Wave w: h columns jcol = j0 + 32w .. +32 (gate rows jcol.., up rows I + jcol..).
// ---------------------------------------------------------------------------
template <int FMT, int NB>
__device__ __forceinline__ void g1_tile(char* sX, const uint16_t* x, const int32_t* prow, int K, int H, int I,
                                        int jcol, bool wave_on, const uint8_t* gq, const SRow<FMT>& gs,
                                        const uint8_t* uq, const SRow<FMT>& us, int row0, int nrows,
                                        uint16_t* __restrict__ h, float* __restrict__ gu_save) {
  using C = Core<FMT, NB>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t roff[C::kInstr];  // byte offset of each staged x row (token perm[p] / K)
#pragma unroll
  for (int i = 0; i < C::kInstr; ++i) {
    const int r = C::staged_row(wave, lane, i);
    roff[i] = (uint32_t)(prow[r < nrows ? r : 0] / K) * (uint32_t)H * 2u;
  }
  f32x16 accG[NB], accU[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    accG[b] = (f32x16){};
    accU[b] = (f32x16){};
  }
  C::run(sX, C::kBufBytes, reinterpret_cast<const char*>(x), roff, H, gq, gs, uq, us, wave_on, accG, accU);
  // lane holds, per token block b and register quad q, the four h columns
  // jcol + 8q + 4*hh + 0..3 of token row 32b + l32.
  // (h == nullptr: the backward's recompute, which keeps g and u instead)
  const int l32 = lane & 31, hh = lane >> 5;
  if (wave_on && h) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int r = 32 * b + l32;
      if (r >= nrows) continue;
      uint16_t* hp = h + (int64_t)(row0 + r) * I + jcol + 4 * hh;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float g = accG[b][4 * q + i], u = accU[b][4 * q + i];
          v[i] = g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
        }
        *reinterpret_cast<uint2*>(hp + 8 * q) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
  if (gu_save) {
    // The backward keeps g and u of every sorted row ([n][2I] fp32), staged
    // through LDS (the token buffers, free once the last DMAs have landed) so
    // that the global stores write whole rows: first g, then u.  Every wave
    // takes part in the barriers.
    constexpr int kPitch = 4 * kG1Cols + 16;
    static_assert(32 * NB * kPitch <= Lds<FMT>::kG2, "g tile fits the LDS array");
    const int j0 = jcol - 32 * wave;
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      __syncthreads();
      if (wave_on) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const f32x16& a = part ? accU[b] : accG[b];
          char* rowp = sX + (32 * b + l32) * kPitch + 4 * (32 * wave + 4 * hh);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(rowp + 4 * 8 * q) = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
      }
      __syncthreads();
      copy_rows<float, kBM, 4 * kG1Cols / 16, kPitch>(sX, nrows, I - j0, gu_save + (int64_t)row0 * 2 * I + part * I + j0,
                                                      2 * I);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void g1_kernel(const uint16_t* __restrict__ x, int32_t K, int32_t E,
                                                     int32_t H, int32_t I, const uint8_t* __restrict__ wq,
                                                     const float* __restrict__ ws, const uint8_t* __restrict__ wsc,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ tile_start,
                                                     const int32_t* __restrict__ perm_idx,
                                                     uint16_t* __restrict__ h, float* __restrict__ gu_save) {
  __shared__ __attribute__((aligned(16))) char sX[Lds<FMT>::kG2];

  int e, mt, ct;
  if (!decode_work(tile_start, E, (I + kG1Cols - 1) / kG1Cols, e, mt, ct)) return;
  int row0, nrows;
  tile_rows(offsets, tile_start, e, mt, &row0, &nrows);
  const int wave = threadIdx.x >> 6, l32 = threadIdx.x & 31;

  const int jcol = ct * kG1Cols + 32 * wave;
  const bool wave_on = jcol < I;  // I % 32 == 0
  // (a wave past the last column streams the expert's first rows, unused)
  const int grow = (wave_on ? jcol : 0) + l32, urow = grow + I;  // rows within the expert
  const int cpr = kNf4Codes<FMT> ? H / 2 : H;                     // code bytes per row

  const uint8_t* gq = wq + ((int64_t)e * 2 * I + grow) * cpr;
  const uint8_t* uq = wq + ((int64_t)e * 2 * I + urow) * cpr;
  const SRow<FMT> gs = srow_at<FMT>(ws, wsc, e, 2 * I, grow, H, 0);
  const SRow<FMT> us = srow_at<FMT>(ws, wsc, e, 2 * I, urow, H, 0);
  const int32_t* prow = perm_idx + row0;
  if (nrows > 192)
    g1_tile<FMT, 8>(sX, x, prow, K, H, I, jcol, wave_on, gq, gs, uq, us, row0, nrows, h, gu_save);
  else if (nrows > 128)
    g1_tile<FMT, 6>(sX, x, prow, K, H, I, jcol, wave_on, gq, gs, uq, us, row0, nrows, h, gu_save);
  else if (nrows > 64)
    g1_tile<FMT, 4>(sX, x, prow, K, H, I, jcol, wave_on, gq, gs, uq, us, row0, nrows, h, gu_save);
  else
    g1_tile<FMT, 2>(sX, x, prow, K, H, I, jcol, wave_on, gq, gs, uq, us, row0, nrows, h, gu_save);
}

// ---------------------------------------------------------------------------
// G2: y[p][n] = w_p * (down_n . h_p) in fp32.  Wave w: output columns
// ncol = n0 + 64w .. +64 (two 32-row MFMA blocks).
// ---------------------------------------------------------------------------
template <int FMT, int NB>
__device__ __forceinline__ void g2_tile(char* sX, const float* sw, const uint16_t* h, int H, int I, int ncol,
                                        bool on, const uint8_t* q0, const SRow<FMT>& s0, const uint8_t* q1,
                                        const SRow<FMT>& s1, int row0, int nrows, uint16_t* __restrict__ y) {
  using C = Core<FMT, NB>;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t roff[C::kInstr];  // byte offset of each staged h row (relative to the tile's first row)
#pragma unroll
  for (int i = 0; i < C::kInstr; ++i) {
    const int r = C::staged_row(wave, lane, i);
    roff[i] = (uint32_t)(r < nrows ? r : 0) * (uint32_t)I * 2u;
  }
  f32x16 acc0[NB], acc1[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    acc0[b] = (f32x16){};
    acc1[b] = (f32x16){};
  }
  C::run(sX, C::kBufBytes, reinterpret_cast<const char*>(h + (int64_t)row0 * I), roff, I, q0, s0, q1, s1, on,
         acc0, acc1);
  const int l32 = lane & 31, hh = lane >> 5;
  // bf16 y through LDS, so that global stores write whole rows (a direct
  // store from the MFMA layout touches 32 rows per instruction)
  constexpr int kPitch = 2 * kG2Rows + 16;  // bytes per staged row (16-B aligned, 8-B writes 2-way at most)
  static_assert(32 * NB * kPitch <= Lds<FMT>::kG2, "y tile fits the LDS array");
  __builtin_amdgcn_s_waitcnt(0);  // token DMAs of the extra prefetched step may still be landing
  __syncthreads();
  if (on) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float wr = sw[32 * b + l32];
      char* rowp = sX + (32 * b + l32) * kPitch + 2 * (64 * wave + 4 * hh);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const f32x16& a = m ? acc1[b] : acc0[b];
          *reinterpret_cast<uint2*>(rowp + 2 * (32 * m + 8 * q)) =
              make_uint2(pack_bf16x2(a[4 * q] * wr, a[4 * q + 1] * wr), pack_bf16x2(a[4 * q + 2] * wr, a[4 * q + 3] * wr));
        }
      }
    }
  }
  __syncthreads();
  const int n0 = ncol - 64 * wave;
  copy_rows<uint16_t, kBM, 2 * kG2Rows / 16, kPitch>(sX, nrows, H - n0, y + (int64_t)row0 * H + n0, H);
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void g2_kernel(const uint16_t* __restrict__ h, const float* __restrict__ wts,
                                                     int32_t E, int32_t H, int32_t I,
                                                     const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                                                     const uint8_t* __restrict__ wsc,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ tile_start,
                                                     const int32_t* __restrict__ perm_idx, uint16_t* __restrict__ y,
                                                     int32_t split) {
  __shared__ __attribute__((aligned(16))) char sX[Lds<FMT>::kG2];
  __shared__ float sw[kBM];

  // split: each token tile's rows in this many balanced parts, one work item
  // each (the parts of a column tile next to each other); an output element
  // is still summed by one wave in the same K order, so the bits do not
  // depend on the split
  int e, mt, ct2;
  if (!decode_work(tile_start, E, split * ((H + kG2Rows - 1) / kG2Rows), e, mt, ct2)) return;
  const int ct = ct2 / split, part = ct2 - ct * split;
  int row0, nrows;
  tile_rows(offsets, tile_start, e, mt, &row0, &nrows);
  {
    const int lo = nrows * part / split, hi = nrows * (part + 1) / split;
    row0 += lo;
    nrows = hi - lo;
  }
  if (nrows <= 0) return;  // a one-row tile's empty part (every wave leaves, before any barrier)
  const int t = threadIdx.x, wave = t >> 6, l32 = t & 31;
  if (t < kBM) sw[t] = (t < nrows) ? wts[perm_idx[row0 + t]] : 0.0f;

  const int ncol = ct * kG2Rows + 64 * wave;  // H % 64 == 0: a wave is all in or all out
  const bool on = ncol < H;
  const int r0 = (on ? ncol : 0) + l32, r1 = r0 + 32;  // rows within the expert
  const int cpr = kNf4Codes<FMT> ? I / 2 : I;

  const uint8_t* q0 = wq + ((int64_t)e * H + r0) * cpr;
  const uint8_t* q1 = wq + ((int64_t)e * H + r1) * cpr;
  const SRow<FMT> s0 = srow_at<FMT>(ws, wsc, e, H, r0, I, 0);
  const SRow<FMT> s1 = srow_at<FMT>(ws, wsc, e, H, r1, I, 0);
  if (nrows > 192)
    g2_tile<FMT, 8>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
  else if (nrows > 128)
    g2_tile<FMT, 6>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
  else if (nrows > 64)
    g2_tile<FMT, 4>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
  else
    g2_tile<FMT, 2>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
}

// ---------------------------------------------------------------------------
// Backward through the frozen packed experts (gradients with respect to the
// hidden states and the routing weights; see moeq_experts_backward):
//   recompute  g, u = G1 of the forward, kept in fp32 (h is not stored)
//   T1         v = down^T dout[t];  dh = w * v;  dg = dh u s (1 + g (1 - s)),
//              du = dh g s  -> dgu = bf16 [dg | du]                 (s = sigmoid(g))
//              and, per column tile, the share sum_c v_c h_c of
//              grad_w[a] = dout[t] . (down h) = v . h, with h = bf16(silu(g) u)
//              formed again from the saved g and u (the forward's bits)
//   BW         grad_w[a] = sum of T1's shares over the column tiles, in order
//   T2         dx = gate_up^T dgu  (fp32, one row per sorted assignment)
//   C1         grad_x[t] = bf16(sum over k in order of dx)
// T1 and T2 are transposed grouped GEMMs: the contraction runs over the rows
// of the packed weight while its NF4 blocks run along the output columns.
//
// tgemm_kernel: out[p][c] = sum_r W_e[r][c] v_p[r] for the tile (expert e, up
// to 256 sorted rows p, 128 output columns c), K steps of 64 weight rows.
// Each K step the workgroup
//   * dequantizes the W tile [64 r][128 c] into LDS in natural layout (every
//     thread: one row's 32 columns, which lie in one NF4 block), from codes
//     it loaded one step earlier;
//   * copies the token tile [256 rows][64 r] into LDS with the LDS DMA (rows
//     XOR-swizzled by 16-B chunk);
// and the MFMA A operand (W^T: 8 consecutive r of one column per lane) is read
// from the natural layout with ds_read_b64_tr_b16, which hands each lane of a
// 16-lane group one column of a 4 x 16 block of 16-bit values: lane L of the
// group points at row L / 4, columns 4 (L % 4) .. +3 of the block, and lane i
// receives column i of all four rows.
//   MODE 1: W = down_e (R = H rows, C = I columns); v_p = dout[perm[p] / K];
//           the epilogue forms dg and du from dh = w_p * acc and the saved g, u,
//           and the tile's share of grad_w, sum over its columns of acc * h.
//   MODE 2: W = gate_up_e (R = 2I, C = H); v_p = dgu[p]; out = dx fp32.
// Waves: wave w owns output columns 64 (w & 1) .. +64 (two 32-column MFMA
// blocks) of token rows 128 (w >> 1) .. +128 (four 32-row blocks).
// ---------------------------------------------------------------------------
constexpr int kTcols = 128;               // output columns per tile
constexpr int kTk = 64;                   // weight rows per K step
constexpr int kTpitch = 2 * kTcols + 32;  // LDS bytes per dequantized W row (padded)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <int FMT, int MODE>
__global__ __launch_bounds__(kThreads) void tgemm_kernel(const uint16_t* __restrict__ vsrc, int32_t Ktop, int32_t E,
                                                        int32_t R, int32_t C, const uint8_t* __restrict__ wq,
                                                        const float* __restrict__ ws,
                                                        const uint8_t* __restrict__ wsc,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ tile_start,
                                                        const int32_t* __restrict__ perm_idx,
                                                        const float* __restrict__ wts,
                                                        const float* __restrict__ gu_save, void* __restrict__ out,
                                                        float* __restrict__ gw_part) {
  // one LDS array: the dequantized W tiles, then the token tiles
  constexpr int kWBytes = kTk * kTpitch, kVBytes = kBM * kTk * 2;
  // (T2 also stages its fp32 output tile here: kBM rows of kTcols floats, padded)
  constexpr int kOutPitch = 4 * kTcols + 16;
  constexpr int kSmem = 2 * kWBytes + 2 * kVBytes > kBM * kOutPitch ? 2 * kWBytes + 2 * kVBytes : kBM * kOutPitch;
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  __shared__ float sw[kBM];
  auto sW = [&](int b) { return smem + b * kWBytes; };
  auto sV = [&](int b) { return smem + 2 * kWBytes + b * kVBytes; };

  int e, mt, ct;
  if (!decode_work(tile_start, E, (C + kTcols - 1) / kTcols, e, mt, ct)) return;
  int row0, nrows;
  tile_rows(offsets, tile_start, e, mt, &row0, &nrows);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int c0 = ct * kTcols;
  if (MODE == 1 && t < kBM) sw[t] = (t < nrows) ? wts[perm_idx[row0 + t]] : 0.0f;
  const int nks = R / kTk;  // R % 64 == 0

  // W tile loader: thread -> row wr of the step, columns wc .. wc + 31
  const int wr = t >> 2;
  const int wc = c0 + 32 * (t & 3);
  const bool wc_in = wc < C;  // C % 64 == 0: a 32-column quarter is wholly in or out
  const int wcc = wc_in ? wc : 0;
  const int64_t cpr = kNf4Codes<FMT> ? C / 2 : C;
  const int64_t spr = kNf4Codes<FMT> ? C / kNf4Block : 1;
  const uint8_t* wrow = wq + ((int64_t)e * R + wr) * cpr + (kNf4Codes<FMT> ? wcc / 2 : wcc);
  const SRow<FMT> srow = srow_at<FMT>(ws, wsc, e, R, wr, C, kNf4Codes<FMT> ? wcc / kNf4Block : 0);
  struct WCodes {
    uint4 a, b;  // NF4: a (32 codes); int8: a, b
    Scale<FMT> s;
    uint32_t m;  // all ones, or zero for a step or column quarter past the end
  };
  // code loads plus scale loads per step
  constexpr int kWLoads = (kNf4Codes<FMT> ? 1 : 2) + SRow<FMT>::kLoads;
  // Loads for step ks (past the last step: step 0's addresses).  They are
  // never behind a branch; a step or columns past the end are zeroed through
  // the scale when the codes are used (a zero scale makes the weights
  // exactly zero).
  auto wfetch = [&](WCodes& c, int ks) {
    const bool in = ks < nks;
    const int64_t kr = in ? (int64_t)ks * kTk : 0;
    const uint4* p = reinterpret_cast<const uint4*>(wrow + kr * cpr);
    c.a = p[0];
    if constexpr (!kNf4Codes<FMT>) c.b = p[1];
    c.s = srow.load(kr * spr);
    uint32_t m = (in && wc_in) ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(m));  // opaque: keeps the select from becoming a branch around the loads
    c.m = m;
  };
  // The dequantization of one step's W row quarter into LDS, cut into work
  // items of a few VALU instructions each so that a K step can slot one item
  // after each MFMA (the same arithmetic and bits as moeq_dequantize):
  //   NF4:  4 table stages, then per 8-column fragment f: 4 stages and its store;
  //   int8: the scale pair, then per fragment f: 2 stages and its store.
  struct WStage {
    float sc;
    Nf4Table tb;
    Nf4FragStages f4;
    FragStages<MOEQ_FMT_INT8_ROWWISE> f8;
    Dequant<MOEQ_FMT_INT8_ROWWISE> d8;
  };
  constexpr int kWItems = kNf4Codes<FMT> ? 4 + 4 * 5 : 1 + 4 * 3;
  auto witem = [&](int j, const WCodes& c, WStage& w, int buf) {
    char* dst = sW(buf) + wr * kTpitch + 64 * (t & 3);
    if constexpr (kNf4Codes<FMT>) {
      if (j < 4) {
        if (j == 0) w.sc = c.s.masked(c.m).value();
        float a = w.sc;
        pin_in(a);
        const uint32_t p0 = pack_bf16x2(__uint_as_float(kNf4LevelBits[4 * j]) * a,
                                        __uint_as_float(kNf4LevelBits[4 * j + 1]) * a);
        const uint32_t p1 = pack_bf16x2(__uint_as_float(kNf4LevelBits[4 * j + 2]) * a,
                                        __uint_as_float(kNf4LevelBits[4 * j + 3]) * a);
        w.tb.lo[j] = perm(p1, p0, 0x06040200u);
        w.tb.hi[j] = perm(p1, p0, 0x07050301u);
        pin_out(w.tb.lo[j]), pin_out(w.tb.hi[j]);
      } else {
        const int f = (j - 4) / 5, k = (j - 4) % 5;
        if (k < 4) {
          if (k == 0) w.f4.w = f == 0 ? c.a.x : (f == 1 ? c.a.y : (f == 2 ? c.a.z : c.a.w));
          w.f4.stage(k, w.tb);
        } else {
          *reinterpret_cast<bf16x8*>(dst + 16 * f) = w.f4.value();
        }
      }
    } else {
      if (j == 0) {
        w.d8.s = c.s.masked(c.m).value();
        w.d8.ns128 = -128.0f * w.d8.s;
      } else {
        const int f = (j - 1) / 3, k = (j - 1) % 3;
        if (k < 2) {
          if (k == 0) {
            const uint4& q = f < 2 ? c.a : c.b;
            w.f8.w[0] = (f & 1) ? q.z : q.x;
            w.f8.w[1] = (f & 1) ? q.w : q.y;
          }
          w.f8.stage(k, w.d8);
        } else {
          *reinterpret_cast<bf16x8*>(dst + 16 * f) = w.f8.value();
        }
      }
    }
  };
  auto wstore = [&](const WCodes& c, int buf) {
    WStage w;
#pragma unroll
    for (int j = 0; j < kWItems; ++j) witem(j, c, w, buf);
  };

  // token tile loader: instruction i of wave w stages rows 8 (4 i + w) .. +7,
  // lane l row 8 (4 i + w) + l / 8, LDS slot l % 8 holding chunk slot ^ ((row / 2) % 8)
  // (rows are 128 B: rows 2r and 2r + 1 lie in different bank halves, so 16
  // consecutive rows read at one chunk hit 16 distinct 16-B bank groups)
  uint32_t voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (4 * i + wave) + (lane >> 3);
    const int rr = r < nrows ? r : 0;
    voff[i] = (MODE == 1) ? (uint32_t)(perm_idx[row0 + rr] / Ktop) * (uint32_t)R * 2u
                          : (uint32_t)(row0 + rr) * (uint32_t)R * 2u;
  }
  const int vchunk = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);  // (row / 2) % 8 of the lane's rows
  const char* vbase = reinterpret_cast<const char*>(vsrc);
  // The DMA target is passed as a bare LDS address: with the array itself
  // the compiler would make every later LDS read wait for all DMAs in flight.
  // The explicit waits before each barrier order them instead.
  uint32_t vlds = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)sV(0);
  asm volatile("" : "+s"(vlds));  // opaque, so it is not folded back into a pointer to the array
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // the LDS target (M0) is scalar
  auto vstage_one = [&](int ks, int buf, int i) {
    const int kk = (ks < nks ? ks * kTk : 0) + 8 * vchunk;
    lds_dma16(vbase + voff[i] + 2 * kk, vlds + buf * kVBytes + (8 * (4 * i + wave_u)) * 128);
  };
  auto vstage = [&](int ks, int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) vstage_one(ks, buf, i);
  };

  // A operand addresses (ds_read_b64_tr_b16): lane L = lane % 16 of group
  // g = lane / 16 points at row 8 (g / 2) + L / 4 (+ 4 for the second read)
  // of the 16-row MFMA step, columns cb + 16 (g % 2) + 4 (L % 4)
  const int g16 = lane >> 4, L16 = lane & 15;
  const int a_off = (8 * (g16 >> 1) + (L16 >> 2)) * kTpitch + 2 * (16 * (g16 & 1) + 4 * (L16 & 3));
  const int cw = 64 * (wave & 1);    // wave's first tile column
  const int tw = 128 * (wave >> 1);  // wave's first tile row

  f32x16 acc[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[m][b] = (f32x16){};

  // Step ks: multiply step ks from buffer buf while staging step ks + 1 into
  // buffer buf ^ 1 (read last in step ks - 1, before the barrier that ended
  // it): after each of the 32 MFMAs one dequantization work item of the codes
  // loaded a step ago, one token DMA after each even MFMA of the first 16,
  // then the loads of step ks + 2's codes.  The code loads are the last loads
  // of the step, so the wait before the barrier can leave exactly them in
  // flight (every older load, the DMAs included, has landed).  The fragments
  // of each 16-row sub-step are read from LDS one sub-step ahead.  Two code
  // register sets in turn.
  constexpr int kSub = kTk / 16;          // MFMA sub-steps per step
  constexpr int kWSlots = kSub * 8;       // MFMAs per step (2 column blocks x 4 token blocks each)
  constexpr int kFetchSlot = 16;          // MFMA after which the next codes load
  static_assert(kWItems <= kWSlots && 2 * 7 < kFetchSlot, "step schedule");
  WCodes ca, cb;
  wfetch(ca, 0);
  vstage(0, 0);
  wstore(ca, 0);  // waits for the codes (and the DMA issued before them)
  wfetch(ca, 1);
  // as at the end of every step: only the codes just requested (used after
  // the first MFMA of step 0) stay in flight
  __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<kWLoads>);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  auto frags = [&](int buf, int s4, bf16x8 (&af)[2], bf16x8 (&bf)[4]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const char* base = sW(buf) + (16 * s4) * kTpitch + 2 * (cw + 32 * m) + a_off;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + 4 * kTpitch));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      af[m] = as_bf16x8(l2.x, l2.y, h2.x, h2.y);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = tw + 32 * b + l32;
      const int slot = (2 * s4 + hh) ^ ((row >> 1) & 7);
      bf[b] = *reinterpret_cast<const bf16x8*>(sV(buf) + row * 128 + slot * 16);
    }
  };
  auto kstep = [&](auto bufc, int ks, WCodes& cn, WCodes& cnn) {
    constexpr int buf = decltype(bufc)::value;
    __builtin_amdgcn_sched_barrier(0);
    WStage w;
    bf16x8 af[2][2], bf[2][4];
    frags(buf, 0, af[0], bf[0]);
#pragma unroll
    for (int s4 = 0; s4 < kSub; ++s4) {
      const int cur = s4 & 1;
      if (s4 + 1 < kSub) frags(buf, s4 + 1, af[cur ^ 1], bf[cur ^ 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = i >> 2, b = i & 3, slot = 8 * s4 + i;
        acc[m][b] = mfma(af[cur][m], bf[cur][b], acc[m][b]);
        if (slot < kWItems) witem(slot, cn, w, buf ^ 1);
        if ((slot & 1) == 0 && slot / 2 < 8) vstage_one(ks + 1, buf ^ 1, slot / 2);
        if (slot == kFetchSlot) wfetch(cnn, ks + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<kWLoads>);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  // two steps per trip with no branch between them; for an odd step count
  // the last trip's second step has zero weights and adds nothing
  for (int ks = 0; ks < nks; ks += 2) {
    kstep(std::integral_constant<int, 0>{}, ks, ca, cb);
    kstep(std::integral_constant<int, 1>{}, ks + 1, cb, ca);
  }

  // epilogue: lane holds, per column block m and token block b, output
  // columns cw + 32 m + 8 q + 4 hh + 0..3 of tile row tw + 32 b + l32
  if constexpr (MODE == 2) {
    // dx through LDS, so that the global stores write whole rows
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[m][b];
          *reinterpret_cast<float4*>(smem + (tw + 32 * b + l32) * kOutPitch + 4 * (cw + 32 * m + 8 * q + 4 * hh)) =
              make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
    __syncthreads();
    copy_rows<float, kBM, 4 * kTcols / 16, kOutPitch>(smem, nrows, C - c0, static_cast<float*>(out) + (int64_t)row0 * C + c0,
                                                      C);
    return;
  }
  if constexpr (MODE == 1) {
    // acc (= down^T dout, unweighted) through LDS, then row by row: a thread
    // takes 4 consecutive columns of a row, so the loads of the saved fp32 g
    // and u and the stores of bf16 dg and du cover whole rows (from the
    // accumulator layout each such load touched 32 rows).  Per element
    // dh = w * acc; the row's share of grad_w adds acc * h over the thread's
    // columns in order, then over the row's 32 lanes in a fixed tree.
    constexpr int kChunks = kTcols / 4;  // 4-column chunks of a tile row (a row: 32 lanes of one wave)
    static_assert(kChunks == 32, "one row per half wave");
    const int nct = (C + kTcols - 1) / kTcols;
    // The g and u loads go eight rows at a time, one group ahead: group 0
    // before the accumulators are staged, group i + 1 before group i is used
    // (a row or columns past the end load row 0 of the tile, column c0, and
    // are masked below).
    constexpr int kIters = kBM * kChunks / kThreads, kGroup = 8, kGroups = kIters / kGroup;
    static_assert(kIters % kGroup == 0, "whole groups");
    float4 g4[2][kGroup], u4[2][kGroup];
    auto gload = [&](int u0, float4 (&gg)[kGroup], float4 (&uu)[kGroup]) {
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const int i = threadIdx.x + (u0 + j) * kThreads, r = i / kChunks, c = c0 + 4 * (i - r * kChunks);
        const bool in = r < nrows && c < C;
        const float* gp = gu_save + (int64_t)(row0 + (in ? r : 0)) * 2 * C + (in ? c : c0);
        gg[j] = *reinterpret_cast<const float4*>(gp);
        uu[j] = *reinterpret_cast<const float4*>(gp + C);
      }
    };
    gload(0, g4[0], u4[0]);
    // The last K step ended in a barrier after every wave's fragment reads
    // and DMAs had completed, so the LDS array is free here.
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[m][b];
          *reinterpret_cast<float4*>(smem + (tw + 32 * b + l32) * kOutPitch + 4 * (cw + 32 * m + 8 * q + 4 * hh)) =
              make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
    __builtin_amdgcn_s_waitcnt(kVmcntLgkmWait<63>);  // this wave's LDS stores only
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      if (gi + 1 < kGroups) gload((gi + 1) * kGroup, g4[(gi + 1) & 1], u4[(gi + 1) & 1]);
#pragma unroll
      for (int j = 0; j < kGroup; ++j) {
        const int i = threadIdx.x + (gi * kGroup + j) * kThreads, r = i / kChunks, k4 = i - r * kChunks;
        const int c = c0 + 4 * k4;
        float share = 0.0f;
        if (r < nrows && c < C) {
          const int64_t p = row0 + r;
          const float w = sw[r];
          const float4 a4 = *reinterpret_cast<const float4*>(smem + r * kOutPitch + 16 * k4);
          const float4 gq = g4[gi & 1][j], uq = u4[gi & 1][j];
          const float av[4] = {a4.x, a4.y, a4.z, a4.w}, gv[4] = {gq.x, gq.y, gq.z, gq.w},
                      uv[4] = {uq.x, uq.y, uq.z, uq.w};
          float dg[4], du[4], hf[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[e]));
            const float dv = w * av[e];
            du[e] = dv * gv[e] * sg;
            dg[e] = dv * uv[e] * sg * (1.0f + gv[e] * (1.0f - sg));
            hf[e] = gv[e] * uv[e] * sg;  // the forward's h before rounding, same operations
          }
          const uint32_t h01 = pack_bf16x2(hf[0], hf[1]), h23 = pack_bf16x2(hf[2], hf[3]);
          const float hv[4] = {__uint_as_float(h01 << 16), __uint_as_float(h01 & 0xffff0000u),
                               __uint_as_float(h23 << 16), __uint_as_float(h23 & 0xffff0000u)};
#pragma unroll
          for (int e = 0; e < 4; ++e) share += av[e] * hv[e];
          uint16_t* o = static_cast<uint16_t*>(out) + p * 2 * C + c;
          *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *reinterpret_cast<uint2*>(o + C) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) share += __shfl_xor(share, o, 64);
        if (k4 == 0 && r < nrows) gw_part[(int64_t)(row0 + r) * nct + ct] = share;
      }
    }
    return;
  }
  static_assert(MODE == 1 || MODE == 2, "T1 or T2");
}

// grad_w[a] = sum over the column tiles ct = 0, 1, ... of T1's shares
// gw_part[slot[a]][ct] (0 for an unrouted assignment), one wave per
// assignment, lanes summed in a fixed tree order.
__global__ __launch_bounds__(kThreads) void gradw_kernel(const float* __restrict__ gw_part,
                                                        const int32_t* __restrict__ slot, int32_t n, int32_t nct,
                                                        float* __restrict__ gw) {
  const int64_t a = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (a >= n) return;
  const int lane = threadIdx.x & 63;
  const int p = slot[a];
  float acc = 0.0f;
  if (p >= 0)
    for (int j = lane; j < nct; j += 64) acc += gw_part[(int64_t)p * nct + j];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) gw[a] = acc;
}


}  // namespace

constexpr int kCUs = 256;  // compute units of an MI355X (8 XCDs x 32)

int32_t forward_tile_rows() { return kBM; }

int32_t backward_col_tiles(int32_t I) { return (I + kTcols - 1) / kTcols; }

template <int FMT>
hipError_t launch_tiled(const ForwardArgs& a, hipStream_t s, hipEvent_t const* ev) {
  const int32_t n = a.T * a.K;
  hipError_t err = a.routed ? launch_tile_start(a.rb.offsets, a.E, kBM, a.rb.tile_start, s)
                            : launch_route(a.idx, n, a.E, kBM, a.rb, s);
  if (err != hipSuccess) return err;
  if (ev) (void)hipEventRecord(ev[1], s);
  // upper bound on the number of token tiles: sum_e ceil(count_e / kBM)
  const int mtiles = (n + kBM - 1) / kBM + a.E;
  const int g1 = round_up(mtiles * ((a.I + kG1Cols - 1) / kG1Cols), kXcds);
  // The down GEMM has few work items when every expert holds one token tile
  // (prefill of a few hundred tokens over few, wide experts): at most one per
  // CU even at the upper bound on token tiles.  Its tiles' rows are then
  // split in two, so the chip fills (the same bits).
  const int g2cols = (a.H + kG2Rows - 1) / kG2Rows;
  const int g2split = mtiles * g2cols <= kCUs ? 2 : 1;
  const int g2 = round_up(mtiles * g2cols * g2split, kXcds);
  const uint8_t* guq = static_cast<const uint8_t*>(a.gu_q);
  const uint8_t* dnq = static_cast<const uint8_t*>(a.dn_q);
  g1_kernel<FMT><<<g1, kThreads, 0, s>>>(a.x, a.K, a.E, a.H, a.I, guq, a.gu_s, a.gu_c, a.rb.offsets,
                                         a.rb.tile_start, a.rb.perm, a.h, a.gu_save);
  if (ev) (void)hipEventRecord(ev[2], s);
  // y rows rounded to bf16 here (the fp32 workspace buffer holds them)
  uint16_t* y16 = reinterpret_cast<uint16_t*>(a.y);
  g2_kernel<FMT><<<g2, kThreads, 0, s>>>(a.h, a.wts, a.E, a.H, a.I, dnq, a.dn_s, a.dn_c, a.rb.offsets,
                                                   a.rb.tile_start, a.rb.perm, y16, g2split);
  if (ev) (void)hipEventRecord(ev[3], s);
  combine_kernel<uint16_t><<<a.T, kThreads, 0, s>>>(y16, a.rb.slot, a.K, a.H, a.out);
  if (ev) (void)hipEventRecord(ev[4], s);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t const* ev) {
  if (ev) (void)hipEventRecord(ev[0], s);
  return a.T * a.K <= kDecodeMax && !a.gu_save ? launch_experts_decode(a, s, ev) : launch_tiled<FMT>(a, s, ev);
}

template <int FMT>
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  const int32_t n = a.T * a.K;
  hipError_t err = launch_route(a.idx, n, a.E, kBM, a.rb, s);
  if (err != hipSuccess) return err;
  const int mtiles = (n + kBM - 1) / kBM + a.E;
  const int g1 = round_up(mtiles * ((a.I + kG1Cols - 1) / kG1Cols), kXcds);
  const int t1 = round_up(mtiles * ((a.I + kTcols - 1) / kTcols), kXcds);
  const int t2 = round_up(mtiles * ((a.H + kTcols - 1) / kTcols), kXcds);
  const uint8_t* guq = static_cast<const uint8_t*>(a.gu_q);
  const uint8_t* dnq = static_cast<const uint8_t*>(a.dn_q);
  const RouteBuffers& r = a.rb;
  if (a.recompute)
    g1_kernel<FMT><<<g1, kThreads, 0, s>>>(a.x, a.K, a.E, a.H, a.I, guq, a.gu_s, a.gu_c, r.offsets, r.tile_start,
                                           r.perm, nullptr, a.gu_save);
  tgemm_kernel<FMT, 1><<<t1, kThreads, 0, s>>>(a.dout, a.K, a.E, a.H, a.I, dnq, a.dn_s, a.dn_c, r.offsets,
                                               r.tile_start, r.perm, a.wts, a.gu_save, a.dgu, a.gw_part);
  gradw_kernel<<<(n + kWaves - 1) / kWaves, kThreads, 0, s>>>(a.gw_part, r.slot, n, backward_col_tiles(a.I),
                                                              a.grad_w);
  tgemm_kernel<FMT, 2><<<t2, kThreads, 0, s>>>(a.dgu, a.K, a.E, 2 * a.I, a.H, guq, a.gu_s, a.gu_c, r.offsets,
                                               r.tile_start, r.perm, nullptr, nullptr, a.dx, nullptr);
  combine_kernel<float><<<a.T, kThreads, 0, s>>>(a.dx, r.slot, a.K, a.H, a.grad_x);
  return hipGetLastError();
}

hipError_t launch_experts_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t const* ev) {
  switch (a.format) {
    case MOEQ_FMT_NF4: return launch_forward<MOEQ_FMT_NF4>(a, s, ev);
    case MOEQ_FMT_NF4_DQ: return launch_forward<MOEQ_FMT_NF4_DQ>(a, s, ev);
    default: return launch_forward<MOEQ_FMT_INT8_ROWWISE>(a, s, ev);
  }
}

hipError_t launch_experts_backward(const BackwardArgs& a, hipStream_t s) {
  switch (a.format) {
    case MOEQ_FMT_NF4: return launch_backward<MOEQ_FMT_NF4>(a, s);
    case MOEQ_FMT_NF4_DQ: return launch_backward<MOEQ_FMT_NF4_DQ>(a, s);
    default: return launch_backward<MOEQ_FMT_INT8_ROWWISE>(a, s);
  }
}

}  // namespace moeq
