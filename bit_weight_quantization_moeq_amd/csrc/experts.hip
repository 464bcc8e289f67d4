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
// Few-assignment path (n <= 512, decode): no routing kernels and no token
// tiles; each workgroup finds its expert and that expert's assignments from
// top_k_index itself, streams weight codes straight from HBM into registers
// and splits K across its waves when few experts are touched (see
// decode_kernel).  h and y rows are indexed by assignment.
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
#include <type_traits>

#include "moeq_internal.h"

namespace moeq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 256;             // sorted assignment rows per tile (at most)
constexpr int kG1Cols = 32 * kWaves; // h columns per G1 tile (each wave: 32 gate + 32 up rows)
constexpr int kG2Rows = 64 * kWaves; // output columns per G2 tile (each wave: 64 down rows)
constexpr int kXcds = 8;

// s_waitcnt immediate that waits until at most N vector-memory loads are
// outstanding and leaves the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
constexpr int kVmcntWait = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
// ... and also until every LDS access of this wave has completed.
template <int N>
constexpr int kVmcntLgkmWait = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4);

template <int FMT>
struct Fmt;
template <>
struct Fmt<MOEQ_FMT_NF4> {
  static constexpr int kStep = 128;  // two NF4 blocks: one per MFMA lane half
};
template <>
struct Fmt<MOEQ_FMT_INT8_ROWWISE> {
  static constexpr int kStep = 64;
};
template <>
struct Fmt<MOEQ_FMT_NF4_DQ> : Fmt<MOEQ_FMT_NF4> {};

// NF4 codes (plain or with double-quantized absmax): 4-bit codes, 64-blocks.
template <int FMT>
constexpr bool kNf4Codes = FMT == MOEQ_FMT_NF4 || FMT == MOEQ_FMT_NF4_DQ;

// One scale as loaded: NF4 / int8 hold the fp32 scale itself; with
// double-quantized absmax, the absmax code and its group's scale, multiplied
// only when the scale is used (after the loads have landed):
// absmax' = fp32(code * group_scale).
template <int FMT>
struct Scale {
  float s;
  __device__ __forceinline__ float value() const { return s; }
  __device__ __forceinline__ Scale masked(uint32_t m) const { return {__uint_as_float(__float_as_uint(s) & m)}; }
  __device__ __forceinline__ Scale or_zero(bool in) const { return {in ? s : 0.0f}; }
};
template <>
struct Scale<MOEQ_FMT_NF4_DQ> {
  uint32_t c;
  float g;
  __device__ __forceinline__ float value() const { return (float)c * g; }
  __device__ __forceinline__ Scale masked(uint32_t m) const { return {c, __uint_as_float(__float_as_uint(g) & m)}; }
  __device__ __forceinline__ Scale or_zero(bool in) const { return {c, in ? g : 0.0f}; }
};

// Where one weight row's scales live.  load(boff): the scale of block boff
// counted from the row's first block (int8: the row scale, boff rows on).
template <int FMT>
struct SRow {
  const float* p;
  static constexpr int kLoads = 1;
  __device__ __forceinline__ Scale<FMT> load(int64_t boff) const { return {p[boff]}; }
};
// Double-quantized absmax: the row's absmax codes, its expert's group scales
// and the row's first block within the expert (groups of 256 blocks of one
// expert).
template <>
struct SRow<MOEQ_FMT_NF4_DQ> {
  const uint8_t* c;
  const float* g;
  int64_t b0;
  static constexpr int kLoads = 2;
  __device__ __forceinline__ Scale<MOEQ_FMT_NF4_DQ> load(int64_t boff) const {
    return {(uint32_t)c[boff], g[(b0 + boff) >> kDqGroupShift]};
  }
};

// Scales of row `row` of expert e, from column block kb0 on, in a tensor of R
// rows per expert and K columns.  ws: fp32 scales (NF4, int8) or group
// scales (double-quantized); wc: absmax codes (double-quantized only).
template <int FMT>
__device__ __forceinline__ SRow<FMT> srow_at(const float* ws, const uint8_t* wc, int e, int R, int row, int K,
                                             int kb0) {
  if constexpr (FMT == MOEQ_FMT_NF4_DQ) {
    const int64_t spr = K / kNf4Block, nb = (int64_t)R * spr;
    return {wc + (int64_t)e * nb + row * spr + kb0, ws + (int64_t)e * dq_groups(nb), row * spr + kb0};
  } else if constexpr (FMT == MOEQ_FMT_NF4) {
    return {ws + ((int64_t)e * R + row) * (K / kNf4Block) + kb0};
  } else {
    return {ws + (int64_t)e * R + row};
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> two bf16 (round to nearest even), lo in the low half: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Anchors for hand-placed VALU work: pin_in makes x look redefined here
// and pin_out makes it look used here (both emit nothing).  Work between a
// stage's pin_in of its inputs and pin_out of its results stays between the
// two points, in program order with the fences around it.
__device__ __forceinline__ void pin_in(uint32_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_in(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin_out(uint32_t x) { asm volatile("" ::"v"(x)); }

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (global_load_lds_dwordx4 with the LDS base in M0).  Written as inline
// assembly so that the compiler does not see an LDS write it cannot order:
// with the builtin it waits for every LDS access in flight (lgkmcnt(0)) at
// each later LDS use, which would also wait for fragment reads issued ahead
// of time.  The caller orders the copy with explicit vmcnt waits before a
// barrier.  The DMA reads M0 one wait state after it is written.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(src)
               : "memory", "m0");
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// NF4 dequantization in registers.
// ---------------------------------------------------------------------------
// Byte tables of the 16 dequantized values of one (row, 64-block):
// T_i = bf16_rne(fp32(level_i * absmax)); lo[q] holds the low bytes of
// T_{4q..4q+3}, hi[q] the high bytes.
struct Nf4Table {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ Nf4Table nf4_table(float a) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    p[j] = pack_bf16x2(__uint_as_float(kNf4LevelBits[2 * j]) * a, __uint_as_float(kNf4LevelBits[2 * j + 1]) * a);
  Nf4Table t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.lo[q] = perm(p[2 * q + 1], p[2 * q], 0x06040200u);
    t.hi[q] = perm(p[2 * q + 1], p[2 * q], 0x07050301u);
  }
  return t;
}

// One dword of packed codes (8 consecutive k; byte m holds k = 2m in its high
// nibble and k = 2m + 1 in its low nibble) -> the A operand [k0 .. k7].
__device__ __forceinline__ bf16x8 nf4_frag(const Nf4Table& t, uint32_t w) {
  // v_perm selectors 8..11 replicate the sign bit of pool bytes 1, 3, 5, 7:
  // with pool {w, w << 8} they give 0xff exactly where a byte of w has bit 7
  // set, i.e. where the high-nibble code is >= 8; shifting w by 4 first does
  // the same for the low-nibble codes.
  const uint32_t me = perm(w, w << 8, 0x0B090A08u);
  const uint32_t mo = perm(w << 4, w << 12, 0x0B090A08u);
  const uint32_t se = (w >> 4) & 0x07070707u, so = w & 0x07070707u;
  // low / high bytes of the values of the even-k codes (k0 k2 k4 k6) and of the
  // odd-k codes (k1 k3 k5 k7)
  const uint32_t le = (me & perm(t.lo[3], t.lo[2], se)) | (~me & perm(t.lo[1], t.lo[0], se));
  const uint32_t he = (me & perm(t.hi[3], t.hi[2], se)) | (~me & perm(t.hi[1], t.hi[0], se));
  const uint32_t lo = (mo & perm(t.lo[3], t.lo[2], so)) | (~mo & perm(t.lo[1], t.lo[0], so));
  const uint32_t ho = (mo & perm(t.hi[3], t.hi[2], so)) | (~mo & perm(t.hi[1], t.hi[0], so));
  // interleave back to k order: low bytes of k0..k3, high bytes of k0..k3, ...
  const uint32_t l03 = perm(lo, le, 0x05010400u), h03 = perm(ho, he, 0x05010400u);
  const uint32_t l47 = perm(lo, le, 0x07030602u), h47 = perm(ho, he, 0x07030602u);
  return as_bf16x8(perm(h03, l03, 0x05010400u), perm(h03, l03, 0x07030602u), perm(h47, l47, 0x05010400u),
                   perm(h47, l47, 0x07030602u));
}

// nf4_frag in four stages of 6 to 8 VALU instructions, so that a GEMM can
// slot one stage between two MFMAs (an MFMA runs for 32 cycles while the
// same wave keeps issuing independent VALU work).  Same arithmetic, same bits.
struct Nf4FragStages {
  static constexpr int kStages = 4;
  uint32_t w, me, mo, se, so, le, he, lo, ho, r[4];
  __device__ __forceinline__ void stage(int k, const Nf4Table& t) {
    if (k == 0) {
      pin_in(w);
      me = perm(w, w << 8, 0x0B090A08u);
      mo = perm(w << 4, w << 12, 0x0B090A08u);
      se = (w >> 4) & 0x07070707u;
      so = w & 0x07070707u;
      pin_out(me), pin_out(mo), pin_out(se), pin_out(so);
    } else if (k == 1) {
      pin_in(me), pin_in(se);
      le = (me & perm(t.lo[3], t.lo[2], se)) | (~me & perm(t.lo[1], t.lo[0], se));
      he = (me & perm(t.hi[3], t.hi[2], se)) | (~me & perm(t.hi[1], t.hi[0], se));
      pin_out(le), pin_out(he);
    } else if (k == 2) {
      pin_in(mo), pin_in(so);
      lo = (mo & perm(t.lo[3], t.lo[2], so)) | (~mo & perm(t.lo[1], t.lo[0], so));
      ho = (mo & perm(t.hi[3], t.hi[2], so)) | (~mo & perm(t.hi[1], t.hi[0], so));
      pin_out(lo), pin_out(ho);
    } else {
      pin_in(le), pin_in(he), pin_in(lo), pin_in(ho);
      const uint32_t l03 = perm(lo, le, 0x05010400u), h03 = perm(ho, he, 0x05010400u);
      const uint32_t l47 = perm(lo, le, 0x07030602u), h47 = perm(ho, he, 0x07030602u);
      r[0] = perm(h03, l03, 0x05010400u);
      r[1] = perm(h03, l03, 0x07030602u);
      r[2] = perm(h47, l47, 0x05010400u);
      r[3] = perm(h47, l47, 0x07030602u);
      pin_out(r[0]), pin_out(r[1]), pin_out(r[2]), pin_out(r[3]);
    }
  }
  __device__ __forceinline__ bf16x8 value() const { return as_bf16x8(r[0], r[1], r[2], r[3]); }
};

// ---------------------------------------------------------------------------
// int8 dequantization in registers: bf16_rne(fp32(q * s)).  q + 128 is the
// unsigned byte of q ^ 0x80, and fma(u, s, -128 s) rounds the exact q * s
// once, exactly like the plain product.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 i8_frag(uint32_t w0, uint32_t w1, float s, float ns128) {
  const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
  float f[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = __builtin_fmaf((float)((u0 >> (8 * j)) & 0xffu), s, ns128);
    f[4 + j] = __builtin_fmaf((float)((u1 >> (8 * j)) & 0xffu), s, ns128);
  }
  return as_bf16x8(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7]));
}

// One weight row's share of a K step for one lane: the packed codes of the
// lane's half of the step and the row scale (NF4: absmax of the 64-block).
template <int FMT>
struct RowCodes {
  uint4 c0, c1;
  Scale<FMT> scale;  // as loaded; sc() is the one to use
  uint32_t m;        // all ones when the step is in range, else zero

  // Exactly kLoads vector loads per call (the K-step pipeline counts on it),
  // always issued, with no branch around them, so that a caller can place
  // them between MFMAs: row_base: codes of the row (always a valid row);
  // srow: scales of the row; k0: K step start; hh: lane half; K: row length;
  // ok: the row is real.  Outside the row or the K range the loads read the
  // row start and the step is zeroed through its scale when consumed (NF4:
  // zero absmax -> all-zero table; int8: zero scale -> the A operand is
  // exactly zero), so nothing waits on the loads here.
  static constexpr int kLoads = 2 + SRow<FMT>::kLoads;
  __device__ __forceinline__ void fetch(const uint8_t* row_base, const SRow<FMT>& srow, int k0, int hh, int K,
                                        bool ok) {
    constexpr int half = Fmt<FMT>::kStep / 2;
    const int kk = k0 + half * hh;
    const bool in = ok && kk < K;
    const int kc = in ? kk : 0;
    const uint4* p = reinterpret_cast<const uint4*>(row_base + (kNf4Codes<FMT> ? kc / 2 : kc));
    c0 = p[0];
    c1 = p[1];
    scale = srow.load(kNf4Codes<FMT> ? kc / kNf4Block : 0);
    m = in ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(m));  // opaque, so the select is not folded into a branch around the loads
  }
  __device__ __forceinline__ Scale<FMT> sc() const { return scale.masked(m); }
  __device__ __forceinline__ uint32_t word(int i) const {
    const uint4& c = (i < 4) ? c0 : c1;
    const int j = i & 3;
    return j == 0 ? c.x : (j == 1 ? c.y : (j == 2 ? c.z : c.w));
  }
};

// Codes for a loop that never branches around its loads: the loads always
// issue (in-range addresses) and a step outside the row or the K range is
// zeroed through its scale alone when it is consumed.  A zero scale makes the
// A operand exactly zero for NF4 (every table entry is a level times zero)
// and for int8.  Masking at use keeps the load registers untouched until
// then, so the memory counter can be waited on partially.
template <int FMT>
struct StreamCodes {
  RowCodes<FMT> raw;
  uint32_t m;
  // row_scale: the int8 row scale, loaded once by the caller (a per-step
  // load of a loop-invariant value would be hoisted to just before the loop
  // and make every step wait for it); unused for NF4.
  __device__ __forceinline__ void fetch(const uint8_t* row_base, const SRow<FMT>& srow, int k0, int hh, int K,
                                        bool ok, float row_scale) {
    constexpr int half = Fmt<FMT>::kStep / 2;
    const int kk = k0 + half * hh;
    const bool in = ok && kk < K;
    const int kc = in ? kk : 0;
    const uint4* p = reinterpret_cast<const uint4*>(row_base + (kNf4Codes<FMT> ? kc / 2 : kc));
    raw.c0 = p[0];
    raw.c1 = p[1];
    if constexpr (kNf4Codes<FMT>)
      raw.scale = srow.load(kc / kNf4Block);
    else
      raw.scale = {row_scale};
    m = in ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(m));  // opaque, so the select is not folded into a branch around the loads
  }
  // The codes and the range mask only, for a caller that loads the scales
  // itself and sets raw.scale before use().
  __device__ __forceinline__ void fetch_codes(const uint8_t* row_base, int k0, int hh, int K, bool ok) {
    constexpr int half = Fmt<FMT>::kStep / 2;
    const int kk = k0 + half * hh;
    const bool in = ok && kk < K;
    const int kc = in ? kk : 0;
    const uint4* p = reinterpret_cast<const uint4*>(row_base + (kNf4Codes<FMT> ? kc / 2 : kc));
    raw.c0 = p[0];
    raw.c1 = p[1];
    m = in ? 0xffffffffu : 0u;
    asm volatile("" : "+v"(m));
  }
  __device__ __forceinline__ RowCodes<FMT> use() const {
    RowCodes<FMT> r = raw;
    r.m = m;
    return r;
  }
};

template <int FMT>
struct Dequant {  // NF4, plain or with double-quantized absmax
  Nf4Table t;
  __device__ __forceinline__ void prepare(const RowCodes<FMT>& r) { t = nf4_table(r.sc().value()); }
  // the same table in kPrepStages pieces: piece q holds levels 4q .. 4q+3
  static constexpr int kPrepStages = 4;
  __device__ __forceinline__ void prep_stage(int q, const RowCodes<FMT>& r) {
    float a = r.sc().value();
    pin_in(a);
    const uint32_t p0 = pack_bf16x2(__uint_as_float(kNf4LevelBits[4 * q]) * a,
                                    __uint_as_float(kNf4LevelBits[4 * q + 1]) * a);
    const uint32_t p1 = pack_bf16x2(__uint_as_float(kNf4LevelBits[4 * q + 2]) * a,
                                    __uint_as_float(kNf4LevelBits[4 * q + 3]) * a);
    t.lo[q] = perm(p1, p0, 0x06040200u);
    t.hi[q] = perm(p1, p0, 0x07050301u);
    pin_out(t.lo[q]), pin_out(t.hi[q]);
  }
  // MFMA step s (0..7) of the K step: codes word s = 8 consecutive k of the block
  __device__ __forceinline__ bf16x8 frag(const RowCodes<FMT>& r, int s) const { return nf4_frag(t, r.word(s)); }
};

// One A fragment computed in stages: begin() takes MFMA step s's codes,
// stage(k) for k = 0 .. kStages-1 in order, then value().
template <int FMT>
struct FragStages {  // NF4, plain or with double-quantized absmax
  static constexpr int kStages = Nf4FragStages::kStages;
  Nf4FragStages f;
  __device__ __forceinline__ void begin(const RowCodes<FMT>& r, int s) { f.w = r.word(s); }
  __device__ __forceinline__ void stage(int k, const Dequant<FMT>& d) { f.stage(k, d.t); }
  __device__ __forceinline__ bf16x8 value() const { return f.value(); }
};

template <>
struct Dequant<MOEQ_FMT_INT8_ROWWISE> {
  float s, ns128;
  __device__ __forceinline__ void prepare(const RowCodes<MOEQ_FMT_INT8_ROWWISE>& r) {
    s = r.sc().value();
    ns128 = -128.0f * s;
  }
  static constexpr int kPrepStages = 1;
  __device__ __forceinline__ void prep_stage(int, const RowCodes<MOEQ_FMT_INT8_ROWWISE>& r) { prepare(r); }
  // MFMA step s (0..3): 8 consecutive int8 codes = words 2s, 2s+1
  __device__ __forceinline__ bf16x8 frag(const RowCodes<MOEQ_FMT_INT8_ROWWISE>& r, int s_) const {
    return i8_frag(r.word(2 * s_), r.word(2 * s_ + 1), s, ns128);
  }
};

// i8_frag in two stages (one code word each), same arithmetic.
template <>
struct FragStages<MOEQ_FMT_INT8_ROWWISE> {
  static constexpr int kStages = 2;
  uint32_t w[2], r[4];
  __device__ __forceinline__ void begin(const RowCodes<MOEQ_FMT_INT8_ROWWISE>& c, int s) {
    w[0] = c.word(2 * s);
    w[1] = c.word(2 * s + 1);
  }
  __device__ __forceinline__ void stage(int k, const Dequant<MOEQ_FMT_INT8_ROWWISE>& d) {
    pin_in(w[k]);
    const uint32_t u = w[k] ^ 0x80808080u;
    float f[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) f[j] = __builtin_fmaf((float)((u >> (8 * j)) & 0xffu), d.s, d.ns128);
    r[2 * k] = pack_bf16x2(f[0], f[1]);
    r[2 * k + 1] = pack_bf16x2(f[2], f[3]);
    pin_out(r[2 * k]), pin_out(r[2 * k + 1]);
  }
  __device__ __forceinline__ bf16x8 value() const { return as_bf16x8(r[0], r[1], r[2], r[3]); }
};

// ---------------------------------------------------------------------------
// Work items: expert-major (expert, group of kTileGroup token tiles, column
// tile, token tile within the group), dealt to the XCDs in contiguous
// ranges.  tile_start = exclusive prefix of per-expert token-tile counts.
// ---------------------------------------------------------------------------
constexpr int kTileGroup = 4;

// Rows [*row0, *row0 + *nrows) of tile mt of expert e: the expert's rows
// split into tile_start[e+1] - tile_start[e] near-equal tiles (at most kBM
// rows each, since the count is ceil(rows / kBM)).
__device__ __forceinline__ void tile_rows(const int32_t* offsets, const int32_t* tile_start, int e, int mt,
                                          int* row0, int* nrows) {
  const int c = offsets[e + 1] - offsets[e];
  const int nt = tile_start[e + 1] - tile_start[e];
  const int lo = (int)((int64_t)mt * c / nt), hi = (int)((int64_t)(mt + 1) * c / nt);
  *row0 = offsets[e] + lo;
  *nrows = hi - lo;
}

__device__ __forceinline__ bool decode_work(const int32_t* tile_start, int E, int ncol, int& e, int& mt,
                                            int& ct) {
  const int total = tile_start[E] * ncol;
  const int per = (total + kXcds - 1) / kXcds;
  const int slot = blockIdx.x / kXcds;
  const int w = (blockIdx.x % kXcds) * per + slot;
  if (slot >= per || w >= total) return false;
  int lo = 0, hi = E - 1;  // largest e with tile_start[e] * ncol <= w
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] * ncol <= w) lo = mid; else hi = mid - 1;
  }
  e = lo;
  const int r = w - tile_start[e] * ncol;
  const int nt = tile_start[e + 1] - tile_start[e];
  // the expert's token tiles in groups of kTileGroup; a group's items run
  // column tile by column tile, so the items in flight on an XCD at once
  // share a few token tiles and a few weight column tiles, each K step of
  // which is fetched once into that XCD's L2
  const int g = r / (kTileGroup * ncol);
  const int gt = min(kTileGroup, nt - g * kTileGroup);
  const int rr = r - g * kTileGroup * ncol;
  ct = rr / gt;
  mt = g * kTileGroup + (rr - ct * gt);
  return true;
}

// ---------------------------------------------------------------------------
// The GEMM core shared by G1 and G2: NB token blocks of 32 rows (the tile's
// 32*NB sorted rows, MFMA B operand, from LDS) times two 32-row weight
// blocks per wave (MFMA A operand, dequantized in registers), accumulated
// over K.
//
// Token rows go global -> LDS directly (global_load_lds_dwordx4: lane l of a
// wave lands 16 B at the wave's LDS base + 16 l), one K step ahead.  One
// instruction of a wave moves whole row segments (4 rows x 256 B for NF4,
// 8 rows x 128 B for int8), so every cache line it touches is used in full.
// The LDS tile is row-major with the 16-B slots of a row XOR-swizzled by the
// row, so the fragment reads (32 consecutive rows, one k chunk) hit distinct
// banks.  The swizzle is the same for every row a lane stages, so a lane's
// source offset within a row is one constant.  Rows past the tile stage a
// valid row (their results are never stored); k past the end meets zero
// weights.
// ---------------------------------------------------------------------------
template <int FMT, int NB>
struct Core {
  // LDS token buffers: three (token DMAs two K steps ahead) when they fit in
  // LDS next to the largest tile's two, else two (one step ahead).
  static constexpr int kNbuf = NB <= 6 ? 3 : 2;
  static constexpr int kStep = Fmt<FMT>::kStep;
  static constexpr int kRows = 32 * NB;
  static constexpr int kCpr = kStep / 8;                  // 16-B chunks per row per step
  static constexpr int kRpi = 64 / kCpr;                  // rows per wave instruction
  static constexpr int kInstr = kRows / (kWaves * kRpi);  // staging instructions per wave per step
  static constexpr int kBufBytes = kRows * kCpr * 16;

  // slot swizzle of row r: conflict-free for 16 consecutive rows
  __device__ __forceinline__ static int swz(int r) { return kCpr == 16 ? (r & 15) : ((r >> 1) & 7); }
  // the tile row staged by lane l of wave w in instruction i
  __device__ __forceinline__ static int staged_row(int w, int l, int i) { return kRpi * (kWaves * i + w) + l / kCpr; }

  // sX: kNbuf LDS buffers of buf_bytes; tbase + roff[i]: byte address of the row staged in
  // instruction i; K: reduction length; (q0, s0) / (q1, s1): this lane's two
  // weight rows.
  __device__ __forceinline__ static void run(char* sX, int buf_bytes, const char* tbase, const uint32_t (&roff)[kInstr],
                                             int K, const uint8_t* q0, const SRow<FMT>& s0, const uint8_t* q1,
                                             const SRow<FMT>& s1, bool wave_on, f32x16 (&acc0)[NB],
                                             f32x16 (&acc1)[NB]) {
    const int t = threadIdx.x, lane = t & 63;
    // wave-uniform, so each DMA's LDS base (M0) is scalar arithmetic rather
    // than a vector result moved to a scalar register per instruction
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l32 = lane & 31, hh = lane >> 5;
    // source chunk of this lane within its row (the same for every instruction)
    const int chunk = (lane % kCpr) ^ swz(staged_row(wave, lane, 0));
    // The DMA target is passed as a bare LDS address: with the array itself
    // the compiler would make LDS reads wait for all DMAs in flight.  The
    // explicit waits before each barrier order them instead.
    uint32_t stage0 = (uint32_t)(size_t)(__attribute__((address_space(3))) char*)(sX + staged_row(wave, 0, 0) * kCpr * 16);
    asm volatile("" : "+s"(stage0));  // opaque, so it is not folded back into a pointer to the array

    // instruction i of the token DMA for K offset k0 into buffer buf
    auto stage_one = [&](int k0, int buf, int i) {
      int kk = k0 + 8 * chunk;
      kk = kk < K ? kk : 0;
      __builtin_amdgcn_global_load_lds(
          tbase + roff[i] + 2 * kk,
          (__attribute__((address_space(3))) void*)(size_t)(stage0 + buf * buf_bytes + i * kWaves * kRpi * kCpr * 16),
          16, 0, 0);
    };
    auto stage = [&](int k0, int buf) {
#pragma unroll
      for (int i = 0; i < kInstr; ++i) stage_one(k0, buf, i);
    };

    // B fragment of token block b at MFMA step s: row 32b + l32, chunk
    // (kCpr/2)*hh + s, stored at slot chunk ^ swz(row) (swz(row) = swz(l32)).
    const int rsw = swz(l32);

    // Registers of one K step: the packed codes of the lane's two weight
    // rows, their dequantization tables and the A fragments of MFMA step 0.
    struct StepRegs {
      RowCodes<FMT> c0, c1;
      Dequant<FMT> d0, d1;
      bf16x8 a0, a1;
    };

    // One K step.  Runs this step's MFMAs from LDS buffer ks % kNbuf with
    // the registers in `cur`, and meanwhile
    //   * loads step ks + 1's codes into `nxt` (first thing in the step),
    //   * starts the token DMAs of step ks + 1 (two buffers) or ks + 2
    //     (three), spread over the first kDmaSub MFMA steps (a burst at the
    //     step start stalls the wave on the memory pipeline),
    //   * dequantizes MFMA step s + 1's A fragments during MFMA step s, and
    //     during the last MFMA step builds step ks + 1's tables and its first
    //     A fragments, so the next step starts on MFMAs right after the
    //     barrier.
    // The VALU work is cut into stages of a few instructions and one slice is
    // placed after each MFMA, fenced so the compiler keeps it there (an MFMA
    // runs for 32 cycles while the wave keeps issuing independent VALU work;
    // left to itself the compiler bunches the VALU work between MFMA bursts).
    // A straight line (no branches around the MFMAs, so the accumulators stay
    // put): a wave with no weight rows multiplies zeros, and the last step
    // prefetches a harmless extra step (zero codes, an in-range row).
    constexpr int kS = kStep / 16;         // MFMA steps per K step
    constexpr int kSlots = 2 * NB;         // MFMAs per MFMA step
    constexpr int kDma0 = 0;                      // first MFMA step that carries token DMAs
    constexpr int kDmaSub = kS - 1;               // MFMA steps that carry them
    constexpr int kFetch0 = kS > 4 ? 1 : 0;       // MFMA steps that load the next step's codes
    constexpr int kFetch1 = kS > 4 ? 3 : 1;
    constexpr int kFragWork = 2 * FragStages<FMT>::kStages;
    constexpr int kPrepWork = 2 * Dequant<FMT>::kPrepStages;
    constexpr int kLastWork = kPrepWork + kFragWork;
    auto kstep = [&](int ks, StepRegs& cur, StepRegs& nxt) {
      const int buf = ks % kNbuf;
      const int dstep = kNbuf == 2 ? ks + 1 : ks + 2;  // the step the DMAs fetch
      const char* xb = sX + buf * buf_bytes + l32 * kCpr * 16;
      auto bfrag = [&](int s_, int b) {
        const int slot = ((kCpr / 2) * hh + s_) ^ rsw;
        return *reinterpret_cast<const bf16x8*>(xb + (32 * b * kCpr + slot) * 16);
      };
      bf16x8 a0 = cur.a0, a1 = cur.a1;
      bf16x8 xf[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) xf[b] = bfrag(0, b);
#pragma unroll
      for (int s = 0; s < kS; ++s) {
        const bool last = s + 1 == kS;
        FragStages<FMT> f0, f1;
        if (!last) {
          f0.begin(cur.c0, s + 1);
          f1.begin(cur.c1, s + 1);
        }
        if (s >= kDma0 && s < kDma0 + kDmaSub) {
#pragma unroll
          for (int i = (s - kDma0) * kInstr / kDmaSub; i < (s - kDma0 + 1) * kInstr / kDmaSub; ++i)
            stage_one(dstep * kStep, dstep % kNbuf, i);
        }
        if (s == kFetch0) nxt.c0.fetch(q0, s0, (ks + 1) * kStep, hh, K, wave_on);
        if (s == kFetch1) nxt.c1.fetch(q1, s1, (ks + 1) * kStep, hh, K, wave_on);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
          const int b = i >> 1;
          if (i & 1)
            acc1[b] = mfma(a1, xf[b], acc1[b]);
          else
            acc0[b] = mfma(a0, xf[b], acc0[b]);
          if (!last) {
            // token block b is done for this MFMA step: read its next fragment
            if (i & 1) xf[b] = bfrag(s + 1, b);
            // frag stages j in [i*W/kSlots, (i+1)*W/kSlots): f0's, then f1's
            constexpr int kF = FragStages<FMT>::kStages;
#pragma unroll
            for (int j = i * kFragWork / kSlots; j < (i + 1) * kFragWork / kSlots; ++j) {
              if (j >= kF)
                f1.stage(j - kF, cur.d1);
              else
                f0.stage(j, cur.d0);
            }
          } else {
            // next K step: its two tables first, then its first A fragments
#pragma unroll
            for (int j = i * kLastWork / kSlots; j < (i + 1) * kLastWork / kSlots; ++j) {
              if (j < kPrepWork) {
                if (j & 1)
                  nxt.d1.prep_stage(j >> 1, nxt.c1);
                else
                  nxt.d0.prep_stage(j >> 1, nxt.c0);
              } else {
                const int k = j - kPrepWork;
                constexpr int kF = FragStages<FMT>::kStages;
                if (k == 0) f0.begin(nxt.c0, 0);
                if (k == kF) f1.begin(nxt.c1, 0);
                if (k >= kF)
                  f1.stage(k - kF, nxt.d1);
                else
                  f0.stage(k, nxt.d0);
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (!last) {
          a0 = f0.value();
          a1 = f1.value();
        } else {
          nxt.a0 = f0.value();
          nxt.a1 = f1.value();
        }
      }
      // Vector loads complete in order.  Two buffers: this step's DMAs (for
      // step ks + 1) are the last loads issued, so wait for all.  Three
      // buffers: the DMAs for step ks + 1 were issued in the previous step and
      // only this step's code loads and DMAs may still be in flight.  No
      // release fence is needed: every LDS read of this step has been
      // consumed by an MFMA above; the acquire fence keeps the next step's
      // LDS reads below the barrier.
      __builtin_amdgcn_s_waitcnt(kVmcntWait<kNbuf == 2 ? 0 : 2 * RowCodes<FMT>::kLoads + kInstr>);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    };

    // two register sets, used in turn (no copies between steps)
    StepRegs ra, rb;
    stage(0, 0);
    if (kNbuf == 3) stage(kStep, 1);
    __builtin_amdgcn_sched_barrier(0);
    ra.c0.fetch(q0, s0, 0, hh, K, wave_on);
    ra.c1.fetch(q1, s1, 0, hh, K, wave_on);
    __builtin_amdgcn_s_waitcnt(0);
    ra.d0.prepare(ra.c0);
    ra.d1.prepare(ra.c1);
    ra.a0 = ra.d0.frag(ra.c0, 0);
    ra.a1 = ra.d1.frag(ra.c1, 0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const int nks = (K + kStep - 1) / kStep;
    int ks = 0;
    for (; ks + 1 < nks; ks += 2) {
      kstep(ks, ra, rb);
      kstep(ks + 1, rb, ra);
    }
    if (ks < nks) kstep(ks, ra, rb);
  }
};

template <int FMT>
struct Lds {
  // bytes per buffer (largest tile), and the LDS all paths fit in
  static constexpr int kBuf = Core<FMT, kBM / 32>::kBufBytes;
  static constexpr int kTotal = 2 * kBuf > 3 * Core<FMT, 6>::kBufBytes ? 2 * kBuf : 3 * Core<FMT, 6>::kBufBytes;
  // G1 and G2 also stage output tiles (kBM rows of 512 B, padded) in the same array
  static constexpr int kYTile = kBM * (2 * kG2Rows + 16);
  static constexpr int kG2 = kTotal > kYTile ? kTotal : kYTile;
};

// Copies a tile staged in LDS out to global memory, whole rows at a time:
// row r (r < nrows <= kRows) of kChunks 16-B chunks at src + r * kPitch goes
// to dst + r * ld (elements of T), chunks whose first element is at or past
// `cols` skipped (cols a multiple of 16 / sizeof(T)).  A fixed, unrolled trip
// count, so the LDS reads are issued ahead of the stores.  Stored straight
// from the MFMA accumulator layout, each store instruction would touch 32
// rows (32 cache lines, a 16-B piece of each).
template <typename T, int kRows, int kChunks, int kPitch>
__device__ __forceinline__ void copy_rows(const char* src, int nrows, int cols, T* __restrict__ dst, int64_t ld) {
  constexpr int kPer = 16 / (int)sizeof(T);  // elements per chunk
  const int total = nrows * kChunks;
#pragma unroll
  for (int u = 0; u < kRows * kChunks / kThreads; ++u) {
    const int c = threadIdx.x + u * kThreads, r = c / kChunks, k = c % kChunks;
    if (c < total && kPer * k < cols)
      *reinterpret_cast<uint4*>(dst + r * ld + kPer * k) = *reinterpret_cast<const uint4*>(src + r * kPitch + 16 * k);
  }
}

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
  const int l32 = lane & 31, hh = lane >> 5;
  if (wave_on) {
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
// Y: float (fp32 y) or uint16_t (y rounded to bf16).
template <int FMT, int NB, typename Y>
__device__ __forceinline__ void g2_tile(char* sX, const float* sw, const uint16_t* h, int H, int I, int ncol,
                                        bool on, const uint8_t* q0, const SRow<FMT>& s0, const uint8_t* q1,
                                        const SRow<FMT>& s1, int row0, int nrows, Y* __restrict__ y) {
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
  if constexpr (sizeof(Y) == 2) {
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
    copy_rows<uint16_t, kBM, 2 * kG2Rows / 16, kPitch>(sX, nrows, H - n0,
                                                      reinterpret_cast<uint16_t*>(y) + (int64_t)row0 * H + n0, H);
    return;
  } else {
    // fp32 y (the backward's unweighted z) the same way, 128 rows per round
    constexpr int kPitch = 4 * kG2Rows + 16;
    constexpr int kRound = 4;  // token blocks per round
    static_assert(32 * kRound * kPitch <= Lds<FMT>::kG2, "y rows fit the LDS array");
    const int n0 = ncol - 64 * wave;
    __builtin_amdgcn_s_waitcnt(0);  // token DMAs of the extra prefetched step may still be landing
#pragma unroll
    for (int b0 = 0; b0 < NB; b0 += kRound) {
      __syncthreads();  // the LDS is free (token buffers, or the previous round's rows)
      if (on) {
#pragma unroll
        for (int b = b0; b < (b0 + kRound < NB ? b0 + kRound : NB); ++b) {
          const float wr = sw[32 * b + l32];
          char* rowp = sX + (32 * (b - b0) + l32) * kPitch + 4 * (64 * wave + 4 * hh);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
              const f32x16& a = m ? acc1[b] : acc0[b];
              *reinterpret_cast<float4*>(rowp + 4 * (32 * m + 8 * q)) =
                  make_float4(a[4 * q] * wr, a[4 * q + 1] * wr, a[4 * q + 2] * wr, a[4 * q + 3] * wr);
            }
          }
        }
      }
      __syncthreads();
      const int rows = nrows - 32 * b0;
      copy_rows<float, 32 * kRound, 4 * kG2Rows / 16, kPitch>(sX, rows < 32 * kRound ? rows : 32 * kRound, H - n0,
                                                              reinterpret_cast<float*>(y) + (int64_t)(row0 + 32 * b0) * H + n0, H);
    }
  }
}

template <int FMT, typename Y>
__global__ __launch_bounds__(kThreads) void g2_kernel(const uint16_t* __restrict__ h, const float* __restrict__ wts,
                                                     int32_t E, int32_t H, int32_t I,
                                                     const uint8_t* __restrict__ wq, const float* __restrict__ ws,
                                                     const uint8_t* __restrict__ wsc,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ tile_start,
                                                     const int32_t* __restrict__ perm_idx, Y* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) char sX[Lds<FMT>::kG2];
  __shared__ float sw[kBM];

  int e, mt, ct;
  if (!decode_work(tile_start, E, (H + kG2Rows - 1) / kG2Rows, e, mt, ct)) return;
  int row0, nrows;
  tile_rows(offsets, tile_start, e, mt, &row0, &nrows);
  const int t = threadIdx.x, wave = t >> 6, l32 = t & 31;
  // wts == nullptr: unit weights (the backward's unweighted y)
  if (t < kBM) sw[t] = (t < nrows) ? (wts ? wts[perm_idx[row0 + t]] : 1.0f) : 0.0f;

  const int ncol = ct * kG2Rows + 64 * wave;  // H % 64 == 0: a wave is all in or all out
  const bool on = ncol < H;
  const int r0 = (on ? ncol : 0) + l32, r1 = r0 + 32;  // rows within the expert
  const int cpr = kNf4Codes<FMT> ? I / 2 : I;

  const uint8_t* q0 = wq + ((int64_t)e * H + r0) * cpr;
  const uint8_t* q1 = wq + ((int64_t)e * H + r1) * cpr;
  const SRow<FMT> s0 = srow_at<FMT>(ws, wsc, e, H, r0, I, 0);
  const SRow<FMT> s1 = srow_at<FMT>(ws, wsc, e, H, r1, I, 0);
  if (nrows > 192)
    g2_tile<FMT, 8, Y>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
  else if (nrows > 128)
    g2_tile<FMT, 6, Y>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
  else if (nrows > 64)
    g2_tile<FMT, 4, Y>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
  else
    g2_tile<FMT, 2, Y>(sX, sw, h, H, I, ncol, on, q0, s0, q1, s1, row0, nrows, y);
}

// ---------------------------------------------------------------------------
// Decode path (few assignments, T*K <= kDecodeMax): no routing kernels and
// no token tiles.  A workgroup owns one touched expert (its blockIdx.x-th, in
// expert order) and RB row blocks of 64 weight rows; it finds the expert and
// the expert's assignments itself from top_k_index (ascending assignment
// order).  Its NW waves are RB row blocks x P parts of K (NW = RB * P, P
// chosen on the host so that few touched experts still fill the chip).  Each
// wave streams its part of its 64 rows' packed codes straight from HBM,
// dequantizes them in registers into the MFMA A operand and multiplies the
// expert's token rows (at most 32 per pass, read from L2 as the B operand).
// The P partial sums of a row block meet in LDS and are added in part order,
// so the result does not depend on timing.  Rows of h and y are indexed by
// assignment, so the combine needs no slot map.
//   G1 (gate_up): row block = gate rows jcol..+32 and up rows I+jcol..+32,
//                 K = H, B rows x[a / K]; h[a][jcol..+32] = bf16(silu(g) * u).
//   G2 (down):    row block = down rows ncol..+64, K = I, B rows h[a];
//                 y[a][ncol..+64] = w_a * acc.
// ---------------------------------------------------------------------------
constexpr int kDecodeMax = 512;

// LDS-only barrier: waits for this wave's LDS traffic, not for its global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// AB: how plain-NF4 absmax reach the lanes -- 0: one load per K step and row;
// 2: a pair per two steps (PAIR below); 8: eight per lane per eight steps
// (OCT below).
template <int FMT, bool G1, int NW, int AB>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const uint16_t* __restrict__ act,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ wts, int32_t n, int32_t Ktop,
                                                        int32_t E, int32_t H, int32_t I, int32_t P,
                                                        const uint8_t* __restrict__ wq,
                                                        const float* __restrict__ ws,
                                                        const uint8_t* __restrict__ wsc,
                                                        uint16_t* __restrict__ hout, float* __restrict__ yout) {
  constexpr int kT = NW * 64;
  constexpr int kJ = kDecodeMax / kT;  // assignments per thread
  constexpr int kStep = Fmt<FMT>::kStep;
  constexpr int kS = kStep / 16;
  __shared__ uint32_t bits[MOEQ_MAX_EXPERTS / 32];
  __shared__ int list[kDecodeMax];
  __shared__ int cnt[kDecodeMax / 64];
  __shared__ float red[NW][2][16][64];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform, so the K loop is scalar
  const int l32 = lane & 31, hh = lane >> 5;

  // 1. this thread's assignments (a = t + j*kT) and the set of touched experts
  int my[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int a = t + j * kT;
    my[j] = a < n ? idx[a] : -1;
  }
  if (t < MOEQ_MAX_EXPERTS / 32) bits[t] = 0u;
  lds_barrier();
#pragma unroll
  for (int j = 0; j < kJ; ++j)
    if (my[j] >= 0 && my[j] < E) atomicOr(&bits[my[j] >> 5], 1u << (my[j] & 31));
  lds_barrier();

  // 2. this block's expert: the blockIdx.x-th touched one (every wave finds it)
  int e = -1;
  {
    const int nw = (E + 31) / 32;
    const uint32_t wbits = (lane < nw) ? bits[lane] : 0u;
    const int c = __popc(wbits);
    int inc = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    const int u = blockIdx.x;
    const uint64_t who = __ballot((inc - c) <= u && u < inc);
    if (who) {
      const int src = __builtin_ctzll(who);
      uint32_t wb = __shfl(wbits, src, 64);
      for (int r = u - (__shfl(inc, src, 64) - __shfl(c, src, 64)); r > 0; --r) wb &= wb - 1;
      e = src * 32 + __builtin_ctz(wb);
    }
    e = __builtin_amdgcn_readfirstlane(e);
  }
  if (e < 0) return;  // the whole block: the bitmap is shared

  // 3. this wave's row block and part of K; start its first codes now
  const int K = G1 ? H : I;
  const int nrb = G1 ? I / 32 : H / 64;  // row blocks of the expert
  const int RB = NW / P;
  const int rbi = blockIdx.y * RB + wave / P, part = wave % P;
  const bool on = rbi < nrb;  // a wave past the last row block streams block 0 and stores nothing
  const int col0 = (on ? rbi : 0) * (G1 ? 32 : 64);
  const int R = G1 ? 2 * I : H;  // rows per expert
  const int r0 = col0 + l32, r1 = G1 ? r0 + I : r0 + 32;  // rows within the expert
  const int cpr = kNf4Codes<FMT> ? K / 2 : K;
  const uint8_t* q0 = wq + ((int64_t)e * R + r0) * cpr;
  const uint8_t* q1 = wq + ((int64_t)e * R + r1) * cpr;
  const SRow<FMT> s0 = srow_at<FMT>(ws, wsc, e, R, r0, K, 0);
  const SRow<FMT> s1 = srow_at<FMT>(ws, wsc, e, R, r1, K, 0);
  // Parts are whole groups of gran K steps: eights when K is a multiple of
  // 1024 and the P parts split the steps into equal eights (the condition
  // under which the host picks AB = 8), else pairs.  The split depends on
  // the shape only, not on AB, so every format sums the same parts.
  constexpr int kTrip = AB == 8 ? 8 : 2;  // steps per loop trip
  constexpr bool PAIR = AB == 2;
  const int nks = (K + kStep - 1) / kStep;
  const int gran = (K % 1024 == 0 && nks % (8 * P) == 0) ? 8 : 2;
  const int nkp = (nks + gran - 1) / gran;  // groups of steps
  const int ks0 = gran * (part * nkp / P), ks1 = min(gran * ((part + 1) * nkp / P), nks);
  // int8: the row scales, first of this wave's loads
  float rs0 = 0.0f, rs1 = 0.0f;
  if constexpr (!kNf4Codes<FMT>) {
    rs0 = s0.p[0];
    rs1 = s1.p[0];
  }
  StreamCodes<FMT> ca0, ca1, cb0, cb1;
  // PAIR (plain NF4, an even number of 64-blocks per row): the absmax of two
  // K steps comes in one 8-byte load per lane and row instead of two 4-byte
  // ones.  Lanes of half hh load the pair of step ks + hh (blocks 2(ks+hh)
  // and 2(ks+hh)+1; row start past the range); one v_permlane32_swap then
  // gives every lane its own block of step ks and of step ks + 1.  Each such
  // load touches one cache line per row of the wave, so halving their number
  // shortens the step.
  float2 pr0 = {}, pr1 = {};
  auto fetch_pair = [&](int ks) {
    if constexpr (PAIR) {
      const int st = ks + hh;
      const int b = st < ks1 ? 2 * st : 0;
      pr0 = *reinterpret_cast<const float2*>(s0.p + b);
      pr1 = *reinterpret_cast<const float2*>(s1.p + b);
    }
  };
  // OCT (plain NF4, the wave's steps a whole number of eights): each lane
  // loads 8 consecutive absmax of each row (32 B) per eight K steps: lane
  // half hh blocks 2 ks + 8 hh .. +7, so the lane pair covers the trip's 16
  // blocks.  Per-step absmax loads would touch each row's absmax line once
  // per two steps, and at long K loops the L2 evicts the line in between
  // (the counter runs showed each absmax byte fetched 4-7 times); here a
  // line is touched once per 8 steps.  At trip step j < 4 one
  // v_permlane32_swap per row of values j of the pair's chunk gives every
  // lane its block of step j and, in the swap's second result, of step
  // j + 4.
  float4 q0a = {}, q0b = {}, q1a = {}, q1b = {};
  auto fetch_oct = [&](int ks) {
    if constexpr (AB == 8) {
      const int b = ks < ks1 ? 2 * ks + 8 * hh : 0;
      q0a = *reinterpret_cast<const float4*>(s0.p + b);
      q0b = *reinterpret_cast<const float4*>(s0.p + b + 4);
      q1a = *reinterpret_cast<const float4*>(s1.p + b);
      q1b = *reinterpret_cast<const float4*>(s1.p + b + 4);
    }
  };
  auto fetch_step = [&](StreamCodes<FMT>& c0, StreamCodes<FMT>& c1, int ks) {
    if constexpr (AB != 0) {
      c0.fetch_codes(q0, ks * kStep, hh, K, ks < ks1);
      c1.fetch_codes(q1, ks * kStep, hh, K, ks < ks1);
    } else {
      c0.fetch(q0, s0, ks * kStep, hh, K, ks < ks1, rs0);
      c1.fetch(q1, s1, ks * kStep, hh, K, ks < ks1, rs1);
    }
  };
  fetch_step(ca0, ca1, ks0);
  fetch_pair(ks0);
  fetch_oct(ks0);

  // 4. the expert's assignments in ascending order: chunk c = a / 64 is
  //    wave c % NW's j = c / NW values
  uint64_t bal[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    bal[j] = __ballot(my[j] == e);
    if (lane == 0) cnt[wave + j * NW] = __popcll(bal[j]);
  }
  lds_barrier();
  int ne = 0;
#pragma unroll
  for (int c = 0; c < kDecodeMax / 64; ++c) ne += cnt[c];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    int base = 0;
    for (int c = 0; c < wave + j * NW; ++c) base += cnt[c];
    if (my[j] == e) list[base + __popcll(bal[j] & ((1ull << lane) - 1ull))] = t + j * kT;
  }
  lds_barrier();

  for (int g = 0; g < ne; g += 32) {
    const int tok = g + l32 < ne ? g + l32 : g;  // lanes past the tokens repeat one (never stored)
    const int a = list[tok];
    const uint16_t* brow = G1 ? act + (int64_t)(a / Ktop) * H : act + (int64_t)a * I;
    if (g > 0) {
      fetch_step(ca0, ca1, ks0);
      fetch_pair(ks0);
      fetch_oct(ks0);
    }

    f32x16 acc0 = (f32x16){}, acc1 = (f32x16){};
    // this lane's half of step ks of the token row: K is a multiple of 64,
    // so the half is wholly in range or wholly past the end (then the row
    // start)
    auto bptr = [&](int ks) {
      const int kb = ks * kStep + (kStep / 2) * hh;
      return reinterpret_cast<const bf16x8*>(brow + (kb < K ? kb : 0));
    };
    // One K step: multiply this step's token fragments, each one replaced
    // by the next step's as soon as its two MFMAs have issued (one register
    // set: 132 VGPRs, three waves per SIMD; the PAIR form needs 152, two
    // waves), then refill this step's code registers two steps ahead.  Loads
    // complete in issue order, so codes stay in flight across a step while
    // the token fragments (L2 hits) are awaited.  Steps past the wave's range
    // load in-range addresses and are zeroed through their scale.
    bf16x8 xa[kS];
    float nx0 = 0.0f, nx1 = 0.0f;  // PAIR: the second step's absmax, after the swap
    float o0[4] = {}, o1[4] = {};  // OCT: the absmax of trip steps 4 .. 7, from the swaps of steps 0 .. 3
    auto oct_at = [](const float4& a, const float4& b, int i) {
      return i < 4 ? (i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : a.w)
                   : (i == 4 ? b.x : i == 5 ? b.y : i == 6 ? b.z : b.w);
    };
    // j: the step's place in its trip (ks - ks0 = j mod kTrip)
    auto kstep = [&](int ks, StreamCodes<FMT>& sc0, StreamCodes<FMT>& sc1, int j) {
      const bool second = (j & 1) != 0;
      // keep each step's arithmetic after the previous step's (hoisting it
      // would wait for codes that are still loading)
      __builtin_amdgcn_sched_barrier(0);
      const bf16x8* pn = bptr(ks + 1);
      if constexpr (PAIR) {
        if (!second) {
          const auto sw0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pr0.x), __float_as_uint(pr0.y), false, false);
          const auto sw1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pr1.x), __float_as_uint(pr1.y), false, false);
          sc0.raw.scale = {__uint_as_float(sw0[0])};
          sc1.raw.scale = {__uint_as_float(sw1[0])};
          nx0 = __uint_as_float(sw0[1]);
          nx1 = __uint_as_float(sw1[1]);
        } else {
          sc0.raw.scale = {nx0};
          sc1.raw.scale = {nx1};
        }
      }
      if constexpr (AB == 8) {
        if (j < 4) {
          const auto sw0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(oct_at(q0a, q0b, 2 * j)),
                                                            __float_as_uint(oct_at(q0a, q0b, 2 * j + 1)), false, false);
          const auto sw1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(oct_at(q1a, q1b, 2 * j)),
                                                            __float_as_uint(oct_at(q1a, q1b, 2 * j + 1)), false, false);
          sc0.raw.scale = {__uint_as_float(sw0[0])};
          sc1.raw.scale = {__uint_as_float(sw1[0])};
          o0[j] = __uint_as_float(sw0[1]);
          o1[j] = __uint_as_float(sw1[1]);
        } else {
          sc0.raw.scale = {o0[j - 4]};
          sc1.raw.scale = {o1[j - 4]};
        }
      }
      const RowCodes<FMT> c0 = sc0.use(), c1 = sc1.use();
      Dequant<FMT> d0, d1;
      d0.prepare(c0);
      d1.prepare(c1);
#pragma unroll
      for (int s_ = 0; s_ < kS; ++s_) {
        acc0 = mfma(d0.frag(c0, s_), xa[s_], acc0);
        acc1 = mfma(d1.frag(c1, s_), xa[s_], acc1);
        xa[s_] = pn[s_];
      }
      fetch_step(sc0, sc1, ks + 2);
      if (!second) fetch_pair(ks + 2);
      // the chunk registers are free after the swap of trip step 3: the next
      // trip's chunk loads from step 4 on
      if (j == 4) fetch_oct(ks - 4 + kTrip);
    };
    {
      const bf16x8* p0 = bptr(ks0);
#pragma unroll
      for (int s_ = 0; s_ < kS; ++s_) xa[s_] = p0[s_];
    }
    fetch_step(cb0, cb1, ks0 + 1);
    // Two steps per trip (eight with OCT absmax), register sets alternating,
    // with no branch between them (a branch there would make the compiler
    // copy or re-load register sets that are still loading, forcing full
    // waits).  Parts are whole pairs (eights) of steps, so only the last part
    // of an odd step count runs a trailing step past the range: its scale is
    // zero, its A operand exactly zero, and it adds nothing.
    if constexpr (AB == 8) {
      for (int ks = ks0; ks < ks1; ks += 8) {
        kstep(ks, ca0, ca1, 0);
        kstep(ks + 1, cb0, cb1, 1);
        kstep(ks + 2, ca0, ca1, 2);
        kstep(ks + 3, cb0, cb1, 3);
        kstep(ks + 4, ca0, ca1, 4);
        kstep(ks + 5, cb0, cb1, 5);
        kstep(ks + 6, ca0, ca1, 6);
        kstep(ks + 7, cb0, cb1, 7);
      }
    } else {
      for (int ks = ks0; ks < ks1; ks += 2) {
        kstep(ks, ca0, ca1, 0);
        kstep(ks + 1, cb0, cb1, 1);
      }
    }

    // the P partial sums of each row block, added in part order
    bool owner = true;
    if (P > 1) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[wave][0][r][lane] = acc0[r];
        red[wave][1][r][lane] = acc1[r];
      }
      lds_barrier();
      owner = part == 0;
      if (owner) {
        // unrolled over the largest P so that the LDS reads are all in flight
#pragma unroll
        for (int p = 1; p < NW; ++p) {
          if (p < P) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              acc0[r] += red[wave + p][0][r][lane];
              acc1[r] += red[wave + p][1][r][lane];
            }
          }
        }
      }
    }
    if (owner && on && g + l32 < ne) {
      // lane holds, per register quad q, rows col0 + 8q + 4*hh + 0..3 of its token
      if (G1) {
        uint16_t* hp = hout + (int64_t)a * I + col0 + 4 * hh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float gg = acc0[4 * q + i], uu = acc1[4 * q + i];
            v[i] = gg * uu * __builtin_amdgcn_rcpf(1.0f + __expf(-gg));
          }
          *reinterpret_cast<uint2*>(hp + 8 * q) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      } else {
        const float wr = wts[a];
        float* yp = yout + (int64_t)a * H + col0 + 4 * hh;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          *reinterpret_cast<float4*>(yp + 8 * q) =
              make_float4(acc0[4 * q] * wr, acc0[4 * q + 1] * wr, acc0[4 * q + 2] * wr, acc0[4 * q + 3] * wr);
          *reinterpret_cast<float4*>(yp + 32 + 8 * q) =
              make_float4(acc1[4 * q] * wr, acc1[4 * q + 1] * wr, acc1[4 * q + 2] * wr, acc1[4 * q + 3] * wr);
        }
      }
    }
    if (P > 1) lds_barrier();  // red is reused by the next token group
  }
}

// Decode combine: out[t] = bf16(sum over k in order of y[t*K + k]), skipping
// unrouted assignments.  One workgroup per token: the routing entries are
// read once into LDS, then each thread keeps the y loads of up to 8
// assignments in flight at once.
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(const float* __restrict__ y,
                                                                 const int32_t* __restrict__ idx, int32_t K,
                                                                 int32_t E, int32_t H, uint16_t* __restrict__ out) {
  __shared__ uint8_t routed[kDecodeMax];
  const int64_t tok = blockIdx.x;
  for (int k = threadIdx.x; k < K; k += kThreads) {
    const int e = idx[tok * K + k];
    routed[k] = e >= 0 && e < E;
  }
  __syncthreads();
  for (int n4 = threadIdx.x; n4 < H / 4; n4 += kThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < K; k0 += 8) {
      bool use[8];
      float4 v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        use[j] = k0 + j < K && routed[k0 + j];
        v[j] = use[j] ? *reinterpret_cast<const float4*>(y + (tok * K + k0 + j) * H + 4 * n4)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (use[j]) {
          acc.x += v[j].x; acc.y += v[j].y; acc.z += v[j].z; acc.w += v[j].w;
        }
      }
    }
    *reinterpret_cast<uint2*>(out + tok * H + 4 * n4) =
        make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

// ---------------------------------------------------------------------------
// C1: out[t] = bf16(y[slot[t*K]] + y[slot[t*K+1]] + ... ) in k order, the
// sum in fp32 over fp32 or bf16 rows of y.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xffff0000u));
}

template <typename Y>
__global__ __launch_bounds__(kThreads) void combine_kernel(const Y* __restrict__ y, const int32_t* __restrict__ slot,
                                                          int32_t K, int32_t H, uint16_t* __restrict__ out) {
  const int64_t tok = blockIdx.x;
  const int32_t* sl = slot + tok * K;
  for (int n4 = threadIdx.x; n4 < H / 4; n4 += kThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k) {
      const int p = sl[k];
      if (p < 0) continue;
      const float4 v = load4(y + (int64_t)p * H + 4 * n4);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *reinterpret_cast<uint2*>(out + tok * H + 4 * n4) =
        make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

// ---------------------------------------------------------------------------
// Backward through the frozen packed experts (gradients with respect to the
// hidden states and the routing weights; see moeq_experts_backward):
//   recompute  g, u, h = G1 of the forward (g and u kept in fp32),
//              z = down h (G2 with unit weights)
//   BW         grad_w[a] = dout[t] . z[a]
//   T1         dh = w * down^T dout[t];  dg = dh u s (1 + g (1 - s)),
//              du = dh g s  -> dgu = bf16 [dg | du]                 (s = sigmoid(g))
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
//           the epilogue forms dg and du from dh = w_p * acc and the saved g, u.
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
                                                        const float* __restrict__ gu_save, void* __restrict__ out) {
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
  // lane l row 8 (4 i + w) + l / 8, LDS slot l % 8 holding chunk slot ^ (row & 7)
  uint32_t voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * (4 * i + wave) + (lane >> 3);
    const int rr = r < nrows ? r : 0;
    voff[i] = (MODE == 1) ? (uint32_t)(perm_idx[row0 + rr] / Ktop) * (uint32_t)R * 2u
                          : (uint32_t)(row0 + rr) * (uint32_t)R * 2u;
  }
  const int vchunk = (lane & 7) ^ ((lane >> 3) & 7);
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
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
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
      const int slot = (2 * s4 + hh) ^ (row & 7);
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
    // dh = w * acc through LDS, then the SwiGLU backward row by row: a
    // thread takes 4 consecutive columns of a row, so the loads of the saved
    // fp32 g and u and the stores of bf16 dg and du cover whole rows (from
    // the accumulator layout each such load touched 32 rows).  The same
    // fp32 operations in the same order as element by element.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const float w = sw[tw + 32 * b + l32];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x16& a = acc[m][b];
          *reinterpret_cast<float4*>(smem + (tw + 32 * b + l32) * kOutPitch + 4 * (cw + 32 * m + 8 * q + 4 * hh)) =
              make_float4(w * a[4 * q], w * a[4 * q + 1], w * a[4 * q + 2], w * a[4 * q + 3]);
        }
    }
    __syncthreads();
    constexpr int kChunks = kTcols / 4;  // 4-column chunks of a tile row
#pragma unroll 4
    for (int u = 0; u < kBM * kChunks / kThreads; ++u) {
      const int i = threadIdx.x + u * kThreads, r = i / kChunks, k4 = i - r * kChunks;
      const int c = c0 + 4 * k4;
      if (r < nrows && c < C) {
        const int64_t p = row0 + r;
        const float4 d4 = *reinterpret_cast<const float4*>(smem + r * kOutPitch + 16 * k4);
        const float4 g4 = *reinterpret_cast<const float4*>(gu_save + p * 2 * C + c);
        const float4 u4 = *reinterpret_cast<const float4*>(gu_save + p * 2 * C + C + c);
        const float dv[4] = {d4.x, d4.y, d4.z, d4.w}, gv[4] = {g4.x, g4.y, g4.z, g4.w},
                    uv[4] = {u4.x, u4.y, u4.z, u4.w};
        float dg[4], du[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[e]));
          du[e] = dv[e] * gv[e] * sg;
          dg[e] = dv[e] * uv[e] * sg * (1.0f + gv[e] * (1.0f - sg));
        }
        uint16_t* o = static_cast<uint16_t*>(out) + p * 2 * C + c;
        *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
        *reinterpret_cast<uint2*>(o + C) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
      }
    }
    return;
  }
  static_assert(MODE == 1 || MODE == 2, "T1 or T2");
}

// grad_w[a] = dout[a / K] . z[slot[a]] (0 for an unrouted assignment), one
// wave per assignment, lanes summed in a fixed tree order.
__global__ __launch_bounds__(kThreads) void gradw_kernel(const uint16_t* __restrict__ dout,
                                                        const float* __restrict__ z,
                                                        const int32_t* __restrict__ slot, int32_t n, int32_t K,
                                                        int32_t H, float* __restrict__ gw) {
  const int64_t a = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (a >= n) return;
  const int lane = threadIdx.x & 63;
  const int p = slot[a];
  float acc = 0.0f;
  if (p >= 0) {
    const uint16_t* d = dout + (a / K) * H;
    const float* zr = z + (int64_t)p * H;
    for (int j = 4 * lane; j < H; j += 256) {
      const uint2 dv = *reinterpret_cast<const uint2*>(d + j);
      const float4 zv = *reinterpret_cast<const float4*>(zr + j);
      acc += __uint_as_float(dv.x << 16) * zv.x + __uint_as_float(dv.x & 0xffff0000u) * zv.y +
             __uint_as_float(dv.y << 16) * zv.z + __uint_as_float(dv.y & 0xffff0000u) * zv.w;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) gw[a] = acc;
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

}  // namespace

int32_t forward_tile_rows() { return kBM; }

// Decode launch shape: 4 waves per workgroup split as RB row blocks x P
// parts of K.  P grows until the touched experts' row blocks give enough
// waves to fill the chip (~6 per CU).
struct DecodeShape {
  int p, rb, gy;
};
DecodeShape decode_shape(int ux, int nrb) {
  const long w1 = (long)ux * nrb;  // waves at P = 1
  const int p = w1 >= 1536 ? 1 : (2 * w1 >= 1536 ? 2 : 4);
  const int rb = kWaves / p;
  return {p, rb, (nrb + rb - 1) / rb};
}

template <int FMT, bool G1>
void launch_decode_gemm(const ForwardArgs& a, int ux, const uint16_t* act, const uint8_t* q, const float* sc,
                        const uint8_t* scc, hipStream_t s) {
  const int32_t n = a.T * a.K;
  const DecodeShape d = decode_shape(ux, G1 ? a.I / 32 : a.H / 64);
  // plain NF4 absmax: in eights when the parts are equal whole eights of K
  // steps (K a multiple of 1024, so the 16-byte chunk loads are aligned and
  // in the row; the kernel splits K the same way), else in pairs when the
  // row holds an even number of blocks
  const int Kr = G1 ? a.H : a.I;
  int ab = 0;
  if constexpr (FMT == MOEQ_FMT_NF4)
    ab = (Kr % 1024 == 0 && (Kr / 128) % (8 * d.p) == 0) ? 8 : ((Kr / kNf4Block) % 2 == 0 ? 2 : 0);
  if (ab == 8)
    decode_kernel<FMT, G1, kWaves, FMT == MOEQ_FMT_NF4 ? 8 : 0><<<dim3(ux, d.gy), kThreads, 0, s>>>(
        act, a.idx, a.wts, n, a.K, a.E, a.H, a.I, d.p, q, sc, scc, a.h, a.y);
  else if (ab == 2)
    decode_kernel<FMT, G1, kWaves, FMT == MOEQ_FMT_NF4 ? 2 : 0><<<dim3(ux, d.gy), kThreads, 0, s>>>(
        act, a.idx, a.wts, n, a.K, a.E, a.H, a.I, d.p, q, sc, scc, a.h, a.y);
  else
    decode_kernel<FMT, G1, kWaves, 0><<<dim3(ux, d.gy), kThreads, 0, s>>>(
        act, a.idx, a.wts, n, a.K, a.E, a.H, a.I, d.p, q, sc, scc, a.h, a.y);
}

template <int FMT>
hipError_t launch_decode(const ForwardArgs& a, hipStream_t s, hipEvent_t const* ev) {
  const int32_t n = a.T * a.K;
  const int ux = a.E < n ? a.E : n;  // at most this many experts are touched
  if (ev) (void)hipEventRecord(ev[1], s);  // no routing stage on this path
  launch_decode_gemm<FMT, true>(a, ux, a.x, static_cast<const uint8_t*>(a.gu_q), a.gu_s, a.gu_c, s);
  if (ev) (void)hipEventRecord(ev[2], s);
  launch_decode_gemm<FMT, false>(a, ux, a.h, static_cast<const uint8_t*>(a.dn_q), a.dn_s, a.dn_c, s);
  if (ev) (void)hipEventRecord(ev[3], s);
  decode_combine_kernel<<<a.T, kThreads, 0, s>>>(a.y, a.idx, a.K, a.E, a.H, a.out);
  if (ev) (void)hipEventRecord(ev[4], s);
  return hipGetLastError();
}

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
  const int g2 = round_up(mtiles * ((a.H + kG2Rows - 1) / kG2Rows), kXcds);
  const uint8_t* guq = static_cast<const uint8_t*>(a.gu_q);
  const uint8_t* dnq = static_cast<const uint8_t*>(a.dn_q);
  g1_kernel<FMT><<<g1, kThreads, 0, s>>>(a.x, a.K, a.E, a.H, a.I, guq, a.gu_s, a.gu_c, a.rb.offsets,
                                         a.rb.tile_start, a.rb.perm, a.h, nullptr);
  if (ev) (void)hipEventRecord(ev[2], s);
  // y rows rounded to bf16 here (the fp32 workspace buffer holds them)
  uint16_t* y16 = reinterpret_cast<uint16_t*>(a.y);
  g2_kernel<FMT, uint16_t><<<g2, kThreads, 0, s>>>(a.h, a.wts, a.E, a.H, a.I, dnq, a.dn_s, a.dn_c, a.rb.offsets,
                                                   a.rb.tile_start, a.rb.perm, y16);
  if (ev) (void)hipEventRecord(ev[3], s);
  combine_kernel<uint16_t><<<a.T, kThreads, 0, s>>>(y16, a.rb.slot, a.K, a.H, a.out);
  if (ev) (void)hipEventRecord(ev[4], s);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_forward(const ForwardArgs& a, hipStream_t s, hipEvent_t const* ev) {
  if (ev) (void)hipEventRecord(ev[0], s);
  return a.T * a.K <= kDecodeMax ? launch_decode<FMT>(a, s, ev) : launch_tiled<FMT>(a, s, ev);
}

template <int FMT>
hipError_t launch_backward(const BackwardArgs& a, hipStream_t s) {
  const int32_t n = a.T * a.K;
  hipError_t err = launch_route(a.idx, n, a.E, kBM, a.rb, s);
  if (err != hipSuccess) return err;
  const int mtiles = (n + kBM - 1) / kBM + a.E;
  const int g1 = round_up(mtiles * ((a.I + kG1Cols - 1) / kG1Cols), kXcds);
  const int g2 = round_up(mtiles * ((a.H + kG2Rows - 1) / kG2Rows), kXcds);
  const int t1 = round_up(mtiles * ((a.I + kTcols - 1) / kTcols), kXcds);
  const int t2 = round_up(mtiles * ((a.H + kTcols - 1) / kTcols), kXcds);
  const uint8_t* guq = static_cast<const uint8_t*>(a.gu_q);
  const uint8_t* dnq = static_cast<const uint8_t*>(a.dn_q);
  const RouteBuffers& r = a.rb;
  g1_kernel<FMT><<<g1, kThreads, 0, s>>>(a.x, a.K, a.E, a.H, a.I, guq, a.gu_s, a.gu_c, r.offsets, r.tile_start,
                                         r.perm, a.h, a.gu_save);
  g2_kernel<FMT, float><<<g2, kThreads, 0, s>>>(a.h, nullptr, a.E, a.H, a.I, dnq, a.dn_s, a.dn_c, r.offsets,
                                                r.tile_start, r.perm, a.zdx);
  gradw_kernel<<<(n + kWaves - 1) / kWaves, kThreads, 0, s>>>(a.dout, a.zdx, r.slot, n, a.K, a.H, a.grad_w);
  tgemm_kernel<FMT, 1><<<t1, kThreads, 0, s>>>(a.dout, a.K, a.E, a.H, a.I, dnq, a.dn_s, a.dn_c, r.offsets,
                                               r.tile_start, r.perm, a.wts, a.gu_save, a.dgu);
  tgemm_kernel<FMT, 2><<<t2, kThreads, 0, s>>>(a.dgu, a.K, a.E, 2 * a.I, a.H, guq, a.gu_s, a.gu_c, r.offsets,
                                               r.tile_start, r.perm, nullptr, nullptr, a.zdx);
  combine_kernel<float><<<a.T, kThreads, 0, s>>>(a.zdx, r.slot, a.K, a.H, a.grad_x);
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
