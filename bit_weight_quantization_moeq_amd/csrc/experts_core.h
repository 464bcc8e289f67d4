// Shared device code of the experts kernels (gfx950): operand types, the
// packed-format loads and in-register dequantization, the tiled-GEMM core
// (the token-tile DMA pipeline and the MFMA K step) and the work-item order.
// Included by experts.hip (tiled forward, backward) and decode.hip
// (few-assignment forward); everything here has internal linkage.
#pragma once
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

// Few-assignment path bound: n = T*K at most this takes the decode kernels.
constexpr int kDecodeMax = 512;

// LDS-only barrier: waits for this wave's LDS traffic, not for its global loads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

int round_up(int x, int m) { return (x + m - 1) / m * m; }

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

}  // namespace
}  // namespace moeq
