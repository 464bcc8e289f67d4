// Few-assignment (decode) path of the routed experts forward (gfx950): the
// gate_up and down launches and the k-ordered combine for n = T*K <= 512
// assignments, straight from packed NF4 / int8 storage.
//
// out[t] = sum_k w[t,k] * down[e] @ (silu(gate[e] x_t) * up[e] x_t), e = idx[t,k]
// (bitsandbytes issue #1849, Description: gate_up_proj [E, 2I, H],
// down_proj [E, H, I], act_fn between them; unsloth-zoo issue #850,
// Suggested fix: the (hidden_states, top_k_index, top_k_weights) interface).
#include <algorithm>

#include "experts_core.h"

namespace moeq {
namespace {

// ---------------------------------------------------------------------------
// Decode path (few assignments, T*K <= kDecodeMax): no routing kernels and
// no token tiles.  A workgroup owns one touched expert (its blockIdx.x-th, in
// expert order) and RB row blocks of 64 weight rows; it finds the expert and
// the expert's assignments itself from top_k_index (ascending assignment
// order).  The assignments go in groups of 32 (one MFMA's columns).  In a
// batch of more than 32 tokens an expert can hold several groups (skewed
// routing); then that workgroup takes the first group only, and the grid
// carries T*K/32 more workgroups (an upper bound on the later groups of all
// experts), the i-th of which takes the i-th later group in expert order, so
// the groups run side by side instead of one after the other.  Its NW waves
// are RB row blocks x P parts of K (NW = RB * P, P chosen on the host so that
// few touched experts still fill the chip).  Each
// wave streams its part of its 64 rows' packed codes straight from HBM,
// dequantizes them in registers into the MFMA A operand and multiplies the
// expert's token rows (at most 32 per pass, read from L2 as the B operand).
// The P partial sums of a row block meet in LDS and are added in part order,
// so the result does not depend on timing.  When even P = 4 leaves the chip
// short of waves, the down launch also splits K across workgroups (grid z,
// Z = 2 or 4): each z slice writes its own copy of y, and the combine adds
// the copies in z order.  Rows of h and y are indexed by assignment, so the
// combine needs no slot map.
//   G1 (gate_up): row block = gate rows jcol..+32 and up rows I+jcol..+32,
//                 K = H, B rows x[a / K]; h[a][jcol..+32] = bf16(silu(g) * u).
//   G2 (down):    row block = down rows ncol..+64, K = I, B rows h[a];
//                 y[a][ncol..+64] = w_a * acc.
// ---------------------------------------------------------------------------
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
                                                        uint16_t* __restrict__ hout, float* __restrict__ yout,
                                                        int32_t nmain) {
  constexpr int kT = NW * 64;
  constexpr int kJ = kDecodeMax / kT;  // assignments per thread
  constexpr int kStep = Fmt<FMT>::kStep;
  constexpr int kS = kStep / 16;
  __shared__ uint32_t bits[MOEQ_MAX_EXPERTS / 32];
  __shared__ int ecnt[MOEQ_MAX_EXPERTS];  // assignments per expert (later-group workgroups only)
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

  // 2. this block's expert: the blockIdx.x-th touched one (every wave finds
  //    it), and its first token group; or, for blockIdx.x >= nmain, the
  //    (blockIdx.x - nmain)-th later group (groups 1, 2, ... of the experts
  //    holding more than 32 assignments, in expert order)
  int e = -1, gfirst = 0;
  const int xb = (int)blockIdx.x - nmain;
  if (xb < 0) {
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
  } else {
    for (int i = t; i < E; i += kT) ecnt[i] = 0;
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (my[j] >= 0 && my[j] < E) atomicAdd(&ecnt[my[j]], 1);
    lds_barrier();
    // lane l covers experts 16 l .. 16 l + 15 (E <= 1024): its later groups,
    // then an inclusive scan over the lanes
    constexpr int kPer = MOEQ_MAX_EXPERTS / 64;
    int loc = 0;
    for (int i = 0; i < kPer; ++i) {
      const int ex = kPer * lane + i;
      const int c = ex < E ? ecnt[ex] : 0;
      loc += c > 32 ? (c - 1) / 32 : 0;
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(inc, o, 64);
      if (lane >= o) inc += v;
    }
    const uint64_t who = __ballot((inc - loc) <= xb && xb < inc);
    if (who) {
      const int src = __builtin_ctzll(who);
      int r = xb - (__shfl(inc, src, 64) - __shfl(loc, src, 64));  // rank within the lane's experts
      for (int i = 0; i < kPer; ++i) {
        const int ex = kPer * src + i;
        const int c = ex < E ? ecnt[ex] : 0;
        const int ng = c > 32 ? (c - 1) / 32 : 0;
        if (r < ng) {
          e = ex;
          gfirst = 32 * (1 + r);
          break;
        }
        r -= ng;
      }
    }
    e = __builtin_amdgcn_readfirstlane(e);
    gfirst = __builtin_amdgcn_readfirstlane(gfirst);
  }
  if (e < 0) return;  // the whole block: the bitmap is shared

  // 3. this wave's row block and part of K; start its first codes now
  const int K = G1 ? H : I;
  const int nrb = G1 ? I / 32 : H / 64;  // row blocks of the expert
  const int RB = NW / P;
  const int rbi = blockIdx.y * RB + wave / P, part = wave % P;
  // K is split into PZ = P * gridDim.z parts: P within the workgroup (their
  // sums added in LDS below) times gridDim.z across workgroups (each writing
  // its own slice of y, added by the combine)
  const int PZ = P * (int)gridDim.z, zpart = (int)blockIdx.z * P + part;
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
  // 1024 and the PZ parts split the steps into equal eights (the condition
  // under which the host picks AB = 8), else pairs.  The split depends on
  // the shape only, not on AB, so every format sums the same parts.
  constexpr int kTrip = AB == 8 ? 8 : 2;  // steps per loop trip
  constexpr bool PAIR = AB == 2;
  const int nks = (K + kStep - 1) / kStep;
  const int gran = (K % 1024 == 0 && nks % (8 * PZ) == 0) ? 8 : 2;
  const int nkp = (nks + gran - 1) / gran;  // groups of steps
  const int ks0 = gran * (zpart * nkp / PZ), ks1 = min(gran * ((zpart + 1) * nkp / PZ), nks);
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
  if (gfirst == 0) {  // a later group's workgroup fetches in the group loop
    fetch_step(ca0, ca1, ks0);
    fetch_pair(ks0);
    fetch_oct(ks0);
  }

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

  // one group per workgroup when later groups have their own workgroups
  const int gend = (int)gridDim.x > nmain ? min(ne, gfirst + 32) : ne;
  for (int g = gfirst; g < gend; g += 32) {
    const int tok = g + l32 < ne ? g + l32 : g;  // lanes past the tokens repeat one (never stored)
    const int a = list[tok];
    const uint16_t* brow = G1 ? act + (int64_t)(a / Ktop) * H : act + (int64_t)a * I;
    if (g > 0) {  // not prefetched above
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
        float* yp = yout + ((int64_t)blockIdx.z * n + a) * H + col0 + 4 * hh;
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
// unrouted assignments, where y[a] is the sum over z in order of the Z slices
// y_z[a] (the down launch's parts of K across workgroups; Z = 1, 2 or 4).
// One workgroup per token; each thread keeps 8 y loads (8 / Z assignments) in
// flight at once.  y rows are indexed by assignment and lie in the workspace
// whether or not the assignment is routed, so the loads do not wait for the
// routing entries (uniform scalar loads, read alongside): an unrouted
// assignment's row, never written, is loaded and left out of the sum.
__global__ __launch_bounds__(kThreads) void decode_combine_kernel(const float* __restrict__ y,
                                                                 const int32_t* __restrict__ idx, int32_t K,
                                                                 int32_t E, int32_t H, int32_t zlog,
                                                                 int64_t zstride, uint16_t* __restrict__ out) {
  const int64_t tok = blockIdx.x;
  const int Z = 1 << zlog, kc = 8 >> zlog;
  for (int n4 = threadIdx.x; n4 < H / 4; n4 += kThreads) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k0 = 0; k0 < K; k0 += kc) {
      bool use[8];
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + (u >> zlog), z = u & (Z - 1);
        const bool in = (u >> zlog) < kc && k < K;
        const int e = in ? idx[tok * K + k] : -1;
        use[u] = in && e >= 0 && e < E;
        v[u] = in ? *reinterpret_cast<const float4*>(y + z * zstride + (tok * K + k) * H + 4 * n4)
                  : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      float4 sk = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int z = u & (Z - 1);
        if (z == 0) {
          sk = v[u];
        } else {
          sk.x += v[u].x; sk.y += v[u].y; sk.z += v[u].z; sk.w += v[u].w;
        }
        if (z == Z - 1 && use[u]) {
          acc.x += sk.x; acc.y += sk.y; acc.z += sk.z; acc.w += sk.w;
        }
      }
    }
    *reinterpret_cast<uint2*>(out + tok * H + 4 * n4) =
        make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

}  // namespace

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

// Parts of K across workgroups (grid z) for the down launch: when even P = 4
// leaves the chip short of waves (few touched experts, e.g. one token of a
// top-2 layer), K is split further, 2 or 4 ways, while every part keeps at
// least a pair of K steps (counted in 128-wide steps for every format, so
// that the workspace size depends on the shape alone).
int decode_z(int ux, int nrb, int p, int64_t I) {
  const int nkp = (int)((I / 128 + 1) / 2);
  int z = 1;
  while (p == kWaves && z < 4 && (long)ux * nrb * p * z < 1536 && p * z * 2 <= nkp) z *= 2;
  return z;
}

template <int FMT, bool G1>
void launch_decode_gemm(const ForwardArgs& a, int ux, const uint16_t* act, const uint8_t* q, const float* sc,
                        const uint8_t* scc, hipStream_t s) {
  const int32_t n = a.T * a.K;
  const DecodeShape d = decode_shape(ux, G1 ? a.I / 32 : a.H / 64);
  const int z = G1 ? 1 : decode_z(ux, a.H / 64, d.p, a.I);
  const int pz = d.p * z;
  // plain NF4 absmax: in eights when the parts are equal whole eights of K
  // steps (K a multiple of 1024, so the 16-byte chunk loads are aligned and
  // in the row; the kernel splits K the same way), else in pairs when the
  // row holds an even number of blocks
  const int Kr = G1 ? a.H : a.I;
  int ab = 0;
  if constexpr (FMT == MOEQ_FMT_NF4)
    ab = (Kr % 1024 == 0 && (Kr / 128) % (8 * pz) == 0) ? 8 : ((Kr / kNf4Block) % 2 == 0 ? 2 : 0);
  // an expert holds at most T assignments, so more than one group of 32 only
  // when T > 32: then n / 32 more workgroups take the later groups
  const int extra = a.T > 32 ? n / 32 : 0;
  const dim3 grid(ux + extra, d.gy, z);
  if (ab == 8)
    decode_kernel<FMT, G1, kWaves, FMT == MOEQ_FMT_NF4 ? 8 : 0><<<grid, kThreads, 0, s>>>(
        act, a.idx, a.wts, n, a.K, a.E, a.H, a.I, d.p, q, sc, scc, a.h, a.y, ux);
  else if (ab == 2)
    decode_kernel<FMT, G1, kWaves, FMT == MOEQ_FMT_NF4 ? 2 : 0><<<grid, kThreads, 0, s>>>(
        act, a.idx, a.wts, n, a.K, a.E, a.H, a.I, d.p, q, sc, scc, a.h, a.y, ux);
  else
    decode_kernel<FMT, G1, kWaves, 0><<<grid, kThreads, 0, s>>>(
        act, a.idx, a.wts, n, a.K, a.E, a.H, a.I, d.p, q, sc, scc, a.h, a.y, ux);
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
  const int z = decode_down_splits(n, a.E, a.H, a.I);
  decode_combine_kernel<<<a.T, kThreads, 0, s>>>(a.y, a.idx, a.K, a.E, a.H, z == 4 ? 2 : (z == 2 ? 1 : 0),
                                                 (int64_t)n * a.H, a.out);
  if (ev) (void)hipEventRecord(ev[4], s);
  return hipGetLastError();
}

int decode_down_splits(int64_t n, int32_t E, int64_t H, int64_t I) {
  if (n > kDecodeMax || n < 1) return 1;
  const int ux = E < n ? E : (int)n;
  return decode_z(ux, (int)(H / 64), decode_shape(ux, (int)(H / 64)).p, I);
}

hipError_t launch_experts_decode(const ForwardArgs& a, hipStream_t s, hipEvent_t const* ev) {
  switch (a.format) {
    case MOEQ_FMT_NF4: return launch_decode<MOEQ_FMT_NF4>(a, s, ev);
    case MOEQ_FMT_NF4_DQ: return launch_decode<MOEQ_FMT_NF4_DQ>(a, s, ev);
    default: return launch_decode<MOEQ_FMT_INT8_ROWWISE>(a, s, ev);
  }
}

}  // namespace moeq
