// Quantize-on-load and dequantize kernels for fused expert tensors (gfx950).
//
// NF4: blockwise absmax over 64 consecutive in_features elements, nearest of
// the 16 NF4 levels, two codes per byte ("MoE Expert Quantization",
// Implementation details; bitsandbytes issue #1849, maintainer thread).
// int8: row-wise absmax, scale absmax/127 ("MoE Expert Quantization",
// Implementation details).
//
// NF4 with double-quantized absmax: the block absmax is itself stored as an
// 8-bit code per block plus one fp32 scale per group of 256 blocks of one
// expert (bitsandbytes issue #1849, Reproduction and maintainer thread:
// double quantization of the statistics; the format is the library's own).
//
// All kernels are HBM-streaming: a 64-block or a row is read once with
// 16-byte loads, reduced across lanes with DPP, and written once.  Since a
// 64-block never straddles a row or an expert, an NF4 tensor is a flat array
// of independent blocks and the plain kernels ignore E/rows/cols entirely;
// the double-quantized ones work per group (one workgroup each).
#include "moeq_internal.h"

namespace moeq {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950), packed.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads: each byte is read once, so bypass cache retention.
__device__ __forceinline__ uint4 ld_stream16(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ld_stream8(const uint2* p) {
  const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(v.x, v.y);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// max over each group of 8 consecutive lanes: quad xor-1, quad xor-2, then
// the half-row mirror exchanges the two quads of the group.
__device__ __forceinline__ float group8_max(float m) {
  m = fmaxf(m, dpp<0xB1>(m));   // quad_perm [1,0,3,2]
  m = fmaxf(m, dpp<0x4E>(m));   // quad_perm [2,3,0,1]
  m = fmaxf(m, dpp<0x141>(m));  // row_half_mirror
  return m;
}

__device__ __forceinline__ float wave_max(float m) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// ---------------------------------------------------------------------------
// NF4 quantize.  Eight lanes own one 64-block (8 bf16 = 16 B each); a wave
// covers 8 consecutive blocks (1 KB) per step and keeps kUnroll steps of
// loads in flight.
// ---------------------------------------------------------------------------
constexpr int kNf4Unroll = 4;

__device__ __forceinline__ uint2 nf4_bucket_entry(int j) {
  const float lo = (float)(j - 17) * 0.0625f;
  const float hi = lo + 0.0625f;
  float thr = 2.0f;  // no threshold in this bucket: the test below is never true
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < 15; ++i) {
    const float t = __uint_as_float(kNf4ThresholdBits[i]);
    base += (t < lo) ? 1u : 0u;
    thr = (t >= lo && t < hi) ? t : thr;
  }
  return make_uint2(__float_as_uint(thr), base);
}

// Code of w in a block with absmax a (a > 0, not tiny): the bucket comes from
// an approximate ratio w * (16/a); the code is the bucket's count of lower
// thresholds plus one exact test w >= a * t (fma(a, t, -w) <= 0 has the sign
// of the exact a*t - w because no underflow is possible for a >= 2^-90).
__device__ __forceinline__ uint32_t nf4_code(float w, float a, float r16, const uint2* tab) {
  const int j = min(max((int)__builtin_fmaf(w, r16, 17.0f), 0), kNf4Buckets - 1);
  const uint2 e = tab[j];
  return e.y + ((__builtin_fmaf(a, __uint_as_float(e.x), -w) <= 0.0f) ? 1u : 0u);
}

// One 64-block per 8 lanes: v holds this lane's 8 consecutive bf16 of the
// block.  Returns the lane's 8 codes as one word (column 2m in the high
// nibble of byte m) and sets a to the block absmax (the same in all 8 lanes).
// Every lane of the wave must call it (the sub-2^-90 rescue votes).
__device__ __forceinline__ uint32_t nf4_block_word(uint4 v, const uint2* tab, float& a_out) {
  float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  float m = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  m = fmaxf(m, fmaxf(fmaxf(fabsf(x[4]), fabsf(x[5])), fmaxf(fabsf(x[6]), fabsf(x[7]))));
  const float a = group8_max(m);

  // Blocks whose absmax is below 2^-90 (rare: denormal-range weights) are
  // scaled by 2^100 first, which is exact and leaves every ratio unchanged.
  float ae = a;
  if (__any(a > 0.0f && a < 0x1p-90f)) {
    const float sc = (a > 0.0f && a < 0x1p-90f) ? 0x1p100f : 1.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] *= sc;
    ae = a * sc;
  }
  ae = (a == 0.0f) ? 1.0f : ae;  // all-zero block: every w is +-0 -> code 7
  const float r16 = 16.0f * __builtin_amdgcn_rcpf(ae);

  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    const uint32_t hi = nf4_code(x[k], ae, r16, tab);
    const uint32_t lo = nf4_code(x[k + 1], ae, r16, tab);
    word |= ((hi << 4) | lo) << (4 * k);
  }
  a_out = a;
  return word;
}

__global__ __launch_bounds__(kThreads) void nf4_quantize_kernel(const uint4* __restrict__ w,
                                                               uint32_t* __restrict__ q,
                                                               float* __restrict__ absmax,
                                                               int64_t nblocks) {
  __shared__ uint2 tab[kNf4Buckets];
  if (threadIdx.x < kNf4Buckets) tab[threadIdx.x] = nf4_bucket_entry(threadIdx.x);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;   // 16-byte slice of the block
  const int grp = lane >> 3;  // block within the wave's 8
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  constexpr int kPerWave = 8 * kNf4Unroll;

  for (int64_t base = wave * kPerWave; base < nblocks; base += nwaves * kPerWave) {
    uint4 v[kNf4Unroll];
#pragma unroll
    for (int u = 0; u < kNf4Unroll; ++u) {
      int64_t b = base + u * 8 + grp;
      b = b < nblocks ? b : nblocks - 1;  // clamp: every lane loads, only valid ones store
      v[u] = ld_stream16(&w[b * 8 + sub]);
    }
#pragma unroll
    for (int u = 0; u < kNf4Unroll; ++u) {
      const int64_t b = base + u * 8 + grp;
      float a;
      const uint32_t word = nf4_block_word(v[u], tab, a);
      if (b < nblocks) {
        q[b * 8 + sub] = word;
        if (sub == 0) absmax[b] = a;
      }
    }
  }
}

// Streaming reference: the launch shape, loads and stores of
// nf4_quantize_kernel (the same 16-byte nontemporal loads of a 64-block by 8
// lanes, 4 steps in flight, 4 B of codes per lane and 4 B of absmax per
// block) with the code decision replaced by an XOR fold.  Its rate is the
// attainable bandwidth for the quantize kernel's byte mix (2 B read, 0.5625 B
// written per element) and access pattern.
__global__ __launch_bounds__(kThreads) void stream_reference_kernel(const uint4* __restrict__ w,
                                                                   uint32_t* __restrict__ q,
                                                                   float* __restrict__ absmax,
                                                                   int64_t nblocks) {
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7, grp = lane >> 3;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  constexpr int kPerWave = 8 * kNf4Unroll;
  for (int64_t base = wave * kPerWave; base < nblocks; base += nwaves * kPerWave) {
    uint4 v[kNf4Unroll];
#pragma unroll
    for (int u = 0; u < kNf4Unroll; ++u) {
      int64_t b = base + u * 8 + grp;
      b = b < nblocks ? b : nblocks - 1;
      v[u] = ld_stream16(&w[b * 8 + sub]);
    }
#pragma unroll
    for (int u = 0; u < kNf4Unroll; ++u) {
      const int64_t b = base + u * 8 + grp;
      const uint32_t word = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      if (b < nblocks) {
        q[b * 8 + sub] = word;
        if (sub == 0) absmax[b] = __uint_as_float(word & 0x3fffffffu);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Double-quantized absmax: one workgroup per group of (at most) 256
// consecutive blocks of one expert.  Thread t owns block t of the group: the
// group maximum m comes from a wave reduction and 4 LDS partials, then
// s2 = fp32(m / 255) and c = rint(fp32(fp32(255 a) / m)) (IEEE division,
// round half to even), exactly the row-wise int8 rule with 255 levels.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void dq_group_encode(float a, int cnt, uint8_t* codes, float* gscale) {
  __shared__ float part[kThreads / 64];
  const int t = threadIdx.x;
  const float m0 = wave_max(t < cnt ? a : 0.0f);
  if ((t & 63) == 0) part[t >> 6] = m0;
  __syncthreads();
  const float m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  if (t < cnt) codes[t] = (m > 0.0f) ? (uint8_t)__builtin_rintf((a * 255.0f) / m) : (uint8_t)0;
  if (t == 0) *gscale = m / 255.0f;
}

// NF4 quantize writing double-quantized absmax: wave w of the group's
// workgroup quantizes blocks 64w .. 64w + 63 (8 per step, 4 steps of loads
// in flight), keeping each absmax in LDS for the group encode.
__global__ __launch_bounds__(kThreads) void nf4dq_quantize_kernel(const uint4* __restrict__ w,
                                                                 uint32_t* __restrict__ q,
                                                                 uint8_t* __restrict__ codes,
                                                                 float* __restrict__ gscale, int64_t nb,
                                                                 int32_t ng) {
  __shared__ uint2 tab[kNf4Buckets];
  __shared__ float sa[MOEQ_DQ_GROUP];
  if (threadIdx.x < kNf4Buckets) tab[threadIdx.x] = nf4_bucket_entry(threadIdx.x);
  __syncthreads();
  const int e = blockIdx.x / ng, g = blockIdx.x - e * ng;
  const int64_t first = (int64_t)e * nb + (int64_t)g * MOEQ_DQ_GROUP;  // first block of the group
  const int cnt = (int)min<int64_t>(MOEQ_DQ_GROUP, nb - (int64_t)g * MOEQ_DQ_GROUP);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & 7, grp = lane >> 3;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    uint4 v[kNf4Unroll];
#pragma unroll
    for (int u = 0; u < kNf4Unroll; ++u) {
      int j = 64 * wave + 32 * half + 8 * u + grp;  // block within the group
      j = j < cnt ? j : cnt - 1;                    // clamp: every lane loads, only valid ones store
      v[u] = ld_stream16(&w[(first + j) * 8 + sub]);
    }
#pragma unroll
    for (int u = 0; u < kNf4Unroll; ++u) {
      const int j = 64 * wave + 32 * half + 8 * u + grp;
      float a;
      const uint32_t word = nf4_block_word(v[u], tab, a);
      if (j < cnt) {
        q[(first + j) * 8 + sub] = word;
        if (sub == 0) sa[j] = a;
      }
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  dq_group_encode(t < cnt ? sa[t] : 0.0f, cnt, codes + first, gscale + (int64_t)e * ng + g);
}

// Double-quantize existing fp32 absmax [E][nb].
__global__ __launch_bounds__(kThreads) void dq_compress_kernel(const float* __restrict__ absmax,
                                                              uint8_t* __restrict__ codes,
                                                              float* __restrict__ gscale, int64_t nb, int32_t ng) {
  const int e = blockIdx.x / ng, g = blockIdx.x - e * ng;
  const int64_t first = (int64_t)e * nb + (int64_t)g * MOEQ_DQ_GROUP;
  const int cnt = (int)min<int64_t>(MOEQ_DQ_GROUP, nb - (int64_t)g * MOEQ_DQ_GROUP);
  const int t = threadIdx.x;
  dq_group_encode(t < cnt ? absmax[first + t] : 0.0f, cnt, codes + first, gscale + (int64_t)e * ng + g);
}

// ---------------------------------------------------------------------------
// int8 row-wise quantize: one wave per row.  Rows of up to 64*kRowChunks*8
// elements stay in registers between the absmax pass and the code pass;
// longer rows are re-read (from L2) for the code pass.
// ---------------------------------------------------------------------------
constexpr int kRowChunks = 8;

__device__ __forceinline__ uint32_t i8_code(float w, float a) {
  // q = round_half_even(fp32(fp32(127 w) / a)); 127 w is exact for bf16 w.
  const float r = __builtin_rintf((w * 127.0f) / a);
  return (uint32_t)((int32_t)r) & 0xffu;
}

__device__ __forceinline__ uint2 i8_codes8(uint4 v, float a) {
  if (a == 0.0f) return make_uint2(0u, 0u);
  const uint32_t c0 = i8_code(bf16_lo(v.x), a), c1 = i8_code(bf16_hi(v.x), a);
  const uint32_t c2 = i8_code(bf16_lo(v.y), a), c3 = i8_code(bf16_hi(v.y), a);
  const uint32_t c4 = i8_code(bf16_lo(v.z), a), c5 = i8_code(bf16_hi(v.z), a);
  const uint32_t c6 = i8_code(bf16_lo(v.w), a), c7 = i8_code(bf16_hi(v.w), a);
  return make_uint2(c0 | (c1 << 8) | (c2 << 16) | (c3 << 24), c4 | (c5 << 8) | (c6 << 16) | (c7 << 24));
}

__device__ __forceinline__ float absmax8(uint4 v) {
  float r = fmaxf(fmaxf(fabsf(bf16_lo(v.x)), fabsf(bf16_hi(v.x))), fmaxf(fabsf(bf16_lo(v.y)), fabsf(bf16_hi(v.y))));
  r = fmaxf(r, fmaxf(fmaxf(fabsf(bf16_lo(v.z)), fabsf(bf16_hi(v.z))), fmaxf(fabsf(bf16_lo(v.w)), fabsf(bf16_hi(v.w)))));
  return r;
}

__global__ __launch_bounds__(kThreads) void int8_quantize_kernel(const uint16_t* __restrict__ w,
                                                                uint8_t* __restrict__ q,
                                                                float* __restrict__ scale,
                                                                int64_t nrows, int32_t cols) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int nch = cols >> 3;  // 8-element chunks per row (cols % 8 == 0)

  for (int64_t row = wave; row < nrows; row += nwaves) {
    const uint4* wr = reinterpret_cast<const uint4*>(w + row * cols);
    uint2* qr = reinterpret_cast<uint2*>(q + row * cols);
    uint4 v[kRowChunks];
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) {
      const int c = lane + 64 * i;
      v[i] = (c < nch) ? ld_stream16(&wr[c]) : make_uint4(0, 0, 0, 0);
      m = fmaxf(m, absmax8(v[i]));
    }
    for (int c = lane + 64 * kRowChunks; c < nch; c += 64) m = fmaxf(m, absmax8(wr[c]));
    const float a = wave_max(m);
    if (lane == 0) scale[row] = a / 127.0f;
#pragma unroll
    for (int i = 0; i < kRowChunks; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) qr[c] = i8_codes8(v[i], a);
    }
    for (int c = lane + 64 * kRowChunks; c < nch; c += 64) qr[c] = i8_codes8(wr[c], a);
  }
}

// ---------------------------------------------------------------------------
// Dequantize: bf16_rne(fp32(level[code] * absmax)) / bf16_rne(fp32(q * scale)).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void nf4_dequantize_kernel(const uint32_t* __restrict__ q,
                                                                 const float* __restrict__ absmax,
                                                                 uint4* __restrict__ out,
                                                                 int64_t nwords) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = __uint_as_float(kNf4LevelBits[threadIdx.x]);
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x; d < nwords; d += stride) {
    const uint32_t c = __builtin_nontemporal_load(&q[d]);
    const float a = absmax[d >> 3];  // 8 words of codes per 64-block
    float v[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t byte = (c >> (8 * m)) & 0xffu;
      v[2 * m] = lv[byte >> 4] * a;
      v[2 * m + 1] = lv[byte & 0xfu] * a;
    }
    out[d] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                        pack_bf16x2(v[6], v[7]));
  }
}

// NF4 with double-quantized absmax: one workgroup per group; the group
// scale is read once and absmax' = fp32(c * s2) per block.
__global__ __launch_bounds__(kThreads) void nf4dq_dequantize_kernel(const uint32_t* __restrict__ q,
                                                                   const uint8_t* __restrict__ codes,
                                                                   const float* __restrict__ gscale,
                                                                   uint4* __restrict__ out, int64_t nb,
                                                                   int32_t ng) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = __uint_as_float(kNf4LevelBits[threadIdx.x]);
  __syncthreads();
  const int e = blockIdx.x / ng, g = blockIdx.x - e * ng;
  const int64_t first = (int64_t)e * nb + (int64_t)g * MOEQ_DQ_GROUP;
  const int cnt = (int)min<int64_t>(MOEQ_DQ_GROUP, nb - (int64_t)g * MOEQ_DQ_GROUP);
  const float s2 = gscale[(int64_t)e * ng + g];
  for (int i = threadIdx.x; i < 8 * cnt; i += kThreads) {  // 8 words of codes per block
    const int64_t d = first * 8 + i;
    const uint32_t c = __builtin_nontemporal_load(&q[d]);
    const float a = (float)codes[first + (i >> 3)] * s2;
    float v[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t byte = (c >> (8 * m)) & 0xffu;
      v[2 * m] = lv[byte >> 4] * a;
      v[2 * m + 1] = lv[byte & 0xfu] * a;
    }
    out[d] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                        pack_bf16x2(v[6], v[7]));
  }
}

__global__ __launch_bounds__(kThreads) void int8_dequantize_kernel(const uint2* __restrict__ q,
                                                                  const float* __restrict__ scale,
                                                                  uint4* __restrict__ out,
                                                                  int64_t nchunks, int32_t chunks_per_row) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks; c += stride) {
    const uint2 v = ld_stream8(&q[c]);
    const float s = scale[c / chunks_per_row];
    float f[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[k] = (float)(int8_t)((v.x >> (8 * k)) & 0xffu) * s;
      f[4 + k] = (float)(int8_t)((v.y >> (8 * k)) & 0xffu) * s;
    }
    out[c] = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                        pack_bf16x2(f[6], f[7]));
  }
}

int grid_for(int64_t items, int64_t per_block, int64_t cap) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

}  // namespace

hipError_t launch_quantize_nf4(const uint16_t* w, uint8_t* q, float* absmax, int64_t nblocks,
                               hipStream_t s) {
  const int grid = grid_for(nblocks, (kThreads / 64) * 8 * kNf4Unroll, 8192);
  nf4_quantize_kernel<<<grid, kThreads, 0, s>>>(reinterpret_cast<const uint4*>(w),
                                                 reinterpret_cast<uint32_t*>(q), absmax, nblocks);
  return hipGetLastError();
}

hipError_t launch_stream_reference(const uint16_t* w, uint8_t* q, float* absmax, int64_t nblocks, hipStream_t s) {
  const int grid = grid_for(nblocks, (kThreads / 64) * 8 * kNf4Unroll, 8192);
  stream_reference_kernel<<<grid, kThreads, 0, s>>>(reinterpret_cast<const uint4*>(w),
                                                     reinterpret_cast<uint32_t*>(q), absmax, nblocks);
  return hipGetLastError();
}

hipError_t launch_quantize_int8(const uint16_t* w, int8_t* q, float* scale, int64_t nrows,
                                int32_t cols, hipStream_t s) {
  const int grid = grid_for(nrows, kThreads / 64, 16384);
  int8_quantize_kernel<<<grid, kThreads, 0, s>>>(w, reinterpret_cast<uint8_t*>(q), scale, nrows, cols);
  return hipGetLastError();
}

hipError_t launch_dequantize_nf4(const uint8_t* q, const float* absmax, uint16_t* out,
                                 int64_t nblocks, hipStream_t s) {
  const int64_t nwords = nblocks * 8;
  const int grid = grid_for(nwords, kThreads, 16384);
  nf4_dequantize_kernel<<<grid, kThreads, 0, s>>>(reinterpret_cast<const uint32_t*>(q), absmax,
                                                   reinterpret_cast<uint4*>(out), nwords);
  return hipGetLastError();
}

hipError_t launch_dequantize_int8(const int8_t* q, const float* scale, uint16_t* out,
                                  int64_t nrows, int32_t cols, hipStream_t s) {
  const int32_t cpr = cols / 8;
  const int64_t nchunks = nrows * cpr;
  const int grid = grid_for(nchunks, kThreads, 16384);
  int8_dequantize_kernel<<<grid, kThreads, 0, s>>>(reinterpret_cast<const uint2*>(q), scale,
                                                    reinterpret_cast<uint4*>(out), nchunks, cpr);
  return hipGetLastError();
}

hipError_t launch_quantize_nf4_dq(const uint16_t* w, uint8_t* q, uint8_t* codes, float* gscale, int32_t E,
                                  int64_t nb, hipStream_t s) {
  const int32_t ng = (int32_t)dq_groups(nb);
  nf4dq_quantize_kernel<<<(unsigned)E * ng, kThreads, 0, s>>>(reinterpret_cast<const uint4*>(w),
                                                               reinterpret_cast<uint32_t*>(q), codes, gscale, nb, ng);
  return hipGetLastError();
}

hipError_t launch_compress_absmax(const float* absmax, uint8_t* codes, float* gscale, int32_t E, int64_t nb,
                                  hipStream_t s) {
  const int32_t ng = (int32_t)dq_groups(nb);
  dq_compress_kernel<<<(unsigned)E * ng, kThreads, 0, s>>>(absmax, codes, gscale, nb, ng);
  return hipGetLastError();
}

hipError_t launch_dequantize_nf4_dq(const uint8_t* q, const uint8_t* codes, const float* gscale, uint16_t* out,
                                    int32_t E, int64_t nb, hipStream_t s) {
  const int32_t ng = (int32_t)dq_groups(nb);
  nf4dq_dequantize_kernel<<<(unsigned)E * ng, kThreads, 0, s>>>(reinterpret_cast<const uint32_t*>(q), codes, gscale,
                                                                 reinterpret_cast<uint4*>(out), nb, ng);
  return hipGetLastError();
}

}  // namespace moeq
