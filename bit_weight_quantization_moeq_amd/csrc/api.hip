// C ABI of libmoeq: host-side validation, workspace layout and dispatch.
// Every check runs before the first HIP call, so a rejected call has no side
// effect; nothing is ever skipped silently (the silent-skip and
// packed-uint8-reaches-float-kernel failures described in bitsandbytes issue
// #1849 and unsloth-zoo issue #850 are what these checks exist to prevent).
#include <string.h>

#include <mutex>

#include "moeq_internal.h"

using namespace moeq;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape / format validation of one qweight descriptor.
bool nf4_codes(int32_t format) { return format == MOEQ_FMT_NF4 || format == MOEQ_FMT_NF4_DQ; }

moeq_status check_qweight(const moeq_qweight* q, int32_t want_format /* 0 = any */) {
  if (!q) return MOEQ_EINVAL;
  if (q->format != MOEQ_FMT_NF4 && q->format != MOEQ_FMT_INT8_ROWWISE && q->format != MOEQ_FMT_NF4_DQ)
    return MOEQ_EFORMAT;
  if (want_format && q->format != want_format) return MOEQ_EFORMAT;
  if (q->num_experts <= 0 || q->rows <= 0 || q->cols <= 0) return MOEQ_EINVAL;
  if (!q->qdata || !q->scales) return MOEQ_EINVAL;
  // absmax codes exactly when the format has them
  if ((q->format == MOEQ_FMT_NF4_DQ) != (q->scale_codes != nullptr)) return MOEQ_EINVAL;
  if (nf4_codes(q->format)) {
    if (q->blocksize != MOEQ_NF4_BLOCKSIZE || q->cols % MOEQ_NF4_BLOCKSIZE != 0) return MOEQ_EBLOCK;
  } else {
    if (q->blocksize != q->cols) return MOEQ_EBLOCK;
    if (q->cols % 8 != 0) return MOEQ_ESHAPE;
  }
  if (!aligned16(q->qdata) || !aligned16(q->scales)) return MOEQ_EALIGN;
  if (q->scale_codes && !aligned16(q->scale_codes)) return MOEQ_EALIGN;
  return MOEQ_OK;
}

int64_t numel(const moeq_qweight* q) { return (int64_t)q->num_experts * q->rows * q->cols; }

// NF4 blocks per expert
int64_t blocks_per_expert(const moeq_qweight* q) { return (int64_t)q->rows * q->cols / kNf4Block; }

// Bytes of codes, fp32 scales and absmax codes of one tensor.
size_t code_bytes(const moeq_qweight* q) { return (size_t)(nf4_codes(q->format) ? numel(q) / 2 : numel(q)); }
size_t scale_bytes(const moeq_qweight* q) {
  const int64_t E = q->num_experts;
  switch (q->format) {
    case MOEQ_FMT_NF4: return sizeof(float) * (size_t)(E * blocks_per_expert(q));
    case MOEQ_FMT_NF4_DQ: return sizeof(float) * (size_t)(E * dq_groups(blocks_per_expert(q)));
    default: return sizeof(float) * (size_t)(E * q->rows);
  }
}
size_t scale_code_bytes(const moeq_qweight* q) {
  return q->format == MOEQ_FMT_NF4_DQ ? (size_t)(q->num_experts * blocks_per_expert(q)) : 0;
}

moeq_status device_status(hipError_t e) { return e == hipSuccess ? MOEQ_OK : MOEQ_EDEVICE; }

constexpr size_t kAlign = 256;
size_t up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Layout {
  size_t chunk_counts, chunk_base, rank, counts, offsets, tile_start, perm, slot, h, y, total;
};

// Workspace carve-up for n = T*K assignments over E experts (h/y only when
// the forward needs them).
Layout layout(int64_t n, int32_t E, int64_t I, int64_t H) {
  Layout L{};
  const int64_t nchunk = route_chunks(n);
  size_t o = 0;
  L.chunk_counts = o; o += up(sizeof(int32_t) * (size_t)(nchunk * E));
  L.chunk_base = o;   o += up(sizeof(int32_t) * (size_t)(nchunk * E));
  L.rank = o;         o += up(sizeof(int32_t) * (size_t)n);
  L.counts = o;       o += up(sizeof(int32_t) * (size_t)E);
  L.offsets = o;      o += up(sizeof(int32_t) * (size_t)(E + 1));
  L.tile_start = o;   o += up(sizeof(int32_t) * (size_t)(E + 1));
  L.perm = o;         o += up(sizeof(int32_t) * (size_t)n);
  L.slot = o;         o += up(sizeof(int32_t) * (size_t)n);
  L.h = o;            o += up(sizeof(uint16_t) * (size_t)(n * I));
  L.y = o;            o += up(sizeof(float) * (size_t)(n * H) * (size_t)decode_down_splits(n, E, H, I));
  L.total = o;
  return L;
}

RouteBuffers route_buffers(void* ws, const Layout& L) {
  char* b = static_cast<char*>(ws);
  RouteBuffers r;
  r.chunk_counts = reinterpret_cast<int32_t*>(b + L.chunk_counts);
  r.chunk_base = reinterpret_cast<int32_t*>(b + L.chunk_base);
  r.rank = reinterpret_cast<int32_t*>(b + L.rank);
  r.counts = reinterpret_cast<int32_t*>(b + L.counts);
  r.offsets = reinterpret_cast<int32_t*>(b + L.offsets);
  r.tile_start = reinterpret_cast<int32_t*>(b + L.tile_start);
  r.perm = reinterpret_cast<int32_t*>(b + L.perm);
  r.slot = reinterpret_cast<int32_t*>(b + L.slot);
  return r;
}

constexpr int64_t kMaxAssignments = int64_t(1) << 24;

// Device-resident scratch for moeq_experts_forward_noalloc: the forward's
// workspace for callers that cannot allocate.  Each GPU the library runs on
// holds its own copy for the life of the process.  Host code never uses the
// array's name as an address (on the host it is only a handle): the device
// address comes from hipGetSymbolAddress, once per device with that device
// current, and is kept per device.
static __device__ __align__(256) unsigned char scratch[MOEQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// The scratch address on the current device (resolved on the first call there).
hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

moeq_status check_forward_shapes(int32_t T, int32_t K, const moeq_qweight* gu, const moeq_qweight* dn) {
  if (T < 0 || K < 1) return MOEQ_EINVAL;
  moeq_status st = check_qweight(gu, 0);
  if (st != MOEQ_OK) return st;
  st = check_qweight(dn, 0);
  if (st != MOEQ_OK) return st;
  if (gu->format != dn->format) return MOEQ_EFORMAT;
  if (gu->num_experts != dn->num_experts) return MOEQ_ESHAPE;
  if (gu->num_experts > MOEQ_MAX_EXPERTS) return MOEQ_ESHAPE;
  if (gu->rows % 2 != 0) return MOEQ_ESHAPE;
  const int32_t I = gu->rows / 2, H = gu->cols;
  if (dn->rows != H || dn->cols != I) return MOEQ_ESHAPE;
  if (H % 64 != 0 || I % 64 != 0) return MOEQ_ESHAPE;
  if ((int64_t)T * K > kMaxAssignments) return MOEQ_ESHAPE;
  // the GEMM kernels address rows of hidden_states with 32-bit byte offsets
  if ((int64_t)T * H * 2 >= (int64_t(1) << 32)) return MOEQ_ESHAPE;
  return MOEQ_OK;
}

}  // namespace

extern "C" {

int32_t moeq_abi_version(void) { return MOEQ_ABI_VERSION; }

const char* moeq_status_string(moeq_status s) {
  switch (s) {
    case MOEQ_OK: return "ok";
    case MOEQ_EINVAL: return "invalid argument (null pointer, non-positive dimension, K < 1, T < 0, or absmax codes given for a format without them)";
    case MOEQ_ESHAPE: return "inconsistent or unsupported shapes";
    case MOEQ_EBLOCK: return "blocksize rule violated (NF4: blocksize 64 and cols % 64 == 0; int8: blocksize == cols)";
    case MOEQ_EFORMAT: return "format tag not what the call needs, or gate_up and down formats differ";
    case MOEQ_EALIGN: return "pointer not 16-byte aligned";
    case MOEQ_EWORKSPACE: return "workspace missing or too small";
    case MOEQ_EDEVICE: return "HIP call failed";
    default: return "unknown status";
  }
}

moeq_status moeq_nf4_codebook(float* out) {
  if (!out) return MOEQ_EINVAL;
  for (int i = 0; i < 16; ++i) memcpy(&out[i], &kNf4LevelBits[i], sizeof(float));
  return MOEQ_OK;
}

moeq_status moeq_quantize_nf4(const uint16_t* w, const moeq_qweight* dst, void* stream) {
  moeq_status st = check_qweight(dst, 0);
  if (st != MOEQ_OK) return st;
  if (!nf4_codes(dst->format)) return MOEQ_EFORMAT;
  if (!w) return MOEQ_EINVAL;
  if (!aligned16(w)) return MOEQ_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dst->format == MOEQ_FMT_NF4_DQ)
    return device_status(launch_quantize_nf4_dq(w, static_cast<uint8_t*>(dst->qdata), dst->scale_codes,
                                                dst->scales, dst->num_experts, blocks_per_expert(dst), s));
  const int64_t nblocks = numel(dst) / kNf4Block;
  return device_status(launch_quantize_nf4(w, static_cast<uint8_t*>(dst->qdata), dst->scales, nblocks, s));
}

moeq_status moeq_stream_reference(const uint16_t* w, const moeq_qweight* dst, void* stream) {
  moeq_status st = check_qweight(dst, MOEQ_FMT_NF4);
  if (st != MOEQ_OK) return st;
  if (!w) return MOEQ_EINVAL;
  if (!aligned16(w)) return MOEQ_EALIGN;
  return device_status(launch_stream_reference(w, static_cast<uint8_t*>(dst->qdata), dst->scales,
                                               numel(dst) / kNf4Block, static_cast<hipStream_t>(stream)));
}

moeq_status moeq_compress_absmax(const moeq_qweight* src, const moeq_qweight* dst, void* stream) {
  moeq_status st = check_qweight(src, MOEQ_FMT_NF4);
  if (st != MOEQ_OK) return st;
  st = check_qweight(dst, MOEQ_FMT_NF4_DQ);
  if (st != MOEQ_OK) return st;
  if (src->num_experts != dst->num_experts || src->rows != dst->rows || src->cols != dst->cols)
    return MOEQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (dst->qdata != src->qdata)
    e = hipMemcpyAsync(dst->qdata, src->qdata, code_bytes(src), hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = launch_compress_absmax(src->scales, dst->scale_codes, dst->scales, src->num_experts,
                               blocks_per_expert(src), s);
  return device_status(e);
}

moeq_status moeq_quantize_int8_rowwise(const uint16_t* w, const moeq_qweight* dst, void* stream) {
  moeq_status st = check_qweight(dst, MOEQ_FMT_INT8_ROWWISE);
  if (st != MOEQ_OK) return st;
  if (!w) return MOEQ_EINVAL;
  if (!aligned16(w)) return MOEQ_EALIGN;
  const int64_t nrows = (int64_t)dst->num_experts * dst->rows;
  return device_status(launch_quantize_int8(w, static_cast<int8_t*>(dst->qdata), dst->scales, nrows,
                                            dst->cols, static_cast<hipStream_t>(stream)));
}

moeq_status moeq_dequantize(const moeq_qweight* src, uint16_t* out, void* stream) {
  moeq_status st = check_qweight(src, 0);
  if (st != MOEQ_OK) return st;
  if (!out) return MOEQ_EINVAL;
  if (!aligned16(out)) return MOEQ_EALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (src->format == MOEQ_FMT_NF4)
    return device_status(launch_dequantize_nf4(static_cast<const uint8_t*>(src->qdata), src->scales, out,
                                               numel(src) / kNf4Block, s));
  if (src->format == MOEQ_FMT_NF4_DQ)
    return device_status(launch_dequantize_nf4_dq(static_cast<const uint8_t*>(src->qdata), src->scale_codes,
                                                  src->scales, out, src->num_experts, blocks_per_expert(src), s));
  return device_status(launch_dequantize_int8(static_cast<const int8_t*>(src->qdata), src->scales, out,
                                              (int64_t)src->num_experts * src->rows, src->cols, s));
}

size_t moeq_experts_forward_workspace_bytes(int32_t T, int32_t K, const moeq_qweight* gu,
                                            const moeq_qweight* dn) {
  if (check_forward_shapes(T, K, gu, dn) != MOEQ_OK) return 0;
  return layout((int64_t)T * K, gu->num_experts, gu->rows / 2, gu->cols).total;
}

moeq_status moeq_experts_forward(const uint16_t* x, const int32_t* idx, const float* wts, int32_t T, int32_t K,
                                 const moeq_qweight* gu, const moeq_qweight* dn, uint16_t* out,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return moeq_experts_forward_timed(x, idx, wts, T, K, gu, dn, out, workspace, workspace_bytes, stream, nullptr);
}

moeq_status moeq_experts_forward_timed(const uint16_t* x, const int32_t* idx, const float* wts, int32_t T,
                                       int32_t K, const moeq_qweight* gu, const moeq_qweight* dn, uint16_t* out,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       void* const* stage_events) {
  moeq_status st = check_forward_shapes(T, K, gu, dn);
  if (st != MOEQ_OK) return st;
  if (T == 0) return MOEQ_OK;
  if (!x || !idx || !wts || !out) return MOEQ_EINVAL;
  if (!aligned16(x) || !aligned16(out)) return MOEQ_EALIGN;
  const int32_t I = gu->rows / 2, H = gu->cols, E = gu->num_experts;
  const Layout L = layout((int64_t)T * K, E, I, H);
  if (!workspace || workspace_bytes < L.total) return MOEQ_EWORKSPACE;
  if (!aligned16(workspace)) return MOEQ_EALIGN;

  ForwardArgs a;
  a.x = x; a.idx = idx; a.wts = wts;
  a.T = T; a.K = K; a.E = E; a.H = H; a.I = I;
  a.format = gu->format;
  a.gu_q = gu->qdata; a.gu_s = gu->scales; a.gu_c = gu->scale_codes;
  a.dn_q = dn->qdata; a.dn_s = dn->scales; a.dn_c = dn->scale_codes;
  a.out = out;
  a.rb = route_buffers(workspace, L);
  a.h = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + L.h);
  a.y = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.y);
  a.routed = false;
  return device_status(launch_experts_forward(a, static_cast<hipStream_t>(stream),
                                             reinterpret_cast<hipEvent_t const*>(stage_events)));
}

moeq_status check_backward_shapes(int32_t T, int32_t K, const moeq_qweight* gu, const moeq_qweight* dn);

moeq_status moeq_experts_forward_save(const uint16_t* x, const int32_t* idx, const float* wts, int32_t T,
                                      int32_t K, const moeq_qweight* gu, const moeq_qweight* dn, uint16_t* out,
                                      float* gu_saved, void* workspace, size_t workspace_bytes, void* stream) {
  // the backward's shape limits, so that what is saved can always be used
  moeq_status st = check_backward_shapes(T, K, gu, dn);
  if (st != MOEQ_OK) return st;
  if (T == 0) return MOEQ_OK;
  if (!x || !idx || !wts || !out || !gu_saved) return MOEQ_EINVAL;
  if (!aligned16(x) || !aligned16(out) || !aligned16(gu_saved)) return MOEQ_EALIGN;
  const int32_t I = gu->rows / 2, H = gu->cols, E = gu->num_experts;
  const Layout L = layout((int64_t)T * K, E, I, H);
  if (!workspace || workspace_bytes < L.total) return MOEQ_EWORKSPACE;
  if (!aligned16(workspace)) return MOEQ_EALIGN;
  ForwardArgs a;
  a.x = x; a.idx = idx; a.wts = wts;
  a.T = T; a.K = K; a.E = E; a.H = H; a.I = I;
  a.format = gu->format;
  a.gu_q = gu->qdata; a.gu_s = gu->scales; a.gu_c = gu->scale_codes;
  a.dn_q = dn->qdata; a.dn_s = dn->scales; a.dn_c = dn->scale_codes;
  a.out = out;
  a.rb = route_buffers(workspace, L);
  a.h = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + L.h);
  a.y = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.y);
  a.routed = false;
  a.gu_save = gu_saved;
  return device_status(launch_experts_forward(a, static_cast<hipStream_t>(stream), nullptr));
}

moeq_status moeq_experts_forward_noalloc(const uint16_t* x, const int32_t* idx, const float* wts, int32_t T,
                                         int32_t K, const moeq_qweight* gu, const moeq_qweight* dn, uint16_t* out,
                                         void* stream) {
  moeq_status st = check_forward_shapes(T, K, gu, dn);
  if (st != MOEQ_OK) return st;
  if (T == 0) return MOEQ_OK;
  if (!x || !idx || !wts || !out) return MOEQ_EINVAL;
  if (!aligned16(x) || !aligned16(out)) return MOEQ_EALIGN;
  const int32_t I = gu->rows / 2, H = gu->cols, E = gu->num_experts;
  const Layout L = layout((int64_t)T * K, E, I, H);
  if (L.total > (size_t)MOEQ_NOALLOC_SCRATCH_BYTES) return MOEQ_EWORKSPACE;
  void* ws = nullptr;
  if (device_scratch(&ws) != hipSuccess || !ws) return MOEQ_EDEVICE;
  return moeq_experts_forward_timed(x, idx, wts, T, K, gu, dn, out, ws, MOEQ_NOALLOC_SCRATCH_BYTES, stream,
                                    nullptr);
}

moeq_status moeq_experts_forward_routed(const uint16_t* x, const int32_t* idx, const float* wts, int32_t T,
                                        int32_t K, const moeq_qweight* gu, const moeq_qweight* dn,
                                        const int32_t* offsets, const int32_t* perm, const int32_t* slot,
                                        uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
  moeq_status st = check_forward_shapes(T, K, gu, dn);
  if (st != MOEQ_OK) return st;
  if (T == 0) return MOEQ_OK;
  if (!x || !idx || !wts || !out || !offsets || !perm || !slot) return MOEQ_EINVAL;
  if (!aligned16(x) || !aligned16(out)) return MOEQ_EALIGN;
  const int32_t I = gu->rows / 2, H = gu->cols, E = gu->num_experts;
  const Layout L = layout((int64_t)T * K, E, I, H);
  if (!workspace || workspace_bytes < L.total) return MOEQ_EWORKSPACE;
  if (!aligned16(workspace)) return MOEQ_EALIGN;
  ForwardArgs a;
  a.x = x; a.idx = idx; a.wts = wts;
  a.T = T; a.K = K; a.E = E; a.H = H; a.I = I;
  a.format = gu->format;
  a.gu_q = gu->qdata; a.gu_s = gu->scales; a.gu_c = gu->scale_codes;
  a.dn_q = dn->qdata; a.dn_s = dn->scales; a.dn_c = dn->scale_codes;
  a.out = out;
  a.rb = route_buffers(workspace, L);
  // the caller's routing replaces the routing stage; only tile_start is derived
  a.rb.offsets = const_cast<int32_t*>(offsets);
  a.rb.perm = const_cast<int32_t*>(perm);
  a.rb.slot = const_cast<int32_t*>(slot);
  a.h = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + L.h);
  a.y = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.y);
  a.routed = true;
  return device_status(launch_experts_forward(a, static_cast<hipStream_t>(stream), nullptr));
}

// Backward workspace: the routing buffers, then T1's grad_w shares fp32
// [n][column tiles of I], g|u fp32 [n][2I] (not when the caller holds them),
// dx fp32 [n][H] and dg|du bf16 [n][2I], 256-B aligned.
struct BwLayout {
  Layout route;
  size_t gwp, gu, dx, dgu, total;
};
BwLayout bw_layout(int64_t n, int32_t E, int64_t I, int64_t H, bool with_gu = true) {
  BwLayout L;
  L.route = layout(n, E, 0, 0);
  size_t o = L.route.total;
  L.gwp = o; o += up(sizeof(float) * (size_t)(n * backward_col_tiles((int32_t)I)));
  L.gu = o;  o += with_gu ? up(sizeof(float) * (size_t)(n * 2 * I)) : 0;
  L.dx = o;  o += up(sizeof(float) * (size_t)(n * H));
  L.dgu = o; o += up(sizeof(uint16_t) * (size_t)(n * 2 * I));
  L.total = o;
  return L;
}

moeq_status check_backward_shapes(int32_t T, int32_t K, const moeq_qweight* gu, const moeq_qweight* dn) {
  moeq_status st = check_forward_shapes(T, K, gu, dn);
  if (st != MOEQ_OK) return st;
  // the transposed GEMMs address rows of dg|du with 32-bit byte offsets
  if ((int64_t)T * K * gu->rows * 2 >= (int64_t(1) << 32)) return MOEQ_ESHAPE;
  return MOEQ_OK;
}

size_t moeq_experts_backward_workspace_bytes(int32_t T, int32_t K, const moeq_qweight* gu,
                                             const moeq_qweight* dn) {
  if (check_backward_shapes(T, K, gu, dn) != MOEQ_OK) return 0;
  return bw_layout((int64_t)T * K, gu->num_experts, gu->rows / 2, gu->cols).total;
}

moeq_status moeq_experts_backward(const uint16_t* x, const int32_t* idx, const float* wts, int32_t T, int32_t K,
                                  const moeq_qweight* gu, const moeq_qweight* dn, const uint16_t* dout,
                                  uint16_t* grad_x, float* grad_w, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  moeq_status st = check_backward_shapes(T, K, gu, dn);
  if (st != MOEQ_OK) return st;
  if (T == 0) return MOEQ_OK;
  if (!x || !idx || !wts || !dout || !grad_x || !grad_w) return MOEQ_EINVAL;
  if (!aligned16(x) || !aligned16(dout) || !aligned16(grad_x)) return MOEQ_EALIGN;
  const int32_t I = gu->rows / 2, H = gu->cols, E = gu->num_experts;
  const BwLayout L = bw_layout((int64_t)T * K, E, I, H);
  if (!workspace || workspace_bytes < L.total) return MOEQ_EWORKSPACE;
  if (!aligned16(workspace)) return MOEQ_EALIGN;
  char* w = static_cast<char*>(workspace);
  BackwardArgs a;
  a.x = x; a.idx = idx; a.wts = wts; a.dout = dout;
  a.T = T; a.K = K; a.E = E; a.H = H; a.I = I;
  a.format = gu->format;
  a.gu_q = gu->qdata; a.gu_s = gu->scales; a.gu_c = gu->scale_codes;
  a.dn_q = dn->qdata; a.dn_s = dn->scales; a.dn_c = dn->scale_codes;
  a.grad_x = grad_x; a.grad_w = grad_w;
  a.rb = route_buffers(workspace, L.route);
  a.gw_part = reinterpret_cast<float*>(w + L.gwp);
  a.gu_save = reinterpret_cast<float*>(w + L.gu);
  a.dx = reinterpret_cast<float*>(w + L.dx);
  a.dgu = reinterpret_cast<uint16_t*>(w + L.dgu);
  return device_status(launch_experts_backward(a, static_cast<hipStream_t>(stream)));
}

size_t moeq_experts_backward_saved_workspace_bytes(int32_t T, int32_t K, const moeq_qweight* gu,
                                                   const moeq_qweight* dn) {
  if (check_backward_shapes(T, K, gu, dn) != MOEQ_OK) return 0;
  return bw_layout((int64_t)T * K, gu->num_experts, gu->rows / 2, gu->cols, false).total;
}

moeq_status moeq_experts_backward_saved(const int32_t* idx, const float* wts, int32_t T, int32_t K,
                                        const moeq_qweight* gu, const moeq_qweight* dn, const float* gu_saved,
                                        const uint16_t* dout, uint16_t* grad_x, float* grad_w, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  moeq_status st = check_backward_shapes(T, K, gu, dn);
  if (st != MOEQ_OK) return st;
  if (T == 0) return MOEQ_OK;
  if (!idx || !wts || !gu_saved || !dout || !grad_x || !grad_w) return MOEQ_EINVAL;
  if (!aligned16(gu_saved) || !aligned16(dout) || !aligned16(grad_x)) return MOEQ_EALIGN;
  const int32_t I = gu->rows / 2, H = gu->cols, E = gu->num_experts;
  const BwLayout L = bw_layout((int64_t)T * K, E, I, H, false);
  if (!workspace || workspace_bytes < L.total) return MOEQ_EWORKSPACE;
  if (!aligned16(workspace)) return MOEQ_EALIGN;
  char* w = static_cast<char*>(workspace);
  BackwardArgs a;
  a.x = nullptr; a.idx = idx; a.wts = wts; a.dout = dout;
  a.T = T; a.K = K; a.E = E; a.H = H; a.I = I;
  a.format = gu->format;
  a.gu_q = gu->qdata; a.gu_s = gu->scales; a.gu_c = gu->scale_codes;
  a.dn_q = dn->qdata; a.dn_s = dn->scales; a.dn_c = dn->scale_codes;
  a.grad_x = grad_x; a.grad_w = grad_w;
  a.rb = route_buffers(workspace, L.route);
  a.gw_part = reinterpret_cast<float*>(w + L.gwp);
  a.gu_save = const_cast<float*>(gu_saved);  // read only: the recompute that writes it is skipped
  a.recompute = false;
  a.dx = reinterpret_cast<float*>(w + L.dx);
  a.dgu = reinterpret_cast<uint16_t*>(w + L.dgu);
  return device_status(launch_experts_backward(a, static_cast<hipStream_t>(stream)));
}

moeq_status moeq_router_topk(const uint16_t* x, const uint16_t* gate, int32_t T, int32_t H, int32_t E, int32_t K,
                             int32_t renormalize, int32_t* idx, float* wts, void* stream) {
  if (T < 0 || H <= 0 || E <= 0 || K < 1) return MOEQ_EINVAL;
  if (H % 64 != 0 || K > E || E > MOEQ_MAX_EXPERTS) return MOEQ_ESHAPE;
  if ((int64_t)T * H * 2 >= (int64_t(1) << 40)) return MOEQ_ESHAPE;
  if (T == 0) return MOEQ_OK;
  if (!x || !gate || !idx || !wts) return MOEQ_EINVAL;
  if (!aligned16(x) || !aligned16(gate)) return MOEQ_EALIGN;
  return device_status(launch_router(x, gate, T, H, E, K, renormalize ? 1 : 0, idx, wts, nullptr, nullptr,
                                     static_cast<hipStream_t>(stream)));
}

// Router + routing workspace: chunk counts and bases [ceil(T/16)][E], the
// per-assignment rank [T*K] and tile_start [E+1], 256-B aligned.
struct RouterLayout {
  size_t chunk_counts, chunk_base, rank, tile_start, total;
};
RouterLayout router_layout(int64_t T, int32_t K, int32_t E) {
  RouterLayout L{};
  const int64_t nchunk = (T + kRouterChunkTokens - 1) / kRouterChunkTokens;
  size_t o = 0;
  L.chunk_counts = o; o += up(sizeof(int32_t) * (size_t)(nchunk * E));
  L.chunk_base = o;   o += up(sizeof(int32_t) * (size_t)(nchunk * E));
  L.rank = o;         o += up(sizeof(int32_t) * (size_t)(T * K));
  L.tile_start = o;   o += up(sizeof(int32_t) * (size_t)(E + 1));
  L.total = o;
  return L;
}

moeq_status check_router_route(int32_t T, int32_t H, int32_t E, int32_t K) {
  if (T < 0 || H <= 0 || E <= 0 || K < 1) return MOEQ_EINVAL;
  if (H % 64 != 0 || K > E || E > MOEQ_MAX_EXPERTS || K > kRouterRankMaxK) return MOEQ_ESHAPE;
  if ((int64_t)T * H * 2 >= (int64_t(1) << 40) || (int64_t)T * K > kMaxAssignments) return MOEQ_ESHAPE;
  return MOEQ_OK;
}

size_t moeq_router_route_workspace_bytes(int32_t T, int32_t H, int32_t E, int32_t K) {
  if (check_router_route(T, H, E, K) != MOEQ_OK) return 0;
  return router_layout(T, K, E).total;
}

moeq_status moeq_router_route(const uint16_t* x, const uint16_t* gate, int32_t T, int32_t H, int32_t E, int32_t K,
                              int32_t renormalize, int32_t* idx, float* wts, int32_t* counts, int32_t* offsets,
                              int32_t* perm, int32_t* slot, void* workspace, size_t workspace_bytes,
                              void* stream) {
  moeq_status st = check_router_route(T, H, E, K);
  if (st != MOEQ_OK) return st;
  if (!counts || !offsets) return MOEQ_EINVAL;
  if (T > 0 && (!x || !gate || !idx || !wts || !perm || !slot)) return MOEQ_EINVAL;
  if (T > 0 && (!aligned16(x) || !aligned16(gate))) return MOEQ_EALIGN;
  const RouterLayout L = router_layout(T, K, E);
  if (!workspace || workspace_bytes < L.total) return MOEQ_EWORKSPACE;
  char* w = static_cast<char*>(workspace);
  RouteBuffers rb;
  rb.chunk_counts = reinterpret_cast<int32_t*>(w + L.chunk_counts);
  rb.chunk_base = reinterpret_cast<int32_t*>(w + L.chunk_base);
  rb.rank = reinterpret_cast<int32_t*>(w + L.rank);
  rb.tile_start = reinterpret_cast<int32_t*>(w + L.tile_start);
  rb.counts = counts;
  rb.offsets = offsets;
  rb.perm = perm;
  rb.slot = slot;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (T > 0)
    e = launch_router(x, gate, T, H, E, K, renormalize ? 1 : 0, idx, wts, rb.rank, rb.chunk_counts, s);
  if (e == hipSuccess)
    e = launch_route_tail(idx, T * K, E, forward_tile_rows(), kRouterChunkTokens * K, rb, s);
  return device_status(e);
}

moeq_status moeq_qweight_copy_async(const moeq_qweight* src, const moeq_qweight* dst, void* stream) {
  moeq_status st = check_qweight(src, 0);
  if (st != MOEQ_OK) return st;
  st = check_qweight(dst, src->format);
  if (st != MOEQ_OK) return st;
  if (src->num_experts != dst->num_experts || src->rows != dst->rows || src->cols != dst->cols)
    return MOEQ_ESHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(dst->qdata, src->qdata, code_bytes(src), hipMemcpyDefault, s);
  if (e == hipSuccess) e = hipMemcpyAsync(dst->scales, src->scales, scale_bytes(src), hipMemcpyDefault, s);
  if (e == hipSuccess && src->scale_codes)
    e = hipMemcpyAsync(dst->scale_codes, src->scale_codes, scale_code_bytes(src), hipMemcpyDefault, s);
  return device_status(e);
}

size_t moeq_route_workspace_bytes(int32_t T, int32_t K, int32_t E) {
  if (T < 0 || K < 1 || E < 1 || E > MOEQ_MAX_EXPERTS || (int64_t)T * K > kMaxAssignments) return 0;
  return layout((int64_t)T * K, E, 0, 0).total;
}

moeq_status moeq_route_buckets(const int32_t* idx, int32_t T, int32_t K, int32_t E, int32_t* counts,
                               int32_t* offsets, int32_t* perm, int32_t* slot, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (T < 0 || K < 1 || E < 1) return MOEQ_EINVAL;
  if (E > MOEQ_MAX_EXPERTS || (int64_t)T * K > kMaxAssignments) return MOEQ_ESHAPE;
  if (!counts || !offsets || (T > 0 && (!idx || !perm || !slot))) return MOEQ_EINVAL;
  const int64_t n = (int64_t)T * K;
  const Layout L = layout(n, E, 0, 0);
  if (!workspace || workspace_bytes < L.total) return MOEQ_EWORKSPACE;
  RouteBuffers rb = route_buffers(workspace, L);
  // The caller's arrays replace the workspace ones for the four outputs.
  rb.counts = counts;
  rb.offsets = offsets;
  rb.perm = perm;
  rb.slot = slot;
  return device_status(launch_route(idx, (int32_t)n, E, forward_tile_rows(), rb, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
