// Host-only stand-ins for the kernel launchers behind the C ABI, for the
// sanitizer build of the validation layer: every stub counts its call and
// launches nothing, so the driver can run without a GPU and check that a
// rejected call reached no launcher.
#include "moeq_internal.h"

int g_launches = 0;

namespace moeq {
namespace {
hipError_t hit() {
  ++g_launches;
  return hipSuccess;
}
}  // namespace

hipError_t launch_quantize_nf4(const uint16_t*, uint8_t*, float*, int64_t, hipStream_t) { return hit(); }
hipError_t launch_stream_reference(const uint16_t*, uint8_t*, float*, int64_t, hipStream_t) { return hit(); }
hipError_t launch_quantize_int8(const uint16_t*, int8_t*, float*, int64_t, int32_t, hipStream_t) { return hit(); }
hipError_t launch_dequantize_nf4(const uint8_t*, const float*, uint16_t*, int64_t, hipStream_t) { return hit(); }
hipError_t launch_dequantize_int8(const int8_t*, const float*, uint16_t*, int64_t, int32_t, hipStream_t) {
  return hit();
}
hipError_t launch_quantize_nf4_dq(const uint16_t*, uint8_t*, uint8_t*, float*, int32_t, int64_t, hipStream_t) {
  return hit();
}
hipError_t launch_compress_absmax(const float*, uint8_t*, float*, int32_t, int64_t, hipStream_t) { return hit(); }
hipError_t launch_dequantize_nf4_dq(const uint8_t*, const uint8_t*, const float*, uint16_t*, int32_t, int64_t,
                                    hipStream_t) {
  return hit();
}
int64_t route_chunks(int64_t n) { return (n + kRouteChunk - 1) / kRouteChunk; }
hipError_t launch_route(const int32_t*, int32_t, int32_t, int32_t, const RouteBuffers&, hipStream_t) { return hit(); }
hipError_t launch_route_tail(const int32_t*, int32_t, int32_t, int32_t, int32_t, const RouteBuffers&, hipStream_t) {
  return hit();
}
hipError_t launch_tile_start(const int32_t*, int32_t, int32_t, int32_t*, hipStream_t) { return hit(); }
hipError_t launch_experts_forward(const ForwardArgs&, hipStream_t, hipEvent_t const*) { return hit(); }
hipError_t launch_experts_backward(const BackwardArgs&, hipStream_t) { return hit(); }
hipError_t launch_router(const uint16_t*, const uint16_t*, int32_t, int32_t, int32_t, int32_t, int32_t, int32_t*,
                         float*, int32_t*, int32_t*, hipStream_t) {
  return hit();
}
int32_t forward_tile_rows() { return 256; }
int32_t backward_col_tiles(int32_t I) { return (I + 127) / 128; }
// The workspace carve-up only needs a count here (the driver checks errors,
// not sizes): one slice of y.
int decode_down_splits(int64_t, int32_t, int64_t, int64_t) { return 1; }
}  // namespace moeq
