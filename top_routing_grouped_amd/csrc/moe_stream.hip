// Streaming read of device memory, a measurement aid for the layer's
// HBM-bound kernels: the rate at which this chip delivers a plain read
// stream (from HBM for a buffer larger than the 256 MB last-level cache,
// from that cache for a smaller one read again), against which the
// kernels' own rates are read.
//
// Each wave reads one 64 KB block in 1 KB requests (lane l takes the 16
// bytes at 16 l of each KB, so every request is whole 128-byte lines), eight
// requests in flight per lane, and folds what it read with XOR into one
// word per lane, which is stored so the loads cannot be elided.
#include "moe_kernels.h"

namespace moe {

namespace {
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBlock = 65536;  // bytes per wave
constexpr int kInFlight = 8;   // 16-byte loads per lane in flight
}  // namespace

__global__ __launch_bounds__(256) void stream_read_kernel(const uint8_t* __restrict__ buf, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const size_t wave = size_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    const uint8_t* base = buf + wave * kBlock + 16 * lane;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int i = 0; i < kBlock / 1024; i += kInFlight) {
        u32x4 v[kInFlight];
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) v[u] = *reinterpret_cast<const u32x4*>(base + 1024 * (i + u));
#pragma unroll
        for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
    }
    sink[wave * 64 + lane] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

size_t stream_read_sink_words(size_t bytes) { return bytes / kBlock * 64; }

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
    const size_t waves = bytes / kBlock;
    if (waves == 0 || waves % 4) return hipErrorInvalidValue;
    stream_read_kernel<<<dim3(unsigned(waves / 4)), dim3(256), 0, s>>>(static_cast<const uint8_t*>(buf), sink);
    return hipGetLastError();
}

}  // namespace moe
