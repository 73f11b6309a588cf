// Measurement aids beside the layer.
//
// Streaming read of device memory, the reference for the layer's
// HBM-bound kernels: the rate at which this chip delivers a plain read
// stream (from HBM for a buffer larger than the 256 MB last-level cache,
// from that cache for a smaller one read again), against which the
// kernels' own rates are read.
//
// Each wave reads one 64 KB block in 1 KB requests (lane l takes the 16
// bytes at 16 l of each KB, so every request is whole 128-byte lines), eight
// requests in flight per lane, and folds what it read with XOR into one
// word per lane, which is stored so the loads cannot be elided.
#include "moe_device.h"
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

// MFMA issue rate, the reference for the MFMA-bound side of the grouped
// GEMMs: every wave runs kChains independent accumulator chains of the
// layer's bf16 MFMA shapes back to back (16x16x32, as the kernels use, or
// 32x32x16), with every operand element equal to `one` (1.0 from the host, a
// kernel argument, so no chain can be folded at compile time).  Each lane
// then stores the sum of its accumulator elements: iterations * kChains *
// (elements per lane) * (reduction per MFMA) when one is 1.
namespace {
constexpr int kChains = 8;
typedef float f32x16 __attribute__((ext_vector_type(16)));
}  // namespace

template <int SHAPE>
__global__ __launch_bounds__(256) void mfma_rate_kernel(float one, int iterations, float* __restrict__ sink) {
    const __bf16 v = __bf16(one);
    const bf16x8 a = {v, v, v, v, v, v, v, v};
    float total = 0.f;
    if constexpr (SHAPE == 0) {
        f32x4 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iterations; ++it)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < kChains; ++c) total += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    } else {
        f32x16 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
        for (int it = 0; it < iterations; ++it)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < kChains; ++c)
#pragma unroll
            for (int e = 0; e < 16; ++e) total += acc[c][e];
    }
    sink[size_t(blockIdx.x) * 256 + threadIdx.x] = total;
}

int mfma_rate_chains() { return kChains; }

// Vector-memory read rate from the L2 by lane pattern, the reference for how a
// kernel maps lanes to addresses.  Every wave reads a 64 KB region laid out
// as 16 rows of 4 KB (the rows of a bf16 matrix with 2048 columns), 64 load
// instructions of 16 bytes per lane per pass, issued in groups of eight:
//   pattern 0, row segments: instruction c reads the 1 KB at 1024 c, lane l
//     the 16 bytes at 16 l (eight consecutive lanes per 128-byte line);
//   pattern 1, MFMA operand order: instruction c reads 64 bytes of each row,
//     lane l row l mod 16 at byte 64 c + 16 (l / 16) (the lanes of one
//     64-byte segment are 16 apart), the order in which a 16x16x32 operand
//     fragment sits in the lanes;
//   pattern 2, row quads: the same 16 x 64 bytes per instruction, lane l row
//     l / 4 at byte 64 c + 16 (l mod 4) (four consecutive lanes per segment).
// A workgroup's four waves read four regions of one 256 KB set, set
// (workgroup / 256) mod 4 of a 1 MiB buffer: after the first pass every XCD's
// L2 (4 MB) holds what its compute units read, which their 32 KB L1s cannot.
// Each workgroup starts its passes at its own chunk (so the workgroups that
// share a compute unit do not read the same lines in step), and each lane
// adds the 32-bit words it read (mod 2^32) into the word it stores.
namespace {
constexpr int kL2Row = 4096;
constexpr int kL2Region = 16 * kL2Row;  // bytes per wave
constexpr int kL2Set = 4 * kL2Region;   // bytes per workgroup
}  // namespace

template <int PATTERN>
__global__ __launch_bounds__(256) void l2_read_kernel(const uint8_t* __restrict__ buf, int iterations,
                                                      uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint8_t* region = buf + size_t((blockIdx.x >> 8) & 3) * kL2Set + size_t(wv) * kL2Region;
    uint32_t lane_off;
    if constexpr (PATTERN == 0) lane_off = 16 * lane;
    else if constexpr (PATTERN == 1) lane_off = (lane & 15) * kL2Row + 16 * (lane >> 4);
    else lane_off = (lane >> 2) * kL2Row + 16 * (lane & 3);
    constexpr uint32_t kStep = PATTERN == 0 ? 1024 : 64;
    const int c0 = int(blockIdx.x * 8u) & 63;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int it = 0; it < iterations; ++it) {
        uint32_t off = lane_off;
        asm volatile("" : "+v"(off));  // a new pass: the loads cannot be hoisted out of it
        for (int i = 0; i < 64; i += kInFlight) {
            u32x4 v[kInFlight];
#pragma unroll
            for (int u = 0; u < kInFlight; ++u)
                v[u] = *reinterpret_cast<const u32x4*>(region + off + kStep * uint32_t((c0 + i + u) & 63));
#pragma unroll
            for (int u = 0; u < kInFlight; ++u) acc += v[u];
        }
    }
    sink[(size_t(blockIdx.x) * 4 + wv) * 64 + lane] = acc.x + acc.y + acc.z + acc.w;
}

size_t l2_read_buffer_bytes() { return size_t(4) * kL2Set; }

hipError_t launch_l2_read(int pattern, int workgroups, int iterations, const void* buf, uint32_t* sink,
                          hipStream_t s) {
    const uint8_t* b = static_cast<const uint8_t*>(buf);
    const dim3 g{unsigned(workgroups)}, t{256u};
    if (pattern == 0) l2_read_kernel<0><<<g, t, 0, s>>>(b, iterations, sink);
    else if (pattern == 1) l2_read_kernel<1><<<g, t, 0, s>>>(b, iterations, sink);
    else l2_read_kernel<2><<<g, t, 0, s>>>(b, iterations, sink);
    return hipGetLastError();
}

hipError_t launch_mfma_rate(int shape, int workgroups, int iterations, float* sink, hipStream_t s) {
    if (shape == 0)
        mfma_rate_kernel<0><<<dim3(unsigned(workgroups)), dim3(256), 0, s>>>(1.0f, iterations, sink);
    else
        mfma_rate_kernel<1><<<dim3(unsigned(workgroups)), dim3(256), 0, s>>>(1.0f, iterations, sink);
    return hipGetLastError();
}

}  // namespace moe
