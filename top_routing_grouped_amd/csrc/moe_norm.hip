// RMS normalisation of the attention residual (Treebeard, "How Treebeard
// routes Qwen3.6 MoE tokens": "Routing math" takes x_t to be the RMS-normalised
// post-attention state; "Editable Mermaid flowchart" and "Pseudocode" apply
// x = rms_norm(attention residual) ahead of the router):
//   x[t, j] = r[t, j] / sqrt(mean_j r[t, j]^2 + eps) * w[j]     (w = 1 without a weight)
// stored once in the activation type (bf16: round to nearest even).
//
// Bound by HBM: each fp32 row is read once and x written once.  One wave per
// row.  Lane l holds elements 4 l + 256 i (16-byte loads: a wave reads 1 KB
// contiguous per instruction) and sums their squares in ascending i with fused
// multiply-adds; a butterfly sum over the wave (fixed pairing, so every lane
// ends with the same bits, independent of timing) gives the row's sum.  Rows
// of up to 4096 elements stay in registers between the sum and the scaling;
// longer rows are read a second time (from L2) in the same order, so both
// forms give identical results.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kNormWaves = 4;
constexpr int kNormMaxJ = 16;  // rows of up to 256 * 16 elements held in registers

template <bool OUTBF>
__device__ __forceinline__ void store_x(void* x, size_t row_off, int i, float4 v, float inv, const float* w) {
    const float4 g = w ? reinterpret_cast<const float4*>(w)[i] : float4{0.f, 0.f, 0.f, 0.f};
    const float a = norm_scale(v.x, inv, w, g.x), b = norm_scale(v.y, inv, w, g.y);
    const float c = norm_scale(v.z, inv, w, g.z), d = norm_scale(v.w, inv, w, g.w);
    if constexpr (OUTBF) {
        uint2 p;
        p.x = pack_bf16x2(a, b);
        p.y = pack_bf16x2(c, d);
        reinterpret_cast<uint2*>(static_cast<uint16_t*>(x) + row_off)[i] = p;
    } else {
        reinterpret_cast<float4*>(static_cast<float*>(x) + row_off)[i] = float4{a, b, c, d};
    }
}

// J: float4 loads per lane when D = 256 J (held in registers); 0: any D % 4 == 0
template <int J, bool OUTBF>
__global__ __launch_bounds__(kNormWaves * 64) void rms_norm_kernel(const float* __restrict__ r,
                                                                   const float* __restrict__ w, float eps, int T,
                                                                   int D, void* __restrict__ x) {
    const int lane = threadIdx.x & 63;
    const int row = int(blockIdx.x) * kNormWaves + int(threadIdx.x >> 6);
    if (row >= T) return;
    const size_t off = size_t(row) * D;
    const float4* rr = reinterpret_cast<const float4*>(r + off);
    if constexpr (J > 0) {
        float s = 0.f;
        float4 v[J];
#pragma unroll
        for (int j = 0; j < J; ++j) v[j] = rr[lane + 64 * j];
#pragma unroll
        for (int j = 0; j < J; ++j) s = sum_sq4(v[j], s);
        const float inv = rms_inv_from_sum(wave_sum(s), D, eps);
#pragma unroll
        for (int j = 0; j < J; ++j) store_x<OUTBF>(x, off, lane + 64 * j, v[j], inv, w);
    } else {
        const float inv = wave_row_rms_inv(r + off, D, eps, lane);
        for (int i = lane; i < D / 4; i += 64) store_x<OUTBF>(x, off, i, rr[i], inv, w);
    }
}

template <int J>
hipError_t launch_j(const float* r, const float* w, float eps, int T, int D, void* x, bool out_bf16, hipStream_t s) {
    const dim3 g(unsigned((T + kNormWaves - 1) / kNormWaves)), b(kNormWaves * 64);
    if (out_bf16)
        rms_norm_kernel<J, true><<<g, b, 0, s>>>(r, w, eps, T, D, x);
    else
        rms_norm_kernel<J, false><<<g, b, 0, s>>>(r, w, eps, T, D, x);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rms_norm(const float* r, const float* w, float eps, int T, int D, void* x, bool out_bf16,
                           hipStream_t s) {
    if (T <= 0) return hipSuccess;
    if (D <= 0 || D % 4) return hipErrorInvalidValue;
    const int J = D % 256 == 0 ? D / 256 : 0;
    switch (J > kNormMaxJ ? 0 : J) {
        case 1: return launch_j<1>(r, w, eps, T, D, x, out_bf16, s);
        case 2: return launch_j<2>(r, w, eps, T, D, x, out_bf16, s);
        case 4: return launch_j<4>(r, w, eps, T, D, x, out_bf16, s);
        case 8: return launch_j<8>(r, w, eps, T, D, x, out_bf16, s);
        case 12: return launch_j<12>(r, w, eps, T, D, x, out_bf16, s);
        case 16: return launch_j<16>(r, w, eps, T, D, x, out_bf16, s);
        default: return launch_j<0>(r, w, eps, T, D, x, out_bf16, s);
    }
}

}  // namespace moe
