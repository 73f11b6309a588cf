// Routing kernels: one wave64 per token selects K experts from the fp32
// router logits (selection rules in moe_select.h), and for small token
// counts a single workgroup that also runs the permute.
//
// Softmax family (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens",
// "Routing math"; edge0 "MoE Routing and Experts", "Softmax top-k"):
//   p = softmax(z) over all E experts, I = TopK(p, K),
//   alpha_i = p_i / max(sum_{j in I} p_j, 2^-14).
// Softmax is strictly increasing, so the top-K is taken on the logits.
// Sigmoid group family (edge0, "Sigmoid group top-k"):
//   s = sigmoid(z) in fp32, sel = s + expert_bias, groups of E/n_group
//   contiguous experts scored by the sum of their two best sel, the best
//   topk_group groups kept, top-K of sel inside them,
//   alpha = routed_scaling * s_I / max(sum s_I, 2^-14)  (bias excluded).
// Selection is K rounds of a wave-wide maximum, ties toward the lower expert
// index, leaving slot k with the k-th best expert: for the softmax family
// over 32-bit order-preserving score keys, the winner being the lowest lane
// that offers the maximum (lanes hold ascending expert ids); for the group
// family over 64-bit keys (score bits << 32 | ~index).
#include "moe_kernels.h"
#include "moe_select.h"

namespace moe {

// One wave per token, blocks of NW tokens; or (softmax family, PAIR) one wave
// per two tokens, blocks of 2 NW, whose selection chains interleave.
// Optionally also the shared-expert gate logit w_shared . x_t of the token
// (Treebeard, "Shared expert computation"), and with `counts` the block's
// pair histogram: counts[block][e] = how many of the block's tokens' slots
// chose expert e (E <= 64 NV).
template <int NV, bool PAIR, int NW>
__global__ __launch_bounds__(NW * 64) void route_select_kernel(SelParams P, GateParams G, int32_t* __restrict__ ids,
                                                               float* __restrict__ wts, int32_t* __restrict__ counts) {
    __shared__ float sel_s[NW][64 * NV];
    __shared__ float sig_s[NW][64 * NV];
    __shared__ int hist[64 * NV];
    constexpr int B = PAIR ? 2 : 1;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t0 = blockIdx.x * NW * B + wave;
    if (counts) {
        for (int e = threadIdx.x; e < P.E; e += NW * 64) hist[e] = 0;
        __syncthreads();
    }
    if (t0 < P.T) {  // wave-uniform; no block-wide barrier inside
        int id[B];
        float w[B];
        int tt[B];
#pragma unroll
        for (int b = 0; b < B; ++b) tt[b] = min(t0 + NW * b, P.T - 1);  // a clamped second token repeats the last
        if (PAIR || P.family == 0) {
            select_softmax_lanes<NV, B>(P, tt, id, w);
        } else {
            select_token<NV>(P, t0, sel_s[wave], sig_s[wave], &id[0], &w[0]);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int t = t0 + NW * b;
            if (t >= P.T) break;
            float gl = 0.f;
            if (G.w) gl = wave_dot_row(G.x, G.w, t, G.D, G.x_f32 != 0);
            if (lane < P.K) {
                const size_t o = size_t(t) * P.K + lane;
                ids[o] = id[b];
                wts[o] = w[b];
                if (P.ids2) P.ids2[o] = id[b];
                if (P.wts2) P.wts2[o] = w[b];
                if (counts) atomicAdd(&hist[id[b]], 1);
            }
            if (G.w && lane == 0) G.out[t] = gl;
        }
    }
    if (counts) {
        __syncthreads();
        for (int e = threadIdx.x; e < P.E; e += NW * 64) counts[size_t(blockIdx.x) * P.E + e] = hist[e];
    }
}

// Small T: every token's selection, then the permute, in one 1024-thread
// workgroup (16 waves take the tokens in turn; the ids stay in LDS).
constexpr int kFusedMaxE = 256;
constexpr int kFusedMaxPairs = 2048;

__global__ __launch_bounds__(kPermThreads) void route_permute_kernel(SelParams P, int32_t* __restrict__ ids,
                                                                     float* __restrict__ wts, PermParams Q) {
    __shared__ float sel_s[kPermWaves][kFusedMaxE];
    __shared__ float sig_s[kPermWaves][kFusedMaxE];
    __shared__ int32_t ids_s[kFusedMaxPairs];
    __shared__ int perm_lds[permute_lds_words(kFusedMaxE)];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int t = wave; t < P.T; t += kPermWaves) {
        int id;
        float w;
        select_token<4>(P, t, sel_s[wave], sig_s[wave], &id, &w);
        if (lane < P.K) {
            const size_t o = size_t(t) * P.K + lane;
            ids[o] = id;
            wts[o] = w;
            if (P.ids2) P.ids2[o] = id;
            if (P.wts2) P.wts2[o] = w;
            ids_s[t * P.K + lane] = id;
        }
    }
    __syncthreads();
    Q.ids = ids_s;
    permute_block(Q, perm_lds);
}

template <int NV>
static void launch_nv(const SelParams& P, const GateParams& G, int32_t* ids, float* wts, hipStream_t s) {
    // many tokens, softmax family: two tokens per wave
    if (P.family == 0 && P.T >= 1024 && NV <= 8)
        route_select_kernel<NV, true, 4><<<(P.T + 7) / 8, 256, 0, s>>>(P, G, ids, wts, nullptr);
    else
        route_select_kernel<NV, false, 4><<<(P.T + 3) / 4, 256, 0, s>>>(P, G, ids, wts, nullptr);
}

// With counts: blocks of kCountWaves waves, so a block's pairs are a chunk
// of the permute from counts.

template <int NV>
static void launch_nv_counts(const SelParams& P, const GateParams& G, int32_t* ids, float* wts, int32_t* counts,
                             hipStream_t s) {
    const int ct = route_chunk_tokens(P.family);
    if (P.family == 0)
        route_select_kernel<NV, true, kCountWaves><<<(P.T + ct - 1) / ct, 64 * kCountWaves, 0, s>>>(P, G, ids, wts,
                                                                                                  counts);
    else
        route_select_kernel<NV, false, kCountWaves><<<(P.T + ct - 1) / ct, 64 * kCountWaves, 0, s>>>(P, G, ids,
                                                                                                   wts, counts);
}

hipError_t launch_route_select_counts(const SelParams& P, const GateParams& G, int32_t* ids, float* weights,
                                      int32_t* counts, hipStream_t s) {
    if (P.T <= 0) return hipSuccess;
    if (!counts || P.E > 256) return hipErrorInvalidValue;
    const int nv = (P.E + 63) / 64;
    if (nv <= 1) launch_nv_counts<1>(P, G, ids, weights, counts, s);
    else if (nv <= 2) launch_nv_counts<2>(P, G, ids, weights, counts, s);
    else launch_nv_counts<4>(P, G, ids, weights, counts, s);
    return hipGetLastError();
}

hipError_t launch_route_select_gate(const SelParams& P, const GateParams& G, int32_t* ids, float* weights,
                                    hipStream_t s) {
    if (P.T <= 0) return hipSuccess;
    const int nv = (P.E + 63) / 64;
    if (nv <= 1) launch_nv<1>(P, G, ids, weights, s);
    else if (nv <= 2) launch_nv<2>(P, G, ids, weights, s);
    else if (nv <= 4) launch_nv<4>(P, G, ids, weights, s);
    else if (nv <= 8) launch_nv<8>(P, G, ids, weights, s);
    else launch_nv<16>(P, G, ids, weights, s);
    return hipGetLastError();
}

hipError_t launch_route_select(const SelParams& P, int32_t* ids, float* weights, hipStream_t s) {
    GateParams G{};
    return launch_route_select_gate(P, G, ids, weights, s);
}

bool route_permute_fusable(int T, int E, int K) { return E <= kFusedMaxE && T * K <= kFusedMaxPairs && T <= 64; }

hipError_t launch_route_permute(const SelParams& P, int32_t* ids, float* weights, const PermParams& Q,
                                hipStream_t s) {
    if (P.T <= 0) return hipSuccess;
    route_permute_kernel<<<1, kPermThreads, 0, s>>>(P, ids, weights, Q);
    return hipGetLastError();
}

// Shared-expert gate logit w_shared . x_t (Treebeard "Shared expert
// computation"); one wave per token, fp32 accumulation.
template <bool F32>
__global__ __launch_bounds__(256) void gate_logit_kernel(const void* __restrict__ x, const void* __restrict__ wv,
                                                         int T, int D, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    float acc = 0.f;
    if constexpr (F32) {
        const float* xr = static_cast<const float*>(x) + size_t(t) * D;
        const float* w = static_cast<const float*>(wv);
        for (int k = lane * 4; k < D; k += 256) {
            const float4 a = *reinterpret_cast<const float4*>(xr + k);
            const float4 b = *reinterpret_cast<const float4*>(w + k);
            acc = fmaf(a.x, b.x, acc);
            acc = fmaf(a.y, b.y, acc);
            acc = fmaf(a.z, b.z, acc);
            acc = fmaf(a.w, b.w, acc);
        }
    } else {
        const uint16_t* xr = static_cast<const uint16_t*>(x) + size_t(t) * D;
        const uint16_t* w = static_cast<const uint16_t*>(wv);
        for (int k = lane * 8; k < D; k += 512) {
            const uint4 a = *reinterpret_cast<const uint4*>(xr + k);
            const uint4 b = *reinterpret_cast<const uint4*>(w + k);
            const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = fmaf(bf16_lo(av[i]), bf16_lo(bv[i]), acc);
                acc = fmaf(bf16_hi(av[i]), bf16_hi(bv[i]), acc);
            }
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) out[t] = acc;
}

hipError_t launch_gate_logit(const void* x, bool x_f32, const void* wvec, int T, int D, float* out, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int blocks = (T + 3) / 4;
    if (x_f32)
        gate_logit_kernel<true><<<blocks, 256, 0, s>>>(x, wvec, T, D, out);
    else
        gate_logit_kernel<false><<<blocks, 256, 0, s>>>(x, wvec, T, D, out);
    return hipGetLastError();
}

}  // namespace moe
