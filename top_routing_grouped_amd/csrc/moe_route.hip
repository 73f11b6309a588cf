// Routing kernels: one wave64 per token selects K experts from the fp32
// router logits.
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
// Selection is K rounds of a wave-wide maximum over 64-bit keys
// (score bits << 32 | ~index), which breaks ties toward the lower index and
// leaves slot k holding the k-th best expert.
#include <math.h>

#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr float kClamp = 0x1p-14f;  // smallest normal fp16

template <int NV>
__global__ __launch_bounds__(256) void route_softmax_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                            int32_t* __restrict__ ids, float* __restrict__ wts) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const float* z = logits + size_t(t) * E;
    float v[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int e = lane + 64 * j;
        v[j] = e < E ? z[e] : -INFINITY;
    }
    float m = v[0];
#pragma unroll
    for (int j = 1; j < NV; ++j) m = fmaxf(m, v[j]);
    m = wave_max(m);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
        if (lane + 64 * j < E) s += __expf(v[j] - m);
    s = wave_sum(s);

    uint32_t taken = 0;
    int my_id = 0;
    float my_z = -INFINITY;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((taken >> j) & 1u)) {
                const uint64_t key = sel_key(v[j], e);
                best = key > best ? key : best;
            }
        }
        best = wave_max_u64(best);
        const int idx = min(max(key_index(best), 0), E - 1);
        if ((idx & 63) == lane) taken |= 1u << (idx >> 6);
        if (lane == k) {
            my_id = idx;
            my_z = key_score(best);
        }
    }
    const float p = lane < K ? __expf(my_z - m) / s : 0.f;
    const float denom = fmaxf(wave_sum(p), kClamp);
    if (lane < K) {
        ids[size_t(t) * K + lane] = my_id;
        wts[size_t(t) * K + lane] = p / denom;
    }
}

template <int NV>
__global__ __launch_bounds__(256) void route_sigmoid_group_kernel(const float* __restrict__ logits, int T, int E,
                                                                  int K, int G, int TG, float scaling,
                                                                  const float* __restrict__ bias,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ wts) {
    __shared__ float sel_s[4][64 * NV];
    __shared__ float sig_s[4][64 * NV];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    const bool live = t < T;  // every wave reaches the barrier below
    const int gs = E / G;

    float sel[NV];
    if (live) {
        const float* z = logits + size_t(t) * E;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = lane + 64 * j;
            if (e < E) {
                const float s = sigmoidf_(z[e]);
                sel[j] = s + (bias ? bias[e] : 0.f);
                sig_s[wave][e] = s;
                sel_s[wave][e] = sel[j];
            } else {
                sel[j] = -INFINITY;
            }
        }
    }
    __syncthreads();
    if (!live) return;

    // group score: sum of the two best selection scores of the group
    float gscore = -INFINITY;
    if (lane < G) {
        float b1 = -INFINITY, b2 = -INFINITY;
        for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
            const float x = sel_s[wave][e];
            if (x > b1) {
                b2 = b1;
                b1 = x;
            } else if (x > b2) {
                b2 = x;
            }
        }
        gscore = b1 + b2;
    }
    uint64_t kept = 0;
    for (int g = 0; g < TG; ++g) {
        uint64_t key = (lane < G && !((kept >> lane) & 1ull)) ? sel_key(gscore, lane) : 0;
        key = wave_max_u64(key);
        kept |= 1ull << min(max(key_index(key), 0), G - 1);
    }

    uint32_t taken = 0;
    int my_id = 0;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((taken >> j) & 1u) && ((kept >> (e / gs)) & 1ull)) {
                const uint64_t key = sel_key(sel[j], e);
                best = key > best ? key : best;
            }
        }
        best = wave_max_u64(best);
        const int idx = min(max(key_index(best), 0), E - 1);
        if ((idx & 63) == lane) taken |= 1u << (idx >> 6);
        if (lane == k) my_id = idx;
    }
    const float s = lane < K ? sig_s[wave][my_id] : 0.f;
    const float denom = fmaxf(wave_sum(s), kClamp);
    if (lane < K) {
        ids[size_t(t) * K + lane] = my_id;
        wts[size_t(t) * K + lane] = scaling * s / denom;
    }
}

template <int NV>
static void launch_nv(const float* logits, int T, int E, int K, int family, int G, int TG, float scaling,
                      const float* bias, int32_t* ids, float* wts, hipStream_t s) {
    const int blocks = (T + 3) / 4;
    if (family == 0)
        route_softmax_kernel<NV><<<blocks, 256, 0, s>>>(logits, T, E, K, ids, wts);
    else
        route_sigmoid_group_kernel<NV><<<blocks, 256, 0, s>>>(logits, T, E, K, G, TG, scaling, bias, ids, wts);
}

hipError_t launch_route_select(const float* logits, int T, int E, int K, int family, int n_group, int topk_group,
                               float routed_scaling, const float* bias, int32_t* ids, float* weights,
                               hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int nv = (E + 63) / 64;
    if (nv <= 1) launch_nv<1>(logits, T, E, K, family, n_group, topk_group, routed_scaling, bias, ids, weights, s);
    else if (nv <= 2) launch_nv<2>(logits, T, E, K, family, n_group, topk_group, routed_scaling, bias, ids, weights, s);
    else if (nv <= 4) launch_nv<4>(logits, T, E, K, family, n_group, topk_group, routed_scaling, bias, ids, weights, s);
    else if (nv <= 8) launch_nv<8>(logits, T, E, K, family, n_group, topk_group, routed_scaling, bias, ids, weights, s);
    else launch_nv<16>(logits, T, E, K, family, n_group, topk_group, routed_scaling, bias, ids, weights, s);
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
