// Down projection fused with the combine, for small token counts, bf16 or
// 4-bit affine group-64 weights (Treebeard,
// "How Treebeard routes Qwen3.6 MoE tokens", "Routed expert computation" and
// "Shared expert computation", last block):
//   out[t, :] = residual[t, :] + sum_{k ascending} alpha[t, k] * (W_down[e_tk] h[t*K + k])
//                              + g_t * (W_shared_down h_shared[t])
// with g_t the sigmoid of the shared gate logit (1 without a gate vector).
//
// A workgroup owns R output features d0 .. d0+R-1 for every token, so it
// alone reads those rows of every selected expert's down matrix (each byte
// once from HBM) and sums a token's units (its K routed pairs in ascending
// k, then the shared expert) in a fixed order: no slot buffer, no second
// launch, no atomics.  With about one token per selected expert a unit is a
// matrix-vector product, done with v_dot2 on the VALU: with L = 64 / R lanes
// per feature, lane (r, s) holds feature d0 + r and the 8-element K blocks
// s, s + L, s + 2L, ... of it (bf16), so a 16-byte load instruction reads
// whole 128-byte lines (R = 8 or 4).  The waves split the
// list of units evenly; a wave's partial sum for a token goes to LDS when the
// token changes and the workgroup adds the waves' partials in wave order.
// The loads of the next one or two units are in flight per wave while a unit
// is used.
#include "moe_device.h"
#include "moe_kernels.h"

#include <type_traits>
#include <utility>

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kDcR = 8;  // output features per workgroup
// bf16 banks with d_ff 512 and at least 64 units (8 per wave): 4 features per
// workgroup, twice the workgroups, half the units walked by each wave in
// turn (Qwen3.6 decode down + combine: T = 32 78.6 -> 77.2 us, T = 8 22.3
// -> 21.8 us; T = 1, with 9 units, 5.4 -> 5.6 us, so it keeps 8; 4-bit
// banks measured no faster with 4: T = 64 53.2 -> 55.3 us)
constexpr int kDcR4 = 4;
constexpr int kDcNarrowUnits = 64;
constexpr int kDcWaves = 8;
constexpr int kDcMaxT = 64;
// Fourth word of a raw (stride 0, byte-addressed) buffer resource on gfx9:
// 32-bit data format; offsets at or past the record count read zero.
constexpr int kRsrcWord3 = 0x00020000;

// Each element goes through a scalar copy before the bit cast: clang's
// __builtin_bit_cast of a vector-element expression (a.y) read element 0.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc) {
    const uint32_t a0 = a.x, a1 = a.y, a2 = a.z, a3 = a.w, b0 = b.x, b1 = b.y, b2 = b.z, b3 = b.w;
    return dot2(a3, b3, dot2(a2, b2, dot2(a1, b1, dot2(a0, b0, acc))));
}

// 4-bit weights: piece j of lane s covers reduction elements 256 j + 32 s ..
// +31 (16 bytes of codes, inside one group of 64); the same 32 h elements are
// 4 loads of 16 bytes.  With w = scale * q + min (edge0, tier table: 4-bit
// affine, group 64),
//   sum_k w_k h_k = scale * sum_k (128 + q_k) h_k + (min - 128 scale) * sum_k h_k,
// and 128 + q is a bf16 number whose bits are 0x4300 | q (exponent 2^7, the
// code in the low mantissa bits), so a pair of codes becomes a bf16 pair with
// one byte permute and one and-or, and both sums are v_dot2 over bf16 pairs:
// no per-weight conversion, fma or rounding of w (about half the VALU work of
// dequantising every weight to bf16 first).
__device__ __forceinline__ float dot_u4_piece(const u32x4& c, float s, float m, const u32x4 (&h)[4], float acc) {
    constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)
    const uint32_t words[4] = {c.x, c.y, c.z, c.w};
    float pv = 0.f, ph = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = words[i], w4 = w >> 4;
        const uint32_t h0 = h[i].x, h1 = h[i].y, h2 = h[i].z, h3 = h[i].w;
        const uint32_t hp[4] = {h0, h1, h2, h3};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            // byte b of w holds codes 2b (low nibble) and 2b+1 (high nibble):
            // bytes 0 and 2 of the permute take byte b of w and of w >> 4
            const uint32_t v = (__builtin_amdgcn_perm(w4, w, 0x0c040c00u + 0x00010001u * b) & 0x000f000fu) | 0x43004300u;
            pv = dot2(v, hp[b], pv);
            ph = dot2(kOnes, hp[b], ph);
        }
    }
    return fmaf(s, pv, fmaf(m - 128.f * s, ph, acc));
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, i>) for i = 0 .. N-1
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// R: output features per workgroup, L = 64 / R lanes per feature; J: 16-byte
// weight loads per lane per unit (bf16: F = 8 L J; U4: F = 32 L J); NB: units
// whose loads are in flight per wave
template <int J, bool U4, int NB, int R = kDcR>
__global__ __launch_bounds__(kDcWaves * 64) void down_combine_kernel(DownCombineArgs a) {
    constexpr int L = 64 / R;  // lanes per feature
    __shared__ float part[kDcWaves][kDcMaxT][R];
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int r = lane / L, s = lane % L;
    const int d0 = blockIdx.x * R;
    const int T = a.T, K = a.K, S = a.has_shared ? 1 : 0, KS = K + S, TK = T * K;
    for (int i = tid; i < kDcWaves * kDcMaxT * R; i += kDcWaves * 64) (&part[0][0][0])[i] = 0.f;

    // the wave's units ub .. ue-1 (at most 64): lane l holds unit ub + l's
    // expert (-1: the shared expert) and scale, read back with readlane
    const int n_units = T * KS;
    const int ub = (wave * n_units) / kDcWaves, ue = ((wave + 1) * n_units) / kDcWaves;
    int u_e = 0;
    float u_sc = 0.f;
    if (ub + lane < ue) {
        const int u = ub + lane, t = u / KS, k = u - t * KS;
        if (k < K) {
            const int e = a.ids[t * K + k];
            const bool ok = e >= 0 && e < a.E;
            u_e = ok ? e : 0;  // scale 0 for an id out of range
            u_sc = ok ? a.wts[t * K + k] : 0.f;
        } else {
            u_e = -1;
            u_sc = a.gate_logit ? sigmoidf_(a.gate_logit[t]) : 1.f;
        }
    }
    __syncthreads();
    const uint16_t* wb = static_cast<const uint16_t*>(a.w);
    const uint16_t* wsb = static_cast<const uint16_t*>(a.ws);
    const uint16_t* hb = static_cast<const uint16_t*>(a.h);
    const int F = U4 ? 32 * L * J : 8 * L * J;

    // unit u: token u / KS, slot u % KS (slot K: the shared expert).  Buffer
    // loads: the unit's row-slice and h row are scalar bases, a lane's byte
    // offset inside them is fixed, so issuing a unit writes no VGPR but the
    // load destinations (address arithmetic on VGPRs made the compiler wait
    // for the loads in flight before reusing their registers).
    const uint32_t w_off = uint32_t((r * F + 8 * s) * 2), h_off = uint32_t(16 * s);
    // 4-bit: lane offsets of the codes, the group scale/min and the h pieces
    const uint32_t c_off = uint32_t(r * (F / 2) + 16 * s), g_off = uint32_t((r * (F / 64) + s / 2) * 2),
                   hq_off = uint32_t(64 * s);
    const uint8_t* cb = static_cast<const uint8_t*>(a.w);
    const uint8_t* csb = static_cast<const uint8_t*>(a.ws);
    auto load_u4 = [&](int u, u32x4 (&cr)[J], uint32_t (&sm)[J], u32x4 (&hr)[J][4]) __attribute__((always_inline)) {
        const int t = u / KS, k = u - t * KS;
        const int e = __builtin_amdgcn_readlane(u_e, u - ub);
        const size_t rowi = e >= 0 ? size_t(e) * a.D + d0 : size_t(d0);
        const uint8_t* crow = (e >= 0 ? cb : csb) + rowi * (F / 2);
        const uint16_t* srow = static_cast<const uint16_t*>(e >= 0 ? a.w_scale : a.ws_scale) + rowi * (F / 64);
        const uint16_t* mrow = static_cast<const uint16_t*>(e >= 0 ? a.w_min : a.ws_min) + rowi * (F / 64);
        const size_t hrow = k < K ? size_t(t) * K + k : size_t(TK) + t;
        const auto rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(crow), 0, R * F / 2, kRsrcWord3);
        const auto rsc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(srow), 0, R * F / 32, kRsrcWord3);
        const auto rmn = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(mrow), 0, R * F / 32, kRsrcWord3);
        const auto rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(hb + hrow * a.h_ld), 0, F * 2, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            cr[j] = __builtin_amdgcn_raw_buffer_load_b128(rc, c_off + 16 * L * j, 0, 0);
            const uint32_t sv = __builtin_amdgcn_raw_buffer_load_b16(rsc, g_off + L * j, 0, 0);
            const uint32_t mv = __builtin_amdgcn_raw_buffer_load_b16(rmn, g_off + L * j, 0, 0);
            sm[j] = sv | (mv << 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) hr[j][i] = __builtin_amdgcn_raw_buffer_load_b128(rh, hq_off + 64 * L * j + 16 * i, 0, 0);
        }
    };
    auto load = [&](int u, u32x4 (&wr)[J], u32x4 (&hr)[J]) __attribute__((always_inline)) {
        const int t = u / KS, k = u - t * KS;
        const int e = __builtin_amdgcn_readlane(u_e, u - ub);
        const uint16_t* wrow = e >= 0 ? wb + (size_t(e) * a.D + d0) * F : wsb + size_t(d0) * F;
        const size_t hrow = k < K ? size_t(t) * K + k : size_t(TK) + t;
        const auto rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(wrow), 0, R * F * 2, kRsrcWord3);
        const auto rh = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(hb + hrow * a.h_ld), 0, F * 2, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < J; ++j) {
            wr[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, w_off + 16 * L * j, 0, 0);
            hr[j] = __builtin_amdgcn_raw_buffer_load_b128(rh, h_off + 16 * L * j, 0, 0);
        }
    };
    auto unit_scale = [&](int u) __attribute__((always_inline)) {
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, u_sc), u - ub));
    };

    float acc = 0.f;
    int cur_t = ub < ue ? ub / KS : 0;
    auto flush = [&]() __attribute__((always_inline)) {
        float v = acc;
#pragma unroll
        for (int m = 1; m < L; m <<= 1) v += __shfl_xor(v, m, 64);
        if (s == 0) part[wave][cur_t][r] = v;
        acc = 0.f;
    };
    auto use = [&](int u, const u32x4 (&wr)[J], const u32x4 (&hr)[J]) __attribute__((always_inline)) {
        const int t = u / KS;
        if (t != cur_t) {
            flush();
            cur_t = t;
        }
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int j = 0; j < J; j += 2) {
            p0 = dot8(wr[j], hr[j], p0);
            if (j + 1 < J) p1 = dot8(wr[j + 1], hr[j + 1], p1);
        }
        acc = fmaf(unit_scale(u), p0 + p1, acc);
    };

    auto use_u4 = [&](int u, const u32x4 (&cr)[J], const uint32_t (&sm)[J], const u32x4 (&hr)[J][4])
                      __attribute__((always_inline)) {
        const int t = u / KS;
        if (t != cur_t) {
            flush();
            cur_t = t;
        }
        float p = 0.f;
#pragma unroll
        for (int j = 0; j < J; ++j) p = dot_u4_piece(cr[j], bf16_lo(sm[j]), bf16_hi(sm[j]), hr[j], p);
        acc = fmaf(unit_scale(u), p, acc);
    };

    // NB units in flight: NB register slots used in rotation (unrolled, so
    // every slot index is a constant).  Slot i holds unit u + i at the top of
    // the loop; step i issues the loads of unit u + i + NB - 1 (clamped: past
    // the end they re-read the last unit, unused) into the slot that step i - 1
    // used, then uses unit u + i.
    if constexpr (U4) {
        if (ub < ue) {
            u32x4 cq[NB][J], hq[NB][J][4];
            uint32_t sq[NB][J];
            static_for<NB - 1>([&](auto ic) { load_u4(min(ub + ic(), ue - 1), cq[ic()], sq[ic()], hq[ic()]); });
            int u = ub;
            for (; u + NB <= ue; u += NB) {
                static_for<NB>([&](auto ic) {
                    constexpr int i = decltype(ic)::value, nx = (i + NB - 1) % NB;
                    load_u4(min(u + i + NB - 1, ue - 1), cq[nx], sq[nx], hq[nx]);
                    use_u4(u + i, cq[i], sq[i], hq[i]);
                });
            }
            static_for<NB - 1>([&](auto ic) {
                if (u + ic() < ue) use_u4(u + ic(), cq[ic()], sq[ic()], hq[ic()]);
            });
            flush();
        }
    } else if (ub < ue) {
        u32x4 wq[NB][J], hq[NB][J];
        static_for<NB - 1>([&](auto ic) { load(min(ub + ic(), ue - 1), wq[ic()], hq[ic()]); });
        int u = ub;
        for (; u + NB <= ue; u += NB) {
            static_for<NB>([&](auto ic) {
                constexpr int i = decltype(ic)::value, nx = (i + NB - 1) % NB;
                load(min(u + i + NB - 1, ue - 1), wq[nx], hq[nx]);
                use(u + i, wq[i], hq[i]);
            });
        }
        static_for<NB - 1>([&](auto ic) {
            if (u + ic() < ue) use(u + ic(), wq[ic()], hq[ic()]);
        });
        flush();
    }
    __syncthreads();

    // waves' partials in wave order, then the residual
    for (int i = tid; i < T * R; i += kDcWaves * 64) {
        const int t = i / R, rr = i % R;
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < kDcWaves; ++w) v += part[w][t][rr];
        const size_t o = size_t(t) * a.D + d0 + rr;
        a.out[o] = a.residual[o] + v;
    }
}

// Units in flight per wave.  Measured at Qwen3.6 shape (d_ff 512): a third
// unit in flight takes 4-bit T = 64 (40 units per wave) from 145 to 141 us per
// layer, but costs bf16 layers 1-1.5 us at T = 1, 8 and 32, and 4-bit layers
// with one or two units per wave about 1 us (its prologue loads the same unit
// twice).  So three for 4-bit banks whose units fit the registers of two waves
// per SIMD (5 J 16-byte loads per lane per unit, J <= 3) when a wave has at
// least 8 units, two otherwise.
constexpr int kDcDeepUnits = 8;

}  // namespace

bool down_combine_supported(int T, int K, int D, int F, int Fs, bool u4) {
    // a wave's units (T * (K + 1) / 8 of them) must fit its 64 lanes
    if (T <= 0 || T > kDcMaxT || D % kDcR || T * (K + 1) > 64 * kDcWaves) return false;
    if (Fs != 0 && Fs != F) return false;
    if (u4) return F == 256 || F == 512 || F == 768 || F == 1024;
    return F == 128 || F == 256 || F == 512 || F == 768 || F == 1024;
}

hipError_t launch_down_combine(const DownCombineArgs& a, hipStream_t s) {
    const bool u4 = a.u4 != 0;
    if (!down_combine_supported(a.T, a.K, a.D, a.F, a.has_shared ? a.F : 0, u4)) return hipErrorInvalidValue;
    if (u4 && (!a.w_scale || !a.w_min || (a.has_shared && (!a.ws_scale || !a.ws_min)))) return hipErrorInvalidValue;
    const dim3 g(unsigned(a.D / kDcR)), b(kDcWaves * 64);
    if (u4) {
        const bool deep = a.T * (a.K + (a.has_shared ? 1 : 0)) >= kDcDeepUnits * kDcWaves;
        switch (a.F / 256) {
            case 1:
                if (deep) down_combine_kernel<1, true, 3><<<g, b, 0, s>>>(a);
                else down_combine_kernel<1, true, 2><<<g, b, 0, s>>>(a);
                break;
            case 2:
                if (deep) down_combine_kernel<2, true, 3><<<g, b, 0, s>>>(a);
                else down_combine_kernel<2, true, 2><<<g, b, 0, s>>>(a);
                break;
            case 3:
                if (deep) down_combine_kernel<3, true, 3><<<g, b, 0, s>>>(a);
                else down_combine_kernel<3, true, 2><<<g, b, 0, s>>>(a);
                break;
            default: down_combine_kernel<4, true, 2><<<g, b, 0, s>>>(a); break;
        }
        return hipGetLastError();
    }
    const int units = a.T * (a.K + (a.has_shared ? 1 : 0));
    switch (a.F / 64) {
        case 2: down_combine_kernel<2, false, 2><<<g, b, 0, s>>>(a); break;
        case 4: down_combine_kernel<4, false, 2><<<g, b, 0, s>>>(a); break;
        case 8:
            if (units >= kDcNarrowUnits) down_combine_kernel<4, false, 2, kDcR4><<<dim3(unsigned(a.D / kDcR4)), b, 0, s>>>(a);
            else down_combine_kernel<8, false, 2><<<g, b, 0, s>>>(a);
            break;
        case 12: down_combine_kernel<12, false, 2><<<g, b, 0, s>>>(a); break;
        default: down_combine_kernel<16, false, 2><<<g, b, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace moe
