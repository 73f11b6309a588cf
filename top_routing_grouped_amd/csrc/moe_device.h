// Device-side helpers for the gfx950 MoE kernels: vector types, bf16
// conversions, wave64 reductions and the MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------ bf16 <-> f32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return uint32_t(__builtin_bit_cast(uint16_t, b));
}
// Two floats -> packed bf16 (lo in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32 (converting the halves one at a time costs a shift and an
// or more per pair).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
// The same rounding with the halves converted one at a time: more instructions,
// but neither float waits in a register for the other (the 4-bit
// dequantisation of the down projections keeps 5 waves per SIMD this way,
// 4 with pack_bf16x2).
__device__ __forceinline__ uint32_t pack_bf16x2_split(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 4-bit codes: the low nibbles (even elements) and the high nibbles (odd
// elements) of a word of 8 codes, one code per byte.  OPAQUE: the two
// registers are hidden from the compiler, so that each byte converts with
// one v_cvt_f32_ubyteN; seeing the masks, it extracts every nibble with a
// bit-field extract before a byte-0 conversion (two instructions a code, but
// only the word stays live: fewer registers).
template <bool OPAQUE>
__device__ __forceinline__ void nibble_bytes(uint32_t w, uint32_t& even, uint32_t& odd) {
    even = w & 0x0f0f0f0fu;
    odd = (w >> 4) & 0x0f0f0f0fu;
    if constexpr (OPAQUE) {
        asm("" : "+v"(even));
        asm("" : "+v"(odd));
    }
}
// The register-streaming 4-bit kernels keep the plain form: with the opaque
// one they hold a wave per SIMD fewer and measured slower (Qwen3.6 shape,
// K = 4: T = 64 layer 136.4 -> 140.5 us, T = 512 219.4 -> 227.6 us); the
// LDS-tiled kernel, whose occupancy its LDS fixes, gained 2-3%.
constexpr bool kU4OpaqueReg = false;

// ------------------------------------------------------------ wave64 reductions
// Butterfly reductions: every lane ends with the same value; the combination
// order is fixed by lane position, so results are deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = __shfl_xor(v, m, kWave);
        v = o > v ? o : v;
    }
    return v;
}

// Faster wave reductions: all-reduce inside each 16-lane row with DPP
// permutations (xor 1, xor 2 by quad permutes; the 8- and 16-lane mirrors),
// then the four row results combined through scalar registers.  Fixed
// combination order, so deterministic; the result is wave-uniform.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i inside 16

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppHalfMirror>(v);
    v += dpp_f32<kDppMirror>(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f32<kDppMirror>(v));
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
    v = max(v, dpp_u32<kDppXor1>(v));
    v = max(v, dpp_u32<kDppXor2>(v));
    v = max(v, dpp_u32<kDppHalfMirror>(v));
    v = max(v, dpp_u32<kDppMirror>(v));
    const uint32_t a = uint32_t(__builtin_amdgcn_readlane(int(v), 0)), b = uint32_t(__builtin_amdgcn_readlane(int(v), 16));
    const uint32_t c = uint32_t(__builtin_amdgcn_readlane(int(v), 32)), d = uint32_t(__builtin_amdgcn_readlane(int(v), 48));
    return max(max(a, b), max(c, d));
}
template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp_u64(uint64_t v) {
    const uint32_t lo = dpp_u32<CTRL>(uint32_t(v)), hi = dpp_u32<CTRL>(uint32_t(v >> 32));
    const uint64_t o = (uint64_t(hi) << 32) | lo;
    return o > v ? o : v;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
    return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
    v = max_dpp_u64<kDppXor1>(v);
    v = max_dpp_u64<kDppXor2>(v);
    v = max_dpp_u64<kDppHalfMirror>(v);
    v = max_dpp_u64<kDppMirror>(v);
    uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16), c = readlane_u64(v, 32), d = readlane_u64(v, 48);
    a = a > b ? a : b;
    c = c > d ? c : d;
    return a > c ? a : c;
}

// Total order on floats as unsigned integers (larger float -> larger key).
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}
// Selection key: higher score first, then lower index.
__device__ __forceinline__ uint64_t sel_key(float score, int idx) {
    return (uint64_t(orderable(score)) << 32) | uint64_t(0xffffffffu - uint32_t(idx));
}
__device__ __forceinline__ int key_index(uint64_t key) { return int(0xffffffffu - uint32_t(key)); }
__device__ __forceinline__ float key_score(uint64_t key) { return from_orderable(uint32_t(key >> 32)); }

// ------------------------------------------------------------ RMS norm pieces
// Shared by every kernel that normalises the attention residual, so that all
// of them produce the same bits: lane l of a wave sums the squares of the
// row's float4 blocks l, l + 64, l + 128, ... in that order, then wave_sum.
__device__ __forceinline__ float sum_sq4(float4 v, float s) {
    s = fmaf(v.x, v.x, s);
    s = fmaf(v.y, v.y, s);
    s = fmaf(v.z, v.z, s);
    return fmaf(v.w, v.w, s);
}
__device__ __forceinline__ float rms_inv_from_sum(float sum_sq, int D, float eps) {
    return 1.0f / sqrtf(sum_sq / float(D) + eps);
}
// Sums of squares of NR fp32 rows of D elements (D % 4 == 0; a null row reads
// as zeros), reduced over the wave.  The loads go out in batches of 8 float4
// per lane and row, all of a batch before any of its sums; blocks past the
// row end read as zero, and adding +0 leaves a sum of squares unchanged, so
// each row's sum is the same sequence of operations as summing its blocks
// lane, lane + 64, ... one at a time.
template <int NR>
__device__ __forceinline__ void wave_rows_sum_sq(const float* const (&rows)[NR], int D, int lane, float (&s)[NR]) {
    constexpr int B = 8;
    const int n4 = D / 4;
#pragma unroll
    for (int r = 0; r < NR; ++r) s[r] = 0.f;
    for (int base = 0; base < n4; base += kWave * B) {
        float4 v[NR][B];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int j = 0; j < B; ++j) {
                const int i = base + lane + kWave * j;
                v[r][j] = (rows[r] && i < n4) ? reinterpret_cast<const float4*>(rows[r])[i] : float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int j = 0; j < B; ++j) s[r] = sum_sq4(v[r][j], s[r]);
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) s[r] = wave_sum(s[r]);
}
// 1 / rms of a D-element fp32 row (D % 4 == 0); every lane gets the value.
__device__ __forceinline__ float wave_row_rms_inv(const float* row, int D, float eps, int lane) {
    const float* rows[1] = {row};
    float s[1];
    wave_rows_sum_sq<1>(rows, D, lane, s);
    return rms_inv_from_sum(s[0], D, eps);
}
// x = (r * inv) * w, or r * inv without a weight
__device__ __forceinline__ float norm_scale(float r, float inv, const float* w, float wv) {
    const float v = r * inv;
    return w ? v * wv : v;
}

__device__ __forceinline__ float sigmoidf_(float v) { return 1.0f / (1.0f + __expf(-v)); }

// A value every lane of the wave holds alike, moved to a scalar register so
// branches on it are scalar and addresses built from it stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace moe
