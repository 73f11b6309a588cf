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
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

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

__device__ __forceinline__ float sigmoidf_(float v) { return 1.0f / (1.0f + __expf(-v)); }

}  // namespace moe
