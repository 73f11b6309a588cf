// Grouped "weight-rows x token-columns" MFMA kernels for the MoE layer.
//
// One kernel template serves every matrix product of the layer:
//   * router logits           z[t, e]   = W_router[e, :] . x[t, :]
//   * routed gate/up + SwiGLU h[p, f]   = SiLU(W_gate[e] x_t)_f * (W_up[e] x_t)_f
//   * routed down x alpha     slot[p,:] = alpha_p * W_down[e] h_p
//   * shared gate/up, shared down (x sigmoid gate)
// (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens": "Routing math",
// "Routed expert computation", "Shared expert computation").
//
// Mapping to CDNA4: the weight matrix is the MFMA "A" operand (16 weight rows
// per wave), the gathered token rows are the "B" operand (16 tokens per
// fragment), so each weight element a wave loads is used against every token
// of the tile and the result for one token sits in 4 consecutive feature
// rows of a lane (one 8/16-byte store).  Both operands are K-contiguous in
// memory.  Because any permutation of the reduction index applied to both
// operands leaves a dot product unchanged, the K order inside a chunk of
// 4 MFMAs is chosen for the load pattern rather than the instruction's own:
// for bf16, MFMA j of a chunk takes 8-element block (q + 4j) of the chunk in
// lane-group q, so each 16-byte load instruction of a wave covers 64
// contiguous bytes of each of its 16 rows; for 4-bit codes (32 weights in 16
// bytes) and fp32 (4 values in 16 bytes) lane-group q takes one contiguous
// 16-byte run, which gives the same 64-byte runs per row.  Weight rows are
// streamed straight from HBM into registers (read once per tile); a
// workgroup's waves split K and reduce their partial sums through LDS in a
// fixed order.
#include "moe_device.h"
#include "moe_kernels.h"
#include "moe_select.h"

#include <type_traits>


namespace moe {

// --------------------------------------------------------------- operands
template <int WK>
struct WTraits;
template <>
struct WTraits<kWF32> {
    static constexpr int KL = 4;  // K elements per lane per chunk
};
template <>
struct WTraits<kWBF16> {
    static constexpr int KL = 32;
};
template <>
struct WTraits<kWU4> {
    static constexpr int KL = 32;
};

// A chunk of one lane's operand: 4 MFMA-ready fragments.
template <bool F32>
struct Frag;
template <>
struct Frag<false> {
    bf16x8 v[4];
};
template <>
struct Frag<true> {
    float v[4];
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }

// K offset of MFMA j's operand block for lane-group q in the chunk at kc.
template <int WK>
__device__ __forceinline__ int kofs(int kc, int q, int j) {
    if constexpr (WK == kWBF16) return kc + (q + 4 * j) * 8;
    else return kc + q * WTraits<WK>::KL + j * (WTraits<WK>::KL / 4);
}

// Weight chunk at chunk base kc for lane-group q (rows: `row` of the bank).
template <int WK>
__device__ __forceinline__ void load_w(Frag<WK == kWF32>& f, const void* w, const void* sc, const void* mn,
                                       size_t row, int K, int kc, int q) {
    if constexpr (WK == kWBF16) {
        const uint16_t* p = static_cast<const uint16_t*>(w) + row * K;
#pragma unroll
        for (int j = 0; j < 4; ++j) f.v[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(p + kofs<WK>(kc, q, j)));
    } else if constexpr (WK == kWF32) {
        const int k = kofs<WK>(kc, q, 0);
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(w) + row * K + k);
        f.v[0] = v.x; f.v[1] = v.y; f.v[2] = v.z; f.v[3] = v.w;
    } else {  // 4-bit affine, group 64: 32 codes (16 bytes) inside one group
        const int k = kofs<WK>(kc, q, 0);
        const u32x4 c = *(
            reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w) + row * (K / 2) + k / 2));

        const size_t g = row * (K / 64) + k / 64;
        const float s = bf16_to_f32(static_cast<const uint16_t*>(sc)[g]);
        const float m = bf16_to_f32(static_cast<const uint16_t*>(mn)[g]);
        const uint32_t words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t packed[4], even, odd;
            nibble_bytes<kU4OpaqueReg>(words[j], even, odd);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float lo = fmaf(s, float((even >> (8 * i)) & 0xffu), m);
                const float hi = fmaf(s, float((odd >> (8 * i)) & 0xffu), m);
                packed[i] = pack_bf16x2_split(lo, hi);
            }
            f.v[j] = as_bf16x8(make_uint4(packed[0], packed[1], packed[2], packed[3]));
        }
    }
}

// 4-bit chunk whose group scale and min come from the LDS staging below
// (word = scale | min << 16); only the codes are loaded from memory.
__device__ __forceinline__ void load_w_u4_staged(Frag<false>& f, const void* w, size_t row, int K, int kc, int q,
                                                 uint32_t sm_word) {
    const int k = kofs<kWU4>(kc, q, 0);
    const u32x4 c = *(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(w) + row * (K / 2) + k / 2));
    const float s = bf16_lo(sm_word), m = bf16_hi(sm_word);
    const uint32_t words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t even, odd;
        nibble_bytes<kU4OpaqueReg>(words[j], even, odd);
        uint32_t packed[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = fmaf(s, float((even >> (8 * i)) & 0xffu), m);
            const float hi = fmaf(s, float((odd >> (8 * i)) & 0xffu), m);
            packed[i] = pack_bf16x2(lo, hi);
        }
        f.v[j] = as_bf16x8(make_uint4(packed[0], packed[1], packed[2], packed[3]));
    }
}

// Activation chunk (bf16 or fp32 rows) in the weights' K order, zeros for an
// absent token (with 1-2 tokens per expert most lanes hold none, and skipping
// their loads measures faster than reading a stand-in row).
template <int WK>
__device__ __forceinline__ void load_x(Frag<WK == kWF32>& f, const void* rowp, int kc, int q) {
    if constexpr (WK == kWF32) {
        if (rowp) {
            const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(rowp) + kofs<WK>(kc, q, 0));
            f.v[0] = v.x; f.v[1] = v.y; f.v[2] = v.z; f.v[3] = v.w;
        } else {
            f.v[0] = f.v[1] = f.v[2] = f.v[3] = 0.f;
        }
    } else {
        if (rowp) {
            const uint16_t* p = static_cast<const uint16_t*>(rowp);
#pragma unroll
            for (int j = 0; j < 4; ++j) f.v[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(p + kofs<WK>(kc, q, j)));
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) f.v[j] = as_bf16x8(make_uint4(0, 0, 0, 0));
        }
    }
}

// Activation chunk straight from an fp32 attention-residual row: x = (r * inv)
// * w rounded to bf16 (the same arithmetic as the RMS-norm kernel, so the
// same bits); xo, when not null, receives the converted x row.
__device__ __forceinline__ void load_x_norm(Frag<false>& f, const float* rowp, const float* w, float inv, int kc,
                                            int q, uint16_t* xo) {
    if (!rowp) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f.v[j] = as_bf16x8(make_uint4(0, 0, 0, 0));
        return;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int k = kofs<kWBF16>(kc, q, j);
        const float4 a = *reinterpret_cast<const float4*>(rowp + k);
        const float4 b = *reinterpret_cast<const float4*>(rowp + k + 4);
        float4 ga = float4{0.f, 0.f, 0.f, 0.f}, gb = ga;
        if (w) {
            ga = *reinterpret_cast<const float4*>(w + k);
            gb = *reinterpret_cast<const float4*>(w + k + 4);
        }
        const u32x4 p = {pack_bf16x2(norm_scale(a.x, inv, w, ga.x), norm_scale(a.y, inv, w, ga.y)),
                         pack_bf16x2(norm_scale(a.z, inv, w, ga.z), norm_scale(a.w, inv, w, ga.w)),
                         pack_bf16x2(norm_scale(b.x, inv, w, gb.x), norm_scale(b.y, inv, w, gb.y)),
                         pack_bf16x2(norm_scale(b.z, inv, w, gb.z), norm_scale(b.w, inv, w, gb.w))};
        f.v[j] = as_bf16x8(p);
        if (xo) *reinterpret_cast<u32x4*>(xo + k) = p;
    }
}

// bf16 chunks loaded quad-wise: a 16-byte load by every lane reads 64
// contiguous bytes of one row per four consecutive lanes (lane l: row
// (l / 4) mod 16, 16-byte piece l mod 4 of the 64), the order in which the
// vector memory path takes a full request per lane quad.  The MFMA order
// (lane 16 q + r: row r, piece q) is restored at use time by a fixed lane
// permutation (quad_order).  Both operands of a chunk take it, so the
// products are the same.
__device__ __forceinline__ void load_w_quad(Frag<false>& f, const uint16_t* w_rows, int K, int kc) {
    const int lane = threadIdx.x & 63;
    const uint16_t* p = w_rows + size_t((lane >> 2) & 15) * K + kc + (lane & 3) * 8;
#pragma unroll
    for (int j = 0; j < 4; ++j) f.v[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(p + 32 * j));
}
__device__ __forceinline__ void load_x_quad(Frag<false>& f, const uint16_t* rowp, int kc) {
    const int lane = threadIdx.x & 63;
    if (rowp) {
        const uint16_t* p = rowp + kc + (lane & 3) * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) f.v[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(p + 32 * j));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) f.v[j] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
}
__device__ __forceinline__ void quad_order(Frag<false>& f) {
    const int lane = threadIdx.x & 63;
    const int src = (4 * (lane & 15) + (lane >> 4)) << 2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 v = __builtin_bit_cast(u32x4, f.v[j]);
        v.x = __builtin_amdgcn_ds_bpermute(src, int(v.x));
        v.y = __builtin_amdgcn_ds_bpermute(src, int(v.y));
        v.z = __builtin_amdgcn_ds_bpermute(src, int(v.z));
        v.w = __builtin_amdgcn_ds_bpermute(src, int(v.w));
        f.v[j] = __builtin_bit_cast(bf16x8, v);
    }
}

template <bool F32>
__device__ __forceinline__ void mma_chunk(f32x4& acc, const Frag<F32>& a, const Frag<F32>& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (F32)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
        else
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v[j], b.v[j], acc, 0, 0, 0);
    }
}

// --------------------------------------------------------------- small-T tiles
// Small T*K (<= 256 pairs): workgroup item 0 is the shared expert (all T
// tokens, when the layer has one); item 1 + a is the a-th distinct expert
// among the routed pairs in ascending expert id, and m-tile z takes its
// pairs [16z, 16z + 16) in ascending pair id.  Every wave derives this on
// its own from the routing ids (a bit set of the experts present in the
// wave's LDS slice, the a-th set bit, ballot ranks of the matching pairs),
// so no workgroup barrier is needed; all waves reach the same answer.
// Returns the row count (0: no work); rows_w[0..count) are pair ids
// (routed) or token ids (shared).
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__device__ int small_tile(const GemmArgs& a, const int32_t* ids, int item, int mt, int* rows_w, int* e_out) {
    __shared__ uint32_t pres_all[4][32];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (item < 0) {  // shared expert: tokens 16*mt + i
        if (lane < 16) rows_w[lane] = 16 * mt + lane;
        *e_out = -1;
        wave_lds_fence();
        return max(0, min(16, a.n_tokens - 16 * mt));
    }
    if (a.direct_pairs) {  // item = one (token, slot) pair, no grouping
        if (mt > 0 || item >= a.n_pairs) return 0;
        const int e = ids[item];
        if (e < 0 || e >= a.n_experts) return 0;
        *e_out = e;
        if (lane == 0) rows_w[0] = item;
        wave_lds_fence();
        return 1;
    }
    uint32_t* pres = pres_all[wave];
    if (lane < 32) pres[lane] = 0;
    wave_lds_fence();
    const int TK = a.n_pairs;
    int idv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int p = lane + 64 * j;
        int e = p < TK ? ids[p] : -1;
        if (e < 0 || e >= a.n_experts) e = -1;
        idv[j] = e;
        if (e >= 0) atomicOr(&pres[e >> 5], 1u << (e & 31));
    }
    wave_lds_fence();
    const uint32_t word = lane < 32 ? pres[lane] : 0u;
    const int c = __popc(word);
    int incl = c;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
    }
    const uint64_t ball = __ballot(lane < 32 && incl > item);
    if (ball == 0) {
        *e_out = -1;
        return 0;
    }
    const int w = __ffsll((unsigned long long)ball) - 1;
    const int before = __builtin_amdgcn_readlane(incl - c, w);
    uint32_t bits = uint32_t(__builtin_amdgcn_readlane(int(word), w));
    for (int i = before; i < item; ++i) bits &= bits - 1;
    const int e = w * 32 + __ffs(bits) - 1;
    *e_out = e;
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int base = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool m = idv[j] == e;
        const uint64_t b = __ballot(m);
        const int pos = base + __popcll(b & lt) - 16 * mt;
        if (m && pos >= 0 && pos < 16) rows_w[pos] = lane + 64 * j;
        base += __popcll(b);
    }
    wave_lds_fence();
    return max(0, min(16, base - 16 * mt));
}

// Softmax top-K selection of all T (<= kFusedSelMaxT) tokens inside a
// small-T gate/up workgroup (the same selection code as the routing launch,
// so the ids are identical): wave w takes tokens w and w + 4 into ids_l;
// workgroup 0 also writes the routing outputs and the shared gate logits.
// Ends with a workgroup barrier.
__device__ void fused_select(const GemmArgs& a, int32_t* ids_l) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int T = a.n_tokens, K = a.topk;
    SelParams P{};
    P.logits = a.sel_logits;
    P.ksplit = a.sel_ksplit;
    P.T = T;
    P.E = a.n_experts;
    P.K = K;
    const int tt[2] = {min(wave, T - 1), min(wave + 4, T - 1)};
    int id[2];
    float w[2];
    select_softmax_lanes<4, 2>(P, tt, id, w);
    const bool first = blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int t = wave + 4 * b;
        if (t < T && lane < K) {
            const int o = t * K + lane;
            ids_l[o] = id[b];
            if (first) {
                a.sel_ids[o] = id[b];
                a.sel_wts[o] = w[b];
                if (a.sel_ids2) a.sel_ids2[o] = id[b];
                if (a.sel_wts2) a.sel_wts2[o] = w[b];
            }
        }
        if (first && a.gate_w && t < T) {
            const float gl = wave_dot_row(a.act, a.gate_w, t, a.K, a.gate_x_f32 != 0);
            if (lane == 0) a.gate_out[t] = gl;
        }
    }
    __syncthreads();
}

// --------------------------------------------------------------- kernel
// MODE: kRoutedGateUp | kRoutedDown | kDenseGateUp | kDenseDown | kDenseStore | kSmallGateUp | kSmallDown
//       | kDenseStoreNorm
// WK: weight kind; OUTBF: output stored as bf16 (else fp32)
// TF: 16-token fragments per tile; WN x WKS waves = 4 (rows x K split);
// RF: 16-row weight fragments per wave (4-bit routed tiles: each token chunk
// a wave loads is used against RF row fragments)
template <int MODE, int WK, bool OUTBF, int TF, int WN, int WKS, int RF = 1>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    constexpr bool F32 = (WK == kWF32);
    constexpr bool SMALL = (MODE == kSmallGateUp || MODE == kSmallDown);
    constexpr bool DUAL = (MODE == kRoutedGateUp || MODE == kDenseGateUp || MODE == kSmallGateUp);
    constexpr bool ROUTED = (MODE == kRoutedGateUp || MODE == kRoutedDown);
    constexpr bool NORM = (MODE == kDenseStoreNorm);
    constexpr bool STORE = (MODE == kDenseStore || NORM);
    static_assert(!NORM || (TF == 1 && WK == kWBF16), "the folded RMS norm takes bf16 16-row tiles");
    constexpr int KL = WTraits<WK>::KL;
    constexpr int SPAN = 4 * KL;
    constexpr int BM = 16 * TF;
    constexpr int NM = DUAL ? 2 : 1;
    static_assert(!SMALL || TF == 1, "small-T tiles are 16 rows");
    static_assert(RF == 1 || (ROUTED && WK == kWU4 && TF == 1 && WKS == 1), "row fragments: 4-bit routed tiles");

    // ---- tile: expert (bank) e, rows [begin, begin + count) or explicit rows (small T)
    __shared__ int srows_all[4][16];
    int* srows = srows_all[threadIdx.x >> 6];
    int e = 0, begin = 0, count;
    bool shared_item = false;
    int N = a.N, K = a.K;
    const void *w0 = a.w0, *s0 = a.s0, *m0 = a.m0, *w1 = a.w1, *s1 = a.s1, *m1 = a.m1;
    if constexpr (SMALL) {
        const int item = int(blockIdx.x) - (a.has_shared ? 1 : 0);
        const int32_t* ids = a.ids;
        if constexpr (MODE == kSmallGateUp) {
            __shared__ int32_t ids_l[kFusedSelMaxT * 64];
            // the shared expert's rows need no routing: of its workgroups only
            // the first (which writes the routing outputs and gate logits)
            // selects, and the others start streaming the shared weights
            // while the routed workgroups select
            const bool first = blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0;
            if (a.fused_sel && (item >= 0 || first)) {
                fused_select(a, ids_l);
                ids = ids_l;
            }
        }
        count = uniform(small_tile(a, ids, item, blockIdx.z, srows, &e));
        e = uniform(e);
        if (count <= 0) return;
        if (item < 0) {
            shared_item = true;
            e = 0;
            w0 = a.sw0; s0 = a.ss0; m0 = a.sm0; w1 = a.sw1; s1 = a.ss1; m1 = a.sm1;
            if constexpr (MODE == kSmallGateUp) N = a.sN; else K = a.sK;
        }
    } else if constexpr (ROUTED) {
        const int tile = blockIdx.x;
        if (tile >= uniform(*a.n_tiles)) return;
        const int4 t = a.tiles[tile];
        e = uniform(t.x); begin = uniform(t.y); count = uniform(t.z);
        if (e < 0 || e >= a.n_banks || begin < 0 || count <= 0 || begin + count > a.n_pairs) return;
    } else {
        begin = blockIdx.x * BM;
        count = min(BM, a.n_rows - begin);
        if (count <= 0) return;
    }
    const int act_ld = a.act_ld > 0 ? a.act_ld : K;
    const int out_ld = a.out_ld > 0 ? a.out_ld : N;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wn = wave % WN;
    const int wk = wave / WN;
    const int q = lane >> 4;
    const int r = lane & 15;
    // dense store may split K over blockIdx.z (partial sums to separate planes)
    const int ksub = STORE ? K / max(a.ksplit, 1) : K;
    const int kbase = STORE ? int(blockIdx.z) * ksub : 0;
    // rows wrow0 + 16 f + (0..15), f < RF (N is a multiple of 16 RF when RF > 1)
    const int wrow0 = blockIdx.y * (16 * WN * RF) + 16 * RF * wn;
    const bool rows_ok = wrow0 < N;

    // ---- token rows of this lane (one per 16-token fragment)
    const void* xrow[TF];
#pragma unroll
    for (int j = 0; j < TF; ++j) {
        const int i = j * 16 + r;
        const void* p = nullptr;
        if (i < count) {
            int arow;
            if constexpr (MODE == kRoutedGateUp) {
                const int pair = a.pairs[begin + i];
                arow = (pair >= 0 && pair < a.n_pairs) ? pair / a.topk : -1;
            } else if constexpr (MODE == kSmallGateUp) {
                arow = shared_item ? srows[i] : srows[i] / a.topk;  // token
            } else if constexpr (MODE == kSmallDown) {
                arow = shared_item ? a.n_pairs + srows[i] : srows[i];  // h row: pair, or T*K + token
            } else {
                arow = begin + i;
            }
            if (arow >= 0 && arow < a.n_act_rows)
                p = (F32 || NORM) ? static_cast<const void*>(static_cast<const float*>(a.act) + size_t(arow) * act_ld)
                        : static_cast<const void*>(static_cast<const uint16_t*>(a.act) + size_t(arow) * act_ld);
        }
        xrow[j] = p;
    }

    f32x4 acc[NM][RF][TF];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int f = 0; f < RF; ++f)
#pragma unroll
            for (int j = 0; j < TF; ++j) acc[m][f][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // routed down: each token column's pair id (its store row and routing
    // weight) is requested before the K loop, so it arrives during it
    [[maybe_unused]] int down_pair[TF];
    if constexpr (MODE == kRoutedDown) {
#pragma unroll
        for (int j = 0; j < TF; ++j) down_pair[j] = a.pairs[begin + min(j * 16 + r, count - 1)];
    }

    // 4-bit gate/up weights: the group scales and mins of this workgroup's
    // weight rows (16 * WN rows over its K range) are staged in LDS once, 16
    // bytes per load where aligned, as (scale | min << 16) words.  Loading the
    // 2-byte values per chunk cost three memory requests per 16 bytes of codes
    // (measured at T = 64: gate/up 109 -> 82 us).  The down projections keep
    // the per-chunk loads: their reduction is short (d_ff), and the staging's
    // extra round trip before the K loop cost more than it saved there.
    constexpr bool U4S = (WK == kWU4) && DUAL;
    constexpr bool PIPE = (WK == kWBF16) && TF == 1 && !NORM;  // double-buffered K trips (below)
    // (RF > 1: reductions up to 2048, so that the staging of 128 rows stays 33 KB)
    constexpr int kU4Groups = RF > 1 ? kU4MaxGroups / 2 : kU4MaxGroups;
    constexpr int kU4Stride = kU4Groups + 1;  // words per row (odd: no bank conflicts)
    __shared__ uint32_t u4_sm[U4S ? NM * 16 * WN * RF * kU4Stride : 1];
    if constexpr (U4S) {
        constexpr int ROWS = 16 * WN * RF;
        const int g0 = kbase / 64, ng = ksub / 64, gpr = K / 64;  // groups: first, count, per row
        if (ng > kU4Groups) return;  // the host rejects such sizes; never index past the staging
        const int row_base = int(blockIdx.y) * ROWS;
        const bool vec = (gpr % 8) == 0 && (g0 % 8) == 0 && (ng % 8) == 0 &&
                         ((reinterpret_cast<uintptr_t>(s0) | reinterpret_cast<uintptr_t>(m0) |
                           reinterpret_cast<uintptr_t>(NM > 1 ? s1 : s0) |
                           reinterpret_cast<uintptr_t>(NM > 1 ? m1 : m0)) % 16) == 0;
        const int per_row = vec ? ng / 8 : ng;  // 16-byte pieces, or single groups
        for (int t = int(threadIdx.x); t < NM * ROWS * per_row; t += 256) {
            const int m = t / (ROWS * per_row), rem = t - m * (ROWS * per_row);
            const int rr = rem / per_row, pc = rem - rr * per_row, row = row_base + rr;
            if (row >= N) continue;
            const uint16_t* sp = static_cast<const uint16_t*>(m == 0 ? s0 : s1);
            const uint16_t* mp = static_cast<const uint16_t*>(m == 0 ? m0 : m1);
            const size_t base = (size_t(e) * N + row) * gpr + g0;
            uint32_t* dst = &u4_sm[(m * ROWS + rr) * kU4Stride];
            if (vec) {
                const u32x4 sv = *reinterpret_cast<const u32x4*>(sp + base + 8 * pc);
                const u32x4 mv = *reinterpret_cast<const u32x4*>(mp + base + 8 * pc);
                const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w}, mw[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dst[8 * pc + 2 * i] = (sw[i] & 0xffffu) | (mw[i] << 16);
                    dst[8 * pc + 2 * i + 1] = (sw[i] >> 16) | (mw[i] & 0xffff0000u);
                }
            } else {
                dst[pc] = uint32_t(sp[base + pc]) | (uint32_t(mp[base + pc]) << 16);
            }
        }
        __syncthreads();
    }
    // this lane's staged word for chunk base kc, matrix m, row fragment f
    auto u4_word = [&](int m, int kc, int f) __attribute__((always_inline)) {
        return u4_sm[(m * 16 * WN * RF + 16 * RF * wn + 16 * f + r) * kU4Stride +
                     (kc - kbase + q * WTraits<WK>::KL) / 64];
    };

    // folded RMS norm (router logits from the attention residual): the first
    // chunk's weights are requested before the residual rows are read for the
    // tokens' 1/rms, so the HBM and L2 round trips overlap.  Then this lane's
    // token scale, and (row block 0, first wave column) where the converted x
    // goes.
    const size_t wrow = size_t(e) * N + wrow0 + r;
    const int kper = ksub / WKS;
    const int kbeg = kbase + wk * kper;
    const int nchunks = kper / SPAN;
    [[maybe_unused]] Frag<F32> w_first;
    [[maybe_unused]] float x_inv = 0.f;
    [[maybe_unused]] uint16_t* x_dst = nullptr;
    if constexpr (NORM) {
        __shared__ float s_inv[16];
        if (rows_ok && nchunks > 0) load_w<WK>(w_first, w0, s0, m0, wrow, K, kbeg, q);
        // rows wave and wave + 4 together (both rows' loads in flight at once)
        for (int i = wave; i < count; i += 8) {
            const float* rows[2] = {static_cast<const float*>(a.act) + size_t(begin + i) * act_ld,
                                    i + 4 < count ? static_cast<const float*>(a.act) + size_t(begin + i + 4) * act_ld
                                                  : nullptr};
            float ss[2];
            wave_rows_sum_sq<2>(rows, K, lane, ss);
            if (lane == 0) {
                s_inv[i] = rms_inv_from_sum(ss[0], K, a.norm_eps);
                if (i + 4 < count) s_inv[i + 4] = rms_inv_from_sum(ss[1], K, a.norm_eps);
            }
        }
        __syncthreads();
        if (r < count) {
            x_inv = s_inv[r];
            if (blockIdx.y == 0 && wn == 0) x_dst = static_cast<uint16_t*>(a.norm_x) + size_t(begin + r) * K;
        }
    }

    if constexpr (NORM) {
        if (rows_ok) {
            for (int c = 0; c < nchunks; ++c) {
                Frag<F32> wa, xb;
                if (c == 0)
                    wa = w_first;
                else
                    load_w<WK>(wa, w0, s0, m0, wrow, K, kbeg + c * SPAN, q);
                load_x_norm(xb, static_cast<const float*>(xrow[0]), a.norm_w, x_inv, kbeg + c * SPAN, q, x_dst);
                mma_chunk<F32>(acc[0][0][0], wa, xb);
            }
        }
    } else if (rows_ok) {
        // U = 2 chunks per trip, all loads before any MFMA: a runtime-count
        // loop with MFMAs (convergent) is not unrolled by the compiler, so
        // without this a wave waits a full memory round trip per chunk.
        // (Measured at decode shapes: 4 chunks per trip halves occupancy for
        // no gain; the launch is bandwidth bound either way.)
        // (RF > 1: one chunk per trip, the same weight bytes in flight)
        constexpr int U = RF > 1 ? 1 : 2;
        auto trip = [&](int c0, auto u_c) __attribute__((always_inline)) {
            constexpr int UU = decltype(u_c)::value;
            Frag<F32> wa[UU][NM][RF];
            Frag<F32> xb[UU][TF];
#pragma unroll
            for (int i = 0; i < UU; ++i) {
                const int kc = kbeg + (c0 + i) * SPAN;
#pragma unroll
                for (int f = 0; f < RF; ++f) {
                    if constexpr (U4S) {
                        load_w_u4_staged(wa[i][0][f], w0, wrow + 16 * f, K, kc, q, u4_word(0, kc, f));
                        load_w_u4_staged(wa[i][1][f], w1, wrow + 16 * f, K, kc, q, u4_word(1, kc, f));
                    } else {
                        load_w<WK>(wa[i][0][f], w0, s0, m0, wrow + 16 * f, K, kc, q);
                        if constexpr (DUAL) load_w<WK>(wa[i][1][f], w1, s1, m1, wrow + 16 * f, K, kc, q);
                    }
                }
#pragma unroll
                for (int j = 0; j < TF; ++j) load_x<WK>(xb[i][j], xrow[j], kc, q);
            }
#pragma unroll
            for (int i = 0; i < UU; ++i)
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int f = 0; f < RF; ++f)
#pragma unroll
                        for (int j = 0; j < TF; ++j) mma_chunk<F32>(acc[m][f][j], wa[i][m][f], xb[i][j]);
        };
        int c = 0;
        if constexpr (PIPE) {
            // bf16, one token fragment: two trip buffers, so that the next
            // trip's loads are in flight while this trip waits and multiplies
            // (a wave otherwise has nothing in flight between receiving a trip
            // and issuing the next).  The last pair of trips is peeled: the
            // loop body has no conditional load.  (4-bit chunks held as loaded
            // and dequantised at use measured slower: 4-bit T = 64 layer 137
            // -> 144 us, one wave per SIMD fewer.)
            Frag<false> wb[2][U][NM];
            Frag<false> xc[2][U][TF];
            // gate/up launches load quad-wise (Qwen3.6 decode layer: T = 32 235.7
            // -> 222.1 us, T = 1 28.9 -> 27.7, T = 8 unchanged); the down
            // projections keep the MFMA order (their short reductions gained
            // nothing and lost to the permutes: routed down at T = 64 82.6 ->
            // 93.3 us)
            constexpr bool QUAD = DUAL;
            // quad-wise loads: the 16 weight rows of the wave's fragment from
            // their first row, the token row of lane (l / 4) mod 16
            const uint16_t* wq0 = static_cast<const uint16_t*>(w0) + (wrow - r) * size_t(K);
            const uint16_t* wq1 = DUAL ? static_cast<const uint16_t*>(w1) + (wrow - r) * size_t(K) : nullptr;
            const uint16_t* xq = nullptr;
            if constexpr (QUAD) {
                const uint64_t xp = reinterpret_cast<uint64_t>(xrow[0]);
                const int src = ((lane >> 2) & 15) << 2;
                const uint32_t lo = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(uint32_t(xp))));
                const uint32_t hi = uint32_t(__builtin_amdgcn_ds_bpermute(src, int(uint32_t(xp >> 32))));
                xq = reinterpret_cast<const uint16_t*>((uint64_t(hi) << 32) | lo);
            }
            auto issue = [&](auto b_c, int t) __attribute__((always_inline)) {
                constexpr int B = decltype(b_c)::value;
#pragma unroll
                for (int i = 0; i < U; ++i) {
                    const int kc = kbeg + (t * U + i) * SPAN;
                    if constexpr (QUAD) {
                        load_w_quad(wb[B][i][0], wq0, K, kc);
                        if constexpr (DUAL) load_w_quad(wb[B][i][1], wq1, K, kc);
                        load_x_quad(xc[B][i][0], xq, kc);
                    } else {
                        load_w<WK>(wb[B][i][0], w0, s0, m0, wrow, K, kc, q);
                        if constexpr (DUAL) load_w<WK>(wb[B][i][1], w1, s1, m1, wrow, K, kc, q);
#pragma unroll
                        for (int j = 0; j < TF; ++j) load_x<WK>(xc[B][i][j], xrow[j], kc, q);
                    }
                }
            };
            auto mmas = [&](auto b_c, int) __attribute__((always_inline)) {
                constexpr int B = decltype(b_c)::value;
                if constexpr (QUAD) {
#pragma unroll
                    for (int i = 0; i < U; ++i) {
#pragma unroll
                        for (int m = 0; m < NM; ++m) quad_order(wb[B][i][m]);
                        quad_order(xc[B][i][0]);
                    }
                }
#pragma unroll
                for (int i = 0; i < U; ++i)
#pragma unroll
                    for (int m = 0; m < NM; ++m)
#pragma unroll
                        for (int j = 0; j < TF; ++j) mma_chunk<F32>(acc[m][0][j], wb[B][i][m], xc[B][i][j]);
            };
            constexpr std::integral_constant<int, 0> I0{};
            constexpr std::integral_constant<int, 1> I1{};
            const int npair = nchunks / (2 * U);
            if (npair > 0) {
                issue(I0, 0);
                for (int p = 0; p + 1 < npair; ++p) {
                    issue(I1, 2 * p + 1);
                    __builtin_amdgcn_sched_barrier(0);
                    mmas(I0, 2 * p);
                    issue(I0, 2 * p + 2);
                    __builtin_amdgcn_sched_barrier(0);
                    mmas(I1, 2 * p + 1);
                }
                issue(I1, 2 * npair - 1);
                __builtin_amdgcn_sched_barrier(0);
                mmas(I0, 2 * npair - 2);
                mmas(I1, 2 * npair - 1);
                c = npair * 2 * U;
            }
        }
        for (; c + U <= nchunks; c += U) trip(c, std::integral_constant<int, U>{});
        for (; c < nchunks; ++c) trip(c, std::integral_constant<int, 1>{});
    }

    // ---- split-K reduction through LDS, fixed order wk = 0, 1, 2, ...
    if constexpr (WKS > 1) {
        constexpr int NACC = NM * TF * 4;
        __shared__ float red[(WKS - 1) * WN * NACC * 64];
        if (wk > 0) {
            float* dst = red + ((wk - 1) * WN + wn) * NACC * 64;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
                for (int j = 0; j < TF; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i) dst[((m * TF + j) * 4 + i) * 64 + lane] = acc[m][0][j][i];
        }
        __syncthreads();
        if (wk == 0) {
#pragma unroll
            for (int s = 1; s < WKS; ++s) {
                const float* src = red + ((s - 1) * WN + wn) * NACC * 64;
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int j = 0; j < TF; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[m][0][j][i] += src[((m * TF + j) * 4 + i) * 64 + lane];
            }
        }
    }
    // ---- epilogue (waves of the first K part): lane holds rows wrow0 + 4q +
    // (0..3) of token column j*16 + r.  (A guarded block rather than early
    // returns: the compiler allocates 4-bit gate/up launches 118 registers
    // this way instead of 152, one more wave per SIMD.)
    if (!rows_ok || wk != 0) return;
#pragma unroll
    for (int rf = 0; rf < RF; ++rf) {
        const int f0 = wrow0 + 16 * rf + 4 * q;
#pragma unroll
        for (int j = 0; j < TF; ++j) {
            const int i = j * 16 + r;
            if (i >= count) continue;
            float v[4];
            size_t dest;
            if constexpr (DUAL) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float g = acc[0][rf][j][t];
                    v[t] = g / (1.0f + __expf(-g)) * acc[1][rf][j][t];
                }
                if constexpr (MODE == kSmallGateUp)
                    dest = shared_item ? size_t(a.n_pairs + srows[i]) : size_t(srows[i]);
                else
                    dest = size_t(begin + i);
            } else if constexpr (MODE == kRoutedDown) {
                const int pair = down_pair[j];
                if (pair < 0 || pair >= a.n_pairs) continue;
                const float s = a.row_scale[pair];
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = s * acc[0][rf][j][t];
                dest = size_t(pair);
            } else if constexpr (MODE == kSmallDown) {
                // slot rows per token: K routed (+ the shared expert in slot K)
                const int id = srows[i];
                const int spt = a.topk + (a.has_shared ? 1 : 0);
                float s;
                if (shared_item) {
                    s = a.gate_logit ? sigmoidf_(a.gate_logit[id]) : 1.0f;
                    dest = size_t(id) * spt + a.topk;
                } else {
                    s = a.row_scale[id];
                    dest = size_t(id / a.topk) * spt + id % a.topk;
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = s * acc[0][rf][j][t];
            } else if constexpr (MODE == kDenseDown) {
                const float s = a.row_scale ? sigmoidf_(a.row_scale[begin + i]) : 1.0f;
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = s * acc[0][rf][j][t];
                dest = size_t(begin + i);
            } else {  // kDenseStore
#pragma unroll
                for (int t = 0; t < 4; ++t) v[t] = acc[0][rf][j][t];
                dest = size_t(blockIdx.z) * a.n_rows + begin + i;
            }
            if constexpr (OUTBF) {
                uint2 pk = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + dest * out_ld + f0) = pk;
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(a.out) + dest * out_ld + f0) =
                    make_float4(v[0], v[1], v[2], v[3]);
            }
        }
    }
}

// --------------------------------------------------------------- launchers
// 4-bit routed 16-token tiles: weight row fragments per wave.  The down
// projection (reduction d_ff) loads as many token bytes as weight bytes per
// row fragment; two fragments per wave halve that (Qwen3.6 4-bit, K = 4,
// T = 512: layer 212.6 -> 198 us; four: no further change).  The gate/up
// keeps one: two measured 2-3 us slower (a wave per SIMD fewer).
constexpr int kU4RowFragsGateUp = 1;
constexpr int kU4RowFragsDown = 2;

// K the waves of a small-T workgroup split: both the routed and the shared
// item must divide evenly, so take the smaller of the two reduction lengths'
// common divisibility (they are both multiples of the chunk span).
static int gcd_k(const GemmArgs& a) {
    int x = a.K, y = a.sK > 0 ? a.sK : a.K;
    while (y) { const int t = x % y; x = y; y = t; }
    return x;
}

template <int MODE, int WK, bool OUTBF>
static hipError_t launch_cfg(const GemmArgs& a, int grid_x, int tf, hipStream_t s) {
    // waves split the workgroup's K range 4, 2 or 1 ways (rows 16, 32, 64)
    constexpr bool SMALL = (MODE == kSmallGateUp || MODE == kSmallDown);
    constexpr bool STORE = (MODE == kDenseStore || MODE == kDenseStoreNorm);
    if (MODE == kDenseStoreNorm && tf != 1) return hipErrorInvalidValue;
    int ks = (STORE && a.ksplit > 1) ? a.ksplit : 1;
    if (SMALL) ks = (a.n_tokens + 15) / 16;  // grid.z = 16-token m-tiles (an expert holds <= T pairs)
    const int kwg = STORE ? a.K / ks : (SMALL && a.has_shared ? gcd_k(a) : a.K);
    if constexpr (SMALL) tf = 1;
    const int nrows = (MODE == kSmallGateUp && a.has_shared && a.sN > a.N) ? a.sN : a.N;
    constexpr int SPAN = 4 * WTraits<WK>::KL;
    const bool ksplit4 = (kwg % (4 * SPAN) == 0);
    const bool ksplit2 = (kwg % (2 * SPAN) == 0);
    const int shape_x = a.shape_grid > 0 ? a.shape_grid : grid_x;  // work items the tile shape is chosen for
    const bool routed16 = (MODE == kRoutedGateUp || MODE == kRoutedDown) && tf == 1;
    if ((SMALL || routed16) && kwg % SPAN == 0 && (long long)shape_x * ((nrows + 63) / 64) >= 512) {
        // enough work items: 64 weight rows per workgroup, no K split
        // (measured at T = 8: a quarter of the workgroups of 16-row, 4-way-K
        // tiles, all resident at once, and the per-workgroup routing decode
        // runs a quarter as often; routed 16-token tiles at medium T: 4-bit
        // T = 512 layer 252 -> 220 us, bf16 T = 256 386 -> 357 us).  Fewer
        // items (T <= 4) keep the 16-row tiles below: 64-row ones would leave
        // ~1 workgroup per CU.
        if constexpr (WK == kWU4 && (MODE == kRoutedGateUp || MODE == kRoutedDown)) {
            constexpr int RF = MODE == kRoutedGateUp ? kU4RowFragsGateUp : kU4RowFragsDown;
            if (RF > 1 && nrows % (64 * RF) == 0 && kwg <= 64 * kU4MaxGroups / 2) {
                // 4-bit routed tiles: each wave 16 * RF weight rows, so a
                // token chunk is loaded once per that many rows
                dim3 g(grid_x, nrows / (64 * RF), ks);
                gemm_kernel<MODE, WK, OUTBF, 1, 4, 1, RF><<<g, 256, 0, s>>>(a);
                return hipGetLastError();
            }
        }
        dim3 g(grid_x, (nrows + 63) / 64, ks);
        gemm_kernel<MODE, WK, OUTBF, 1, 4, 1><<<g, 256, 0, s>>>(a);
    } else if (tf == 1 || SMALL) {
        if (ksplit4) {
            dim3 g(grid_x, (nrows + 15) / 16, ks);
            gemm_kernel<MODE, WK, OUTBF, 1, 1, 4><<<g, 256, 0, s>>>(a);
        } else if (ksplit2) {
            dim3 g(grid_x, (nrows + 31) / 32, ks);
            gemm_kernel<MODE, WK, OUTBF, 1, 2, 2><<<g, 256, 0, s>>>(a);
        } else {
            dim3 g(grid_x, (nrows + 63) / 64, ks);
            gemm_kernel<MODE, WK, OUTBF, 1, 4, 1><<<g, 256, 0, s>>>(a);
        }
    } else if constexpr (!SMALL && MODE != kDenseStoreNorm) {
        if (ksplit4) {
            dim3 g(grid_x, (nrows + 15) / 16, ks);
            gemm_kernel<MODE, WK, OUTBF, 4, 1, 4><<<g, 256, 0, s>>>(a);
        } else {
            dim3 g(grid_x, (nrows + 63) / 64, ks);
            gemm_kernel<MODE, WK, OUTBF, 4, 4, 1><<<g, 256, 0, s>>>(a);
        }
    }
    return hipGetLastError();
}

template <int MODE>
static hipError_t dispatch_wk(const GemmArgs& a, int wkind, bool outbf, int grid_x, int tf, hipStream_t s) {
    if (wkind == kWBF16)
        return outbf ? launch_cfg<MODE, kWBF16, true>(a, grid_x, tf, s) : launch_cfg<MODE, kWBF16, false>(a, grid_x, tf, s);
    if (wkind == kWU4)
        return outbf ? launch_cfg<MODE, kWU4, true>(a, grid_x, tf, s) : launch_cfg<MODE, kWU4, false>(a, grid_x, tf, s);
    return launch_cfg<MODE, kWF32, false>(a, grid_x, tf, s);
}

// 4-bit affine group-64 matrix [rows][K] -> bf16 [rows][K] (scale * q + min,
// rounded to nearest even: the value every 4-bit GEMM here multiplies).  One
// thread per 32 codes (one 16-byte load, four 16-byte stores); K % 64 == 0.
__global__ __launch_bounds__(256) void dequant_u4_kernel(const uint8_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scale,
                                                         const uint16_t* __restrict__ mn, long long n_pieces, int K,
                                                         uint16_t* __restrict__ out) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_pieces) return;
    const long long e = i * 32;  // first element: row e / K, column e % K (a piece lies in one group)
    const u32x4 c = *reinterpret_cast<const u32x4*>(codes + e / 2);
    const float sc = bf16_to_f32(scale[e / 64]), m = bf16_to_f32(mn[e / 64]);
    const uint32_t words[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t even, odd, packed[4];
        nibble_bytes<false>(words[j], even, odd);
#pragma unroll
        for (int b = 0; b < 4; ++b)
            packed[b] = pack_bf16x2(fmaf(sc, float((even >> (8 * b)) & 0xffu), m),
                                    fmaf(sc, float((odd >> (8 * b)) & 0xffu), m));
        *reinterpret_cast<u32x4*>(out + e + 8 * j) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
}

hipError_t launch_dequant_u4(const void* codes, const void* scale, const void* min, int rows, int K, void* out,
                             hipStream_t s) {
    if (rows <= 0 || K <= 0) return hipSuccess;
    if (K % 64) return hipErrorInvalidValue;
    const long long n = (long long)rows * K / 32;
    dequant_u4_kernel<<<unsigned((n + 255) / 256), 256, 0, s>>>(
        static_cast<const uint8_t*>(codes), static_cast<const uint16_t*>(scale), static_cast<const uint16_t*>(min), n,
        K, static_cast<uint16_t*>(out));
    return hipGetLastError();
}

hipError_t launch_gemm(int mode, int wkind, bool outbf, const GemmArgs& a, int grid_x, int tf, hipStream_t s) {
    if (grid_x <= 0) return hipSuccess;
    switch (mode) {
        case kSmallGateUp: return dispatch_wk<kSmallGateUp>(a, wkind, outbf, grid_x, tf, s);
        case kSmallDown: return dispatch_wk<kSmallDown>(a, wkind, outbf, grid_x, tf, s);
        case kRoutedGateUp: return dispatch_wk<kRoutedGateUp>(a, wkind, outbf, grid_x, tf, s);
        case kRoutedDown: return dispatch_wk<kRoutedDown>(a, wkind, outbf, grid_x, tf, s);
        case kDenseGateUp: return dispatch_wk<kDenseGateUp>(a, wkind, outbf, grid_x, tf, s);
        case kDenseDown: return dispatch_wk<kDenseDown>(a, wkind, outbf, grid_x, tf, s);
        default:
            // router logits: bf16 or fp32 weights, fp32 output
            return dispatch_wk<kDenseStore>(a, wkind == kWF32 ? kWF32 : kWBF16, false, grid_x, tf, s);
        case kDenseStoreNorm:
            if (wkind != kWBF16) return hipErrorInvalidValue;
            return launch_cfg<kDenseStoreNorm, kWBF16, false>(a, grid_x, tf, s);
    }
}

}  // namespace moe
