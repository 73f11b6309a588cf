// Device functions shared by the routing kernels: per-token top-K selection
// (one wave64 per token) and the single-workgroup permute.
//
// Selection (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens", "Routing
// math"; edge0 "MoE Routing and Experts", "Routing families"):
//   softmax family: p = softmax(z) over all E experts, I = TopK(p, K),
//     alpha_i = p_i / max(sum_{j in I} p_j, 2^-14).  Softmax is strictly
//     increasing, so the top-K is taken on the logits.
//   sigmoid group family: s = sigmoid(z) in fp32, sel = s + expert_bias,
//     groups of E/n_group contiguous experts scored by the sum of their two
//     best sel, the best topk_group groups kept, top-K of sel inside them,
//     alpha = routed_scaling * s_I / max(sum s_I, 2^-14)  (bias excluded).
// K rounds of a wave-wide maximum break ties toward the lower index and put
// the k-th best in slot k: 32-bit order-preserving score keys plus one ballot
// for the lowest offering lane in the softmax family (select_softmax_lanes),
// 64-bit keys (score bits << 32 | ~index) in the group family (select_token).
//
// Permute (Treebeard, "Intel SYCL path", steps 1-4): count the pairs per
// expert, offsets by exclusive scan, active-expert list, stable scatter of
// flat pair ids t*K + k (ballot per id bit finds equal experts inside a
// wave; earlier waves' counts and a running cursor give the position), and
// the GEMM tile list over active experts.
#pragma once

#include <math.h>

#include "moe_device.h"

namespace moe {

constexpr float kClamp = 0x1p-14f;  // smallest normal fp16

// Softmax-family routing weight of slot `lane` < K, whose logit z the lane
// holds (slot 0 holds the largest logit m):
//   alpha_k = p_k / max(sum_{j in I} p_j, 2^-14),  p = softmax(z) over all E.
// The full softmax denominator cancels, and the floor cannot bind: the K
// largest of E probabilities sum to at least K / E >= 2^-10 (the library
// accepts E <= 1024).  So alpha_k is
// exp(z_k - m) / sum_{j in I} exp(z_j - m): K exponentials, one wave sum,
// no pass over all E experts.
__device__ __forceinline__ float softmax_topk_weight(float z, int K) {
    const int lane = threadIdx.x & 63;
    const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(z), 0));
    const float e = lane < K ? __expf(z - m) : 0.f;
    return e / wave_sum_dpp(e);
}

// Orders LDS accesses of one wave (lanes of a wave exchange data through LDS).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

struct SelParams {
    const float* logits;  // [ksplit][T][E]
    int ksplit;
    int T, E, K;
    int family;  // 0 softmax, 1 sigmoid group
    int G, TG;
    float scaling;
    const float* bias;
    int32_t* ids2;  // optional second copy of the outputs
    float* wts2;
};

// w . x_t for one token, fp32 accumulation, result in every lane.
__device__ __forceinline__ float wave_dot_row(const void* x, const void* w, int t, int D, bool f32) {
    const int lane = threadIdx.x & 63;
    float acc = 0.f;
    if (f32) {
        const float* xr = static_cast<const float*>(x) + size_t(t) * D;
        const float* wr = static_cast<const float*>(w);
        for (int k = lane * 4; k < D; k += 256) {
            const float4 a = *reinterpret_cast<const float4*>(xr + k);
            const float4 b = *reinterpret_cast<const float4*>(wr + k);
            acc = fmaf(a.x, b.x, acc);
            acc = fmaf(a.y, b.y, acc);
            acc = fmaf(a.z, b.z, acc);
            acc = fmaf(a.w, b.w, acc);
        }
    } else {
        const uint16_t* xr = static_cast<const uint16_t*>(x) + size_t(t) * D;
        const uint16_t* wr = static_cast<const uint16_t*>(w);
        for (int k = lane * 8; k < D; k += 512) {
            const uint4 a = *reinterpret_cast<const uint4*>(xr + k);
            const uint4 b = *reinterpret_cast<const uint4*>(wr + k);
            const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc = fmaf(bf16_lo(av[i]), bf16_lo(bv[i]), acc);
                acc = fmaf(bf16_hi(av[i]), bf16_hi(bv[i]), acc);
            }
        }
    }
    return wave_sum_dpp(acc);
}

// Logits of token t for lane's experts lane + 64 j (-inf past E): the K-split
// partial planes summed in order.
template <int NV>
__device__ __forceinline__ void token_logits(const SelParams& P, int t, float (&v)[NV]) {
    const int lane = threadIdx.x & 63;
    const int E = P.E;
    const size_t stride = size_t(P.T) * E;
    const size_t row = size_t(t) * E;
    // all partial logits are loaded before any is summed (one memory round
    // trip): the loads are unconditional, from clamped addresses, so that no
    // branch or register reuse puts a wait between them
    constexpr int kMaxSplit = 8;
    float part[NV][kMaxSplit];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int e = min(lane + 64 * j, E - 1);
#pragma unroll
        for (int s = 0; s < kMaxSplit; ++s) {
            const float* src = P.logits + row + e + min(s, P.ksplit - 1) * stride;
            part[j][s] = *src;
        }
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        float acc = part[j][0];
#pragma unroll
        for (int s = 1; s < kMaxSplit; ++s)
            if (s < P.ksplit) acc += part[j][s];
        v[j] = lane + 64 * j < E ? acc : -INFINITY;
    }
}

// Selects the experts of a token from its logits v (token_logits); lane
// k < K returns slot k in (*id, *w).  sel_s/sig_s: this wave's LDS scratch of
// 64*NV floats each (sigmoid family).
template <int NV>
__device__ __forceinline__ void select_from_logits(const SelParams& P, float (&v)[NV], float* sel_s, float* sig_s,
                                                   int* id_out, float* w_out) {
    const int lane = threadIdx.x & 63;
    const int E = P.E, K = P.K;
    uint32_t taken = 0;
    int my_id = 0;
    if (P.family == 0) {
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
            best = wave_max_u64_dpp(best);
            const int idx = min(max(key_index(best), 0), E - 1);
            if ((idx & 63) == lane) taken |= 1u << (idx >> 6);
            if (lane == k) {
                my_id = idx;
                my_z = key_score(best);
            }
        }
        *id_out = my_id;
        *w_out = softmax_topk_weight(my_z, K);
        return;
    }
    // sigmoid group top-k
    const int G = P.G, gs = E / G;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int e = lane + 64 * j;
        if (e < E) {
            const float s = sigmoidf_(v[j]);
            v[j] = s + (P.bias ? P.bias[e] : 0.f);
            sig_s[e] = s;
            sel_s[e] = v[j];
        }
    }
    wave_lds_sync();
    float gscore = -INFINITY;
    if (lane < G) {
        float b1 = -INFINITY, b2 = -INFINITY;
        for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
            const float x = sel_s[e];
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
    for (int g = 0; g < P.TG; ++g) {
        uint64_t key = (lane < G && !((kept >> lane) & 1ull)) ? sel_key(gscore, lane) : 0;
        key = wave_max_u64_dpp(key);
        kept |= 1ull << min(max(key_index(key), 0), G - 1);
    }
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const int e = lane + 64 * j;
            if (e < E && !((taken >> j) & 1u) && ((kept >> (e / gs)) & 1ull)) {
                const uint64_t key = sel_key(v[j], e);
                best = key > best ? key : best;
            }
        }
        best = wave_max_u64_dpp(best);
        const int idx = min(max(key_index(best), 0), E - 1);
        if ((idx & 63) == lane) taken |= 1u << (idx >> 6);
        if (lane == k) my_id = idx;
    }
    const float s = lane < K ? sig_s[my_id] : 0.f;
    const float denom = fmaxf(wave_sum_dpp(s), kClamp);
    *id_out = my_id;
    *w_out = P.scaling * s / denom;
    wave_lds_sync();  // sel_s/sig_s are reused by the wave's next token
}

// Softmax family top-K of B tokens at once (B = 1 or 2; their dependent
// reduction chains interleave).  Lane l holds the logits of experts NV*l ..
// NV*l + NV - 1, so a lower lane always holds lower expert ids: each round,
// every lane offers its best untaken expert (ties to the lower id), the wave
// takes the maximum of the 32-bit order-preserving score keys, and the lowest
// lane offering that maximum (one ballot) holds the winner.  Lane k < K
// returns slot k in (id[b], w[b]).
template <int NV, int B>
__device__ __forceinline__ void select_softmax_lanes(const SelParams& P, const int (&t)[B], int (&id)[B],
                                                     float (&w)[B]) {
    const int lane = threadIdx.x & 63;
    const int E = P.E, K = P.K;
    const size_t stride = size_t(P.T) * E;
    const bool valid = NV * lane < E;  // E % 16 == 0: all or none of a lane's experts exist
    float v[B][NV];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int j = 0; j < NV; ++j) v[b][j] = 0.f;
    {
        // every load unconditional, from clamped addresses (no branch or
        // register reuse puts a wait between them); masked afterwards
        constexpr int kMaxSplit = 8;
        float part[B][kMaxSplit][NV];
        const int l = valid ? lane : 0;
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int s = 0; s < kMaxSplit; ++s) {
                {
                    const float* src = P.logits + min(s, P.ksplit - 1) * stride + size_t(t[b]) * E + NV * l;
                    if constexpr (NV == 1) {
                        part[b][s][0] = *src;
                    } else {
#pragma unroll
                        for (int j = 0; j < NV; j += 2) {
                            const float2 u = *reinterpret_cast<const float2*>(src + j);
                            part[b][s][j] = u.x;
                            part[b][s][j + 1] = u.y;
                        }
                    }
                }
            }
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int s = 0; s < kMaxSplit; ++s)
                if (s < P.ksplit)
#pragma unroll
                    for (int j = 0; j < NV; ++j) v[b][j] += part[b][s][j];
#pragma unroll
        for (int b = 0; b < B; ++b)
#pragma unroll
            for (int j = 0; j < NV; ++j) v[b][j] = valid ? v[b][j] : 0.f;
    }
    // each lane's keys sorted once, descending, by adjacent swaps on a
    // strictly greater key (stable: equal keys keep the lower expert first);
    // a round then offers the lane's head, and the winning lane shifts its
    // list (no rescan of the lane's keys per round)
    uint32_t sk[B][NV];
    int sj[B][NV];
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            sk[b][j] = valid ? orderable(v[b][j]) : 0u;  // any real score orders above 0
            sj[b][j] = j;
        }
#pragma unroll
    for (int pass = 0; pass < NV - 1; ++pass)
#pragma unroll
        for (int i = 0; i < NV - 1 - pass; ++i)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const bool sw = sk[b][i + 1] > sk[b][i];
                const uint32_t ka = sk[b][i], kb = sk[b][i + 1];
                const int ja = sj[b][i], jb = sj[b][i + 1];
                sk[b][i] = sw ? kb : ka;
                sk[b][i + 1] = sw ? ka : kb;
                sj[b][i] = sw ? jb : ja;
                sj[b][i + 1] = sw ? ja : jb;
            }
    int my_id[B];
    uint32_t my_key[B];
#pragma unroll
    for (int b = 0; b < B; ++b) { my_id[b] = 0; my_key[b] = 0; }
    for (int k = 0; k < K; ++k) {
        uint32_t mx[B];
#pragma unroll
        for (int b = 0; b < B; ++b) mx[b] = wave_max_u32_dpp(sk[b][0]);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const uint64_t ball = __ballot(sk[b][0] == mx[b]);
            const int wl = __ffsll((unsigned long long)ball) - 1;
            const int wj = __builtin_amdgcn_readlane(sj[b][0], wl);
            if (lane == wl) {
#pragma unroll
                for (int i = 0; i + 1 < NV; ++i) {
                    sk[b][i] = sk[b][i + 1];
                    sj[b][i] = sj[b][i + 1];
                }
                sk[b][NV - 1] = 0u;
            }
            if (lane == k) {
                my_id[b] = NV * wl + wj;
                my_key[b] = mx[b];
            }
        }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
        id[b] = my_id[b];
        w[b] = softmax_topk_weight(from_orderable(my_key[b]), K);
    }
}

// Selects token t's experts; lane k < K returns slot k in (*id, *w).
template <int NV>
__device__ __forceinline__ void select_token(const SelParams& P, int t, float* sel_s, float* sig_s, int* id_out,
                                             float* w_out) {
    float v[NV];
    token_logits<NV>(P, t, v);
    select_from_logits<NV>(P, v, sel_s, sig_s, id_out, w_out);
}

// ------------------------------------------------------------------ permute
constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

// Exclusive scan over the 1024 threads of the block.  `sh` holds >= 16 ints.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    if (wave == 0) {
        int w = lane < kPermWaves ? sh[lane] : 0;
#pragma unroll
        for (int d = 1; d < kPermWaves; d <<= 1) {
            const int o = __shfl_up(w, d, 64);
            if (lane >= d) w += o;
        }
        if (lane < kPermWaves) sh[lane] = w;
    }
    __syncthreads();
    const int excl = (wave > 0 ? sh[wave - 1] : 0) + inc - v;
    *total = sh[kPermWaves - 1];
    __syncthreads();
    return excl;
}

// GEMM tiles of expert e (rows [begin, begin+cnt)) from tile index `start`;
// tiles past max_tiles are dropped.  Field w packs the expert's first tile
// and tile count (start * 65536 + n) so the GEMM can order its work by
// weight block; -1 when they do not fit.
__device__ __forceinline__ void write_tiles(int4* tiles, int start, int e, int begin, int cnt, int tile_rows,
                                            int max_tiles) {
    const int nt = (cnt + tile_rows - 1) / tile_rows;
    const int w = (start < 32768 && nt < 65536 && start + nt <= max_tiles) ? start * 65536 + nt : -1;
    for (int j = 0, r = 0; r < cnt; ++j, r += tile_rows) {
        const int ti = start + j;
        if (ti >= max_tiles) break;
        tiles[ti] = make_int4(e, begin + r, min(tile_rows, cnt - r), w);
    }
}

struct PermParams {
    const int32_t* ids;  // [n_pairs] (global or LDS)
    int n_pairs, E, id_bits;
    int32_t* offsets;
    int32_t* active;
    int32_t* n_active;
    int32_t* sorted_pairs;
    int4* tiles;
    int32_t* n_tiles;
    int tile_rows, max_tiles;
    int32_t* chunk_base;  // [ceil(n_pairs / kPermChunk)][E] scratch of the chunked permute
};

// Pairs per chunk of the chunked (many-pair) permute.
constexpr int kPermChunk = 1024;
inline int perm_chunks(int n_pairs) { return (n_pairs + kPermChunk - 1) / kPermChunk; }

// LDS words the permute needs for E experts.
__host__ __device__ constexpr size_t permute_lds_words(int E) { return size_t(3 * E + 32) + size_t(kPermWaves) * E / 2; }

// Whole-block permute; `lds` holds permute_lds_words(E) words.  Called by
// all 1024 threads of the block.
__device__ __forceinline__ void permute_block(const PermParams& P, int* lds) {
    const int E = P.E;
    int* cnt = lds;             // [E]
    int* base = cnt + E;        // [E]
    int* cursor = base + E;     // [E]
    int* sh = cursor + E;       // [32]
    uint16_t* wcnt = reinterpret_cast<uint16_t*>(sh + 32);  // [16][E]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < E; e += kPermThreads) {
        cnt[e] = 0;
        cursor[e] = 0;
    }
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < P.n_pairs; p += kPermThreads) {
        const int e = P.ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();

    const int c = tid < E ? cnt[tid] : 0;
    int total;
    const int off = block_exclusive_scan(c, &total, sh);
    int n_act;
    const int apos = block_exclusive_scan(c > 0 ? 1 : 0, &n_act, sh);
    const int nt = (c + P.tile_rows - 1) / P.tile_rows;
    int tiles_total;
    const int tstart = block_exclusive_scan(nt, &tiles_total, sh);
    if (tid < E) {
        base[tid] = off;
        P.offsets[tid] = off;
        if (c > 0) {
            P.active[apos] = tid;
            if (P.tiles) write_tiles(P.tiles, tstart, tid, off, c, P.tile_rows, P.max_tiles);
        }
    }
    if (tid == 0) {
        P.offsets[E] = total;
        *P.n_active = n_act;
        if (P.n_tiles) *P.n_tiles = min(tiles_total, P.max_tiles);
    }
    __syncthreads();

    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r0 = 0; r0 < P.n_pairs; r0 += kPermThreads) {
        const int p = r0 + tid;
        int e = p < P.n_pairs ? P.ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        if (!valid) e = 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < P.id_bits; ++b) {
            const bool bit = (e >> b) & 1;
            const uint64_t bb = __ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        const int rank = __popcll(peers & lt_mask);
        const int wc = __popcll(peers);
        if (valid && rank == 0) wcnt[wave * E + e] = uint16_t(wc);
        __syncthreads();
        if (valid) {
            int before = 0;
            for (int w = 0; w < wave; ++w) before += wcnt[w * E + e];
            P.sorted_pairs[base[e] + cursor[e] + before + rank] = p;
        }
        __syncthreads();
        if (valid && rank == 0) {
            atomicAdd(&cursor[e], wc);
            wcnt[wave * E + e] = 0;
        }
        __syncthreads();
    }
}

}  // namespace moe
