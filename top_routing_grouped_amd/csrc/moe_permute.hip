// Permute pre-pass and combine.
//
// Permute (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens", "Intel SYCL
// path", steps 1-4): count the T*K (token, slot) pairs per expert, turn the
// counts into offsets and an active-expert list, pack every flat pair id
// t*K + k under its expert, and list the GEMM tiles over active experts only.
// One 1024-thread workgroup: histogram with LDS atomics, block scans, then a
// stable scatter: inside a wave, lanes holding the same expert are found with
// one ballot per id bit; earlier waves' counts and a running cursor per
// expert give every pair its position, so pairs stay in ascending pair-id
// order inside each expert (the order a stable sort by expert gives).
//
// Combine (Treebeard, "Shared expert computation", last block):
//   out = residual + (sum_{k ascending} slot[t, k, :] + shared[t, :]).
#include "moe_device.h"
#include "moe_kernels.h"
#include "moe_select.h"

namespace moe {

__global__ __launch_bounds__(kPermThreads) void permute_kernel(PermParams P) {
    extern __shared__ int smem[];
    permute_block(P, smem);
}

size_t permute_smem_bytes(int E) { return permute_lds_words(E) * 4; }

int id_bits_for(int E) {
    int bits = 1;
    while ((1 << bits) < E) ++bits;
    return bits;
}

int max_tiles_for(int n_pairs, int E, int tile_rows) {
    const long long act = E < n_pairs ? E : n_pairs;
    return int(((long long)n_pairs + act * (tile_rows - 1)) / tile_rows);
}

// Many pairs: one workgroup per expert.  Every workgroup builds the full
// per-expert histogram in LDS (the same in all of them), takes its expert's
// offset, active-list slot and first tile from prefix sums over the smaller
// experts, and gathers its expert's pair ids in ascending order with
// per-wave ballots.  No cross-workgroup communication, so the result is the
// same stable order as the single-workgroup permute.
__global__ __launch_bounds__(kPermThreads) void permute_wide_kernel(PermParams P) {
    extern __shared__ int hist[];  // [E] then 32 scratch ints
    int* sh = hist + P.E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int E = P.E, me = blockIdx.x;
    for (int e = tid; e < E; e += kPermThreads) hist[e] = 0;
    __syncthreads();
    for (int p = tid; p < P.n_pairs; p += kPermThreads) {
        const int e = P.ids[p];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    const int c = tid < E ? hist[tid] : 0;
    const int nt = (c + P.tile_rows - 1) / P.tile_rows;
    int total, n_act, n_tiles;
    const int off = block_exclusive_scan(c, &total, sh);
    const int apos = block_exclusive_scan(c > 0 ? 1 : 0, &n_act, sh);
    const int tpos = block_exclusive_scan(nt, &n_tiles, sh);
    __shared__ int mine[4];
    if (tid == me) {
        mine[0] = off;
        mine[1] = c;
        mine[2] = apos;
        mine[3] = tpos;
    }
    __syncthreads();
    const int base = mine[0], cnt = mine[1];
    if (tid == 0) {
        P.offsets[me] = base;
        if (cnt > 0) {
            P.active[mine[2]] = me;
            if (P.tiles) write_tiles(P.tiles, mine[3], me, base, cnt, P.tile_rows, P.max_tiles);
        }
        if (me == 0) {
            P.offsets[E] = total;
            *P.n_active = n_act;
            if (P.n_tiles) *P.n_tiles = min(n_tiles, P.max_tiles);
        }
    }
    if (cnt == 0) return;  // uniform
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    int running = 0;
    for (int r0 = 0; r0 < P.n_pairs; r0 += kPermThreads) {
        const int p = r0 + tid;
        const bool m = p < P.n_pairs && P.ids[p] == me;
        const uint64_t b = __ballot(m);
        if (lane == 0) sh[wave] = __popcll(b);
        __syncthreads();
        int before = running, sum = 0;
        for (int w = 0; w < kPermWaves; ++w) {
            const int v = sh[w];
            if (w < wave) before += v;
            sum += v;
        }
        if (m) P.sorted_pairs[base + before + __popcll(b & lt)] = p;
        running += sum;
        __syncthreads();
    }
}

hipError_t launch_permute(const PermParams& P, hipStream_t s) {
    if (P.n_pairs >= 4096) {
        permute_wide_kernel<<<P.E, kPermThreads, size_t(P.E + 32) * 4, s>>>(P);
    } else {
        permute_kernel<<<1, kPermThreads, permute_smem_bytes(P.E), s>>>(P);
    }
    return hipGetLastError();
}

// Tile list from given permute outputs (used when the caller supplies them).
__global__ __launch_bounds__(kPermThreads) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                                   const int32_t* __restrict__ active,
                                                                   const int32_t* __restrict__ n_active_p, int E,
                                                                   int n_pairs, int4* __restrict__ tiles,
                                                                   int32_t* __restrict__ n_tiles, int max_tiles,
                                                                   int tile_rows) {
    __shared__ int sh[32];
    const int tid = threadIdx.x;
    const int n_active = min(max(*n_active_p, 0), E);
    int e = -1, begin = 0, cnt = 0;
    if (tid < n_active) {
        e = active[tid];
        if (e >= 0 && e < E) {
            begin = offsets[e];
            const int end = offsets[e + 1];
            if (begin >= 0 && end >= begin && end <= n_pairs) cnt = end - begin;
        }
    }
    const int nt = (cnt + tile_rows - 1) / tile_rows;
    int total;
    const int start = block_exclusive_scan(nt, &total, sh);
    if (cnt > 0) write_tiles(tiles, start, e, begin, cnt, tile_rows, max_tiles);
    if (tid == 0) *n_tiles = min(total, max_tiles);
}

hipError_t launch_build_tiles(const int32_t* offsets, const int32_t* active, const int32_t* n_active, int E,
                              int n_pairs, int4* tiles, int32_t* n_tiles, int max_tiles, int tile_rows,
                              hipStream_t s) {
    build_tiles_kernel<<<1, kPermThreads, 0, s>>>(offsets, active, n_active, E, n_pairs, tiles, n_tiles, max_tiles,
                                                   tile_rows);
    return hipGetLastError();
}

// ------------------------------------------------------------------ combine
template <bool BF>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ slots, const float* __restrict__ shared,
                                                      const float* residual, float* out, int T, int K, int D) {
    const int dq = D / 4;
    const long long n = (long long)T * dq;
    for (long long i = blockIdx.x * 256ll + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
        const int t = int(i / dq);
        const int d = int(i % dq) * 4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k = 0; k < K; ++k) {
            const size_t o = (size_t(t) * K + k) * D + d;
            if constexpr (BF) {
                const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(slots) + o);
                acc.x += bf16_lo(u.x);
                acc.y += bf16_hi(u.x);
                acc.z += bf16_lo(u.y);
                acc.w += bf16_hi(u.y);
            } else {
                const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(slots) + o);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
        }
        const size_t o = size_t(t) * D + d;
        if (shared) {
            const float4 sv = *reinterpret_cast<const float4*>(shared + o);
            acc.x += sv.x;
            acc.y += sv.y;
            acc.z += sv.z;
            acc.w += sv.w;
        }
        const float4 rv = *reinterpret_cast<const float4*>(residual + o);
        *reinterpret_cast<float4*>(out + o) = make_float4(rv.x + acc.x, rv.y + acc.y, rv.z + acc.z, rv.w + acc.w);
    }
}

hipError_t launch_combine(const void* slots, bool slots_bf16, const float* shared, const float* residual, float* out,
                          int T, int K, int D, hipStream_t s) {
    const long long n = (long long)T * (D / 4);
    if (n <= 0) return hipSuccess;
    const long long nb = (n + 255) / 256;
    const int blocks = int(nb < 4096 ? nb : 4096);
    if (slots_bf16)
        combine_kernel<true><<<blocks, 256, 0, s>>>(slots, shared, residual, out, T, K, D);
    else
        combine_kernel<false><<<blocks, 256, 0, s>>>(slots, shared, residual, out, T, K, D);
    return hipGetLastError();
}

}  // namespace moe
