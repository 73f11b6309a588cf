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

namespace moe {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

// Exclusive scan over the 1024 threads of the block.  `sh` holds >= 16 ints.
__device__ int block_exclusive_scan(int v, int* total, int* sh) {
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

// Writes the GEMM tiles of expert e (rows [begin, begin+cnt)) starting at
// tile index `start`; returns nothing.  Tiles past max_tiles are dropped.
__device__ void write_tiles(int4* tiles, int start, int e, int begin, int cnt, int tile_rows, int max_tiles) {
    for (int j = 0, r = 0; r < cnt; ++j, r += tile_rows) {
        const int ti = start + j;
        if (ti >= max_tiles) break;
        tiles[ti] = make_int4(e, begin + r, min(tile_rows, cnt - r), 0);
    }
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(const int32_t* __restrict__ ids, int n_pairs, int E,
                                                               int id_bits, int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ active,
                                                               int32_t* __restrict__ n_active,
                                                               int32_t* __restrict__ sorted_pairs,
                                                               int4* __restrict__ tiles, int32_t* __restrict__ n_tiles,
                                                               int tile_rows, int max_tiles) {
    extern __shared__ int smem[];
    int* cnt = smem;             // [E]
    int* base = cnt + E;         // [E]
    int* cursor = base + E;      // [E]
    int* sh = cursor + E;        // [32]
    uint16_t* wcnt = reinterpret_cast<uint16_t*>(sh + 32);  // [16][E]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < E; e += kPermThreads) {
        cnt[e] = 0;
        cursor[e] = 0;
    }
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
    __syncthreads();
    for (int p = tid; p < n_pairs; p += kPermThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();

    // offsets, active list and tile list (E <= 1024: one expert per thread)
    const int c = tid < E ? cnt[tid] : 0;
    int total;
    const int off = block_exclusive_scan(c, &total, sh);
    int n_act;
    const int apos = block_exclusive_scan(c > 0 ? 1 : 0, &n_act, sh);
    const int nt = (c + tile_rows - 1) / tile_rows;
    int tiles_total;
    const int tstart = block_exclusive_scan(nt, &tiles_total, sh);
    if (tid < E) {
        base[tid] = off;
        offsets[tid] = off;
        if (c > 0) {
            active[apos] = tid;
            if (tiles) write_tiles(tiles, tstart, tid, off, c, tile_rows, max_tiles);
        }
    }
    if (tid == 0) {
        offsets[E] = total;
        *n_active = n_act;
        if (n_tiles) *n_tiles = min(tiles_total, max_tiles);
    }
    __syncthreads();

    // stable scatter, 1024 pairs per round
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r0 = 0; r0 < n_pairs; r0 += kPermThreads) {
        const int p = r0 + tid;
        int e = p < n_pairs ? ids[p] : -1;
        const bool valid = e >= 0 && e < E;
        if (!valid) e = 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < id_bits; ++b) {
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
            sorted_pairs[base[e] + cursor[e] + before + rank] = p;
        }
        __syncthreads();
        if (valid && rank == 0) {
            atomicAdd(&cursor[e], wc);
            wcnt[wave * E + e] = 0;
        }
        __syncthreads();
    }
}

size_t permute_smem_bytes(int E) { return size_t(3 * E + 32) * 4 + size_t(kPermWaves) * E * 2; }

hipError_t launch_permute(const int32_t* ids, int n_pairs, int E, int32_t* offsets, int32_t* active,
                          int32_t* n_active, int32_t* sorted_pairs, int4* tiles, int32_t* n_tiles, int tile_rows,
                          hipStream_t s) {
    int bits = 0;
    while ((1 << bits) < E) ++bits;
    if (bits == 0) bits = 1;
    const long long act = E < n_pairs ? E : n_pairs;
    const long long mt = ((long long)n_pairs + act * (tile_rows - 1)) / tile_rows;
    permute_kernel<<<1, kPermThreads, permute_smem_bytes(E), s>>>(ids, n_pairs, E, bits, offsets, active, n_active,
                                                                   sorted_pairs, tiles, n_tiles, tile_rows, int(mt));
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
