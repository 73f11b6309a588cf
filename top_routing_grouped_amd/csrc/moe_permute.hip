// Permute pre-pass and combine.
//
// Permute (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens", "Intel SYCL
// path", steps 1-4): count the T*K (token, slot) pairs per expert, turn the
// counts into offsets and an active-expert list, pack every flat pair id
// t*K + k under its expert, and list the GEMM tiles over active experts only.
// Up to 4096 pairs, one 1024-thread workgroup: histogram with LDS atomics,
// block scans, then a stable scatter: inside a wave, lanes holding the same
// expert are found with one ballot per id bit; earlier waves' counts and a
// running cursor per expert give every pair its position, so pairs stay in
// ascending pair-id order inside each expert (the order a stable sort by
// expert gives).  More pairs: the chunked permute below.
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

// Many pairs: three launches over chunks of kPermChunk pairs.
//  1. count: each chunk's per-expert histogram (LDS atomics) -> chunk_base[c][e];
//  2. scan (one workgroup, threads over experts x slices of chunks): per
//     expert, the exclusive prefix over chunks and the total; the totals give
//     offsets, the active list and the tile list, and chunk_base[c][e] becomes
//     the position of chunk c's first pair of expert e;
//  3. scatter: each chunk ranks its pairs within their expert (ballots over
//     the id bits inside a wave, earlier waves' counts through LDS) and writes
//     them from chunk_base, so pairs stay in ascending pair-id order inside
//     each expert (the order a stable sort by expert gives).
__global__ __launch_bounds__(256) void permute_count_kernel(PermParams P) {
    extern __shared__ int hist[];  // [E]
    const int E = P.E, c = blockIdx.x, tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) hist[e] = 0;
    __syncthreads();
    const int p0 = c * kPermChunk, p1 = min(P.n_pairs, p0 + kPermChunk);
    for (int p = p0 + tid; p < p1; p += 256) {
        const int e = P.ids[p];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = tid; e < E; e += 256) P.chunk_base[size_t(c) * E + e] = hist[e];
}

__global__ __launch_bounds__(kPermThreads) void permute_scan_kernel(PermParams P, int nchunks) {
    __shared__ int sh[32];
    __shared__ int part[kPermThreads];  // per (slice, expert): the slice's count of the expert's pairs
    __shared__ int off_l[kPermThreads];  // per expert: its offset
    // Thread (slice sl, expert e) = tid: the chunks split into S contiguous
    // slices, one per group of E threads; a thread's first G chunk counts are
    // loaded in one round trip (unconditional loads from clamped addresses)
    // and kept in registers for the second pass.
    constexpr int G = 16;
    const int E = P.E, tid = threadIdx.x;
    const int S = max(1, kPermThreads / E);
    const int e = tid % E, sl = tid / E;
    const bool act = sl < S;
    const int per = (nchunks + S - 1) / S;
    const int c0 = act ? min(nchunks, sl * per) : nchunks, c1 = min(nchunks, c0 + per);
    int v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = P.chunk_base[size_t(min(c0 + i, nchunks - 1)) * E + e];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < G; ++i) sum += c0 + i < c1 ? v[i] : 0;
    for (int c = c0 + G; c < c1; ++c) sum += P.chunk_base[size_t(c) * E + e];  // slices longer than G
    part[tid] = act ? sum : 0;
    __syncthreads();
    int total = 0, before = 0;
    if (act) {
        for (int q = 0; q < S; ++q) {
            const int n = part[q * E + e];
            total += n;
            before += q < sl ? n : 0;
        }
    }
    const int cnt = tid < E ? total : 0;
    int all, n_act, n_tiles;
    const int off = block_exclusive_scan(cnt, &all, sh);
    const int apos = block_exclusive_scan(cnt > 0 ? 1 : 0, &n_act, sh);
    const int nt = (cnt + P.tile_rows - 1) / P.tile_rows;
    const int tpos = block_exclusive_scan(P.tiles ? nt : 0, &n_tiles, sh);
    if (tid < E) {
        P.offsets[tid] = off;
        off_l[tid] = off;
        if (cnt > 0) {
            P.active[apos] = tid;
            if (P.tiles) write_tiles(P.tiles, tpos, tid, off, cnt, P.tile_rows, P.max_tiles);
        }
    }
    __syncthreads();
    if (act) {
        // chunk c's first pair of expert e goes to off + (its pairs in chunks < c)
        int run = off_l[e] + before;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            if (c0 + i < c1) {
                P.chunk_base[size_t(c0 + i) * E + e] = run;
                run += v[i];
            }
        }
        for (int c = c0 + G; c < c1; ++c) {
            const int n = P.chunk_base[size_t(c) * E + e];
            P.chunk_base[size_t(c) * E + e] = run;
            run += n;
        }
    }
    if (tid == 0) {
        P.offsets[E] = all;
        *P.n_active = n_act;
        if (P.n_tiles) *P.n_tiles = min(n_tiles, P.max_tiles);
    }
}

static_assert(kPermChunk == kPermThreads, "one pair per thread in the scatter");

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(PermParams P) {
    extern __shared__ uint16_t wcnt[];  // [kPermWaves][E]
    const int E = P.E, c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int p = c * kPermChunk + tid;  // one pair per thread (kPermChunk == kPermThreads)
    int e = p < P.n_pairs ? P.ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    if (!valid) e = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < P.id_bits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
    }
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt);
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
    __syncthreads();
    if (valid && rank == 0) wcnt[wave * E + e] = uint16_t(__popcll(peers));
    __syncthreads();
    if (valid) {
        int before = 0;
        for (int w = 0; w < wave; ++w) before += wcnt[w * E + e];
        P.sorted_pairs[P.chunk_base[size_t(c) * E + e] + before + rank] = p;
    }
}

hipError_t launch_permute(const PermParams& P, hipStream_t s) {
    if (P.n_pairs >= 4096 && P.chunk_base) {
        const int nc = perm_chunks(P.n_pairs);
        permute_count_kernel<<<nc, 256, size_t(P.E) * 4, s>>>(P);
        permute_scan_kernel<<<1, kPermThreads, 0, s>>>(P, nc);
        permute_scatter_kernel<<<nc, kPermThreads, size_t(kPermWaves) * P.E * 2, s>>>(P);
    } else {
        permute_kernel<<<1, kPermThreads, permute_smem_bytes(P.E), s>>>(P);
    }
    return hipGetLastError();
}

// The permute from per-chunk expert counts that an earlier launch wrote
// (the routing launch of many tokens counts each workgroup's pairs): one
// launch.  Block b takes R = 1024 / chunk_pairs consecutive chunks (one pair
// per thread).  Every block sums all chunk counts itself (threads over
// experts x slices of chunks, each thread's counts loaded in round trips of
// 16), so it knows every expert's offset and how many of the expert's pairs
// lie in chunks before its own; block 0 also writes the offsets, the active
// list and the tile list.  The scatter ranks pairs as permute_scatter_kernel
// does (stable: ascending pair id inside each expert).
constexpr int kCountsMaxE = 256;

__global__ __launch_bounds__(kPermThreads) void permute_from_counts_kernel(PermParams P, int n_chunks,
                                                                           int chunk_pairs) {
    __shared__ int sh[32];
    __shared__ int part_all[kPermThreads];
    __shared__ int part_before[kPermThreads];
    __shared__ int base_l[kCountsMaxE];
    __shared__ uint16_t wcnt[kPermWaves * kCountsMaxE];
    constexpr int G = 16;
    const int E = P.E, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = kPermThreads / chunk_pairs;
    const int cb = blockIdx.x * R;  // first chunk of this block
    const int S = kPermThreads / E;
    const int e = tid % E, sl = tid / E;
    const bool act = sl < S;
    const int per = (n_chunks + S - 1) / S;
    const int c0 = act ? min(n_chunks, sl * per) : n_chunks, c1 = min(n_chunks, c0 + per);
    int all = 0, before = 0;
    for (int c = c0; c < c1; c += G) {
        int v[G];
#pragma unroll
        for (int i = 0; i < G; ++i) v[i] = P.chunk_base[size_t(min(c + i, n_chunks - 1)) * E + e];
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const int n = c + i < c1 ? v[i] : 0;
            all += n;
            before += c + i < cb ? n : 0;
        }
    }
    part_all[tid] = act ? all : 0;
    part_before[tid] = act ? before : 0;
    for (int i = tid; i < kPermWaves * E; i += kPermThreads) wcnt[i] = 0;
    __syncthreads();
    int total = 0, bef = 0;
    if (tid < E) {
        for (int s = 0; s < S; ++s) {
            total += part_all[s * E + tid];
            bef += part_before[s * E + tid];
        }
    }
    int n_all, n_act, n_tiles;
    const int off = block_exclusive_scan(total, &n_all, sh);
    const int apos = block_exclusive_scan(total > 0 ? 1 : 0, &n_act, sh);
    const int nt = (total + P.tile_rows - 1) / P.tile_rows;
    const int tpos = block_exclusive_scan(P.tiles ? nt : 0, &n_tiles, sh);
    if (tid < E) {
        base_l[tid] = off + bef;
        if (blockIdx.x == 0) {
            P.offsets[tid] = off;
            if (total > 0) {
                P.active[apos] = tid;
                if (P.tiles) write_tiles(P.tiles, tpos, tid, off, total, P.tile_rows, P.max_tiles);
            }
        }
    }
    if (blockIdx.x == 0 && tid == 0) {
        P.offsets[E] = n_all;
        *P.n_active = n_act;
        if (P.n_tiles) *P.n_tiles = min(n_tiles, P.max_tiles);
    }
    __syncthreads();
    const int p = cb * chunk_pairs + tid;
    int ex = (tid < R * chunk_pairs && p < P.n_pairs) ? P.ids[p] : -1;
    const bool valid = ex >= 0 && ex < E;
    if (!valid) ex = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < P.id_bits; ++b) {
        const bool bit = (ex >> b) & 1;
        const uint64_t bb = __ballot(bit);
        peers &= bit ? bb : ~bb;
    }
    const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt);
    if (valid && rank == 0) wcnt[wave * E + ex] = uint16_t(__popcll(peers));
    __syncthreads();
    if (valid) {
        int bw = 0;
        for (int w = 0; w < wave; ++w) bw += wcnt[w * E + ex];
        P.sorted_pairs[base_l[ex] + bw + rank] = p;
    }
}

hipError_t launch_permute_from_counts(const PermParams& P, int n_chunks, int chunk_pairs, hipStream_t s) {
    if (P.E <= 0 || P.E > kCountsMaxE || chunk_pairs <= 0 || chunk_pairs > kPermThreads || n_chunks <= 0 ||
        !P.chunk_base)
        return hipErrorInvalidValue;
    const int R = kPermThreads / chunk_pairs;
    permute_from_counts_kernel<<<(n_chunks + R - 1) / R, kPermThreads, 0, s>>>(P, n_chunks, chunk_pairs);
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
