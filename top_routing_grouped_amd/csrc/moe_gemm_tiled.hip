// LDS-tiled bf16 MFMA kernels for the grouped expert GEMMs at large token
// counts (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens", "Routed
// expert computation" and "Shared expert computation"; the per-expert
// grouping follows the "Intel SYCL path": one tile works on one active
// expert's packed pairs, so each weight block is loaded for up to 128 of them).
//
// Workgroup tile: 128 weight rows x 128 token rows, K in steps of 64.  Two
// LDS buffers and two register buffers: the global loads of step k+2 are
// issued while step k's MFMAs run and step k+1's data moves from registers to
// LDS, one barrier per step.  For gate/up the 128 weight rows are 64 gate
// rows and the same 64 up rows, so each lane ends with matching gate and up
// accumulators and applies SwiGLU in registers.  4 waves in a 2 x 2 grid;
// each wave owns 64 weight rows x 64 tokens as 4 x 4 fragments of
// v_mfma_f32_16x16x32_bf16 (weights = A, tokens = B); token fragments past
// the tile's row count issue no MFMAs.  LDS rows are 128 bytes with the
// 16-byte pieces of row r XOR-swizzled by (r/2) mod 8, so both the 8-lanes-
// per-row stores and the 16-rows-per-fragment reads of a wave touch 16
// distinct 4-bank groups.
#include "moe_device.h"
#include "moe_kernels.h"

#include <type_traits>

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int BW = 128;       // weight rows per tile
constexpr int BT = 128;       // token rows per tile
constexpr int BK = 64;        // K per step
constexpr int kThreads = 256;

// LDS row layout: 0 = rows padded to 144 bytes, 1 = 128-byte rows with the
// 16-byte pieces XOR-swizzled by (r/2) mod 8, 2 = swizzled by r mod 8.
#ifndef MOE_TILED_LDS_LAYOUT
#define MOE_TILED_LDS_LAYOUT 1
#endif
// global prefetch distance in K steps (1 or 2)
#ifndef MOE_TILED_PREFETCH
#define MOE_TILED_PREFETCH 2
#endif
constexpr int kLayout = MOE_TILED_LDS_LAYOUT;
constexpr int kPrefetch = MOE_TILED_PREFETCH;
constexpr int RS = kLayout == 0 ? BK + 8 : BK;  // LDS row stride (elements)

// element offset of 16-byte piece p of LDS row r
__device__ __forceinline__ int lds_off(int r, int p) {
    if constexpr (kLayout == 0) return r * RS + (p << 3);
    else if constexpr (kLayout == 1) return r * RS + ((p ^ ((r >> 1) & 7)) << 3);
    else return r * RS + ((p ^ (r & 7)) << 3);
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base));
}

}  // namespace

template <int MODE, bool OUTBF>
__global__ __launch_bounds__(kThreads, 2) void gemm_tiled_kernel(GemmArgs a) {
    constexpr bool DUAL = (MODE == kRoutedGateUp || MODE == kDenseGateUp);
    constexpr bool ROUTED = (MODE == kRoutedGateUp || MODE == kRoutedDown);
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BW * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BT * RS];

    // XCD-aware order: workgroups are dispatched to the 8 XCDs round-robin,
    // so block b runs on XCD b % 8.  Each XCD takes one contiguous run of the
    // (tile, row block) work list, row block fastest: the row blocks of a
    // token tile (same gathered token rows) and neighbouring tiles of the same
    // expert (same weight rows) then share that XCD's L2.
    constexpr bool DUAL_ = DUAL;
    const int nrb = DUAL_ ? (a.N + 63) / 64 : (a.N + BW - 1) / BW;
    const int n_tiles_real = ROUTED ? uniform(*a.n_tiles) : (a.n_rows + BT - 1) / BT;
    const int n_items = n_tiles_real * nrb;
    const int chunk = (n_items + 7) / 8;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local >= chunk) return;
    const int item = xcd * chunk + local;
    if (item >= n_items) return;
    const int tile = item / nrb;
    const int row_blk = item - tile * nrb;

    int e = 0, begin, count;
    if constexpr (ROUTED) {
        const int4 t = a.tiles[tile];
        e = uniform(t.x); begin = uniform(t.y); count = uniform(t.z);
        if (e < 0 || e >= a.n_banks || begin < 0 || count <= 0 || begin + count > a.n_pairs) return;
    } else {
        begin = tile * BT;
        count = min(BT, a.n_rows - begin);
        if (count <= 0) return;
    }
    const int N = a.N, K = a.K;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, r = lane & 15;
    const int wm = wave & 1, wn = wave >> 1;
    // weight-row block row_blk: gate/up covers features [64*row_blk, +64) of both banks

    // ---- global load assignment: 4 pieces of 16 B per thread per operand
    // piece p = tid + 256*i: row p/8, 16-byte column p%8 (8 threads per 128-byte row segment)
    const uint16_t* wsrc[4];
    const uint16_t* xsrc[4];
    int lrow[4], lcol[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + kThreads * i;
        const int row = p >> 3, col = (p & 7) * 8;
        lrow[i] = row;
        lcol[i] = col;
        const uint16_t* wb;
        int wr;
        if constexpr (DUAL) {
            wb = static_cast<const uint16_t*>(row < 64 ? a.w0 : a.w1);
            wr = row_blk * 64 + (row & 63);
        } else {
            wb = static_cast<const uint16_t*>(a.w0);
            wr = row_blk * BW + row;
        }
        // Every load is unconditional (no branch, so no wait for older loads
        // inside the K loop): absent weight rows and token rows read a valid
        // row instead; they only feed output rows / token columns that are
        // never stored.
        wsrc[i] = wb + (size_t(e) * N + min(wr, N - 1)) * K + col;
        int arow = -1;
        if (row < count) {
            if constexpr (MODE == kRoutedGateUp) {
                const int pair = a.pairs[begin + row];
                arow = (pair >= 0 && pair < a.n_pairs) ? pair / a.topk : -1;
            } else {
                arow = begin + row;
            }
        }
        if (arow < 0 || arow >= a.n_act_rows) arow = 0;
        xsrc[i] = static_cast<const uint16_t*>(a.act) + size_t(arow) * K + col;
    }

    u32x4 wreg[2][4], xreg[2][4];
    auto gload = [&](int rb, int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wreg[rb][i] = *reinterpret_cast<const u32x4*>(wsrc[i] + k0);
            xreg[rb][i] = *reinterpret_cast<const u32x4*>(xsrc[i] + k0);
        }
    };
    int soff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) soff[i] = lds_off(lrow[i], lcol[i] >> 3);
    auto lstore = [&](int rb, int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<u32x4*>(&As[buf][soff[i]]) = wreg[rb][i];
            *reinterpret_cast<u32x4*>(&Bs[buf][soff[i]]) = xreg[rb][i];
        }
    };

    // wave's fragment rows inside the tile
    int arow_l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (DUAL)  // frags 0,1: gate rows; 2,3: the matching up rows
            arow_l[i] = (i >= 2 ? 64 : 0) + wm * 32 + (i & 1) * 16 + r;
        else
            arow_l[i] = wm * 64 + i * 16 + r;
    }
    const int brow_l = wn * 64 + r;
    // token fragments of this wave that hold at least one row
    const int nfrag = uniform(min(4, max(0, (count - wn * 64 + 15) / 16)));

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    // One K step: MFMAs from LDS buffer `cur`.  FULL: all 4 token fragments
    // hold rows (no per-fragment test inside the loop).
    auto compute = [&](int cur, auto full) {
        constexpr bool FULL = decltype(full)::value;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = lds_frag(&As[cur][lds_off(arow_l[i], ks * 4 + q)]);
#pragma unroll
            for (int j = 0; j < 4; ++j) bfr[j] = lds_frag(&Bs[cur][lds_off(brow_l + j * 16, ks * 4 + q)]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (!FULL && j >= nfrag) break;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
        }
    };
    auto main_loop = [&](auto full) {
        if constexpr (kPrefetch == 1) {
            gload(0, 0);
            lstore(0, 0);
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                const int cur = kt & 1;
                if (kt + 1 < nk) gload(0, (kt + 1) * BK);
                compute(cur, full);
                if (kt + 1 < nk) lstore(0, cur ^ 1);
                __syncthreads();
            }
        } else {
            // register buffers alternate with the K step; the loop is unrolled by
            // two so each buffer index is a compile-time constant.  The steady
            // state has no conditional load (a branch there makes the compiler
            // wait for the loads in flight); sched_barrier keeps each step's
            // prefetch at the top of the step, ahead of its MFMAs.
            gload(0, 0);
            if (nk > 1) gload(1, BK);
            lstore(0, 0);
            __syncthreads();
            int kt = 0;
            for (; kt + 3 < nk; kt += 2) {
                gload(0, (kt + 2) * BK);
                __builtin_amdgcn_sched_barrier(0);
                compute(0, full);
                lstore(1, 1);
                __syncthreads();
                gload(1, (kt + 3) * BK);
                __builtin_amdgcn_sched_barrier(0);
                compute(1, full);
                lstore(0, 0);
                __syncthreads();
            }
            // tail: 1 step (nk == 1), else 2 or 3 steps left; register buffer 1
            // holds step kt + 1 when nk > 1
            const int left = nk - kt;
            if (left == 3) gload(0, (kt + 2) * BK);
            compute(0, full);
            if (left >= 2) {
                lstore(1, 1);
                __syncthreads();
                compute(1, full);
                if (left == 3) {
                    lstore(0, 0);
                    __syncthreads();
                    compute(0, full);
                }
            }
        }
    };
    // the branch is on a wave-uniform value; a workgroup's waves may take
    // different branches (both reach the same barriers)
    if (nfrag == 4)
        main_loop(std::true_type{});
    else
        main_loop(std::false_type{});

    // ---- epilogue: lane holds rows (4q .. 4q+3) of fragment i, token column r of fragment j
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int tok = wn * 64 + j * 16 + r;
        if (tok >= count) continue;
        if constexpr (DUAL) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int f = row_blk * 64 + wm * 32 + i * 16 + 4 * q;
                if (f >= N) continue;
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float g = acc[i][j][t];
                    v[t] = g / (1.0f + __expf(-g)) * acc[i + 2][j][t];
                }
                const size_t o = size_t(begin + tok) * N + f;
                if constexpr (OUTBF)
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) =
                        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
                else
                    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o) = make_float4(v[0], v[1], v[2], v[3]);
            }
        } else {
            size_t dest;
            float s = 1.0f;
            if constexpr (MODE == kRoutedDown) {
                const int pair = a.pairs[begin + tok];
                if (pair < 0 || pair >= a.n_pairs) continue;
                dest = size_t(pair);
                s = a.row_scale[pair];
            } else if constexpr (MODE == kDenseDown) {
                dest = size_t(begin + tok);
                if (a.row_scale) s = sigmoidf_(a.row_scale[begin + tok]);
            } else {
                dest = size_t(begin + tok);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = row_blk * BW + wm * 64 + i * 16 + 4 * q;
                if (d >= N) continue;
                const float v0 = s * acc[i][j][0], v1 = s * acc[i][j][1], v2 = s * acc[i][j][2], v3 = s * acc[i][j][3];
                const size_t o = dest * N + d;
                if constexpr (OUTBF)
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + o) =
                        make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                else
                    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o) = make_float4(v0, v1, v2, v3);
            }
        }
    }
}

int tiled_rows() { return BT; }

hipError_t launch_gemm_tiled(int mode, bool outbf, const GemmArgs& a, int grid_x, hipStream_t s) {
    if (grid_x <= 0) return hipSuccess;
    const bool dual = (mode == kRoutedGateUp || mode == kDenseGateUp);
    const long long nrb = dual ? (a.N + 63) / 64 : (a.N + BW - 1) / BW;
    const long long items = (long long)grid_x * nrb;
    const dim3 g(unsigned(8 * ((items + 7) / 8)));
    switch (mode) {
        case kRoutedGateUp: gemm_tiled_kernel<kRoutedGateUp, true><<<g, kThreads, 0, s>>>(a); break;
        case kRoutedDown:
            if (outbf) gemm_tiled_kernel<kRoutedDown, true><<<g, kThreads, 0, s>>>(a);
            else gemm_tiled_kernel<kRoutedDown, false><<<g, kThreads, 0, s>>>(a);
            break;
        case kDenseGateUp: gemm_tiled_kernel<kDenseGateUp, true><<<g, kThreads, 0, s>>>(a); break;
        case kDenseDown: gemm_tiled_kernel<kDenseDown, false><<<g, kThreads, 0, s>>>(a); break;
        default: gemm_tiled_kernel<kDenseStore, false><<<g, kThreads, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace moe
