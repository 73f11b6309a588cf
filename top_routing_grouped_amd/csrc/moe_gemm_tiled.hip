// LDS-tiled bf16 MFMA kernels for the grouped expert GEMMs at large token
// counts (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens", "Routed
// expert computation" and "Shared expert computation"; the per-expert
// grouping follows the "Intel SYCL path": one tile works on one active
// expert's packed pairs, so each weight block is loaded once for up to a
// whole tile of them).
//
// Workgroup tile: BW weight rows x BT token rows, K in steps of 64, NW waves
// in a WM x WN grid; each wave owns (BW/WM) weight rows x (BT/WN) tokens as
// fragments of v_mfma_f32_16x16x32_bf16 (weights = A, tokens = B); token
// fragments past the tile's row count issue no MFMAs.  Two LDS buffers and
// PF register buffers: the global loads of step k+PF are issued while step
// k's MFMAs run, one barrier per step.  For gate/up the BW weight rows are
// BW/2 gate rows and the same BW/2 up rows, so each lane ends with matching
// gate and up accumulators and applies SwiGLU in registers.  LDS rows are 128
// bytes with the 16-byte pieces of row r XOR-swizzled by (r/2) mod 8, so both
// the 8-lanes-per-row stores and the 16-rows-per-fragment reads of a wave
// touch 16 distinct 4-bank groups.
//
// The kernel is bound by how many bytes the memory system keeps in flight for
// it (loaded latency is microseconds): the step time is about the latency
// divided by the number of steps in flight, so the tile is as large, and the
// register prefetch as deep, as the LDS and the register file allow.
#include "moe_device.h"
#include "moe_kernels.h"

#include <algorithm>
#include <type_traits>

namespace moe {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = 64;  // K per step
constexpr int RS = BK;  // LDS row stride (elements)

// Tile configuration: BW weight rows x BT tokens, NW waves as WM x WN, PF
// register prefetch stages, MINB workgroups per CU for the launch bounds.
template <int BW_, int BT_, int WM_, int WN_, int PF_, int MINB_>
struct Cfg {
    static constexpr int BW = BW_, BT = BT_, WM = WM_, WN = WN_, NW = WM_ * WN_, PF = PF_, MINB = MINB_;
    static constexpr int THREADS = NW * 64;
    static constexpr int FM = BW / WM / 16;  // weight fragments per wave
    static constexpr int FT = BT / WN / 16;  // token fragments per wave
    static constexpr int LA = BW * 8 / THREADS;  // 16-byte weight pieces per thread per step
    static constexpr int LB = BT * 8 / THREADS;  // 16-byte token pieces per thread per step
    static_assert(LA * THREADS == BW * 8 && LB * THREADS == BT * 8, "whole pieces per thread");
    static_assert(FM % 2 == 0, "gate/up pairs of fragments");
};
// Routed experts: 256 x 128, 8 waves of 64 x 64, two register stages ahead
// (64 accumulators + 2 x 24 staging registers + operands per lane fit the
// 256 registers of 2 waves per SIMD without spilling).  Measured at T = 4096
// against 256 x 256 (one stage: fewer steps in flight), 128 x 128 (two
// workgroups per CU: twice the bytes per MFMA) and 16-wave shapes (spills).
using CfgLarge = Cfg<256, 128, 4, 2, 2, 1>;
// 4-bit routed experts: the same tile with the 8 waves as 8 x 1, so that
// each weight fragment is dequantised by one wave only (measured at Qwen3.6
// shape, K = 4: T = 4096 layer 539 -> 484 us, T = 2048 363 -> 343 us against
// 4 x 2; 2 x 4: 662 and 470 us)
#ifndef MOE_U4_WM
#define MOE_U4_WM 8
#endif
using CfgU4 = Cfg<256, 128, MOE_U4_WM, 8 / MOE_U4_WM, 2, 1>;
// 4-bit experts with fewer pairs: 64-token tiles, whose smaller LDS stages
// leave room for a deeper ring (the weights, a quarter of the bf16 bytes,
// need more K steps in flight to keep enough bytes in flight)
using CfgU4M = Cfg<256, 64, MOE_U4_WM, 8 / MOE_U4_WM, 2, 1>;
// Dense products (shared expert, router logits): 128 x 128, 4 waves of
// 64 x 64, one register stage ahead, 2 workgroups per CU (a dense T = 4096
// product has too few 256 x 128 tiles to fill the chip).
using CfgSmall = Cfg<128, 128, 2, 2, 1, 2>;

// element offset of 16-byte piece p of LDS row r
__device__ __forceinline__ int lds_off(int r, int p) { return r * RS + ((p ^ ((r >> 1) & 7)) << 3); }

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* base) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base));
}

}  // namespace

template <int MODE, bool OUTBF, class C>
__global__ __launch_bounds__(C::THREADS, C::MINB) void gemm_tiled_kernel(GemmArgs a) {
    constexpr int BW = C::BW, BT = C::BT, WM = C::WM, FM = C::FM, FT = C::FT, LA = C::LA, LB = C::LB;
    constexpr int THREADS = C::THREADS, PF = C::PF;
    constexpr bool DUAL = (MODE == kRoutedGateUp || MODE == kDenseGateUp);
    constexpr bool ROUTED = (MODE == kRoutedGateUp || MODE == kRoutedDown);
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BW * RS];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BT * RS];

    // Work order: weight-stationary inside each expert (row block major,
    // the expert's token tiles fastest), so a weight block is fetched from
    // HBM once and re-read from L2 by the expert's other token tiles; the
    // gathered token rows (a few MiB) stay in the last-level cache.  XCD-aware:
    // workgroups are dispatched to the 8 XCDs round-robin, so block b runs on
    // XCD b % 8, and each XCD takes one contiguous run of the work list.
    constexpr int ROWS = DUAL ? BW / 2 : BW;  // output rows of a row block
    const int nrb = (a.N + ROWS - 1) / ROWS;
    const int n_tiles_real = ROUTED ? uniform(*a.n_tiles) : (a.n_rows + BT - 1) / BT;
    // dense store (router logits): K split ksplit ways into partial planes
    const int ksplit = (MODE == kDenseStore) ? max(a.ksplit, 1) : 1;
    const int n_items = n_tiles_real * nrb * ksplit;
    const int chunk = (n_items + 7) / 8;
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local >= chunk) return;
    const int item_k = xcd * chunk + local;
    if (item_k >= n_items) return;
    const int kz = item_k % ksplit, item = item_k / ksplit;
    // the expert's tiles [first, first + nt) own items [first*nrb, (first+nt)*nrb)
    int first = 0, nt = n_tiles_real;
    if constexpr (ROUTED) {
        const int w = uniform(a.tiles[item / nrb].w);
        first = w >> 16;
        nt = w & 0xffff;
        const int off = item - first * nrb;
        if (w < 0 || nt <= 0 || off < 0 || off >= nt * nrb) {  // no expert extent: plain order
            first = item / nrb;
            nt = 1;
        }
    }
    const int off = item - first * nrb;
    int row_blk = off / nt;
    int tile = first + (off - row_blk * nt);
    if (!ROUTED && a.tile_major) {
        tile = item / nrb;
        row_blk = item - tile * nrb;
    }

    int e = 0, begin, count;
    if constexpr (ROUTED) {
        const int4 t = a.tiles[tile];
        e = uniform(t.x); begin = uniform(t.y); count = uniform(t.z);
        if (e < 0 || e >= a.n_banks || begin < 0 || count <= 0 || count > BT || begin + count > a.n_pairs) return;
    } else {
        begin = tile * BT;
        count = min(BT, a.n_rows - begin);
        if (count <= 0) return;
    }
    const int N = a.N, K = a.K;
    const int klen = K / ksplit, kbase = kz * klen;  // this block's K range
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int q = lane >> 4, r = lane & 15;
    const int wm = wave % WM, wn = wave / WM;

    // ---- global load assignment: piece p = tid + THREADS*i is row p/8,
    // 16-byte column p%8 (8 threads per 128-byte row segment of a K step)
    const uint16_t* wsrc[LA];
    const uint16_t* xsrc[LB];
    int soff_a[LA], soff_b[LB];
#pragma unroll
    for (int i = 0; i < LA; ++i) {
        const int p = tid + THREADS * i;
        const int row = p >> 3, col = (p & 7) * 8;
        soff_a[i] = lds_off(row, col >> 3);
        const uint16_t* wb;
        int wr;
        if constexpr (DUAL) {
            wb = static_cast<const uint16_t*>(row < BW / 2 ? a.w0 : a.w1);
            wr = row_blk * (BW / 2) + (row & (BW / 2 - 1));
        } else {
            wb = static_cast<const uint16_t*>(a.w0);
            wr = row_blk * BW + row;
        }
        // Every load is unconditional (no branch, so no wait for older loads
        // inside the K loop): absent weight rows and token rows read a valid
        // row instead; they only feed output rows / token columns that are
        // never stored.
        wsrc[i] = wb + (size_t(e) * N + min(wr, N - 1)) * K + kbase + col;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int p = tid + THREADS * i;
        const int row = p >> 3, col = (p & 7) * 8;
        soff_b[i] = lds_off(row, col >> 3);
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
        xsrc[i] = static_cast<const uint16_t*>(a.act) + size_t(arow) * K + kbase + col;
    }

    u32x4 wreg[PF][LA], xreg[PF][LB];
    auto gload = [&](int rb, int k0) {
#pragma unroll
        for (int i = 0; i < LA; ++i) wreg[rb][i] = *reinterpret_cast<const u32x4*>(wsrc[i] + k0);
#pragma unroll
        for (int i = 0; i < LB; ++i) xreg[rb][i] = *reinterpret_cast<const u32x4*>(xsrc[i] + k0);
    };
    auto lstore = [&](int rb, int buf) {
#pragma unroll
        for (int i = 0; i < LA; ++i) *reinterpret_cast<u32x4*>(&As[buf][soff_a[i]]) = wreg[rb][i];
#pragma unroll
        for (int i = 0; i < LB; ++i) *reinterpret_cast<u32x4*>(&Bs[buf][soff_b[i]]) = xreg[rb][i];
    };

    // wave's fragment rows inside the tile
    int arow_l[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if constexpr (DUAL)  // the first FM/2 fragments: gate rows; the rest: the matching up rows
            arow_l[i] = (i >= FM / 2 ? BW / 2 : 0) + wm * (BW / 2 / WM) + (i % (FM / 2)) * 16 + r;
        else
            arow_l[i] = wm * (BW / WM) + i * 16 + r;
    }
    const int brow_l = wn * (BT / C::WN) + r;
    // token fragments of this wave that hold at least one row
    const int nfrag = uniform(min(FT, max(0, (count - wn * (BT / C::WN) + 15) / 16)));

    f32x4 acc[FM][FT];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = klen / BK;
    // One K step: MFMAs from LDS buffer `cur`.  FULL: all token fragments
    // hold rows (no per-fragment test inside the loop).
    auto compute = [&](int cur, auto full) {
        constexpr bool FULL = decltype(full)::value;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            bf16x8 af[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = lds_frag(&As[cur][lds_off(arow_l[i], ks * 4 + q)]);
#pragma unroll
            for (int j = 0; j < FT; ++j) {
                if (!FULL && j >= nfrag) break;
                const bf16x8 bfr = lds_frag(&Bs[cur][lds_off(brow_l + j * 16, ks * 4 + q)]);
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr, acc[i][j], 0, 0, 0);
            }
        }
    };
    auto main_loop = [&](auto full) {
        if constexpr (PF == 1) {
            gload(0, 0);
            lstore(0, 0);
            __syncthreads();
            for (int kt = 0; kt < nk; ++kt) {
                const int cur = kt & 1;
                if (kt + 1 < nk) gload(0, (kt + 1) * BK);
                __builtin_amdgcn_sched_barrier(0);
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
    if (nfrag == FT)
        main_loop(std::true_type{});
    else
        main_loop(std::false_type{});

    // ---- epilogue: lane holds rows (4q .. 4q+3) of fragment i, token column r of fragment j
#pragma unroll
    for (int j = 0; j < FT; ++j) {
        const int tok = wn * (BT / C::WN) + j * 16 + r;
        if (tok >= count) continue;
        if constexpr (DUAL) {
#pragma unroll
            for (int i = 0; i < FM / 2; ++i) {
                const int f = row_blk * (BW / 2) + wm * (BW / 2 / WM) + i * 16 + 4 * q;
                if (f >= N) continue;
                float v[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float g = acc[i][j][t];
                    v[t] = g / (1.0f + __expf(-g)) * acc[i + FM / 2][j][t];
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
            } else {  // dense store: partial plane kz
                dest = size_t(kz) * a.n_rows + begin + tok;
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int d = row_blk * BW + wm * (BW / WM) + i * 16 + 4 * q;
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

// Routed experts, persistent.  With an expert's d_ff-long K (down) an item
// is only a few K steps, and the plain kernel waits on memory several times
// per item: decoding the item (two dependent loads), the token rows, the
// first K steps, and the pair ids and routing weights of its stores.  Here
// one workgroup per CU walks its XCD's run of items (the same weight-
// stationary order) and hides all of that behind the previous item: the
// item list is decoded into LDS once, the pair ids that locate token rows
// (gate/up, two items ahead) and the next item's store targets (down) are
// loaded while the current item's K loop runs, and the next item's first two
// K steps are loaded during the current item's last two.  Loads are buffer
// loads from scalar bases (the weight block, the token matrix) with fixed
// per-lane offsets, so switching items changes no VGPR address, and the
// weight rows past the matrix read zero (record count of the resource).
constexpr int kPersistMaxItems = 64;  // items per workgroup (LDS table)
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format (gfx9)

// ---- K steps straight into LDS
// The K steps go from global memory straight into a ring of three LDS stages
// (buffer loads with the LDS bit: lane i's 16 bytes land at the stage's
// address + 16 i, so each lane loads the piece that the XOR swizzle puts at
// its slot), two steps ahead: no staging registers and no LDS write
// instructions.  Waits are explicit: the vector memory counter retires in
// order, so "at most N newer operations in flight" is exact when every
// operation between two waits has a fixed count per wave.  Per K step each
// wave issues kDmaPerStep loads; the stores of an item are kStores buffer
// stores (masked elements go to an offset past the buffer, which the
// hardware drops) and the next item's prefetch is a fixed number of loads.
// The barrier is a bare s_barrier: the workgroup fence of __syncthreads would
// wait for every load in flight.
template <int N>
__device__ __forceinline__ void vm_wait_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0 << 8) | (7 << 4) | (N & 15));
}
__device__ __forceinline__ void bare_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))
// 16 bytes per lane from a buffer straight into LDS at dst + 16 * lane.  A
// plain device function: inside the kernel template the builtin made the
// host compilation pass drop the kernel's launch stub without a diagnostic.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff, int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(dst), 16, voff, soff, 0, 0);
}
// Fragment reads from the ring are inline asm: the compiler, seeing a plain
// LDS read while DMA into the same array is in flight, waits for every load
// in flight (it cannot tell the stages apart).  After the asm reads, an
// explicit lgkmcnt(0) wait that names the fragments as operands keeps their
// uses (the MFMAs) behind it.
__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ uint32_t ds_read4(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ u32x2 ds_read8(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ uint32_t ds_read_u16(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_u16 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}
__device__ __forceinline__ void lgkm_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void tie(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(u32x2& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie(uint32_t& v) { asm volatile("" : "+v"(v)); }
// 4 bytes per lane from a buffer straight into LDS at dst + 4 * lane
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(dst), 4, voff, 0, 0, 0);
}
constexpr uint32_t kDropOffset = 0x80000000u;  // past every buffer: the store is dropped

// KS: K elements per step (64 or 32); NST: LDS stages, the DMA running
// PD = NST - 1 steps ahead of the MFMAs.  U4G > 0: 4-bit affine group-64
// weights whose rows hold at most U4G groups (below); 0: bf16 weights.
//
// 4-bit weights: a K step is one group of 64 codes, 32 bytes of each weight
// row, so the A part of a stage is a quarter of the bf16 one.  The group
// scales and mins of an item's rows (one contiguous block of each array,
// [rows][K/64] bf16, as they lie in memory) go into one of two LDS buffers
// by DMA in the first K step of the item before (the barrier of that step
// is the one after which no wave reads that buffer for the item before
// it).  Each lane dequantises its A fragment (8 codes -> bf16 of
// scale * q + min, the rounding of the register-streaming kernels) right
// before the MFMAs that use it, so every code is dequantised once per wave
// that holds its row and used against all of the wave's token fragments.
// The K order inside a step differs from the bf16 one: lane-group q takes
// the 16 contiguous codes at 16q (8 bytes, one LDS read for both 32-wide
// MFMA steps), so its token operand is the 16-byte pieces 2q and 2q+1.
template <int MODE, bool OUTBF, class C, int KS, int NST, int U4G>
__global__ __launch_bounds__(C::THREADS, 1) void gemm_routed_dma_kernel(GemmArgs a) {
    constexpr int BW = C::BW, BT = C::BT, WM = C::WM, WN = C::WN, FM = C::FM, FT = C::FT;
    constexpr int NW = C::NW;
    constexpr bool DUAL = (MODE == kRoutedGateUp);
    constexpr bool U4 = U4G > 0;
    constexpr int ROWS = DUAL ? BW / 2 : BW;
    constexpr int PD = NST - 1;             // steps in flight ahead of the one computed
    constexpr int RSK = KS;                 // LDS row stride (elements)
    constexpr int PPR = KS / 8;             // 16-byte pieces per LDS row
    constexpr int RPC = 64 / PPR;           // rows one 64-lane DMA call covers
    constexpr int ARB = U4 ? KS / 2 : KS * 2;  // bytes of an A row per K step
    constexpr int ARPC = 1024 / ARB;        // A rows one 64-lane DMA call covers
    constexpr int AEL = BW * ARB / 2;       // elements of the A part of a stage
    constexpr int STAGE = AEL + BT * RSK;   // elements: A rows then B rows
    constexpr int AJ = BW / ARPC / NW;      // ARPC-row A blocks per wave per step
    constexpr int BJ = BT / RPC / NW;       // RPC-row B blocks per wave per step
    constexpr int kDmaPerStep = AJ + BJ;
    constexpr int kStores = DUAL ? FT * FM / 2 : FT * FM;
    constexpr int kPrefetch = DUAL ? 1 : 2 * FT;
    // 4-bit scale staging: NSA arrays (gate scale, gate min, up scale, up
    // min; down: scale, min) of ROWS x U4G bf16 per buffer, kSc DMA calls
    // of 1 KB per wave per item
    constexpr int NSA = DUAL ? 4 : 2;
    constexpr int SCB = U4 ? ROWS * U4G * 2 : 0;  // bytes per array
    constexpr int CPA = SCB / 1024;               // DMA calls per array
    constexpr int kSc = U4 ? NSA * CPA / NW : 0;
    static_assert(KS == 32 || KS == 64, "K steps of one or two 32-wide MFMA steps");
    static_assert(!U4 || KS == 64, "4-bit: a K step is one group of 64");
    static_assert(!U4 || (SCB % 1024 == 0 && kSc * NW == NSA * CPA && CPA % kSc == 0),
                  "whole scale DMA calls per wave, each wave's inside one array");
    static_assert(MODE == kRoutedGateUp || MODE == kRoutedDown, "routed modes");
    static_assert(AJ * ARPC * NW == BW && BJ * RPC * NW == BT, "whole row blocks per wave");
    static_assert(!DUAL || (NW / 2) * AJ * ARPC == BW / 2, "a wave's A rows lie in the gate or the up half");
    static_assert((PD - 1) * kDmaPerStep + kStores + kPrefetch + kSc < 64 && PD * kDmaPerStep < 64, "vmcnt range");
    static_assert(RPC * BJ <= 64, "one pair id per lane covers the wave's B rows");
    __shared__ __attribute__((aligned(16))) uint16_t lds[NST][STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t sc_lds[U4 ? 2 : 1][U4 ? NSA * SCB : 16];
    __shared__ int4 items[kPersistMaxItems];
    // gate/up: pair ids of the item after next, 64 per wave (one DMA per item)
    __shared__ uint32_t pair_ids[DUAL ? NW * 64 : 1];

    const int N = a.N, K = a.K, nk = K / KS;
    const int nrb = (N + ROWS - 1) / ROWS;
    const int n_items = uniform(*a.n_tiles) * nrb;
    const int chunk = (n_items + 7) / 8;
    const int xcd = blockIdx.x & 7, l = blockIdx.x >> 3, nl = gridDim.x >> 3;
    const int it0 = xcd * chunk + l, it_end = min((xcd + 1) * chunk, n_items);
    const int n_mine = uniform(it0 < it_end ? min(kPersistMaxItems, (it_end - it0 + nl - 1) / nl) : 0);
    if (n_mine == 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int q = lane >> 4, r = lane & 15;
    const int wm = wave % WM, wn = wave / WM;

    if (tid < n_mine) {
        const int item = it0 + nl * tid;
        const int w = a.tiles[item / nrb].w;
        int first = w >> 16, nt = w & 0xffff;
        const int o0 = item - first * nrb;
        if (w < 0 || nt <= 0 || o0 < 0 || o0 >= nt * nrb) {
            first = item / nrb;
            nt = 1;
        }
        const int off = item - first * nrb, row_blk = off / nt, tile = first + (off - row_blk * nt);
        const int4 t = a.tiles[tile];
        const bool ok = t.x >= 0 && t.x < a.n_banks && t.y >= 0 && t.z > 0 && t.z <= BT && t.y + t.z <= a.n_pairs;
        items[tid] = ok ? make_int4(t.x, t.y, t.z, row_blk) : make_int4(0, 0, 0, 0);
    }
    __syncthreads();

    // ---- this lane's DMA pieces: A block j covers tile rows wave*RPC*AJ +
    // RPC*j .. + RPC-1, lane = PPR * (row in block) + slot; the slot holds
    // logical 16-byte piece slot ^ ((row >> 1) & (PPR - 1))
    uint32_t aoff[AJ];
    int brow[BJ], bpiece[BJ];
#pragma unroll
    for (int j = 0; j < AJ; ++j) {
        if constexpr (U4) {  // 4-bit rows: 2 pieces per step, unswizzled
            const int ra = wave * ARPC * AJ + ARPC * j + lane / 2;
            aoff[j] = uint32_t((DUAL ? (ra & (BW / 2 - 1)) : ra) * (K / 2) + 16 * (lane & 1));
        } else {
            const int ra = wave * RPC * AJ + RPC * j + lane / PPR;
            const int p = (lane % PPR) ^ ((ra >> 1) & (PPR - 1));
            aoff[j] = uint32_t(((DUAL ? (ra & (BW / 2 - 1)) : ra) * K + 8 * p) * 2);
        }
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
        brow[j] = wave * RPC * BJ + RPC * j + lane / PPR;
        bpiece[j] = (lane % PPR) ^ ((brow[j] >> 1) & (PPR - 1));
    }
    const bool up_wave = DUAL && wave * ARPC * AJ >= BW / 2;
    const auto rs_x = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.act), 0,
                                                        uint32_t(size_t(a.n_act_rows) * K * 2), kRsrcWord3);
    const auto rs_out = __builtin_amdgcn_make_buffer_rsrc(
        a.out, 0, uint32_t(size_t(a.n_pairs) * N * (OUTBF ? 2 : 4)), kRsrcWord3);
    const auto rs_pairs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.pairs), 0,
                                                            uint32_t(a.n_pairs) * 4u, kRsrcWord3);
    // this wave's weight rows of an item (gate/up: gate or up half by wave)
    auto w_rsrc = [&](int4 it) __attribute__((always_inline)) {
        const int r0 = it.w * ROWS;
        const void* bank = up_wave ? a.w1 : a.w0;
        constexpr int EB = U4 ? 1 : 4;  // (bytes per element) x 2
        const uint8_t* p = static_cast<const uint8_t*>(bank) + (size_t(it.x) * N + r0) * K * EB / 2;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0,
                                                 uint32_t(min(ROWS, N - r0) * K * EB / 2), kRsrcWord3);
    };
    // 4-bit: the group scales and mins of an item's rows into scale buffer
    // buf; wave w's kSc calls lie in one array
    const int G = K / 64;
    auto scale_dma = [&](int4 it, int buf) __attribute__((always_inline)) {
        if constexpr (U4) {
            const int r0 = it.w * ROWS;
            const int arr = (wave * kSc) / CPA, ch0 = (wave * kSc) % CPA;
            const void* base = arr == 0 ? a.s0 : arr == 1 ? a.m0 : arr == 2 ? a.s1 : a.m1;
            const uint8_t* p = static_cast<const uint8_t*>(base) + (size_t(it.x) * N + r0) * G * 2;
            const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), 0,
                                                              uint32_t(min(ROWS, N - r0) * G * 2), kRsrcWord3);
            uint8_t* dst = &sc_lds[buf][arr * SCB + ch0 * 1024];
#pragma unroll
            for (int j = 0; j < kSc; ++j) dma16(rs, dst + j * 1024, uint32_t((ch0 + j) * 1024 + 16 * lane), 0);
        }
    };
    auto item_at = [&](int m) __attribute__((always_inline)) {
        const int4 t = items[m];
        return make_int4(uniform(t.x), uniform(t.y), uniform(t.z), uniform(t.w));
    };
    auto pair_index = [&](int4 it, int row) __attribute__((always_inline)) {
        return it.y + (row < it.z ? row : 0);
    };
    // byte offset of this lane's piece of a token row; rows past the tile
    // (partial tiles: every cold expert's, each expert's last) get an
    // offset past the buffer's records, which the hardware answers with
    // zeros and no memory request (their columns are never stored)
    auto x_offset = [&](int j, int pair_or_row, bool valid) __attribute__((always_inline)) {
        int arow = pair_or_row;
        if constexpr (DUAL) arow = (pair_or_row >= 0 && pair_or_row < a.n_pairs) ? pair_or_row / a.topk : -1;
        if (!valid || arow < 0 || arow >= a.n_act_rows) return kDropOffset;
        return uint32_t((arow * K + 8 * bpiece[j]) * 2);
    };
    // K step kt of an item into LDS stage st
    auto dma = [&](int st, const __amdgpu_buffer_rsrc_t& rw, const uint32_t (&xo)[BJ], int kt)
                   __attribute__((always_inline)) {
        const int so = kt * KS * 2;
        uint16_t* base = &lds[st][0];
#pragma unroll
        for (int j = 0; j < AJ; ++j)
            dma16(rw, base + (wave * ARPC * AJ + ARPC * j) * (ARB / 2), aoff[j], kt * ARB);
#pragma unroll
        for (int j = 0; j < BJ; ++j)
            dma16(rs_x, base + (AEL + (wave * RPC * BJ + RPC * j) * RSK), xo[j], so);
    };
    // element offset of 16-byte piece p of LDS row r of a stage
    auto soff = [](int r, int p) __attribute__((always_inline)) { return r * RSK + ((p ^ ((r >> 1) & (PPR - 1))) << 3); };

    int arow_l[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if constexpr (DUAL)
            arow_l[i] = (i >= FM / 2 ? BW / 2 : 0) + wm * (BW / 2 / WM) + (i % (FM / 2)) * 16 + r;
        else
            arow_l[i] = wm * (BW / WM) + i * 16 + r;
    }
    const int brow_l = wn * (BT / WN) + r;
    f32x4 acc[FM][FT];
    constexpr int NKS = KS / 32;  // 32-wide MFMA steps per K step
    // byte offsets of the wave's fragments inside a stage: [ks][fragment]
    // (4-bit A: one 8-byte read per fragment for both ks, at aofs[0])
    uint32_t aofs[NKS][FM], bofs[NKS][FT];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
            aofs[ks][i] = U4 ? uint32_t(arow_l[i] * ARB + 8 * q) : uint32_t(soff(arow_l[i], ks * 4 + q) * 2);
#pragma unroll
        for (int jj = 0; jj < FT; ++jj)
            bofs[ks][jj] = uint32_t((AEL + soff(brow_l + jj * 16, U4 ? 2 * q + ks : ks * 4 + q)) * 2);
    }
    // 4-bit: byte offset of fragment i's row scale in a scale buffer (its
    // min is SCB further)
    uint32_t scofs[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int arr = (DUAL && i >= FM / 2) ? 2 : 0;
        const int row = DUAL ? (arow_l[i] & (BW / 2 - 1)) : arow_l[i];
        scofs[i] = uint32_t(arr * SCB + row * G * 2);
    }
    const uint32_t lds0 = lds_byte_addr(&lds[0][0]);
    const uint32_t sc0 = lds_byte_addr(&sc_lds[0][0]);
    auto compute_u4 = [&](int st, auto nf_c, int kt, int buf) __attribute__((always_inline)) {
        constexpr int NF = decltype(nf_c)::value;
        if constexpr (NF > 0) {
            const uint32_t sb = lds0 + uint32_t(st * STAGE * 2);
            const uint32_t scb = sc0 + uint32_t(buf * NSA * SCB + 2 * kt);
            u32x2 cw[FM];
            uint32_t sw[FM], mw[FM];
            u32x4 bfv[NKS][NF];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                cw[i] = ds_read8(sb + aofs[0][i]);
                sw[i] = ds_read_u16(scb + scofs[i]);
                mw[i] = ds_read_u16(scb + scofs[i] + SCB);
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int jj = 0; jj < NF; ++jj) bfv[ks][jj] = ds_read16(sb + bofs[ks][jj]);
            lgkm_wait_all();
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                tie(cw[i]);
                tie(sw[i]);
                tie(mw[i]);
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int jj = 0; jj < NF; ++jj) tie(bfv[ks][jj]);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const float sc = bf16_lo(sw[i]), mn = bf16_lo(mw[i]);
                    const uint32_t w = ks == 0 ? cw[i].x : cw[i].y;
                    uint32_t even, odd;
                    nibble_bytes<true>(w, even, odd);
                    u32x4 af;
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        af[b] = pack_bf16x2(fmaf(sc, float((even >> (8 * b)) & 0xffu), mn),
                                            fmaf(sc, float((odd >> (8 * b)) & 0xffu), mn));
#pragma unroll
                    for (int jj = 0; jj < NF; ++jj)
                        acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, af), __builtin_bit_cast(bf16x8, bfv[ks][jj]), acc[i][jj], 0, 0, 0);
                }
            }
        }
    };
    auto compute = [&](int st, auto nf_c) __attribute__((always_inline)) {
        constexpr int NF = decltype(nf_c)::value;
        const uint32_t sb = lds0 + uint32_t(st * STAGE * 2);
        u32x4 af[NKS][FM], bfv[NKS][NF > 0 ? NF : 1];
        auto reads = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < FM; ++i) af[ks][i] = ds_read16(sb + aofs[ks][i]);
#pragma unroll
            for (int jj = 0; jj < NF; ++jj) bfv[ks][jj] = ds_read16(sb + bofs[ks][jj]);
        };
        auto ready = [&](int ks) __attribute__((always_inline)) {
            lgkm_wait_all();
#pragma unroll
            for (int i = 0; i < FM; ++i) tie(af[ks][i]);
#pragma unroll
            for (int jj = 0; jj < NF; ++jj) tie(bfv[ks][jj]);
        };
        auto mfmas = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
            for (int jj = 0; jj < NF; ++jj)
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[ks][i]),
                                                                         __builtin_bit_cast(bf16x8, bfv[ks][jj]),
                                                                         acc[i][jj], 0, 0, 0);
        };
        if constexpr (NF > 0) {
            reads(0);
            ready(0);
            if constexpr (NKS == 2) {
                reads(1);  // in flight during the first half's MFMAs
                mfmas(0);
                ready(1);
                mfmas(1);
            } else {
                mfmas(0);
            }
        }
    };

    // ---- prologue: first item's token rows and store targets, its first two
    // K steps, and kStores dropped stores so every item starts with the same
    // count of operations in flight
    int4 cur = item_at(0);
    uint32_t xo_cur[BJ], xo_nxt[BJ];
    int ep_cur[FT], ep_nxt[FT];
    float es_cur[FT];
    {
        const int4 n1 = item_at(min(1, n_mine - 1));
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
            const int v = DUAL ? a.pairs[pair_index(cur, brow[j])] : cur.y + brow[j];
            xo_cur[j] = x_offset(j, v, brow[j] < cur.z);
            const int v1 = DUAL ? a.pairs[pair_index(n1, brow[j])] : n1.y + brow[j];
            xo_nxt[j] = x_offset(j, v1, brow[j] < n1.z);
        }
    }
    if constexpr (!DUAL) {
#pragma unroll
        for (int j = 0; j < FT; ++j) ep_cur[j] = a.pairs[pair_index(cur, wn * (BT / WN) + j * 16 + r)];
    }
    auto rw_cur = w_rsrc(cur);
    scale_dma(cur, 0);
#pragma unroll
    for (int st = 0; st < PD; ++st) dma(st, rw_cur, xo_cur, st);
#pragma unroll
    for (int i = 0; i < kStores; ++i) {  // distinct offsets: identical stores would be merged
        if constexpr (OUTBF || DUAL)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, rs_out, kDropOffset + 16u * i, 0, 0);
        else
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, rs_out, kDropOffset + 16u * i, 0, 0);
    }
    int g = 0;  // global K step: LDS stage g % NST

    // Token-row offsets are formed one item ahead of their first DMA: the
    // pair ids of the item after next go into LDS by DMA at an item's top
    // and are turned into offsets right after the wait that ends its K loop
    // (which leaves only that loop's newest DMA in flight, so they have
    // landed; the wave reads only what it loaded itself).  Plain loads there
    // cost a full memory round trip per item: the compiler drained the
    // memory counter ahead of each item's K loop when that loop used them,
    // and at the K loop's end otherwise (its wait model does not count the
    // LDS DMA).
    for (int m = 0; m < n_mine; ++m) {
        const int4 nxt = item_at(min(m + 1, n_mine - 1));
        const auto rw_nxt = w_rsrc(nxt);
        // item-top prefetch, kPrefetch loads: the pair ids of the item after
        // next (gate/up: its token rows) or the next item's store rows
        // (down), and this item's routing weights
        const int4 nx2 = item_at(min(m + 2, n_mine - 1));
        if constexpr (DUAL)  // lane l: the pair id of the wave's row l mod RPC BJ (past the end: zero)
            dma4(rs_pairs, &pair_ids[wave * 64], uint32_t(nx2.y + wave * RPC * BJ + (lane & (RPC * BJ - 1))) * 4u);
        if constexpr (!DUAL) {
#pragma unroll
            for (int jj = 0; jj < FT; ++jj) {
                ep_nxt[jj] = a.pairs[pair_index(nxt, wn * (BT / WN) + jj * 16 + r)];
                const int pc = ep_cur[jj];
                es_cur[jj] = a.row_scale[(pc >= 0 && pc < a.n_pairs) ? pc : 0];
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jj = 0; jj < FT; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int nfrag = uniform(min(FT, max(0, (cur.z - wn * (BT / WN) + 15) / 16)));

        auto run = [&](auto nf_c) __attribute__((always_inline)) {
            auto step = [&](int kt, bool first) __attribute__((always_inline)) {
                // one DMA call with its operands selected element by element:
                // two calls on the two arrays were merged by the compiler into
                // one call on a selected array address, which put both arrays
                // in scratch memory
                const int st = (g + PD) % NST;
                const bool same = kt + PD < nk;
                uint32_t xo_s[BJ];
#pragma unroll
                for (int jj = 0; jj < BJ; ++jj) xo_s[jj] = same ? xo_cur[jj] : xo_nxt[jj];
                dma(st, same ? rw_cur : rw_nxt, xo_s, same ? kt + PD : kt + PD - nk);
                if constexpr (U4) {
                    if (first) scale_dma(nxt, (m + 1) & 1);
                    compute_u4(g % NST, nf_c, kt, m & 1);
                } else {
                    compute(g % NST, nf_c);
                }
                ++g;
            };
            // Newer than step kt's DMA at its wait: kt < PD: the DMA of
            // steps kt+1 .. PD-1 (issued by the previous item), the previous
            // item's stores, this item's prefetch and the DMA of steps 0 ..
            // kt-1, i.e. (PD-1) steps' DMA + stores + prefetch, plus the
            // scale DMA issued in step 0 for kt >= 1; kt = PD: the scale DMA
            // and PD-1 steps' DMA; later steps: PD-1 steps' DMA
            vm_wait_lgkm0<(PD - 1) * kDmaPerStep + kStores + kPrefetch>();
            bare_barrier();
            step(0, true);
#pragma unroll
            for (int kt = 1; kt < PD; ++kt) {
                vm_wait_lgkm0<(PD - 1) * kDmaPerStep + kStores + kPrefetch + kSc>();
                bare_barrier();
                step(kt, false);
            }
            if (nk > PD) {
                vm_wait_lgkm0<(PD - 1) * kDmaPerStep + kSc>();
                bare_barrier();
                step(PD, false);
            }
            for (int kt = PD + 1; kt < nk; ++kt) {
                vm_wait_lgkm0<(PD - 1) * kDmaPerStep>();
                bare_barrier();
                step(kt, false);
            }
        };
        auto dispatch = [&](auto self, auto nf_c) __attribute__((always_inline)) {
            constexpr int NF = decltype(nf_c)::value;
            if constexpr (NF == 0)
                run(nf_c);
            else if (nfrag == NF)
                run(nf_c);
            else
                self(self, std::integral_constant<int, NF - 1>{});
        };
        dispatch(dispatch, std::integral_constant<int, FT>{});
        // exactly the PD newest steps' DMA may be in flight here; everything
        // older (the prefetch) is complete
        vm_wait_lgkm0<PD * kDmaPerStep>();
        uint32_t xo_nn[BJ];
        if constexpr (DUAL) {
            uint32_t pid[BJ];
#pragma unroll
            for (int jj = 0; jj < BJ; ++jj)
                pid[jj] = ds_read4(lds_byte_addr(&pair_ids[wave * 64]) + 4u * uint32_t(brow[jj] - wave * RPC * BJ));
            lgkm_wait_all();
#pragma unroll
            for (int jj = 0; jj < BJ; ++jj) {
                tie(pid[jj]);
                xo_nn[jj] = x_offset(jj, int(pid[jj]), brow[jj] < nx2.z);
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < BJ; ++jj) xo_nn[jj] = x_offset(jj, nx2.y + brow[jj], brow[jj] < nx2.z);
        }

        // ---- stores: kStores buffer stores per wave, masked ones dropped
        const int begin = cur.y, count = cur.z, row_blk = cur.w;
#pragma unroll
        for (int j = 0; j < FT; ++j) {
            const int tok = wn * (BT / WN) + j * 16 + r;
            const bool tok_ok = tok < count;
            if constexpr (DUAL) {
#pragma unroll
                for (int i = 0; i < FM / 2; ++i) {
                    const int f = row_blk * (BW / 2) + wm * (BW / 2 / WM) + i * 16 + 4 * q;
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float gt = acc[i][j][t];
                        v[t] = gt / (1.0f + __expf(-gt)) * acc[i + FM / 2][j][t];
                    }
                    const uint32_t o = (tok_ok && f < N) ? uint32_t(((begin + tok) * N + f) * 2) : kDropOffset;
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])},
                                                          rs_out, o, 0, 0);
                }
            } else {
                const int pair = ep_cur[j];
                const bool ok = tok_ok && pair >= 0 && pair < a.n_pairs;
                const float s = es_cur[j];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int d = row_blk * BW + wm * (BW / WM) + i * 16 + 4 * q;
                    const bool st_ok = ok && d < N;
                    const float v0 = s * acc[i][j][0], v1 = s * acc[i][j][1], v2 = s * acc[i][j][2],
                                v3 = s * acc[i][j][3];
                    if constexpr (OUTBF) {
                        const uint32_t o = st_ok ? uint32_t((pair * N + d) * 2) : kDropOffset;
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)},
                                                              rs_out, o, 0, 0);
                    } else {
                        const uint32_t o = st_ok ? uint32_t((pair * N + d) * 4) : kDropOffset;
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4{__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)},
                            rs_out, o, 0, 0);
                    }
                }
            }
        }
        cur = nxt;
        rw_cur = rw_nxt;
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
            xo_cur[j] = xo_nxt[j];
            xo_nxt[j] = xo_nn[j];
        }
        if constexpr (!DUAL) {
#pragma unroll
            for (int j = 0; j < FT; ++j) ep_cur[j] = ep_nxt[j];
        }
    }
    vm_wait_lgkm0<0>();
}

int tiled_rows() { return CfgLarge::BT; }
int tiled_rows_dense() { return CfgSmall::BT; }

template <class C>
static hipError_t launch_cfg(int mode, bool outbf, const GemmArgs& a, int grid_x, hipStream_t s) {
    const bool dual = (mode == kRoutedGateUp || mode == kDenseGateUp);
    const int rows = dual ? C::BW / 2 : C::BW;
    const long long nrb = (a.N + rows - 1) / rows;
    const long long items = (long long)grid_x * nrb * (mode == kDenseStore ? std::max(a.ksplit, 1) : 1);
    const dim3 g(unsigned(8 * ((items + 7) / 8)));
    const dim3 b(C::THREADS);
    switch (mode) {
        case kRoutedGateUp: gemm_tiled_kernel<kRoutedGateUp, true, C><<<g, b, 0, s>>>(a); break;
        case kRoutedDown:
            if (outbf) gemm_tiled_kernel<kRoutedDown, true, C><<<g, b, 0, s>>>(a);
            else gemm_tiled_kernel<kRoutedDown, false, C><<<g, b, 0, s>>>(a);
            break;
        case kDenseGateUp: gemm_tiled_kernel<kDenseGateUp, true, C><<<g, b, 0, s>>>(a); break;
        case kDenseDown: gemm_tiled_kernel<kDenseDown, false, C><<<g, b, 0, s>>>(a); break;
        default: gemm_tiled_kernel<kDenseStore, false, C><<<g, b, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

// Routed modes use the large tile (grid_x = routed tiles of tiled_rows()
// pairs); dense modes the small one (grid_x = token tiles of
// tiled_rows_dense() tokens).
// Persistent routed launch: one workgroup per CU (at most), each XCD's 32
// taking its run of items in turn.  Needs whole K steps (at least NST - 1
// per item; 4-bit: NST, so that an item's scale DMA, issued in its first
// step, is older than the next item's first K step), byte offsets inside
// 32 bits and at most kPersistMaxItems items per workgroup.
#ifndef MOE_PERSIST_KS
#define MOE_PERSIST_KS 64
#endif
constexpr int kPersistKS = MOE_PERSIST_KS;           // K per step of the persistent kernel
constexpr int kPersistNST = kPersistKS == 64 ? 3 : 6;  // LDS stages: 144 KB either way
constexpr int kU4NST = 3;                            // 4-bit: 72 KB of stages + 64 KB of scales
#ifndef MOE_U4M_NST
#define MOE_U4M_NST 4
#endif
constexpr int kU4MNST = MOE_U4M_NST;                 // 64-token tiles: 64 KB of stages + 64 KB of scales
constexpr int kU4MaxGroupsTiled = 32;                // 4-bit rows: K up to 2048
constexpr int kU4DownSmallGroups = 8;                // 4-bit down rows up to K = 512: smaller scale buffers

static int persist_groups(int mode, bool u4, int N, int K, int max_tiles, int n_act_rows, int n_pairs, bool outbf,
                          int nst) {
    using C = CfgLarge;
    const int KS = u4 ? 64 : kPersistKS, NST = nst;
    const int rows = mode == kRoutedGateUp ? C::BW / 2 : C::BW;
    if (N <= 0 || K <= 0 || max_tiles <= 0) return 0;
    const long long max_items = (long long)max_tiles * ((N + rows - 1) / rows);
    const long long per_xcd = (max_items + 7) / 8;
    const int nl = int(std::min<long long>(32, per_xcd));
    if (nl <= 0 || K % KS || K / KS < (u4 ? NST : NST - 1) || (per_xcd + nl - 1) / nl > kPersistMaxItems) return 0;
    if ((unsigned long long)n_act_rows * K * 2 >= (1ull << 32) || (unsigned long long)rows * K * 2 >= (1ull << 32))
        return 0;
    // stores address the output with 32-bit offsets below the drop offset
    if ((unsigned long long)n_pairs * N * (outbf || mode == kRoutedGateUp ? 2 : 4) >= (1ull << 31)) return 0;
    if (u4 && K / 64 > kU4MaxGroupsTiled) return 0;
    return nl;
}

int tiled_rows_u4_medium() { return CfgU4M::BT; }

bool routed_tiled_u4_fits(int mode, int tile_rows, int N, int K, int max_tiles, int n_act_rows, int n_pairs,
                          bool outbf) {
    if (tile_rows != CfgU4::BT && tile_rows != CfgU4M::BT) return false;
    const int nst = tile_rows == CfgU4::BT ? kU4NST : kU4MNST;
    return persist_groups(mode, true, N, K, max_tiles, n_act_rows, n_pairs, outbf, nst) > 0;
}

template <class U, int NST>
static void launch_u4(int mode, bool outbf, const GemmArgs& a, dim3 g, hipStream_t s) {
    static_assert(U::BW == CfgLarge::BW && U::THREADS == CfgLarge::THREADS, "same weight rows and threads");
    constexpr int GU = kU4MaxGroupsTiled, GD = kU4DownSmallGroups;
    const dim3 b(U::THREADS);
    if (mode == kRoutedGateUp) gemm_routed_dma_kernel<kRoutedGateUp, true, U, 64, NST, GU><<<g, b, 0, s>>>(a);
    else if (a.K / 64 <= GD) {
        if (outbf) gemm_routed_dma_kernel<kRoutedDown, true, U, 64, NST, GD><<<g, b, 0, s>>>(a);
        else gemm_routed_dma_kernel<kRoutedDown, false, U, 64, NST, GD><<<g, b, 0, s>>>(a);
    } else {
        if (outbf) gemm_routed_dma_kernel<kRoutedDown, true, U, 64, NST, GU><<<g, b, 0, s>>>(a);
        else gemm_routed_dma_kernel<kRoutedDown, false, U, 64, NST, GU><<<g, b, 0, s>>>(a);
    }
}

// u4: 0 = bf16 weights, else the 4-bit token tile rows (CfgU4 or CfgU4M)
static bool launch_persist(int mode, bool outbf, int u4, const GemmArgs& a, int max_tiles, hipStream_t s) {
    using C = CfgLarge;
    const int nst = u4 == 0 ? kPersistNST : u4 == CfgU4::BT ? kU4NST : kU4MNST;
    if (u4 != 0 && u4 != CfgU4::BT && u4 != CfgU4M::BT) return false;
    const int nl = persist_groups(mode, u4 != 0, a.N, a.K, max_tiles, a.n_act_rows, a.n_pairs, outbf, nst);
    if (nl <= 0) return false;
    const dim3 g(unsigned(8 * nl)), b(C::THREADS);
    if (u4 == CfgU4::BT) {
        launch_u4<CfgU4, kU4NST>(mode, outbf, a, g, s);
        return true;
    }
    if (u4 == CfgU4M::BT) {
        launch_u4<CfgU4M, kU4MNST>(mode, outbf, a, g, s);
        return true;
    }
    constexpr int KS = kPersistKS, NST = kPersistNST;
    if (mode == kRoutedGateUp) gemm_routed_dma_kernel<kRoutedGateUp, true, C, KS, NST, 0><<<g, b, 0, s>>>(a);
    else if (outbf) gemm_routed_dma_kernel<kRoutedDown, true, C, KS, NST, 0><<<g, b, 0, s>>>(a);
    else gemm_routed_dma_kernel<kRoutedDown, false, C, KS, NST, 0><<<g, b, 0, s>>>(a);
    return true;
}

hipError_t launch_gemm_tiled(int mode, bool outbf, const GemmArgs& a, int grid_x, hipStream_t s) {
    if (grid_x <= 0) return hipSuccess;
    if ((mode == kRoutedGateUp || mode == kRoutedDown) && launch_persist(mode, outbf, 0, a, grid_x, s))
        return hipGetLastError();
    if (mode == kRoutedGateUp || mode == kRoutedDown) return launch_cfg<CfgLarge>(mode, outbf, a, grid_x, s);
    // Dense products (shared expert, router logits) take their items token
    // tile by token tile: each XCD (a contiguous run of items) then reads its
    // own rows of the activations and every weight row block, instead of one
    // row block against all the activations.  Measured on the skewed T = 4096
    // prefill: bytes fetched from beyond L2 per launch 139 -> 50 MB (shared
    // gate/up), 36 -> 21 MB (shared down), 38 -> 25 MB (router logits).
    GemmArgs t = a;
    t.tile_major = 1;
    return launch_cfg<CfgSmall>(mode, outbf, t, grid_x, s);
}

hipError_t launch_gemm_routed_u4(int mode, bool outbf, int tile_rows, const GemmArgs& a, int max_tiles,
                                 hipStream_t s) {
    if (max_tiles <= 0) return hipSuccess;
    if (mode != kRoutedGateUp && mode != kRoutedDown) return hipErrorInvalidValue;
    if (!launch_persist(mode, outbf, tile_rows, a, max_tiles, s)) return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
