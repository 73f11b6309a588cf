// Internal launch interface between the C ABI layer (moe_api.cpp) and the
// HIP kernels.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// weight kinds
enum { kWF32 = 0, kWBF16 = 1, kWU4 = 2 };

// GEMM modes (see moe_gemm.hip)
enum {
    kRoutedGateUp = 0,  // tiles from the permute; x rows gathered via pair/topk; SwiGLU -> h[pos]
    kRoutedDown = 1,    // tiles from the permute; h rows in permuted order; alpha * . -> slot[pair]
    kDenseGateUp = 2,   // all T rows; SwiGLU -> h[t]
    kDenseDown = 3,     // all T rows; sigmoid(gate logit) * . (or 1) -> out[t]
    kDenseStore = 4,    // all T rows; plain fp32 store (router logits)
    kSmallGateUp = 5,   // small T*K: tile derived from topk ids in-kernel; shared expert as item 0
    kSmallDown = 6,     // small T*K: same tiles; writes slot rows t*(K+1)+k, shared to slot K
    kDenseStoreNorm = 7 // router logits from the fp32 attention residual, RMS norm folded in (bf16, 16-row tiles)
};

struct GemmArgs {
    const void* w0;  // weight bank [n_banks][N][K] (u4: codes [n_banks][N][K/2])
    const void* s0;  // u4 scale [n_banks][N][K/64] bf16
    const void* m0;  // u4 min
    const void* w1;  // second bank (gate/up modes: up)
    const void* s1;
    const void* m1;
    int N, K;
    int n_banks;
    const void* act;  // activation rows [n_act_rows][K]
    int n_act_rows;
    const int4* tiles;  // routed modes: {expert, begin, count, 0}
    const int* n_tiles;
    int n_rows;         // dense modes: number of rows (tokens)
    const int* pairs;   // routed modes: sorted flat pair ids
    int n_pairs;        // T*K
    int topk;
    void* out;              // [rows][N] fp32 or bf16 (dense store: [ksplit][rows][N])
    const float* row_scale; // routed down: weights[pair]; dense down: gate logits or null
    int ksplit;             // dense store only: K split across blockIdx.z (partial sums)
    // small-T modes
    const int32_t* ids;     // topk ids [T*K]
    int n_tokens;
    int n_experts;
    int has_shared;
    const void* sw0; const void* ss0; const void* sm0;  // shared gate (or shared down)
    const void* sw1; const void* ss1; const void* sm1;  // shared up
    const float* gate_logit;  // [T] shared gate logits or null (s = 1)
    int sN, sK;               // shared item: output rows (gate/up) / reduction length (down)
    int act_ld, out_ld;       // row strides when they differ from K / N (0 = default)
    // small-T gate/up with the softmax top-K selection folded in: every
    // workgroup selects from the router's partial logits into LDS, and
    // workgroup 0 writes the routing outputs and the shared gate logits
    int fused_sel;
    const float* sel_logits;  // [sel_ksplit][T][n_experts] partial logits
    int sel_ksplit;
    int32_t* sel_ids;         // [T*K] outputs (workspace)
    float* sel_wts;
    int32_t* sel_ids2;        // optional caller copies
    float* sel_wts2;
    const void* gate_w;       // shared gate vector [K] (null: no gate logits)
    int gate_x_f32;
    float* gate_out;          // [T]
    int direct_pairs;         // small-T gate/up: one work item per (token, slot) pair
    int shape_grid;           // small T: item count the tile shape is chosen for (0: grid_x)
    // kDenseStoreNorm: act is the fp32 residual [n_rows][K]; x = (r * (1/rms)) * norm_w
    // is rounded to bf16 on the fly, and the row-block-0 workgroups write it to norm_x
    const float* norm_w;      // [K] or null (ones)
    float norm_eps;
    void* norm_x;             // [n_rows][K] bf16
    // LDS-tiled dense modes: work items in token-tile-major order (row block
    // fastest), so each XCD reads its own slice of the activation rows
    int tile_major;
};
// Largest T for which the small-T gate/up launch does the selection itself.
constexpr int kFusedSelMaxT = 8;
// 4-bit weights: largest count of 64-element groups in a GEMM workgroup's K
// range (reduction lengths up to 4096), the size of the LDS scale staging.
constexpr int kU4MaxGroups = 64;

hipError_t launch_gemm(int mode, int wkind, bool outbf, const GemmArgs& a, int grid_x, int tf, hipStream_t s);
// 4-bit affine group-64 matrix [rows][K] (codes, scale, min) -> bf16 [rows][K]
hipError_t launch_dequant_u4(const void* codes, const void* scale, const void* min, int rows, int K, void* out,
                             hipStream_t s);
// bf16 LDS-tiled variant; K % 64 == 0.  Routed modes: tiles of tiled_rows()
// pairs (256 weight rows x 128 tokens per workgroup); dense modes: token
// tiles of tiled_rows_dense() (128 x 128).
hipError_t launch_gemm_tiled(int mode, bool outbf, const GemmArgs& a, int grid_x, hipStream_t s);
int tiled_rows();
int tiled_rows_dense();
// 4-bit affine group-64 banks on the persistent LDS-tiled kernel (routed
// modes, tiles of tiled_rows() or tiled_rows_u4_medium() pairs): whether the
// shape fits it (K % 64 == 0, K <= 2048, at least as many K steps as LDS
// stages, offsets inside 32 bits, the item table), and the launch
// (hipErrorInvalidValue when it does not fit; nothing launched).
int tiled_rows_u4_medium();
bool routed_tiled_u4_fits(int mode, int tile_rows, int N, int K, int max_tiles, int n_act_rows, int n_pairs,
                          bool outbf);
hipError_t launch_gemm_routed_u4(int mode, bool outbf, int tile_rows, const GemmArgs& a, int max_tiles,
                                 hipStream_t s);

// routing (parameter blocks in moe_select.h)
struct SelParams;
struct PermParams;
hipError_t launch_route_select(const SelParams& P, int32_t* ids, float* weights, hipStream_t s);
bool route_permute_fusable(int T, int E, int K);
// shared-gate logit per token inside the selection kernel (small T path)
struct GateParams { const void* x; const void* w; int D; int x_f32; float* out; };
hipError_t launch_route_select_gate(const SelParams& P, const GateParams& G, int32_t* ids, float* weights,
                                    hipStream_t s);
hipError_t launch_route_permute(const SelParams& P, int32_t* ids, float* weights, const PermParams& Q,
                                hipStream_t s);
hipError_t launch_gate_logit(const void* x, bool x_f32, const void* wvec, int T, int D, float* out, hipStream_t s);
// Selection that also counts each block's pairs per expert: block c takes
// route_chunk_tokens(family) tokens (16 waves: two tokens per wave in the
// softmax family, one in the group family) and writes counts[c][e] (how
// many of its tokens' slots chose expert e), the first pass of
// launch_permute_from_counts.  E <= 256.
constexpr int kCountWaves = 16;
inline int route_chunk_tokens(int family) { return family == 0 ? 2 * kCountWaves : kCountWaves; }
hipError_t launch_route_select_counts(const SelParams& P, const GateParams& G, int32_t* ids, float* weights,
                                      int32_t* counts, hipStream_t s);

// permute (tiles may be null)
hipError_t launch_permute(const PermParams& P, hipStream_t s);
// The permute from per-chunk expert counts (chunk c = pairs c*chunk_pairs ..,
// counts [n_chunks][E] in P.chunk_base, as launch_route_select_counts writes
// them): one launch; E <= 256, chunk_pairs <= 1024.
hipError_t launch_permute_from_counts(const PermParams& P, int n_chunks, int chunk_pairs, hipStream_t s);
int id_bits_for(int E);
int max_tiles_for(int n_pairs, int E, int tile_rows);
hipError_t launch_build_tiles(const int32_t* offsets, const int32_t* active, const int32_t* n_active, int E,
                              int n_pairs, int4* tiles, int32_t* n_tiles, int max_tiles, int tile_rows,
                              hipStream_t s);

// combine: out = residual + (sum_k slot[t,k,:] + shared[t,:])
// Small T, bf16 weights: down projection and combine in one launch.
// out[t, :] = residual[t, :] + sum_k wts[t*K+k] * W_down[ids[t*K+k]] h[t*K+k]
//            + sigmoid(gate_logit[t]) * W_shared_down h[T*K + t]   (gate 1 if NULL).
struct DownCombineArgs {
    const void* h;            // [T*K + T][h_ld] bf16: routed pair rows, then shared rows
    int h_ld;
    const int32_t* ids;       // [T*K]
    const float* wts;         // [T*K]
    const void* w;            // routed down bank [E][D][F] bf16
    const void* ws;           // shared down [D][F] bf16 (has_shared)
    const float* gate_logit;  // [T] or NULL
    const float* residual;    // [T][D]
    float* out;               // [T][D]
    int T, K, E, D, F, has_shared;
    // 4-bit affine group-64 banks (u4 != 0): w / ws hold the codes [.., D, F/2];
    // scale and min bf16 [.., D, F/64]
    int u4;
    const void* w_scale;
    const void* w_min;
    const void* ws_scale;
    const void* ws_min;
};
bool down_combine_supported(int T, int K, int D, int F, int Fs, bool u4);
hipError_t launch_down_combine(const DownCombineArgs& a, hipStream_t s);
hipError_t launch_combine(const void* slots, bool slots_bf16, const float* shared, const float* residual,
                          float* out, int T, int K, int D, hipStream_t s);
// small T: the slot rows hold K routed slots + the shared expert (K+1 per token)

// Streaming read of `bytes` (a multiple of 256 KiB) at buf; one XOR word per
// lane of each 64 KB block into sink (stream_read_sink_words(bytes) words).
size_t stream_read_sink_words(size_t bytes);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
// MFMA issue-rate loop (shape 0: 16x16x32 bf16, 1: 32x32x16 bf16): workgroups
// of 4 waves, `iterations` rounds of mfma_rate_chains() MFMAs per wave, one
// float per lane into sink (workgroups * 256 floats).
int mfma_rate_chains();
hipError_t launch_mfma_rate(int shape, int workgroups, int iterations, float* sink, hipStream_t s);
// L2 read rate by lane pattern (0 row segments, 1 MFMA operand order, 2 row
// quads): workgroups of 4 waves, each wave `iterations` passes over a 64 KB
// region of a buffer of l2_read_buffer_bytes(); one word per lane into sink
// (workgroups * 256 words).
size_t l2_read_buffer_bytes();
hipError_t launch_l2_read(int pattern, int workgroups, int iterations, const void* buf, uint32_t* sink,
                          hipStream_t s);

// x[t, :] = r[t, :] / sqrt(mean(r[t, :]^2) + eps) * w (w may be NULL: ones);
// x bf16 (out_bf16) or fp32.  D % 4 == 0; r, w, x 16-byte aligned.
hipError_t launch_rms_norm(const float* r, const float* w, float eps, int T, int D, void* x, bool out_bf16,
                           hipStream_t s);

}  // namespace moe
