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
    kDenseStore = 4     // all T rows; plain fp32 store (router logits)
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
};

hipError_t launch_gemm(int mode, int wkind, bool outbf, const GemmArgs& a, int grid_x, int tf, hipStream_t s);

// routing (parameter blocks in moe_select.h)
struct SelParams;
struct PermParams;
hipError_t launch_route_select(const SelParams& P, int32_t* ids, float* weights, hipStream_t s);
bool route_permute_fusable(int T, int E, int K);
hipError_t launch_route_permute(const SelParams& P, int32_t* ids, float* weights, const PermParams& Q,
                                hipStream_t s);
hipError_t launch_gate_logit(const void* x, bool x_f32, const void* wvec, int T, int D, float* out, hipStream_t s);

// permute (tiles may be null)
hipError_t launch_permute(const PermParams& P, hipStream_t s);
int id_bits_for(int E);
int max_tiles_for(int n_pairs, int E, int tile_rows);
hipError_t launch_build_tiles(const int32_t* offsets, const int32_t* active, const int32_t* n_active, int E,
                              int n_pairs, int4* tiles, int32_t* n_tiles, int max_tiles, int tile_rows,
                              hipStream_t s);

// combine: out = residual + (sum_k slot[t,k,:] + shared[t,:])
hipError_t launch_combine(const void* slots, bool slots_bf16, const float* shared, const float* residual,
                          float* out, int T, int K, int D, hipStream_t s);

}  // namespace moe
