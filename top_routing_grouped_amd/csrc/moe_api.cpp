// C ABI of the MoE layer library: argument checks, workspace carving, launch
// sequencing and the two-stream fork/join of the shared expert.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/moe.h"
#include "moe_kernels.h"
#include "moe_select.h"


namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

#define HIP_TRY(expr)                                                                         \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

int wkind_of(moe_dtype d) {
    return d == MOE_F32 ? moe::kWF32 : d == MOE_BF16 ? moe::kWBF16 : moe::kWU4;
}

// K elements per chunk a wave consumes: fp32 16, bf16/u4 128.
int kspan_of(moe_dtype expert) { return expert == MOE_F32 ? 16 : 128; }

// Routed GEMM tiles: bf16 experts averaging >= 16 pairs use the persistent
// LDS-tiled kernel (128-token tiles: an expert's weights are read once per
// tile, where 16-token tiles read them up to 8 times; measured at T = 1024,
// K = 8: 765 -> 378 us per layer); 4-bit and fp32 experts averaging >= 64
// pairs use 64-token register tiles; fewer pairs use 16-token tiles (weights
// streamed straight into registers).
bool routed_large(const moe_config& c) {
    const int64_t per_expert = c.expert_dtype == MOE_BF16 ? 16 : 64;
    return (int64_t)c.n_tokens * c.top_k >= per_expert * c.n_experts;
}
int64_t max_tiles(int64_t n_pairs, int E, int tile_rows) {
    const int64_t act = std::min<int64_t>(E, n_pairs);
    return (n_pairs + act * (tile_rows - 1)) / tile_rows;
}
// 4-bit banks averaging at least kU4TiledMinPairs pairs per expert use the
// persistent LDS-tiled kernel (codes and group scales staged in LDS) where
// both routed GEMMs fit it: 128-token tiles from kU4Bt128MinPairs pairs per
// expert, 64-token tiles (a deeper ring) below; fewer pairs keep the
// register tiles.  Measured at Qwen3.6 shape, K = 4 (pairs per expert:
// layer us): register tiles 8: 212.6, 16: 328; 64-token tiles 1.6: 163.5
// (register 136.7), 8: 221.4, 16: 234.4, 32: 264.0, 64: 404.2; 128-token
// tiles 16: 251.6, 32: 281.9, 64: 349.5.
#ifndef MOE_U4_TILED_MIN_PAIRS
#define MOE_U4_TILED_MIN_PAIRS 16
#endif
#ifndef MOE_U4_BT128_MIN_PAIRS
#define MOE_U4_BT128_MIN_PAIRS 64
#endif
constexpr int kU4TiledMinPairs = MOE_U4_TILED_MIN_PAIRS;
constexpr int kU4Bt128MinPairs = MOE_U4_BT128_MIN_PAIRS;
// token tile rows of the tiled 4-bit schedule, 0 when the layer does not take it
int routed_u4_tile_rows(const moe_config& c) {
    if (c.expert_dtype != MOE_U4_AFFINE_G64) return 0;
    const int64_t TK = (int64_t)c.n_tokens * c.top_k;
    if (TK < (int64_t)kU4TiledMinPairs * c.n_experts || TK >= (int64_t(1) << 31)) return 0;
    const int rows = TK >= (int64_t)kU4Bt128MinPairs * c.n_experts ? moe::tiled_rows() : moe::tiled_rows_u4_medium();
    const int mt = int(max_tiles(TK, c.n_experts, rows));
    const bool fits =
        moe::routed_tiled_u4_fits(moe::kRoutedGateUp, rows, c.d_ff, c.d_model, mt, c.n_tokens, int(TK), true) &&
        moe::routed_tiled_u4_fits(moe::kRoutedDown, rows, c.d_model, c.d_ff, mt, int(TK), int(TK), false);
    return fits ? rows : 0;
}
bool routed_tiled_u4(const moe_config& c) { return routed_u4_tile_rows(c) > 0; }
bool routed_tiled(const moe_config& c) {
    return (routed_large(c) && c.expert_dtype == MOE_BF16) || routed_tiled_u4(c);
}
int routed_tf(const moe_config& c) { return routed_large(c) ? 4 : 1; }
int routed_tile_rows(const moe_config& c) {
    if (const int u = routed_u4_tile_rows(c)) return u;
    return routed_tiled(c) ? moe::tiled_rows() : 16 * routed_tf(c);
}
int dense_tf(const moe_config& c) { return c.n_tokens >= 64 ? 4 : 1; }
bool dense_tiled(const moe_config& c, moe_dtype d) { return c.n_tokens >= 128 && d == MOE_BF16; }
// 4-bit shared expert from T = 128: its three matrices are dequantised to
// bf16 into the workspace (6 MiB at Qwen3.6 shape, a few us) and it runs on
// the LDS-tiled bf16 kernels.  The register-streaming 4-bit kernels re-read
// each 64-token tile of activations for every 16 weight rows (Qwen3.6 4-bit,
// K = 4, T = 4096: shared gate/up 92 us and down 212 us on the aux stream).
bool shared_dequant(const moe_config& c) {
    return c.expert_dtype == MOE_U4_AFFINE_G64 && c.d_ff_shared > 0 && dense_tiled(c, MOE_BF16);
}
// Small T*K: one stream; every GEMM workgroup finds its expert and pairs from
// the routing ids itself (no permute launch) and the shared expert is an
// extra work item of the routed launches.
bool small_path(const moe_config& c) {
    return !routed_large(c) && !routed_tiled_u4(c) && (int64_t)c.n_tokens * c.top_k <= 256;
}
int h_ld(const moe_config& c) { return std::max(c.d_ff, c.d_ff_shared); }
// Small path with bf16 or 4-bit weights: the down projection and the combine
// are one launch (each workgroup owns a slice of output features for every
// token).
bool down_combine_fused(const moe_config& c) {
    return small_path(c) && (c.expert_dtype == MOE_BF16 || c.expert_dtype == MOE_U4_AFFINE_G64) &&
           moe::down_combine_supported(c.n_tokens, c.top_k, c.d_model, c.d_ff, c.d_ff_shared,
                                       c.expert_dtype == MOE_U4_AFFINE_G64);
}

// Router logits: for small T, K is split over up to 8 workgroups (partial
// planes the selection sums), each split a whole number of 4-wave chunks; 1
// when no such split exists (a split must divide d_model exactly, or part of
// the reduction would be dropped).
int router_ksplit(const moe_config& c) {
    if (dense_tiled(c, c.router_dtype)) {
        // LDS-tiled logits: enough K splits for ~256 workgroups, each a
        // multiple of the 64-wide K step
        const long long items = (long long)((c.n_tokens + moe::tiled_rows_dense() - 1) / moe::tiled_rows_dense()) *
                                ((c.n_experts + moe::tiled_rows_dense() - 1) / moe::tiled_rows_dense());
        int s = int(std::min<long long>(8, std::max<long long>(1, (256 + items - 1) / items)));
        while (s > 1 && c.d_model % (s * 64)) --s;
        return s;
    }
    if (c.n_tokens > 64) return 1;
    const int per = 4 * kspan_of(c.router_dtype == MOE_F32 ? MOE_F32 : MOE_BF16);
    for (int s = 8; s > 1; --s)
        if (c.d_model % (s * per) == 0) return s;
    return 1;
}

// Many pairs (E <= 256): the selection launch also counts each block's pairs
// per expert, and the permute is one launch from those counts, in place of a
// count launch, a single-workgroup scan and a scatter launch (Qwen3.6
// prefill shape, T = 4096: selection 11.4 + permute 5.2 + 9.6 + 5.2 us ->
// 14.5 + 13.5 us).
int count_chunk_tokens(const moe_config& c) { return moe::route_chunk_tokens(int(c.family)); }
bool permute_counts(const moe_config& c) {
    return !small_path(c) && c.n_experts <= 256 && (int64_t)c.n_tokens * c.top_k >= 4 * moe::kPermChunk &&
           count_chunk_tokens(c) * c.top_k <= moe::kPermThreads;
}
int count_chunks(const moe_config& c) { return (c.n_tokens + count_chunk_tokens(c) - 1) / count_chunk_tokens(c); }

struct Layout {
    size_t chunk_base, logits, gate_logit, ids, wts, offsets, active, n_active, n_tiles, pairs, tiles, h, slots, hs, ys, xn,
        sw, total;
};

Layout layout(const moe_config& c) {
    const size_t T = c.n_tokens, E = c.n_experts, K = c.top_k, D = c.d_model, F = c.d_ff, Fs = c.d_ff_shared;
    const size_t TK = T * K;
    const size_t hb = c.expert_dtype == MOE_F32 ? 4 : 2;
    const size_t mt = size_t(max_tiles(TK, int(E), routed_tile_rows(c)));
    Layout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o += align256(bytes);
        return at;
    };
    L.chunk_base = take(size_t(std::max(moe::perm_chunks(int(TK)), permute_counts(c) ? count_chunks(c) : 0)) * E * 4);
    L.logits = take(size_t(router_ksplit(c)) * T * E * 4);
    L.gate_logit = take(T * 4);
    L.ids = take(TK * 4);
    L.wts = take(TK * 4);
    L.offsets = take((E + 1) * 4);
    L.active = take(E * 4);
    L.n_active = take(4);
    L.n_tiles = take(4);
    L.pairs = take(TK * 4);
    L.tiles = take(mt * 16);
    const size_t Fh = size_t(std::max(c.d_ff, c.d_ff_shared));
    L.h = take(std::max(TK * F, (TK + T) * Fh) * hb);
    L.slots = take(std::max(TK * D, T * (K + 1) * D) * hb);
    L.hs = take(T * Fs * hb);
    L.ys = take(T * D * 4);
    L.xn = take(T * D * (c.act_dtype == MOE_F32 ? 4 : 2));  // normalised x (moe_layer_forward_norm)
    L.sw = take(shared_dequant(c) ? 3 * Fs * D * 2 : 0);    // dequantised shared gate, up, down (bf16)
    L.total = o;
    return L;
}

// The value a C caller stored in an enum-typed field or argument, read as
// the 32-bit integer the ABI passes: C allows any int there, and loading an
// out-of-range value through the C++ enum type is undefined.
template <class E>
int32_t raw(const E& v) {
    static_assert(sizeof(E) == sizeof(int32_t), "enums are 32-bit in this ABI");
    int32_t r;
    std::memcpy(&r, &v, sizeof r);
    return r;
}

moe_status check_config(const moe_config* c) {
    if (!c) return fail(MOE_ERR_INVALID_ARGUMENT, "config is NULL");
    const int32_t family = raw(c->family), act = raw(c->act_dtype), rdt = raw(c->router_dtype),
                  edt = raw(c->expert_dtype);
    if (c->n_tokens < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "n_tokens < 0");
    if (c->d_model <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->d_ff <= 0 || c->d_ff_shared < 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "sizes must be positive (d_ff_shared >= 0)");
    if (c->top_k > c->n_experts) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k > n_experts");
    if (c->top_k > 32) return fail(MOE_ERR_UNSUPPORTED, "top_k > 32");
    if (c->n_experts > 1024 || c->n_experts % 16) return fail(MOE_ERR_UNSUPPORTED, "n_experts must be a multiple of 16, <= 1024");
    if ((int64_t)c->n_tokens * c->top_k > (int64_t(1) << 30)) return fail(MOE_ERR_UNSUPPORTED, "n_tokens * top_k too large");
    if (family != MOE_ROUTE_SOFTMAX_TOPK && family != MOE_ROUTE_SIGMOID_GROUP_TOPK)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown routing family");
    if (family == MOE_ROUTE_SIGMOID_GROUP_TOPK) {
        const int E = c->n_experts, G = c->n_group, TG = c->topk_group;
        if (G < 1 || G > 64) return fail(MOE_ERR_INVALID_ARGUMENT, "n_group must be in [1, 64]");
        if (E % G || E / G < 2) return fail(MOE_ERR_INVALID_ARGUMENT, "n_experts must split into n_group groups of >= 2");
        if (TG < 1 || TG > G) return fail(MOE_ERR_INVALID_ARGUMENT, "topk_group must be in [1, n_group]");
        if (c->top_k > TG * (E / G)) return fail(MOE_ERR_INVALID_ARGUMENT, "top_k exceeds the experts of the kept groups");
        if (!(std::isfinite(c->routed_scaling) && c->routed_scaling > 0.f))
            return fail(MOE_ERR_INVALID_ARGUMENT, "routed_scaling must be finite and > 0");
    }
    const bool f32 = act == MOE_F32;
    if (act != MOE_F32 && act != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "act_dtype must be F32 or BF16");
    if (rdt != act) return fail(MOE_ERR_UNSUPPORTED, "router_dtype must equal act_dtype");
    if (f32 ? edt != MOE_F32 : (edt != MOE_BF16 && edt != MOE_U4_AFFINE_G64))
        return fail(MOE_ERR_UNSUPPORTED, "expert_dtype must be F32 with F32 activations, BF16 or U4_AFFINE_G64 with BF16");
    if (edt == MOE_U4_AFFINE_G64 &&
        (c->d_model > 64 * moe::kU4MaxGroups || c->d_ff > 64 * moe::kU4MaxGroups ||
         c->d_ff_shared > 64 * moe::kU4MaxGroups))
        return fail(MOE_ERR_UNSUPPORTED, "4-bit weights: d_model, d_ff and d_ff_shared must be <= %d",
                    64 * moe::kU4MaxGroups);
    const int span = edt == MOE_F32 ? 16 : 128;
    if (c->d_model % span || c->d_ff % span || c->d_ff_shared % span)
        return fail(MOE_ERR_UNSUPPORTED, "d_model, d_ff, d_ff_shared must be multiples of %d for this dtype", span);
    return MOE_OK;
}

moe_status check_ws(const moe_config& c, void* ws, size_t ws_bytes) {
    const size_t need = layout(c).total;
    if (ws_bytes < need) return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < %zu bytes", ws_bytes, need);
    if (!ws) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    return MOE_OK;
}

bool matrix_ok(const moe_matrix& m, moe_dtype d) {
    if (!m.w) return false;
    if (d == MOE_U4_AFFINE_G64 && (!m.scale || !m.min)) return false;
    return true;
}

moe_status check_weights(const moe_config& c, const moe_weights* w, bool routed, bool shared) {
    if (!w) return fail(MOE_ERR_INVALID_ARGUMENT, "weights is NULL");
    if (routed && !(matrix_ok(w->gate, c.expert_dtype) && matrix_ok(w->up, c.expert_dtype) &&
                    matrix_ok(w->down, c.expert_dtype)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "routed gate/up/down bank pointer is NULL");
    if (shared && c.d_ff_shared > 0 &&
        !(matrix_ok(w->shared_gate, c.expert_dtype) && matrix_ok(w->shared_up, c.expert_dtype) &&
          matrix_ok(w->shared_down, c.expert_dtype)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared expert matrix pointer is NULL");
    return MOE_OK;
}

moe::GemmArgs gemm_args(const moe_matrix& m0, const moe_matrix* m1, int N, int K, int n_banks) {
    moe::GemmArgs a{};
    a.w0 = m0.w; a.s0 = m0.scale; a.m0 = m0.min;
    if (m1) { a.w1 = m1->w; a.s1 = m1->scale; a.m1 = m1->min; }
    a.N = N; a.K = K; a.n_banks = n_banks;
    return a;
}

template <class T>
T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

// RMS norm of the attention residual folded into the router-logits launch:
// small T with bf16 activations (16-token tiles; the launch converts the
// residual rows it reads and writes x for the later launches).
struct NormFold {
    const float* residual;
    const float* w;
    float eps;
    void* x;
};
bool norm_fusable(const moe_config& c) {
    return small_path(c) && c.act_dtype == MOE_BF16 && c.router_dtype == MOE_BF16 &&
           !dense_tiled(c, c.router_dtype) && dense_tf(c) == 1;
}

// ---- stages (arguments already validated)
moe_status stage_logits(const moe_config& c, const Layout& L, void* ws, const void* x, const void* router,
                        hipStream_t s, const NormFold* nf = nullptr) {
    const int T = c.n_tokens;
    moe_matrix rm{router, nullptr, nullptr};
    moe::GemmArgs a = gemm_args(rm, nullptr, c.n_experts, c.d_model, 1);
    a.act = x; a.n_act_rows = T; a.n_rows = T;
    a.out = at<float>(ws, L.logits);
    a.ksplit = router_ksplit(c);
    if (nf) {
        a.act = nf->residual;
        a.norm_w = nf->w; a.norm_eps = nf->eps; a.norm_x = nf->x;
        HIP_TRY(moe::launch_gemm(moe::kDenseStoreNorm, moe::kWBF16, false, a, (T + 15) / 16, 1, s));
        return MOE_OK;
    }
    if (dense_tiled(c, c.router_dtype)) {
        HIP_TRY(moe::launch_gemm_tiled(moe::kDenseStore, false, a, (T + moe::tiled_rows_dense() - 1) / moe::tiled_rows_dense(), s));
        return MOE_OK;
    }
    const int tf = dense_tf(c);
    HIP_TRY(moe::launch_gemm(moe::kDenseStore, c.router_dtype == MOE_F32 ? moe::kWF32 : moe::kWBF16, false, a,
                             (T + 16 * tf - 1) / (16 * tf), tf, s));
    return MOE_OK;
}

moe::SelParams sel_params(const moe_config& c, const Layout& L, void* ws, const float* bias,
                          int32_t* ids2 = nullptr, float* wts2 = nullptr) {
    moe::SelParams P{};
    P.ids2 = ids2;
    P.wts2 = wts2;
    P.logits = at<float>(ws, L.logits);
    P.ksplit = router_ksplit(c);
    P.T = c.n_tokens; P.E = c.n_experts; P.K = c.top_k;
    P.family = int(c.family);
    P.G = c.n_group; P.TG = c.topk_group; P.scaling = c.routed_scaling;
    P.bias = c.family == MOE_ROUTE_SIGMOID_GROUP_TOPK ? bias : nullptr;
    return P;
}

moe::PermParams perm_params(const moe_config& c, const int32_t* ids, int32_t* offsets, int32_t* active,
                            int32_t* n_active, int32_t* sorted_pairs, int4* tiles, int32_t* n_tiles, int tile_rows,
                            int32_t* chunk_base) {
    moe::PermParams Q{};
    Q.chunk_base = chunk_base;
    Q.ids = ids;
    Q.n_pairs = c.n_tokens * c.top_k;
    Q.E = c.n_experts;
    Q.id_bits = moe::id_bits_for(c.n_experts);
    Q.offsets = offsets; Q.active = active; Q.n_active = n_active; Q.sorted_pairs = sorted_pairs;
    Q.tiles = tiles; Q.n_tiles = n_tiles;
    Q.tile_rows = tile_rows;
    Q.max_tiles = moe::max_tiles_for(Q.n_pairs, c.n_experts, tile_rows);
    return Q;
}

moe_status stage_route(const moe_config& c, const Layout& L, void* ws, const void* x, const void* router,
                       const float* bias, int32_t* ids, float* wts, hipStream_t s) {
    if (moe_status st = stage_logits(c, L, ws, x, router, s)) return st;
    HIP_TRY(moe::launch_route_select(sel_params(c, L, ws, bias), ids, wts, s));
    return MOE_OK;
}

moe_status stage_gateup(const moe_config& c, const Layout& L, void* ws, const void* x, const moe_weights& w,
                        const int32_t* pairs, const int4* tiles, const int32_t* n_tiles, hipStream_t s) {
    const int T = c.n_tokens, K = c.top_k, TK = T * K;
    const int tf = routed_tf(c);
    const int grid = int(max_tiles(TK, c.n_experts, 16 * tf));
    moe::GemmArgs a = gemm_args(w.gate, &w.up, c.d_ff, c.d_model, c.n_experts);
    a.act = x; a.n_act_rows = T;
    a.tiles = tiles; a.n_tiles = n_tiles; a.pairs = pairs; a.n_pairs = TK; a.topk = K;
    a.out = at<void>(ws, L.h);
    if (routed_tiled_u4(c)) {
        HIP_TRY(moe::launch_gemm_routed_u4(moe::kRoutedGateUp, true, routed_tile_rows(c), a,
                                           int(max_tiles(TK, c.n_experts, routed_tile_rows(c))), s));
        return MOE_OK;
    }
    if (routed_tiled(c)) {
        HIP_TRY(moe::launch_gemm_tiled(moe::kRoutedGateUp, true, a, int(max_tiles(TK, c.n_experts, routed_tile_rows(c))), s));
        return MOE_OK;
    }
    HIP_TRY(moe::launch_gemm(moe::kRoutedGateUp, wkind_of(c.expert_dtype), c.expert_dtype != MOE_F32, a, grid, tf, s));
    return MOE_OK;
}

moe_status stage_down(const moe_config& c, const Layout& L, void* ws, const moe_weights& w, const int32_t* pairs,
                      const int4* tiles, const int32_t* n_tiles, const float* wts, void* slot_out, bool slot_bf16,
                      hipStream_t s) {
    const int T = c.n_tokens, K = c.top_k, TK = T * K;
    const int tf = routed_tf(c);
    const int grid = int(max_tiles(TK, c.n_experts, 16 * tf));
    moe::GemmArgs d = gemm_args(w.down, nullptr, c.d_model, c.d_ff, c.n_experts);
    d.act = at<void>(ws, L.h); d.n_act_rows = TK;
    d.tiles = tiles; d.n_tiles = n_tiles; d.pairs = pairs; d.n_pairs = TK; d.topk = K;
    d.out = slot_out; d.row_scale = wts;
    if (routed_tiled_u4(c)) {
        HIP_TRY(moe::launch_gemm_routed_u4(moe::kRoutedDown, slot_bf16, routed_tile_rows(c), d,
                                           int(max_tiles(TK, c.n_experts, routed_tile_rows(c))), s));
        return MOE_OK;
    }
    if (routed_tiled(c)) {
        HIP_TRY(moe::launch_gemm_tiled(moe::kRoutedDown, slot_bf16, d, int(max_tiles(TK, c.n_experts, routed_tile_rows(c))), s));
        return MOE_OK;
    }
    HIP_TRY(moe::launch_gemm(moe::kRoutedDown, wkind_of(c.expert_dtype), slot_bf16, d, grid, tf, s));
    return MOE_OK;
}

moe::GemmArgs small_args(const moe_config& c, const Layout& L, void* ws, const moe_weights& w, bool gateup) {
    moe::GemmArgs a{};
    const int T = c.n_tokens, K = c.top_k, TK = T * K;
    a.ids = at<int32_t>(ws, L.ids);
    a.n_pairs = TK; a.n_tokens = T; a.n_experts = c.n_experts; a.topk = K; a.n_banks = c.n_experts;
    a.has_shared = c.d_ff_shared > 0;
    const moe_matrix& r0 = gateup ? w.gate : w.down;
    a.w0 = r0.w; a.s0 = r0.scale; a.m0 = r0.min;
    if (gateup) { a.w1 = w.up.w; a.s1 = w.up.scale; a.m1 = w.up.min; }
    if (a.has_shared) {
        const moe_matrix& q0 = gateup ? w.shared_gate : w.shared_down;
        a.sw0 = q0.w; a.ss0 = q0.scale; a.sm0 = q0.min;
        if (gateup) { a.sw1 = w.shared_up.w; a.ss1 = w.shared_up.scale; a.sm1 = w.shared_up.min; }
    }
    if (gateup) {
        a.N = c.d_ff; a.sN = c.d_ff_shared; a.K = c.d_model; a.sK = c.d_model;
        a.n_act_rows = T;
        a.out_ld = h_ld(c);
    } else {
        a.N = c.d_model; a.sN = c.d_model; a.K = c.d_ff; a.sK = c.d_ff_shared > 0 ? c.d_ff_shared : c.d_ff;
        a.n_act_rows = TK + T;
        a.act_ld = h_ld(c);
        a.row_scale = at<float>(ws, L.wts);
        a.gate_logit = w.shared_gate_vec ? at<float>(ws, L.gate_logit) : nullptr;
    }
    return a;
}

// The small-T gate/up launch does the softmax selection itself (saving the
// routing launch) for up to kFusedSelMaxT tokens.
bool select_fused(const moe_config& c) {
    return small_path(c) && c.family == MOE_ROUTE_SOFTMAX_TOPK && c.n_tokens <= moe::kFusedSelMaxT &&
           c.n_experts <= 256 && c.top_k <= 64;
}

moe_status stage_small_gateup(const moe_config& c, const Layout& L, void* ws, const void* x, const moe_weights& w,
                              hipStream_t s, const moe::SelParams* sel = nullptr,
                              const moe::GateParams* gate = nullptr) {
    moe::GemmArgs a = small_args(c, L, ws, w, true);
    a.act = x;
    a.out = at<void>(ws, L.h);
    if (sel) {
        a.fused_sel = 1;
        a.sel_logits = sel->logits;
        a.sel_ksplit = sel->ksplit;
        a.sel_ids = at<int32_t>(ws, L.ids);
        a.sel_wts = at<float>(ws, L.wts);
        a.sel_ids2 = sel->ids2;
        a.sel_wts2 = sel->wts2;
        if (gate && gate->w) {
            a.gate_w = gate->w;
            a.gate_x_f32 = gate->x_f32;
            a.gate_out = gate->out;
        }
    }
    const int grid = (a.has_shared ? 1 : 0) + std::min(c.n_experts, c.n_tokens * c.top_k);
    HIP_TRY(moe::launch_gemm(moe::kSmallGateUp, wkind_of(c.expert_dtype), c.expert_dtype != MOE_F32, a, grid, 1, s));
    return MOE_OK;
}

// At most 32 pairs the layer runs gate/up with one work item per pair (no
// grouping decode): nearly every pair has its own expert there, and the
// measured stage is 2-4% faster (T <= 4 at Qwen3.6 shape, K = 8); from about
// 48 pairs grouping pays (20% at 64).  h is the same bit for bit.
constexpr int kDirectGateUpMaxPairs = 32;
bool direct_gateup(const moe_config& c) { return small_path(c) && c.n_tokens * c.top_k <= kDirectGateUpMaxPairs; }

// The same stage with one work item per (token, slot) pair (no grouping);
// with `sel`, the selection runs inside the launch as in the grouped one.
moe_status stage_small_gateup_direct(const moe_config& c, const Layout& L, void* ws, const void* x,
                                     const moe_weights& w, hipStream_t s, const moe::SelParams* sel = nullptr,
                                     const moe::GateParams* gate = nullptr) {
    moe::GemmArgs a = small_args(c, L, ws, w, true);
    a.act = x;
    a.out = at<void>(ws, L.h);
    a.direct_pairs = 1;
    if (sel) {
        a.fused_sel = 1;
        a.sel_logits = sel->logits;
        a.sel_ksplit = sel->ksplit;
        a.sel_ids = at<int32_t>(ws, L.ids);
        a.sel_wts = at<float>(ws, L.wts);
        a.sel_ids2 = sel->ids2;
        a.sel_wts2 = sel->wts2;
        if (gate && gate->w) {
            a.gate_w = gate->w;
            a.gate_x_f32 = gate->x_f32;
            a.gate_out = gate->out;
        }
    }
    // the grouped launch's tile shape, so both compute each h element alike
    a.shape_grid = (a.has_shared ? 1 : 0) + std::min(c.n_experts, c.n_tokens * c.top_k);
    const int grid = (a.has_shared ? 1 : 0) + c.n_tokens * c.top_k;
    HIP_TRY(moe::launch_gemm(moe::kSmallGateUp, wkind_of(c.expert_dtype), c.expert_dtype != MOE_F32, a, grid, 1, s));
    return MOE_OK;
}

// Small-T down projection into slot rows (K routed + the shared expert per
// token), grouped by expert or, with `direct`, one work item per (token,
// slot) pair (each pair reads its expert's rows; same tile shape, so the same
// slot values).
moe_status stage_small_down(const moe_config& c, const Layout& L, void* ws, const moe_weights& w, hipStream_t s,
                            bool direct = false) {
    moe::GemmArgs a = small_args(c, L, ws, w, false);
    a.act = at<void>(ws, L.h);
    a.out = at<void>(ws, L.slots);
    const int grouped = (a.has_shared ? 1 : 0) + std::min(c.n_experts, c.n_tokens * c.top_k);
    int grid = grouped;
    if (direct) {
        a.direct_pairs = 1;
        a.shape_grid = grouped;
        grid = (a.has_shared ? 1 : 0) + c.n_tokens * c.top_k;
    }
    HIP_TRY(moe::launch_gemm(moe::kSmallDown, wkind_of(c.expert_dtype), c.expert_dtype != MOE_F32, a, grid, 1, s));
    return MOE_OK;
}

// The small-T down projection fused with the combine (bf16 or 4-bit banks).
moe::DownCombineArgs down_combine_args(const moe_config& c, const Layout& L, void* ws, const moe_weights& w,
                                       const float* residual, float* out) {
    const bool has_shared = c.d_ff_shared > 0;
    moe::DownCombineArgs d{};
    d.h = at<void>(ws, L.h); d.h_ld = h_ld(c);
    d.ids = at<int32_t>(ws, L.ids); d.wts = at<float>(ws, L.wts);
    d.w = w.down.w; d.ws = has_shared ? w.shared_down.w : nullptr;
    d.gate_logit = has_shared && w.shared_gate_vec ? at<float>(ws, L.gate_logit) : nullptr;
    d.residual = residual; d.out = out;
    d.T = c.n_tokens; d.K = c.top_k; d.E = c.n_experts; d.D = c.d_model; d.F = c.d_ff;
    d.has_shared = has_shared ? 1 : 0;
    if (c.expert_dtype == MOE_U4_AFFINE_G64) {
        d.u4 = 1;
        d.w_scale = w.down.scale; d.w_min = w.down.min;
        if (has_shared) { d.ws_scale = w.shared_down.scale; d.ws_min = w.shared_down.min; }
    }
    return d;
}

moe_status stage_experts(const moe_config& c, const Layout& L, void* ws, const void* x, const moe_weights& w,
                         const int32_t* pairs, const int4* tiles, const int32_t* n_tiles, const float* wts,
                         void* slot_out, bool slot_bf16, hipStream_t s) {
    if (moe_status st = stage_gateup(c, L, ws, x, w, pairs, tiles, n_tiles, s)) return st;
    return stage_down(c, L, ws, w, pairs, tiles, n_tiles, wts, slot_out, slot_bf16, s);
}

moe_status stage_shared(const moe_config& c, const Layout& L, void* ws, const void* x, const moe_weights& w,
                        float* shared_out, hipStream_t s) {
    const int T = c.n_tokens;
    const int tf = dense_tf(c);
    const int grid = (T + 16 * tf - 1) / (16 * tf);
    const int wk = wkind_of(c.expert_dtype);
    const bool hbf = c.expert_dtype != MOE_F32;
    const float* gl = nullptr;
    if (w.shared_gate_vec) {
        HIP_TRY(moe::launch_gate_logit(x, c.act_dtype == MOE_F32, w.shared_gate_vec, T, c.d_model,
                                       at<float>(ws, L.gate_logit), s));
        gl = at<float>(ws, L.gate_logit);
    }
    void* hs = at<void>(ws, L.hs);
    moe_matrix sg = w.shared_gate, su = w.shared_up, sd = w.shared_down;
    if (shared_dequant(c)) {
        const int Fs = c.d_ff_shared, D = c.d_model;
        uint16_t* base = at<uint16_t>(ws, L.sw);
        const moe_matrix* src[3] = {&w.shared_gate, &w.shared_up, &w.shared_down};
        moe_matrix* dst[3] = {&sg, &su, &sd};
        for (int i = 0; i < 3; ++i) {
            uint16_t* o = base + size_t(i) * Fs * D;
            const int rows = i < 2 ? Fs : D, K = i < 2 ? D : Fs;
            HIP_TRY(moe::launch_dequant_u4(src[i]->w, src[i]->scale, src[i]->min, rows, K, o, s));
            *dst[i] = moe_matrix{o, nullptr, nullptr};
        }
    }
    moe::GemmArgs a = gemm_args(sg, &su, c.d_ff_shared, c.d_model, 1);
    a.act = x; a.n_act_rows = T; a.n_rows = T; a.out = hs;
    moe::GemmArgs d = gemm_args(sd, nullptr, c.d_model, c.d_ff_shared, 1);
    d.act = hs; d.n_act_rows = T; d.n_rows = T; d.out = shared_out; d.row_scale = gl;
    if (dense_tiled(c, c.expert_dtype) || shared_dequant(c)) {
        const int g = (T + moe::tiled_rows_dense() - 1) / moe::tiled_rows_dense();
        HIP_TRY(moe::launch_gemm_tiled(moe::kDenseGateUp, true, a, g, s));
        HIP_TRY(moe::launch_gemm_tiled(moe::kDenseDown, false, d, g, s));
        return MOE_OK;
    }
    HIP_TRY(moe::launch_gemm(moe::kDenseGateUp, wk, hbf, a, grid, tf, s));
    HIP_TRY(moe::launch_gemm(moe::kDenseDown, wk, false, d, grid, tf, s));
    return MOE_OK;
}

constexpr int kMaxDev = 64;
thread_local hipEvent_t g_ev_fork[kMaxDev] = {};
thread_local hipEvent_t g_ev_join[kMaxDev] = {};

moe_status fork_join_events(hipEvent_t* fork, hipEvent_t* join) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDev) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
    if (!g_ev_fork[dev]) HIP_TRY(hipEventCreateWithFlags(&g_ev_fork[dev], hipEventDisableTiming));
    if (!g_ev_join[dev]) HIP_TRY(hipEventCreateWithFlags(&g_ev_join[dev], hipEventDisableTiming));
    *fork = g_ev_fork[dev];
    *join = g_ev_join[dev];
    return MOE_OK;
}


// x [T, D] act_dtype against a [T, D] fp32 tensor
bool overlaps(const void* x, const moe_config& c, const float* t) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(t);
    const size_t n = size_t(c.n_tokens) * c.d_model;
    const size_t xa = n * (c.act_dtype == MOE_F32 ? 4 : 2), tb = n * 4;
    return a < b + tb && b < a + xa;
}

moe_status check_norm(const moe_config& c, const float* residual, const float* w, float eps, const void* x) {
    if (!(std::isfinite(eps) && eps > 0.f)) return fail(MOE_ERR_INVALID_ARGUMENT, "eps must be finite and > 0");
    if (!residual || !x) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    auto mis = [](const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 != 0; };
    if (mis(residual) || mis(x) || (w && mis(w)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "residual, norm_weight and x must be 16-byte aligned");
    if (overlaps(x, c, residual)) return fail(MOE_ERR_INVALID_ARGUMENT, "x overlaps residual");
    return MOE_OK;
}

moe_status layer_forward_impl(const moe_config& c, const moe_weights* weights, const void* x, const float* residual,
                              float* out, int32_t* topk_ids_out, float* topk_weights_out, void* ws,
                              hipStream_t stream, hipStream_t aux_stream, const NormFold* nf = nullptr) {
    const Layout L = layout(c);
    const bool has_shared = c.d_ff_shared > 0;
    const bool slot_bf16 = c.expert_dtype != MOE_F32;
    int32_t* ids = at<int32_t>(ws, L.ids);
    float* wts = at<float>(ws, L.wts);
    const moe::SelParams P = sel_params(c, L, ws, weights->expert_bias, topk_ids_out, topk_weights_out);

    if (small_path(c)) {
        // one stream: logits -> selection (+ shared gate logit; inside the
        // gate/up launch for T <= kFusedSelMaxT) -> gate/up -> down (+ combine)
        if (moe_status st = stage_logits(c, L, ws, x, weights->router, stream, nf)) return st;
        moe::GateParams G{};
        if (has_shared && weights->shared_gate_vec) {
            G.x = x; G.w = weights->shared_gate_vec; G.D = c.d_model; G.x_f32 = c.act_dtype == MOE_F32;
            G.out = at<float>(ws, L.gate_logit);
        }
        const bool fuse = select_fused(c);
        if (!fuse) HIP_TRY(moe::launch_route_select_gate(P, G, ids, wts, stream));
        if (direct_gateup(c)) {
            if (moe_status st = stage_small_gateup_direct(c, L, ws, x, *weights, stream, fuse ? &P : nullptr, &G))
                return st;
        } else if (moe_status st = stage_small_gateup(c, L, ws, x, *weights, stream, fuse ? &P : nullptr, &G)) {
            return st;
        }
        if (down_combine_fused(c)) {
            HIP_TRY(moe::launch_down_combine(down_combine_args(c, L, ws, *weights, residual, out), stream));
            return MOE_OK;
        }
        if (moe_status st = stage_small_down(c, L, ws, *weights, stream)) return st;
        HIP_TRY(moe::launch_combine(at<void>(ws, L.slots), slot_bf16, nullptr, residual, out, c.n_tokens,
                                    c.top_k + (has_shared ? 1 : 0), c.d_model, stream));
        return MOE_OK;
    }

    float* ys = has_shared ? at<float>(ws, L.ys) : nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    const bool fork = has_shared && aux_stream && aux_stream != stream;
    if (fork) {
        if (moe_status st = fork_join_events(&ev_fork, &ev_join)) return st;
        HIP_TRY(hipEventRecord(ev_fork, stream));
        HIP_TRY(hipStreamWaitEvent(aux_stream, ev_fork, 0));
        if (moe_status st = stage_shared(c, L, ws, x, *weights, ys, aux_stream)) return st;
        HIP_TRY(hipEventRecord(ev_join, aux_stream));
    } else if (has_shared) {
        if (moe_status st = stage_shared(c, L, ws, x, *weights, ys, stream)) return st;
    }

    const int tile_rows = routed_tile_rows(c);
    int32_t* pairs = at<int32_t>(ws, L.pairs);
    int4* tiles = at<int4>(ws, L.tiles);
    int32_t* nt = at<int32_t>(ws, L.n_tiles);
    const moe::PermParams Q = perm_params(c, ids, at<int32_t>(ws, L.offsets), at<int32_t>(ws, L.active),
                                          at<int32_t>(ws, L.n_active), pairs, tiles, nt, tile_rows,
                                          at<int32_t>(ws, L.chunk_base));
    if (moe_status st = stage_logits(c, L, ws, x, weights->router, stream)) return st;
    if (permute_counts(c)) {
        moe::GateParams G{};
        HIP_TRY(moe::launch_route_select_counts(P, G, ids, wts, Q.chunk_base, stream));
        HIP_TRY(moe::launch_permute_from_counts(Q, count_chunks(c), count_chunk_tokens(c) * c.top_k, stream));
    } else if (moe::route_permute_fusable(c.n_tokens, c.n_experts, c.top_k)) {
        HIP_TRY(moe::launch_route_permute(P, ids, wts, Q, stream));
    } else {
        HIP_TRY(moe::launch_route_select(P, ids, wts, stream));
        HIP_TRY(moe::launch_permute(Q, stream));
    }
    void* slots = at<void>(ws, L.slots);
    if (moe_status st = stage_experts(c, L, ws, x, *weights, pairs, tiles, nt, wts, slots, slot_bf16, stream))
        return st;
    if (fork) HIP_TRY(hipStreamWaitEvent(stream, ev_join, 0));
    HIP_TRY(moe::launch_combine(slots, slot_bf16, ys, residual, out, c.n_tokens, c.top_k, c.d_model, stream));
    return MOE_OK;
}

// Scratch memory of moe_layer_forward_noalloc, for callers that cannot
// allocate: one array per device, held by the loaded library until the
// process ends.  Its name denotes a host-side stand-in in host code; host
// code uses only the device address that hipGetSymbolAddress returns for the
// current device (kept per device in g_scratch_ptr).
constexpr size_t kScratchBytes = size_t(32) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDev] = {};

// Device address of this device's scratch array (looked up once per device,
// with that device current).
moe_status scratch_ptr(void** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDev) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p || reinterpret_cast<uintptr_t>(p) % 256)
            return fail(MOE_ERR_HIP, "scratch array address %p is not 256-byte aligned", p);
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status status) {
    switch (raw(status)) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
    *bytes = layout(*cfg).total;
    return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* router, const float* expert_bias,
                     int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes, moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!x || !router || !topk_ids || !topk_weights) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    if (moe_status st = check_ws(*cfg, ws, ws_bytes)) return st;
    (void)hipGetLastError();
    return stage_route(*cfg, layout(*cfg), ws, x, router, expert_bias, topk_ids, topk_weights, stream);
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t* expert_offsets,
                       int32_t* active_experts, int32_t* n_active, int32_t* sorted_pairs, void* ws, size_t ws_bytes,
                       moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!topk_ids || !expert_offsets || !active_experts || !n_active || !sorted_pairs)
        return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    // the chunked permute's scratch, when the caller gives a workspace
    int32_t* chunk_base = nullptr;
    if (ws && ws_bytes >= layout(*cfg).total && reinterpret_cast<uintptr_t>(ws) % 256 == 0)
        chunk_base = at<int32_t>(ws, layout(*cfg).chunk_base);
    (void)hipGetLastError();
    HIP_TRY(moe::launch_permute(perm_params(*cfg, topk_ids, expert_offsets, active_experts, n_active, sorted_pairs,
                                            nullptr, nullptr, 16, chunk_base),
                                stream));
    return MOE_OK;
}

moe_status moe_experts(const moe_config* cfg, const void* x, const moe_weights* weights,
                       const int32_t* expert_offsets, const int32_t* active_experts, const int32_t* n_active,
                       const int32_t* sorted_pairs, const float* topk_weights, float* slot_out, void* ws,
                       size_t ws_bytes, moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!x || !expert_offsets || !active_experts || !n_active || !sorted_pairs || !topk_weights || !slot_out)
        return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    if (moe_status st = check_weights(*cfg, weights, true, false)) return st;
    if (moe_status st = check_ws(*cfg, ws, ws_bytes)) return st;
    (void)hipGetLastError();
    const Layout L = layout(*cfg);
    const int TK = cfg->n_tokens * cfg->top_k;
    const int tile_rows = routed_tile_rows(*cfg);
    int4* tiles = at<int4>(ws, L.tiles);
    int32_t* nt = at<int32_t>(ws, L.n_tiles);
    HIP_TRY(moe::launch_build_tiles(expert_offsets, active_experts, n_active, cfg->n_experts, TK, tiles, nt,
                                    int(max_tiles(TK, cfg->n_experts, tile_rows)), tile_rows, stream));
    return stage_experts(*cfg, L, ws, x, *weights, sorted_pairs, tiles, nt, topk_weights, slot_out, false, stream);
}

moe_status moe_shared_expert(const moe_config* cfg, const void* x, const moe_weights* weights, float* shared_out,
                             void* ws, size_t ws_bytes, moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->d_ff_shared == 0) return fail(MOE_ERR_INVALID_ARGUMENT, "d_ff_shared == 0: no shared expert");
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!x || !shared_out) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    if (moe_status st = check_weights(*cfg, weights, false, true)) return st;
    if (moe_status st = check_ws(*cfg, ws, ws_bytes)) return st;
    (void)hipGetLastError();
    return stage_shared(*cfg, layout(*cfg), ws, x, *weights, shared_out, stream);
}

moe_status moe_combine(const moe_config* cfg, const float* slot_out, const float* shared_out, const float* residual,
                       float* out, moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!slot_out || !residual || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    (void)hipGetLastError();
    HIP_TRY(moe::launch_combine(slot_out, false, shared_out, residual, out, cfg->n_tokens, cfg->top_k, cfg->d_model,
                                stream));
    return MOE_OK;
}

moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* weights, const void* x, const float* residual,
                             float* out, int32_t* topk_ids_out, float* topk_weights_out, void* ws, size_t ws_bytes,
                             moe_stream_t stream, moe_stream_t aux_stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!x || !residual || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    if (!weights || !weights->router) return fail(MOE_ERR_INVALID_ARGUMENT, "router weights are NULL");
    if (moe_status st = check_weights(*cfg, weights, true, true)) return st;
    if (moe_status st = check_ws(*cfg, ws, ws_bytes)) return st;
    (void)hipGetLastError();
    return layer_forward_impl(*cfg, weights, x, residual, out, topk_ids_out, topk_weights_out, ws, stream, aux_stream);
}

moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* weights, const void* x,
                                     const float* residual, float* out, int32_t* topk_ids_out,
                                     float* topk_weights_out, moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!x || !residual || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    if (!weights || !weights->router) return fail(MOE_ERR_INVALID_ARGUMENT, "router weights are NULL");
    if (moe_status st = check_weights(*cfg, weights, true, true)) return st;
    const size_t need = layout(*cfg).total;
    if (need > kScratchBytes)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL,
                    "this layer needs %zu bytes of scratch; the allocation-free entry has %zu (use "
                    "moe_layer_forward with a workspace)", need, kScratchBytes);
    void* ws = nullptr;
    if (moe_status st = scratch_ptr(&ws)) return st;
    (void)hipGetLastError();
    // one stream: no fork/join events are created
    return layer_forward_impl(*cfg, weights, x, residual, out, topk_ids_out, topk_weights_out, ws, stream, nullptr);
}

moe_status moe_layer_forward_direct(const moe_config* cfg, const moe_weights* weights, const void* x,
                                    const float* residual, float* out, int32_t* topk_ids_out,
                                    float* topk_weights_out, void* ws, size_t ws_bytes, moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!x || !residual || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    if (!weights || !weights->router) return fail(MOE_ERR_INVALID_ARGUMENT, "router weights are NULL");
    if (moe_status st = check_weights(*cfg, weights, true, true)) return st;
    if (moe_status st = check_ws(*cfg, ws, ws_bytes)) return st;
    const moe_config& c = *cfg;
    if (!small_path(c))
        return fail(MOE_ERR_UNSUPPORTED, "direct execution needs T*K <= 256 (and few pairs per expert); got %d pairs",
                    c.n_tokens * c.top_k);
    (void)hipGetLastError();
    const Layout L = layout(c);
    const bool has_shared = c.d_ff_shared > 0;
    int32_t* ids = at<int32_t>(ws, L.ids);
    float* wts = at<float>(ws, L.wts);
    const moe::SelParams P = sel_params(c, L, ws, weights->expert_bias, topk_ids_out, topk_weights_out);
    if (moe_status st = stage_logits(c, L, ws, x, weights->router, stream)) return st;
    moe::GateParams G{};
    if (has_shared && weights->shared_gate_vec) {
        G.x = x; G.w = weights->shared_gate_vec; G.D = c.d_model; G.x_f32 = c.act_dtype == MOE_F32;
        G.out = at<float>(ws, L.gate_logit);
    }
    const bool fuse = select_fused(c);
    if (!fuse) HIP_TRY(moe::launch_route_select_gate(P, G, ids, wts, stream));
    if (moe_status st = stage_small_gateup_direct(c, L, ws, x, *weights, stream, fuse ? &P : nullptr, &G)) return st;
    if (moe_status st = stage_small_down(c, L, ws, *weights, stream, true)) return st;
    HIP_TRY(moe::launch_combine(at<void>(ws, L.slots), c.expert_dtype != MOE_F32, nullptr, residual, out, c.n_tokens,
                                c.top_k + (has_shared ? 1 : 0), c.d_model, stream));
    return MOE_OK;
}

moe_status moe_rms_norm(const moe_config* cfg, const float* residual, const float* norm_weight, float eps, void* x,
                        moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (moe_status st = check_norm(*cfg, residual, norm_weight, eps, x)) return st;
    (void)hipGetLastError();
    HIP_TRY(moe::launch_rms_norm(residual, norm_weight, eps, cfg->n_tokens, cfg->d_model, x,
                                 cfg->act_dtype != MOE_F32, stream));
    return MOE_OK;
}

moe_status moe_layer_forward_norm(const moe_config* cfg, const moe_weights* weights, const float* norm_weight,
                                  float eps, const float* residual, void* x_out, float* out, int32_t* topk_ids_out,
                                  float* topk_weights_out, void* ws, size_t ws_bytes, moe_stream_t stream,
                                  moe_stream_t aux_stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!residual || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL tensor argument");
    if (!weights || !weights->router) return fail(MOE_ERR_INVALID_ARGUMENT, "router weights are NULL");
    if (moe_status st = check_weights(*cfg, weights, true, true)) return st;
    if (moe_status st = check_ws(*cfg, ws, ws_bytes)) return st;
    const moe_config& c = *cfg;
    void* x = x_out ? x_out : at<void>(ws, layout(c).xn);
    if (moe_status st = check_norm(c, residual, norm_weight, eps, x)) return st;
    if (x_out && overlaps(x_out, c, out)) return fail(MOE_ERR_INVALID_ARGUMENT, "x_out overlaps out");
    (void)hipGetLastError();
    if (norm_fusable(c)) {
        const NormFold nf{residual, norm_weight, eps, x};
        return layer_forward_impl(c, weights, x, residual, out, topk_ids_out, topk_weights_out, ws, stream,
                                  aux_stream, &nf);
    }
    HIP_TRY(moe::launch_rms_norm(residual, norm_weight, eps, c.n_tokens, c.d_model, x, c.act_dtype != MOE_F32, stream));
    return layer_forward_impl(c, weights, x, residual, out, topk_ids_out, topk_weights_out, ws, stream, aux_stream);
}

moe_status moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, moe_stream_t stream) {
    g_err[0] = 0;
    if (!buf || !sink) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL buffer or sink");
    if (reinterpret_cast<uintptr_t>(buf) % 16) return fail(MOE_ERR_INVALID_ARGUMENT, "buf must be 16-byte aligned");
    if (bytes == 0 || bytes % (size_t(1) << 18))
        return fail(MOE_ERR_INVALID_ARGUMENT, "bytes (%zu) must be a non-zero multiple of 262144", bytes);
    if (sink_words < moe::stream_read_sink_words(bytes))
        return fail(MOE_ERR_INVALID_ARGUMENT, "sink holds %zu words, %zu needed", sink_words,
                    moe::stream_read_sink_words(bytes));
    (void)hipGetLastError();
    HIP_TRY(moe::launch_stream_read(buf, bytes, sink, stream));
    return MOE_OK;
}

moe_status moe_mfma_rate(int32_t shape, int32_t workgroups, int32_t iterations, float* sink, size_t sink_words,
                         moe_stream_t stream) {
    g_err[0] = 0;
    if (shape != 0 && shape != 1) return fail(MOE_ERR_INVALID_ARGUMENT, "shape %d is not 0 or 1", int(shape));
    if (workgroups < 1 || workgroups > 65536)
        return fail(MOE_ERR_INVALID_ARGUMENT, "workgroups %d outside 1 .. 65536", int(workgroups));
    // at most 2^16 rounds: every accumulator and partial sum of a lane stays
    // an exact fp32 integer, so the sink holds the stated value
    if (iterations < 1 || iterations > (1 << 16))
        return fail(MOE_ERR_INVALID_ARGUMENT, "iterations %d outside 1 .. 65536", int(iterations));
    if (!sink) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL sink");
    if (sink_words < size_t(workgroups) * 256)
        return fail(MOE_ERR_INVALID_ARGUMENT, "sink holds %zu floats, %zu needed", sink_words, size_t(workgroups) * 256);
    (void)hipGetLastError();
    HIP_TRY(moe::launch_mfma_rate(shape, workgroups, iterations, sink, stream));
    return MOE_OK;
}

moe_status moe_l2_read_rate(int32_t pattern, int32_t workgroups, int32_t iterations, const void* buf,
                            size_t buf_bytes, uint32_t* sink, size_t sink_words, moe_stream_t stream) {
    g_err[0] = 0;
    if (pattern < 0 || pattern > 2) return fail(MOE_ERR_INVALID_ARGUMENT, "pattern %d is not 0, 1 or 2", int(pattern));
    if (workgroups < 1 || workgroups > 65536)
        return fail(MOE_ERR_INVALID_ARGUMENT, "workgroups %d outside 1 .. 65536", int(workgroups));
    if (iterations < 1 || iterations > (1 << 16))
        return fail(MOE_ERR_INVALID_ARGUMENT, "iterations %d outside 1 .. 65536", int(iterations));
    if (!buf || reinterpret_cast<uintptr_t>(buf) % 16)
        return fail(MOE_ERR_INVALID_ARGUMENT, "buf must be a 16-byte aligned device pointer");
    if (buf_bytes < moe::l2_read_buffer_bytes())
        return fail(MOE_ERR_INVALID_ARGUMENT, "buf holds %zu bytes, %zu needed", buf_bytes, moe::l2_read_buffer_bytes());
    if (!sink) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL sink");
    if (sink_words < size_t(workgroups) * 256)
        return fail(MOE_ERR_INVALID_ARGUMENT, "sink holds %zu words, %zu needed", sink_words, size_t(workgroups) * 256);
    (void)hipGetLastError();
    HIP_TRY(moe::launch_l2_read(pattern, workgroups, iterations, buf, sink, stream));
    return MOE_OK;
}

moe_status moe_layer_stage(const moe_config* cfg, const moe_weights* weights, const void* x, moe_stage stage,
                           void* ws, size_t ws_bytes, moe_stream_t stream) {
    g_err[0] = 0;
    if (moe_status st = check_config(cfg)) return st;
    if (cfg->n_tokens == 0) return MOE_OK;
    if (!x || !weights || !weights->router) return fail(MOE_ERR_INVALID_ARGUMENT, "NULL argument");
    if (moe_status st = check_weights(*cfg, weights, true, true)) return st;
    if (moe_status st = check_ws(*cfg, ws, ws_bytes)) return st;
    (void)hipGetLastError();
    const moe_config& c = *cfg;
    const Layout L = layout(c);
    int32_t* pairs = at<int32_t>(ws, L.pairs);
    int4* tiles = at<int4>(ws, L.tiles);
    int32_t* nt = at<int32_t>(ws, L.n_tiles);
    const int32_t stage_v = raw(stage);
    switch (stage_v) {
        case MOE_STAGE_ROUTER_LOGITS: return stage_logits(c, L, ws, x, weights->router, stream);
        case MOE_STAGE_GATE_UP:
        case MOE_STAGE_GATE_UP_DIRECT: {
            const bool direct = stage_v == MOE_STAGE_GATE_UP_DIRECT;
            if (!small_path(c)) {
                if (direct) return fail(MOE_ERR_UNSUPPORTED, "the direct gate/up stage needs the small-T path");
                return stage_gateup(c, L, ws, x, *weights, pairs, tiles, nt, stream);
            }
            if (!select_fused(c))
                return direct || direct_gateup(c) ? stage_small_gateup_direct(c, L, ws, x, *weights, stream)
                                                  : stage_small_gateup(c, L, ws, x, *weights, stream);
            // the launch the layer runs: selection (and the shared gate
            // logit) from the router logits in ws, then gate/up
            const moe::SelParams P = sel_params(c, L, ws, weights->expert_bias);
            moe::GateParams G{};
            if (c.d_ff_shared > 0 && weights->shared_gate_vec) {
                G.x = x; G.w = weights->shared_gate_vec; G.D = c.d_model; G.x_f32 = c.act_dtype == MOE_F32;
                G.out = at<float>(ws, L.gate_logit);
            }
            return direct || direct_gateup(c) ? stage_small_gateup_direct(c, L, ws, x, *weights, stream, &P, &G)
                                              : stage_small_gateup(c, L, ws, x, *weights, stream, &P, &G);
        }
        case MOE_STAGE_DOWN_GROUPED:
        case MOE_STAGE_DOWN_DIRECT:
            if (!small_path(c)) return fail(MOE_ERR_UNSUPPORTED, "the unfused small-T down stages need the small-T path");
            return stage_small_down(c, L, ws, *weights, stream, stage_v == MOE_STAGE_DOWN_DIRECT);
        case MOE_STAGE_DOWN:
            if (down_combine_fused(c)) {
                // the layer's own launch, writing into the workspace (y_shared region,
                // [T, D] fp32, also standing in for the residual)
                float* y = at<float>(ws, L.ys);
                HIP_TRY(moe::launch_down_combine(down_combine_args(c, L, ws, *weights, y, y), stream));
                return MOE_OK;
            }
            if (small_path(c)) return stage_small_down(c, L, ws, *weights, stream);
            return stage_down(c, L, ws, *weights, pairs, tiles, nt, at<float>(ws, L.wts), at<void>(ws, L.slots),
                              c.expert_dtype != MOE_F32, stream);
    }
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown stage %d", int(stage_v));
}

}  // extern "C"
