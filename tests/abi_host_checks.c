/* Host-side argument checks of every entry point in include/moe.h, called as
 * a C program calls them, against a build of the C ABI layer with
 * AddressSanitizer and UndefinedBehaviorSanitizer on its host code
 * (tests/test_abi_sanitized.py builds and runs it).  Every call below fails
 * (or succeeds with n_tokens == 0) in the host checks, before any HIP call:
 * nothing touches a GPU.  Fake device pointers are never dereferenced.
 * Enum-typed fields and arguments also receive values outside their
 * enumerators, as C allows.  Prints one line per failed check and exits
 * non-zero if any failed. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static int g_failed = 0;
#define CHECK(expr, want)                                                                              \
    do {                                                                                               \
        const moe_status got_ = (expr);                                                                \
        if (got_ != (want)) {                                                                          \
            printf("FAIL line %d: %s -> %d (%s), want %d\n", __LINE__, #expr, (int)got_,               \
                   moe_last_error(), (int)(want));                                                     \
            ++g_failed;                                                                                \
        }                                                                                              \
    } while (0)

static moe_config cfg6(int T, int D, int E, int K, int F, int Fs) {
    moe_config c;
    memset(&c, 0, sizeof(c));
    c.n_tokens = T; c.d_model = D; c.n_experts = E; c.top_k = K; c.d_ff = F; c.d_ff_shared = Fs;
    c.family = MOE_ROUTE_SOFTMAX_TOPK; c.n_group = 1; c.topk_group = 1; c.routed_scaling = 1.0f;
    c.act_dtype = MOE_BF16; c.router_dtype = MOE_BF16; c.expert_dtype = MOE_BF16;
    return c;
}
static moe_config cfg(int T) { return cfg6(T, 2048, 256, 8, 512, 512); }

int main(void) {
    void* const fake = (void*)((uintptr_t)1 << 20); /* aligned, never dereferenced */
    void* const fake2 = (void*)((uintptr_t)1 << 24);
    void* const ws = (void*)((uintptr_t)1 << 28);
    const float* ff = (const float*)fake;
    float* fo = (float*)fake2;
    int32_t* ip = (int32_t*)fake;
    size_t n = 0;

    /* ---- configs */
    moe_config c = cfg(8);
    CHECK(moe_workspace_size(&c, &n), MOE_OK);
    const size_t need = n;
    CHECK(moe_workspace_size(NULL, &n), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_workspace_size(&c, NULL), MOE_ERR_INVALID_ARGUMENT);
    struct { moe_config c; moe_status want; } bad[] = {
        {cfg6(8, 2048, 256, 0, 512, 512), MOE_ERR_INVALID_ARGUMENT}, {cfg6(8, 2048, 64, 33, 512, 512), MOE_ERR_UNSUPPORTED},
        {cfg6(8, 2048, 250, 8, 512, 512), MOE_ERR_UNSUPPORTED},      {cfg6(8, 2048, 2048, 8, 512, 512), MOE_ERR_UNSUPPORTED},
        {cfg6(-1, 2048, 256, 8, 512, 512), MOE_ERR_INVALID_ARGUMENT}, {cfg6(8, 2000, 256, 8, 512, 512), MOE_ERR_UNSUPPORTED},
        {cfg6(8, 2048, 256, 8, 96, 512), MOE_ERR_UNSUPPORTED},       {cfg6(8, 2048, 256, 8, 512, -1), MOE_ERR_INVALID_ARGUMENT},
        {cfg6(8, 0, 256, 8, 512, 512), MOE_ERR_INVALID_ARGUMENT},     {cfg6(1 << 30, 2048, 256, 8, 512, 512), MOE_ERR_UNSUPPORTED}};
    for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) CHECK(moe_workspace_size(&bad[i].c, &n), bad[i].want);
    moe_config s = cfg6(8, 2048, 128, 8, 512, 512);
    s.family = MOE_ROUTE_SIGMOID_GROUP_TOPK; s.n_group = 8; s.topk_group = 4; s.routed_scaling = 2.5f;
    CHECK(moe_workspace_size(&s, &n), MOE_OK);
    moe_config s2 = s; s2.n_group = 6; CHECK(moe_workspace_size(&s2, &n), MOE_ERR_INVALID_ARGUMENT);
    s2 = s; s2.topk_group = 9; CHECK(moe_workspace_size(&s2, &n), MOE_ERR_INVALID_ARGUMENT);
    s2 = s; s2.routed_scaling = NAN; CHECK(moe_workspace_size(&s2, &n), MOE_ERR_INVALID_ARGUMENT);
    s2 = s; s2.routed_scaling = -1.0f; CHECK(moe_workspace_size(&s2, &n), MOE_ERR_INVALID_ARGUMENT);
    s2 = s; s2.family = (moe_route_family)7; CHECK(moe_workspace_size(&s2, &n), MOE_ERR_INVALID_ARGUMENT);
    s2 = s; s2.family = (moe_route_family)-1; CHECK(moe_workspace_size(&s2, &n), MOE_ERR_INVALID_ARGUMENT);
    moe_config u4 = cfg6(8, 2048, 256, 4, 512, 512); u4.expert_dtype = MOE_U4_AFFINE_G64;
    CHECK(moe_workspace_size(&u4, &n), MOE_OK);
    moe_config u4big = u4; u4big.d_model = 8192; CHECK(moe_workspace_size(&u4big, &n), MOE_ERR_UNSUPPORTED);
    moe_config mix = cfg(8); mix.router_dtype = MOE_F32; CHECK(moe_workspace_size(&mix, &n), MOE_ERR_UNSUPPORTED);
    mix = cfg(8); mix.act_dtype = MOE_U4_AFFINE_G64; CHECK(moe_workspace_size(&mix, &n), MOE_ERR_UNSUPPORTED);
    mix = cfg(8); mix.expert_dtype = (moe_dtype)1000; CHECK(moe_workspace_size(&mix, &n), MOE_ERR_UNSUPPORTED);
    mix = cfg(8); mix.act_dtype = mix.router_dtype = (moe_dtype)-5; CHECK(moe_workspace_size(&mix, &n), MOE_ERR_UNSUPPORTED);

    /* ---- weights records */
    moe_weights w, none, wu, missing;
    memset(&w, 0, sizeof(w));
    memset(&none, 0, sizeof(none));
    w.router = fake;
    w.gate.w = w.up.w = w.down.w = fake;
    w.shared_gate.w = w.shared_up.w = w.shared_down.w = fake;
    wu = w; /* 4-bit banks without their scales and mins */
    missing = w; missing.shared_down.w = NULL;

    /* ---- routing and permute */
    CHECK(moe_route(&c, NULL, fake, NULL, (int32_t*)fake2, fo, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_route(&c, fake, fake, NULL, (int32_t*)fake2, fo, ws, 16, NULL), MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_route(&c, fake, fake, NULL, (int32_t*)fake2, fo, (void*)4100, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_route(&c, fake, fake, NULL, (int32_t*)fake2, fo, NULL, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_permute(&c, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_permute(NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_ERR_INVALID_ARGUMENT);

    /* ---- experts, shared expert, combine */
    CHECK(moe_experts(&c, fake, &none, ip, ip, ip, ip, ff, fo, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_experts(&c, fake, NULL, ip, ip, ip, ip, ff, fo, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_experts(&c, fake, &w, ip, ip, ip, ip, ff, NULL, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_experts(&u4, fake, &wu, ip, ip, ip, ip, ff, fo, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    moe_config c0 = cfg6(8, 2048, 256, 8, 512, 0);
    CHECK(moe_shared_expert(&c0, fake, &w, fo, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_shared_expert(&c, fake, &missing, fo, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_combine(&c, NULL, NULL, ff, fo, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_combine(NULL, ff, NULL, ff, fo, NULL), MOE_ERR_INVALID_ARGUMENT);

    /* ---- whole-layer entries */
    CHECK(moe_layer_forward(&c, &none, fake, ff, fo, NULL, NULL, ws, need, NULL, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_layer_forward(&c, &w, NULL, ff, fo, NULL, NULL, ws, need, NULL, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_layer_forward(&c, &w, fake, ff, fo, NULL, NULL, ws, need - 1, NULL, NULL), MOE_ERR_WORKSPACE_TOO_SMALL);
    CHECK(moe_layer_forward_direct(&c, &w, fake, NULL, fo, NULL, NULL, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    moe_config big = cfg(64); /* 512 pairs: beyond the direct schedule */
    CHECK(moe_workspace_size(&big, &n), MOE_OK);
    CHECK(moe_layer_forward_direct(&big, &w, fake, ff, fo, NULL, NULL, ws, n, NULL), MOE_ERR_UNSUPPORTED);
    moe_config huge = cfg(512); /* scratch need above the allocation-free entry's array */
    CHECK(moe_layer_forward_noalloc(&huge, &w, fake, ff, fo, NULL, NULL, NULL), MOE_ERR_WORKSPACE_TOO_SMALL);
    if (strlen(moe_last_error()) == 0) {
        printf("FAIL: no message for the refused allocation-free call\n");
        ++g_failed;
    }
    CHECK(moe_layer_forward_noalloc(&c, &none, fake, ff, fo, NULL, NULL, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_layer_stage(&c, &w, NULL, MOE_STAGE_GATE_UP, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_layer_stage(&c, &w, fake, MOE_STAGE_GATE_UP, ws, 8, NULL), MOE_ERR_WORKSPACE_TOO_SMALL);

    /* ---- RMS norm entries */
    const float bad_eps[] = {0.0f, -1e-6f, INFINITY, NAN};
    for (int i = 0; i < 4; ++i) CHECK(moe_rms_norm(&c, ff, NULL, bad_eps[i], fake2, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_rms_norm(&c, ff, NULL, 1e-6f, NULL, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_rms_norm(&c, (const float*)(((uintptr_t)1 << 20) + 8), NULL, 1e-6f, fake2, NULL),
          MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_rms_norm(&c, ff, NULL, 1e-6f, (void*)(((uintptr_t)1 << 20) + 256), NULL),
          MOE_ERR_INVALID_ARGUMENT); /* x overlaps the residual */
    CHECK(moe_layer_forward_norm(&c, &w, NULL, 0.0f, ff, NULL, fo, NULL, NULL, ws, need, NULL, NULL),
          MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_layer_forward_norm(&c, &w, NULL, 1e-6f, ff, (void*)(((uintptr_t)1 << 24) + 64), fo, NULL, NULL, ws,
                                 need, NULL, NULL),
          MOE_ERR_INVALID_ARGUMENT); /* x_out overlaps out */

    /* ---- zero tokens: every entry returns MOE_OK and launches nothing */
    moe_config z = cfg(0);
    CHECK(moe_route(&z, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    CHECK(moe_permute(&z, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    CHECK(moe_experts(&z, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    CHECK(moe_combine(&z, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    CHECK(moe_layer_forward(&z, &none, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL), MOE_OK);
    CHECK(moe_layer_forward_noalloc(&z, &none, NULL, NULL, NULL, NULL, NULL, NULL), MOE_OK);
    CHECK(moe_layer_forward_direct(&z, &none, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL), MOE_OK);
    CHECK(moe_rms_norm(&z, NULL, NULL, 1e-6f, NULL, NULL), MOE_OK);

    /* ---- an unknown stage and status */
    CHECK(moe_layer_stage(&c, &w, fake, (moe_stage)99, ws, need, NULL), MOE_ERR_INVALID_ARGUMENT);
    /* streaming read: NULL buffers, misalignment, sizes off the 256 KiB grid, a short sink */
    uint32_t* sink = (uint32_t*)(((uintptr_t)1 << 20) + 64);
    CHECK(moe_stream_read(NULL, 1 << 18, sink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_stream_read(fake, 1 << 18, NULL, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_stream_read((const void*)(((uintptr_t)1 << 20) + 8), 1 << 18, sink, 256, NULL),
          MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_stream_read(fake, 0, sink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_stream_read(fake, (1 << 18) + 1024, sink, 1 << 20, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_stream_read(fake, 1 << 18, sink, 255, NULL), MOE_ERR_INVALID_ARGUMENT);
    /* MFMA issue-rate loop: shapes, counts and sinks off its grid */
    float* fsink = (float*)(((uintptr_t)1 << 20) + 64);
    CHECK(moe_mfma_rate(2, 1, 1, fsink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_mfma_rate(0, 0, 1, fsink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_mfma_rate(0, 1, 0, fsink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_mfma_rate(1, 1, (1 << 16) + 1, fsink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_mfma_rate(0, 2, 1, fsink, 511, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_mfma_rate(0, 1, 1, NULL, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    /* L2 read-rate loop: patterns, counts, buffers and sinks off its grid */
    CHECK(moe_l2_read_rate(3, 1, 1, fake, 1 << 20, sink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_l2_read_rate(0, 65537, 1, fake, 1 << 20, sink, (size_t)65537 * 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_l2_read_rate(1, 1, (1 << 16) + 1, fake, 1 << 20, sink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_l2_read_rate(2, 1, 1, NULL, 1 << 20, sink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_l2_read_rate(2, 1, 1, (const void*)(((uintptr_t)1 << 20) + 8), 1 << 20, sink, 256, NULL),
          MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_l2_read_rate(0, 1, 1, fake, (1 << 20) - 16, sink, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_l2_read_rate(0, 1, 1, fake, 1 << 20, NULL, 256, NULL), MOE_ERR_INVALID_ARGUMENT);
    CHECK(moe_l2_read_rate(0, 2, 1, fake, 1 << 20, sink, 511, NULL), MOE_ERR_INVALID_ARGUMENT);
    const int codes[] = {MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP,
                         99, -3};
    for (int i = 0; i < 7; ++i) {
        const char* t = moe_status_string((moe_status)codes[i]);
        if (!t || !*t) {
            printf("FAIL: empty status string for %d\n", codes[i]);
            ++g_failed;
        }
    }
    printf("%s: %d failed\n", g_failed ? "FAILED" : "ok", g_failed);
    return g_failed ? 1 : 0;
}
