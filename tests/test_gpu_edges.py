"""GPU parity at the edges of what the library accepts, against the fp64 oracle:
the largest expert count and top-k (E = 1024, K = 32, both routing families,
every schedule from the small-T path to the tiled large-T path), top-1
routing, K = E (every expert selected: a dense softmax mixture), and a router
that ties every expert, so that every token takes experts 0..K-1 (the lowest
index wins, [T] "Routing math" reading R1) and K experts each receive all T
pairs (one expert spanning many GEMM tiles)."""
import numpy as np
import pytest

from tests.gpu_harness import TOL, check_layer, check_route, compare_tokens, make_case, run_layer, spec_of

pytestmark = pytest.mark.gpu

SMALL_DIMS = dict(d_model=256, d_ff=128, d_ff_shared=128)


def _layer_vs_oracle(case):
    out, ids, wts = run_layer(case)
    z, rt = case.oracle_route()
    flagged, _ = check_route(case, ids, wts, z, rt)
    toks = compare_tokens(case, ids)
    err = check_layer(case, out, ids, tokens=toks)
    print(f"layer output compared on {toks.size} of {case.spec.n_tokens} tokens")
    return ids, wts, flagged, err


@pytest.mark.parametrize("family,T", [("softmax", 3), ("softmax", 200), ("softmax", 2048),
                                      ("sigmoid_group", 3), ("sigmoid_group", 200)])
def test_layer_max_experts_and_top_k(family, T):
    if family == "softmax":
        spec = spec_of("qwen_decode", n_tokens=T, n_experts=1024, top_k=32, **SMALL_DIMS)
    else:
        spec = spec_of("sigmoid_group", n_tokens=T, n_experts=1024, n_group=16, topk_group=4, top_k=32,
                       **SMALL_DIMS)
    ids, _, flagged, err = _layer_vs_oracle(make_case(spec))
    assert ids.min() >= 0 and ids.max() < 1024
    print(f"{family} E=1024 K=32 T={T}: {flagged} near-tie tokens, y_moe normwise error {err:.2e}")


@pytest.mark.parametrize("T", [1, 37, 1000])
def test_layer_top1(T):
    spec = spec_of("qwen_decode", n_tokens=T, n_experts=64, top_k=1, **SMALL_DIMS)
    _, wts, _, err = _layer_vs_oracle(make_case(spec))
    np.testing.assert_allclose(wts, 1.0, rtol=1e-6)  # one selected expert carries the whole weight
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("T", [5, 300])
def test_layer_every_expert_selected(T):
    spec = spec_of("qwen_decode", n_tokens=T, n_experts=16, top_k=16, **SMALL_DIMS)
    ids, wts, _, _ = _layer_vs_oracle(make_case(spec))
    assert (np.sort(ids, axis=1) == np.arange(16)[None]).all()
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=1e-5)


@pytest.mark.parametrize("dtype,T", [("bf16", 37), ("bf16", 700), ("bf16", 5000), ("u4", 37), ("u4", 700)])
def test_layer_all_tied_router_hot_experts(dtype, T):
    base = "qwen_decode" if dtype == "bf16" else "qwen_u4"
    spec = spec_of(base, n_tokens=T, n_experts=32, top_k=4, **SMALL_DIMS)
    case = make_case(spec, cache_key=("tied", dtype, T))
    case.w.router.zero_()
    case.wr64[:] = 0.0
    out, ids, wts = run_layer(case)
    assert (ids == np.arange(4)[None]).all()  # all logits equal: the lowest indices win
    np.testing.assert_allclose(wts, 0.25, rtol=1e-6)
    err = check_layer(case, out, ids, tokens=compare_tokens(case, ids))
    print(f"{dtype} T={T}: experts 0..3 with {T} pairs each, y_moe normwise error {err:.2e}")


@pytest.mark.parametrize("dtype,F", [("bf16", 128), ("bf16", 256), ("bf16", 768), ("bf16", 1024),
                                     ("u4", 256), ("u4", 768), ("u4", 1024)])
@pytest.mark.parametrize("T", [3, 16])
def test_layer_fused_down_combine_every_d_ff(dtype, F, T):
    """Each d_ff the fused small-T down + combine launch takes (bf16: 128 ..
    1024; 4-bit: multiples of 256) against the oracle, with one and with
    several units per wave (T = 16, K = 4 and the shared expert: 80 units,
    the 4-bit launch's three-units-in-flight schedule)."""
    base = "qwen_decode" if dtype == "bf16" else "qwen_u4"
    spec = spec_of(base, n_tokens=T, d_model=256, n_experts=32, top_k=4, d_ff=F, d_ff_shared=F)
    _, _, _, err = _layer_vs_oracle(make_case(spec))
    print(f"{dtype} d_ff={F} T={T}: y_moe normwise error {err:.2e}")


def test_layer_max_tokens_qwen_prefill():
    """T = 32768 at Qwen3.6 shape with skewed routing (262144 pairs): the
    routed down projection has 8 row blocks x more than 2048 token tiles of
    128 pairs, more items than the persistent launch's per-workgroup table
    holds (8 XCDs x 32 workgroups x 64), so it runs the non-persistent tiled
    kernel; every token's routing against the oracle, the layer output on
    the first and last pair of every 128-pair token tile of every active
    expert (so every GEMM work item) plus random tokens."""
    T = 32768
    case = make_case(spec_of("qwen_prefill_skew", n_tokens=T))
    s = case.spec
    assert 8 * (s.n_tokens * s.top_k // 128) >= 8 * 32 * 64  # down items: past the persistent table
    ids, wts, flagged, err = _layer_vs_oracle(case)
    print(f"qwen_prefill_skew T={T}: {flagged} near-tie tokens, y_moe normwise error {err:.2e}")


@pytest.mark.parametrize("G,TG,K,bias,T", [
    (1, 1, 8, True, 5), (1, 1, 8, True, 300),  # one group: plain sigmoid top-k of score + bias
    (8, 8, 8, True, 37),  # every group kept
    (8, 1, 8, True, 37),  # one group kept: all K experts of the best group (groups of 8)
    (32, 4, 6, True, 37),  # groups of 2: a group's score is the sum of its two experts
    (8, 4, 8, False, 37), (8, 4, 8, False, 1000),  # no expert_bias, routed_scaling 1
])
def test_layer_sigmoid_group_degenerate(G, TG, K, bias, T):
    """The group top-k family at its degenerate settings, 64 experts, against
    the oracle (small-T and, at T = 300 / 1000, the medium and tiled paths)."""
    spec = spec_of("sigmoid_group", n_tokens=T, n_experts=64, n_group=G, topk_group=TG, top_k=K,
                   bias_var=0.1 if bias else 0.0, routed_scaling=2.5 if bias else 1.0, **SMALL_DIMS)
    case = make_case(spec, cache_key=("sigmoid_degenerate", G, TG, K, bias))
    if not bias:  # the NULL expert_bias pointer (the generator draws zeros)
        case.w.expert_bias = None
        case.bias64 = None
    ids, wts, flagged, err = _layer_vs_oracle(case)
    assert err <= TOL["bf16"]
    if TG == 1:  # every token's experts lie in one group
        assert (ids // (64 // G) == ids[:, :1] // (64 // G)).all()
    print(f"G={G} TG={TG} K={K} bias={bias} T={T}: {flagged} near-tie tokens, y_moe normwise error {err:.2e}")


# Token counts on both sides of every switch of the schedule at E=32, K=4:
# selection folded into the gate/up launch (T <= 8), dense 64-token tiles
# (T >= 64), the small-T path (T*K <= 256), the tiled router and shared expert
# (T >= 128), the tiled routed GEMMs (bf16: T*K >= 16 E; 4-bit with d_ff 128,
# too short a reduction for the tiled 4-bit kernel: 64-token register tiles
# from T*K >= 64 E) and the chunked permute (T*K >= 4096).
BOUNDARY_T = [8, 9, 63, 64, 65, 127, 128, 129, 511, 512, 513, 1023, 1024]


@pytest.mark.parametrize("dtype", ["bf16", "u4", "sigmoid"])
@pytest.mark.parametrize("T", BOUNDARY_T)
def test_layer_schedule_boundaries(dtype, T):
    base = {"bf16": "qwen_decode", "u4": "qwen_u4", "sigmoid": "sigmoid_group"}[dtype]
    extra = dict(n_group=4, topk_group=2) if dtype == "sigmoid" else {}
    spec = spec_of(base, n_tokens=T, d_model=256, n_experts=32, top_k=4, d_ff=128, d_ff_shared=128, **extra)
    case = make_case(spec, cache_key=("boundaries", dtype))
    out, ids, wts = run_layer(case)
    z, rt = case.oracle_route()
    check_route(case, ids, wts, z, rt)
    check_layer(case, out, ids)


# The permute that runs from the selection launch's per-block pair counts
# (from 4096 pairs, E <= 256; blocks of 32 tokens in the softmax family, 16
# in the group family): expert counts whose thread slices divide unevenly,
# a last chunk of a few tokens, several chunks per permute block, and one
# chunk per block (32 tokens x K = 32 = 1024 pairs).
COUNTS_CASES = [
    ("qwen_decode", 1030, dict(n_experts=16, top_k=4)),  # 33 chunks, the last of 6 tokens; 64 slices of experts
    ("qwen_decode", 517, dict(n_experts=48, top_k=8, d_ff_shared=0)),  # 4 chunks per block, 5 blocks
    ("qwen_decode", 130, dict(n_experts=256, top_k=32)),  # one chunk per block
    ("sigmoid_group", 600, dict(n_experts=64, n_group=8, topk_group=4, top_k=8)),  # 16-token chunks
    ("qwen_u4", 1100, dict(n_experts=80, top_k=4)),  # 4-bit experts on the same permute
]


@pytest.mark.parametrize("base,T,kw", COUNTS_CASES)
def test_layer_permute_from_block_counts(base, T, kw):
    dims = dict(SMALL_DIMS)
    dims.update(kw)
    spec = spec_of(base, n_tokens=T, **dims)
    assert T * spec.top_k >= 4096 and spec.n_experts <= 256
    case = make_case(spec, cache_key=("counts", base, T))
    out, ids, wts = run_layer(case)
    z, rt = case.oracle_route()
    flagged, _ = check_route(case, ids, wts, z, rt)
    err = check_layer(case, out, ids)
    assert err <= TOL[spec.expert_dtype]
    print(f"{base} T={T} {kw}: {flagged} near-tie tokens, y_moe normwise error {err:.2e}")
