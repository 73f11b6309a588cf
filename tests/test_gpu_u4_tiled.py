"""GPU parity of 4-bit affine group-64 layers on the persistent LDS-tiled routed
GEMMs (codes and group scales staged in LDS; 64-token tiles up to 64 pairs
per expert, 128-token tiles from there), which take 4-bit layers averaging
at least 16 pairs per expert when both routed GEMMs fit them: every token's
routing and layer output against the fp64 oracle (edge0 page, tier table:
4-bit affine, group 64; Treebeard page, "Routed expert computation").  The shapes cover the switch point, the smallest
reduction the layer gives it (four K steps), rows past a partial row block,
both scale-buffer sizes of the down projection, the largest gate/up
reduction (32 groups), experts spanning many token tiles and skewed
routing."""
import numpy as np
import pytest

from tests.gpu_harness import TOL, check_layer, check_route, compare_tokens, make_case, run_layer, spec_of

pytestmark = pytest.mark.gpu


def _layer_vs_oracle(case):
    out, ids, wts = run_layer(case)
    z, rt = case.oracle_route()
    flagged, _ = check_route(case, ids, wts, z, rt)
    toks = compare_tokens(case, ids)
    assert toks.size == case.spec.n_tokens
    err = check_layer(case, out, ids, tokens=toks)
    return ids, flagged, err


def _tiled(spec):
    """Whether the layer takes the tiled 4-bit routed GEMMs (mirrors the
    library's rule: >= 16 pairs per expert, reductions of 3..32 groups;
    the layer takes multiples of 128 only, so at least 4)."""
    pairs = spec.n_tokens * spec.top_k
    return (pairs >= 16 * spec.n_experts and spec.d_model % 64 == 0 and spec.d_ff % 64 == 0
            and 3 <= spec.d_model // 64 <= 32 and 3 <= spec.d_ff // 64 <= 32)


@pytest.mark.parametrize("T", [127, 128, 300, 511, 512, 3000])
def test_u4_tiled_switch_point(T):
    """E = 32, K = 4: T = 127 keeps the 16-token register tiles, T >= 128
    takes the tiled kernel, with 64-token tiles below 64 pairs per expert
    (T < 512) and 128-token tiles from there."""
    spec = spec_of("qwen_u4", n_tokens=T, d_model=256, n_experts=32, top_k=4, d_ff=256, d_ff_shared=256)
    assert _tiled(spec) == (T >= 128)
    _, flagged, err = _layer_vs_oracle(make_case(spec))
    assert err <= TOL["u4"]
    print(f"4-bit T={T} (tiled: {_tiled(spec)}): {flagged} near-tie tokens, y_moe normwise error {err:.2e}")


@pytest.mark.parametrize("D,F,E,K,T", [
    (384, 384, 16, 4, 900),     # down: 1.5 row blocks of 256 (the second partial), 6 groups
    (2048, 1024, 16, 2, 512),   # gate/up 32 groups (the largest), down 16 groups (the larger scale buffer)
    (512, 2048, 16, 2, 400),    # down 32 groups (64-token tiles)
])
def test_u4_tiled_shapes(D, F, E, K, T):
    spec = spec_of("qwen_u4", n_tokens=T, d_model=D, n_experts=E, top_k=K, d_ff=F, d_ff_shared=F)
    assert _tiled(spec)
    _, flagged, err = _layer_vs_oracle(make_case(spec))
    assert err <= TOL["u4"]
    print(f"4-bit D={D} F={F} E={E} K={K} T={T}: {flagged} near-tie tokens, y_moe normwise error {err:.2e}")


def test_u4_tiled_hot_experts():
    """A router that ties every expert: experts 0..3 each take all 3000
    tokens (24 token tiles each, the last one partial)."""
    T = 3000
    spec = spec_of("qwen_u4", n_tokens=T, d_model=256, n_experts=32, top_k=4, d_ff=256, d_ff_shared=256)
    case = make_case(spec, cache_key=("u4_tiled_tied", T))
    case.w.router.zero_()
    case.wr64[:] = 0.0
    out, ids, wts = run_layer(case)
    assert (ids == np.arange(4)[None]).all()
    np.testing.assert_allclose(wts, 0.25, rtol=1e-6)
    err = check_layer(case, out, ids, tokens=compare_tokens(case, ids))
    assert err <= TOL["u4"]
    print(f"4-bit tied router T={T}: y_moe normwise error {err:.2e}")


@pytest.mark.parametrize("T", [2048, 4096])
def test_u4_tiled_qwen_skewed(T):
    """Qwen3.6 shape with 4-bit experts, K = 4 and the skewed routing of the
    prefill workload (hot experts with many tiles, cold ones with one
    partial tile)."""
    spec = spec_of("qwen_prefill_skew", n_tokens=T, top_k=4, expert_dtype="u4")
    assert _tiled(spec)
    _, flagged, err = _layer_vs_oracle(make_case(spec))
    assert err <= TOL["u4"]
    print(f"4-bit skewed Qwen T={T}: {flagged} near-tie tokens, y_moe normwise error {err:.2e}")
