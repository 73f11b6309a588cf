"""GPU parity of the direct (per-pair) layer schedule, moe_layer_forward_direct,
against the fp64 oracle: the small-batch execution where every (token, slot)
pair is its own work item in both routed projections (Treebeard, "Intel SYCL
path": below a few token columns, one pair at a time instead of bucketing by
expert).  Every token's routing and output is compared; the routing also
equals the grouped schedule's bit for bit."""
import numpy as np
import pytest
import torch

from tests.gpu_harness import TOL, check_layer, check_route, make_case, run_layer, spec_of
from top_routing_grouped_amd import moe

pytestmark = pytest.mark.gpu

SMALL = {
    "small_f32": ("tiny_f32", dict(d_model=64, n_experts=32, top_k=4, d_ff=32, d_ff_shared=48)),
    "small_bf16": ("qwen_decode", dict(d_model=256, n_experts=32, top_k=4, d_ff=128, d_ff_shared=128)),
    "small_bf16_noshared": ("qwen_decode", dict(d_model=256, n_experts=48, top_k=6, d_ff=256, d_ff_shared=0)),
    "small_sigmoid": ("sigmoid_group", dict(d_model=256, n_experts=32, n_group=4, topk_group=2, top_k=4,
                                            d_ff=128, d_ff_shared=128)),
    "small_u4": ("qwen_u4", dict(d_model=256, n_experts=32, top_k=4, d_ff=128, d_ff_shared=128)),
}
CASES = ([("qwen_decode", {}, T) for T in (1, 2, 4, 8, 16, 32)] + [("qwen_u4", {}, T) for T in (1, 8, 64)]
         + [("sigmoid_group", {}, T) for T in (1, 8, 32)] + [("tiny_f32", {}, 4)]
         + [(SMALL[n][0], SMALL[n][1], T) for n in SMALL for T in (1, 9, 37)])


def run_direct(case):
    s = case.spec
    cfg = moe.config_from_spec(s)
    ws = moe.alloc_workspace(cfg)
    ids = torch.full((s.n_tokens, s.top_k), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((s.n_tokens, s.top_k), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.full_like(case.r, float("nan"))
    moe.layer_forward_direct(cfg, moe.weights_struct(case.w), case.x, case.r, out, ids, wts, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), wts.cpu().numpy()


@pytest.mark.parametrize("base,kw,T", CASES)
def test_direct_layer_matches_oracle(base, kw, T):
    print(f"direct {base} {kw} T={T}", flush=True)
    case = make_case(spec_of(base, n_tokens=T, **kw))
    out, ids, wts = run_direct(case)
    z, rt = case.oracle_route()
    check_route(case, ids, wts, z, rt)
    err = check_layer(case, out, ids)
    # the grouped schedule selects identically and lands within the same tolerance
    g_out, g_ids, g_wts = run_layer(case, aux=False)
    assert np.array_equal(ids, g_ids) and np.array_equal(wts.view(np.uint32), g_wts.view(np.uint32))
    if case.spec.expert_dtype == "f32":  # both take the unfused down and the combine
        assert np.array_equal(out.view(np.uint32), g_out.view(np.uint32))
    print(f"direct {base} T={T}: y_moe normwise error {err:.2e} (gate {TOL[case.spec.expert_dtype]})")


def test_direct_layer_refuses_large_batches():
    case = make_case(spec_of("qwen_decode", n_tokens=64))  # 512 pairs: the grouped large-T schedule
    cfg = moe.config_from_spec(case.spec)
    ws = moe.alloc_workspace(cfg)
    out = torch.empty_like(case.r)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_forward_direct(cfg, moe.weights_struct(case.w), case.x, case.r, out, None, None, ws)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
