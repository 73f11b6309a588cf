"""GPU test of moe_layer_forward_noalloc, the entry point that allocates
nothing (its scratch is a fixed array inside the library), against
moe_layer_forward with a caller workspace on the same inputs: routing ids,
routing weights and layer output bit for bit, on two calls in a row with the
second on fewer tokens (the array keeps the first call's contents), plus the
refusal of a layer whose scratch need exceeds the array."""
import numpy as np
import pytest
import torch

from tests.gpu_harness import make_case, spec_of
from top_routing_grouped_amd import moe

pytestmark = pytest.mark.gpu

SMALL_BF16 = dict(d_model=256, n_experts=32, top_k=4, d_ff=128, d_ff_shared=128)


def _outputs(case):
    s = case.spec
    out = torch.full_like(case.r, float("nan"))
    ids = torch.full((s.n_tokens, s.top_k), -1, dtype=torch.int32, device="cuda")
    wts = torch.full((s.n_tokens, s.top_k), float("nan"), dtype=torch.float32, device="cuda")
    return out, ids, wts


def _with_workspace(case):
    cfg = moe.config_from_spec(case.spec)
    ws = moe.alloc_workspace(cfg)
    out, ids, wts = _outputs(case)
    moe.layer_forward(cfg, moe.weights_struct(case.w), case.x, case.r, out, ids, wts, ws)
    torch.cuda.synchronize()
    return out, ids, wts


def _noalloc(case):
    cfg = moe.config_from_spec(case.spec)
    out, ids, wts = _outputs(case)
    moe.layer_forward_noalloc(cfg, moe.weights_struct(case.w), case.x, case.r, out, ids, wts)
    torch.cuda.synchronize()
    return out, ids, wts


def _same_bits(a, b):
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int32), v.view(torch.int32))


@pytest.mark.parametrize("base,kw,T1,T2", [
    ("qwen_decode", {}, 32, 8),  # small-T path, selection folded into gate/up
    ("qwen_u4", {}, 512, 64),  # 4-bit register-tiled path, 23 MiB of scratch
    ("sigmoid_group", {}, 200, 3),  # group top-k family
    ("qwen_decode", SMALL_BF16, 700, 37),  # tiled routed GEMMs on one stream, then the small path
])
def test_noalloc_matches_workspace_entry(base, kw, T1, T2):
    print(f"noalloc {base} {kw} T={T1} then T={T2}", flush=True)
    first = make_case(spec_of(base, n_tokens=T1, **kw))
    second = make_case(spec_of(base, n_tokens=T2, **kw))
    got1 = _noalloc(first)
    got2 = _noalloc(second)  # fewer tokens, over the first call's scratch contents
    _same_bits(got1, _with_workspace(first))
    _same_bits(got2, _with_workspace(second))
    assert torch.isfinite(got2[0]).all()


def test_noalloc_refuses_a_layer_beyond_its_scratch():
    case = make_case(spec_of("qwen_decode", n_tokens=512))
    cfg = moe.config_from_spec(case.spec)
    assert moe.workspace_size(cfg) > 32 << 20
    out, ids, wts = _outputs(case)
    with pytest.raises(moe.MoeError) as e:
        moe.layer_forward_noalloc(cfg, moe.weights_struct(case.w), case.x, case.r, out, ids, wts)
    assert e.value.status == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.isnan(out).all() and (ids == -1).all()  # nothing was launched
