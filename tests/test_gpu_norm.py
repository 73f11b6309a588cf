"""GPU parity of the RMS normalisation of the attention residual and of the
layer entry that starts from that residual, against the fp64 oracle.

x = r / sqrt(mean(r^2) + eps) * w is computed by the kernel in fp32 and stored
once in the activation type.  Comparison rule for x:
  * bf16: bit-exact wherever the exact value is farther than the kernel's
    error bound from a bf16 rounding boundary; inside that band either of the
    two neighbouring bf16 values is correct (the decision is taken in fp32,
    whose sum order the oracle does not reproduce);
  * fp32: within the error bound of the exact value.
The bound: a lane sums D/64 squares with fused multiply-adds, six butterfly
additions follow, then the mean, the eps addition, the square root (which
halves the relative error), the reciprocal and two products:
((D/64 + 8)/2 + 4) units of 2^-24, taken twice over as margin.

The layer's output is compared with the oracle layer run on the oracle's own
x.  Where x may differ (elements inside the band), the routing weights of that
token are allowed the change that difference can make: |dz_e| <= sum_j
max_e |W_router[e, j]| |dx_j|, and renormalised weights move by at most twice
the largest |dz| in relative terms.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from oracle.inputs import to_numpy, widen_tensor
from synth import make_attention_residual
from tests.gpu_harness import (TOL, check_layer, compare_tokens, logit_error_bound, make_case, normwise_err,
                               score_interval, spec_of, valid_selection, _order_consistent, WEIGHT_RTOL)
from top_routing_grouped_amd import moe

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
EPS = 1e-6

SMALL = {
    "small_f32": ("tiny_f32", dict(d_model=64, n_experts=32, top_k=4, d_ff=32, d_ff_shared=48)),
    "small_bf16": ("qwen_decode", dict(d_model=256, n_experts=32, top_k=4, d_ff=128, d_ff_shared=128)),
    "small_sigmoid": ("sigmoid_group", dict(d_model=256, n_experts=32, n_group=4, topk_group=2, top_k=4,
                                            d_ff=128, d_ff_shared=128)),
    "small_u4": ("qwen_u4", dict(d_model=256, n_experts=32, top_k=4, d_ff=128, d_ff_shared=128)),
}


def _spec(name, T, **kw):
    if name in SMALL:
        base, over = SMALL[name]
        return spec_of(base, n_tokens=T, **over, **kw)
    return spec_of(name, n_tokens=T, **kw)


def norm_error_bound(D: int) -> float:
    return 2.0 * ((D / 64 + 8) / 2 + 4) * U


def _special_rows(r: torch.Tensor, huge: bool):
    """Row 0 zero, row 1 dominated by eps, row 2 (norm-only tests) of very large magnitude."""
    T = r.shape[0]
    if T >= 2:
        r[0] = 0.0
        r[1] *= 1e-7
    if huge and T >= 3:
        r[2] *= 1e10
    return r


def check_normed_x(x_gpu: torch.Tensor, r64: np.ndarray, w64, eps: float, act: str) -> np.ndarray:
    """Checks x against the oracle; returns |dx| bounds per element (0 where x
    is fixed exactly)."""
    exact = O.rms_norm(r64, w64, eps)
    rel = norm_error_bound(r64.shape[1])
    if act == "f32":
        got = to_numpy(x_gpu).astype(np.float64)
        tol = (rel + U) * np.abs(exact)
        bad = np.abs(got - exact) > tol
        assert not bad.any(), f"{bad.sum()} fp32 elements outside the bound, first {np.argwhere(bad)[:3]}"
        return 2 * tol
    want = O.round_bf16(exact)
    bits = to_numpy(x_gpu)
    near = O.bf16_boundary_distance(exact) <= rel
    far_bad = (bits != O.bf16_bits(want)) & ~near
    assert not far_bad.any(), (f"{far_bad.sum()} bf16 elements differ away from a rounding boundary, first "
                               f"{np.argwhere(far_bad)[:3]}")
    got = O.bf16_bits_to_f64(bits)
    lo, hi = O.round_bf16(exact * (1 - rel)), O.round_bf16(exact * (1 + rel))
    near_bad = near & (got != lo) & (got != hi)
    assert not near_bad.any(), f"{near_bad.sum()} bf16 elements are neither neighbour of the boundary"
    return np.where(near, np.abs(hi - lo), 0.0)


def run_norm(spec, r: torch.Tensor, w, eps=EPS):
    cfg = moe.config_from_spec(spec)
    x = torch.full((spec.n_tokens, spec.d_model), float("nan"), device="cuda",
                   dtype=torch.float32 if spec.act_dtype == "f32" else torch.bfloat16)
    moe.rms_norm(cfg, r, w, eps, x)
    torch.cuda.synchronize()
    return x


# ------------------------------------------------------------------ x alone
NORM_CASES = [("qwen_decode", 1, {}), ("qwen_decode", 8, {}), ("qwen_prefill_skew", 4096, {}),
              ("small_bf16", 301, {}), ("small_f32", 37, {}), ("tiny_f32", 5, dict(d_model=2048)),
              ("qwen_decode", 3, dict(d_model=4224)), ("qwen_decode", 2, dict(d_model=8192)),
              ("qwen_decode", 67, dict(d_model=256))]


@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("name,T,kw", NORM_CASES)
def test_rms_norm_matches_oracle(name, T, kw, weighted):
    spec = _spec(name, T, **kw)
    r, w = make_attention_residual(spec, "cuda")
    r = _special_rows(r, huge=True)
    w = w if weighted else None
    x = run_norm(spec, r, w)
    delta = check_normed_x(x, widen_tensor(r), None if w is None else widen_tensor(w), EPS, spec.act_dtype)
    if spec.act_dtype == "bf16":
        print(f"{name} T={T} D={spec.d_model}: {int((delta > 0).sum())} of {delta.size} elements "
              f"within the rounding band")
    if T >= 2:
        assert torch.all(x[0] == 0)


def test_rms_norm_eps_and_scale():
    """eps enters inside the root: a constant row c gives c / sqrt(c^2 + eps)."""
    spec = spec_of("qwen_decode", n_tokens=4, d_model=512)
    r = torch.tensor([[2.0], [-0.5], [1e-3], [30.0]], device="cuda").expand(4, 512).contiguous()
    for eps in (1e-6, 0.25):
        x = run_norm(spec, r, None, eps).float().cpu().numpy()
        c = np.array([2.0, -0.5, 1e-3, 30.0], dtype=np.float32).astype(np.float64)
        want = O.round_bf16(c / np.sqrt(c * c + eps))
        np.testing.assert_array_equal(x, np.repeat(want[:, None], 512, axis=1))


# ------------------------------------------------------------------ the layer from the residual
def run_layer_norm(case, r, w, eps=EPS, x_out=True, aux=True, out_alias=False):
    s = case.spec
    cfg = moe.config_from_spec(s)
    ws = moe.alloc_workspace(cfg)
    ids = torch.empty((s.n_tokens, s.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((s.n_tokens, s.top_k), dtype=torch.float32, device="cuda")
    x = torch.empty((s.n_tokens, s.d_model), device="cuda",
                    dtype=torch.float32 if s.act_dtype == "f32" else torch.bfloat16) if x_out else None
    rr = r.clone()
    out = rr if out_alias else torch.empty_like(rr)
    stream = torch.cuda.Stream()
    aux_stream = torch.cuda.Stream() if aux else None
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        moe.layer_forward_norm(cfg, moe.weights_struct(case.w), w, eps, rr, out, x_out=x, ids_out=ids,
                               weights_out=wts, ws=ws, stream=stream, aux_stream=aux_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), wts.cpu().numpy(), x


LAYER_CASES = [("small_bf16", 1), ("small_bf16", 37), ("small_bf16", 301), ("small_f32", 37), ("small_f32", 700),
               ("small_u4", 37), ("small_sigmoid", 37), ("qwen_decode", 8), ("qwen_decode", 32),
               ("qwen_prefill_skew", 4096)]


def check_layer_from_residual(case, r, w, out, ids, wts, x, tag):
    """The layer entry's x, routing and output against the oracle run from
    residual r (see the module docstring for the rounding-band allowances)."""
    spec = case.spec
    T = spec.n_tokens
    name = tag
    r64, w64 = widen_tensor(r), widen_tensor(w)
    delta = check_normed_x(x, r64, w64, EPS, spec.act_dtype)
    x_or = O.normed_activation(r64, w64, EPS, spec.act_dtype)
    ocase = dataclasses.replace(case, x64=x_or, r64=r64)

    # routing: ids exact on tokens away from near-ties; weights within the
    # change that the x band can make
    toks = compare_tokens(ocase, ids)
    z = O.router_logits(x_or[toks], case.wr64)
    rt = O.route(z, spec.family, spec.top_k, case.bias64, spec.n_group, spec.topk_group, spec.routed_scaling)
    dz = delta[toks] @ np.abs(case.wr64).max(axis=0)
    wtol = WEIGHT_RTOL + 2.0 * dz * (1 + 1e-3)
    g_ids, g_wts = ids[toks], wts[toks]
    differ = (g_ids != rt.ids).any(axis=1)
    strict = ~rt.flags & (dz == 0)
    # away from near-ties and x bands: the set exact, the slot order one that
    # fp32 logit error can give
    dzb = logit_error_bound(spec, x_or[toks], case.wr64)
    for i in np.flatnonzero(differ & strict):
        assert sorted(g_ids[i]) == sorted(rt.ids[i]), f"token {toks[i]}: {g_ids[i]} vs {rt.ids[i]}, no near-tie"
        lo, hi = score_interval(spec, z[i], dzb[i], case.bias64)
        assert _order_consistent(lo, hi, g_ids[i]), f"token {toks[i]}: slot order {g_ids[i]} vs {rt.ids[i]}"
    for i in np.flatnonzero(differ & ~strict):
        # a score moves by at most p * (e^(2 dz) - 1) (softmax) or dz / 4 per
        # sigmoid, twice that for a group score
        widen = 2.1 * dz[i] * rt.score[i].max() if spec.family == "softmax" else 0.5 * dz[i]
        assert valid_selection(spec, z[i], case.bias64, g_ids[i], eps=O.TIE_EPS + widen), \
            f"token {toks[i]}: invalid selection {g_ids[i]}"
    same = ~differ
    rel = np.abs(g_wts - rt.weights) / np.abs(rt.weights)
    assert np.all(rel[same].max(axis=1, initial=0) <= wtol[same]), f"weights rel err {rel[same].max():.3e}"
    err = check_layer(ocase, out, ids, tokens=toks)
    print(f"{name} T={T}: y_moe normwise error {err:.2e} (gate {TOL[spec.expert_dtype]}) over {toks.size} tokens; "
          f"{int((dz > 0).sum())} with x inside a rounding band, {int((differ & strict).sum())} order-relaxed")
    return err


@pytest.mark.parametrize("name,T", LAYER_CASES)
def test_layer_forward_norm_matches_oracle(name, T):
    spec = _spec(name, T)
    case = make_case(spec)
    r, w = make_attention_residual(spec, "cuda")
    r = _special_rows(r, huge=False)
    out, ids, wts, x = run_layer_norm(case, r, w)
    check_layer_from_residual(case, r, w, out, ids, wts, x, name)
    if T >= 2:  # the zero row: x = 0, every projection 0, out = residual + y(0) = 0
        assert np.all(out[0] == 0.0)


@pytest.mark.parametrize("name,T", [("small_bf16", 37), ("small_u4", 8), ("small_sigmoid", 301),
                                    ("qwen_decode", 8)])
def test_chained_layers_match_oracle_layer_by_layer(name, T):
    """Three layers chained as a decoder stack runs them: one workspace, the
    output written over the residual it was computed from, each layer with its
    own RMS-norm weight.  Each layer is checked against the oracle run from
    the residual the GPU fed it (the previous layer's GPU output)."""
    spec = _spec(name, T)
    case = make_case(spec)
    cfg = moe.config_from_spec(spec)
    ws = moe.alloc_workspace(cfg)
    wstruct = moe.weights_struct(case.w)
    res, _ = make_attention_residual(spec, "cuda")
    ids = torch.empty((T, spec.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, spec.top_k), dtype=torch.float32, device="cuda")
    x = torch.empty((T, spec.d_model), device="cuda",
                    dtype=torch.float32 if spec.act_dtype == "f32" else torch.bfloat16)
    stream, aux = torch.cuda.Stream(), torch.cuda.Stream()
    for layer in range(3):
        _, nw = make_attention_residual(spec, "cuda", weight_seed=4242 + layer)
        r_in = res.clone()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            moe.layer_forward_norm(cfg, wstruct, nw, EPS, res, res, x_out=x, ids_out=ids, weights_out=wts,
                                   ws=ws, stream=stream, aux_stream=aux)
        torch.cuda.synchronize()
        check_layer_from_residual(case, r_in, nw, res.cpu().numpy(), ids.cpu().numpy(), wts.cpu().numpy(), x,
                                  f"{name} layer {layer}")


@pytest.mark.parametrize("name,T", [("qwen_decode", 1), ("qwen_decode", 8), ("qwen_decode", 32), ("small_bf16", 37),
                                    ("small_u4", 37), ("small_sigmoid", 37), ("small_bf16", 301), ("small_f32", 700),
                                    ("small_f32", 37), ("qwen_prefill_skew", 4096)])
def test_layer_forward_norm_is_norm_then_layer(name, T):
    """Bitwise: the entry equals moe_rms_norm followed by moe_layer_forward, with
    x in the caller's buffer or in the workspace, out aliasing the residual or
    not, with or without the second stream.  Small T with bf16 activations
    folds the normalisation into the router launch (x converted on the fly and
    written there); the others run the RMS-norm launch first."""
    spec = _spec(name, T)
    case = make_case(spec)
    r, w = make_attention_residual(spec, "cuda")
    a_out, a_ids, a_wts, a_x = run_layer_norm(case, r, w)
    x = run_norm(spec, r, w)
    cfg = moe.config_from_spec(spec)
    ws = moe.alloc_workspace(cfg)
    out = torch.empty_like(r)
    ids = torch.empty((T, spec.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, spec.top_k), dtype=torch.float32, device="cuda")
    moe.layer_forward(cfg, moe.weights_struct(case.w), x, r, out, ids, wts, ws)
    torch.cuda.synchronize()
    assert torch.equal(a_x.view(torch.int16) if a_x.dtype == torch.bfloat16 else a_x.view(torch.int32),
                       x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32))
    for u, v in [(a_out, out.cpu().numpy()), (a_ids, ids.cpu().numpy()), (a_wts, wts.cpu().numpy())]:
        assert np.array_equal(u.view(np.uint32) if u.dtype == np.float32 else u,
                              v.view(np.uint32) if v.dtype == np.float32 else v)
    for kw in (dict(x_out=False), dict(out_alias=True), dict(aux=False)):
        b = run_layer_norm(case, r, w, **kw)
        for u, v in zip((a_out, a_ids, a_wts), b[:3]):
            assert np.array_equal(u.view(np.uint32) if u.dtype == np.float32 else u,
                                  v.view(np.uint32) if v.dtype == np.float32 else v), kw


def test_layer_forward_norm_without_weight_matches_oracle():
    """norm_weight NULL means ones."""
    spec = _spec("qwen_decode", 8)
    case = make_case(spec)
    r, _ = make_attention_residual(spec, "cuda")
    out, ids, wts, x = run_layer_norm(case, r, None)
    r64 = widen_tensor(r)
    check_normed_x(x, r64, None, EPS, "bf16")
    ocase = dataclasses.replace(case, x64=O.normed_activation(r64, None, EPS, "bf16"), r64=r64)
    err = check_layer(ocase, out, ids)
    assert err <= TOL["bf16"]
    assert normwise_err(out.astype(np.float64), ocase.oracle_layer(ids=ids).out) <= TOL["bf16"]
