"""Helpers for the GPU parity tests: run the HIP library through its C ABI
and compare with the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import dataclasses
import itertools
from typing import Optional

import numpy as np
import torch

from oracle import moe_oracle as O
from oracle.inputs import banks_from, widen_tensor
from synth import WORKLOADS, LayerSpec, make_tokens, make_weights
from top_routing_grouped_amd import moe

TOL = {"f32": 1e-4, "bf16": 2e-2, "u4": 2e-2}  # normwise per-token relative error gate on y_moe
WEIGHT_RTOL = 1e-5


def spec_of(name: str, **kw) -> LayerSpec:
    return dataclasses.replace(WORKLOADS[name], **kw)


@dataclasses.dataclass
class Case:
    spec: LayerSpec
    w: object  # synth LayerWeights on the GPU
    x: torch.Tensor
    r: torch.Tensor
    # oracle-side fp64 views
    x64: np.ndarray
    r64: np.ndarray
    wr64: np.ndarray
    bias64: Optional[np.ndarray]
    banks: O.Banks

    def oracle_route(self, tokens=None):
        xs = self.x64 if tokens is None else self.x64[tokens]
        z = O.router_logits(xs, self.wr64)
        s = self.spec
        return z, O.route(z, s.family, s.top_k, self.bias64, s.n_group, s.topk_group, s.routed_scaling)

    def oracle_layer(self, tokens=None, ids=None):
        s = self.spec
        return O.layer_forward(self.x64, self.r64, self.wr64, self.banks, s.family, s.top_k, self.bias64,
                               s.n_group, s.topk_group, s.routed_scaling, tokens=tokens, ids=ids)


_WEIGHT_CACHE = {}


def make_case(spec: LayerSpec, device="cuda", token_seed=None, cache_key=None) -> Case:
    key = cache_key or (spec.name, spec.d_model, spec.n_experts, spec.d_ff, spec.d_ff_shared, spec.expert_dtype,
                        spec.top_k, spec.skew_var)
    if key not in _WEIGHT_CACHE:
        _WEIGHT_CACHE.clear()  # keep one layer's weights resident at a time
        _WEIGHT_CACHE[key] = make_weights(spec, device)
    w = _WEIGHT_CACHE[key]
    x, r = make_tokens(spec, device, seed=token_seed)
    lazy = spec.n_experts * spec.d_ff * spec.d_model > (1 << 24)
    return Case(spec, w, x, r, widen_tensor(x), widen_tensor(r), widen_tensor(w.router),
                None if w.expert_bias is None else widen_tensor(w.expert_bias), banks_from(w, lazy=lazy))


def normwise_err(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(got - ref).max(axis=1) / den).max())


def run_route(case: Case):
    s = case.spec
    cfg = moe.config_from_spec(s)
    ws = moe.alloc_workspace(cfg)
    ids = torch.full((s.n_tokens, s.top_k), -7, dtype=torch.int32, device="cuda")
    wts = torch.full((s.n_tokens, s.top_k), -7.0, dtype=torch.float32, device="cuda")
    moe.route(cfg, case.x, case.w.router, case.w.expert_bias, ids, wts, ws)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), wts.cpu().numpy()


def _valid_topk(score, chosen, k, cand=None, eps=O.TIE_EPS, ordered=False):
    """chosen is a valid top-k of score (restricted to cand) up to eps; with
    ordered, also in descending score order up to eps (the slot order)."""
    idx = np.arange(score.size) if cand is None else np.asarray(cand)
    if not set(chosen) <= set(idx.tolist()) or len(set(chosen)) != k:
        return False
    srt = np.sort(score[idx])[::-1]
    kth = srt[k - 1]
    nxt = srt[k] if k < idx.size else -np.inf
    rest = [e for e in idx if e not in set(chosen)]
    if ordered and any(score[a] < score[b] - eps for a, b in zip(chosen[:-1], chosen[1:])):
        return False
    return all(score[e] >= kth - eps for e in chosen) and all(score[e] <= nxt + eps for e in rest)


def valid_selection(spec: LayerSpec, z_row: np.ndarray, bias, chosen, eps: float = O.TIE_EPS) -> bool:
    """Whether a selection (in slot order) is one of the near-tied valid
    answers (scores within eps) for a flagged token."""
    if spec.family == "softmax":
        return _valid_topk(O.softmax(z_row[None])[0], list(chosen), spec.top_k, eps=eps, ordered=True)
    E, G, TG = spec.n_experts, spec.n_group, spec.topk_group
    gs = E // G
    sel = O.sigmoid(z_row) + (0 if bias is None else bias)
    gsc = O.group_scores(sel[None], G)[0]
    for S in itertools.combinations(range(G), TG):
        if not _valid_topk(gsc, list(S), TG, eps=eps):
            continue
        cand = [e for g in S for e in range(g * gs, (g + 1) * gs)]
        if _valid_topk(sel, list(chosen), spec.top_k, cand, eps=eps, ordered=True):
            return True
    return False


U32 = 2.0 ** -24  # fp32 unit roundoff


def logit_error_bound(spec: LayerSpec, x64: np.ndarray, wr64: np.ndarray) -> np.ndarray:
    """[n, E] bound on |z_gpu - z| for the GPU's fp32 router logits.

    A logit is a sum of D products, exact for bf16 operands (8-bit
    significands, a 16-bit product fits fp32's 24) and rounded once each for
    fp32 operands.  The bf16 kernels sum them as MFMA dot products of 32
    products (counted as up to 32 roundings, however the unit adds them),
    accumulated over at most D/32 steps within a K-split plane, and up to 8
    planes added at the end: a chain of at most d = D/32 + 40 roundings.  An
    fp32 router may sum in any order: d = D.  Each rounding is charged 2u of
    the running sum's magnitude (u = 2^-24; twice round-to-nearest's bound,
    for an accumulator that might not round to nearest), so
    |dz_e| <= 2 d u sum_j |W_ej x_j|."""
    D = spec.d_model
    d = D if spec.router_dtype == "f32" else min(D, D // 32 + 40)
    return 2.0 * d * U32 * (np.abs(x64) @ np.abs(wr64).T)


def _order_consistent(lo: np.ndarray, hi: np.ndarray, order) -> bool:
    """Whether the slots `order` are in descending order of some scores
    within [lo, hi] (for interval scores: hi of every earlier slot >= lo of
    every later one)."""
    best_hi = np.inf  # smallest hi among the earlier slots
    for e in order:
        if lo[e] > best_hi:
            return False
        best_hi = min(best_hi, hi[e])
    return True


def score_interval(spec: LayerSpec, z_row: np.ndarray, dz_row: np.ndarray, bias):
    """Range of the selection score each expert can take with its logit off
    by at most dz: the logit itself for the softmax family (softmax is
    increasing, and the GPU ranks logits), sigmoid(z) + bias for the group
    family (plus 4 ulps of the fp32 sigmoid and the bias addition)."""
    if spec.family == "softmax":
        return z_row - dz_row, z_row + dz_row
    b = 0.0 if bias is None else bias
    lo = O.sigmoid(z_row - dz_row) + b
    hi = O.sigmoid(z_row + dz_row) + b
    slack = 4 * U32 * (np.abs(lo) + np.abs(hi))
    return lo - slack, hi + slack


def check_route(case: Case, ids, wts, z, rt, x64=None):
    """Routing against the oracle.

    * Tokens not flagged (their k-th/(k+1)-th score gap, and the group family's
      kept/dropped group-score gap, is at least 1e-4): the selected set is
      bit-exact.  The slot order (descending score) is bit-exact too, except
      where the GPU's order is one that fp32 logits within
      logit_error_bound of the exact ones could give; those tokens are counted
      and reported as order-relaxed.
    * Flagged tokens: a valid top-K under a 1e-4 score perturbation, in
      descending order within it.
    * Weights within 1e-5 relative on every unflagged token.
    Returns (flagged, order_relaxed) token counts."""
    s = case.spec
    x64 = case.x64 if x64 is None else x64
    fixed = ~rt.flags
    differ = (ids != rt.ids).any(axis=1)
    sets_differ = np.flatnonzero(fixed & (np.sort(ids, axis=1) != np.sort(rt.ids, axis=1)).any(axis=1))
    assert sets_differ.size == 0, (f"{sets_differ.size} unflagged tokens select another set, first "
                                   f"{sets_differ[:5]}: {ids[sets_differ[:2]]} vs {rt.ids[sets_differ[:2]]}")
    relaxed = np.flatnonzero(fixed & differ)
    if relaxed.size:
        dz = logit_error_bound(s, x64[relaxed], case.wr64)
        for i, t in enumerate(relaxed):
            lo, hi = score_interval(s, z[t], dz[i], case.bias64)
            assert _order_consistent(lo, hi, ids[t]), (
                f"token {t}: slot order {ids[t]} against {rt.ids[t]} is not explained by fp32 logit error "
                f"(bound {dz[i][ids[t]].max():.2e})")
    for t in np.flatnonzero(rt.flags & differ):
        assert valid_selection(s, z[t], case.bias64, ids[t]), f"token {t}: invalid near-tie selection {ids[t]}"
    # the oracle's weights in the GPU's slot order (same set on every token compared)
    set_fixed = np.flatnonzero(fixed)
    want = np.empty((set_fixed.size, ids.shape[1]))
    for i, t in enumerate(set_fixed):
        pos = {int(e): j for j, e in enumerate(rt.ids[t])}
        want[i] = rt.weights[t, [pos[int(e)] for e in ids[t]]]
    rel = np.abs(wts[set_fixed] - want) / np.abs(want)
    assert rel.size == 0 or rel.max() <= WEIGHT_RTOL, f"weights rel err {rel.max():.3e}"
    n_flag, n_relax = int(rt.flags.sum()), int(relaxed.size)
    print(f"routing: {ids.shape[0]} tokens, {n_flag} flagged near-ties, {n_relax} order-relaxed "
          f"(slot order within the fp32 logit bound), {int((rt.flags & differ).sum())} flagged with other ids")
    return n_flag, n_relax


FULL_COMPARE_FLOPS = 4e11  # oracle expert work compared on every token (seconds in fp64)


def compare_tokens(case: Case, ids: np.ndarray, tile: int = 128, n_random: int = 48, seed: int = 0) -> np.ndarray:
    """Tokens whose layer (or expert) output is compared with the oracle.
    Every token when the oracle's expert work (6 T K D F flops) is at most
    FULL_COMPARE_FLOPS.  Beyond that: the first and the last pair of every
    `tile`-pair token tile of every active expert, in the permuted order of
    `ids` (so every GEMM work item, and each expert's last, partial tile, has
    compared rows), plus the first and last token and n_random random ones."""
    s = case.spec
    T = s.n_tokens
    if 6.0 * T * s.top_k * s.d_model * s.d_ff <= FULL_COMPARE_FLOPS:
        return np.arange(T)
    perm = O.permute(ids, s.n_experts)
    picks = []
    for e in perm.active:
        a, b = int(perm.offsets[e]), int(perm.offsets[e + 1])
        starts = np.arange(a, b, tile)
        picks += [perm.sorted_pairs[starts], perm.sorted_pairs[np.minimum(starts + tile, b) - 1]]
    rng = np.random.default_rng(seed)
    extra = np.concatenate([[0, T - 1], rng.choice(T, min(n_random, T), replace=False)])
    return np.unique(np.concatenate(picks + [extra * s.top_k]) // s.top_k)


def run_layer(case: Case, aux: bool = True, out_alias: bool = False):
    s = case.spec
    cfg = moe.config_from_spec(s)
    ws = moe.alloc_workspace(cfg)
    ids = torch.empty((s.n_tokens, s.top_k), dtype=torch.int32, device="cuda")
    wts = torch.empty((s.n_tokens, s.top_k), dtype=torch.float32, device="cuda")
    r = case.r.clone()
    out = r if out_alias else torch.empty_like(r)
    stream = torch.cuda.Stream()
    aux_stream = torch.cuda.Stream() if aux else None
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        moe.layer_forward(cfg, moe.weights_struct(case.w), case.x, r, out, ids, wts, ws, stream=stream,
                          aux_stream=aux_stream)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ids.cpu().numpy(), wts.cpu().numpy()


def check_layer(case: Case, out: np.ndarray, ids: np.ndarray, tokens=None):
    """Gate: per-token normwise error of y_moe = out - r against the oracle
    (re-run with the GPU's ids for tokens whose near-tied ids differ)."""
    s = case.spec
    toks = np.arange(s.n_tokens) if tokens is None else np.asarray(tokens)
    ref = case.oracle_layer(tokens=toks, ids=ids)
    y = out[toks].astype(np.float64) - case.r64[toks]
    err = normwise_err(y, ref.y_moe)
    err_out = normwise_err(out[toks].astype(np.float64), ref.out)
    tol = TOL[s.expert_dtype]
    assert err <= tol, f"y_moe normwise error {err:.3e} > {tol}"
    assert err_out <= tol
    return err
