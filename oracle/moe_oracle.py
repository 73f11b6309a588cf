"""Plain fp64 CPU oracle for one sparse mixture-of-experts layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library (no kernels,
headers, helpers, tables or constant generators) and imports nothing from it.

Every step is the plain definition written out in float64 with NumPy; inputs
(float32, bf16 bit patterns, 4-bit affine codes) are first widened exactly.

Sources (page titles and sections; the pages print no code we follow):
  [T]  Treebeard, "How Treebeard routes Qwen3.6 MoE tokens":
       "Routing math" (router logits, softmax, top-k, renormalisation with
       the 2^-14 clamp, equivalence with a softmax over the selected logits),
       "Routed expert computation" (SwiGLU expert and weighted routed sum),
       "Shared expert computation" (sigmoid-gated shared expert, branch sum
       and residual add), "Treebeard's execution optimization" / "Intel SYCL
       path" (count pairs per expert, offsets and active-expert list, pack
       (token, slot) pairs, write back to the original token and slot).
  [E]  edge0, "MoE Routing and Experts": "Experts" (expert formula),
       "Routing families" (softmax top-k; sigmoid group top-k with
       expert_bias, n_group, topk_group, routed_scaling), tier table
       ("4-bit affine, group 64").

Readings where the pages are silent:
  * selection ties go to the lowest expert index (groups: lowest group
    index); slots are ordered by descending score;
  * the sigmoid family uses the same max(sum, 2^-14) guard as the softmax
    family, applied before the routed_scaling multiply;
  * groups are contiguous blocks of E / n_group experts;
  * SiLU(v) = v * sigmoid(v);
  * a missing shared gate vector means s_t = 1;
  * 4-bit affine group 64: w = scale * q + min, q in [0, 15], groups of 64
    consecutive input elements, two codes per byte with the even element in
    the low nibble, scale and min in bf16;
  * the permuted pair order is stable (ascending flat pair id t*K + k inside
    each expert);
  * RMS normalisation of the attention residual ([T] "Routing math": x is the
    post-attention RMS-normalised hidden state; "Editable Mermaid flowchart"
    and "Pseudocode": x = rms_norm(attention residual)) is
    x = r / sqrt(mean_j r_j^2 + eps) * w, with eps inside the square root, an
    optional per-feature weight w (absent: ones) applied after the division,
    and x stored once in the activation type (bf16: round to nearest even from
    the exact value) that every consumer of x reads.

Pins: every function here is pinned by tests/test_oracle_pins.py against
closed forms, hand-derived fixtures (tests/golden/), brute force on tiny
inputs, invariants the pages state, and library routines for the special
cases that reduce to them.  That includes the weights of given selections
(softmax_weights_for, sigmoid_weights_for) and the layer run on given ids in
both routing families (hand-derived values in tests/golden/), and the lazy,
per-expert widening of the banks in oracle/inputs.py (equal to the eager
widening).  The numeric value of a full layer at model shape has no printed
worked example on the pages; it rests on those pins.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

CLAMP = 2.0 ** -14  # smallest normal fp16, the renormalisation floor ([T] "Routing math")
# Near-tie threshold.  A token is flagged when the gap at the selection
# boundary (k-th against (k+1)-th score, and for the group family the
# kept/dropped group scores) is below it: the selected set itself is then not
# fixed at fp32 precision of the logits.
TIE_EPS = 1e-4


# ---------------------------------------------------------------- widening
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16/int16) -> float64, exactly."""
    b = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def dequant_u4_g64(codes: np.ndarray, scale_bits: np.ndarray, min_bits: np.ndarray) -> np.ndarray:
    """4-bit affine, group 64 ([E] tier table): w = scale * q + min in fp64.

    codes [..., rows, n_in/2] uint8, even input element in the low nibble;
    scale_bits/min_bits [..., rows, n_in/64] bf16 bit patterns."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = (codes & 0x0F).astype(np.float64)
    hi = (codes >> 4).astype(np.float64)
    q = np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    n_in = q.shape[-1]
    scale = bf16_bits_to_f64(scale_bits)
    mn = bf16_bits_to_f64(min_bits)
    qg = q.reshape(*q.shape[:-1], n_in // 64, 64)
    w = qg * scale[..., None] + mn[..., None]
    return w.reshape(q.shape)


def widen(arr, dtype: str) -> np.ndarray:
    """'f32' arrays or 'bf16' bit patterns -> float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(arr, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- RMS normalisation
def rms_norm(r: np.ndarray, weight: Optional[np.ndarray] = None, eps: float = 1e-6) -> np.ndarray:
    """x_t = r_t / sqrt(mean_j r_t[j]^2 + eps), times weight if given ([T]
    "Routing math": x_t is the RMS-normalised post-attention state;
    "Pseudocode": x = rms_norm(attention residual)).  Rows are the last axis."""
    r = np.asarray(r, dtype=np.float64)
    ms = np.mean(r * r, axis=-1, keepdims=True)
    x = r / np.sqrt(ms + eps)
    if weight is not None:
        x = x * np.asarray(weight, dtype=np.float64)
    return x


def _bf16_quantum(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values (8 significant bits, fp32's exponent range) at
    the binade of v: 2^(E-7) for |v| in [2^E, 2^(E+1)), E >= -126; 2^-133 below."""
    _, e = np.frexp(v)  # v = m 2^e, 0.5 <= |m| < 1, so E = e - 1
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def round_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even, directly
    from the exact value (no intermediate fp32 rounding).  Returns float64
    holding bf16 values; magnitudes past the largest bf16 become inf."""
    v = np.asarray(v, dtype=np.float64)
    q = _bf16_quantum(v)
    out = np.rint(v / q) * q  # v / q is exact (power-of-two scale); rint ties to even
    big = np.abs(out) >= 2.0 ** 128
    return np.where(big, np.copysign(np.inf, v), out)


def bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of float64 values that are bf16 values."""
    v = np.asarray(v, dtype=np.float64)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v, equal_nan=True), "not bf16 values"
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_boundary_distance(v: np.ndarray) -> np.ndarray:
    """Relative distance |v - m| / |v| from v to the nearest bf16 rounding
    boundary m (a midpoint between adjacent bf16 values); inf for v = 0."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    q = _bf16_quantum(a)
    n = np.floor(a / q)
    d = np.abs(a - (n + 0.5) * q)  # the midpoint of the step holding a
    # in the first step of a binade the boundary below is a quarter step down
    # (the spacing below is half as large)
    _, e = np.frexp(a)
    binade_start = (n * q == np.ldexp(1.0, e - 1)) & (e - 1 > -126)
    d = np.where(binade_start, np.minimum(d, a - (n * q - 0.25 * q)), d)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(a == 0, np.inf, d / a)


def normed_activation(r: np.ndarray, weight: Optional[np.ndarray], eps: float, act_dtype: str) -> np.ndarray:
    """x as the layer stores it: rms_norm rounded once to the activation type
    ('bf16': round_bf16; 'f32': nearest fp32)."""
    x = rms_norm(r, weight, eps)
    if act_dtype == "bf16":
        return round_bf16(x)
    if act_dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    raise ValueError(act_dtype)


# ---------------------------------------------------------------- routing
def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """z_t = W_router^T x_t ([T] "Routing math"); W_router stored [E, D], so z = x @ W.T."""
    return x @ w_router.T


def sigmoid(v: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-v))


def silu(v: np.ndarray) -> np.ndarray:
    """SiLU(v) = v * sigmoid(v)."""
    return v * sigmoid(v)


def softmax(z: np.ndarray) -> np.ndarray:
    """Full softmax over the last axis ([T] "Routing math"; [E] step 1 of softmax top-k)."""
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=-1, keepdims=True)


def _rank_desc(score: np.ndarray) -> np.ndarray:
    """Indices of a 1-D score in descending order, ties -> lower index."""
    return np.argsort(-score, kind="stable")


@dataclasses.dataclass
class Route:
    ids: np.ndarray  # [T, K] int32, slots by descending selection score
    weights: np.ndarray  # [T, K] float64 routing weights alpha
    flags: np.ndarray  # [T] bool near-tie at the selection boundary
    score: np.ndarray  # [T, E] float64 selection score (p, or sigmoid + bias)


def softmax_topk(z: np.ndarray, k: int) -> Route:
    """Softmax top-k with renormalisation and the 2^-14 clamp ([T] "Routing
    math"; [E] "Softmax top-k"): p = softmax(z); I = TopK(p, k);
    alpha_i = p_i / max(sum_{j in I} p_j, 2^-14)."""
    T, E = z.shape
    p = softmax(z)
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    flags = np.zeros(T, dtype=bool)
    for t in range(T):
        order = _rank_desc(p[t])
        sel = order[:k]
        ids[t] = sel
        denom = max(p[t, sel].sum(), CLAMP)
        w[t] = p[t, sel] / denom
        if k < E:
            flags[t] = (p[t, order[k - 1]] - p[t, order[k]]) < TIE_EPS
    return Route(ids, w, flags, p)


def softmax_weights_for(z: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Renormalised softmax weights of given (possibly non-oracle) selections."""
    p = softmax(z)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    return sel / np.maximum(sel.sum(axis=1, keepdims=True), CLAMP)


def group_scores(sel: np.ndarray, n_group: int) -> np.ndarray:
    """Per group of E/n_group contiguous experts: sum of its two largest
    selection scores ([E] "Sigmoid group top-k", step 3)."""
    T, E = sel.shape
    g = sel.reshape(T, n_group, E // n_group)
    top2 = -np.sort(-g, axis=-1)[..., :2]
    return top2.sum(axis=-1)


def sigmoid_group_topk(z: np.ndarray, bias: Optional[np.ndarray], k: int, n_group: int,
                       topk_group: int, routed_scaling: float) -> Route:
    """DeepSeek-V3 style sigmoid group top-k ([E] "Sigmoid group top-k"):
    s = sigmoid(z); sel = s + bias; keep the topk_group groups with the largest
    sum of their two best sel; top-k of sel inside kept groups;
    alpha = routed_scaling * s_I / max(sum s_I, 2^-14) (bias excluded)."""
    T, E = z.shape
    if E % n_group or E // n_group < 2:
        raise ValueError("E must split into n_group groups of >= 2 experts")
    gsize = E // n_group
    s = sigmoid(z)
    b = np.zeros(E) if bias is None else np.asarray(bias, dtype=np.float64)
    sel = s + b[None, :]
    gsc = group_scores(sel, n_group)
    ids = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    flags = np.zeros(T, dtype=bool)
    for t in range(T):
        gorder = _rank_desc(gsc[t])
        kept = np.sort(gorder[:topk_group])
        cand = np.concatenate([np.arange(g * gsize, (g + 1) * gsize) for g in kept])
        corder = cand[_rank_desc(sel[t, cand])]
        chosen = corder[:k]
        ids[t] = chosen
        denom = max(s[t, chosen].sum(), CLAMP)
        w[t] = routed_scaling * s[t, chosen] / denom
        f = False
        if topk_group < n_group:
            f |= (gsc[t, gorder[topk_group - 1]] - gsc[t, gorder[topk_group]]) < TIE_EPS
        if k < len(cand):
            f |= (sel[t, corder[k - 1]] - sel[t, corder[k]]) < TIE_EPS
        flags[t] = f
    return Route(ids, w, flags, sel)


def sigmoid_weights_for(z: np.ndarray, ids: np.ndarray, routed_scaling: float) -> np.ndarray:
    """Weights of given (possibly non-oracle) selections in the sigmoid group
    family ([E] "Sigmoid group top-k", steps 4-5): the raw sigmoid scores of
    the selected experts (bias excluded), renormalised with the 2^-14 floor,
    times routed_scaling."""
    s = np.take_along_axis(sigmoid(z), ids.astype(np.int64), axis=1)
    return routed_scaling * s / np.maximum(s.sum(axis=1, keepdims=True), CLAMP)


# ---------------------------------------------------------------- permute
@dataclasses.dataclass
class Permutation:
    offsets: np.ndarray  # [E+1] int32
    active: np.ndarray  # [n_active] int32, ascending expert ids with count > 0
    n_active: int
    sorted_pairs: np.ndarray  # [T*K] int32 flat pair ids t*K + k


def permute(ids: np.ndarray, n_experts: int) -> Permutation:
    """Counting pass of the grouped path ([T] "Intel SYCL path", steps 1-3):
    count pairs per expert, prefix-sum into offsets, list the active experts,
    pack the flat (token, slot) pair ids under their expert (stable)."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    active = np.flatnonzero(counts).astype(np.int32)
    order = np.argsort(flat, kind="stable").astype(np.int32)
    return Permutation(offsets, active, int(active.size), order)


# ---------------------------------------------------------------- experts
def swiglu(x: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """expert(x) = down(SiLU(gate(x)) * up(x)) ([T] "Routed expert computation";
    [E] "Experts").  x [n, D]; w_gate, w_up [F, D]; w_down [D, F] -> [n, D]."""
    g = x @ w_gate.T
    u = x @ w_up.T
    h = silu(g) * u
    return h @ w_down.T


@dataclasses.dataclass
class Banks:
    """fp64 views of the weights.  Banks may be given lazily via callables
    returning [F, D] / [D, F] slices for one expert (to avoid widening all)."""
    gate: object
    up: object
    down: object
    shared_gate: Optional[np.ndarray] = None
    shared_up: Optional[np.ndarray] = None
    shared_down: Optional[np.ndarray] = None
    shared_gate_vec: Optional[np.ndarray] = None

    def expert(self, e: int):
        def pick(bank):
            return bank(e) if callable(bank) else bank[e]
        return pick(self.gate), pick(self.up), pick(self.down)


def routed_slots(x: np.ndarray, ids: np.ndarray, alpha: np.ndarray, banks: Banks,
                 tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """alpha_{t,k} * e_{I_{t,k}}(x_t) for every (token, slot) -> [n, K, D].
    Grouped by expert: each selected expert's rows of x are gathered and run
    through one matmul chain, then written back to their (token, slot)."""
    if tokens is None:
        tokens = np.arange(x.shape[0])
    ids_s = ids[tokens]
    n, K = ids_s.shape
    out = np.zeros((n, K, x.shape[1]), dtype=np.float64)
    flat = ids_s.ravel()
    for e in np.unique(flat):
        pairs = np.flatnonzero(flat == e)
        rows, slots = pairs // K, pairs % K
        wg, wu, wd = banks.expert(int(e))
        o = swiglu(x[tokens[rows]], wg, wu, wd)
        out[rows, slots] = alpha[tokens[rows], slots][:, None] * o
    return out


def shared_expert(x: np.ndarray, banks: Banks) -> np.ndarray:
    """y_shared = s_t * W_down_sh^T(SiLU(W_gate_sh^T x) * W_up_sh^T x),
    s_t = sigmoid(w_shared^T x) ([T] "Shared expert computation"); s_t = 1
    when there is no gate vector; zeros when there is no shared expert."""
    if banks.shared_gate is None:
        return np.zeros_like(x)
    e = swiglu(x, banks.shared_gate, banks.shared_up, banks.shared_down)
    if banks.shared_gate_vec is None:
        return e
    s = sigmoid(x @ banks.shared_gate_vec)
    return s[:, None] * e


def combine(residual: np.ndarray, slots: np.ndarray, y_shared: np.ndarray) -> np.ndarray:
    """r_next = r + (y_routed + y_shared), y_routed = sum over slots in
    ascending order ([T] "Shared expert computation", last block)."""
    y_routed = np.zeros(slots.shape[0:1] + slots.shape[2:], dtype=np.float64)
    for k in range(slots.shape[1]):
        y_routed = y_routed + slots[:, k]
    return residual + (y_routed + y_shared)


@dataclasses.dataclass
class LayerResult:
    out: np.ndarray  # [n, D]
    y_moe: np.ndarray  # [n, D] = y_routed + y_shared
    slots: np.ndarray  # [n, K, D]
    y_shared: np.ndarray  # [n, D]
    route: Route  # routing of the computed tokens
    z: np.ndarray  # [n, E] logits of the computed tokens
    tokens: np.ndarray


def route(z: np.ndarray, family: str, k: int, bias=None, n_group=1, topk_group=1,
          routed_scaling=1.0) -> Route:
    if family == "softmax":
        return softmax_topk(z, k)
    if family == "sigmoid_group":
        return sigmoid_group_topk(z, bias, k, n_group, topk_group, routed_scaling)
    raise ValueError(family)


def weights_for(z: np.ndarray, ids: np.ndarray, family: str, routed_scaling=1.0) -> np.ndarray:
    if family == "softmax":
        return softmax_weights_for(z, ids)
    return sigmoid_weights_for(z, ids, routed_scaling)


def layer_forward(x: np.ndarray, residual: np.ndarray, w_router: np.ndarray, banks: Banks,
                  family: str, k: int, bias=None, n_group=1, topk_group=1, routed_scaling=1.0,
                  tokens: Optional[np.ndarray] = None, ids: Optional[np.ndarray] = None) -> LayerResult:
    """One MoE layer forward ([T] "The short version", steps 1-8).

    x, residual, w_router and banks are float64.  `tokens` restricts the
    expert/combine work to a subset of rows (routing is per token, so the
    subset's result equals the full run's rows).  `ids` [T, K] (indexed like
    x) substitutes given selections; their weights are then recomputed from
    the oracle's own scores."""
    if tokens is None:
        tokens = np.arange(x.shape[0])
    tokens = np.asarray(tokens)
    z = router_logits(x[tokens], w_router)
    r = route(z, family, k, bias, n_group, topk_group, routed_scaling)
    if ids is not None:
        ids_t = np.asarray(ids)[tokens]
        r = Route(ids_t.astype(np.int32), weights_for(z, ids_t, family, routed_scaling), r.flags, r.score)
    local = np.arange(tokens.size)
    slots = routed_slots(x[tokens], r.ids, r.weights, banks, local)
    ys = shared_expert(x[tokens], banks)
    out = combine(residual[tokens], slots, ys)
    return LayerResult(out, out - residual[tokens], slots, ys, r, z, tokens)


def layer_forward_dense(x: np.ndarray, residual: np.ndarray, w_router: np.ndarray, banks: Banks,
                        family: str, k: int, bias=None, n_group=1, topk_group=1,
                        routed_scaling=1.0) -> np.ndarray:
    """The same layer as a dense mixture over all E experts: every expert runs
    on every token, and a [T, E] weight matrix that is zero off each token's
    selection contracts their outputs ([T] "Routing math": the routing weights
    of unselected experts are zero; "Routed expert computation": y_routed is
    the weighted sum of expert outputs; "Shared expert computation": the gated
    shared branch and the residual sum).  It shares neither the gathering by
    expert nor the (token, slot) write-back with layer_forward, and costs E/K
    times its expert work: for small inputs."""
    T, D = x.shape
    E = w_router.shape[0]
    z = x @ w_router.T
    rt = route(z, family, k, bias, n_group, topk_group, routed_scaling)
    A = np.zeros((T, E))
    for t in range(T):
        A[t, rt.ids[t]] = rt.weights[t]
    mats = [banks.expert(e) for e in range(E)]
    Wg = np.stack([m[0] for m in mats])  # [E, F, D]
    Wu = np.stack([m[1] for m in mats])
    Wd = np.stack([m[2] for m in mats])  # [E, D, F]
    G = np.einsum("td,efd->tef", x, Wg)
    U = np.einsum("td,efd->tef", x, Wu)
    H = G / (1.0 + np.exp(-G)) * U
    Y = np.einsum("tef,edf->ted", H, Wd)  # every expert's output for every token
    y_routed = np.einsum("te,ted->td", A, Y)
    y_shared = np.zeros((T, D))
    if banks.shared_gate is not None:
        gs = x @ banks.shared_gate.T
        us = x @ banks.shared_up.T
        y_shared = (gs / (1.0 + np.exp(-gs)) * us) @ banks.shared_down.T
        if banks.shared_gate_vec is not None:
            y_shared = y_shared / (1.0 + np.exp(-(x @ banks.shared_gate_vec)))[:, None]
    return residual + (y_routed + y_shared)
