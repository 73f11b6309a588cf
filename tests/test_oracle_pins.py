"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test ties an oracle function to something other than itself: values
derived by hand (tests/golden/), closed forms stated on the pages, brute force
over all subsets on tiny inputs, invariants, and special cases that reduce to
library routines (torch softmax / SiLU, NumPy sorting).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
LN = {"ln3": math.log(3.0), "ln2": math.log(2.0)}


def _ev(expr):
    """Evaluate a hand-derived fixture expression (numbers, + - * / ( ), ln2, ln3)."""
    if isinstance(expr, (int, float)):
        return float(expr)
    allowed = set("0123456789.+-*/() ")
    names = expr
    for k in LN:
        names = names.replace(k, "")
    assert set(names) <= allowed, expr
    return float(eval(expr, {"__builtins__": {}}, LN))  # noqa: S307 - restricted alphabet


def _arr(nested):
    return np.vectorize(_ev, otypes=[np.float64])(np.array(nested, dtype=object))


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_layer(rng, T, D, E, K, F, Fs, gated=True):
    x = rng.standard_normal((T, D))
    r = rng.standard_normal((T, D))
    wr = rng.standard_normal((E, D)) / math.sqrt(D)
    banks = O.Banks(rng.standard_normal((E, F, D)) / math.sqrt(D),
                    rng.standard_normal((E, F, D)) / math.sqrt(D),
                    rng.standard_normal((E, D, F)) / math.sqrt(F),
                    rng.standard_normal((Fs, D)) / math.sqrt(D) if Fs else None,
                    rng.standard_normal((Fs, D)) / math.sqrt(D) if Fs else None,
                    rng.standard_normal((D, Fs)) / math.sqrt(Fs) if Fs else None,
                    rng.standard_normal(D) / math.sqrt(D) if (Fs and gated) else None)
    return x, r, wr, banks


# ------------------------------------------------------------- golden fixtures
def test_golden_softmax_layer_by_hand():
    g = _load("softmax_layer_hand.json")
    x, r = _arr(g["x"]), _arr(g["residual"])
    banks = O.Banks(_arr(g["gate"]), _arr(g["up"]), _arr(g["down"]), _arr(g["shared_gate"]),
                    _arr(g["shared_up"]), _arr(g["shared_down"]), _arr(g["shared_gate_vec"]))
    res = O.layer_forward(x, r, _arr(g["router"]), banks, "softmax", g["shape"]["K"])
    np.testing.assert_array_equal(res.route.ids, np.array(g["expected_ids"]))
    np.testing.assert_allclose(res.route.weights, _arr(g["expected_weights"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(res.out, _arr(g["expected_out"]), rtol=0, atol=1e-12)
    # the dense-mixture formulation reproduces the same hand values
    dense = O.layer_forward_dense(x, r, _arr(g["router"]), banks, "softmax", g["shape"]["K"])
    np.testing.assert_allclose(dense, _arr(g["expected_out"]), rtol=0, atol=1e-12)


def test_golden_sigmoid_group_by_hand():
    g = _load("sigmoid_group_hand.json")
    sh = g["shape"]
    z = O.router_logits(_arr(g["x"]), _arr(g["router"]))
    rt = O.sigmoid_group_topk(z, _arr(g["expert_bias"]), sh["K"], sh["n_group"], sh["topk_group"],
                              sh["routed_scaling"])
    np.testing.assert_array_equal(rt.ids, np.array(g["expected_ids"]))
    np.testing.assert_allclose(rt.weights, _arr(g["expected_weights"]), rtol=0, atol=1e-14)
    # negative control: ranking groups by their single best score picks another group
    sel = O.sigmoid(z) + _arr(g["expert_bias"])[None]
    top1 = sel.reshape(2, sh["n_group"], -1).max(axis=-1)
    kept = int(np.argmax(top1[0]))
    members = np.arange(kept * 2, kept * 2 + 2)
    alt = members[np.argsort(-sel[0, members], kind="stable")][: sh["K"]]
    assert list(alt) == g["top1_group_rule_ids_token0"] != list(rt.ids[0])


def _sigmoid_layer_fixture():
    g = _load("sigmoid_group_layer_hand.json")
    sh = g["shape"]
    banks = O.Banks(_arr(g["gate"]), _arr(g["up"]), _arr(g["down"]), _arr(g["shared_gate"]), _arr(g["shared_up"]),
                    _arr(g["shared_down"]), None)
    args = dict(bias=_arr(g["expert_bias"]), n_group=sh["n_group"], topk_group=sh["topk_group"],
                routed_scaling=sh["routed_scaling"])
    return g, sh, banks, args


def test_golden_sigmoid_group_layer_by_hand():
    g, sh, banks, args = _sigmoid_layer_fixture()
    x, r, wr = _arr(g["x"]), _arr(g["residual"]), _arr(g["router"])
    res = O.layer_forward(x, r, wr, banks, "sigmoid_group", sh["K"], **args)
    np.testing.assert_array_equal(res.route.ids, np.array(g["expected_ids"]))
    np.testing.assert_allclose(res.route.weights, _arr(g["expected_weights"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(res.out, _arr(g["expected_out"]), rtol=0, atol=1e-12)
    dense = O.layer_forward_dense(x, r, wr, banks, "sigmoid_group", sh["K"], **args)
    np.testing.assert_allclose(dense, _arr(g["expected_out"]), rtol=0, atol=1e-12)


def test_golden_sigmoid_group_layer_given_ids_by_hand():
    """The layer on given selections (one token's set is not the rule's
    choice, the other's slots are swapped): weights from the raw sigmoid
    scores of the given set times routed_scaling, outputs by hand."""
    g, sh, banks, args = _sigmoid_layer_fixture()
    x, r, wr = _arr(g["x"]), _arr(g["residual"]), _arr(g["router"])
    given = np.array(g["given_ids"])
    res = O.layer_forward(x, r, wr, banks, "sigmoid_group", sh["K"], ids=given, **args)
    np.testing.assert_array_equal(res.route.ids, given)
    np.testing.assert_allclose(res.route.weights, _arr(g["given_weights"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(res.out, _arr(g["given_out"]), rtol=0, atol=1e-12)
    z = O.router_logits(x, wr)
    np.testing.assert_allclose(O.sigmoid_weights_for(z, given, sh["routed_scaling"]), _arr(g["given_weights"]),
                               rtol=0, atol=1e-15)
    # negative controls: the biased score, or no routed_scaling, give other weights
    s_sel = np.take_along_axis(O.sigmoid(z), given, axis=1)
    b_sel = args["bias"][given]
    by_sel = 2.5 * (s_sel + b_sel) / (s_sel + b_sel).sum(axis=1, keepdims=True)
    unscaled = s_sel / s_sel.sum(axis=1, keepdims=True)
    for wrong in (by_sel, unscaled):
        assert np.abs(wrong - _arr(g["given_weights"])).max() > 0.05


def test_sigmoid_weights_for_equals_the_rule_on_its_own_selection():
    rng = np.random.default_rng(31)
    for E, G, tg, K, scale in [(128, 8, 4, 8, 2.5), (32, 4, 2, 4, 1.0), (16, 1, 1, 3, 0.7)]:
        z = rng.standard_normal((60, E)) * 1.5
        b = rng.standard_normal(E) * 0.3
        rt = O.sigmoid_group_topk(z, b, K, G, tg, scale)
        np.testing.assert_allclose(O.sigmoid_weights_for(z, rt.ids, scale), rt.weights, rtol=1e-15, atol=0)
        np.testing.assert_allclose(O.weights_for(z, rt.ids, "sigmoid_group", scale), rt.weights, rtol=1e-15, atol=0)
        # slot order follows the given ids
        rev = rt.ids[:, ::-1]
        np.testing.assert_allclose(O.sigmoid_weights_for(z, rev, scale), rt.weights[:, ::-1], rtol=1e-15, atol=0)


def test_sigmoid_given_ids_layer_reproduces_the_unforced_layer():
    rng = np.random.default_rng(32)
    x, r, wr, banks = _rand_layer(rng, 10, 32, 16, 4, 16, 16, gated=False)
    kw = dict(bias=rng.standard_normal(16) * 0.3, n_group=4, topk_group=2, routed_scaling=2.5)
    full = O.layer_forward(x, r, wr, banks, "sigmoid_group", 4, **kw)
    again = O.layer_forward(x, r, wr, banks, "sigmoid_group", 4, ids=full.route.ids, **kw)
    np.testing.assert_array_equal(again.route.ids, full.route.ids)
    np.testing.assert_allclose(again.route.weights, full.route.weights, rtol=1e-15, atol=0)
    np.testing.assert_allclose(again.out, full.out, rtol=0, atol=1e-14)
    # swapped slot order: the same sum up to fp64 rounding
    swapped = O.layer_forward(x, r, wr, banks, "sigmoid_group", 4, ids=full.route.ids[:, ::-1], **kw)
    np.testing.assert_allclose(swapped.out, full.out, rtol=0, atol=1e-13)
    sub = np.array([7, 2])
    part = O.layer_forward(x, r, wr, banks, "sigmoid_group", 4, tokens=sub, ids=full.route.ids, **kw)
    np.testing.assert_allclose(part.out, full.out[sub], rtol=0, atol=1e-14)


@pytest.mark.parametrize("dtype", ["bf16", "u4", "f32"])
def test_lazy_banks_equal_eager_widening(dtype):
    """The per-expert (lazy) widening the full-shape tests use returns exactly
    the eager widening's slice for every expert and matrix; bf16 also equals
    torch's own bf16 -> float64 conversion."""
    import dataclasses
    from oracle.inputs import banks_from
    from synth import WORKLOADS, make_weights
    base = {"bf16": "qwen_decode", "u4": "qwen_u4", "f32": "tiny_f32"}[dtype]
    spec = dataclasses.replace(WORKLOADS[base], d_model=128, n_experts=16, d_ff=64, d_ff_shared=64, top_k=4)
    w = make_weights(spec)
    eager, lazy = banks_from(w), banks_from(w, lazy=True)
    assert callable(lazy.gate) and not callable(eager.gate)
    for e in range(spec.n_experts):
        for a, b in zip(eager.expert(e), lazy.expert(e)):
            np.testing.assert_array_equal(a, b)
    if dtype == "bf16":
        np.testing.assert_array_equal(eager.gate, w.gate.w.double().numpy())
        np.testing.assert_array_equal(lazy.expert(5)[2], w.down.w[5].double().numpy())
    for name in ("shared_gate", "shared_up", "shared_down"):
        np.testing.assert_array_equal(getattr(eager, name), getattr(lazy, name))


def test_golden_u4_dequant_by_hand():
    g = _load("u4_affine_g64_hand.json")
    codes = np.array([g["codes_row0_bytes"][0]] * 32 + [g["codes_row0_bytes"][1]] * 32, dtype=np.uint8)[None]
    w = O.dequant_u4_g64(codes, np.array([g["scale_bits_row0"]], dtype=np.uint16),
                         np.array([g["min_bits_row0"]], dtype=np.uint16))
    assert w.shape == (1, 128)
    np.testing.assert_array_equal(w[0, :64].reshape(32, 2), np.tile(g["expected_row0_group0_pair"], (32, 1)))
    np.testing.assert_array_equal(w[0, 64:].reshape(32, 2), np.tile(g["expected_row0_group1_pair"], (32, 1)))


def test_golden_permute_by_hand():
    g = _load("permute_hand.json")
    p = O.permute(np.array(g["ids"]), g["n_experts"])
    np.testing.assert_array_equal(p.offsets, g["expected_offsets"])
    np.testing.assert_array_equal(p.active, g["expected_active"])
    assert p.n_active == len(g["expected_active"])
    np.testing.assert_array_equal(p.sorted_pairs, g["expected_sorted_pairs"])


def test_bf16_widening_exact():
    # bit patterns with known values: 1.0, -2.0, 0.5, smallest subnormal, max finite
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0001, 0x7F7F], dtype=np.uint16)
    v = O.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.5
    assert v[3] == 2.0 ** -133
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127
    t = torch.tensor([1.0, -2.0, 0.5, 3.140625], dtype=torch.bfloat16)
    np.testing.assert_array_equal(O.bf16_bits_to_f64(t.view(torch.int16).numpy()), t.double().numpy())


# ------------------------------------------------------------- routing invariants
@pytest.mark.parametrize("E,K", [(16, 4), (256, 8), (256, 4), (8, 8)])
def test_renorm_sums_to_one_and_selected_softmax_form(E, K):
    rng = np.random.default_rng(E * 10 + K)
    z = rng.standard_normal((64, E)) * 2.0
    rt = O.softmax_topk(z, K)
    np.testing.assert_allclose(rt.weights.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    # the global denominator cancels: alpha = exp(z_i) / sum_{j in I} exp(z_j)
    zs = np.take_along_axis(z, rt.ids.astype(np.int64), axis=1)
    closed = np.exp(zs) / np.exp(zs).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(rt.weights, closed, rtol=1e-12, atol=0)
    # the 2^-14 clamp never binds for softmax: the top-K mass is >= K/E
    assert (np.sort(rt.score, axis=1)[:, ::-1][:, :K].sum(axis=1) >= K / E - 1e-15).all()


def test_softmax_matches_library_routine():
    rng = np.random.default_rng(7)
    z = rng.standard_normal((32, 256)) * 3
    np.testing.assert_allclose(O.softmax(z), torch.softmax(torch.from_numpy(z), dim=1).numpy(), rtol=1e-13, atol=0)


def _is_topk(score, S, K):
    """Defining property of the top-K set with ties to the lower index."""
    rest = [j for j in range(score.size) if j not in S]
    return len(S) == K and all((score[i] > score[j]) or (score[i] == score[j] and i < j)
                               for i in S for j in rest)


@pytest.mark.parametrize("tied", [False, True])
def test_topk_brute_force_tiny(tied):
    rng = np.random.default_rng(11 + tied)
    E, K = 16, 4
    for trial in range(40):
        z = rng.integers(-2, 3, E).astype(np.float64) if tied else rng.standard_normal(E)
        rt = O.softmax_topk(z[None], K)
        winners = [S for S in itertools.combinations(range(E), K) if _is_topk(rt.score[0], S, K)]
        assert len(winners) == 1
        assert sorted(rt.ids[0].tolist()) == list(winners[0])
        # slot order: descending score, ties -> lower index
        ids = rt.ids[0]
        for a, b in zip(ids[:-1], ids[1:]):
            assert rt.score[0, a] > rt.score[0, b] or (rt.score[0, a] == rt.score[0, b] and a < b)
        # ranking by probability equals ranking by logit
        assert list(ids) == list(np.lexsort((np.arange(E), -z))[:K])


def test_all_tie_softmax():
    rt = O.softmax_topk(np.zeros((3, 256)), 8)
    np.testing.assert_array_equal(rt.ids, np.tile(np.arange(8), (3, 1)))
    np.testing.assert_array_equal(rt.weights, np.full((3, 8), 1 / 8))
    assert rt.flags.all()


def _brute_group(z, b, K, G, tg, scale):
    E = z.size
    gs = E // G
    s = 1 / (1 + np.exp(-z))
    sel = s + b
    # "sum of the two best" by brute force over all pairs of distinct members
    gscore = np.array([max(sel[i] + sel[j] for i, j in itertools.combinations(range(g * gs, (g + 1) * gs), 2))
                       for g in range(G)])
    kept = [Gs for Gs in itertools.combinations(range(G), tg) if _is_topk(gscore, Gs, tg)]
    assert len(kept) == 1
    cand = [e for g in kept[0] for e in range(g * gs, (g + 1) * gs)]
    masked = np.where(np.isin(np.arange(E), cand), sel, -np.inf)
    S = [S for S in itertools.combinations(cand, K) if _is_topk(masked, S, K)]
    assert len(S) == 1
    w = scale * s[list(S[0])] / max(s[list(S[0])].sum(), 2.0 ** -14)
    return set(S[0]), dict(zip(S[0], w))


@pytest.mark.parametrize("E,G,tg,K", [(16, 4, 2, 4), (16, 8, 3, 3), (12, 3, 1, 2), (16, 4, 4, 5)])
def test_group_topk_brute_force(E, G, tg, K):
    rng = np.random.default_rng(E + G + tg + K)
    for trial in range(25):
        z = rng.standard_normal(E) if trial % 3 else rng.integers(-1, 2, E).astype(float)
        b = rng.standard_normal(E) * 0.3 if trial % 2 else np.zeros(E)
        rt = O.sigmoid_group_topk(z[None], b, K, G, tg, 2.5)
        S, w = _brute_group(z, b, K, G, tg, 2.5)
        assert set(rt.ids[0].tolist()) == S
        for slot, e in enumerate(rt.ids[0]):
            assert abs(rt.weights[0, slot] - w[int(e)]) < 1e-13
        np.testing.assert_allclose(rt.weights.sum(), 2.5, rtol=1e-13)


def test_group_rule_degenerates_to_plain_topk():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((50, 128))
    b = rng.standard_normal(128) * 0.3
    sel = 1 / (1 + np.exp(-z)) + b
    plain = np.stack([np.lexsort((np.arange(128), -row))[:8] for row in sel])
    for G, tg in [(8, 8), (1, 1)]:
        rt = O.sigmoid_group_topk(z, b, 8, G, tg, 2.5)
        np.testing.assert_array_equal(rt.ids, plain)


def test_bias_selects_but_does_not_weight():
    rng = np.random.default_rng(5)
    z = rng.standard_normal((40, 128))
    b = rng.standard_normal(128) * 0.3
    base = O.sigmoid_group_topk(z, b, 8, 8, 4, 2.5)
    shifted = O.sigmoid_group_topk(z, b + 0.75, 8, 8, 4, 2.5)
    np.testing.assert_array_equal(base.ids, shifted.ids)
    np.testing.assert_allclose(base.weights, shifted.weights, rtol=0, atol=0)
    # a +10 bias forces expert 77 into every token; its weight uses the raw score only
    b2 = b.copy()
    b2[77] += 10
    forced = O.sigmoid_group_topk(z, b2, 8, 8, 4, 2.5)
    s = 1 / (1 + np.exp(-z))
    for t in range(z.shape[0]):
        ids = forced.ids[t]
        assert ids[0] == 77
        np.testing.assert_allclose(forced.weights[t], 2.5 * s[t, ids] / s[t, ids].sum(), rtol=1e-13)
        # negative control: weighting by the biased score would differ
        assert not np.allclose(forced.weights[t], 2.5 * (s[t, ids] + b2[ids]) / (s[t, ids] + b2[ids]).sum())


def test_all_tie_sigmoid_group():
    rt = O.sigmoid_group_topk(np.zeros((2, 128)), np.zeros(128), 8, 8, 4, 2.5)
    np.testing.assert_array_equal(rt.ids, np.tile(np.arange(8), (2, 1)))
    np.testing.assert_array_equal(rt.weights, np.full((2, 8), 2.5 / 8))


def test_sigmoid_clamp_binds_only_when_scores_vanish():
    z = np.full((1, 16), -30.0)
    z[0, :4] += np.array([0.5, 0.25, 0.125, 0.0])
    rt = O.sigmoid_group_topk(z, None, 4, 4, 2, 2.5)
    s = 1 / (1 + np.exp(-z[0, rt.ids[0]]))
    assert s.sum() < 2.0 ** -14
    assert rt.weights.sum() < 2.5 * 1e-6  # the floor keeps the weights tiny instead of renormalising to 2.5
    np.testing.assert_allclose(rt.weights[0] / rt.weights[0].sum(), s / s.sum(), rtol=1e-12)


# ------------------------------------------------------------- permute
def test_permute_brute_force():
    rng = np.random.default_rng(9)
    for T, E, K in [(1, 8, 2), (7, 16, 4), (33, 64, 8), (100, 5, 5)]:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)])
        p = O.permute(ids, E)
        buckets = {e: [] for e in range(E)}
        for t in range(T):
            for k in range(K):
                buckets[int(ids[t, k])].append(t * K + k)
        flat = [q for e in range(E) for q in buckets[e]]
        assert p.sorted_pairs.tolist() == flat
        assert p.offsets[-1] == T * K and sorted(flat) == list(range(T * K))
        assert p.offsets.tolist() == [0] + list(np.cumsum([len(buckets[e]) for e in range(E)]))
        assert p.active.tolist() == [e for e in range(E) if buckets[e]]


# ------------------------------------------------------------- textbook reductions
def _torch_swiglu(x, wg, wu, wd):
    xt = torch.from_numpy(x)
    h = torch.nn.functional.silu(xt @ torch.from_numpy(wg).T) * (xt @ torch.from_numpy(wu).T)
    return (h @ torch.from_numpy(wd).T).numpy()


def test_single_expert_is_plain_swiglu_ffn():
    rng = np.random.default_rng(21)
    x, r, wr, banks = _rand_layer(rng, 6, 32, 1, 1, 16, 0)
    res = O.layer_forward(x, r, wr, banks, "softmax", 1)
    np.testing.assert_array_equal(res.route.weights, np.ones((6, 1)))
    ffn = _torch_swiglu(x, banks.gate[0], banks.up[0], banks.down[0])
    np.testing.assert_allclose(res.out, r + ffn, rtol=1e-12, atol=1e-12)


def test_k_equals_e_is_dense_softmax_mixture():
    rng = np.random.default_rng(22)
    T, D, E, F = 5, 24, 6, 8
    x, r, wr, banks = _rand_layer(rng, T, D, E, E, F, 0)
    res = O.layer_forward(x, r, wr, banks, "softmax", E)
    p = torch.softmax(torch.from_numpy(x @ wr.T), dim=1).numpy()
    dense = sum(p[:, e:e + 1] * _torch_swiglu(x, banks.gate[e], banks.up[e], banks.down[e]) for e in range(E))
    np.testing.assert_allclose(res.y_moe, dense, rtol=1e-11, atol=1e-12)


def test_zero_gate_vector_halves_shared_expert():
    rng = np.random.default_rng(23)
    x, r, wr, banks = _rand_layer(rng, 4, 16, 4, 2, 8, 8)
    banks.shared_gate_vec = np.zeros(16)
    ys = O.shared_expert(x, banks)
    np.testing.assert_allclose(ys, 0.5 * _torch_swiglu(x, banks.shared_gate, banks.shared_up, banks.shared_down),
                               rtol=1e-13, atol=1e-16)
    # sigmoid(0) = 1/2 exactly: the gated output is exactly half the ungated one
    banks.shared_gate_vec = None
    np.testing.assert_array_equal(ys, 0.5 * O.shared_expert(x, banks))


def test_grouped_and_dense_formulations_agree():
    rng = np.random.default_rng(24)
    x, r, wr, banks = _rand_layer(rng, 9, 64, 16, 4, 32, 32)
    for fam, kw in [("softmax", {}), ("sigmoid_group",
                                       dict(bias=rng.standard_normal(16) * 0.3, n_group=4, topk_group=2,
                                            routed_scaling=2.5))]:
        a = O.layer_forward(x, r, wr, banks, fam, 4, **kw).out
        b = O.layer_forward_dense(x, r, wr, banks, fam, 4, **kw)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_token_subset_and_given_ids_consistent():
    rng = np.random.default_rng(25)
    x, r, wr, banks = _rand_layer(rng, 12, 32, 8, 2, 16, 16)
    full = O.layer_forward(x, r, wr, banks, "softmax", 2)
    sub = np.array([3, 0, 11])
    part = O.layer_forward(x, r, wr, banks, "softmax", 2, tokens=sub)
    np.testing.assert_allclose(part.out, full.out[sub], rtol=0, atol=1e-14)
    again = O.layer_forward(x, r, wr, banks, "softmax", 2, ids=full.route.ids)
    np.testing.assert_allclose(again.out, full.out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(O.softmax_weights_for(full.z, full.route.ids), full.route.weights, rtol=1e-15)


# ------------------------------------------------------------- RMS normalisation
def _ev_pow(expr):
    """Fixture expression with ** allowed (hand-derived numbers only)."""
    if isinstance(expr, (int, float)):
        return float(expr)
    assert set(expr) <= set("0123456789.+-*/() "), expr
    return float(eval(expr, {"__builtins__": {}}, {}))  # noqa: S307 - restricted alphabet


def test_golden_rms_norm_by_hand():
    g = _load("rms_norm_hand.json")
    for c in g["cases"]:
        w = None if c["weight"] is None else np.array(c["weight"], dtype=np.float64)
        got = O.rms_norm(np.array(c["r"], dtype=np.float64), w, c["eps"])
        want = np.vectorize(_ev_pow, otypes=[np.float64])(np.array(c["x"], dtype=object))
        np.testing.assert_allclose(got, want, rtol=1e-15, atol=1e-15, err_msg=c["derivation"])


def test_golden_bf16_rounding_by_hand():
    g = _load("rms_norm_hand.json")
    for c in g["bf16_cases"]:
        v = np.array([_ev_pow(c["v"])])
        with np.errstate(over="ignore"):
            bits = O.bf16_bits(O.round_bf16(v))[0]
        assert bits == int(c["bits"], 16), (c["v"], hex(bits), c["why"])


@pytest.mark.parametrize("alpha", [1e-3, 0.37, 7.5, 1e4])
def test_rms_norm_scale_invariance(alpha):
    """rms_norm(alpha r; alpha^2 eps) = rms_norm(r; eps) for alpha > 0: the
    mean square scales by alpha^2 and eps sits inside the square root with it."""
    rng = np.random.default_rng(5)
    r = rng.standard_normal((6, 96)) * rng.uniform(0.1, 30, (6, 1))
    w = rng.standard_normal(96)
    for eps in (0.0, 1e-6, 0.5):
        np.testing.assert_allclose(O.rms_norm(alpha * r, w, eps * alpha ** 2), O.rms_norm(r, w, eps),
                                   rtol=1e-12, atol=1e-14)


def test_rms_norm_mean_square_closed_form():
    """Unit weight: mean(x^2) = ms / (ms + eps); a weight multiplies afterwards."""
    rng = np.random.default_rng(6)
    r = rng.standard_normal((5, 64)) * 3
    ms = (r * r).mean(axis=1)
    for eps in (0.0, 1e-6, 2.0):
        x = O.rms_norm(r, None, eps)
        np.testing.assert_allclose((x * x).mean(axis=1), ms / (ms + eps), rtol=1e-13)
        assert np.all(np.sign(x) == np.sign(r))
    w = rng.uniform(0.5, 2.0, 64)
    np.testing.assert_allclose(O.rms_norm(r, w, 1e-6) / w, O.rms_norm(r, None, 1e-6), rtol=1e-14)


def test_round_bf16_matches_library_on_fp32_values():
    """For values that are fp32 numbers, rounding to bf16 is what torch's
    float32 -> bfloat16 conversion (round to nearest even) gives."""
    rng = np.random.default_rng(7)
    m = rng.uniform(-2, 2, 20000)
    ex = rng.integers(-140, 120, 20000)
    v32 = np.ldexp(m, ex).astype(np.float32)
    # exact ties: a bf16 value plus half its spacing (even and odd neighbours)
    base = rng.integers(0x0080, 0x7F00, 4000, dtype=np.uint32) << np.uint32(16)
    ties = (base | np.uint32(0x8000)).view(np.float32)
    v32 = np.concatenate([v32, ties, -ties, np.float32([0.0, 1.0, -1.0])])
    lib = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = O.bf16_bits(O.round_bf16(v32.astype(np.float64)))
    assert np.array_equal(ours, lib)


def test_round_bf16_rounds_once_from_the_exact_value():
    """A value just above a tie rounds up even when its fp32 rounding would land
    on the tie (rounding via fp32 first would give the even neighbour)."""
    v = np.array([1 + 2.0 ** -8 + 2.0 ** -30, -(3 + 2.0 ** -7 + 2.0 ** -30)])
    assert np.array_equal(v.astype(np.float32).astype(np.float64), [1 + 2.0 ** -8, -(3 + 2.0 ** -7)])
    np.testing.assert_array_equal(O.round_bf16(v), [1 + 2.0 ** -7, -(3 + 2.0 ** -6)])


def test_bf16_boundary_distance_brackets_the_rounding_switch():
    """Inside the returned distance every value rounds alike; just past it the
    rounding changes (so the distance is that of the nearest boundary)."""
    rng = np.random.default_rng(8)
    v = np.ldexp(rng.uniform(0.5, 1.0, 5000), rng.integers(-20, 20, 5000)) * rng.choice([-1.0, 1.0], 5000)
    d = O.bf16_boundary_distance(v)
    inside_lo, inside_hi = O.round_bf16(v * (1 - 0.99 * d)), O.round_bf16(v * (1 + 0.99 * d))
    assert np.array_equal(inside_lo, inside_hi)
    outside_lo, outside_hi = O.round_bf16(v * (1 - 1.01 * d)), O.round_bf16(v * (1 + 1.01 * d))
    assert np.all(outside_lo != outside_hi)
    np.testing.assert_array_equal(O.bf16_boundary_distance(np.array([1.0, 1.5, 1 - 2.0 ** -9, 0.0])),
                                  [2.0 ** -9, 2.0 ** -8 / 1.5, 0.0, np.inf])


def test_normed_activation_rounds_once_per_dtype():
    rng = np.random.default_rng(9)
    r = rng.standard_normal((3, 128)) * 5
    x = O.rms_norm(r, None, 1e-6)
    np.testing.assert_array_equal(O.normed_activation(r, None, 1e-6, "f32"), x.astype(np.float32).astype(np.float64))
    b = O.normed_activation(r, None, 1e-6, "bf16")
    assert np.all(np.abs(b - x) <= 2.0 ** -8 * np.abs(x))
    O.bf16_bits(b)  # every element is a bf16 value
