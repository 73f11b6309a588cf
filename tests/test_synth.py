"""The seeded input generator: shapes, determinism and the 4-bit quantiser's error bound."""
import math

import numpy as np
import torch

from synth import WORKLOADS, make_tokens, make_weights, quantize_u4_g64
from oracle.moe_oracle import dequant_u4_g64
from oracle.inputs import to_numpy


def _small(name, **kw):
    import dataclasses
    base = WORKLOADS[name]
    return dataclasses.replace(base, **kw)


def test_shapes_and_determinism():
    spec = _small("qwen_decode", d_model=128, n_experts=16, d_ff=64, d_ff_shared=64, n_tokens=5)
    a, b = make_weights(spec), make_weights(spec)
    for ta, tb in zip(a.all_tensors(), b.all_tensors()):
        assert torch.equal(ta, tb)
    assert a.router.shape == (16, 128) and a.router.dtype == torch.bfloat16
    assert a.gate.w.shape == (16, 64, 128) and a.down.w.shape == (16, 128, 64)
    assert a.shared_gate_vec.shape == (128,)
    x, r = make_tokens(spec)
    assert x.shape == (5, 128) and x.dtype == torch.bfloat16 and r.dtype == torch.float32
    rms = x.float().square().mean(dim=1).sqrt()
    assert torch.allclose(rms, torch.ones(5), atol=1e-2)


def test_skew_constant_feature():
    spec = _small("qwen_prefill_skew", d_model=128, n_experts=16, d_ff=64, d_ff_shared=64, n_tokens=64)
    x, _ = make_tokens(spec)
    v = x[:, -1].float()
    assert (v > 0.7).all() and (v < 1.4).all()


def test_u4_quantiser_error_bound():
    g = torch.Generator().manual_seed(1)
    w = torch.randn(8, 16, 256, generator=g) / math.sqrt(256)
    m = quantize_u4_g64(w)
    assert m.w.dtype == torch.uint8 and m.w.shape == (8, 16, 128)
    assert m.scale.shape == (8, 16, 4) and m.scale.dtype == torch.bfloat16
    deq = dequant_u4_g64(to_numpy(m.w), to_numpy(m.scale), to_numpy(m.min))
    wg = w.double().numpy().reshape(8, 16, 4, 64)
    exact_scale = (wg.max(-1) - wg.min(-1)) / 15
    sc = m.scale.double().numpy()
    mn = m.min.double().numpy()
    bound = sc / 2 + np.abs(mn - wg.min(-1)) + 15 * np.abs(exact_scale - sc) + 1e-7
    err = np.abs(deq.reshape(8, 16, 4, 64) - wg).max(-1)
    assert (err <= bound).all()


def test_sigmoid_workload_has_bias_and_no_shared_gate():
    spec = _small("sigmoid_group", d_model=64, d_ff=32, d_ff_shared=32, n_tokens=4)
    wts = make_weights(spec)
    assert wts.expert_bias is not None and wts.expert_bias.shape == (128,)
    assert wts.shared_gate_vec is None
