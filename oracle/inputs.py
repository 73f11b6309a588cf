"""Widen layer inputs held as torch tensors into the oracle's float64 arrays.

TEST INFRASTRUCTURE ONLY (see moe_oracle.py).  Accepts any object with the
attributes of a layer-weights record (router, expert_bias, gate, up, down,
shared_gate, shared_up, shared_down, shared_gate_vec; matrices carry w, scale,
min); it imports nothing from the library or the input generator.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import Banks, bf16_bits_to_f64, dequant_u4_g64


def to_numpy(t) -> np.ndarray:
    """torch tensor (any device) -> numpy; bf16 becomes its uint16 bit pattern."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen_tensor(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(to_numpy(t))
    return to_numpy(t).astype(np.float64)


def widen_matrix(m, index=None) -> np.ndarray:
    """A weight matrix (f32/bf16 tensor, or u4 codes + bf16 scale/min) -> fp64,
    optionally only bank entry `index`."""
    pick = (lambda t: t[index]) if index is not None else (lambda t: t)
    if m.scale is not None:
        return dequant_u4_g64(to_numpy(pick(m.w)), to_numpy(pick(m.scale)), to_numpy(pick(m.min)))
    return widen_tensor(pick(m.w))


class _LazyBank:
    """Widens one expert's matrix on demand (no cache: each expert is used once per call)."""

    def __init__(self, m):
        self.m = m

    def __call__(self, e):
        return widen_matrix(self.m, e)


def banks_from(weights, lazy: bool = False) -> Banks:
    def bank(m):
        return _LazyBank(m) if lazy else widen_matrix(m)

    def opt(m):
        return None if m is None else widen_matrix(m)

    return Banks(bank(weights.gate), bank(weights.up), bank(weights.down),
                 opt(weights.shared_gate), opt(weights.shared_up), opt(weights.shared_down),
                 None if weights.shared_gate_vec is None else widen_tensor(weights.shared_gate_vec))
