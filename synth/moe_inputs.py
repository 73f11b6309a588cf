"""Seeded synthetic inputs for one sparse-MoE layer forward.

This module only *draws* inputs: it holds none of the layer's arithmetic
(no routing, no expert math, no dequantisation).  Both the HIP library's
tests/bench and the fp64 oracle receive the tensors produced here; neither
side imports the other.

Shapes follow the model facts on the pages:
  * Qwen3.6-35B-A3B: d_model 2048, 256 routed experts, top-8, expert and
    shared intermediate 512, softmax routing with a gated shared expert
    (Treebeard, "How Treebeard routes Qwen3.6 MoE tokens", "Model constants"
    table and the GGUF metadata block under "Source map").
  * edge0 tiers: the 35b tier uses softmax top-4 with 4-bit affine group-64
    weights, the 8b tier 128 experts with sigmoid group top-k, n_group 8,
    topk_group 4, routed_scaling 2.5 (edge0 "MoE Routing and Experts", tier
    table and "Routing families").

Recipe (every tensor is drawn with torch's generator on the requested device;
the same seed on the same device type gives the same tensor):
  * weight seed = 1000 * workload id; token seed = 1000 * workload id + T.
  * draw order: router, per-expert skew offsets or expert_bias, gate bank,
    up bank, down bank, shared gate, shared up, shared down, shared gate
    vector; then (token generator) hidden, residual.
  * weights: standard normal float32 draws times 1/sqrt(fan_in) (variance
    1/fan_in; fan_in = d_model for router/gate/up/shared-gate-vector, d_ff or
    d_ff_shared for down), then rounded to bf16 (round-to-nearest-even) for
    bf16 workloads, kept float32 for the fp32 workload.
  * 4-bit affine group-64 workload: the float32 draws are quantised per group
    of 64 consecutive *input* elements: min = bf16(min w), scale =
    bf16((max w - min w) / 15), q = clamp(round_half_even((w - min) / scale),
    0, 15) (q = 0 where scale == 0); two codes per byte, even element in the
    low nibble.  Routed and shared banks are quantised; the router and the
    shared gate vector stay bf16.
  * hidden x: g ~ N(0,1) [T, D], divided by its row RMS (eps 0), rounded to
    bf16; the fp32 tiny workload uses plain N(0,1) float32.  In the skewed
    prefill workload g[:, D-1] is set to 1 before the RMS step and the
    router's last column receives a per-expert offset b_e ~ N(0, var 1.5), so
    b_e acts as a logit-space offset (load skew, some experts idle).
  * residual ~ N(0,1) float32.
  * attention residual for the entry that normalises it (make_attention_residual):
    r_t = s_t g_t with g_t drawn as for the hidden state above (N(0,1); last
    column 1 in the skewed workload) and s_t = 4 exp(N(0,1)) a per-token
    magnitude (rows of very different scale); token seed 1000 * id + T + 500.
    RMS-norm weight 1 + 0.1 N(0,1) float32, seed 1000 * id + 999 (+ a layer
    index for chained layers).
  * sigmoid-group workload: expert_bias ~ N(0, var 0.1) float32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

WORKLOAD_IDS = {
    "tiny_f32": 1,
    "qwen_decode": 2,
    "qwen_prefill_skew": 3,
    "sigmoid_group": 4,
    "qwen_u4": 5,
}


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Static description of one MoE layer workload."""

    name: str
    n_tokens: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    d_ff_shared: int  # 0 => no shared expert
    family: str  # "softmax" | "sigmoid_group"
    n_group: int = 1
    topk_group: int = 1
    routed_scaling: float = 1.0
    act_dtype: str = "bf16"  # "f32" | "bf16"
    router_dtype: str = "bf16"  # "f32" | "bf16"
    expert_dtype: str = "bf16"  # "f32" | "bf16" | "u4"
    shared_gate: bool = True
    skew_var: float = 0.0
    bias_var: float = 0.0

    @property
    def workload_id(self) -> int:
        return WORKLOAD_IDS[self.name]

    def with_tokens(self, n_tokens: int) -> "LayerSpec":
        return dataclasses.replace(self, n_tokens=n_tokens)


_QWEN = dict(d_model=2048, n_experts=256, d_ff=512, d_ff_shared=512, family="softmax")

WORKLOADS = {
    "tiny_f32": LayerSpec("tiny_f32", 4, 64, 16, 4, 32, 32, "softmax",
                          act_dtype="f32", router_dtype="f32", expert_dtype="f32"),
    "qwen_decode": LayerSpec("qwen_decode", 8, top_k=8, **_QWEN),
    "qwen_prefill_skew": LayerSpec("qwen_prefill_skew", 4096, top_k=8, skew_var=1.5, **_QWEN),
    "sigmoid_group": LayerSpec("sigmoid_group", 2048, 2048, 128, 8, 512, 512, "sigmoid_group",
                               n_group=8, topk_group=4, routed_scaling=2.5,
                               shared_gate=False, bias_var=0.1),
    "qwen_u4": LayerSpec("qwen_u4", 64, top_k=4, expert_dtype="u4", **_QWEN),
}

# token counts each workload is exercised at
WORKLOAD_TOKENS = {
    "tiny_f32": (4,),
    "qwen_decode": (1, 8, 32),
    "qwen_prefill_skew": (4096,),
    "sigmoid_group": (2048,),
    "qwen_u4": (1, 64, 512),
}


@dataclasses.dataclass
class Matrix:
    """A weight matrix (or bank).  For u4: w = codes uint8 [..., rows, in/2],
    scale/min bf16 [..., rows, in/64]; otherwise w is f32/bf16 [..., rows, in]."""

    w: torch.Tensor
    scale: Optional[torch.Tensor] = None
    min: Optional[torch.Tensor] = None

    def tensors(self):
        return [t for t in (self.w, self.scale, self.min) if t is not None]


@dataclasses.dataclass
class LayerWeights:
    router: torch.Tensor  # [E, D]
    expert_bias: Optional[torch.Tensor]  # [E] f32
    gate: Matrix  # [E, F, D]
    up: Matrix  # [E, F, D]
    down: Matrix  # [E, D, F]
    shared_gate: Optional[Matrix]  # [Fs, D]
    shared_up: Optional[Matrix]  # [Fs, D]
    shared_down: Optional[Matrix]  # [D, Fs]
    shared_gate_vec: Optional[torch.Tensor]  # [D]

    def all_tensors(self):
        out = [self.router]
        if self.expert_bias is not None:
            out.append(self.expert_bias)
        for m in (self.gate, self.up, self.down, self.shared_gate, self.shared_up, self.shared_down):
            if m is not None:
                out.extend(m.tensors())
        if self.shared_gate_vec is not None:
            out.append(self.shared_gate_vec)
        return out


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, std: float, gen, device) -> torch.Tensor:
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return t.mul_(std)


def _to_dtype(t: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return t.contiguous()
    if dtype == "bf16":
        return t.to(torch.bfloat16).contiguous()  # round-to-nearest-even
    raise ValueError(dtype)


def quantize_u4_g64(w: torch.Tensor) -> Matrix:
    """Affine 4-bit quantiser, groups of 64 consecutive elements of the last
    (input) dimension; see the module docstring for the rule."""
    *lead, n_in = w.shape
    if n_in % 64:
        raise ValueError("input dim must be a multiple of 64")
    g = w.reshape(*lead, n_in // 64, 64).float()
    gmin = g.amin(dim=-1)
    gmax = g.amax(dim=-1)
    mn = gmin.to(torch.bfloat16)
    sc = ((gmax - gmin) / 15.0).to(torch.bfloat16)
    scf = sc.float().unsqueeze(-1)
    q = torch.where(scf > 0, torch.round((g - mn.float().unsqueeze(-1)) / torch.where(scf > 0, scf, torch.ones_like(scf))),
                    torch.zeros_like(g))
    q = q.clamp_(0, 15).to(torch.uint8).reshape(*lead, n_in)
    codes = (q[..., 0::2] | (q[..., 1::2] << 4)).contiguous()
    return Matrix(codes, sc.contiguous(), mn.contiguous())


def _bank(shape, fan_in: int, dtype: str, gen, device) -> Matrix:
    w = _normal(shape, 1.0 / math.sqrt(fan_in), gen, device)
    if dtype == "u4":
        m = quantize_u4_g64(w)
        del w
        return m
    return Matrix(_to_dtype(w, dtype))


def make_weights(spec: LayerSpec, device="cpu", seed: Optional[int] = None) -> LayerWeights:
    """Draw one layer's weights (see the module docstring for the recipe)."""
    seed = 1000 * spec.workload_id if seed is None else seed
    gen = _gen(seed, device)
    D, E, F, Fs = spec.d_model, spec.n_experts, spec.d_ff, spec.d_ff_shared
    router = _normal((E, D), 1.0 / math.sqrt(D), gen, device)
    expert_bias = None
    if spec.skew_var > 0:
        offs = _normal((E,), math.sqrt(spec.skew_var), gen, device)
        router[:, D - 1] += offs
    if spec.family == "sigmoid_group":
        expert_bias = _normal((E,), math.sqrt(spec.bias_var), gen, device) if spec.bias_var > 0 \
            else torch.zeros(E, device=device)
    router = _to_dtype(router, spec.router_dtype)
    gate = _bank((E, F, D), D, spec.expert_dtype, gen, device)
    up = _bank((E, F, D), D, spec.expert_dtype, gen, device)
    down = _bank((E, D, F), F, spec.expert_dtype, gen, device)
    sg = su = sd = sv = None
    if Fs > 0:
        sg = _bank((Fs, D), D, spec.expert_dtype, gen, device)
        su = _bank((Fs, D), D, spec.expert_dtype, gen, device)
        sd = _bank((D, Fs), Fs, spec.expert_dtype, gen, device)
        if spec.shared_gate:
            sv = _to_dtype(_normal((D,), 1.0 / math.sqrt(D), gen, device), spec.router_dtype)
    return LayerWeights(router, expert_bias, gate, up, down, sg, su, sd, sv)


def make_tokens(spec: LayerSpec, device="cpu", seed: Optional[int] = None):
    """Draw hidden states x [T, D] and residual r [T, D] float32."""
    T, D = spec.n_tokens, spec.d_model
    seed = 1000 * spec.workload_id + T if seed is None else seed
    gen = _gen(seed, device)
    g = torch.randn((T, D), generator=gen, device=device, dtype=torch.float32)
    if spec.act_dtype == "f32":
        x = g.contiguous()
    else:
        if spec.skew_var > 0:
            g[:, D - 1] = 1.0
        rms = g.square().mean(dim=1, keepdim=True).sqrt()
        x = (g / rms).to(torch.bfloat16).contiguous()
    r = torch.randn((T, D), generator=gen, device=device, dtype=torch.float32)
    return x, r



def make_attention_residual(spec: LayerSpec, device="cpu", seed: Optional[int] = None,
                            weight_seed: Optional[int] = None):
    """Draw an attention residual r [T, D] float32 and an RMS-norm weight [D]
    float32 (the inputs of the layer entry that normalises r itself)."""
    T, D = spec.n_tokens, spec.d_model
    seed = 1000 * spec.workload_id + T + 500 if seed is None else seed
    gen = _gen(seed, device)
    g = torch.randn((T, D), generator=gen, device=device, dtype=torch.float32)
    if spec.skew_var > 0:
        g[:, D - 1] = 1.0
    mag = 4.0 * torch.exp(torch.randn((T, 1), generator=gen, device=device, dtype=torch.float32))
    r = (g * mag).contiguous()
    wgen = _gen(1000 * spec.workload_id + 999 if weight_seed is None else weight_seed, device)
    w = (1.0 + 0.1 * torch.randn((D,), generator=wgen, device=device, dtype=torch.float32)).contiguous()
    return r, w
