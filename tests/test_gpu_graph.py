"""Captured HIP graphs of the layer entries: every replay equals an eager
forward on the same inputs, bit for bit.  Each graph is replayed several
times, with the program's own eager work (other forwards, unrelated device
writes, synchronisations) between replays and new inputs copied into the
captured buffers before some of them, so state a launch leaves behind
(counters, flags, workspace contents) cannot carry from one replay into the
next unnoticed."""
import pytest
import torch

from synth import make_attention_residual, make_tokens
from tests.gpu_harness import make_case, spec_of
from top_routing_grouped_amd import moe

pytestmark = pytest.mark.gpu

CASES = [
    ("qwen_decode", 8, {}),  # small T, selection folded into gate/up, fused down + combine
    ("qwen_u4", 37, {}),  # small T, 4-bit, separate selection
    ("qwen_decode", 300, {}),  # medium T, 16-token tiles
    ("qwen_decode", 1500, {}),  # large T: tiled router, chunked permute, persistent GEMMs, aux-stream fork
    ("sigmoid_group", 301, dict(n_group=4, topk_group=2)),
]
DIMS = dict(d_model=256, n_experts=32, top_k=4, d_ff=128, d_ff_shared=128)


def _bufs(spec):
    T = spec.n_tokens
    return (torch.empty(T, spec.d_model, dtype=torch.float32, device="cuda"),
            torch.empty(T, spec.top_k, dtype=torch.int32, device="cuda"),
            torch.empty(T, spec.top_k, dtype=torch.float32, device="cuda"))


@pytest.mark.parametrize("name,T,extra", CASES)
def test_layer_forward_graph_replays(name, T, extra):
    spec = spec_of(name, n_tokens=T, **DIMS, **extra)
    case = make_case(spec, cache_key=("graph", name, T))
    cfg = moe.config_from_spec(spec)
    w = moe.weights_struct(case.w)
    ws = moe.alloc_workspace(cfg)
    x, r = case.x.clone(), case.r.clone()
    out, ids, wts = _bufs(spec)
    s, aux = torch.cuda.Stream(), torch.cuda.Stream()

    def eager(xi, ri):
        o, i, ww = _bufs(spec)
        ews = moe.alloc_workspace(cfg)
        moe.layer_forward(cfg, w, xi, ri, o, i, ww, ews, stream=torch.cuda.current_stream(), aux_stream=aux)
        torch.cuda.synchronize()
        return o, i, ww

    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up: the library creates its fork/join events
        moe.layer_forward(cfg, w, x, r, out, ids, wts, ws, stream=s, aux_stream=aux)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.layer_forward(cfg, w, x, r, out, ids, wts, ws, stream=s, aux_stream=aux)
    torch.cuda.synchronize()

    inputs = [(case.x, case.r)] + [make_tokens(spec, "cuda", seed=77 + i) for i in range(2)]
    for rep in range(4):
        xi, ri = inputs[rep % len(inputs)]
        x.copy_(xi)
        r.copy_(ri)
        out.fill_(float("nan"))
        ids.fill_(-7)
        ws.fill_(0xAB)  # scribble over the workspace between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o, i, ww = eager(xi, ri)  # eager work between replays, on fresh buffers
        assert torch.equal(ids, i), f"replay {rep}: ids differ"
        assert torch.equal(wts.view(torch.int32), ww.view(torch.int32)), f"replay {rep}: weights differ"
        assert torch.equal(out.view(torch.int32), o.view(torch.int32)), f"replay {rep}: out differs"


@pytest.mark.parametrize("T", [8, 300])
def test_layer_forward_norm_graph_replays(T):
    spec = spec_of("qwen_decode", n_tokens=T, **DIMS)
    case = make_case(spec, cache_key=("graph_norm", T))
    cfg = moe.config_from_spec(spec)
    w = moe.weights_struct(case.w)
    ws = moe.alloc_workspace(cfg)
    res, nw = make_attention_residual(spec, "cuda")
    res = res.clone()
    out, ids, wts = _bufs(spec)
    s = torch.cuda.Stream()
    eps = 1e-6
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe.layer_forward_norm(cfg, w, nw, eps, res, out, ids_out=ids, weights_out=wts, ws=ws, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.layer_forward_norm(cfg, w, nw, eps, res, out, ids_out=ids, weights_out=wts, ws=ws, stream=s)
    torch.cuda.synchronize()
    for rep in range(4):
        ri = res.clone() if rep % 2 == 0 else res * 0.5 + 0.25
        res.copy_(ri)
        out.fill_(float("nan"))
        ws.fill_(0x5C)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o, i, ww = _bufs(spec)
        moe.layer_forward_norm(cfg, w, nw, eps, ri, o, ids_out=i, weights_out=ww,
                               ws=moe.alloc_workspace(cfg), stream=torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(ids, i) and torch.equal(out.view(torch.int32), o.view(torch.int32)), f"replay {rep}"
