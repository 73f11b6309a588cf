#!/usr/bin/env python3
"""Throughput of one sparse-MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one whole layer forward (routing, permute, routed gate/up +
SwiGLU, routed down x alpha, shared expert, combine + residual) over one
batch of T tokens, launched as one captured HIP graph of the library's
moe_layer_forward.  Steps rotate over L layer instances that are distinct
device copies of the seeded weights, each with its own seeded tokens (so
the routing differs per instance and no instance's weights stay cached in
the 256 MB last-level cache).  Inputs are resident in HBM before the timed
region, which is bracketed by device synchronisation and HIP events.

Prints one JSON line: tokens/s of the Qwen3.6-35B-A3B layer at decode shape
(T = 8), the roofline of its dominant kernel (routed gate/up GEMM as the layer
launches it, timed with HIP events over re-launches on the same routing),
the fp64 oracle timed on the host cores on a bounded sample, and the
T = 4096 skewed prefill layer as a secondary entry.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from synth import WORKLOAD_TOKENS, WORKLOADS, make_attention_residual, make_tokens, make_weights  # noqa: E402
from top_routing_grouped_amd import moe  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE layer tokens/s, Qwen3.6 shape at T=8 and T=4096; % of HBM / MFMA roofline"
BYTES_PER_PARAM = {"f32": 4.0, "bf16": 2.0, "u4": 0.5 + 4.0 / 64}
NORM_EPS = 1e-6  # RMS-norm epsilon of the chained layers (the pages give none)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def clone_weights(w):
    import copy
    c = copy.copy(w)
    c.router = w.router.clone()
    c.expert_bias = None if w.expert_bias is None else w.expert_bias.clone()
    for name in ("gate", "up", "down", "shared_gate", "shared_up", "shared_down"):
        m = getattr(w, name)
        if m is not None:
            mm = copy.copy(m)
            mm.w = m.w.clone()
            mm.scale = None if m.scale is None else m.scale.clone()
            mm.min = None if m.min is None else m.min.clone()
            setattr(c, name, mm)
    c.shared_gate_vec = None if w.shared_gate_vec is None else w.shared_gate_vec.clone()
    return c


class Instance:
    def __init__(self, spec, w, seed):
        self.spec = spec
        self.w = w
        self.ws_struct = moe.weights_struct(w)
        self.x, self.r = make_tokens(spec, "cuda", seed=seed)
        self.cfg = moe.config_from_spec(spec)
        self.ws = moe.alloc_workspace(self.cfg)
        self.out = torch.empty_like(self.r)
        self.ids = torch.empty(spec.n_tokens, spec.top_k, dtype=torch.int32, device="cuda")
        self.wts = torch.empty(spec.n_tokens, spec.top_k, dtype=torch.float32, device="cuda")
        self.graph = None
        self.direct = False  # the direct (per-pair) schedule instead of the grouped one

    def forward(self, aux):
        if self.direct:
            moe.layer_forward_direct(self.cfg, self.ws_struct, self.x, self.r, self.out, self.ids, self.wts, self.ws)
        else:
            moe.layer_forward(self.cfg, self.ws_struct, self.x, self.r, self.out, self.ids, self.wts, self.ws,
                              aux_stream=aux)

    def stage(self, stage):
        moe.layer_stage(self.cfg, self.ws_struct, self.x, stage, self.ws)

    def n_active(self):
        return int(np.unique(self.ids.cpu().numpy()).size)


def layer_bytes(spec, n_active):
    T, D, E, F, Fs = spec.n_tokens, spec.d_model, spec.n_experts, spec.d_ff, spec.d_ff_shared
    bw = BYTES_PER_PARAM[spec.expert_dtype]
    br = 4.0 if spec.router_dtype == "f32" else 2.0
    bx = 4.0 if spec.act_dtype == "f32" else 2.0
    gate_vec = D * br if spec.shared_gate and Fs else 0
    return E * D * br + n_active * 3 * D * F * bw + 3 * D * Fs * bw + gate_vec + T * D * bx + 2 * T * D * 4


def layer_flops(spec):
    T, D, E, K, F, Fs = spec.n_tokens, spec.d_model, spec.n_experts, spec.top_k, spec.d_ff, spec.d_ff_shared
    return 2.0 * T * (E * D + K * 3 * D * F + 3 * D * Fs + (D if spec.shared_gate and Fs else 0))


def shared_in_routed_launch(spec):
    """Small T*K: the library runs the shared expert inside the routed launches
    (its small-T path: T*K <= 256 pairs and fewer than 16 pairs per expert on
    average for bf16 banks, 64 for 4-bit and fp32 banks)."""
    T, K, E = spec.n_tokens, spec.top_k, spec.n_experts
    per_expert = 16 if spec.expert_dtype == "bf16" else 64
    return T * K <= 256 and T * K < per_expert * E and spec.d_ff_shared > 0


def gateup_bytes(spec, n_active):
    """Algorithmic bytes of one routed gate/up launch: the active experts' gate
    and up matrices read once (plus the shared expert's when the launch carries
    it), the token rows read, the bf16 SwiGLU rows written."""
    T, D, K, F, Fs = spec.n_tokens, spec.d_model, spec.top_k, spec.d_ff, spec.d_ff_shared
    bw = BYTES_PER_PARAM[spec.expert_dtype]
    shared = shared_in_routed_launch(spec)
    return (n_active * 2 * D * F * bw + (2 * D * Fs * bw if shared else 0) + T * D * 2
            + (T * K * F + (T * Fs if shared else 0)) * 2)


def gateup_flops(spec):
    shared = shared_in_routed_launch(spec)
    return 2.0 * spec.n_tokens * 2 * spec.d_model * (spec.top_k * spec.d_ff + (spec.d_ff_shared if shared else 0))


def build_instances(spec, L, log_prefix):
    t0 = time.time()
    base = make_weights(spec, "cuda")
    ws = [base] + [clone_weights(base) for _ in range(L - 1)]
    torch.cuda.synchronize()
    tok_seed = 1000 * spec.workload_id + spec.n_tokens
    insts = [Instance(spec, w, tok_seed + 7919 * i) for i, w in enumerate(ws)]
    log(f"{log_prefix}: {L} instances built in {time.time() - t0:.1f}s "
        f"({torch.cuda.memory_allocated() / 2**30:.1f} GiB on device)")
    return insts


def chain_length(steps, L):
    """Layers per captured chain: the largest divisor of `steps` not above L,
    so that exactly `steps` forwards run as whole chains."""
    return max(d for d in range(1, min(L, steps) + 1) if steps % d == 0)


def capture_chain(insts, aux, cap):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for inst in insts:
            inst.forward(aux)
    return g


def time_layer(insts, steps, warmup, protocol_chains=20):
    """Per-layer time of the layer forward, measured two ways.

    Timed region: exactly `steps` forwards, run as whole captured chains of
    Lc = chain_length(steps, L) distinct instances (a decoder stack's launch
    pattern) after at least 5 warm-up chains (or `warmup` forwards, whichever
    is more), bracketed by synchronisation and HIP events.  Protocol
    measurement (outside the timed region): `protocol_chains` replays of the
    chain of all L instances, each timed alone; the median is reported.
    Replays of both graphs are first checked bit for bit against the eager
    forwards."""
    aux = torch.cuda.Stream()
    # eager warm-up (creates the library's fork/join events), then capture
    for inst in insts:
        inst.forward(aux)
    torch.cuda.synchronize()
    ref_out = [inst.out.clone() for inst in insts]
    cap = torch.cuda.Stream()
    L = len(insts)
    Lc = chain_length(steps, L)
    full = capture_chain(insts, aux, cap)
    part = full if Lc == L else capture_chain(insts[:Lc], aux, cap)
    for inst in insts:  # single-layer graphs for the isolated and cold latencies
        inst.graph = capture_chain([inst], aux, cap)
    torch.cuda.synchronize()
    for g, n in ((full, L), (part, Lc), (full, L)):
        for inst in insts:
            inst.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for inst, ref in zip(insts[:n], ref_out):
            if not torch.equal(inst.out.view(torch.int32), ref.view(torch.int32)):
                raise RuntimeError("graph replay differs from the eager forward")
    for _ in range(max(5, -(-warmup // Lc))):
        part.replay()
    torch.cuda.synchronize()
    n_chain = steps // Lc
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n_chain):
        part.replay()
    end.record()
    torch.cuda.synchronize()
    total = start.elapsed_time(end) / steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(protocol_chains + 1)]
    evs[0].record()
    for c in range(protocol_chains):
        full.replay()
        evs[c + 1].record()
    torch.cuda.synchronize()
    per_chain = sorted(evs[c].elapsed_time(evs[c + 1]) / L for c in range(protocol_chains))
    return {"ms": total, "chain_layers": Lc, "chains_timed": n_chain,
            "median_ms": per_chain[len(per_chain) // 2], "protocol_chains": protocol_chains, "protocol_layers": L}


def single_layer_ms(insts, reps=10, flush_bytes=0):
    """Latency of one layer launched alone (its single-layer graph) after the
    GPU has drained: median over `reps` instances.  With flush_bytes, a buffer
    of that size (never written, so none of its lines is dirty) is read first:
    it evicts the layer's data from the last-level cache and replaces the TLB
    entries of the weights.  (A flush that writes the buffer leaves the cache
    full of dirty lines, and the layer then pays for writing them back: 142
    against 90 us at decode T = 8.)"""
    flush = torch.empty(max(flush_bytes, 4) // 4, dtype=torch.float32, device="cuda")
    times = []
    for i in range(reps):
        inst = insts[i % len(insts)]
        if flush_bytes:
            flush.amax()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        inst.graph.replay()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    del flush
    return sorted(times)[len(times) // 2]


def time_stage(insts, stage, reps, repeats=5, spread=None):
    """Average duration of one stage launch (or of a sequence of stage
    launches, given a tuple), re-launched `reps` times in one captured graph
    over the instances' real routing; HIP events on the replay stream.  The
    graph is replayed `repeats` times after a warm-up replay and the median
    replay is returned (a list passed as `spread` receives every replay's
    per-launch time)."""
    L = len(insts)
    stages = stage if isinstance(stage, tuple) else (stage,)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for i in range(reps):
            for st in stages:
                insts[i % L].stage(st)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    per = []
    for _ in range(max(1, repeats)):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        g.replay()
        end.record()
        torch.cuda.synchronize()
        per.append(start.elapsed_time(end) / reps)
    if spread is not None:
        spread.extend(per)
    return float(np.median(per))


def source_hash():
    """Hash of what the library's machine code is built from: the HIP and C++
    sources, the public header and the build options."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "top_routing_grouped_amd")
    csrc = os.path.join(pkg, "csrc")
    inc = os.path.join(ROOT, "include")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    files += [os.path.join(inc, f) for f in sorted(os.listdir(inc))]
    files.append(os.path.join(pkg, "build.py"))
    for p in files:
        with open(p, "rb") as fh:
            h.update(os.path.relpath(p, ROOT).encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_record(kernel_key, workload, launch_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel and workload, if it was taken from the current sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        recs = json.load(f)
    rec = recs.get(f"{kernel_key}/{workload}")
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def host_description():
    """CPU model, the BLAS library NumPy uses, and the thread count the oracle
    runs with: the cores this process may run on (its affinity mask), capped
    by OMP_NUM_THREADS when that is set (the CPU share of a shared host)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        cores = min(cores, int(omp))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "blas": blas, "cores": cores}


def cpu_baseline(inst, seconds):
    """The fp64 oracle (as it stands) on the host cores: full layer forwards
    over instance 0's tokens, repeated for about `seconds` (at least once),
    with BLAS limited to the cores host_description() reports."""
    from oracle import moe_oracle as O
    from oracle.inputs import banks_from, widen_tensor
    host = host_description()
    spec = inst.spec
    host_w = clone_weights_to_host(inst.w)
    banks = banks_from(host_w, lazy=True)
    x64, r64 = widen_tensor(inst.x), widen_tensor(inst.r)
    wr = widen_tensor(host_w.router)
    bias = None if host_w.expert_bias is None else widen_tensor(host_w.expert_bias)
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=host["cores"], user_api="blas")
    except Exception:  # pragma: no cover
        limiter = None
    reps, t0 = 0, time.time()
    while True:
        O.layer_forward(x64, r64, wr, banks, spec.family, spec.top_k, bias, spec.n_group, spec.topk_group,
                        spec.routed_scaling)
        reps += 1
        if time.time() - t0 >= seconds:
            break
    dt = time.time() - t0
    if limiter is not None:
        limiter.unregister()
    return {"value": reps * spec.n_tokens / dt, "unit": "tokens/s", "cores": host["cores"], "kind": "oracle",
            "cpu_model": host["cpu_model"], "blas": host["blas"],
            "sample": f"{reps} full layer forwards of the same workload (T={spec.n_tokens}) in float64 NumPy, "
                      f"{dt:.1f} s wall clock; weights widened from bf16 per expert inside each call"}


def clone_weights_to_host(w):
    import copy
    c = copy.copy(w)
    c.router = w.router.cpu()
    c.expert_bias = None if w.expert_bias is None else w.expert_bias.cpu()
    for name in ("gate", "up", "down", "shared_gate", "shared_up", "shared_down"):
        m = getattr(w, name)
        if m is not None:
            mm = copy.copy(m)
            mm.w = m.w.cpu()
            mm.scale = None if m.scale is None else m.scale.cpu()
            mm.min = None if m.min is None else m.min.cpu()
            setattr(c, name, mm)
    c.shared_gate_vec = None if w.shared_gate_vec is None else w.shared_gate_vec.cpu()
    return c


def copy_calibration(nbytes=1 << 30):
    """One device-to-device copy of `nbytes` (reads and writes nbytes each),
    whose counter readings scale FETCH_SIZE / WRITE_SIZE to bytes."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy calibration: {nbytes} bytes")


def stream_ops(src, dst, out):
    """(name, launch, bytes moved) of the streaming reference: a copy of src
    into dst, and a sum of src into the 0-d tensor out."""
    n = src.numel() * src.element_size()
    return (("copy", lambda: dst.copy_(src), 2 * n), ("read", lambda: torch.sum(src, dim=0, out=out), n))


def hbm_reference(nbytes=1 << 30, reps=10):
    """The chip's streaming rate, as a reference for the roofline fractions:
    through torch's kernels a device-to-device copy of `nbytes` (reads and
    writes nbytes) and a read-only pass (a sum over `nbytes` of fp32), each
    over distinct buffers larger than the 256 MB last-level cache; and the
    library's streaming read (moe_stream_read) of the same buffer and of a
    128 MiB slice of it read again (served by the last-level cache); HIP
    events around the launches."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    out = torch.empty((), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    res = {}
    for name, fn, moved in stream_ops(src, dst, out):
        fn()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        res[f"{name}_GBps"] = round(moved * reps / (s.elapsed_time(e) / 1e3) / 1e9, 1)
    # the library's own streaming read (whole 128-byte lines per request, eight
    # 16-byte loads per lane in flight): from HBM over the 1 GiB buffer, and
    # from the last-level cache over a 128 MiB slice read again
    sink = torch.empty(nbytes // 1024, dtype=torch.int32, device="cuda")
    llc = src[: (128 << 20) // 4]
    for name, buf, n in (("stream_read", src, reps), ("llc_read", llc, 4 * reps)):
        moe.stream_read(buf, sink)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            moe.stream_read(buf, sink)
        e.record()
        torch.cuda.synchronize()
        res[f"{name}_GBps"] = round(buf.numel() * 4 * n / (s.elapsed_time(e) / 1e3) / 1e9, 1)
    res["llc_bytes"] = 128 << 20
    # one launch per 256 MiB slice, the slices in turn (each read from HBM): a
    # read of about the decode gate/up's bytes, its launch ramp and tail included
    q = (256 << 20) // 4
    slices = [src[i * q:(i + 1) * q] for i in range(src.numel() // q)]
    if slices:
        moe.stream_read(slices[-1], sink)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 4 * reps
        s.record()
        for i in range(n):
            moe.stream_read(slices[i % len(slices)], sink)
        e.record()
        torch.cuda.synchronize()
        res["stream_read_256MiB_GBps"] = round((256 << 20) * n / (s.elapsed_time(e) / 1e3) / 1e9, 1)
    del src, dst, sink, llc, slices
    torch.cuda.empty_cache()
    res["bytes"] = nbytes
    return res


MFMA_SHAPES = ((0, "16x16x32_bf16", 2 * 16 * 16 * 32), (1, "32x32x16_bf16", 2 * 32 * 32 * 16))


def mfma_reference(reps=5):
    """The chip's bf16 MFMA issue rate, as a reference for the MFMA fractions:
    the library's issue-rate loop (moe_mfma_rate: 8 independent accumulator
    chains per wave, back-to-back MFMAs) for the 16x16x32 shape the grouped
    GEMMs use and for 32x32x16, with one wave on each SIMD (256 workgroups of
    4 waves) and two; about a millisecond per launch, HIP events around
    `reps` launches after a warm-up one."""
    res = {}
    for shape, name, flops in MFMA_SHAPES:
        iters = 20000 if shape == 0 else 10000
        for wgs, label in ((256, "1_wave_per_simd"), (512, "2_waves_per_simd")):
            sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
            moe.mfma_rate(shape, wgs, iters, sink)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                moe.mfma_rate(shape, wgs, iters, sink)
            e.record()
            torch.cuda.synchronize()
            total = wgs * 4 * iters * 8 * flops * reps
            res[f"mfma_{name}_{label}_TFLOPs"] = round(total / (s.elapsed_time(e) / 1e3) / 1e12, 1)
    res["peak_TFLOPs"] = BF16_PEAK_TFLOPS
    return res


L2_PATTERNS = ((0, "row_segments"), (1, "mfma_operand_order"), (2, "row_quads"))
SHADER_CLOCK_GHZ = 2.4  # MI355X peak engine clock


def l2_read_reference(reps=5, iterations=32):
    """Vector-memory read rate from the L2 for the three lane-to-address
    patterns of the library's L2 read loop (moe_l2_read_rate: 16-byte loads,
    each wave 64 KB of 4 KB rows per pass, a 1 MiB set every XCD's L2 holds):
    eight consecutive lanes per 128-byte line, the 16x16x32 MFMA operand
    order, and four consecutive lanes per 64-byte segment; 4 and 16 waves per
    compute unit (256 and 1024 workgroups).  Bytes per clock per compute unit
    at the peak engine clock, HIP events around `reps` launches after a
    warm-up one."""
    buf = torch.zeros(1 << 18, dtype=torch.int32, device="cuda")
    res = {}
    for wgs, label in ((256, "4_waves_per_cu"), (1024, "16_waves_per_cu")):
        sink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")
        for pattern, name in L2_PATTERNS:
            moe.l2_read_rate(pattern, wgs, iterations, buf, sink)
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                moe.l2_read_rate(pattern, wgs, iterations, buf, sink)
            e.record()
            torch.cuda.synchronize()
            nbytes = wgs * 4 * 65536 * iterations * reps
            per_s = nbytes / (s.elapsed_time(e) / 1e3)
            res[f"{name}_{label}_B_per_clk_per_CU"] = round(per_s / (SHADER_CLOCK_GHZ * 1e9 * 256), 1)
    res["clock_GHz"] = SHADER_CLOCK_GHZ
    return res


def run_workload(name, T, L, steps, warmup, stage_reps):
    spec = WORKLOADS[name].with_tokens(T)
    insts = build_instances(spec, L, f"{name} T={T}")
    tl = time_layer(insts, steps, warmup)
    ms, ms_median = tl["ms"], tl["median_ms"]
    alone_ms = single_layer_ms(insts)
    cold_ms = single_layer_ms(insts, flush_bytes=512 << 20)
    n_act = [inst.n_active() for inst in insts]
    mean_act = float(np.mean(n_act))
    byts = float(np.mean([layer_bytes(spec, a) for a in n_act]))
    flops = layer_flops(spec)
    t = ms / 1e3
    # the routed gate/up launch the layer runs (selection folded in where the
    # layer folds it), re-launched back to back over the instances' routing
    stage_spread = []
    stage_ms = time_stage(insts, moe.STAGE_GATE_UP, stage_reps, spread=stage_spread)
    gu_bytes = float(np.mean([gateup_bytes(spec, a) for a in n_act]))
    gu_flops = gateup_flops(spec)
    gu_t = stage_ms / 1e3
    t_hbm, t_mfma = byts / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
    res = {
        "spec": spec, "insts": insts, "ms_per_step": ms, "tokens_per_s": T / t,
        "median_chain_us_per_layer": ms_median * 1e3, "cold_layer_us": cold_ms * 1e3,
        "alone_layer_us": alone_ms * 1e3, "timing": tl,
        "mfma_ceiling": t_mfma / max(t_hbm, t_mfma),
        "n_active_mean": mean_act, "layer_bytes": byts, "layer_flops": flops,
        "layer_hbm_frac": byts / t / (HBM_PEAK_GBS * 1e9), "layer_mfma_frac": flops / t / (BF16_PEAK_TFLOPS * 1e12),
        "gateup_ms": stage_ms, "gateup_spread_ms": stage_spread, "gateup_bytes": gu_bytes, "gateup_flops": gu_flops,
        "gateup_gbs": gu_bytes / gu_t / 1e9, "gateup_tflops": gu_flops / gu_t / 1e12,
    }
    log(f"{name} T={T}: {ms * 1e3:.1f} us/layer, {T / t:,.0f} tok/s, n_active {mean_act:.1f}, "
        f"layer {byts / t / 1e9:,.0f} GB/s ({res['layer_hbm_frac']:.1%} HBM), "
        f"{flops / t / 1e12:.1f} TFLOP/s ({res['layer_mfma_frac']:.1%} MFMA, ceiling {res['mfma_ceiling']:.1%}); "
        f"{tl['chains_timed']} chains of {tl['chain_layers']} timed; median of {tl['protocol_chains']} chains of "
        f"{tl['protocol_layers']} {ms_median * 1e3:.1f} us/layer; single layer alone {alone_ms * 1e3:.1f} us, "
        f"after a cache flush {cold_ms * 1e3:.1f} us; gate/up {stage_ms * 1e3:.1f} us = "
        f"{res['gateup_gbs']:,.0f} GB/s, {res['gateup_tflops']:.1f} TFLOP/s")
    return res


def time_chain(spec, L, steps, warmup):
    """A stack of L distinct layers at one token count, each starting from the
    attention residual: layer l normalises r_l (its own RMS-norm weight) and
    writes r_(l+1) = r_l + y_moe, which layer l+1 reads.  One workspace serves
    every layer (calls are ordered on one stream).  Captured as one graph;
    returns us per layer (mean over the timed replays) and the median replay."""
    t0 = time.time()
    base = make_weights(spec, "cuda")
    ws_list = [base] + [clone_weights(base) for _ in range(L - 1)]
    structs = [moe.weights_struct(w) for w in ws_list]
    r0, _ = make_attention_residual(spec, "cuda")
    gammas = [make_attention_residual(spec.with_tokens(1), "cuda", weight_seed=1000 * spec.workload_id + 999 + l)[1]
              for l in range(L)]
    bufs = [r0] + [torch.empty_like(r0) for _ in range(L)]
    cfg = moe.config_from_spec(spec)
    wsp = moe.alloc_workspace(cfg)

    def run():
        for l in range(L):
            moe.layer_forward_norm(cfg, structs[l], gammas[l], NORM_EPS, bufs[l], bufs[l + 1], ws=wsp)

    run()
    torch.cuda.synchronize()
    ref = bufs[L].clone()
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        run()
    for _ in range(2):
        bufs[L].fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(bufs[L].view(torch.int32), ref.view(torch.int32)):
            raise RuntimeError("chained graph replay differs from the eager chain")
    log(f"chain of {L} layers (T={spec.n_tokens}) built in {time.time() - t0:.1f}s")
    for _ in range(max(1, warmup // L)):
        g.replay()
    torch.cuda.synchronize()
    n = max(1, steps // L)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    evs[0].record()
    for i in range(n):
        g.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) / L for i in range(n))
    total = evs[0].elapsed_time(evs[-1]) / (n * L)
    del g, ws_list, structs, bufs
    torch.cuda.empty_cache()
    return total * 1e3, per[len(per) // 2] * 1e3


def norm_bytes(spec):
    """Algorithmic bytes of one RMS-norm launch: the fp32 residual read, x
    written in the activation type, the fp32 weight read."""
    T, D = spec.n_tokens, spec.d_model
    return T * D * 4 + T * D * (4 if spec.act_dtype == "f32" else 2) + D * 4


def time_norm(spec, reps, rotate_bytes=384 << 20):
    """Average duration of one moe_rms_norm launch (captured graph of `reps`
    launches over enough distinct residual buffers to exceed the last-level
    cache), HIP events on the replay stream."""
    r, w = make_attention_residual(spec, "cuda")
    nbuf = max(1, min(reps, -(-rotate_bytes // r.numel() // 4)))
    rs = [r] + [r * (1.0 + 1e-3 * i) for i in range(1, nbuf)]
    x = torch.empty(r.shape, device="cuda", dtype=torch.float32 if spec.act_dtype == "f32" else torch.bfloat16)
    cfg = moe.config_from_spec(spec)
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for i in range(reps):
            moe.rms_norm(cfg, rs[i % nbuf], w, NORM_EPS, x)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    del rs, g
    torch.cuda.empty_cache()
    gbs = norm_bytes(spec) / (ms / 1e3) / 1e9
    rec = {"kernel": "RMS norm of the attention residual", "n_tokens": spec.n_tokens, "launch_us": round(ms * 1e3, 2),
           "algorithmic_bytes": norm_bytes(spec), "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(gbs / HBM_PEAK_GBS, 4), "bound": "hbm"}
    if spec.n_tokens == 4096:
        rec["traffic"] = traffic_record("rms_norm", "qwen_T4096", norm_bytes(spec))
    return rec


def chained_decode(args, dec_us):
    """Entry for the 40-layer chain at decode shape with the normalisation in
    each layer, beside the RMS-norm launch measured alone (T = 8 and 4096)."""
    spec = WORKLOADS["qwen_decode"].with_tokens(8)
    L = args.instances
    us, us_med = time_chain(spec, L, args.steps, args.warmup)
    n8 = time_norm(spec, args.stage_reps)
    n4k = time_norm(WORKLOADS["qwen_prefill_skew"].with_tokens(4096), max(8, args.stage_reps // 4))
    log(f"chain: {us:.1f} us/layer (median replay {us_med:.1f}) with the norm; independent layers {dec_us:.1f}; "
        f"norm alone {n8['launch_us']:.1f} us at T=8, {n4k['launch_us']:.1f} us = {n4k['achieved']:,.0f} GB/s "
        f"at T=4096")
    return {"workload": f"{L} chained Qwen3.6-35B-A3B MoE layers at T=8: each normalises the attention residual "
                        f"(RMS norm, eps {NORM_EPS:g}, per-layer weight) and feeds r + y_moe to the next",
            "layers": L, "us_per_layer": round(us, 2), "median_replay_us_per_layer": round(us_med, 2),
            "tokens_per_s": round(8 / (us * 1e-6), 1),
            "independent_layers_us_per_layer": round(dec_us, 2),
            "norm_T8": n8, "norm_T4096": n4k}


def prefill_roofline(pre):
    """Roofline of the prefill gate/up launch, bound chosen by its algorithmic
    intensity against the chip's ridge point (bf16 MFMA peak / HBM peak)."""
    intensity = pre["gateup_flops"] / pre["gateup_bytes"]
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma = {"achieved": round(pre["gateup_tflops"], 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre["gateup_tflops"] / BF16_PEAK_TFLOPS, 4)}
    hbm = {"achieved": round(pre["gateup_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(pre["gateup_gbs"] / HBM_PEAK_GBS, 4)}
    bound, other = ("mfma", hbm) if intensity > ridge else ("hbm", mfma)
    r = {"kernel": "routed gate/up GEMM + SwiGLU", "bound": bound}
    r.update(mfma if bound == "mfma" else hbm)
    r.update({"intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1),
              "other": other, "launch_us": round(pre["gateup_ms"] * 1e3, 2),
              "algorithmic_bytes": round(pre["gateup_bytes"]), "algorithmic_flops": round(pre["gateup_flops"]),
              "traffic": traffic_record("gateup", "qwen_prefill_T4096", pre["gateup_bytes"])})
    return r


def crossover(args):
    """Direct execution (every (token, slot) pair its own work item, reading
    its expert's weights) against grouped execution (the pairs of an expert
    share one read of its weights) at decode shape, on the same routing: the
    whole layer (moe_layer_forward_direct against moe_layer_forward, each as
    captured chains of the 40 instances) and the routed gate/up stage alone.
    Prints one JSON line per T with the bytes the two would move without
    caches and the measured times."""
    for T in (1, 2, 3, 4, 6, 8, 16, 32):
        spec = WORKLOADS["qwen_decode"].with_tokens(T)
        insts = build_instances(spec, min(args.instances, 40), f"crossover T={T}")
        grouped = time_layer(insts, args.steps, args.warmup)
        g_stage = time_stage(insts, moe.STAGE_GATE_UP, args.stage_reps)
        d_stage = time_stage(insts, moe.STAGE_GATE_UP_DIRECT, args.stage_reps)
        dn = {k: time_stage(insts, st, args.stage_reps) for k, st in
              (("fused", moe.STAGE_DOWN), ("grouped", moe.STAGE_DOWN_GROUPED), ("direct", moe.STAGE_DOWN_DIRECT))}
        g_ids = [inst.ids.clone() for inst in insts]
        for inst in insts:
            inst.direct = True
        direct = time_layer(insts, args.steps, args.warmup)
        if not all(torch.equal(a, inst.ids) for a, inst in zip(g_ids, insts)):
            raise RuntimeError("direct and grouped schedules selected different experts")
        n_act = float(np.mean([inst.n_active() for inst in insts]))
        wb = 3 * spec.d_model * spec.d_ff * BYTES_PER_PARAM[spec.expert_dtype]
        line = {"study": "layer, direct vs grouped", "n_tokens": T, "pairs": T * spec.top_k,
                "n_active_mean": round(n_act, 2), "routed_weight_bytes_grouped": round(n_act * wb),
                "routed_weight_bytes_direct_uncached": round(T * spec.top_k * wb),
                "grouped_us_per_layer": round(grouped["ms"] * 1e3, 2),
                "direct_us_per_layer": round(direct["ms"] * 1e3, 2),
                "grouped_median_us": round(grouped["median_ms"] * 1e3, 2),
                "direct_median_us": round(direct["median_ms"] * 1e3, 2),
                "direct_over_grouped": round(direct["median_ms"] / grouped["median_ms"], 3),
                "gate_up_stage_grouped_us": round(g_stage * 1e3, 2), "gate_up_stage_direct_us": round(d_stage * 1e3, 2),
                "down_stage_fused_combine_us": round(dn["fused"] * 1e3, 2),
                "down_stage_grouped_us": round(dn["grouped"] * 1e3, 2),
                "down_stage_direct_us": round(dn["direct"] * 1e3, 2)}
        print(json.dumps(line), flush=True)
        log(f"T={T}: layer grouped {line['grouped_median_us']} us, direct {line['direct_median_us']} us "
            f"({line['direct_over_grouped']}x); gate/up stage {line['gate_up_stage_grouped_us']} / "
            f"{line['gate_up_stage_direct_us']} us; down stage fused+combine / grouped / direct "
            f"{line['down_stage_fused_combine_us']} / {line['down_stage_grouped_us']} / {line['down_stage_direct_us']} us")
        del insts
        torch.cuda.empty_cache()


def all_configs(args):
    """One JSON line per workload and token count of the parity
    configurations, with the same protocol as the headline: chained graph
    over distinct layer instances (40 up to T = 512, 4 beyond), actual
    n_active, algorithmic bytes and flops, both roofline fractions, the
    attainable MFMA ceiling, the routed gate/up launch alone."""
    for name, Ts in WORKLOAD_TOKENS.items():
        for T in Ts:
            big = T > 512
            L = min(args.instances, 4) if big else args.instances
            steps = max(80, args.steps // 10) if big else args.steps
            warmup = max(20, args.warmup // 10) if big else args.warmup
            res = run_workload(name, T, L, steps, warmup, max(8, args.stage_reps // 4) if big else args.stage_reps)
            spec = res["spec"]
            print(json.dumps({
                "workload": name, "n_tokens": T, "d_model": spec.d_model, "n_experts": spec.n_experts,
                "top_k": spec.top_k, "d_ff": spec.d_ff, "d_ff_shared": spec.d_ff_shared, "routing": spec.family,
                "expert_dtype": spec.expert_dtype, "layer_instances": L,
                "us_per_layer": round(res["ms_per_step"] * 1e3, 2), "tokens_per_s": round(res["tokens_per_s"], 1),
                "median_chain_us_per_layer": round(res["median_chain_us_per_layer"], 2),
                "cold_layer_us": round(res["cold_layer_us"], 2), "n_active_mean": round(res["n_active_mean"], 2),
                "layer_algorithmic_bytes": round(res["layer_bytes"]),
                "layer_algorithmic_flops": round(res["layer_flops"]),
                "layer_hbm_frac": round(res["layer_hbm_frac"], 4), "layer_mfma_frac": round(res["layer_mfma_frac"], 4),
                "mfma_ceiling": round(res["mfma_ceiling"], 4), "gateup_us": round(res["gateup_ms"] * 1e3, 2),
                "gateup_hbm_frac": round(res["gateup_gbs"] / HBM_PEAK_GBS, 4),
                "gateup_mfma_frac": round(res["gateup_tflops"] / BF16_PEAK_TFLOPS, 4)}), flush=True)
            del res
            torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--instances", type=int, default=40)
    ap.add_argument("--stage-reps", type=int, default=64)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="profiling aid: finish with a 1 GiB device-to-device copy (known bytes for counter scaling)")
    ap.add_argument("--crossover", action="store_true",
                    help="small-T study: the layer (and its gate/up stage) with one work item per (token, slot) "
                         "pair versus grouped by expert, T = 1..32 at decode shape; one JSON line per T")
    ap.add_argument("--no-chain", action="store_true")
    ap.add_argument("--configs", action="store_true",
                    help="one JSON line per parity configuration (every workload and token count)")
    ap.add_argument("--workload", default=None, help="with --tokens: run this one workload (profiling aid)")
    ap.add_argument("--tokens", type=int, default=None)
    ap.add_argument("--only", choices=["decode", "prefill", "chain"], default=None,
                    help="profiling aid: run one workload and print its log line only")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    moe.lib()

    if args.crossover:
        crossover(args)
        return
    if args.configs:
        all_configs(args)
        return
    if args.workload:
        T = args.tokens or WORKLOADS[args.workload].n_tokens
        big = T > 512
        run_workload(args.workload, T, min(args.instances, 4) if big else args.instances, args.steps, args.warmup,
                     args.stage_reps)
        if args.copy_calibration:
            copy_calibration()
        return
    if args.only == "chain":
        chained_decode(args, float("nan"))
        if args.copy_calibration:
            copy_calibration()
        return
    if args.only == "prefill":
        run_workload("qwen_prefill_skew", 4096, min(args.instances, 4), args.steps, args.warmup, args.stage_reps)
        if args.copy_calibration:
            copy_calibration()
        return
    dec = run_workload("qwen_decode", 8, args.instances, args.steps, args.warmup, args.stage_reps)
    if args.only == "decode":
        if args.copy_calibration:
            copy_calibration()
        return
    spec = dec["spec"]
    gu_traffic = traffic_record("gateup", "qwen_decode_T8", dec["gateup_bytes"])
    line = {
        "metric": METRIC,
        "value": round(dec["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Qwen3.6-35B-A3B MoE layer forward, decode shape",
                   "n_tokens": 8, "d_model": spec.d_model, "n_experts": spec.n_experts, "top_k": spec.top_k,
                   "d_ff": spec.d_ff, "d_ff_shared": spec.d_ff_shared, "routing": "softmax top-k, 2^-14 clamp",
                   "shared_gate": True, "layer_instances": args.instances,
                   "n_active_mean": round(dec["n_active_mean"], 2),
                   "layer_algorithmic_bytes": round(dec["layer_bytes"]),
                   "layer_algorithmic_flops": round(dec["layer_flops"]),
                   "layer_hbm_frac": round(dec["layer_hbm_frac"], 4),
                   "layer_mfma_frac": round(dec["layer_mfma_frac"], 4),
                   "mfma_ceiling": round(dec["mfma_ceiling"], 4),
                   "timed_chain_layers": dec["timing"]["chain_layers"],
                   "timed_chains": dec["timing"]["chains_timed"],
                   "median_chain_us_per_layer": round(dec["median_chain_us_per_layer"], 2),
                   "median_over": f"{dec['timing']['protocol_chains']} chains of {dec['timing']['protocol_layers']} "
                                  f"layers, outside the timed region",
                   "alone_layer_us": round(dec["alone_layer_us"], 2),
                   "cold_layer_us": round(dec["cold_layer_us"], 2)},
        "roofline": {"kernel": "routed gate/up GEMM + SwiGLU (selection folded in, as the layer launches it)",
                     "bound": "hbm",
                     "achieved": round(dec["gateup_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec["gateup_gbs"] / HBM_PEAK_GBS, 4),
                     "traffic": gu_traffic, "launch_us": round(dec["gateup_ms"] * 1e3, 3),
                     "launch_us_measured_as": f"{args.stage_reps} re-launches of the layer's gate/up launch in a "
                                              "captured graph over the instances' routing, HIP events on its stream; "
                                              f"median of {len(dec['gateup_spread_ms'])} replays",
                     "launch_us_replays": [round(v * 1e3, 2) for v in dec["gateup_spread_ms"]],
                     "algorithmic_bytes": round(dec["gateup_bytes"])},
    }
    line["hbm_reference"] = hbm_reference()
    line["mfma_reference"] = mfma_reference()
    line["l2_read_reference"] = l2_read_reference()
    if not args.no_chain:
        line["chained_decode"] = chained_decode(args, dec["ms_per_step"] * 1e3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(dec["insts"][0], args.cpu_seconds)
    # the decode instances (40 layer copies, about 60 GB) are released before
    # the prefill workload is built
    del dec
    torch.cuda.empty_cache()
    if not args.no_prefill:
        pre = run_workload("qwen_prefill_skew", 4096, 4, max(80, args.steps // 10), max(20, args.warmup // 10),
                           max(8, args.stage_reps // 4))
        line["secondary"] = {
            "workload": "Qwen3.6-35B-A3B MoE layer forward, prefill T=4096, skewed routing",
            "value": round(pre["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(pre["ms_per_step"], 6), "n_active_mean": round(pre["n_active_mean"], 2),
            "layer_mfma_frac": round(pre["layer_mfma_frac"], 4), "layer_hbm_frac": round(pre["layer_hbm_frac"], 4),
            "mfma_ceiling": round(pre["mfma_ceiling"], 4), "layer_algorithmic_bytes": round(pre["layer_bytes"]),
            "layer_algorithmic_flops": round(pre["layer_flops"]),
            "timed_chain_layers": pre["timing"]["chain_layers"], "timed_chains": pre["timing"]["chains_timed"],
            "median_chain_us_per_layer": round(pre["median_chain_us_per_layer"], 2),
            "alone_layer_us": round(pre["alone_layer_us"], 2),
            "cold_layer_us": round(pre["cold_layer_us"], 2),
            "roofline": prefill_roofline(pre),
        }
        if not args.no_cpu_baseline:
            line["secondary"]["cpu_baseline"] = cpu_baseline(pre["insts"][0], args.cpu_seconds)
        del pre
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
