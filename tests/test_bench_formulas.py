"""The roofline denominators bench.py divides by, against the per-layer
formulas written out by hand: bytes = router E*D*b_r + each active expert's
three matrices once + the shared expert's + the gate vector + x + residual in
and out; flops = 2*T*(E*D + K*3*D*F + 3*D*F_s + D).  CPU only."""
import dataclasses
import subprocess
import sys

import pytest

bench = pytest.importorskip("bench")
from synth import WORKLOADS  # noqa: E402


def test_layer_flops_per_token_qwen():
    s = WORKLOADS["qwen_decode"].with_tokens(1)
    # 2 * (256*2048 + 8*3*2048*512 + 3*2048*512 + 2048) = 57.68 MFLOP per token
    assert bench.layer_flops(s) == 2 * (256 * 2048 + 8 * 3 * 2048 * 512 + 3 * 2048 * 512 + 2048) == 57675776


def test_layer_bytes_qwen_decode_and_u4():
    s = WORKLOADS["qwen_decode"].with_tokens(8)
    want = 256 * 2048 * 2 + 57 * 3 * 2048 * 512 * 2 + 3 * 2048 * 512 * 2 + 2048 * 2 + 8 * 2048 * 2 + 2 * 8 * 2048 * 4
    assert bench.layer_bytes(s, 57) == want
    u = WORKLOADS["qwen_u4"].with_tokens(64)
    bw = 0.5 + 4 / 64  # codes plus bf16 scale and min per 64 weights
    want = 256 * 2048 * 2 + 100 * 3 * 2048 * 512 * bw + 3 * 2048 * 512 * bw + 2048 * 2 + 64 * 2048 * 2 \
        + 2 * 64 * 2048 * 4
    assert bench.layer_bytes(u, 100) == pytest.approx(want, rel=1e-15)


def test_gateup_bytes_and_flops():
    s = WORKLOADS["qwen_decode"].with_tokens(8)  # small T: the launch also carries the shared expert
    assert bench.shared_in_routed_launch(s)
    assert bench.gateup_bytes(s, 57) == 57 * 2 * 2048 * 512 * 2 + 2 * 2048 * 512 * 2 + 8 * 2048 * 2 \
        + (8 * 8 * 512 + 8 * 512) * 2
    assert bench.gateup_flops(s) == 2 * 8 * 2 * 2048 * (8 * 512 + 512)
    p = WORKLOADS["qwen_prefill_skew"].with_tokens(4096)  # large T: shared expert on the aux stream
    assert not bench.shared_in_routed_launch(p)
    assert bench.gateup_bytes(p, 186) == 186 * 2 * 2048 * 512 * 2 + 4096 * 2048 * 2 + 4096 * 8 * 512 * 2
    assert bench.gateup_flops(p) == 2 * 4096 * 2 * 2048 * 8 * 512


def test_small_path_rule_matches_library():
    """The bench's small-T rule is the library's: at most 256 pairs, and below
    16 pairs per expert (bf16) or 64 (4-bit, fp32) on average."""
    s = dataclasses.replace(WORKLOADS["qwen_decode"], n_experts=16, top_k=8, n_tokens=32)  # 256 pairs, 16 per expert
    assert not bench.shared_in_routed_launch(s)
    assert bench.shared_in_routed_launch(dataclasses.replace(s, n_tokens=31))
    u = dataclasses.replace(s, expert_dtype="u4")
    assert bench.shared_in_routed_launch(u)  # 4-bit: tiled only from 64 pairs per expert


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in (r.stdout + r.stderr)


def test_chain_length_divides_steps_within_the_instances():
    assert bench.chain_length(20, 40) == 20
    assert bench.chain_length(800, 40) == 40
    assert bench.chain_length(50, 40) == 25
    assert bench.chain_length(41, 40) == 1
    for steps in range(1, 120):
        c = bench.chain_length(steps, 40)
        assert steps % c == 0 and 1 <= c <= 40


def test_streaming_reference_ops_run_and_count_bytes():
    import torch
    src = torch.arange(1024, dtype=torch.float32)
    dst, out = torch.empty_like(src), torch.empty(())
    ops = bench.stream_ops(src, dst, out)
    assert [o[0] for o in ops] == ["copy", "read"] and [o[2] for o in ops] == [8192, 4096]
    for _, fn, _ in ops:
        fn()
    assert torch.equal(dst, src) and out.item() == float(sum(range(1024)))


def test_host_description_reports_cores_and_blas():
    d = bench.host_description()
    assert d["cores"] >= 1 and isinstance(d["cpu_model"], str) and isinstance(d["blas"], str)
