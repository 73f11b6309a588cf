"""CPU checks of the C ABI: the library loads, exports what include/moe.h
declares, its structs match the binding's layout, and host-side argument
checks return the documented codes without launching anything."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from top_routing_grouped_amd import moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    L = moe.lib()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(moe.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", moe._LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), n


def test_struct_layout_matches_header():
    prog = r"""
#include <stdio.h>
#include <stddef.h>
#include "moe.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu\n", sizeof(moe_config), offsetof(moe_config, routed_scaling),
         offsetof(moe_config, expert_dtype), sizeof(moe_matrix), sizeof(moe_weights),
         offsetof(moe_weights, shared_gate_vec));
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write(prog)
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c11", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        got = list(map(int, subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()))
    want = [ctypes.sizeof(moe.MoeConfig), moe.MoeConfig.routed_scaling.offset, moe.MoeConfig.expert_dtype.offset,
            ctypes.sizeof(moe.MoeMatrix), ctypes.sizeof(moe.MoeWeights), moe.MoeWeights.shared_gate_vec.offset]
    assert got == want


def _cfg(**kw):
    base = dict(n_tokens=8, d_model=2048, n_experts=256, top_k=8, d_ff=512, d_ff_shared=512)
    base.update(kw)
    return moe.make_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(top_k=0), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(top_k=300), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(top_k=33, n_experts=64), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=250), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=2048), moe.MOE_ERR_UNSUPPORTED),
    (dict(n_tokens=-1), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(d_model=2000), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=96), moe.MOE_ERR_UNSUPPORTED),
    (dict(d_ff_shared=-1), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(expert_dtype="f32"), moe.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype="f32", router_dtype="f32", expert_dtype="bf16"), moe.MOE_ERR_UNSUPPORTED),
    (dict(router_dtype="f32"), moe.MOE_ERR_UNSUPPORTED),
    (dict(family="sigmoid_group", n_experts=128, n_group=6, topk_group=4), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(family="sigmoid_group", n_experts=128, n_group=8, topk_group=9), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(family="sigmoid_group", n_experts=128, n_group=8, topk_group=0), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(family="sigmoid_group", n_experts=128, n_group=8, topk_group=1, top_k=17), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(family="sigmoid_group", n_experts=128, n_group=128, topk_group=4), moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(family="sigmoid_group", n_experts=128, n_group=8, topk_group=4, routed_scaling=0.0),
     moe.MOE_ERR_INVALID_ARGUMENT),
    (dict(family="sigmoid_group", n_experts=128, n_group=8, topk_group=4, routed_scaling=float("nan")),
     moe.MOE_ERR_INVALID_ARGUMENT),
])
def test_config_validation_codes(kw, code):
    n = ctypes.c_size_t(0)
    st = moe.lib().moe_workspace_size(ctypes.byref(_cfg(**kw)), ctypes.byref(n))
    assert st == code, moe.lib().moe_last_error()
    assert moe.lib().moe_last_error()


def test_valid_configs_and_workspace_grows_with_tokens():
    sizes = [moe.workspace_size(_cfg(n_tokens=t)) for t in (1, 8, 4096)]
    assert sizes[0] < sizes[1] < sizes[2]
    moe.workspace_size(_cfg(family="sigmoid_group", n_experts=128, n_group=8, topk_group=4, routed_scaling=2.5))
    moe.workspace_size(_cfg(expert_dtype="u4", top_k=4))
    moe.workspace_size(_cfg(act_dtype="f32", router_dtype="f32", expert_dtype="f32", d_model=64, d_ff=32,
                            d_ff_shared=32, n_experts=16, top_k=4))


def test_null_and_workspace_errors_without_launch():
    L = moe.lib()
    cfg = _cfg()
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below fails its host checks
    # null tensors
    assert L.moe_route(ctypes.byref(cfg), None, fake, None, fake, fake, fake, 1 << 30, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    # workspace too small
    assert L.moe_route(ctypes.byref(cfg), fake, fake, None, fake, fake, fake, 16, None) == \
        moe.MOE_ERR_WORKSPACE_TOO_SMALL
    # misaligned workspace
    need = moe.workspace_size(cfg)
    assert L.moe_route(ctypes.byref(cfg), fake, fake, None, fake, fake, ctypes.c_void_p(4100), need, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    # null weights / missing u4 scale
    w = moe.MoeWeights()
    assert L.moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), fake, fake, fake, None, None, fake, need,
                               None, None) == moe.MOE_ERR_INVALID_ARGUMENT
    cu4 = _cfg(expert_dtype="u4", top_k=4)
    w = moe.MoeWeights(4096, None, moe.MoeMatrix(4096, None, None), moe.MoeMatrix(4096, 4096, 4096),
                       moe.MoeMatrix(4096, 4096, 4096))
    assert L.moe_experts(ctypes.byref(cu4), fake, ctypes.byref(w), fake, fake, fake, fake, fake, fake, fake,
                         moe.workspace_size(cu4), None) == moe.MOE_ERR_INVALID_ARGUMENT
    # shared expert requested without one
    c0 = _cfg(d_ff_shared=0)
    assert L.moe_shared_expert(ctypes.byref(c0), fake, ctypes.byref(w), fake, fake, 1 << 30, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    # config NULL
    assert L.moe_combine(None, fake, None, fake, fake, None) == moe.MOE_ERR_INVALID_ARGUMENT


def test_rms_norm_argument_errors_without_launch():
    L = moe.lib()
    cfg = _cfg(n_tokens=8)
    fake, fake2 = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24)  # never dereferenced
    E = moe.MOE_ERR_INVALID_ARGUMENT
    for eps in (0.0, -1e-6, float("inf"), float("nan")):
        assert L.moe_rms_norm(ctypes.byref(cfg), fake, None, eps, fake2, None) == E
    assert L.moe_rms_norm(ctypes.byref(cfg), None, None, 1e-6, fake2, None) == E
    assert L.moe_rms_norm(ctypes.byref(cfg), fake, None, 1e-6, None, None) == E
    assert L.moe_rms_norm(ctypes.byref(cfg), ctypes.c_void_p((1 << 20) + 8), None, 1e-6, fake2, None) == E
    assert L.moe_rms_norm(ctypes.byref(cfg), fake, ctypes.c_void_p(4100), 1e-6, fake2, None) == E
    # x overlapping the residual rows
    assert L.moe_rms_norm(ctypes.byref(cfg), fake, None, 1e-6, ctypes.c_void_p((1 << 20) + 256), None) == E
    assert L.moe_rms_norm(None, fake, None, 1e-6, fake2, None) == E
    # the layer entry: bad eps, missing residual, x_out overlapping out
    need = moe.workspace_size(cfg)
    w = moe.MoeWeights(4096, None, moe.MoeMatrix(4096, None, None), moe.MoeMatrix(4096, None, None),
                       moe.MoeMatrix(4096, None, None), moe.MoeMatrix(4096, None, None),
                       moe.MoeMatrix(4096, None, None), moe.MoeMatrix(4096, None, None))
    ws = ctypes.c_void_p(1 << 28)
    def call(eps=1e-6, residual=fake, x_out=None, out=fake2):
        return L.moe_layer_forward_norm(ctypes.byref(cfg), ctypes.byref(w), None, eps, residual, x_out, out,
                                        None, None, ws, need, None, None)
    assert call(eps=0.0) == E
    assert call(residual=None) == E
    assert call(x_out=ctypes.c_void_p((1 << 24) + 64)) == E
    assert L.moe_layer_forward_norm(ctypes.byref(cfg), ctypes.byref(w), None, 1e-6, fake, None, fake2, None, None,
                                    ws, 16, None, None) == moe.MOE_ERR_WORKSPACE_TOO_SMALL


def test_mfma_rate_argument_errors_without_launch():
    """The MFMA issue-rate aid rejects shapes, sizes and sinks off its grid
    before any launch (the sink pointer is never dereferenced)."""
    L = moe.lib()
    E = moe.MOE_ERR_INVALID_ARGUMENT
    fake = ctypes.c_void_p(1 << 20)
    assert L.moe_mfma_rate(2, 1, 1, fake, 256, None) == E
    assert L.moe_mfma_rate(-1, 1, 1, fake, 256, None) == E
    assert L.moe_mfma_rate(0, 0, 1, fake, 256, None) == E
    assert L.moe_mfma_rate(0, 65537, 1, fake, 65537 * 256, None) == E
    assert L.moe_mfma_rate(1, 1, 0, fake, 256, None) == E
    assert L.moe_mfma_rate(1, 1, (1 << 16) + 1, fake, 256, None) == E
    assert L.moe_mfma_rate(0, 2, 1, fake, 511, None) == E
    assert L.moe_mfma_rate(0, 1, 1, None, 256, None) == E


def test_l2_read_rate_argument_errors_without_launch():
    """The L2 read-rate aid rejects patterns, sizes, buffers and sinks off its
    grid before any launch (the pointers are never dereferenced)."""
    L = moe.lib()
    E = moe.MOE_ERR_INVALID_ARGUMENT
    buf, sink = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 24)
    MiB = 1 << 20
    assert L.moe_l2_read_rate(3, 1, 1, buf, MiB, sink, 256, None) == E
    assert L.moe_l2_read_rate(-1, 1, 1, buf, MiB, sink, 256, None) == E
    assert L.moe_l2_read_rate(0, 0, 1, buf, MiB, sink, 256, None) == E
    assert L.moe_l2_read_rate(0, 65537, 1, buf, MiB, sink, 65537 * 256, None) == E
    assert L.moe_l2_read_rate(1, 1, 0, buf, MiB, sink, 256, None) == E
    assert L.moe_l2_read_rate(1, 1, (1 << 16) + 1, buf, MiB, sink, 256, None) == E
    assert L.moe_l2_read_rate(2, 1, 1, None, MiB, sink, 256, None) == E
    assert L.moe_l2_read_rate(2, 1, 1, ctypes.c_void_p((1 << 20) + 8), MiB, sink, 256, None) == E
    assert L.moe_l2_read_rate(0, 1, 1, buf, MiB - 16, sink, 256, None) == E
    assert L.moe_l2_read_rate(0, 1, 1, buf, MiB, None, 256, None) == E
    assert L.moe_l2_read_rate(0, 2, 1, buf, MiB, sink, 511, None) == E


def test_noalloc_entry_host_checks_without_launch():
    """The allocation-free layer entry rejects bad arguments and layers whose
    scratch need exceeds its 32 MiB array before any HIP call."""
    L = moe.lib()
    fake = ctypes.c_void_p(4096)  # never dereferenced
    w = moe.MoeWeights(4096, None, moe.MoeMatrix(4096, None, None), moe.MoeMatrix(4096, None, None),
                       moe.MoeMatrix(4096, None, None), moe.MoeMatrix(4096, None, None),
                       moe.MoeMatrix(4096, None, None), moe.MoeMatrix(4096, None, None))
    big = moe.make_config(512, 2048, 256, 8, 512, 512)
    assert moe.workspace_size(big) > 32 << 20
    assert L.moe_layer_forward_noalloc(ctypes.byref(big), ctypes.byref(w), fake, fake, fake, None, None, None) == \
        moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert b"32" in L.moe_last_error() or b"33554432" in L.moe_last_error()
    small = moe.make_config(8, 2048, 256, 8, 512, 512)
    assert L.moe_layer_forward_noalloc(ctypes.byref(small), ctypes.byref(w), None, fake, fake, None, None, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_layer_forward_noalloc(ctypes.byref(small), None, fake, fake, fake, None, None, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert L.moe_layer_forward_noalloc(None, ctypes.byref(w), fake, fake, fake, None, None, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    zero = moe.make_config(0, 2048, 256, 8, 512, 512)
    assert L.moe_layer_forward_noalloc(ctypes.byref(zero), ctypes.byref(w), None, None, None, None, None, None) == \
        moe.MOE_OK


def test_zero_tokens_is_ok_without_launch():
    L = moe.lib()
    cfg = _cfg(n_tokens=0)
    w = moe.MoeWeights()
    assert L.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert L.moe_permute(ctypes.byref(cfg), None, None, None, None, None, None, 0, None) == moe.MOE_OK
    assert L.moe_combine(ctypes.byref(cfg), None, None, None, None, None) == moe.MOE_OK
    assert L.moe_layer_forward(ctypes.byref(cfg), ctypes.byref(w), None, None, None, None, None, None, 0,
                               None, None) == moe.MOE_OK
    assert L.moe_rms_norm(ctypes.byref(cfg), None, None, 1e-6, None, None) == moe.MOE_OK
    assert L.moe_layer_forward_norm(ctypes.byref(cfg), ctypes.byref(w), None, 1e-6, None, None, None, None, None,
                                    None, 0, None, None) == moe.MOE_OK


def test_status_strings():
    L = moe.lib()
    for code, name in [(0, b"MOE_OK"), (1, b"MOE_ERR_INVALID_ARGUMENT"), (2, b"MOE_ERR_UNSUPPORTED"),
                       (3, b"MOE_ERR_WORKSPACE_TOO_SMALL"), (4, b"MOE_ERR_HIP")]:
        assert L.moe_status_string(code) == name


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(ImportError):
        moe.lib()
