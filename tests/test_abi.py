"""The C-ABI library without a GPU: it loads, exports every entry point that
include/moe.h declares, and rejects bad arguments on the host before any
launch.  Pointers here are fake; every case is one the checks must refuse, so
no kernel is ever launched."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_38_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4
A = 0x100000  # a fake, 16-byte aligned "device" address
MIS = A + 4   # a fake misaligned one


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = moe.load()
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_kernel_names():
    lib = moe.load()
    for s in range(6):
        assert lib.moe_status_string(s)
    assert lib.moe_kernel_name(5) == b"ffn_gate_up"
    assert lib.moe_kernel_name(11) == b"router_losses"
    assert lib.moe_kernel_name(99) == b"?"


def _ws(p):
    return moe.moe_workspace_size(p)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), INVALID), (dict(T=-3), INVALID), (dict(top_k=9), INVALID), (dict(top_k=0), INVALID),
    (dict(n_experts=2000, top_k=2), UNSUPPORTED), (dict(d_model=100), UNSUPPORTED),
    (dict(d_ff=1410), UNSUPPORTED), (dict(dtype=7), UNSUPPORTED), (dict(flags=4), INVALID),
    (dict(flags=3), OK),
    (dict(n_experts=64, top_k=33), UNSUPPORTED), (dict(T=1 << 29, top_k=2), UNSUPPORTED),
    (dict(dtype=0, T=1 << 20, top_k=2, d_model=2048), UNSUPPORTED),
    (dict(dtype=0, T=1 << 20, top_k=2, d_model=1024), OK),
])
def test_problem_checks(kw, status):
    base = dict(T=64, d_model=128, n_experts=8, top_k=2, d_ff=256, dtype=1, capacity=-1, flags=0)
    base.update(kw)
    p = moe.MoEProblem(**base)
    out = ctypes.c_size_t(0)
    assert moe.load().moe_workspace_size(ctypes.byref(p), ctypes.byref(out)) == status


def test_workspace_sizes_grow_with_the_problem():
    small = moe.problem(64, 128, 8, 2, 256, "bf16")
    big = moe.problem(8192, 4096, 8, 2, 14336, "bf16")
    assert 0 < _ws(small) < _ws(big)
    assert moe.moe_dispatch_workspace_size(big) > 0
    assert moe.moe_expert_ffn_workspace_size(big) > 0
    assert moe.moe_route_workspace_size(big) >= 8 * 4


def test_forward_rejects_bad_arguments():
    lib = moe.load()
    p = moe.problem(64, 128, 8, 2, 256, "bf16")
    need = _ws(p)
    P = ctypes.byref(p)
    # null required pointer
    assert lib.moe_forward(P, None, A, A, A, A, None, A, None, A, need, None) == INVALID
    # misaligned pointer
    assert lib.moe_forward(P, MIS, A, A, A, A, None, A, None, A, need, None) == ALIGN
    # workspace too small / missing
    assert lib.moe_forward(P, A, A, A, A, A, None, A, None, A, need - 1, None) == WORKSPACE
    assert lib.moe_forward(P, A, A, A, A, A, None, A, None, None, need, None) == WORKSPACE
    # misaligned optional debug pointer
    dbg = moe.MoEDebugOut(logits=MIS)
    assert lib.moe_forward(P, A, A, A, A, A, None, A, ctypes.byref(dbg), A, need, None) == ALIGN
    bad = moe.problem(64, 128, 8, 9, 256, "bf16")
    assert lib.moe_forward(ctypes.byref(bad), A, A, A, A, A, None, A, None, A, need, None) == INVALID


def test_step_calls_reject_bad_arguments():
    lib = moe.load()
    p = moe.problem(64, 128, 8, 2, 256, "bf16")
    P = ctypes.byref(p)
    # route: missing ids; prob_sum without workspace; router weight missing with x
    assert lib.moe_route(P, A, A, None, A, None, None, None, A, None, 0, None) == INVALID
    assert lib.moe_route(P, A, A, None, A, None, A, A, A, None, 0, None) == WORKSPACE
    assert lib.moe_route(P, A, None, None, A, None, None, A, A, None, 0, None) == INVALID
    # dispatch: x given without x_perm; workspace too small
    dws = moe.moe_dispatch_workspace_size(p)
    assert lib.moe_dispatch(P, A, A, A, A, A, A, A, None, A, dws, None) == INVALID
    assert lib.moe_dispatch(P, A, None, A, A, A, A, A, None, A, dws - 1, None) == WORKSPACE
    assert lib.moe_dispatch(P, MIS, None, A, A, A, A, A, None, A, dws, None) == ALIGN
    # ffn: missing weight; combine: missing output
    fws = moe.moe_expert_ffn_workspace_size(p)
    assert lib.moe_expert_ffn(P, A, A, A, None, A, A, A, A, fws, None) == INVALID
    assert lib.moe_expert_ffn(P, A, A, A, A, A, A, A, None, fws, None) == WORKSPACE
    assert lib.moe_combine(P, A, A, A, None, None) == INVALID
    assert lib.moe_aux_loss(P, None, A, A, None) == INVALID
    assert lib.moe_bias_update(P, A, ctypes.c_float(1e-3), None, None) == INVALID


def test_router_losses_rejects_bad_arguments():
    lib = moe.load()
    p = moe.problem(64, 128, 8, 2, 256, "bf16")
    P = ctypes.byref(p)
    ws = moe.moe_router_losses_workspace_size(p)
    assert ws >= 4 * 9
    # no output requested; aux without counts; workspace too small; misaligned scores
    assert lib.moe_router_losses(P, A, None, A, A, None, None, A, ws, None) == INVALID
    assert lib.moe_router_losses(P, A, None, A, None, None, A, A, ws, None) == INVALID
    assert lib.moe_router_losses(P, A, None, A, A, A, A, A, ws - 1, None) == WORKSPACE
    assert lib.moe_router_losses(P, MIS, None, A, A, A, A, A, ws, None) == ALIGN
    assert lib.moe_router_losses(P, A, None, None, A, A, A, A, ws, None) == INVALID


def test_combine_concat_rejects_bad_arguments():
    lib = moe.load()
    p = moe.problem(64, 128, 8, 2, 256, "bf16")
    P = ctypes.byref(p)
    ws = moe.moe_combine_concat_workspace_size(p)
    assert ws >= 64 * 2 * 128 * 2  # the concatenated rows at least
    assert moe.moe_combine_concat_workspace_size(moe.problem(4096, 128, 8, 2, 256, "bf16")) > ws
    assert lib.moe_combine_concat(P, None, A, A, A, A, ws, None) == INVALID
    assert lib.moe_combine_concat(P, A, A, None, A, A, ws, None) == INVALID
    assert lib.moe_combine_concat(P, A, A, A, A, A, ws - 1, None) == WORKSPACE
    assert lib.moe_combine_concat(P, A, A, A, A, MIS, ws, None) == ALIGN
    assert lib.moe_combine_concat(P, MIS, A, A, A, A, ws, None) == ALIGN


def test_timer_hook_bookkeeping():
    lib = moe.load()
    n = ctypes.c_int(-1)
    assert lib.moe_set_kernel_timer(5, None, None, 0, ctypes.byref(n)) == OK and n.value == 0
    assert lib.moe_set_kernel_timer(5, None, None, 3, None) == INVALID
    assert lib.moe_set_kernel_timer(42, None, None, 0, None) == INVALID
    assert lib.moe_set_kernel_timer(5, None, None, -1, ctypes.byref(n)) == OK and n.value == 0


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_LIB", None)
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "libmoe.so"))
    with pytest.raises(RuntimeError, match="missing"):
        moe.load()


def test_chunked_forward_checks():
    lib = moe.load()
    p = moe.problem(1000, 128, 8, 2, 256, "bf16")
    P = ctypes.byref(p)
    ws = moe.moe_forward_chunked_workspace_size(p, 256)
    assert 0 < ws < moe.moe_workspace_size(p)
    assert moe.moe_forward_chunked_workspace_size(p, 5000) == moe.moe_workspace_size(p)
    # capacity is a per-batch rule: refused
    pc = moe.problem(1000, 128, 8, 2, 256, "bf16", capacity=100)
    assert lib.moe_forward_chunked(ctypes.byref(pc), 256, A, A, A, A, A, None, A, None, A, ws, None) == UNSUPPORTED
    # bad chunk, small workspace, per-batch debug output
    assert lib.moe_forward_chunked(P, 0, A, A, A, A, A, None, A, None, A, ws, None) == INVALID
    assert lib.moe_forward_chunked(P, 256, A, A, A, A, A, None, A, None, A, ws - 1, None) == WORKSPACE
    dbg = moe.MoEDebugOut(counts=A)
    assert lib.moe_forward_chunked(P, 256, A, A, A, A, A, None, A, ctypes.byref(dbg), A, ws, None) == INVALID


def test_peaks_library_exports_every_declared_function():
    """libmoepeaks.so (the measurement probes of include/moe_peaks.h) loads
    and exports what its header declares; no kernel is launched."""
    from mixture_experts_layer_38_amd import peaks
    text = open(os.path.join(ROOT, "include", "moe_peaks.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = sorted(set(re.findall(r"\b(peak_[a-z_]+)\s*\(", text)))
    assert len(names) == 6
    lib = peaks.load()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.peak_mfma_flops(4, 1) == 4 * 4 * 8 * 2.0 * 32 * 32 * 16
    assert lib.peak_stream_read(None, 1 << 20, 1, None, None) == 1  # refused on the host
    assert lib.peak_mfma_loop(A, 3, 1, A, None) == 1                 # iters not a multiple of 4


def test_noalloc_refuses_oversized_problems_on_the_host():
    """moe_forward_noalloc checks the problem's workspace against its static
    array before it touches the GPU: an oversized problem is refused, so no
    kernel is launched with these fake pointers."""
    lib = moe.load()
    p = moe.problem(8192, 4096, 8, 2, 14336, "bf16")
    assert _ws(p) > moe.MOE_NOALLOC_WS_BYTES
    assert lib.moe_forward_noalloc(ctypes.byref(p), A, A, A, A, A, None, A, None, None) == WORKSPACE
    assert lib.moe_forward_noalloc(ctypes.byref(p), None, A, A, A, A, None, A, None, None) == INVALID
