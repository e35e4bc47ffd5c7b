"""The C-ABI library loads and exports every declared symbol (no GPU needed).

Only host-pure entry points are called here (dg_temperature, dg_reveal_count,
dg_workspace_bytes, dg_moe_workspace_bytes), and entry points with a NULL context, which
refuse before touching a device; nothing launches a kernel.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import dg_inputs as di
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import block_ar_canvas_amd as dg

    if not os.path.exists(dg.lib_path()):
        from block_ar_canvas_amd.build import build
        build()
    return dg._load()


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "dg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert len(syms) >= 15
    cdll = ctypes.CDLL(os.path.join(ROOT, "block_ar_canvas_amd", "libdg.so"))
    for s in syms:
        assert hasattr(cdll, s), s


def test_seven_calls_declared():
    syms = declared_symbols()
    for s in ("dg_canvas_attn", "dg_logits_entropy", "dg_entropy_accept", "dg_renoise",
              "dg_selfcond", "dg_stop_test", "dg_commit_kv"):
        assert s in syms


def test_temperature_matches_oracle(lib):
    import block_ar_canvas_amd as dg

    for N in (1, 2, 8, 48, 64):
        for k in range(N):
            assert np.float32(dg.temperature(k, N)) == O.temperature(k, N)
    assert dg.temperature(47, 48) == np.float32(0.4)
    assert dg.temperature(0, 48) == np.float32(0.8)


def test_reveal_count_matches_oracle(lib):
    import block_ar_canvas_amd as dg

    for C, N in ((256, 48), (16, 8), (100, 7), (1000, 48), (0, 3), (5, 9)):
        sched = O.reveal_schedule(C, N)
        assert [dg.reveal_count(C, N, t) for t in range(N)] == sched
        assert dg.reveal_count(C, N, N + 3) == C
    assert lib.dg_reveal_count(4, 0, 0) == -1
    assert lib.dg_reveal_count(-1, 4, 0) == -1


def test_workspace_bytes(lib):
    import block_ar_canvas_amd as dg

    for i in range(5):
        cfg = di.config(i)
        n = dg.workspace_bytes(cfg, cfg.Pcap)
        # p~ alone is C x V bf16
        assert n >= cfg.C * cfg.V * 2
    big = di.config(2)
    assert dg.workspace_bytes(big, 262400) >= dg.workspace_bytes(big, 8448)
    with pytest.raises(dg.DGError):
        dg.workspace_bytes(big.with_(hd=48), 1024)


def test_moe_workspace_bytes(lib):
    import block_ar_canvas_amd as dg

    md = dg.MoeDims(2048, 128, 8, 512, 1024)
    n = dg.moe_workspace_bytes(md, 256)
    # at least: fp32 router logits, the grouped hidden rows and expert outputs (bf16)
    assert n >= 256 * 128 * 4 + 256 * 8 * (512 + 2048) * 2
    assert dg.moe_workspace_bytes(md, 512) > n
    assert dg.moe_workspace_bytes(md, 1024) > 0           # C * K = 8192, the limit
    for bad, C in ((dg.MoeDims(64, 16, 20, 32, 64), 8),   # K > E
                   (dg.MoeDims(64, 16, 4, 40, 64), 8),    # Fe not a multiple of 32
                   (dg.MoeDims(64, 300, 4, 32, 64), 8),   # E > 256
                   (dg.MoeDims(64, 16, 33, 32, 64), 8),   # K > 32
                   (dg.MoeDims(2048, 128, 8, 512, 1024), 1025),   # C > 1024
                   (dg.MoeDims(64, 64, 16, 32, 64), 600)):        # C * K > 8192
        with pytest.raises(dg.DGError):
            dg.moe_workspace_bytes(bad, C)


def test_binding_rejects_host_tensors(lib):
    import torch

    import block_ar_canvas_amd as dg

    with pytest.raises((ValueError, TypeError)):
        dg._ptr(torch.zeros(4), torch.float32, "x")


def test_binding_flag_may_be_pinned_host_only(lib):
    """Only the stop flag may live in host memory, and only if it is pinned."""
    import torch

    import block_ar_canvas_amd as dg

    with pytest.raises(ValueError):
        dg._ptr(torch.zeros(1, dtype=torch.int32), torch.int32, "flag", pinned_ok=True)
    with pytest.raises(ValueError):
        dg._ptr(torch.zeros(4), torch.float32, "x", pinned_ok=False)


def test_loop_workspace_bytes(lib):
    import block_ar_canvas_amd as dg

    for i in range(5):
        cfg = di.config(i)
        n = dg.loop_workspace_bytes(cfg)
        # tokens, entropy, two argmax buffers (4 B each), acceptance, z and A (bf16 rows)
        assert n >= cfg.C * (4 * 4 + 1) + 2 * 2 * cfg.C * cfg.d
        assert n % 256 == 0
    with pytest.raises(dg.DGError):
        dg.loop_workspace_bytes(di.config(2).with_(hd=48))


def test_run_canvas_refuses_a_null_context(lib):
    # a NULL context is refused before anything touches a device
    steps, P = ctypes.c_int32(0), ctypes.c_int64(0)
    d = lib.dg_run_canvas.argtypes[1]._type_()
    st = lib.dg_run_canvas(None, ctypes.byref(d), None, None, None, 0, 0, None, lib.dg_run_canvas.argtypes[8](), None,
                           None, None, None, ctypes.byref(steps), ctypes.byref(P))
    assert st == 1                                      # DG_ERR_NULL


def test_combined_sampler_calls_refuse_a_null_context(lib):
    # the one-launch acceptance/renoise/stop call and the one beside self-conditioning's
    # reduce are refused with DG_ERR_NULL before anything touches a device
    st = lib.dg_accept_renoise_stop(None, 1, 16, 100, None, 0.1, None, None, None, 1, 0, 0, 0.005, 8,
                                    None, None, None, None)
    assert st == 1
    import block_ar_canvas_amd as dg
    d = dg.Dims(V=512, d=64, C=16, Hq=4, Hkv=2, hd=16, F=128)
    a = dg.AcceptArgs()
    st = lib.dg_selfcond_accept(None, ctypes.byref(d), None, None, None, None, None, ctypes.byref(a))
    assert st == 1
