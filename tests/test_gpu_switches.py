"""The debug switches read from the environment at every call: PTG_LOG prints each launch's
tile configuration to stderr; PTG_CHECK runs the device-side check of group offsets, user
offsets or user indices before a call that depends on them, and returns its error instead of
launching (the output stays untouched)."""
import numpy as np
import pytest
import torch

import pipelined_tiled_gemm_amd as ptg
from pipelined_tiled_gemm_amd import _ffi
from parity import dev, dev_bf16, int_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _clean(monkeypatch):
    monkeypatch.delenv("PTG_LOG", raising=False)
    monkeypatch.delenv("PTG_CHECK", raising=False)
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0


def test_log_prints_each_launch(capfd, monkeypatch):
    rng = np.random.default_rng(1)
    A, B = dev_bf16(int_bf16(rng, (512, 256))), dev_bf16(int_bf16(rng, (384, 256)))
    monkeypatch.setenv("PTG_LOG", "1")
    ptg.gemm(A, B, b_layout=ptg.B_NK)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    cfg = ptg.describe_config(512, 384, 256, ptg.B_NK)
    assert f"[ptg] ptg_gemm M=512 N=384 K=256 NK bf16: tile {cfg['BM']}x{cfg['BN']}x{cfg['BK']}" in err
    monkeypatch.setenv("PTG_LOG", "0")
    ptg.gemm(A, B, b_layout=ptg.B_NK)
    torch.cuda.synchronize()
    assert "[ptg]" not in capfd.readouterr().err


def _expect_device_check(fn, out):
    with pytest.raises(ptg.PtgError) as e:
        fn()
    assert _ffi.STATUS_NAMES[e.value.status] == "PTG_ERR_DEVICE_CHECK"
    torch.cuda.synchronize()
    assert bool(torch.isnan(out.float()).all()), "the call launched although its check failed"


def test_check_refuses_bad_group_offsets(monkeypatch):
    rng = np.random.default_rng(2)
    G, M, K, N = 4, 300, 64, 128
    X = dev_bf16(int_bf16(rng, (M, K)))
    W = dev_bf16(int_bf16(rng, (G, K, N)))
    dY = dev_bf16(int_bf16(rng, (M, N)))
    bad = dev(np.array([0, 100, 50, 200, M], dtype=np.int32))     # not nondecreasing
    good = dev(np.array([0, 50, 100, 200, M], dtype=np.int32))
    monkeypatch.setenv("PTG_CHECK", "1")
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _expect_device_check(lambda: ptg.grouped_gemm(X, W, bad, out=Y), Y)
    ws = torch.empty(ptg.grouped_gemm_split_workspace(), dtype=torch.uint8, device="cuda")
    _expect_device_check(lambda: ptg.grouped_gemm(X, W, bad, out=Y, workspace=ws), Y)
    dW = torch.full((G, K, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    _expect_device_check(lambda: ptg.grouped_gemm_wgrad(X, dY, bad, out=dW), dW)
    # valid offsets: the same result as without the switch
    checked = ptg.grouped_gemm(X, W, good, out_dtype=torch.float32)
    monkeypatch.delenv("PTG_CHECK")
    plain = ptg.grouped_gemm(X, W, good, out_dtype=torch.float32)
    assert torch.equal(checked, plain)


def test_check_refuses_bad_user_offsets_and_indices(monkeypatch):
    rng = np.random.default_rng(3)
    monkeypatch.setenv("PTG_CHECK", "1")
    # attention: user offsets must run from 0 to Mc
    U, Mc, H, D, L = 3, 40, 1, 128, 64
    Q = dev_bf16(int_bf16(rng, (Mc, H, D)))
    K = dev_bf16(int_bf16(rng, (U, L, H, D)))
    V = dev_bf16(int_bf16(rng, (U, L, H, D)))
    O = torch.full((Mc, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    bad_off = dev(np.array([0, 10, 20, Mc + 5], dtype=np.int32))
    _expect_device_check(lambda: ptg.ikbo_attention(Q, K, V, bad_off, out=O), O)
    # broadcast: every user index in [0, U)
    Ku, Kc, N = 64, 64, 128
    Xu, Xc = dev_bf16(int_bf16(rng, (U, Ku))), dev_bf16(int_bf16(rng, (Mc, Kc)))
    W = dev_bf16(int_bf16(rng, (Ku + Kc, N)))
    idx = np.arange(Mc, dtype=np.int32) % U
    idx[7] = U
    Y = torch.full((Mc, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    for fn in (ptg.broadcast_gemm, ptg.broadcast_gemm_noalloc):
        _expect_device_check(lambda: fn(Xu, Xc, dev(idx), W, out=Y), Y)
    Xu2 = dev_bf16(int_bf16(rng, (U, 128)))
    W2 = dev_bf16(int_bf16(rng, (128 + Kc, N)))
    _expect_device_check(lambda: ptg.broadcast_gemm_fused(Xu2, Xc, dev(idx), W2, out=Y), Y)
