"""GPU parity of the mixture-of-experts backward products against the fp64 CPU oracle.

Weight gradient dW_g = X_g^T . dY_g (ptg_grouped_gemm_wgrad): the reduction runs over each
expert's rows, so the cases cover empty experts (dW_g = 0), experts of one row, reduction
tails that are not multiples of 8, ragged m and n tiles, and (at full size) the 64-expert
Zipf(1.1) routing of the forward workload; the workgroups take tiles from a queue in a small
caller workspace, whose prior content must not matter.  Input gradient dX_g = dY_g . W_g^T is the grouped
GEMM with the forward weights read as N x K.
"""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import check, dev, dev_bf16, exact, int_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_watchdog():
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0, "a pipeline wait timed out"


def offsets_of(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


def sentinel_out(G, K, N, dtype, guard=4096):
    """dW followed by a guard band, both filled with NaN: every element of dW must be written,
    nothing after it."""
    buf = torch.full((G * K * N + guard,), float("nan"), dtype=dtype, device="cuda")
    return buf, buf[: G * K * N].view(G, K, N)


def guard_untouched(buf, G, K, N):
    tail = buf[G * K * N:]
    assert torch.isnan(tail).all().item(), "the kernel wrote past dW"


# reduction lengths: tails of 44, 1, 63, 2 rows past whole 64-row steps; several empty experts
COUNTS = np.array([300, 0, 1, 129, 0, 0, 64, 511, 2, 0])


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K,N", [(520, 392), (256, 256), (8, 8)])
def test_wgrad_small(out_dtype, K, N):
    w = wl.wgrad(61, len(COUNTS), int(COUNTS.sum()), K, N, counts=COUNTS)
    buf, dW = sentinel_out(w.G, K, N, out_dtype)
    ptg.grouped_gemm_wgrad(dev_bf16(w.X), dev_bf16(w.dY), dev(w.offsets), out=dW)
    v = oracle.grouped_wgrad(w.X, w.dY, w.offsets)
    # the reduction length is the largest expert's row count
    check(dW.reshape(w.G * K, N), v, int(COUNTS.max()), f"wgrad K={K} N={N} {out_dtype}")
    guard_untouched(buf, w.G, K, N)
    for g in np.flatnonzero(COUNTS == 0):
        assert (dW[g] == 0).all().item(), f"empty expert {g} must get dW = 0"


def test_wgrad_integer_exact():
    """Integer X and dY: every partial sum is an exact integer in fp32, so the fp32 result must
    equal the oracle bit for bit (no lost, repeated or misplaced row of any expert)."""
    counts = np.array([700, 3, 0, 65, 1, 257])
    G, K, N = len(counts), 776, 264
    M = int(counts.sum())
    rng = np.random.default_rng(62)
    X, dY = int_bf16(rng, (M, K)), int_bf16(rng, (M, N))
    off = offsets_of(counts)
    dW = ptg.grouped_gemm_wgrad(dev_bf16(X), dev_bf16(dY), dev(off), out_dtype=torch.float32)
    exact(dW.reshape(G * K, N), oracle.grouped_wgrad(X, dY, off), "wgrad integer")


def test_wgrad_one_hot_rows():
    """X[r] = e_{c(r)}: dW_g[i] is the sum of the rows of dY_g whose hot column is i; pins
    which expert, which row of X and which row of dY meet in every product."""
    counts = np.array([90, 0, 300, 7])
    G, K, N = len(counts), 264, 136
    M = int(counts.sum())
    rng = np.random.default_rng(63)
    hot = rng.integers(0, K, M)
    X = wl.f32_to_bf16_bits(np.eye(K, dtype=np.float32)[hot])
    dY = int_bf16(rng, (M, N))
    off = offsets_of(counts)
    want = np.zeros((G, K, N))
    dy = wl.bf16_bits_to_f32(dY).astype(np.float64)
    for g in range(G):
        for r in range(int(off[g]), int(off[g + 1])):
            want[g, hot[r]] += dy[r]
    for out_dtype in (torch.float32, torch.bfloat16):
        dW = ptg.grouped_gemm_wgrad(dev_bf16(X), dev_bf16(dY), dev(off), out_dtype=out_dtype)
        exact(dW, want, f"one-hot {out_dtype}")


def test_wgrad_no_rows_at_all():
    """M_total = 0: every expert is empty and dW is all zeros."""
    G, K, N = 5, 264, 136
    off = np.zeros(G + 1, np.int32)
    buf, dW = sentinel_out(G, K, N, torch.float32)
    X = torch.empty((0, K), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, N), dtype=torch.bfloat16, device="cuda")
    ptg.grouped_gemm_wgrad(X, dY, dev(off), out=dW)
    assert (dW == 0).all().item()
    guard_untouched(buf, G, K, N)


def test_wgrad_equals_gemm_on_transposed_slices():
    """Invariant: each expert's gradient equals the plain GEMM of an explicitly transposed copy
    of X_g with dY_g (GPU against GPU, bit-exact on integer data).  The plain GEMM needs its
    reduction length to be a multiple of 8, hence the row counts."""
    counts = np.array([136, 0, 520, 8])
    G, K, N = len(counts), 512, 264
    M = int(counts.sum())
    rng = np.random.default_rng(64)
    X, dY = int_bf16(rng, (M, K)), int_bf16(rng, (M, N))
    off = offsets_of(counts)
    Xd, dYd = dev_bf16(X), dev_bf16(dY)
    dW = ptg.grouped_gemm_wgrad(Xd, dYd, dev(off), out_dtype=torch.float32)
    for g in range(G):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi == lo:
            continue
        XT = Xd[lo:hi].t().contiguous()
        ref = ptg.gemm(XT, dYd[lo:hi].contiguous(), b_layout=ptg.B_KN, out_dtype=torch.float32)
        assert torch.equal(dW[g], ref), f"expert {g}"


def test_wgrad_repeat_is_bit_identical():
    w = wl.wgrad(65, len(COUNTS), int(COUNTS.sum()), 520, 392, counts=COUNTS)
    X, dY, off = dev_bf16(w.X), dev_bf16(w.dY), dev(w.offsets)
    a = ptg.grouped_gemm_wgrad(X, dY, off, out_dtype=torch.float32)
    b = ptg.grouped_gemm_wgrad(X, dY, off, out_dtype=torch.float32)
    assert torch.equal(a, b)


def test_wgrad_workspace_content_does_not_matter():
    """The tile queue is reset on the stream before every launch: a workspace full of arbitrary
    bytes, and one reused by back-to-back calls, give the same bits."""
    w = wl.wgrad(68, len(COUNTS), int(COUNTS.sum()), 520, 392, counts=COUNTS)
    X, dY, off = dev_bf16(w.X), dev_bf16(w.dY), dev(w.offsets)
    ws = torch.full((ptg.grouped_gemm_wgrad_workspace(),), 0xA5, dtype=torch.uint8, device="cuda")
    a = ptg.grouped_gemm_wgrad(X, dY, off, out_dtype=torch.float32, workspace=ws)
    ws.fill_(0xFF)
    b = ptg.grouped_gemm_wgrad(X, dY, off, out_dtype=torch.float32, workspace=ws)
    c = ptg.grouped_gemm_wgrad(X, dY, off, out_dtype=torch.float32, workspace=ws)
    assert torch.equal(a, b) and torch.equal(b, c)
    check(a.reshape(w.G * w.K, w.N), oracle.grouped_wgrad(w.X, w.dY, w.offsets), int(COUNTS.max()), "workspace")


def test_wgrad_rejects_bad_arguments():
    X = torch.zeros((16, 12), dtype=torch.bfloat16, device="cuda")  # K = 12: not a multiple of 8
    dY = torch.zeros((16, 8), dtype=torch.bfloat16, device="cuda")
    off = dev(np.array([0, 16], np.int32))
    with pytest.raises(ptg.PtgError):
        ptg.grouped_gemm_wgrad(X, dY, off)
    X = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    with pytest.raises(ptg.PtgError):
        ptg.grouped_gemm_wgrad(X, dY, off, workspace=small)


def test_dgrad_is_grouped_gemm_nk():
    """dX_g = dY_g . W_g^T: the grouped GEMM with the forward's K x N weights as layout NK."""
    counts = np.array([200, 0, 3, 317])
    G, K, N = len(counts), 392, 264   # forward: X [M x K], W_g [K x N], dY [M x N]
    M = int(counts.sum())
    rng = np.random.default_rng(66)
    dY = wl.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    W = wl.f32_to_bf16_bits((rng.standard_normal((G, K, N)) * 0.02).astype(np.float32))
    off = offsets_of(counts)
    v = oracle.grouped_gemm(dY, W, wl.B_NK, off)
    for out_dtype in (torch.float32, torch.bfloat16):
        dX = ptg.grouped_gemm(dev_bf16(dY), dev_bf16(W), dev(off), w_layout=ptg.B_NK, out_dtype=out_dtype)
        check(dX, v, N, f"dgrad {out_dtype}")


def test_moe_wgrad_full_size_sampled():
    """The benchmarked backward workload (64 experts, 16384 rows, K = 4096, N = 1536, rank-Zipf
    routing), in the benchmarked launch: sampled rows of dW (the first, last and a random row
    of every expert's K x N block, plus random rows), bf16 output and its fp32 twin."""
    w = wl.moe_wgrad()
    rng = np.random.default_rng(67)
    rows = set(rng.integers(0, w.G * w.K, 96).tolist())
    for g in range(w.G):
        rows |= {g * w.K, g * w.K + w.K - 1, g * w.K + int(rng.integers(0, w.K))}
    rows = np.array(sorted(rows), dtype=np.int64)
    v = oracle.grouped_wgrad(w.X, w.dY, w.offsets, rows=rows)
    X, dY, off = dev_bf16(w.X), dev_bf16(w.dY), dev(w.offsets)
    idx = torch.from_numpy(rows).cuda()
    Kred = int(w.counts.max())
    for out_dtype in (torch.bfloat16, torch.float32):
        dW = ptg.grouped_gemm_wgrad(X, dY, off, out_dtype=out_dtype)
        check(dW.reshape(w.G * w.K, w.N)[idx], v, Kred, f"moe wgrad {out_dtype}")
        del dW
        torch.cuda.empty_cache()
