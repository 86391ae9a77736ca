"""GPU parity with one operand larger than 4 GiB: the tiles far into it sit more than 2^32
bytes past its start, where the 64-bit tile bases and the per-tile buffer descriptors must
still address the right rows (the largest operands the entry points accept are bounded per
tile, not per operand).  Inputs are small integers drawn on the GPU from a seeded generator,
so every sampled output row is exact in fp32 and compared bit for bit with the oracle; the
samples include the rows whose byte offsets cross 2^31 and 2^32 and the last row."""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import dev, dev_bf16, exact, host_bits, int_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_watchdog():
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0, "a pipeline wait timed out"


def int_bf16_gpu(shape, seed):
    """Integers in [-4, 4] as bfloat16, drawn on the GPU from a seeded generator."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t = torch.randint(-4, 5, shape, dtype=torch.int16, device="cuda", generator=g)
    return t.to(torch.bfloat16)


def crossing_rows(M, row_bytes, extra):
    rows = {0, M - 1, *extra}
    for b in (1 << 31, 1 << 32):
        r = b // row_bytes
        rows |= {r - 1, r, r + 1}
    return torch.tensor(sorted(r for r in rows if 0 <= r < M), dtype=torch.int64, device="cuda")


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
def test_dense_a_beyond_4gib(layout):
    M, K, N = 300_032 + 40, 8192, 256     # A: 4.9 GB; ragged last m-tile
    A = int_bf16_gpu((M, K), 21)
    assert A.numel() * 2 > (1 << 32)
    rng = np.random.default_rng(22)
    Bh = int_bf16(rng, (K, N) if layout == wl.B_KN else (N, K))
    out = ptg.gemm(A, dev_bf16(Bh), b_layout=layout, out_dtype=torch.float32)
    rows = crossing_rows(M, K * 2, [M - 41, M - 40])
    v = oracle.gemm(host_bits(A[rows]), Bh, layout)
    exact(out[rows], v, f"dense A beyond 4 GiB, layout={layout}")
    del A, out
    torch.cuda.empty_cache()


def test_grouped_x_beyond_4gib():
    counts = np.array([250_000, 0, 350_000])
    G, K, N = len(counts), 4096, 256
    M = int(counts.sum())                 # X: 4.9 GB
    X = int_bf16_gpu((M, K), 23)
    assert X.numel() * 2 > (1 << 32)
    rng = np.random.default_rng(24)
    Wh = int_bf16(rng, (G, K, N))
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    out = ptg.grouped_gemm(X, dev_bf16(Wh), dev(off), out_dtype=torch.float32)
    rows = crossing_rows(M, K * 2, [249_999, 250_000]).cpu().numpy()
    grp = np.searchsorted(off, rows, side="right") - 1
    for g in np.unique(grp):
        rg = torch.from_numpy(rows[grp == g]).cuda()
        v = oracle.gemm(host_bits(X[rg]), Wh[g], wl.B_KN)
        exact(out[rg], v, f"grouped X beyond 4 GiB, expert {g}")
    del X, out
    torch.cuda.empty_cache()


def test_wgrad_reduction_window_just_under_2gib():
    """Weight gradient at its largest accepted operand: X of 2^31 - 8192 bytes (one tile's
    descriptor spans an expert's whole row range, so X and dY are bounded by 2 GiB), one expert
    reducing over 261,143 rows.  Columns of dW[g] depend only on the same columns of X, so the
    oracle takes the sampled columns of X; integer data, exact in fp32."""
    K, N = 4096, 256
    M = (1 << 31) // (K * 2) - 1
    counts = np.array([M - 1000, 1000])
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    X = int_bf16_gpu((M, K), 25)
    dY = int_bf16_gpu((M, N), 26)
    dW = ptg.grouped_gemm_wgrad(X, dY, dev(off), out_dtype=torch.float32)
    ks = torch.tensor([0, 1, 255, 256, 2047, 2048, 4095], dtype=torch.int64, device="cuda")
    v = oracle.grouped_wgrad(host_bits(X[:, ks].contiguous()), host_bits(dY), off)
    got = dW[:, ks, :].reshape(len(counts) * len(ks), N)
    exact(got, v, "wgrad reduction over a 2 GiB window")
    del X, dY, dW
    torch.cuda.empty_cache()
