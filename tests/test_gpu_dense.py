"""GPU parity of the dense pipelined GEMM (ptg_gemm) against the fp64 CPU oracle.

Sizes span several tiles with ragged M, N and K tails in both tile configurations (the
128 x 128 one used for small problems and the 256 x 256 one used once a problem has 128 or
more such tiles), both B layouts, every epilogue and both output types.  The 8192^3
workload is checked on sampled rows in the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import check, dev, dev_bf16, exact, host_bits, host_f32, int_bf16, sample_rows

pytestmark = pytest.mark.gpu

EPIS = [wl.EPI_NONE, wl.EPI_BIAS, wl.EPI_SILU, wl.EPI_BIAS_SILU]


@pytest.fixture(autouse=True)
def _no_watchdog():
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0, "a pipeline wait timed out"


def run_dense(w: wl.Dense, out_dtype=torch.float32, epi=None, rows=None):
    epi = w.epi if epi is None else epi
    A, B = dev_bf16(w.A), dev_bf16(w.B)
    bias = dev(w.bias) if w.bias is not None else None
    out = ptg.gemm(A, B, b_layout=w.b_layout, out_dtype=out_dtype, bias=bias, epi=epi)
    v = oracle.gemm(w.A, w.B, w.b_layout, w.bias, epi, rows=rows)
    return out, v


def test_config1_single_gemm_256():
    """256^3, U(-1,1) bf16, fp32 output, no epilogue: every element against the oracle."""
    w = wl.config1()
    out, v = run_dense(w, torch.float32)
    check(out, v, w.K, "config1")


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("epi", EPIS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_medium_tiles_ragged(layout, epi, out_dtype):
    """M, N, K tails in every direction (K = 328 leaves an 8-deep last k-step)."""
    w = wl.dense(11 + layout, 200, 136, 328, dist="uniform", b_layout=layout, with_bias=True)
    out, v = run_dense(w, out_dtype, epi)
    check(out, v, w.K, f"dense 200x136x328 layout={layout} epi={epi}")


@pytest.mark.parametrize("shape", [(128, 128, 64), (256, 128, 64), (384, 128, 8), (200, 520, 72),
                                   (2560, 2560, 136)])
def test_medium_tiles_both_consumer_groups(shape):
    """The medium tile runs alternate tiles on two consumer groups: one tile (the second group
    only sees the end), two, three (odd), a ragged grid, and 400 tiles (some workgroups run two,
    one per group) on integer data, bit-exact against the oracle."""
    M, N, K = shape
    rng = np.random.default_rng(M + N + K)
    A, B = int_bf16(rng, (M, K)), int_bf16(rng, (K, N))
    assert ptg.describe_config(M, N, K, wl.B_KN)["BM"] == 128
    out = ptg.gemm(dev_bf16(A), dev_bf16(B), b_layout=wl.B_KN, out_dtype=torch.float32)
    exact(out, oracle.gemm(A, B, wl.B_KN), f"medium {shape}")


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("shape", [(4352, 4352, 72), (2304, 2304, 72)])
def test_last_round_split_by_columns(shape, layout):
    """Tile counts that leave most workgroups idle in the last round, whose tiles then run as
    column halves on two workgroups (on an MI355X: 289 large tiles, the last 33 split; 324
    medium tiles, the last 68 split).  Integer data, bit-exact against the oracle, guard rows
    untouched."""
    M, N, K = shape
    rng = np.random.default_rng(M + K)
    A = int_bf16(rng, (M, K))
    B = int_bf16(rng, (K, N) if layout == wl.B_KN else (N, K))
    buf = torch.full((M + 2, N), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[1:M + 1]
    ptg.gemm(dev_bf16(A), dev_bf16(B), b_layout=layout, out=out)
    exact(out, oracle.gemm(A, B, layout), f"dense last round split {shape} layout={layout}")
    assert bool(torch.isnan(buf[0]).all()) and bool(torch.isnan(buf[M + 1]).all()), "guard rows written"


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("epi", [wl.EPI_NONE, wl.EPI_BIAS_SILU])
def test_large_tiles_ragged(layout, epi):
    """Large-tile path (>= 128 tiles of 256 x 256) with ragged M, N and K; sampled rows."""
    M, N, K = 4096 + 40, 2048 + 24, 264
    assert ptg.describe_config(M, N, K, layout)["BM"] == 256
    w = wl.dense(21 + layout, M, N, K, dist="normal", b_layout=layout, scale=K ** -0.5,
                 with_bias=True)
    rows = np.concatenate([sample_rows(M, 96, 1), np.arange(M - 40, M)])
    rows = np.unique(rows)
    for out_dtype in (torch.float32, torch.bfloat16):
        out, v = run_dense(w, out_dtype, epi, rows=rows)
        check(out[torch.from_numpy(rows).cuda()], v, K, f"large {M}x{N}x{K} {out_dtype}")


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("shape", [(1000, 1032, 1096), (4096, 4096, 1024)])
def test_integer_exact(layout, shape):
    """Integer entries: any summation order is exact in fp32, so the result is bit-exact.
    Pins the whole pipeline: no k-step lost, repeated or read from a stale ring slot.  Every
    element is compared."""
    M, N, K = shape
    rng = np.random.default_rng(M + K + layout)
    A = int_bf16(rng, (M, K))
    Bkn = int_bf16(rng, (K, N))
    B = Bkn if layout == wl.B_KN else np.ascontiguousarray(Bkn.T)
    out = ptg.gemm(dev_bf16(A), dev_bf16(B), b_layout=layout, out_dtype=torch.float32)
    exact(out, oracle.gemm(A, B, layout), f"integer {shape}")


def test_integer_exact_8192_full():
    """The headline shape and launch configuration (8192^3, B stored N x K, large tiles) on
    integer entries in [-4, 4]: every partial sum is an integer below 2^24, exact in fp32 in
    any order, so the whole 8192 x 8192 output must equal the oracle bit for bit (fp32
    output), and the bf16 output must be its correct rounding.  The same B stored K x N (its
    transpose, the other form of the kernel) must give the same fp32 output."""
    M = N = K = 8192
    rng = np.random.default_rng(8192)
    A = int_bf16(rng, (M, K))
    B = int_bf16(rng, (N, K))
    assert ptg.describe_config(M, N, K, wl.B_NK)["BM"] == 256
    dA, dB = dev_bf16(A), dev_bf16(B)
    out = ptg.gemm(dA, dB, b_layout=wl.B_NK, out_dtype=torch.float32)
    out16 = ptg.gemm(dA, dB, b_layout=wl.B_NK, out_dtype=torch.bfloat16)
    dBt = dB.t().contiguous()
    del dB
    out_kn = ptg.gemm(dA, dBt, b_layout=wl.B_KN, out_dtype=torch.float32)
    del dA, dBt
    v = oracle.gemm(A, B, wl.B_NK)
    exact(out, v, "integer 8192^3 fp32")
    exact(out16, v, "integer 8192^3 bf16")
    exact(out_kn, v, "integer 8192^3 fp32, B stored K x N")


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_identity_and_permutation(layout, out_dtype):
    rng = np.random.default_rng(5)
    M, K = 300, 264
    A = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (M, K)).astype(np.float32))
    eye = wl.f32_to_bf16_bits(np.eye(K, dtype=np.float32))
    out = ptg.gemm(dev_bf16(A), dev_bf16(eye), b_layout=layout, out_dtype=out_dtype)
    exact(out, wl.bf16_bits_to_f32(A).astype(np.float64), "A.I")
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.float32)
    P[perm, np.arange(K)] = 1.0          # (A P)[:, j] = A[:, perm[j]]
    Pb = wl.f32_to_bf16_bits(P)
    Pl = Pb if layout == wl.B_KN else np.ascontiguousarray(Pb.T)
    out = ptg.gemm(dev_bf16(A), dev_bf16(Pl), b_layout=layout, out_dtype=out_dtype)
    exact(out, wl.bf16_bits_to_f32(A).astype(np.float64)[:, perm], "A.P")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_guard_bands_and_strides(out_dtype):
    """Output written through a strided view inside a NaN-filled buffer: every element of
    the view is written, nothing outside it is touched."""
    rng = np.random.default_rng(8)
    M, N, K = 130, 72, 96
    A = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (M, K)).astype(np.float32))
    B = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (K, N)).astype(np.float32))
    big = torch.full((M + 2, N + 24), float("nan"), dtype=out_dtype, device="cuda")
    view = big[1:M + 1, 8:8 + N]
    ptg.gemm(dev_bf16(A), dev_bf16(B), out=view)
    v = oracle.gemm(A, B, wl.B_KN)
    check(view, v, K, "strided view")
    g = big.float().cpu()
    inside = torch.zeros_like(g, dtype=torch.bool)
    inside[1:M + 1, 8:8 + N] = True
    assert torch.isnan(g[~inside]).all(), "guard band overwritten"
    assert not torch.isnan(g[inside]).any(), "element of the output left unwritten"


def test_strided_inputs():
    """lda and ldb larger than the row length (views into wider buffers)."""
    rng = np.random.default_rng(9)
    M, N, K = 257, 96, 136
    Aw = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (M, K + 40)).astype(np.float32))
    Bw = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (K, N + 16)).astype(np.float32))
    A, B = dev_bf16(Aw)[:, 8:8 + K], dev_bf16(Bw)[:, :N]
    out = ptg.gemm(A, B, out_dtype=torch.float32)
    v = oracle.gemm(np.ascontiguousarray(Aw[:, 8:8 + K]), np.ascontiguousarray(Bw[:, :N]), wl.B_KN)
    check(out, v, K, "strided inputs")


def test_degenerate_sizes():
    A = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda")
    assert ptg.gemm(A, B).shape == (0, 32)
    A = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((64, 0), dtype=torch.bfloat16, device="cuda")
    assert ptg.gemm(A, B).shape == (16, 0)
    # a single row, single column block, shortest legal K
    w = wl.dense(3, 1, 8, 8, dist="uniform")
    out, v = run_dense(w, torch.float32)
    check(out, v, 8, "1x8x8")


def test_repeat_is_deterministic():
    w = wl.dense(4, 700, 520, 1000, dist="normal", b_layout=wl.B_NK)
    A, B = dev_bf16(w.A), dev_bf16(w.B)
    o1 = ptg.gemm(A, B, b_layout=wl.B_NK, out_dtype=torch.float32)
    o2 = ptg.gemm(A, B, b_layout=wl.B_NK, out_dtype=torch.float32)
    assert torch.equal(o1, o2)


def test_config2_8192_sampled():
    """The benchmarked workload: 8192^3, B stored N x K, N(0,1)/sqrt(K) entries.
    bf16 output (as benchmarked) and its fp32 twin, on sampled rows."""
    w = wl.config2()
    A, B = dev_bf16(w.A), dev_bf16(w.B)
    rows = sample_rows(w.M, 62, 3)
    v = oracle.gemm(w.A, w.B, wl.B_NK, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    for out_dtype in (torch.bfloat16, torch.float32):
        out = ptg.gemm(A, B, b_layout=wl.B_NK, out_dtype=out_dtype)
        check(out[idx], v, w.K, f"config2 {out_dtype}")
