"""GPU parity of the one-role dense kernel (every wave both copies and computes; 256 x 256 x 32
tiles in five LDS slots) against the fp64 CPU oracle.

ptg_gemm takes this kernel when K is a multiple of 32 and the output has at least 128 tiles of
256 x 256 (or more tiles of 128 x 128 than the device has CUs), with B stored N x K or K x N (whose fragments are read with transposing LDS reads).  The cases cover every remainder of the unrolled k-loop (ten
32-deep steps per pass: one to ten steps after zero, one or two passes), output grids whose 16 x 16 tile blocks and 4-row strips are partial
(including the reversed odd block rows), ragged M and N, every epilogue and both output types,
and strided operands and outputs inside guard bands.  Integer data make the fp32 result exact
in any summation order, so those cases are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import check, dev, dev_bf16, exact, int_bf16, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_watchdog():
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0, "a range check of the kernel fired"


def onerole(M, N, K, layout=wl.B_NK) -> bool:
    return ptg.describe_config(M, N, K, layout)["producers"] == 0


def b_of(rng, N, K, layout):
    return int_bf16(rng, (N, K) if layout == wl.B_NK else (K, N))


LAYOUTS = [wl.B_NK, wl.B_KN]


def test_routing():
    assert onerole(8192, 8192, 8192)
    assert onerole(4096, 2048, 32)
    assert onerole(8192, 8192, 8192, wl.B_KN)
    assert not onerole(4096, 4096, 264)                # K not a multiple of 32
    assert not onerole(4096, 4096, 264, wl.B_KN)
    assert not onerole(2048, 2048, 1024)               # 64 tiles; 256 medium tiles fill one round
    assert onerole(2304, 2304, 512)                    # 81 tiles; 324 medium tiles need two rounds
    assert onerole(4096, 1536, 4096, wl.B_KN)          # 96 tiles
    cfg = ptg.describe_config(8192, 8192, 8192, wl.B_NK)
    assert (cfg["BM"], cfg["BN"], cfg["BK"], cfg["stages"]) == (256, 256, 32, 5)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("steps", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 15, 20, 21])
def test_every_loop_remainder_integer_exact(steps, layout):
    """K = 32 steps: the unrolled loop runs ten steps per pass and finishes with one to ten;
    copies go in pairs of steps (odd step counts leave a pair half past K).  4096 x 2048 (128
    tiles, one round), every element bit-exact in fp32 and bf16."""
    M, N, K = 4096, 2048, 32 * steps
    assert onerole(M, N, K, layout)
    rng = np.random.default_rng(100 + steps + layout)
    A, B = int_bf16(rng, (M, K)), b_of(rng, N, K, layout)
    dA, dB = dev_bf16(A), dev_bf16(B)
    v = oracle.gemm(A, B, layout)
    exact(ptg.gemm(dA, dB, b_layout=layout, out_dtype=torch.float32), v, f"K={K} layout={layout} fp32")
    exact(ptg.gemm(dA, dB, b_layout=layout, out_dtype=torch.bfloat16), v, f"K={K} layout={layout} bf16")


@pytest.mark.parametrize("shape", [(4196, 2088, 96),       # 17 x 9 tiles: a one-row last block row
                                   (8392, 4392, 64),       # 33 x 18: reversed odd block rows whose
                                                           # narrow last block column comes first
                                   (4100, 8200, 160),      # 17 x 33: three block columns, the last
                                                           # one tile wide
                                   (4600, 3000, 128)])     # 18 x 12: a last strip of two tile rows
@pytest.mark.parametrize("layout", LAYOUTS)
def test_tile_order_edges_integer_exact(shape, layout):
    """Output grids whose tile blocks and strips are partial: every tile is computed exactly
    once (the output is NaN-filled first) and every element is bit-exact."""
    M, N, K = shape
    assert onerole(M, N, K, layout)
    rng = np.random.default_rng(M + N + K + layout)
    A, B = int_bf16(rng, (M, K)), b_of(rng, N, K, layout)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ptg.gemm(dev_bf16(A), dev_bf16(B), b_layout=layout, out=out)
    exact(out, oracle.gemm(A, B, layout), f"one-role {shape} layout={layout}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("epi", [wl.EPI_NONE, wl.EPI_BIAS, wl.EPI_SILU, wl.EPI_BIAS_SILU])
def test_epilogues_ragged(epi, layout):
    """Ragged M and N, N(0,1)/sqrt(K) data, every epilogue, both output types; sampled rows
    plus the whole last (partial) row of tiles against the oracle."""
    M, N, K = 4096 + 40, 2048 + 24, 288
    assert onerole(M, N, K, layout)
    w = wl.dense(31 + layout, M, N, K, dist="normal", b_layout=layout, scale=K ** -0.5, with_bias=True)
    A, B, bias = dev_bf16(w.A), dev_bf16(w.B), dev(w.bias)
    rows = np.unique(np.concatenate([sample_rows(M, 64, 2), np.arange(M - 40, M)]))
    v = oracle.gemm(w.A, w.B, layout, w.bias, epi, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    for out_dtype in (torch.float32, torch.bfloat16):
        out = ptg.gemm(A, B, b_layout=layout, out_dtype=out_dtype, bias=bias, epi=epi)
        check(out[idx], v, K, f"one-role epi={epi} layout={layout} {out_dtype}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_strided_operands_and_guard_bands(out_dtype, layout):
    """lda, ldb > K and ldc > N (views into wider buffers); the output view sits inside a
    NaN-filled buffer: every element of the view is written, nothing around it."""
    M, N, K = 4096 + 8, 2048 + 16, 128
    assert onerole(M, N, K, layout)
    rng = np.random.default_rng(77 + layout)
    Aw = int_bf16(rng, (M, K + 24))
    if layout == wl.B_NK:
        Bw = int_bf16(rng, (N, K + 40))
        Bh = np.ascontiguousarray(Bw[:, 16:16 + K])
        B = dev_bf16(Bw)[:, 16:16 + K]
    else:
        Bw = int_bf16(rng, (K, N + 40))
        Bh = np.ascontiguousarray(Bw[:, 16:16 + N])
        B = dev_bf16(Bw)[:, 16:16 + N]
    A = dev_bf16(Aw)[:, 8:8 + K]
    big = torch.full((M + 2, N + 24), float("nan"), dtype=out_dtype, device="cuda")
    view = big[1:M + 1, 8:8 + N]
    ptg.gemm(A, B, b_layout=layout, out=view)
    v = oracle.gemm(np.ascontiguousarray(Aw[:, 8:8 + K]), Bh, layout)
    exact(view, v, "one-role strided")
    g = big.float()
    inside = torch.zeros_like(g, dtype=torch.bool)
    inside[1:M + 1, 8:8 + N] = True
    assert bool(torch.isnan(g[~inside]).all()), "guard band overwritten"


@pytest.mark.parametrize("layout", LAYOUTS)
def test_fewer_large_tiles_than_half_the_chip(layout):
    """A grid of 9 x 9 large tiles (81, under 128, but 324 medium tiles: more than one round),
    ragged in M and N, integer data, bit-exact."""
    M, N, K = 2304 - 40, 2304 - 8, 384
    assert onerole(M, N, K, layout)
    rng = np.random.default_rng(2304 + layout)
    A, B = int_bf16(rng, (M, K)), b_of(rng, N, K, layout)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ptg.gemm(dev_bf16(A), dev_bf16(B), b_layout=layout, out=out)
    exact(out, oracle.gemm(A, B, layout), f"one-role 81 tiles layout={layout}")


def test_repeat_and_layouts_agree():
    """Two calls give the same bits; on integer data B stored N x K and its transpose stored
    K x N give the same result, and so does the two-role kernel (K not a multiple of 32: the
    same product with 8 zero columns of A and rows of B appended)."""
    M, N, K = 4096, 4096, 512
    rng = np.random.default_rng(5)
    A, Bnk = int_bf16(rng, (M, K)), int_bf16(rng, (N, K))
    dA = dev_bf16(A)
    dB = dev_bf16(Bnk)
    o1 = ptg.gemm(dA, dB, b_layout=wl.B_NK, out_dtype=torch.float32)
    o2 = ptg.gemm(dA, dB, b_layout=wl.B_NK, out_dtype=torch.float32)
    assert torch.equal(o1, o2)
    o3 = ptg.gemm(dA, dB.t().contiguous(), b_layout=wl.B_KN, out_dtype=torch.float32)
    assert torch.equal(o1, o3)
    assert not onerole(M, N, K + 8)
    zA = torch.cat([dA, torch.zeros((M, 8), dtype=torch.bfloat16, device="cuda")], 1)
    zB = torch.cat([dB, torch.zeros((N, 8), dtype=torch.bfloat16, device="cuda")], 1)
    o4 = ptg.gemm(zA, zB, b_layout=wl.B_NK, out_dtype=torch.float32)
    assert torch.equal(o1, o4)
