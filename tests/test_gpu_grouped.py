"""GPU parity of the grouped (mixture-of-experts) GEMM against the fp64 CPU oracle.

Expert row ranges come from device-resident int32 offsets with empty groups, groups
smaller than a tile, and (at full size) the 64-expert Zipf(1.1) routing of the workload.
Group bookkeeping is pinned bit-exactly with W_g = (g + 1) I.
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
    assert ptg.watchdog(clear=True) == 0, "a pipeline wait timed out"


def run_grouped(w: wl.Grouped, out_dtype, epi, rows=None):
    out = ptg.grouped_gemm(dev_bf16(w.X), dev_bf16(w.W), dev(w.offsets), w_layout=w.w_layout,
                           out_dtype=out_dtype, bias=dev(w.bias) if w.bias is not None else None,
                           epi=epi)
    v = oracle.grouped_gemm(w.X, w.W, w.w_layout, w.offsets, w.bias, epi, rows=rows)
    return out, v


COUNTS = np.array([300, 0, 1, 129, 0, 0, 64, 511, 2, 0])


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("epi", [wl.EPI_NONE, wl.EPI_BIAS_SILU])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_small(layout, epi, out_dtype):
    w = wl.grouped(31, len(COUNTS), int(COUNTS.sum()), 200, 136, w_layout=layout,
                   with_bias=True, counts=COUNTS)
    out, v = run_grouped(w, out_dtype, epi)
    check(out, v, w.K, f"grouped layout={layout} epi={epi}")


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
def test_grouped_scaled_identity_pins_groups(layout):
    """W_g = (g+1) I with integer X: row r must equal (g(r)+1) X[r] exactly."""
    counts = np.array([5, 0, 130, 1, 0, 257, 3, 0])
    G, K = len(counts), 128
    M = int(counts.sum())
    rng = np.random.default_rng(4)
    X = int_bf16(rng, (M, K))
    W = np.stack([wl.f32_to_bf16_bits((g + 1) * np.eye(K, dtype=np.float32)) for g in range(G)])
    if layout == wl.B_NK:
        W = np.ascontiguousarray(W.transpose(0, 2, 1))
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    for out_dtype in (torch.float32, torch.bfloat16):
        out = ptg.grouped_gemm(dev_bf16(X), dev_bf16(W), dev(off), w_layout=layout, out_dtype=out_dtype)
        grp = np.repeat(np.arange(G), counts)
        exact(out, (grp[:, None] + 1) * wl.bf16_bits_to_f32(X).astype(np.float64), "scaled identity")


def test_grouped_equals_per_group_gemm():
    """Invariant: the grouped result equals a plain GEMM per expert (GPU against GPU)."""
    rng = np.random.default_rng(6)
    counts = np.array([77, 0, 256, 3, 190])
    G, K, N = len(counts), 192, 264
    M = int(counts.sum())
    X = int_bf16(rng, (M, K))
    W = int_bf16(rng, (G, K, N))
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    Xd, Wd = dev_bf16(X), dev_bf16(W)
    out = ptg.grouped_gemm(Xd, Wd, dev(off), out_dtype=torch.float32)
    for g in range(G):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            one = ptg.gemm(Xd[lo:hi], Wd[g], out_dtype=torch.float32)
            assert torch.equal(out[lo:hi], one)


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
def test_grouped_tile_boundaries_guard_rows(layout):
    """Experts of exactly 128 and 256 rows and one more or one less (the split between the
    half tiles, whose upper consumer waves idle, and the full tiles), an empty expert and a
    one-row expert: integer data, bit-exact against the oracle, guard rows untouched."""
    counts = np.array([128, 256, 129, 0, 257, 384, 127, 1])
    G, K, N = len(counts), 136, 264
    M = int(counts.sum())
    rng = np.random.default_rng(9)
    X = int_bf16(rng, (M, K))
    W = int_bf16(rng, (G, K, N) if layout == wl.B_KN else (G, N, K))
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    buf = torch.full((M + 2, N), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[1:M + 1]
    ptg.grouped_gemm(dev_bf16(X), dev_bf16(W), dev(off), w_layout=layout, out=out)
    exact(out, oracle.grouped_gemm(X, W, layout, off), f"grouped tile boundaries layout={layout}")
    assert bool(torch.isnan(buf[0]).all()) and bool(torch.isnan(buf[M + 1]).all()), "guard rows written"


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
def test_grouped_last_round_split_by_columns(layout):
    """A last round with idle workgroups: its full tiles run as two column halves on two
    workgroups (on an MI355X, 328 tiles on 256 workgroups: 64 full tiles split into 128 units,
    then 8 half tiles).  Integer data, bit-exact against the oracle, guard rows untouched."""
    counts = np.array([40 * 256, 100])
    G, K, N = len(counts), 72, 2048
    M = int(counts.sum())
    rng = np.random.default_rng(13)
    X = int_bf16(rng, (M, K))
    W = int_bf16(rng, (G, K, N) if layout == wl.B_KN else (G, N, K))
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    buf = torch.full((M + 2, N), float("nan"), dtype=torch.float32, device="cuda")
    out = buf[1:M + 1]
    ptg.grouped_gemm(dev_bf16(X), dev_bf16(W), dev(off), w_layout=layout, out=out)
    exact(out, oracle.grouped_gemm(X, W, layout, off), f"grouped last round split, layout={layout}")
    assert bool(torch.isnan(buf[0]).all()) and bool(torch.isnan(buf[M + 1]).all()), "guard rows written"


def test_grouped_every_tile_split_when_the_grid_exceeds_the_tiles():
    """The grid is sized from an upper bound on the tile count (every group may add a partial
    m-tile), so a small problem can have fewer tiles than workgroups: then every full tile runs
    as two column halves (here 4 tiles, 8 units).  Integer data, bit-exact."""
    counts = np.array([512, 0, 0, 0, 0, 0, 0, 0])
    G, K, N = len(counts), 72, 512
    M = int(counts.sum())
    rng = np.random.default_rng(14)
    X = int_bf16(rng, (M, K))
    W = int_bf16(rng, (G, K, N))
    off = np.zeros(G + 1, np.int32)
    off[1:] = np.cumsum(counts)
    out = ptg.grouped_gemm(dev_bf16(X), dev_bf16(W), dev(off), out_dtype=torch.float32)
    exact(out, oracle.grouped_gemm(X, W, wl.B_KN, off), "grouped, every tile split")


def test_grouped_single_group_is_dense():
    w = wl.grouped(8, 1, 333, 136, 200, counts=np.array([333]))
    out, v = run_grouped(w, torch.float32, wl.EPI_NONE)
    dense = ptg.gemm(dev_bf16(w.X), dev_bf16(w.W[0]), out_dtype=torch.float32)
    check(out, v, w.K, "single group")
    assert torch.equal(out, dense)


def test_grouped_check_helper():
    off = torch.tensor([0, 3, 2, 5], dtype=torch.int32, device="cuda")
    with pytest.raises(ptg.PtgError) as e:
        ptg.grouped_gemm_check(off, 5)
    assert e.value.status == 5
    ptg.grouped_gemm_check(torch.tensor([0, 2, 2, 5], dtype=torch.int32, device="cuda"), 5)


@pytest.mark.parametrize("reading", ["rank", "sampled"])
def test_config3_moe_sampled(reading):
    """64 experts, 16384 rows (Zipf(1.1) routing), K = 4096, N = 1536; bf16 output and the
    fp32 twin on sampled rows: first and last row of every live group plus random rows."""
    w = wl.config3(reading)
    rows = set(sample_rows(w.M_total, 64, 7).tolist())
    for g in range(w.G):
        if w.counts[g] > 0:
            rows |= {int(w.offsets[g]), int(w.offsets[g + 1]) - 1}
    rows = np.array(sorted(rows), dtype=np.int64)
    v = oracle.grouped_gemm(w.X, w.W, w.w_layout, w.offsets, rows=rows)
    X, W, off = dev_bf16(w.X), dev_bf16(w.W), dev(w.offsets)
    idx = torch.from_numpy(rows).cuda()
    for out_dtype in (torch.bfloat16, torch.float32):
        out = ptg.grouped_gemm(X, W, off, out_dtype=out_dtype)
        check(out[idx], v, w.K, f"config3 {reading} {out_dtype}")


# ------------------------------------------------------------------------------------------
# reduction split of the last round (ptg_grouped_gemm_split)
# ------------------------------------------------------------------------------------------
def split_workspace(garbage=True):
    ws = torch.empty(ptg.grouped_gemm_split_workspace(), dtype=torch.uint8, device="cuda")
    if garbage:
        ws.random_(0, 256)     # its content on entry does not matter
    return ws


def offsets_of(counts):
    off = np.zeros(len(counts) + 1, np.int32)
    off[1:] = np.cumsum(counts)
    return off


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_grouped_split_reduction_of_half_tiles(layout, out_dtype):
    """32 experts of 300 rows between empty ones, K = 512, N = 1536: on an MI355X 192 full and
    192 half tiles, so the last round's 128 half tiles run as 256 reduction halves, combined in
    a workspace filled with random bytes.  Integer data (every partial sum exact): bit-exact
    against the oracle, guard rows untouched; a second call on the same workspace too."""
    counts = np.array([300, 0] * 16 + [0, 300] * 16)
    G, K, N = len(counts), 512, 1536
    M = int(counts.sum())
    rng = np.random.default_rng(21 + layout)
    X = int_bf16(rng, (M, K))
    W = int_bf16(rng, (G, K, N) if layout == wl.B_KN else (G, N, K))
    off = offsets_of(counts)
    v = oracle.grouped_gemm(X, W, layout, off)
    ws = split_workspace()
    dX, dW, doff = dev_bf16(X), dev_bf16(W), dev(off)
    for call in range(2):
        buf = torch.full((M + 2, N), float("nan"), dtype=out_dtype, device="cuda")
        out = buf[1:M + 1]
        ptg.grouped_gemm(dX, dW, doff, w_layout=layout, out=out, workspace=ws)
        exact(out, v, f"split half tiles layout={layout} call {call}")
        assert bool(torch.isnan(buf[0].float()).all()) and bool(torch.isnan(buf[M + 1].float()).all())


def test_grouped_split_reduction_of_full_tiles_and_bias():
    """N = 1288 (not a multiple of the tile width, so no column split): one expert of 50 full
    m-tiles gives 300 tiles, and the last round's 44 full tiles run as reduction halves; the
    bias + SiLU epilogue runs once, on the combined sum.  Against the oracle, fp32 output."""
    counts = np.array([50 * 256, 0, 0])
    G, K, N = len(counts), 256, 1288
    w = wl.grouped(22, G, int(counts.sum()), K, N, with_bias=True, counts=counts)
    out = ptg.grouped_gemm(dev_bf16(w.X), dev_bf16(w.W), dev(w.offsets), out_dtype=torch.float32,
                           bias=dev(w.bias), epi=wl.EPI_BIAS_SILU, workspace=split_workspace())
    v = oracle.grouped_gemm(w.X, w.W, w.w_layout, w.offsets, w.bias, wl.EPI_BIAS_SILU)
    check(out, v, K, "split full tiles, bias + silu")


@pytest.mark.parametrize("reading", ["rank", "sampled"])
def test_config3_moe_split(reading):
    """The MoE workload through ptg_grouped_gemm_split, on sampled rows (first and last row of
    every live expert).  Rank-Zipf routing ends on 106 half tiles that run as reduction halves:
    within tolerance, and not bit-identical to the unsplit launch (the halves really ran
    separately).  Zipf-sampled routing ends on full tiles, split by columns only: bit-identical
    to the unsplit launch."""
    w = wl.config3(reading)
    rows = set(sample_rows(w.M_total, 64, 8).tolist())
    for g in range(w.G):
        if w.counts[g] > 0:
            rows |= {int(w.offsets[g]), int(w.offsets[g + 1]) - 1}
    rows = np.array(sorted(rows), dtype=np.int64)
    v = oracle.grouped_gemm(w.X, w.W, w.w_layout, w.offsets, rows=rows)
    X, W, off = dev_bf16(w.X), dev_bf16(w.W), dev(w.offsets)
    idx = torch.from_numpy(rows).cuda()
    ws = split_workspace()
    for out_dtype in (torch.bfloat16, torch.float32):
        out = ptg.grouped_gemm(X, W, off, out_dtype=out_dtype, workspace=ws)
        check(out[idx], v, w.K, f"config3 split {reading} {out_dtype}")
    plain = ptg.grouped_gemm(X, W, off, out_dtype=torch.float32)
    if reading == "rank":
        assert not torch.equal(out, plain)
    else:
        assert torch.equal(out, plain)
