"""GPU parity of the in-kernel broadcast GEMM and of the pointer-array grouped GEMM (a batch of
independent problems in one launch)."""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import check, dev, dev_bf16, exact, host_f32, int_bf16, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_watchdog():
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0, "a pipeline wait timed out"


def run_broadcast(w: wl.Broadcast, out_dtype, epi, rows=None):
    out = ptg.broadcast_gemm(dev_bf16(w.Xu), dev_bf16(w.Xc), dev(w.idx), dev_bf16(w.W),
                             w_layout=w.w_layout, out_dtype=out_dtype,
                             bias=dev(w.bias) if w.bias is not None else None, epi=epi)
    v = oracle.broadcast_gemm(w.Xu, w.Xc, w.idx, w.W, w.w_layout, w.bias, epi, rows=rows)
    return out, v


# ------------------------------------------------------------------------------------------
# broadcast
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
@pytest.mark.parametrize("epi", [wl.EPI_NONE, wl.EPI_BIAS_SILU])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shuffle", [False, True])
def test_broadcast_small(layout, epi, out_dtype, shuffle):
    w = wl.broadcast(41, 5, 264, 136, 200, cmin=1, cmax=300, w_layout=layout, with_bias=True,
                     shuffle=shuffle)
    out, v = run_broadcast(w, out_dtype, epi)
    check(out, v, w.Ku + w.Kc, f"broadcast layout={layout} epi={epi} shuffle={shuffle}")


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
def test_broadcast_block_identities(layout):
    """W = [I; 0] returns Xu[idx] exactly (pins the gather); W = [0; I] returns Xc."""
    rng = np.random.default_rng(3)
    U, Ku, Kc, Mc = 7, 128, 128, 555
    Xu = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (U, Ku)).astype(np.float32))
    Xc = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (Mc, Kc)).astype(np.float32))
    idx = rng.integers(0, U, Mc).astype(np.int32)
    top = wl.f32_to_bf16_bits(np.concatenate([np.eye(Ku), np.zeros((Kc, Ku))]).astype(np.float32))
    bot = wl.f32_to_bf16_bits(np.concatenate([np.zeros((Ku, Kc)), np.eye(Kc)]).astype(np.float32))
    for W, want in ((top, wl.bf16_bits_to_f32(Xu).astype(np.float64)[idx]),
                    (bot, wl.bf16_bits_to_f32(Xc).astype(np.float64))):
        Wl = W if layout == wl.B_KN else np.ascontiguousarray(W.T)
        for out_dtype in (torch.float32, torch.bfloat16):
            out = ptg.broadcast_gemm(dev_bf16(Xu), dev_bf16(Xc), dev(idx), dev_bf16(Wl),
                                     w_layout=layout, out_dtype=out_dtype)
            exact(out, want, "block identity")


def test_broadcast_equals_materialised_gemm():
    """Invariant: broadcast equals a plain GEMM on the explicitly materialised input."""
    rng = np.random.default_rng(12)
    U, Ku, Kc, N, Mc = 6, 192, 64, 136, 901
    Xu, Xc = int_bf16(rng, (U, Ku)), int_bf16(rng, (Mc, Kc))
    W = int_bf16(rng, (Ku + Kc, N))
    idx = rng.integers(0, U, Mc).astype(np.int32)
    out = ptg.broadcast_gemm(dev_bf16(Xu), dev_bf16(Xc), dev(idx), dev_bf16(W), out_dtype=torch.float32)
    Z = np.concatenate([Xu[idx], Xc], axis=1)
    ref = ptg.gemm(dev_bf16(Z), dev_bf16(W), out_dtype=torch.float32)
    assert torch.equal(out, ref)


@pytest.mark.parametrize("Ku", [8, 72, 2048, 2056])
def test_broadcast_split_user_phase(Ku):
    """The user product is split along Ku (up to 32 slices of whole 64-deep k-steps, the last
    possibly short) and the partials summed in slice order: against the oracle, and
    bit-identical from call to call (the sum does not depend on timing)."""
    w = wl.broadcast(61 + Ku, 3, Ku, 40, 136, cmin=1, cmax=90, w_layout=wl.B_NK, with_bias=True)
    out, v = run_broadcast(w, torch.float32, wl.EPI_BIAS)
    check(out, v, w.Ku + w.Kc, f"broadcast split user phase Ku={Ku}")
    again, _ = run_broadcast(w, torch.float32, wl.EPI_BIAS)
    assert torch.equal(out, again)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_broadcast_large_tiles_runs_of_users_guard_rows(out_dtype):
    """Candidate phase on the large tiles (at least 128 tiles of 256 x 256) with candidates in
    runs of one user, as in the workload, so that most waves gather a single user row of P, and
    a ragged last tile: integer data, bit-exact against the oracle, and the rows around the
    output (NaN sentinels) untouched."""
    rng = np.random.default_rng(12)
    U, Ku, Kc, N = 7, 64, 72, 1024
    counts = rng.integers(300, 2500, U)
    idx = np.repeat(np.arange(U), counts).astype(np.int32)
    Mc = int(idx.size)
    assert Mc % 256 != 0 and ptg.describe_config(Mc, N, Kc, wl.B_KN)["BM"] == 256
    Xu, Xc, W = int_bf16(rng, (U, Ku)), int_bf16(rng, (Mc, Kc)), int_bf16(rng, (Ku + Kc, N))
    buf = torch.full((Mc + 2, N), float("nan"), dtype=out_dtype, device="cuda")
    out = buf[1:Mc + 1]
    ptg.broadcast_gemm(dev_bf16(Xu), dev_bf16(Xc), dev(idx), dev_bf16(W), out=out)
    v = oracle.broadcast_gemm(Xu, Xc, idx, W, wl.B_KN)
    exact(out, v, f"broadcast large tiles, runs of users, {out_dtype}")
    assert bool(torch.isnan(buf[0]).all()) and bool(torch.isnan(buf[Mc + 1]).all()), "guard rows written"


@pytest.mark.parametrize("U,Ku,Kc,N,layout", [
    (61, 1000, 200, 712, wl.B_KN),   # 8 user slices (the last short), 8 reduction rows per unit
    (61, 1000, 200, 712, wl.B_NK),
    (256, 136, 72, 264, wl.B_KN),    # the most users in one m-tile, 3 slices
    (7, 72, 40, 136, wl.B_NK),       # 2 slices (the second 8 deep), one ragged column block
])
def test_broadcast_fused_exact(U, Ku, Kc, N, layout):
    """The one-launch form: user units write partial products, reduction units sum them into P
    once every partial of their column block has arrived, candidate tiles start from P once
    their column block is ready.  Integer data with a bias, candidates in runs of one user, a
    ragged last column block and tile: bit-exact against the oracle in both output types; the
    rows around the output (NaN sentinels) untouched; a second call on the same workspace (whose
    flags, partials and P the first call left behind) bit-identical."""
    rng = np.random.default_rng(U * 7 + N + layout)
    counts = rng.integers(1, 2 * 4000 // U, U)  # about 4000 candidates
    idx = np.repeat(np.arange(U), counts).astype(np.int32)
    Mc = int(idx.size)
    Xu, Xc = int_bf16(rng, (U, Ku)), int_bf16(rng, (Mc, Kc))
    W = int_bf16(rng, (Ku + Kc, N))
    Wl = W if layout == wl.B_KN else np.ascontiguousarray(W.T)
    bias = rng.integers(-8, 9, N).astype(np.float32)
    v = oracle.broadcast_gemm(Xu, Xc, idx, Wl, layout, bias, wl.EPI_BIAS)
    ws = torch.empty(ptg.broadcast_gemm_fused_workspace(U, N), dtype=torch.uint8, device="cuda")
    args = (dev_bf16(Xu), dev_bf16(Xc), dev(idx), dev_bf16(Wl))
    for out_dtype in (torch.float32, torch.bfloat16):
        first = None
        for call in range(2):
            buf = torch.full((Mc + 2, N), float("nan"), dtype=out_dtype, device="cuda")
            out = buf[1:Mc + 1]
            ptg.broadcast_gemm_fused(*args, w_layout=layout, out=out, bias=dev(bias), epi=wl.EPI_BIAS,
                                     workspace=ws)
            exact(out, v, f"broadcast U={U} Ku={Ku} N={N} layout={layout} {out_dtype} call {call}")
            assert bool(torch.isnan(buf[0]).all()) and bool(torch.isnan(buf[Mc + 1]).all()), "guard rows written"
            if first is None:
                first = out.clone()
            else:
                assert torch.equal(first, out), "second call differs"


@pytest.mark.parametrize("shuffle", [False, True])
def test_broadcast_fused_silu_matches_oracle(shuffle):
    """The one-launch form with the fused bias and SiLU on N(0,1) data, candidates in runs of
    one user or shuffled, against the fp64 oracle."""
    w = wl.broadcast(77, 40, 768, 320, 1024, cmin=20, cmax=400, w_layout=wl.B_NK, with_bias=True,
                     shuffle=shuffle)
    out = ptg.broadcast_gemm_fused(dev_bf16(w.Xu), dev_bf16(w.Xc), dev(w.idx), dev_bf16(w.W),
                                   w_layout=w.w_layout, out_dtype=torch.float32, bias=dev(w.bias),
                                   epi=wl.EPI_BIAS_SILU)
    v = oracle.broadcast_gemm(w.Xu, w.Xc, w.idx, w.W, w.w_layout, w.bias, wl.EPI_BIAS_SILU)
    check(out, v, w.Ku + w.Kc, f"broadcast fused, bias + SiLU, shuffle={shuffle}")


def test_broadcast_fused_full_workload_integer_exact():
    """The 64-user workload's shapes and user run lengths (81,403 candidates, [2048 | 512] ->
    1024) on integer data, where every sum is exact: the one-launch form equals the
    stream-ordered path on every element, and both equal the oracle on sampled rows (the first
    and last candidate of every user among them)."""
    w = wl.config4()
    rng = np.random.default_rng(44)
    Xu, Xc = int_bf16(rng, (w.U, w.Ku), -2, 2), int_bf16(rng, (w.Mc, w.Kc), -2, 2)
    W = int_bf16(rng, (w.Ku + w.Kc, w.N), -2, 2)
    bias = rng.integers(-8, 9, w.N).astype(np.float32)
    args = (dev_bf16(Xu), dev_bf16(Xc), dev(w.idx), dev_bf16(W))
    kw = dict(w_layout=wl.B_KN, out_dtype=torch.float32, bias=dev(bias), epi=wl.EPI_BIAS)
    plain = ptg.broadcast_gemm(*args, **kw)
    fused = ptg.broadcast_gemm_fused(*args, **kw)
    assert torch.equal(plain, fused), "the one-launch form differs from the stream-ordered path"
    starts = np.concatenate([[0], np.cumsum(w.counts)])
    rows = set(sample_rows(w.Mc, 48, 5).tolist()) | set(starts[:-1].tolist()) | set((starts[1:] - 1).tolist())
    rows = np.array(sorted(rows), dtype=np.int64)
    v = oracle.broadcast_gemm(Xu, Xc, w.idx, W, wl.B_KN, bias, wl.EPI_BIAS, rows=rows)
    exact(fused[torch.from_numpy(rows).cuda()], v, "broadcast fused, full workload, sampled rows")


def test_broadcast_fused_refuses_what_one_launch_cannot_do():
    """More users than one m-tile, or a user reduction of one k-step, is refused (the
    stream-ordered ptg_broadcast_gemm covers them)."""
    rng = np.random.default_rng(5)
    for U, Ku in ((300, 256), (4, 64)):
        Xu, Xc = int_bf16(rng, (U, Ku)), int_bf16(rng, (10, 64))
        W = int_bf16(rng, (Ku + 64, 128))
        idx = (np.arange(10) % U).astype(np.int32)
        with pytest.raises(ptg.PtgError):
            ptg.broadcast_gemm_fused(dev_bf16(Xu), dev_bf16(Xc), dev(idx), dev_bf16(W))


def test_broadcast_check_helper():
    idx = torch.tensor([0, 1, 4, 2], dtype=torch.int32, device="cuda")
    with pytest.raises(ptg.PtgError) as e:
        ptg.broadcast_gemm_check(4, idx)
    assert e.value.status == 5
    ptg.broadcast_gemm_check(5, idx)


def test_config4_ikbo_sampled():
    """64 users (Xu 64 x 2048), 81403 candidates (Xc x 512), W 2560 x 1024, bf16 output and
    its fp32 twin, on sampled rows including the first and last candidate of every user."""
    w = wl.config4()
    starts = np.concatenate([[0], np.cumsum(w.counts)])
    rows = set(sample_rows(w.Mc, 64, 9).tolist()) | set(starts[:-1].tolist()) | set((starts[1:] - 1).tolist())
    rows = np.array(sorted(rows), dtype=np.int64)
    v = oracle.broadcast_gemm(w.Xu, w.Xc, w.idx, w.W, w.w_layout, rows=rows)
    args = (dev_bf16(w.Xu), dev_bf16(w.Xc), dev(w.idx), dev_bf16(w.W))
    idx = torch.from_numpy(rows).cuda()
    for fn in (ptg.broadcast_gemm, ptg.broadcast_gemm_fused):
        for out_dtype in (torch.bfloat16, torch.float32):
            out = fn(*args, out_dtype=out_dtype)
            check(out[idx], v, w.Ku + w.Kc, f"config4 {fn.__name__} {out_dtype}")


# ------------------------------------------------------------------------------------------
# batch of independent problems
# ------------------------------------------------------------------------------------------
def run_batch(pl: wl.ProblemList, out_dtype, rows_per=None):
    probs, outs = [], []
    for p in pl.problems:
        C = torch.empty((p.M, p.N), dtype=out_dtype, device="cuda")
        probs.append((dev_bf16(p.A), dev_bf16(p.B), C, dev(p.bias)))
        outs.append(C)
    ptg.grouped_gemm_ptr_array(probs, pl.epi)
    vs = oracle.problem_list(pl.problems, pl.epi, rows_per)
    return outs, vs


@pytest.mark.parametrize("epi", [wl.EPI_NONE, wl.EPI_BIAS_SILU])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_batch_small(epi, out_dtype):
    pl = wl.problem_list(51, 9, mmin=1, mmax=300, nk_choices=(8, 136, 256), epi=epi)
    outs, vs = run_batch(pl, out_dtype)
    for i, (o, v) in enumerate(zip(outs, vs)):
        check(o, v, pl.problems[i].K, f"batch problem {i}")


def test_batch_prepare_once_run_twice():
    """The recorded batch can be re-run without re-preparing (no host work on run)."""
    pl = wl.problem_list(52, 5, mmin=64, mmax=200)
    probs, outs = [], []
    for p in pl.problems:
        C = torch.empty((p.M, p.N), dtype=torch.float32, device="cuda")
        probs.append((dev_bf16(p.A), dev_bf16(p.B), C, dev(p.bias)))
        outs.append(C)
    ws = torch.empty(ptg.grouped_gemm_ptr_array_workspace(len(probs)), dtype=torch.uint8, device="cuda")
    ptg.grouped_gemm_ptr_array_prepare(probs, pl.epi, ws)
    ptg.grouped_gemm_ptr_array_run(len(probs), ws, torch.float32, pl.epi)
    first = [o.clone() for o in outs]
    for o in outs:
        o.zero_()
    ptg.grouped_gemm_ptr_array_run(len(probs), ws, torch.float32, pl.epi)
    for a, b in zip(first, outs):
        assert torch.equal(a, b)
    vs = oracle.problem_list(pl.problems, pl.epi)
    for i, (o, v) in enumerate(zip(outs, vs)):
        check(o, v, pl.problems[i].K, f"problem {i}")


def test_batch_each_equals_standalone_gemm():
    pl = wl.problem_list(53, 6, mmin=1, mmax=700)
    probs = []
    for p in pl.problems:
        probs.append((dev_bf16(p.A), dev_bf16(p.B), torch.empty((p.M, p.N), dtype=torch.float32,
                      device="cuda"), dev(p.bias)))
    ptg.grouped_gemm_ptr_array(probs, pl.epi)
    for A, B, C, bias in probs:
        one = ptg.gemm(A, B, out_dtype=torch.float32, bias=bias, epi=pl.epi)
        assert torch.allclose(C, one, rtol=0, atol=0) or torch.equal(C, one)


def test_config5_recsys_batch_sampled():
    """1024 problems (M ~ U{64..1024}, N, K in {128, 256, 512}) in one persistent launch with
    the fused bias + SiLU epilogue; bf16 output and fp32 twin, sampled rows of every problem."""
    pl = wl.config5()
    rows_per = [sample_rows(p.M, 3, 100 + i) for i, p in enumerate(pl.problems)]
    vs = oracle.problem_list(pl.problems, pl.epi, rows_per)
    for out_dtype in (torch.bfloat16, torch.float32):
        probs, outs = [], []
        for p in pl.problems:
            C = torch.empty((p.M, p.N), dtype=out_dtype, device="cuda")
            probs.append((dev_bf16(p.A), dev_bf16(p.B), C, dev(p.bias)))
            outs.append(C)
        ptg.grouped_gemm_ptr_array(probs, pl.epi)
        for i, (o, v) in enumerate(zip(outs, vs)):
            check(o[torch.from_numpy(rows_per[i]).cuda()], v, pl.problems[i].K, f"config5 problem {i}")


def _small_batch(seed, n, out_dtype=torch.float32, epi=wl.EPI_BIAS_SILU):
    pl = wl.problem_list(seed, n, mmin=1, mmax=300, nk_choices=(8, 136, 256), epi=epi)
    probs, outs = [], []
    for p in pl.problems:
        C = torch.full((p.M, p.N), float("nan"), dtype=out_dtype, device="cuda")
        probs.append((dev_bf16(p.A), dev_bf16(p.B), C, dev(p.bias)))
        outs.append(C)
    return pl, probs, outs


def test_ptr_array_caller_array_reused_at_once():
    """The host problem array may be overwritten as soon as the call returns: the table was
    staged before the call returned, and the launch reads the staged copy."""
    import ctypes
    from pipelined_tiled_gemm_amd import _ffi
    pl, probs, outs = _small_batch(61, 7)
    arr, _ = ptg._problem_array(probs, pl.epi)
    ws = torch.empty(ptg.grouped_gemm_ptr_array_workspace(len(probs)), dtype=torch.uint8, device="cuda")
    L = _ffi.load()
    st = L.ptg_grouped_gemm_ptr_array(len(probs), arr, 1, pl.epi, ws.data_ptr(), ws.numel(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, ptg.last_error()
    ctypes.memset(arr, 0xFF, ctypes.sizeof(arr))      # garbage, before the stream has run
    torch.cuda.synchronize()
    vs = oracle.problem_list(pl.problems, pl.epi)
    for i, (o, v) in enumerate(zip(outs, vs)):
        check(o, v, pl.problems[i].K, f"problem {i}")


def test_ptr_array_many_calls_in_flight():
    """More back-to-back calls than the library keeps staging buffers (8), each with its own
    workspace, without a synchronisation between them: every call's table stays intact."""
    batches = [_small_batch(70 + k, 3 + k % 4) for k in range(20)]
    for pl, probs, _ in batches:
        ptg.grouped_gemm_ptr_array(probs, pl.epi)
    torch.cuda.synchronize()
    for k, (pl, probs, outs) in enumerate(batches):
        vs = oracle.problem_list(pl.problems, pl.epi)
        for i, (o, v) in enumerate(zip(outs, vs)):
            check(o, v, pl.problems[i].K, f"batch {k} problem {i}")


@pytest.mark.parametrize("change", ["epi", "dtype", "count"])
def test_ptr_array_run_with_another_table_is_refused_on_device(change):
    """A run whose epilogue, output type or count differs from what its table was written for
    writes nothing (the outputs keep their NaN fill) and sets watchdog bit 2."""
    pl, probs, outs = _small_batch(81, 5, epi=wl.EPI_NONE)
    ws = torch.empty(ptg.grouped_gemm_ptr_array_workspace(len(probs) + 1), dtype=torch.uint8, device="cuda")
    ptg.grouped_gemm_ptr_array_prepare(probs, wl.EPI_NONE, ws)
    torch.cuda.synchronize()
    epi = wl.EPI_SILU if change == "epi" else wl.EPI_NONE
    dtype = torch.bfloat16 if change == "dtype" else torch.float32
    count = len(probs) + 1 if change == "count" else len(probs)
    ptg.grouped_gemm_ptr_array_run(count, ws, dtype, epi)
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 2
    for o in outs:
        assert bool(torch.isnan(o).all()), "a refused launch wrote output"
    # the same table with matching arguments runs
    ptg.grouped_gemm_ptr_array_run(len(probs), ws, torch.float32, wl.EPI_NONE)
    vs = oracle.problem_list(pl.problems, wl.EPI_NONE)
    for i, (o, v) in enumerate(zip(outs, vs)):
        check(o, v, pl.problems[i].K, f"problem {i}")


def test_ptr_array_outputs_of_one_dtype():
    pl, probs, outs = _small_batch(91, 3)
    probs[1] = (probs[1][0], probs[1][1], probs[1][2].to(torch.bfloat16), probs[1][3])
    with pytest.raises(TypeError):
        ptg.grouped_gemm_ptr_array(probs, pl.epi)
    probs[1] = (probs[1][0], probs[1][1], outs[1], probs[1][3][:-8])
    with pytest.raises(ValueError):
        ptg.grouped_gemm_ptr_array(probs, pl.epi)     # bias shorter than N


def test_checks_concurrent_streams_and_watchdog():
    """The device-data checks on two streams at once each see their own result, and a set
    watchdog word makes a check fail."""
    good = torch.tensor([0, 3, 3, 10], dtype=torch.int32, device="cuda")
    bad = torch.tensor([0, 5, 3, 10], dtype=torch.int32, device="cuda")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(20):
        ptg.grouped_gemm_check(good, 10, stream=s1)
        with pytest.raises(ptg.PtgError):
            ptg.grouped_gemm_check(bad, 10, stream=s2)
    idx = torch.tensor([0, 1, 2, 1], dtype=torch.int32, device="cuda")
    ptg.broadcast_gemm_check(3, idx, stream=s1)
    with pytest.raises(ptg.PtgError):
        ptg.broadcast_gemm_check(2, idx, stream=s2)
