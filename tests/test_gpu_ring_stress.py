"""Ring-handoff stress: the library's test build libptg_delay.so (the same sources compiled with
PTG_DELAY_INJECT=1) pauses for a pseudo-random 0 to 8192 shader cycles before every fill signal,
release and wait of the LDS ring, in producers and consumers alike.  The handoff rule (a
producer never overwrites a slot still being read, a consumer never reads a slot before its
copy has landed; the yuxiaoba.github.io reading notes on "How We Built TLX", section "Tensor
expressions with explicit handoffs") must hold under any such timing, so on integer data every
result stays bit-exact against the oracle: a slot overwritten early or read stale would change
a sum.

Cases: the large tile (two 64 KB slots, register-staged producers) on long reductions (64
k-steps per tile) in both B layouts; the one-role kernel (five 32 KB slots that change hands
at a per-step barrier; the stress build pauses each wave before that barrier and between its
copies and fragment reads); the medium tile (four slots, buffer-to-LDS producers, two
ping-pong consumer groups); the grouped GEMM with empty experts and a column-split last round;
the weight gradient's dynamic tile queue; the pointer-array batch; the broadcast GEMM's one-launch
form, whose reduction units and candidate tiles wait on other workgroups' results.
"""
import contextlib

import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from pipelined_tiled_gemm_amd import _ffi, build
from parity import dev, dev_bf16, exact, int_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def delay_lib():
    return _ffi.open_library(build.variant_path("delay"))


@contextlib.contextmanager
def using(lib):
    """Route the binding's calls to `lib` (argument marshalling is the binding's own)."""
    saved = _ffi._lib
    _ffi._lib = lib
    try:
        yield
    finally:
        _ffi._lib = saved


@pytest.fixture(autouse=True)
def _no_watchdog(delay_lib):
    with using(delay_lib):
        ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    with using(delay_lib):
        assert ptg.watchdog(clear=True) == 0, "a pipeline wait of the stress build gave up"


@pytest.mark.parametrize("layout,K,stages,producers", [(wl.B_NK, 4104, 2, 4),   # two-role (K mod 32 = 8)
                                                       (wl.B_KN, 4104, 2, 4),   # two-role
                                                       (wl.B_NK, 4096, 5, 0),   # one-role
                                                       (wl.B_KN, 4096, 5, 0)])  # one-role
def test_stress_large_tile_long_k(delay_lib, layout, K, stages, producers):
    """Large tiles over a long K in the stress build: the two-role ring (producer and consumer
    waves hand slots over through LDS counters) and the one-role kernel (every wave copies and
    computes; slots change hands at the per-step barrier), each with pauses that skew the waves."""
    M = N = 4096
    rng = np.random.default_rng(K + layout)
    A = int_bf16(rng, (M, K))
    B = int_bf16(rng, (N, K) if layout == wl.B_NK else (K, N))
    cfg = ptg.describe_config(M, N, K, layout)
    assert (cfg["stages"], cfg["producers"]) == (stages, producers)
    dA, dB = dev_bf16(A), dev_bf16(B)
    with using(delay_lib):
        out = ptg.gemm(dA, dB, b_layout=layout, out_dtype=torch.float32)
    exact(out, oracle.gemm(A, B, layout), f"stress large 4096x4096x{K} layout={layout}")


def test_stress_is_slower_than_the_product_build(delay_lib):
    """The pauses are really there: the same call takes longer in the stress build."""
    M = N = 4096
    K = 2048
    rng = np.random.default_rng(7)
    dA, dB = dev_bf16(int_bf16(rng, (M, K))), dev_bf16(int_bf16(rng, (N, K)))
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def timed(n=5):
        ptg.gemm(dA, dB, b_layout=wl.B_NK, out=out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            ptg.gemm(dA, dB, b_layout=wl.B_NK, out=out)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    t_prod = timed()
    with using(delay_lib):
        t_stress = timed()
    print(f"product build {t_prod:.3f} ms, stress build {t_stress:.3f} ms")
    assert t_stress > 1.1 * t_prod


def test_stress_medium_tile_ping_pong(delay_lib):
    M, N, K = 1000, 1032, 2048
    rng = np.random.default_rng(11)
    A, B = int_bf16(rng, (M, K)), int_bf16(rng, (K, N))
    assert ptg.describe_config(M, N, K, wl.B_KN)["stages"] == 4
    with using(delay_lib):
        out = ptg.gemm(dev_bf16(A), dev_bf16(B), b_layout=wl.B_KN, out_dtype=torch.float32)
    exact(out, oracle.gemm(A, B, wl.B_KN), "stress medium")


def test_stress_grouped(delay_lib):
    """Experts of 0, 1, 128, 129, 300, 0, 700 and 2000 rows (empty, half and full tiles)."""
    counts = np.array([0, 1, 128, 129, 300, 0, 700, 2000])
    G, K, N = len(counts), 1024, 512
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rng = np.random.default_rng(12)
    X = int_bf16(rng, (int(off[-1]), K))
    W = int_bf16(rng, (G, K, N))
    Y = torch.full((int(off[-1]), N), float("nan"), dtype=torch.float32, device="cuda")
    with using(delay_lib):
        ptg.grouped_gemm(dev_bf16(X), dev_bf16(W), dev(off), out=Y)
    exact(Y, oracle.grouped_gemm(X, W, wl.B_KN, off), "stress grouped")


def test_stress_wgrad_queue(delay_lib):
    counts = np.array([40, 0, 300, 1, 513, 64])
    G, K, N = len(counts), 512, 256
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rng = np.random.default_rng(13)
    X = int_bf16(rng, (int(off[-1]), K))
    dY = int_bf16(rng, (int(off[-1]), N))
    with using(delay_lib):
        dW = ptg.grouped_gemm_wgrad(dev_bf16(X), dev_bf16(dY), dev(off), out_dtype=torch.float32)
    exact(dW.reshape(G * K, N), oracle.grouped_wgrad(X, dY, off), "stress wgrad")


def test_stress_ptr_array(delay_lib):
    rng = np.random.default_rng(14)
    shapes = [(1, 8, 8), (300, 256, 520), (129, 136, 64), (700, 128, 1024), (64, 512, 256)]
    probs, host = [], []
    for M, N, K in shapes:
        A, B = int_bf16(rng, (M, K)), int_bf16(rng, (K, N))
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        probs.append((dev_bf16(A), dev_bf16(B), C))
        host.append((A, B))
    with using(delay_lib):
        ptg.grouped_gemm_ptr_array(probs, wl.EPI_NONE)
    for i, ((A, B), p) in enumerate(zip(host, probs)):
        exact(p[2], oracle.gemm(A, B, wl.B_KN), f"stress batch problem {i}")


def test_stress_grouped_split_reduction(delay_lib):
    """The last round's half tiles as reduction halves (ptg_grouped_gemm_split): under the pauses
    either half may finish first; the combined sums stay bit-exact on integer data."""
    counts = np.array([300, 0] * 16 + [0, 300] * 16)
    G, K, N = len(counts), 512, 1536
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rng = np.random.default_rng(15)
    X = int_bf16(rng, (int(off[-1]), K))
    W = int_bf16(rng, (G, K, N))
    v = oracle.grouped_gemm(X, W, wl.B_KN, off)
    with using(delay_lib):
        ws = torch.empty(ptg.grouped_gemm_split_workspace(), dtype=torch.uint8, device="cuda")
        for _ in range(3):
            Y = torch.full((int(off[-1]), N), float("nan"), dtype=torch.float32, device="cuda")
            ptg.grouped_gemm(dev_bf16(X), dev_bf16(W), dev(off), out=Y, workspace=ws)
            exact(Y, v, "stress grouped split")


def test_stress_broadcast_fused(delay_lib):
    """User units, reduction units and candidate tiles of one launch, with the pauses shifting
    which workgroup reaches which unit when: bit-exact, twice on one workspace."""
    rng = np.random.default_rng(64)
    U, Ku, Kc, N = 64, 2048, 512, 1024
    idx = np.repeat(np.arange(U), rng.integers(10, 40, U)).astype(np.int32)
    Mc = int(idx.size)
    Xu, Xc, W = int_bf16(rng, (U, Ku)), int_bf16(rng, (Mc, Kc)), int_bf16(rng, (Ku + Kc, N))
    bias = rng.integers(-8, 9, N).astype(np.float32)
    v = oracle.broadcast_gemm(Xu, Xc, idx, W, wl.B_KN, bias, wl.EPI_BIAS)
    with using(delay_lib):
        ws = torch.empty(ptg.broadcast_gemm_fused_workspace(U, N), dtype=torch.uint8, device="cuda")
        for call in range(2):
            out = ptg.broadcast_gemm_fused(dev_bf16(Xu), dev_bf16(Xc), dev(idx), dev_bf16(W),
                                           out_dtype=torch.float32, bias=dev(bias), epi=wl.EPI_BIAS,
                                           workspace=ws)
            exact(out, v, f"stress broadcast fused, call {call}")
