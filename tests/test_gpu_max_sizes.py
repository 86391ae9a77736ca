"""Parity at the library's maximum counts, where its bookkeeping lives in LDS: 1024 expert groups
(grouped GEMM, its split form and the weight gradient), 2048 problems in one pointer-array launch,
and 1024 users for the IKBO attention.  Integer data make the GEMMs exact, so every element is
compared bit for bit against the oracle; counts include empty groups, empty-ish problems and users
without candidates."""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import dev, dev_bf16, exact, host_f32, int_bf16

pytestmark = pytest.mark.gpu

MAX_GROUPS = 1024
MAX_BATCH = 2048


@pytest.fixture(autouse=True)
def _no_watchdog():
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0, "a pipeline wait timed out"


def _offsets(counts):
    return np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)


@pytest.mark.parametrize("layout", [wl.B_KN, wl.B_NK])
def test_grouped_1024_groups_exact(layout):
    rng = np.random.default_rng(1024 + layout)
    counts = rng.integers(0, 40, MAX_GROUPS)
    counts[rng.integers(0, MAX_GROUPS, 200)] = 0          # many empty experts
    counts[7] = 700                                         # one expert of several tiles
    off = _offsets(counts)
    M, K, N = int(off[-1]), 64, 136
    X = int_bf16(rng, (M, K))
    W = int_bf16(rng, (MAX_GROUPS, K, N) if layout == wl.B_KN else (MAX_GROUPS, N, K))
    bias = rng.integers(-4, 5, (MAX_GROUPS, N)).astype(np.float32)
    v = oracle.grouped_gemm(X, W, layout, off, bias, wl.EPI_BIAS)
    args = (dev_bf16(X), dev_bf16(W), dev(off))
    kw = dict(w_layout=layout, out_dtype=torch.float32, bias=dev(bias), epi=wl.EPI_BIAS)
    exact(ptg.grouped_gemm(*args, **kw), v, f"grouped, 1024 groups, layout {layout}")
    ws = torch.empty(ptg.grouped_gemm_split_workspace(), dtype=torch.uint8, device="cuda")
    exact(ptg.grouped_gemm(*args, workspace=ws, **kw), v, f"grouped split, 1024 groups, layout {layout}")


def test_wgrad_1024_groups_exact():
    rng = np.random.default_rng(2024)
    counts = rng.integers(0, 30, MAX_GROUPS)
    counts[rng.integers(0, MAX_GROUPS, 300)] = 0
    off = _offsets(counts)
    M, K, N = int(off[-1]), 72, 64
    X, dY = int_bf16(rng, (M, K)), int_bf16(rng, (M, N))
    dW = ptg.grouped_gemm_wgrad(dev_bf16(X), dev_bf16(dY), dev(off), out_dtype=torch.float32)
    v = oracle.grouped_wgrad(X, dY, off)
    exact(dW.reshape(MAX_GROUPS * K, N), v, "weight gradient, 1024 groups")


def test_ptr_array_2048_problems_exact():
    rng = np.random.default_rng(2048)
    probs, dev_probs, outs = [], [], []
    for p in range(MAX_BATCH):
        m = int(rng.integers(1, 80))
        n = int(rng.choice((8, 64, 136)))
        k = int(rng.choice((8, 64, 200)))
        A, B = int_bf16(rng, (m, k)), int_bf16(rng, (k, n))
        bias = rng.integers(-4, 5, n).astype(np.float32)
        probs.append(wl.Problem(m, n, k, A, B, bias))
        C = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda")
        dev_probs.append((dev_bf16(A), dev_bf16(B), C, dev(bias)))
        outs.append(C)
    ptg.grouped_gemm_ptr_array(dev_probs, wl.EPI_BIAS)
    vs = oracle.problem_list(probs, wl.EPI_BIAS)
    for i, (o, v) in enumerate(zip(outs, vs)):
        exact(o, v, f"problem {i} of 2048")


def test_attention_1024_users():
    rng = np.random.default_rng(1025)
    U, H, D, L = MAX_GROUPS, 1, 128, 64
    counts = rng.integers(0, 12, U)
    counts[rng.integers(0, U, 100)] = 0                     # users without candidates
    off = _offsets(counts)
    Mc = int(off[-1])
    Q = wl.f32_to_bf16_bits(rng.standard_normal((Mc, H, D)).astype(np.float32))
    K = wl.f32_to_bf16_bits(rng.standard_normal((U, L, H, D)).astype(np.float32))
    V = wl.f32_to_bf16_bits(rng.standard_normal((U, L, H, D)).astype(np.float32))
    scale = 1.0 / np.sqrt(D)
    O = ptg.ikbo_attention(dev_bf16(Q), dev_bf16(K), dev_bf16(V), dev(off), scale=scale, out_dtype=torch.float32)
    v = oracle.ikbo_attention(Q, K, V, off, scale).reshape(Mc, H, D)
    got = host_f32(O).astype(np.float64).reshape(Mc, H, D)
    tol = 2.0 ** -8 * float(np.abs(wl.bf16_bits_to_f32(V)).max())
    assert float(np.abs(got - v).max()) <= tol, "attention, 1024 users"
