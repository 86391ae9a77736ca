"""GPU parity of IKBO attention (ptg_ikbo_attention) against the fp64 CPU oracle.

Tolerance.  The second product takes the softmax weights P as bfloat16 MFMA operands (round to
nearest even, relative error at most 2^-9 per weight) while the normaliser is summed from the
fp32 weights, so every output element is within 2^-9 max|V| of the exact result, plus fp32
accumulation error.  The tests allow 2^-8 max|V| per element for fp32 output; bf16 output must
be within one bf16 step of the correctly rounded oracle value or within that same bound.
Exact cases: zero keys (uniform weights 1.0) with integer values and a power-of-two context
length give the mean of the values exactly; one overwhelming key returns its value row exactly.

Norm check.  The weight errors are independent, at most 2^-9 relative each, so the error of
an output row is about 2^-9 / sqrt(3) of sqrt(sum_j p_j^2 v_j^2) / l, which is also the size of
the row itself when the values have random signs: the relative Frobenius error over a case is
about 1.1e-3.  The tests require at most 2^-8 (fp32 output) and 2^-8 + 2^-9 (bf16 output, whose
rounding adds at most 2^-9 relative).  A dropped, repeated or stale key block moves a row by
about 1/L of a value, several percent of a typical row at L = 1024, and fails it, where the
per-element bound alone would not notice.
"""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import dev, dev_bf16, exact, host_bits, host_f32, int_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _no_watchdog():
    ptg.watchdog(clear=True)
    yield
    torch.cuda.synchronize()
    assert ptg.watchdog(clear=True) == 0, "a pipeline wait timed out"


def bound(V):
    return 2.0 ** -8 * float(np.abs(wl.bf16_bits_to_f32(V)).max())


def check_norm(got, v, limit, what):
    nv = float(np.linalg.norm(v))
    if nv > 0:
        rel = float(np.linalg.norm(got - v)) / nv
        assert rel <= limit, f"{what}: relative Frobenius error {rel:.3e} > {limit:.3e}"


def check_attn(out, v, V, what):
    tol = bound(V)
    if out.dtype == torch.float32:
        got = host_f32(out).astype(np.float64)
        assert np.all(np.isfinite(got)), what
        err = float(np.abs(got - v).max())
        assert err <= tol, f"{what}: max error {err:.3e} > {tol:.3e}"
        check_norm(got, v, 2.0 ** -8, what)
    else:
        got = host_bits(out).reshape(v.shape)
        ref = oracle.round_bf16(v)
        key = lambda b: np.where(b.astype(np.int64) & 0x8000, -(b.astype(np.int64) & 0x7FFF), b.astype(np.int64) & 0x7FFF)
        step = np.abs(key(got) - key(ref))
        near = np.abs(wl.bf16_bits_to_f32(got).astype(np.float64) - v) <= tol
        bad = ~((step <= 1) | near)
        assert not bad.any(), f"{what}: {int(bad.sum())} elements out of bound"
        check_norm(wl.bf16_bits_to_f32(got).astype(np.float64), v, 2.0 ** -8 + 2.0 ** -9, what)


def run(w, out_dtype, rows=None, guard=0):
    buf = torch.full((w.Mc * w.H * w.D + guard,), float("nan"), dtype=out_dtype, device="cuda")
    O = buf[: w.Mc * w.H * w.D].view(w.Mc, w.H, w.D)
    ptg.ikbo_attention(dev_bf16(w.Q), dev_bf16(w.K), dev_bf16(w.V), dev(w.offsets), scale=w.scale, out=O)
    if guard:
        torch.cuda.synchronize()
        assert torch.isnan(buf[w.Mc * w.H * w.D:]).all().item(), "wrote past O"
    return O


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("L", [64, 192])
def test_attention_small(out_dtype, L):
    """Users of 1, 0, 127, 128, 129 and 300 candidates (partial, full and empty candidate blocks,
    idle query rows), 3 heads."""
    w = wl.attention(71, 6, 3, 128, L, counts=np.array([1, 0, 127, 128, 129, 300]))
    O = run(w, out_dtype, guard=4096)
    v = oracle.ikbo_attention(w.Q, w.K, w.V, w.offsets, w.scale)
    check_attn(O, v, w.V, f"attention L={L} {out_dtype}")


def test_attention_negative_scale():
    """A negative scale (the running maximum is then taken over the negated scores)."""
    w = wl.attention(76, 3, 2, 128, 128, counts=np.array([90, 200, 5]))
    for out_dtype in (torch.float32, torch.bfloat16):
        O = ptg.ikbo_attention(dev_bf16(w.Q), dev_bf16(w.K), dev_bf16(w.V), dev(w.offsets), scale=-0.3,
                               out_dtype=out_dtype)
        v = oracle.ikbo_attention(w.Q, w.K, w.V, w.offsets, -0.3)
        check_attn(O, v, w.V, f"negative scale {out_dtype}")


def test_attention_rising_scores():
    """Scores that climb about 6 (log2 units) per 64-key block and reach 48: the running maximum
    the kernel keeps may trail the true one for a block (weights up to 2^8) and must catch up
    within the context, so both the kept and the rescaled paths run, per query and head."""
    counts = np.array([70, 129, 3])
    U, H, D, L = len(counts), 2, 128, 512
    rng = np.random.default_rng(77)
    Mc = int(counts.sum())
    off = np.zeros(U + 1, np.int32)
    off[1:] = np.cumsum(counts)
    Qf = np.zeros((Mc, H, D), np.float32)
    Qf[:, :, 0] = rng.uniform(0.5, 1.0, (Mc, H))
    Qf[:, :, 1:] = rng.normal(0.0, 0.05, (Mc, H, D - 1))
    Kf = rng.normal(0.0, 0.05, (U, L, H, D)).astype(np.float32)
    ramp = np.arange(L, dtype=np.float32) * (6.0 / 64.0 / float(np.log2(np.e)))
    Kf[:, :, :, 0] = ramp[None, :, None] + rng.normal(0.0, 0.3, (U, L, H))
    Q, K = wl.f32_to_bf16_bits(Qf), wl.f32_to_bf16_bits(Kf)
    V = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (U, L, H, D)).astype(np.float32))
    v = oracle.ikbo_attention(Q, K, V, off, 1.0)
    for out_dtype in (torch.float32, torch.bfloat16):
        O = ptg.ikbo_attention(dev_bf16(Q), dev_bf16(K), dev_bf16(V), dev(off), scale=1.0, out_dtype=out_dtype)
        check_attn(O, v, V, f"rising scores {out_dtype}")


def test_attention_zero_keys_give_the_mean_exactly():
    """K = 0: every weight is exactly 1, so O is the plain mean of the user's value rows; with
    integer values and L = 128 that mean is exact in fp32 (pins the value path per user and head)."""
    counts = np.array([3, 200, 0, 131])
    U, H, D, L = len(counts), 2, 128, 128
    rng = np.random.default_rng(72)
    Mc = int(counts.sum())
    off = np.zeros(U + 1, np.int32)
    off[1:] = np.cumsum(counts)
    Q = int_bf16(rng, (Mc, H, D))
    K = np.zeros((U, L, H, D), np.uint16)
    V = int_bf16(rng, (U, L, H, D))
    O = ptg.ikbo_attention(dev_bf16(Q), dev_bf16(K), dev_bf16(V), dev(off), scale=0.1, out_dtype=torch.float32)
    mean = wl.bf16_bits_to_f32(V).astype(np.float64).mean(axis=1)       # [U, H, D]
    user = np.repeat(np.arange(U), counts)
    exact(O, mean[user], "zero keys")


def test_attention_one_overwhelming_key_selects_its_value():
    """Q = e_0 and K[u, j] = 128 e_0 for j = j_u only, scale 1: the other weights are e^-128,
    which underflows to zero in fp32, so O[c] = V[u, j_u] exactly (pins which key and which user
    each candidate sees).  (With e^-64 the weights stay representable, and the matrix cores'
    fp32 accumulation, which does not round to nearest, can leave a power of two one ulp low.)"""
    counts = np.array([130, 5, 0, 64])
    U, H, D, L = len(counts), 3, 128, 256
    rng = np.random.default_rng(73)
    Mc = int(counts.sum())
    off = np.zeros(U + 1, np.int32)
    off[1:] = np.cumsum(counts)
    Qf = np.zeros((Mc, H, D), np.float32)
    Qf[:, :, 0] = 1.0
    Kf = np.zeros((U, L, H, D), np.float32)
    pick = rng.integers(0, L, (U, H))
    for u in range(U):
        for h in range(H):
            Kf[u, pick[u, h], h, 0] = 128.0
    V = wl.f32_to_bf16_bits(rng.uniform(-1, 1, (U, L, H, D)).astype(np.float32))
    for out_dtype in (torch.float32, torch.bfloat16):
        O = ptg.ikbo_attention(dev_bf16(wl.f32_to_bf16_bits(Qf)), dev_bf16(wl.f32_to_bf16_bits(Kf)), dev_bf16(V),
                               dev(off), scale=1.0, out_dtype=out_dtype)
        v = wl.bf16_bits_to_f32(V).astype(np.float64)
        user = np.repeat(np.arange(U), counts)
        want = np.stack([v[user[c], pick[user[c], np.arange(H)], np.arange(H)] for c in range(Mc)])
        exact(O, want, f"dominant key {out_dtype}")


def test_attention_repeat_is_bit_identical():
    w = wl.attention(74, 3, 2, 128, 128, counts=np.array([50, 260, 7]))
    a = run(w, torch.float32)
    b = run(w, torch.float32)
    assert torch.equal(a, b)


def test_attention_rejects_bad_shapes():
    Q = torch.zeros((4, 1, 64), dtype=torch.bfloat16, device="cuda")       # D = 64
    K = torch.zeros((1, 64, 1, 64), dtype=torch.bfloat16, device="cuda")
    off = dev(np.array([0, 4], np.int32))
    with pytest.raises(ptg.PtgError):
        ptg.ikbo_attention(Q, K, K, off)
    Q = torch.zeros((4, 1, 128), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((1, 96, 1, 128), dtype=torch.bfloat16, device="cuda")  # L = 96
    with pytest.raises(ptg.PtgError):
        ptg.ikbo_attention(Q, K, K, off)


def test_ikbo_attention_workload_sampled():
    """The benchmarked workload (64 users, C_u ~ U{256..2048}, L = 1024, 4 heads of 128) in the
    benchmarked launch: the first and last candidate of every user plus random candidates, bf16
    output and its fp32 twin."""
    w = wl.ikbo_attention_workload()
    rng = np.random.default_rng(75)
    rows = set(rng.integers(0, w.Mc, 64).tolist())
    for u in range(w.U):
        if w.counts[u] > 0:
            rows |= {int(w.offsets[u]), int(w.offsets[u + 1]) - 1}
    rows = np.array(sorted(rows), dtype=np.int64)
    v = oracle.ikbo_attention(w.Q, w.K, w.V, w.offsets, w.scale, rows=rows)
    Q, K, V, off = dev_bf16(w.Q), dev_bf16(w.K), dev_bf16(w.V), dev(w.offsets)
    idx = torch.from_numpy(rows).cuda()
    for out_dtype in (torch.bfloat16, torch.float32):
        O = ptg.ikbo_attention(Q, K, V, off, scale=w.scale, out_dtype=out_dtype)
        check_attn(O[idx], v, w.V, f"ikbo attention {out_dtype}")
