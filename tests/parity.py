"""Comparison helpers for the GPU parity tests (test infrastructure: uses the oracle).

Tolerances.  For float32 outputs: relative Frobenius error <= 1e-5 and max elementwise
error <= 1e-4 * sqrt(K) against the oracle's double result v.  For bfloat16 outputs the
rounding alone exceeds those bounds, so each element must be within one bfloat16 step of
the oracle's correctly rounded RNE(v) (a float32 accumulation error may cross a rounding
boundary), or within 1e-4 * sqrt(K) of v (values near zero).  Integer-exact inputs, the
identity/permutation cases and all row/group/user bookkeeping are compared bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import workloads as wl

REL_FRO = 1e-5
ABS_PER_SQRT_K = 1e-4


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bfloat16 bit patterns -> bfloat16 tensor on the GPU (same bytes)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def dev(arr: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr)).to("cuda")


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bfloat16 tensor -> uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def _key(b: np.ndarray) -> np.ndarray:
    """Order-preserving integer key of bfloat16 bit patterns (+0 and -0 share key 0)."""
    b = b.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def check_f32(got: np.ndarray, v: np.ndarray, K: int, what: str = "") -> None:
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == v.shape, (got.shape, v.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = got - v
    nv = float(np.linalg.norm(v))
    nd = float(np.linalg.norm(diff))
    if nv > 0:
        assert nd / nv <= REL_FRO, f"{what}: relative Frobenius error {nd / nv:.3e} > {REL_FRO}"
    else:
        assert nd == 0.0, f"{what}: expected zeros"
    md = float(np.max(np.abs(diff))) if diff.size else 0.0
    assert md <= ABS_PER_SQRT_K * math.sqrt(K), f"{what}: max error {md:.3e} > {ABS_PER_SQRT_K}*sqrt({K})"


def check_bf16(got_bits: np.ndarray, v: np.ndarray, K: int, what: str = "") -> None:
    got_bits = np.asarray(got_bits, dtype=np.uint16)
    assert got_bits.shape == v.shape, (got_bits.shape, v.shape)
    ref = oracle.round_bf16(v)
    step = np.abs(_key(got_bits) - _key(ref))
    near = np.abs(wl.bf16_bits_to_f32(got_bits).astype(np.float64) - v) <= ABS_PER_SQRT_K * math.sqrt(K)
    bad = ~((step <= 1) | near)
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements beyond one bf16 step; first at "
                           f"{np.argwhere(bad)[0].tolist()}")


def check(out: torch.Tensor, v: np.ndarray, K: int, what: str = "") -> None:
    if out.dtype == torch.float32:
        check_f32(host_f32(out), v, K, what)
    else:
        check_bf16(host_bits(out), v, K, what)


def exact(out: torch.Tensor, v: np.ndarray, what: str = "") -> None:
    """Bit-exact comparison: v must be representable in the output dtype."""
    if out.dtype == torch.float32:
        got = host_f32(out).astype(np.float64)
        assert np.array_equal(got, v), f"{what}: not bit-exact ({int((got != v).sum())} differ)"
    else:
        got = host_bits(out)
        want = oracle.round_bf16(v)
        assert np.array_equal(_key(got), _key(want)), f"{what}: not bit-exact"


def int_bf16(rng, shape, lo=-4, hi=4) -> np.ndarray:
    """Small integers: exact in bfloat16; sums of up to 2^20 of their products stay exact in fp32."""
    return wl.f32_to_bf16_bits(rng.integers(lo, hi + 1, shape).astype(np.float32))


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and n random rows (sorted, unique) for checks at full size."""
    rng = np.random.default_rng(seed)
    rows = {0, max(M - 1, 0)} | set(rng.integers(0, max(M, 1), n).tolist())
    return np.array(sorted(r for r in rows if r < M), dtype=np.int64)
