"""Seeded synthetic inputs for the pipelined tiled GEMM and its grouped and broadcast forms.

This module is the only code shared by the CPU oracle (``oracle/``) and the GPU path
(``pipelined_tiled_gemm_amd``).  It draws random numbers and quantises them to bfloat16;
it holds none of the GEMM arithmetic.

Every generator follows one rule: draws are made with ``numpy.random.default_rng(seed)``
(PCG64) in float64, in a fixed order, then rounded to float32 and then to bfloat16 with
round-to-nearest-even.  A bfloat16 array is returned as its raw ``uint16`` bit patterns so
that both sides receive exactly the same bytes.  "N(0, s)" means standard deviation s.

The five workloads stand in for the pages' production cases (How We Built TLX: "TLX in
Production" table; Case Study 2 "In-Kernel Broadcast Optimization"; Case Study 3
"Distributed Grouped GEMM"): no dataset is involved, only these synthetic shapes.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import List, Optional

import numpy as np

# Layout codes, shared vocabulary with the C ABI: B stored K x N row-major, or N x K row-major.
B_KN = 0
B_NK = 1

# Epilogue codes.
EPI_NONE = 0
EPI_BIAS = 1
EPI_SILU = 2
EPI_BIAS_SILU = 3

_CHUNK_ELEMS = 1 << 23  # rows are drawn in chunks of about 8M values to bound host memory


# ----------------------------------------------------------------------------------------
# bfloat16 bit helpers (input quantisation only)
# ----------------------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns.

    Inputs are finite by construction; NaN is kept a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _quantise(x64: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(x64.astype(np.float32))


def _draw_rows(rng, rows: int, cols: int, kind: str, scale: float = 1.0) -> np.ndarray:
    """Draw a rows x cols matrix in row chunks (same stream as one call) and quantise it."""
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        if kind == "uniform":
            x = rng.uniform(-1.0, 1.0, (r1 - r0, cols))
        elif kind == "normal":
            x = rng.standard_normal((r1 - r0, cols))
        else:
            raise ValueError(kind)
        if scale != 1.0:
            x = x * scale
        out[r0:r1] = _quantise(x)
    return out


def digest(*arrays) -> str:
    """SHA-256 over the raw bytes of the given arrays (fixture pinning)."""
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()


# ----------------------------------------------------------------------------------------
# Workload containers
# ----------------------------------------------------------------------------------------
@dataclasses.dataclass
class Dense:
    """C = epi(A.B + bias); A is M x K row-major, B is K x N (KN) or N x K (NK)."""
    M: int
    N: int
    K: int
    A: np.ndarray            # uint16 [M, K]
    B: np.ndarray            # uint16 [K, N] or [N, K]
    b_layout: int
    bias: Optional[np.ndarray] = None   # float32 [N]
    epi: int = EPI_NONE
    out_dtype: str = "f32"


@dataclasses.dataclass
class Grouped:
    """Y[r] = epi(X[r].W_g + bias_g) for rows r of group g: off[g] <= r < off[g+1]."""
    G: int
    M_total: int
    N: int
    K: int
    X: np.ndarray            # uint16 [M_total, K]
    W: np.ndarray            # uint16 [G, K, N] (KN) or [G, N, K] (NK)
    w_layout: int
    counts: np.ndarray       # int64 [G]
    offsets: np.ndarray      # int32 [G + 1]
    bias: Optional[np.ndarray] = None   # float32 [G, N]
    epi: int = EPI_NONE
    out_dtype: str = "bf16"


@dataclasses.dataclass
class Wgrad:
    """dW[g] = X_g^T . dY_g over the rows r of group g: off[g] <= r < off[g+1]."""
    G: int
    M_total: int
    K: int
    N: int
    X: np.ndarray            # uint16 [M_total, K]
    dY: np.ndarray           # uint16 [M_total, N]
    counts: np.ndarray       # int64 [G]
    offsets: np.ndarray      # int32 [G + 1]
    out_dtype: str = "bf16"


@dataclasses.dataclass
class Attention:
    """O[c] = softmax(scale Q[c] . K[u]^T) . V[u] per head, u the user of candidate c."""
    U: int
    Mc: int
    H: int
    D: int
    L: int
    Q: np.ndarray            # uint16 [Mc, H, D]
    K: np.ndarray            # uint16 [U, L, H, D]
    V: np.ndarray            # uint16 [U, L, H, D]
    counts: np.ndarray       # int64 [U] candidates per user
    offsets: np.ndarray      # int32 [U + 1]
    scale: float
    out_dtype: str = "bf16"


@dataclasses.dataclass
class Broadcast:
    """Y[r] = epi([Xu[idx[r]] | Xc[r]].W + bias), W is (Ku + Kc) x N (KN) or N x (Ku + Kc) (NK)."""
    U: int
    Mc: int
    Ku: int
    Kc: int
    N: int
    Xu: np.ndarray           # uint16 [U, Ku]
    Xc: np.ndarray           # uint16 [Mc, Kc]
    idx: np.ndarray          # int32 [Mc]
    W: np.ndarray            # uint16
    w_layout: int
    counts: np.ndarray       # int64 [U] candidates per user
    bias: Optional[np.ndarray] = None
    epi: int = EPI_NONE
    out_dtype: str = "bf16"


@dataclasses.dataclass
class Problem:
    M: int
    N: int
    K: int
    A: np.ndarray            # uint16 [M, K]
    B: np.ndarray            # uint16 [K, N] (KN)
    bias: Optional[np.ndarray]  # float32 [N]


@dataclasses.dataclass
class ProblemList:
    """Independent problems Y_p = epi(A_p.B_p + bias_p), all B_p stored K x N."""
    problems: List[Problem]
    epi: int = EPI_BIAS_SILU
    out_dtype: str = "bf16"


# ----------------------------------------------------------------------------------------
# Generators
# ----------------------------------------------------------------------------------------
def dense(seed: int, M: int, N: int, K: int, *, dist: str = "uniform", b_layout: int = B_KN,
          scale: float = 1.0, out_dtype: str = "f32", epi: int = EPI_NONE,
          with_bias: bool = False) -> Dense:
    """Draw A [M x K], then B (stored as its layout dictates), then the optional bias N(0, 0.1)."""
    rng = np.random.default_rng(seed)
    A = _draw_rows(rng, M, K, dist, scale)
    if b_layout == B_KN:
        B = _draw_rows(rng, K, N, dist, scale)
    else:
        B = _draw_rows(rng, N, K, dist, scale)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32) if with_bias else None
    return Dense(M, N, K, A, B, b_layout, bias, epi, out_dtype)


def config1() -> Dense:
    """Single dense GEMM, 256 cubed, U(-1,1) bf16, fp32 output, no epilogue (seed 1)."""
    return dense(1, 256, 256, 256, dist="uniform", b_layout=B_KN, out_dtype="f32")


def config2(M: int = 8192, N: int = 8192, K: int = 8192, seed: int = 2) -> Dense:
    """Dense GEMM with B stored transposed (N x K), entries N(0,1)/sqrt(K), bf16 output (seed 2)."""
    return dense(seed, M, N, K, dist="normal", b_layout=B_NK, scale=1.0 / np.sqrt(K),
                 out_dtype="bf16")


def zipf_rank_weights(G: int, s: float) -> np.ndarray:
    """Rank-Zipf expert weights p_e proportional to (e + 1)^-s, normalised."""
    p = (np.arange(G, dtype=np.float64) + 1.0) ** (-s)
    return p / p.sum()


def grouped(seed: int, G: int, M_total: int, K: int, N: int, *, reading: str = "rank",
            zipf_s: float = 1.1, w_layout: int = B_KN, w_std: float = 0.02,
            x_dist: str = "normal", out_dtype: str = "bf16", epi: int = EPI_NONE,
            with_bias: bool = False, counts: Optional[np.ndarray] = None) -> Grouped:
    """Draw group counts (multinomial over Zipf weights), then X, then W, then the optional bias.

    reading="rank": weights (e+1)^-s over the G experts.  reading="sampled": weights are
    rng.zipf(s, G) draws, normalised (this makes most groups empty).  An explicit ``counts``
    vector skips the draw.
    """
    rng = np.random.default_rng(seed)
    if counts is None:
        if reading == "rank":
            p = zipf_rank_weights(G, zipf_s)
        elif reading == "sampled":
            w = rng.zipf(zipf_s, G).astype(np.float64)
            p = w / w.sum()
        else:
            raise ValueError(reading)
        counts = rng.multinomial(M_total, p).astype(np.int64)
    else:
        counts = np.asarray(counts, dtype=np.int64)
        assert counts.sum() == M_total and len(counts) == G
    offsets = np.zeros(G + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    X = _draw_rows(rng, M_total, K, x_dist)
    if w_layout == B_KN:
        W = _draw_rows(rng, G * K, N, "normal", w_std).reshape(G, K, N)
    else:
        W = _draw_rows(rng, G * N, K, "normal", w_std).reshape(G, N, K)
    bias = (rng.standard_normal((G, N)) * 0.1).astype(np.float32) if with_bias else None
    return Grouped(G, M_total, N, K, X, W, w_layout, counts, offsets, bias, epi, out_dtype)


def config3(reading: str = "rank") -> Grouped:
    """MoE grouped GEMM: 64 experts, 16384 rows, K=4096, N=1536, weights N(0,0.02) (seed 3)."""
    return grouped(3, 64, 16384, 4096, 1536, reading=reading)


def wgrad(seed: int, G: int, M_total: int, K: int, N: int, *, reading: str = "rank",
          zipf_s: float = 1.1, x_dist: str = "normal", dy_dist: str = "normal",
          out_dtype: str = "bf16", counts: Optional[np.ndarray] = None) -> Wgrad:
    """Weight gradient of the grouped GEMM: draw the group counts and X exactly as ``grouped``
    does with the same seed (same routing, same activations), then dY [M_total x N] in place
    of the weights."""
    rng = np.random.default_rng(seed)
    if counts is None:
        if reading == "rank":
            p = zipf_rank_weights(G, zipf_s)
        elif reading == "sampled":
            w = rng.zipf(zipf_s, G).astype(np.float64)
            p = w / w.sum()
        else:
            raise ValueError(reading)
        counts = rng.multinomial(M_total, p).astype(np.int64)
    else:
        counts = np.asarray(counts, dtype=np.int64)
        assert counts.sum() == M_total and len(counts) == G
    offsets = np.zeros(G + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    X = _draw_rows(rng, M_total, K, x_dist)
    dY = _draw_rows(rng, M_total, N, dy_dist)
    return Wgrad(G, M_total, K, N, X, dY, counts, offsets, out_dtype)


def moe_wgrad(reading: str = "rank") -> Wgrad:
    """Backward of the MoE workload: routing and X of the 64-expert, 16384-row, K = 4096,
    N = 1536 grouped GEMM (seed 3), dY ~ N(0,1); dW is 64 x 4096 x 1536."""
    return wgrad(3, 64, 16384, 4096, 1536, reading=reading)


def broadcast(seed: int, U: int, Ku: int, Kc: int, N: int, *, cmin: int = 256, cmax: int = 2048,
              w_layout: int = B_KN, w_std: float = 0.02, out_dtype: str = "bf16",
              epi: int = EPI_NONE, with_bias: bool = False, shuffle: bool = False) -> Broadcast:
    """Draw C_u ~ U{cmin..cmax} per user, then Xu, Xc ~ N(0,1), then W ~ N(0, w_std).

    Candidates are contiguous by user (idx nondecreasing) unless ``shuffle`` permutes the
    candidate rows with one more draw.
    """
    rng = np.random.default_rng(seed)
    counts = rng.integers(cmin, cmax + 1, U).astype(np.int64)
    Mc = int(counts.sum())
    Xu = _draw_rows(rng, U, Ku, "normal")
    Xc = _draw_rows(rng, Mc, Kc, "normal")
    if w_layout == B_KN:
        W = _draw_rows(rng, Ku + Kc, N, "normal", w_std)
    else:
        W = _draw_rows(rng, N, Ku + Kc, "normal", w_std)
    idx = np.repeat(np.arange(U, dtype=np.int32), counts)
    bias = (rng.standard_normal(N) * 0.1).astype(np.float32) if with_bias else None
    if shuffle:
        perm = rng.permutation(Mc)
        idx = np.ascontiguousarray(idx[perm])
        Xc = np.ascontiguousarray(Xc[perm])
    return Broadcast(U, Mc, Ku, Kc, N, Xu, Xc, idx, W, w_layout, counts, bias, epi, out_dtype)


def config4() -> Broadcast:
    """IKBO linear compression: 64 users, Xu 64x2048, Xc (sum C_u)x512, W 2560x1024 (seed 4)."""
    return broadcast(4, 64, 2048, 512, 1024)


def attention(seed: int, U: int, H: int, D: int, L: int, *, cmin: int = 256, cmax: int = 2048,
              counts: Optional[np.ndarray] = None, out_dtype: str = "bf16") -> Attention:
    """Draw C_u ~ U{cmin..cmax} per user (unless ``counts`` is given), then Q, K, V ~ N(0,1);
    candidates contiguous by user; scale 1/sqrt(D)."""
    rng = np.random.default_rng(seed)
    if counts is None:
        counts = rng.integers(cmin, cmax + 1, U).astype(np.int64)
    else:
        counts = np.asarray(counts, dtype=np.int64)
        assert len(counts) == U
    Mc = int(counts.sum())
    offsets = np.zeros(U + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    Q = _draw_rows(rng, Mc * H, D, "normal").reshape(Mc, H, D)
    K = _draw_rows(rng, U * L * H, D, "normal").reshape(U, L, H, D)
    V = _draw_rows(rng, U * L * H, D, "normal").reshape(U, L, H, D)
    return Attention(U, Mc, H, D, L, Q, K, V, counts, offsets, 1.0 / float(np.sqrt(D)), out_dtype)


def ikbo_attention_workload() -> Attention:
    """IKBO attention: 64 users with C_u ~ U{256..2048} candidates (seed 7), user context of
    L = 1024 keys, 4 heads of dimension 128."""
    return attention(7, 64, 4, 128, 1024)


def attention_flops(w: Attention) -> float:
    """Two products (Q.K^T and P.V) of 2 Mc L D flops per head."""
    return 4.0 * w.Mc * w.L * w.D * w.H


def attention_bytes(w: Attention) -> float:
    """Q and O once per candidate, K and V once per user."""
    ob = out_bytes(w.out_dtype)
    return (2.0 + ob) * w.Mc * w.H * w.D + 2.0 * 2.0 * w.U * w.L * w.H * w.D


def problem_list(seed: int, P: int, *, mmin: int = 64, mmax: int = 1024,
                 nk_choices=(128, 256, 512), epi: int = EPI_BIAS_SILU,
                 out_dtype: str = "bf16") -> ProblemList:
    """First draw all shapes (M_p, N_p, K_p), then per problem A_p, B_p ~ U(-1,1), bias_p ~ N(0,0.1)."""
    rng = np.random.default_rng(seed)
    shapes = []
    for _ in range(P):
        m = int(rng.integers(mmin, mmax + 1))
        n = int(rng.choice(nk_choices))
        k = int(rng.choice(nk_choices))
        shapes.append((m, n, k))
    probs = []
    for (m, n, k) in shapes:
        A = _draw_rows(rng, m, k, "uniform")
        B = _draw_rows(rng, k, n, "uniform")
        bias = (rng.standard_normal(n) * 0.1).astype(np.float32)
        probs.append(Problem(m, n, k, A, B, bias))
    return ProblemList(probs, epi, out_dtype)


def config5() -> ProblemList:
    """RecSys small-shape batch: 1024 GEMMs, M~U{64..1024}, N,K in {128,256,512}, bias+SiLU (seed 5)."""
    return problem_list(5, 1024)


# ----------------------------------------------------------------------------------------
# Algorithmic work and compulsory bytes (for throughput reporting)
# ----------------------------------------------------------------------------------------
def out_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def dense_flops(M, N, K) -> float:
    return 2.0 * M * N * K


def dense_bytes(M, N, K, out_dtype="bf16", bias=False) -> float:
    return 2.0 * (M * K + K * N) + out_bytes(out_dtype) * M * N + (4.0 * N if bias else 0.0)


def grouped_flops(w: Grouped) -> float:
    return 2.0 * w.M_total * w.N * w.K


def grouped_bytes(w: Grouped) -> float:
    live = int((w.counts > 0).sum())
    return 2.0 * (w.M_total * w.K + live * w.K * w.N) + out_bytes(w.out_dtype) * w.M_total * w.N


def wgrad_flops(w: Wgrad) -> float:
    return 2.0 * w.M_total * w.K * w.N


def wgrad_bytes(w: Wgrad) -> float:
    """X and dY read once, every expert's K x N gradient written (zeros for empty experts)."""
    return 2.0 * w.M_total * (w.K + w.N) + out_bytes(w.out_dtype) * w.G * w.K * w.N


def broadcast_flops(w: Broadcast) -> float:
    """Algorithmic work of the decomposed form: user part once per user plus candidate part."""
    return 2.0 * w.U * w.Ku * w.N + 2.0 * w.Mc * w.Kc * w.N


def broadcast_flops_materialised(w: Broadcast) -> float:
    return 2.0 * w.Mc * (w.Ku + w.Kc) * w.N


def broadcast_bytes(w: Broadcast) -> float:
    return (2.0 * (w.U * w.Ku + w.Mc * w.Kc + (w.Ku + w.Kc) * w.N) + 4.0 * w.Mc
            + out_bytes(w.out_dtype) * w.Mc * w.N)


def problem_list_flops(w: ProblemList) -> float:
    return sum(2.0 * p.M * p.N * p.K for p in w.problems)


def problem_list_bytes(w: ProblemList) -> float:
    ob = out_bytes(w.out_dtype)
    return sum(2.0 * (p.M * p.K + p.K * p.N) + ob * p.M * p.N + 4.0 * p.N for p in w.problems)
