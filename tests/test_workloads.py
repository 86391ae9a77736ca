"""The seeded input generators: bfloat16 quantisation, determinism and pinned workload facts."""
import json
import os

import numpy as np
import pytest
import torch

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "workload_fixtures.json")


@pytest.fixture(scope="module")
def fx():
    with open(GOLDEN) as f:
        return json.load(f)


def test_bf16_quantisation_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000),
        np.array([0.0, -0.0, 1.0, -1.0, 3.4e38, -3.4e38, 1e-40, -1e-40, 1.00390625, 1.01171875],
                 np.float32),
    ]).astype(np.float32)
    mine = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_decode_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        vals = wl.bf16_bits_to_f32(bits)
    finite = np.isfinite(vals)
    assert np.array_equal(wl.f32_to_bf16_bits(vals[finite]), bits[finite])


def test_chunked_draws_equal_single_draw(monkeypatch):
    ref = wl.dense(42, 37, 29, 53, dist="normal", b_layout=wl.B_KN)
    monkeypatch.setattr(wl, "_CHUNK_ELEMS", 100)
    got = wl.dense(42, 37, 29, 53, dist="normal", b_layout=wl.B_KN)
    assert np.array_equal(ref.A, got.A) and np.array_equal(ref.B, got.B)


def test_determinism_and_digests(fx):
    c1 = wl.config1()
    assert (c1.M, c1.N, c1.K, c1.b_layout, c1.out_dtype) == (256, 256, 256, wl.B_KN, "f32")
    assert wl.digest(c1.A, c1.B) == fx["config1_digest"]
    small = wl.dense(100, 33, 40, 24, dist="normal", b_layout=wl.B_NK, scale=0.5)
    assert wl.digest(small.A, small.B) == fx["dense_small_digest"]
    a = wl.f32_to_bf16_bits(np.float32(1.0)).item()
    assert a == 0x3F80
    vals = wl.bf16_bits_to_f32(c1.A)
    assert vals.min() >= -1.0 and vals.max() <= 1.0


def test_grouped_counts(fx):
    # the generator's own draw (small K, N so that only the counts matter)
    g = wl.grouped(3, 64, 16384, 8, 8)
    assert g.counts.tolist() == fx["config3_counts_rank_zipf"]
    assert g.offsets[0] == 0 and g.offsets[-1] == 16384
    assert np.all(np.diff(g.offsets) >= 0) and g.offsets.dtype == np.int32
    assert min(g.counts) == 35 and (g.counts == 0).sum() == 0 and g.counts[0] == 4090
    s = wl.grouped(3, 64, 16384, 8, 8, reading="sampled")
    assert s.counts.tolist() == fx["config3_counts_sampled_zipf"]
    assert (s.counts > 0).sum() == 1


def test_broadcast_counts(fx):
    b = wl.broadcast(4, 64, 8, 8, 8)
    assert b.counts.tolist() == fx["config4_candidates_per_user"]
    assert b.Mc == 81403
    assert np.array_equal(b.idx, np.repeat(np.arange(64), b.counts))
    sh = wl.broadcast(4, 64, 8, 8, 8, shuffle=True)
    assert sorted(sh.idx.tolist()) == b.idx.tolist()


def test_wgrad_workload(fx):
    """The weight-gradient workload draws the forward MoE routing and X, then dY."""
    w = wl.wgrad(3, 64, 16384, 8, 8)
    g = wl.grouped(3, 64, 16384, 8, 8)
    assert w.counts.tolist() == fx["config3_counts_rank_zipf"]
    assert np.array_equal(w.X, g.X) and np.array_equal(w.offsets, g.offsets)
    assert w.dY.shape == (16384, 8)
    small = wl.wgrad(30, 5, 300, 16, 24, counts=np.array([100, 0, 7, 150, 43]))
    assert wl.digest(small.X, small.dY) == fx["wgrad_small_digest"]


def test_attention_workload(fx):
    a = wl.attention(7, 64, 1, 128, 64)
    assert a.counts.tolist() == fx["attention_candidates_per_user"]
    assert a.Mc == 77801 and a.offsets[-1] == 77801
    assert a.Q.shape == (77801, 1, 128) and a.K.shape == (64, 64, 1, 128)
    assert a.scale == pytest.approx(128 ** -0.5)
    small = wl.attention(70, 3, 2, 128, 64, counts=np.array([5, 0, 9]))
    assert wl.digest(small.Q, small.K, small.V) == fx["attention_small_digest"]


def test_problem_list_shapes(fx):
    shapes = fx["config5_shapes"]
    assert len(shapes) == 1024 and sum(s[0] for s in shapes) == 560558
    assert shapes[:3] == [[708, 512, 128], [840, 256, 256], [669, 128, 512]]
    small = wl.problem_list(5, 6)
    assert [[p.M, p.N, p.K] for p in small.problems] == shapes[:6]
    for p in small.problems:
        assert p.A.shape == (p.M, p.K) and p.B.shape == (p.K, p.N) and p.bias.shape == (p.N,)
        assert p.bias.dtype == np.float32


def test_work_counts():
    assert wl.dense_flops(8192, 8192, 8192) == pytest.approx(1.0995e12, rel=1e-4)
    assert wl.dense_bytes(8192, 8192, 8192, "bf16") == pytest.approx(402.7e6, rel=1e-3)
