"""The C ABI on the CPU: the library loads, exports every entry point include/ptg.h declares,
and rejects invalid calls with the documented status before touching any device.

Pointers passed here are never dereferenced: every call below fails host-side validation
(or is a documented no-op) before a HIP call would be made.
"""
import ctypes
import os
import re

import pytest

from pipelined_tiled_gemm_amd import _ffi, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = 0x10000  # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def L():
    return _ffi.load()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "ptg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ptg_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert len(decl) >= 15
    assert set(decl) == set(_ffi.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


def test_exports_are_c_symbols():
    out = os.popen(f"nm -D --defined-only {_ffi.LIB_PATH}").read()
    syms = set(re.findall(r"\bT (ptg_\w+)", out))
    assert set(declared_functions()) <= syms


def test_status_strings(L):
    for code, name in _ffi.STATUS_NAMES.items():
        assert L.ptg_status_string(code).decode() == name
    assert L.ptg_version() >= 1


def gemm(L, M=64, N=64, K=64, A=P, lda=None, B=P, ldb=None, layout=0, C=P, ldc=None, dtype=0,
         bias=None, epi=0):
    lda = K if lda is None else lda
    ldb = (N if layout == 0 else K) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return L.ptg_gemm(M, N, K, A, lda, B, ldb, layout, C, ldc, dtype, bias, epi, None)


def test_gemm_validation(L):
    assert gemm(L, M=-1) == INVALID
    assert gemm(L, K=0) == UNSUPPORTED
    assert gemm(L, N=12) == UNSUPPORTED
    assert gemm(L, K=20) == UNSUPPORTED
    assert gemm(L, A=None) == INVALID
    assert gemm(L, C=None) == INVALID
    assert gemm(L, A=P + 2) == UNSUPPORTED
    assert gemm(L, lda=32) == INVALID
    assert gemm(L, ldb=8) == INVALID
    assert gemm(L, ldc=72 + 4) == UNSUPPORTED      # bf16 rows must stay 16-byte aligned
    assert gemm(L, layout=7) == UNSUPPORTED
    assert gemm(L, dtype=9) == UNSUPPORTED
    assert gemm(L, epi=4) == UNSUPPORTED
    assert gemm(L, epi=1, bias=None) == INVALID      # BIAS needs a bias vector
    assert gemm(L, M=1 << 31) == UNSUPPORTED
    assert "ptg_gemm" in L.ptg_last_error().decode()
    # empty problems are valid no-ops that never reach the device
    assert gemm(L, M=0, A=None, B=None, C=None) == OK
    assert gemm(L, N=0, A=None, B=None, C=None) == OK


def test_grouped_validation(L):
    def g(G=4, M=64, N=64, K=64, X=P, W=P, layout=0, off=P, Y=P, dtype=0, bias=None, epi=0):
        return L.ptg_grouped_gemm(G, M, N, K, X, W, layout, off, Y, dtype, bias, epi, None)
    assert g(G=0) == INVALID
    assert g(G=1025) == UNSUPPORTED
    assert g(K=0) == UNSUPPORTED
    assert g(off=None) == INVALID
    assert g(off=P + 2) == UNSUPPORTED
    assert g(X=P + 8) == UNSUPPORTED
    assert g(epi=3, bias=None) == INVALID
    assert g(M=0, X=None, W=None, Y=None, off=None) == OK


def _problems(n, dtype_rows=64):
    arr = (_ffi.ProblemStruct * n)()
    for i in range(n):
        s = arr[i]
        s.M, s.N, s.K = 64, 64, 64
        s.A = s.B = s.C = P
        s.lda = s.ldb = s.ldc = 64
    return arr


def test_ptr_array_validation(L):
    n = 3
    need = L.ptg_grouped_gemm_ptr_array_workspace(n)
    assert need >= 256 + 16 + n * 80
    assert L.ptg_grouped_gemm_ptr_array_workspace(0) == 0
    arr = _problems(n)
    for fn in (L.ptg_grouped_gemm_ptr_array_prepare, L.ptg_grouped_gemm_ptr_array):
        assert fn(0, arr, 0, 0, P, need, None) == INVALID
        assert fn(n, None, 0, 0, P, need, None) == INVALID
        assert fn(2049, arr, 0, 0, P, 1 << 30, None) == UNSUPPORTED
        assert fn(n, arr, 0, 0, P, need - 1, None) == WORKSPACE
        assert fn(n, arr, 0, 0, None, need, None) == WORKSPACE
        assert fn(n, arr, 0, 0, P + 8, need, None) == UNSUPPORTED
        assert fn(n, arr, 5, 0, P, need, None) == UNSUPPORTED       # bad output dtype
        assert fn(n, arr, 0, 4, P, need, None) == UNSUPPORTED       # bad epilogue
        arr[1].K = 12
        assert fn(n, arr, 0, 0, P, need, None) == UNSUPPORTED
        assert "problem 1" in L.ptg_last_error().decode()
        arr[1].K = 64
        arr[2].lda = 8
        assert fn(n, arr, 0, 0, P, need, None) == INVALID
        arr[2].lda = 64
        assert fn(n, arr, 0, 1, P, need, None) == INVALID           # bias missing
    assert L.ptg_grouped_gemm_ptr_array_run(n, P, need - 1, 0, 0, None) == WORKSPACE
    assert L.ptg_grouped_gemm_ptr_array_run(n, P, need, 5, 0, None) == UNSUPPORTED
    assert L.ptg_grouped_gemm_ptr_array_run(n, P, need, 0, 9, None) == UNSUPPORTED
    assert L.ptg_grouped_gemm_ptr_array_run(0, P, need, 0, 0, None) == INVALID
    assert L.ptg_grouped_gemm_ptr_array_run(2049, P, 1 << 30, 0, 0, None) == UNSUPPORTED


def test_ptr_array_output_extent(L):
    """An output row stride whose 256-row tile needs 2^31 bytes or more is refused; the limit
    depends on the output element size (fp32 rows are twice as wide)."""
    n = 2
    need = L.ptg_grouped_gemm_ptr_array_workspace(n)
    arr = _problems(n)
    # bf16: (255 * ldc + 256) * 2 < 2^31  <=>  ldc <= 4210751 (as a multiple of 8: 4210744).  At the limit
    # problem 0 passes, and the call stops at problem 1, made invalid so that nothing runs.
    arr[1].K = 12
    arr[0].ldc = 4210744
    assert L.ptg_grouped_gemm_ptr_array_prepare(n, arr, 0, 0, P, need, None) == UNSUPPORTED
    assert "problem 1" in L.ptg_last_error().decode()
    arr[0].ldc = 4210752
    assert L.ptg_grouped_gemm_ptr_array_prepare(n, arr, 0, 0, P, need, None) == UNSUPPORTED
    assert "problem 0" in L.ptg_last_error().decode()
    arr[1].K = 64
    assert L.ptg_grouped_gemm_ptr_array_prepare(n, arr, 0, 0, P, need, None) == UNSUPPORTED
    arr[0].ldc = 2105376                                           # fp32: at most 2105368
    assert L.ptg_grouped_gemm_ptr_array_prepare(n, arr, 1, 0, P, need, None) == UNSUPPORTED
    arr[0].ldc = 1 << 31                                           # 32-bit ldc
    assert L.ptg_grouped_gemm_ptr_array_prepare(n, arr, 0, 0, P, need, None) == UNSUPPORTED


def test_gemm_output_extent(L):
    # the output tile bound of ptg_gemm, per element size
    assert gemm(L, N=64, ldc=4210752) == UNSUPPORTED
    assert gemm(L, N=64, ldc=2105376, dtype=1) == UNSUPPORTED
    assert gemm(L, N=64, ldc=1 << 31) == UNSUPPORTED


def test_grouped_output_extent(L):
    def g(N, dtype):
        return L.ptg_grouped_gemm(4, 64, N, 64, P, P, 0, P, P, dtype, None, 0, None)
    # Y is dense (ld = N): the output tile bound caps N; W's K x N tile is checked too, so the
    # output check is what fails for the fp32 output at an N that passes for bf16 W
    assert g(2105376, 1) == UNSUPPORTED
    assert "output" in L.ptg_last_error().decode()


def test_broadcast_validation(L):
    U, N = 4, 64
    need = L.ptg_broadcast_gemm_workspace(U, N)
    # P plus one partial per slice of the split user phase (one 128 x 128 tile -> 32 slices)
    assert need == U * N * 4 * (1 + 32)
    # a user product with 256 or more tiles runs unsplit: P alone
    assert L.ptg_broadcast_gemm_workspace(16 * 256, 16 * 256) == 16 * 256 * 16 * 256 * 4

    def b(U=U, Mc=100, Ku=64, Kc=32, N=N, Xu=P, Xc=P, idx=P, W=P, layout=0, Y=P, dtype=0,
          bias=None, epi=0, ws=P, wsb=need):
        return L.ptg_broadcast_gemm(U, Mc, Ku, Kc, N, Xu, Xc, idx, W, layout, Y, dtype, bias, epi,
                                    ws, wsb, None)
    assert b(U=0) == INVALID
    assert b(Kc=0) == UNSUPPORTED
    assert b(Ku=12) == UNSUPPORTED
    assert b(idx=None) == INVALID
    assert b(wsb=need - 4) == WORKSPACE
    assert b(ws=None) == WORKSPACE
    assert b(Mc=0, Xu=None, Xc=None, idx=None, W=None, Y=None, ws=None, wsb=0) == OK
    # P (U x N fp32) is addressed with 31-bit offsets: U * N * 4 >= 2^31 is refused
    bigU, bigN = 1 << 17, 4096
    assert b(U=bigU, N=bigN, wsb=1 << 62) == UNSUPPORTED
    assert "P (U x N fp32)" in L.ptg_last_error().decode()


def test_broadcast_fused_validation(L):
    U, N = 4, 64
    need = L.ptg_broadcast_gemm_fused_workspace(U, N)
    # 4 KB of 64-bit sync words, the arrival flags (8 per slice and 256-column block, up to 32
    # slices) in 4 KB pages, then P and 32 partial products
    sync = (4096 + 1 * 32 * 8 * 4 + 4095) // 4096 * 4096
    assert need == sync + U * N * 4 * (1 + 32)

    def f(U=U, Mc=100, Ku=192, Kc=64, N=N, Xu=P, Xc=P, idx=P, W=P, layout=0, Y=P, dtype=0,
          bias=None, epi=0, ws=P, wsb=need):
        return L.ptg_broadcast_gemm_fused(U, Mc, Ku, Kc, N, Xu, Xc, idx, W, layout, Y, dtype, bias, epi,
                                          ws, wsb, None)
    assert f(U=0) == INVALID
    assert f(idx=None) == INVALID
    # one m-tile of users, at least two 64-deep slices of Ku, the sync words in their block
    assert f(U=257, wsb=1 << 40) == UNSUPPORTED
    assert "one launch" in L.ptg_last_error().decode()
    assert f(Ku=64) == UNSUPPORTED
    assert f(N=511 * 256 + 8, wsb=1 << 40) == UNSUPPORTED
    assert f(wsb=need - 16) == WORKSPACE
    assert f(ws=P + 8) == UNSUPPORTED
    assert f(Mc=0, Xu=None, Xc=None, idx=None, W=None, Y=None, ws=None, wsb=0) == OK


def test_wgrad_validation(L):
    need = L.ptg_grouped_gemm_wgrad_workspace()
    assert need == 256

    def w(G=4, M=100, K=64, N=32, X=P, dY=P, off=P, dW=P, dtype=0, ws=P, wsb=need):
        return L.ptg_grouped_gemm_wgrad(G, M, K, N, X, dY, off, dW, dtype, ws, wsb, None)
    assert w(G=0) == INVALID
    assert w(G=1025) == UNSUPPORTED
    assert w(M=-1) == INVALID
    assert w(K=12) == UNSUPPORTED
    assert w(N=20) == UNSUPPORTED
    assert w(dtype=7) == UNSUPPORTED
    assert w(X=None) == INVALID
    assert w(off=None) == INVALID
    assert w(dW=None) == INVALID
    assert w(ws=None) == WORKSPACE
    assert w(wsb=need - 1) == WORKSPACE
    assert w(ws=P + 8) == UNSUPPORTED
    assert w(off=P + 2) == UNSUPPORTED
    assert w(M=1 << 31) == UNSUPPORTED
    assert w(K=0, X=None, dY=None, dW=None, off=None, ws=None) == OK   # empty output: no-op
    assert w(N=0, X=None, dY=None, dW=None, off=None, ws=None) == OK


def test_attention_validation(L):
    def a(U=2, Mc=10, H=2, D=128, Lk=64, scale=0.088, Q=P, K=P, V=P, off=P, O=P, dtype=0):
        return L.ptg_ikbo_attention(U, Mc, H, D, Lk, scale, Q, K, V, off, O, dtype, None)
    assert a(U=0) == INVALID
    assert a(U=1025) == UNSUPPORTED
    assert a(H=0) == INVALID
    assert a(D=64) == UNSUPPORTED
    assert a(Lk=96) == UNSUPPORTED
    assert a(Lk=0) == INVALID
    assert a(dtype=5) == UNSUPPORTED
    assert a(scale=float("inf")) == INVALID
    assert a(scale=float("nan")) == INVALID
    assert a(Q=None) == INVALID
    assert a(off=None) == INVALID
    assert a(off=P + 2) == UNSUPPORTED
    assert a(O=P + 8) == UNSUPPORTED
    assert a(Mc=0, Q=None, K=None, V=None, off=None, O=None) == OK


def test_describe_config(L):
    cfg = (ctypes.c_int32 * 6)()
    assert L.ptg_describe_config(8192, 8192, 8192, 1, cfg) == OK
    big = list(cfg)
    assert big[:2] == [256, 256] and big[4] + big[5] <= 16
    assert L.ptg_describe_config(256, 256, 256, 0, cfg) == OK
    assert list(cfg)[:2] == [128, 128]
    assert L.ptg_describe_config(1, 1, 1, 0, None) == INVALID


def test_build_compiles_every_source_with_its_flags():
    # every source under csrc/ that is a translation unit is built, and only the GEMM kernels
    # take the max-ilp scheduler (the attention kernel keeps the default one)
    units = sorted(f for f in os.listdir(build.CSRC) if f.endswith((".hip", ".cpp")))
    assert units == sorted(build.SOURCES)
    ilp = "-amdgpu-sched-strategy=max-ilp"
    assert ilp in build.compile_flags(source="ptg_kernels.hip")
    assert ilp not in build.compile_flags(source="ptg_attention.hip")
    assert ilp not in build.compile_flags()
    for src in build.SOURCES:
        flags = build.compile_flags(source=src)
        assert "--offload-arch=gfx950" in flags and "-packed-fp32-ops" in flags


def test_broadcast_noalloc_validation(L):
    """Host-side refusals of the entry point that allocates nothing: the usual argument checks,
    and a workspace need beyond its 16 MiB scratch array."""
    def b(U=4, Mc=100, Ku=64, Kc=32, N=64, Xu=P, Xc=P, idx=P, W=P, layout=0, Y=P, dtype=0, bias=None, epi=0):
        return L.ptg_broadcast_gemm_noalloc(U, Mc, Ku, Kc, N, Xu, Xc, idx, W, layout, Y, dtype, bias, epi, None)
    assert b(U=0) == INVALID
    assert b(Kc=0) == UNSUPPORTED
    assert b(idx=None) == INVALID
    assert b(epi=1) == INVALID                      # bias missing
    assert b(Mc=0, Xu=None, Xc=None, idx=None, W=None, Y=None) == OK
    U, N = 256, 4096
    assert L.ptg_broadcast_gemm_workspace(U, N) > 16 << 20
    assert b(U=U, N=N) == UNSUPPORTED
    assert "16777216" in L.ptg_last_error().decode()


def test_grouped_split_validation(L):
    def g(G=4, M=64, N=64, K=64, X=P, W=P, layout=0, off=P, Y=P, dtype=0, bias=None, epi=0, ws=P, wsb=1 << 30):
        return L.ptg_grouped_gemm_split(G, M, N, K, X, W, layout, off, Y, dtype, bias, epi, ws, wsb, None)
    assert g(G=0) == INVALID
    assert g(K=0) == UNSUPPORTED
    assert g(off=None) == INVALID
    assert g(ws=None) == WORKSPACE
    assert g(ws=P + 8) == UNSUPPORTED
    assert g(M=0, X=None, W=None, Y=None, off=None, ws=None) == OK
