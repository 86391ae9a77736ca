"""Pipelined tiled GEMM for AMD Instinct MI355X (gfx950): Python binding of libptg.so.

Each function has the name of a C ABI entry point (include/ptg.h) without the ``ptg_``
prefix and only marshals arguments: tensors become device pointers, torch's current HIP
stream becomes the ``stream`` argument, and a non-OK status raises :class:`PtgError`.
All work runs in the library's kernels; there is no fallback path, and a missing
libptg.so raises ImportError at the first call.

PyTorch provides device memory and streams only.  bfloat16 tensors carry the bf16
operands; outputs are float32 or bfloat16 tensors.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _ffi

__all__ = [
    "PtgError", "B_KN", "B_NK", "EPI_NONE", "EPI_BIAS", "EPI_SILU", "EPI_BIAS_SILU",
    "gemm", "grouped_gemm", "grouped_gemm_split_workspace", "grouped_gemm_check", "grouped_gemm_wgrad", "grouped_gemm_wgrad_workspace", "ikbo_attention",
    "grouped_gemm_ptr_array_workspace", "grouped_gemm_ptr_array", "grouped_gemm_ptr_array_prepare",
    "grouped_gemm_ptr_array_run", "broadcast_gemm_workspace", "broadcast_gemm", "broadcast_gemm_noalloc",
    "broadcast_gemm_fused_workspace", "broadcast_gemm_fused",
    "broadcast_gemm_check", "watchdog", "version", "describe_config", "status_string",
    "last_error", "library_path",
]

B_KN, B_NK = 0, 1
EPI_NONE, EPI_BIAS, EPI_SILU, EPI_BIAS_SILU = 0, 1, 2, 3
_BF16, _F32 = 0, 1


class PtgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_ffi.STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def _lib():
    return _ffi.load()


def library_path() -> str:
    return _ffi.LIB_PATH


def status_string(status: int) -> str:
    return _lib().ptg_status_string(status).decode()


def last_error() -> str:
    return _lib().ptg_last_error().decode()


def version() -> int:
    return int(_lib().ptg_version())


def _check(status: int) -> None:
    if status != _ffi.PTG_OK:
        raise PtgError(status, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return _BF16
    if dtype == torch.float32:
        return _F32
    raise ValueError(f"output dtype must be bfloat16 or float32, not {dtype}")


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dims: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dimensions, got {t.dim()}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def _rowmajor_ld(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a row-major matrix view (unit stride along the last axis)."""
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError(f"{name} must be row-major (unit stride in the last dimension)")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def _bias_for(bias: Optional[torch.Tensor], epi: int, n: int, name: str, dims: int = 1):
    """The bias an epilogue reads (float32, on the GPU, contiguous, at least n entries), or
    None when the epilogue reads none."""
    if epi not in (EPI_BIAS, EPI_BIAS_SILU):
        return None
    if bias is None:
        raise ValueError(f"the epilogue needs a {name}")
    _need(bias, name, torch.float32, dims)
    if not bias.is_contiguous() or bias.numel() < n:
        raise ValueError(f"{name} must be contiguous with at least {n} entries")
    return bias


def describe_config(M: int, N: int, K: int, b_layout: int = B_KN):
    cfg = (ctypes.c_int32 * 6)()
    _check(_lib().ptg_describe_config(M, N, K, b_layout, cfg))
    return dict(zip(("BM", "BN", "BK", "stages", "consumers", "producers"), list(cfg)))


def watchdog(clear: bool = True) -> int:
    v = ctypes.c_uint32(0)
    _check(_lib().ptg_watchdog(ctypes.byref(v), 1 if clear else 0))
    return int(v.value)


# ------------------------------------------------------------------------------------------
def gemm(A: torch.Tensor, B: torch.Tensor, *, b_layout: int = B_KN, out: Optional[torch.Tensor] = None,
         out_dtype: torch.dtype = torch.bfloat16, bias: Optional[torch.Tensor] = None,
         epi: int = EPI_NONE, stream=None) -> torch.Tensor:
    """C = epi(A.B + bias).  A [M, K] bf16; B [K, N] (B_KN) or [N, K] (B_NK) bf16."""
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, K = A.shape
    N = B.shape[1] if b_layout == B_KN else B.shape[0]
    kb = B.shape[0] if b_layout == B_KN else B.shape[1]
    if kb != K:
        raise ValueError(f"inner dimensions differ: A has K={K}, B has {kb}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=A.device)
    _need(out, "out", out.dtype, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError(f"out must be [{M}, {N}]")
    bias = _bias_for(bias, epi, N, "bias")
    _check(_lib().ptg_gemm(M, N, K, _ptr(A), _rowmajor_ld(A, "A"), _ptr(B), _rowmajor_ld(B, "B"),
                           b_layout, _ptr(out), _rowmajor_ld(out, "out"), _dtype_code(out.dtype),
                           _ptr(bias), epi, _stream(stream)))
    return out


def grouped_gemm_split_workspace() -> int:
    return int(_lib().ptg_grouped_gemm_split_workspace())


def grouped_gemm(X: torch.Tensor, W: torch.Tensor, group_offsets: torch.Tensor, *,
                 w_layout: int = B_KN, out: Optional[torch.Tensor] = None,
                 out_dtype: torch.dtype = torch.bfloat16, bias: Optional[torch.Tensor] = None,
                 epi: int = EPI_NONE, workspace: Optional[torch.Tensor] = None,
                 stream=None) -> torch.Tensor:
    """Y[r] = epi(X[r].W[g] + bias[g]) for offsets[g] <= r < offsets[g+1] (offsets on device).
    With `workspace` (uint8, device, at least grouped_gemm_split_workspace() bytes) the call is
    ptg_grouped_gemm_split: the last round of tiles may run as two units per tile."""
    _need(X, "X", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 3)
    _need(group_offsets, "group_offsets", torch.int32, 1)
    M, K = X.shape
    G = W.shape[0]
    N = W.shape[2] if w_layout == B_KN else W.shape[1]
    if group_offsets.shape[0] != G + 1:
        raise ValueError("group_offsets must have G + 1 entries")
    if not (X.is_contiguous() and W.is_contiguous() and group_offsets.is_contiguous()):
        raise ValueError("X, W and group_offsets must be contiguous")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    if not out.is_contiguous() or tuple(out.shape) != (M, N):
        raise ValueError(f"out must be a contiguous [{M}, {N}] tensor")
    if bias is not None and epi in (EPI_BIAS, EPI_BIAS_SILU) and tuple(bias.shape) != (G, N):
        raise ValueError(f"bias must be [{G}, {N}]")
    bias = _bias_for(bias, epi, G * N, "bias", dims=2)
    if workspace is None:
        _check(_lib().ptg_grouped_gemm(G, M, N, K, _ptr(X), _ptr(W), w_layout, _ptr(group_offsets),
                                       _ptr(out), _dtype_code(out.dtype), _ptr(bias), epi, _stream(stream)))
    else:
        _check(_lib().ptg_grouped_gemm_split(G, M, N, K, _ptr(X), _ptr(W), w_layout, _ptr(group_offsets),
                                             _ptr(out), _dtype_code(out.dtype), _ptr(bias), epi,
                                             _ptr(workspace), _workspace_bytes(workspace), _stream(stream)))
    return out


def grouped_gemm_wgrad_workspace() -> int:
    return int(_lib().ptg_grouped_gemm_wgrad_workspace())


def grouped_gemm_wgrad(X: torch.Tensor, dY: torch.Tensor, group_offsets: torch.Tensor, *,
                       out: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """dW[g] = X_g^T . dY_g over rows offsets[g] <= r < offsets[g+1] (offsets on device);
    returns dW of shape [G, K, N], zero for groups without rows.  `workspace` (uint8, device,
    at least grouped_gemm_wgrad_workspace() bytes) holds the tile queue; one is taken from
    torch's allocator when none is given."""
    _need(X, "X", torch.bfloat16, 2)
    _need(dY, "dY", torch.bfloat16, 2)
    _need(group_offsets, "group_offsets", torch.int32, 1)
    M, K = X.shape
    if dY.shape[0] != M:
        raise ValueError("X and dY must have the same number of rows")
    N = dY.shape[1]
    G = group_offsets.shape[0] - 1
    if not (X.is_contiguous() and dY.is_contiguous() and group_offsets.is_contiguous()):
        raise ValueError("X, dY and group_offsets must be contiguous")
    if out is None:
        out = torch.empty((G, K, N), dtype=out_dtype, device=X.device)
    if not out.is_contiguous() or tuple(out.shape) != (G, K, N):
        raise ValueError(f"out must be a contiguous [{G}, {K}, {N}] tensor")
    if workspace is None:
        workspace = torch.empty(grouped_gemm_wgrad_workspace(), dtype=torch.uint8, device=X.device)
    _check(_lib().ptg_grouped_gemm_wgrad(G, M, K, N, _ptr(X), _ptr(dY), _ptr(group_offsets), _ptr(out),
                                         _dtype_code(out.dtype), _ptr(workspace), workspace.numel(),
                                         _stream(stream)))
    return out


def ikbo_attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, user_offsets: torch.Tensor, *,
                   scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.bfloat16, stream=None) -> torch.Tensor:
    """O[c] = softmax(scale Q[c] . K[u]^T) . V[u] per head, u the user of candidate c
    (offsets[u] <= c < offsets[u+1], on device).  Q [Mc, H, D]; K, V [U, L, H, D]; D = 128."""
    _need(Q, "Q", torch.bfloat16, 3)
    _need(K, "K", torch.bfloat16, 4)
    _need(V, "V", torch.bfloat16, 4)
    _need(user_offsets, "user_offsets", torch.int32, 1)
    Mc, H, D = Q.shape
    U, L = K.shape[0], K.shape[1]
    if tuple(K.shape) != (U, L, H, D) or tuple(V.shape) != tuple(K.shape):
        raise ValueError("K and V must be [U, L, H, D] matching Q's H and D")
    if user_offsets.shape[0] != U + 1:
        raise ValueError("user_offsets must have U + 1 entries")
    if not (Q.is_contiguous() and K.is_contiguous() and V.is_contiguous() and user_offsets.is_contiguous()):
        raise ValueError("Q, K, V and user_offsets must be contiguous")
    if scale is None:
        scale = float(D) ** -0.5
    if out is None:
        out = torch.empty((Mc, H, D), dtype=out_dtype, device=Q.device)
    if not out.is_contiguous() or tuple(out.shape) != (Mc, H, D):
        raise ValueError(f"out must be a contiguous [{Mc}, {H}, {D}] tensor")
    _check(_lib().ptg_ikbo_attention(U, Mc, H, D, L, float(scale), _ptr(Q), _ptr(K), _ptr(V), _ptr(user_offsets),
                                     _ptr(out), _dtype_code(out.dtype), _stream(stream)))
    return out


def grouped_gemm_check(group_offsets: torch.Tensor, M_total: int, stream=None) -> None:
    """Raises PtgError (PTG_ERR_DEVICE_CHECK) when the device offsets break the precondition."""
    _need(group_offsets, "group_offsets", torch.int32, 1)
    _check(_lib().ptg_grouped_gemm_check(group_offsets.shape[0] - 1, M_total, _ptr(group_offsets),
                                         _stream(stream)))


def grouped_gemm_ptr_array_workspace(count: int) -> int:
    return int(_lib().ptg_grouped_gemm_ptr_array_workspace(count))


def _problem_array(problems: Sequence, epi: int):
    """The ptg_problem array of [(A, B, C[, bias]), ...] (B stored K x N) and the one output
    dtype every C shares."""
    if len(problems) == 0:
        raise ValueError("at least one problem is needed")
    arr = (_ffi.ProblemStruct * len(problems))()
    out_dtype = None
    for i, pr in enumerate(problems):
        A, B, C = pr[0], pr[1], pr[2]
        bias = pr[3] if len(pr) > 3 else None
        _need(A, f"A[{i}]", torch.bfloat16, 2)
        _need(B, f"B[{i}]", torch.bfloat16, 2)
        if not isinstance(C, torch.Tensor) or C.dim() != 2 or C.device.type != "cuda":
            raise ValueError(f"C[{i}] must be a 2-D GPU tensor")
        if out_dtype is None:
            out_dtype = C.dtype
        elif C.dtype != out_dtype:
            raise TypeError(f"C[{i}] is {C.dtype}, but C[0] is {out_dtype}: every output of a batch "
                            "must have one dtype")
        _dtype_code(C.dtype)
        M, K = A.shape
        N = B.shape[1]
        if B.shape[0] != K or tuple(C.shape) != (M, N):
            raise ValueError(f"problem {i}: shapes do not match")
        if epi in (EPI_BIAS, EPI_BIAS_SILU):
            if bias is None:
                raise ValueError(f"problem {i}: the epilogue needs a bias")
            _need(bias, f"bias[{i}]", torch.float32, 1)
            if not bias.is_contiguous() or bias.numel() < N:
                raise ValueError(f"bias[{i}] must be contiguous with at least N = {N} entries")
        else:
            bias = None
        s = arr[i]
        s.M, s.N, s.K = M, N, K
        s.A, s.B, s.C, s.bias = _ptr(A), _ptr(B), _ptr(C), _ptr(bias)
        s.lda, s.ldb, s.ldc = _rowmajor_ld(A, "A"), _rowmajor_ld(B, "B"), _rowmajor_ld(C, "C")
    return arr, out_dtype


def _workspace_bytes(workspace: torch.Tensor) -> int:
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return workspace.numel() * workspace.element_size()


def grouped_gemm_ptr_array(problems: Sequence, epi: int = EPI_NONE, workspace: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    """C_p = epi(A_p . B_p + bias_p) for problems [(A, B, C[, bias]), ...] (B stored K x N, every C
    of one dtype) in one persistent launch; returns the workspace used."""
    arr, out_dtype = _problem_array(problems, epi)
    if workspace is None:
        workspace = torch.empty(grouped_gemm_ptr_array_workspace(len(problems)), dtype=torch.uint8,
                                device=problems[0][0].device)
    _check(_lib().ptg_grouped_gemm_ptr_array(len(problems), arr, _dtype_code(out_dtype), epi, _ptr(workspace),
                                             _workspace_bytes(workspace), _stream(stream)))
    return workspace


def grouped_gemm_ptr_array_prepare(problems: Sequence, epi: int, workspace: torch.Tensor, stream=None) -> None:
    """Write the table of problems [(A, B, C[, bias]), ...] into a device workspace."""
    arr, out_dtype = _problem_array(problems, epi)
    _check(_lib().ptg_grouped_gemm_ptr_array_prepare(len(problems), arr, _dtype_code(out_dtype), epi,
                                                     _ptr(workspace), _workspace_bytes(workspace),
                                                     _stream(stream)))


def grouped_gemm_ptr_array_run(count: int, workspace: torch.Tensor, out_dtype: torch.dtype, epi: int,
                               stream=None) -> None:
    """Launch the batch whose table `workspace` holds (written by grouped_gemm_ptr_array_prepare)."""
    _check(_lib().ptg_grouped_gemm_ptr_array_run(count, _ptr(workspace), _workspace_bytes(workspace),
                                                 _dtype_code(out_dtype), epi, _stream(stream)))


def broadcast_gemm_workspace(U: int, N: int) -> int:
    return int(_lib().ptg_broadcast_gemm_workspace(U, N))


def _broadcast_args(Xu, Xc, user_idx, W, w_layout, out, out_dtype, bias, epi):
    _need(Xu, "Xu", torch.bfloat16, 2)
    _need(Xc, "Xc", torch.bfloat16, 2)
    _need(W, "W", torch.bfloat16, 2)
    _need(user_idx, "user_idx", torch.int32, 1)
    U, Ku = Xu.shape
    Mc, Kc = Xc.shape
    N = W.shape[1] if w_layout == B_KN else W.shape[0]
    kw = W.shape[0] if w_layout == B_KN else W.shape[1]
    if kw != Ku + Kc:
        raise ValueError(f"W must have Ku + Kc = {Ku + Kc} rows of reduction, has {kw}")
    if user_idx.shape[0] != Mc:
        raise ValueError("user_idx must have one entry per candidate row")
    for t, name in ((Xu, "Xu"), (Xc, "Xc"), (W, "W"), (user_idx, "user_idx")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out is None:
        out = torch.empty((Mc, N), dtype=out_dtype, device=Xc.device)
    if not out.is_contiguous() or tuple(out.shape) != (Mc, N):
        raise ValueError(f"out must be a contiguous [{Mc}, {N}] tensor")
    bias = _bias_for(bias, epi, N, "bias")
    return (U, Mc, Ku, Kc, N, _ptr(Xu), _ptr(Xc), _ptr(user_idx), _ptr(W), w_layout, _ptr(out),
            _dtype_code(out.dtype), _ptr(bias), epi), out


def broadcast_gemm(Xu: torch.Tensor, Xc: torch.Tensor, user_idx: torch.Tensor, W: torch.Tensor, *,
                   w_layout: int = B_KN, out: Optional[torch.Tensor] = None,
                   out_dtype: torch.dtype = torch.bfloat16, bias: Optional[torch.Tensor] = None,
                   epi: int = EPI_NONE, workspace: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Y[r] = epi([Xu[user_idx[r]] | Xc[r]].W + bias) without materialising Xu[user_idx]."""
    args, out = _broadcast_args(Xu, Xc, user_idx, W, w_layout, out, out_dtype, bias, epi)
    U, N = args[0], args[4]
    if workspace is None:
        workspace = torch.empty(max(broadcast_gemm_workspace(U, N), 16), dtype=torch.uint8,
                                device=Xc.device)
    _check(_lib().ptg_broadcast_gemm(*args, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))
    return out


def broadcast_gemm_fused_workspace(U: int, N: int) -> int:
    return int(_lib().ptg_broadcast_gemm_fused_workspace(U, N))


def broadcast_gemm_fused(Xu: torch.Tensor, Xc: torch.Tensor, user_idx: torch.Tensor, W: torch.Tensor, *,
                         w_layout: int = B_KN, out: Optional[torch.Tensor] = None,
                         out_dtype: torch.dtype = torch.bfloat16, bias: Optional[torch.Tensor] = None,
                         epi: int = EPI_NONE, workspace: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """broadcast_gemm as one persistent launch (user units, reduction units, candidate tiles)."""
    args, out = _broadcast_args(Xu, Xc, user_idx, W, w_layout, out, out_dtype, bias, epi)
    U, N = args[0], args[4]
    if workspace is None:
        workspace = torch.empty(max(broadcast_gemm_fused_workspace(U, N), 16), dtype=torch.uint8,
                                device=Xc.device)
    _check(_lib().ptg_broadcast_gemm_fused(*args, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(stream)))
    return out


def broadcast_gemm_noalloc(Xu: torch.Tensor, Xc: torch.Tensor, user_idx: torch.Tensor, W: torch.Tensor, *,
                           out: torch.Tensor, w_layout: int = B_KN, bias: Optional[torch.Tensor] = None,
                           epi: int = EPI_NONE, stream=None) -> torch.Tensor:
    """broadcast_gemm without a workspace and without any allocation (the caller passes `out`):
    the library's own per-GPU scratch array holds P (calls overlapping on one GPU race)."""
    if out is None:
        raise ValueError("out is required: this call allocates nothing")
    args, out = _broadcast_args(Xu, Xc, user_idx, W, w_layout, out, out.dtype, bias, epi)
    _check(_lib().ptg_broadcast_gemm_noalloc(*args, _stream(stream)))
    return out


def broadcast_gemm_check(U: int, user_idx: torch.Tensor, stream=None) -> None:
    """Raises PtgError (PTG_ERR_DEVICE_CHECK) when an index is outside [0, U)."""
    _need(user_idx, "user_idx", torch.int32, 1)
    _check(_lib().ptg_broadcast_gemm_check(U, user_idx.shape[0], _ptr(user_idx), _stream(stream)))
