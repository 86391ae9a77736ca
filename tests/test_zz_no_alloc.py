"""The entry point that allocates nothing, ptg_broadcast_gemm_noalloc, against the entry point it
is a variant of, ptg_broadcast_gemm (same kernels; P and the partial products in the library's
per-GPU scratch array instead of a caller's workspace): two calls in a row, the second smaller,
each bit-identical to ptg_broadcast_gemm on the same inputs, and both within the oracle's
tolerance.  Sizes beyond the scratch array are refused."""
import numpy as np
import pytest
import torch

import oracle
import pipelined_tiled_gemm_amd as ptg
import workloads as wl
from parity import check, dev, dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(w):
    return dev_bf16(w.Xu), dev_bf16(w.Xc), dev(w.idx), dev_bf16(w.W)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_broadcast_gemm_twice(out_dtype):
    ptg.watchdog(clear=True)
    # first call: 16 users, ragged candidates, bias + SiLU; second: fewer users and candidates,
    # so it reads only part of what the first left in the scratch array
    big = wl.broadcast(301, 16, 1024, 256, 512, cmin=1, cmax=700, with_bias=True, shuffle=True)
    small = wl.broadcast(302, 5, 256, 136, 264, cmin=1, cmax=200, with_bias=True)
    for w in (big, small):
        Xu, Xc, idx, W = _inputs(w)
        bias = dev(w.bias)
        ref = ptg.broadcast_gemm(Xu, Xc, idx, W, out_dtype=out_dtype, bias=bias, epi=wl.EPI_BIAS_SILU)
        out = torch.full_like(ref, float("nan"))
        ptg.broadcast_gemm_noalloc(Xu, Xc, idx, W, out=out, bias=bias, epi=wl.EPI_BIAS_SILU)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16) if out_dtype == torch.bfloat16 else out,
                           ref.view(torch.int16) if out_dtype == torch.bfloat16 else ref), \
            f"noalloc differs from broadcast_gemm (U={w.U}, Mc={w.Mc})"
        v = oracle.broadcast_gemm(w.Xu, w.Xc, w.idx, w.W, w.w_layout, w.bias, wl.EPI_BIAS_SILU)
        check(out, v, w.Ku + w.Kc, f"noalloc U={w.U} Mc={w.Mc}")
    assert ptg.watchdog(clear=True) == 0


def test_noalloc_refuses_sizes_beyond_its_scratch():
    # U x N x 4 x (1 + slices) above 16 MiB: 256 users x 4096 outputs need 4 MiB for P alone
    # and the split user phase's partials on top
    U, N = 256, 4096
    assert ptg.broadcast_gemm_workspace(U, N) > 16 << 20
    Xu = torch.zeros((U, 64), dtype=torch.bfloat16, device="cuda")
    Xc = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(8, dtype=torch.int32, device="cuda")
    W = torch.zeros((128, N), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((8, N), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ptg.PtgError) as e:
        ptg.broadcast_gemm_noalloc(Xu, Xc, idx, W, out=out)
    assert e.value.status == 2
