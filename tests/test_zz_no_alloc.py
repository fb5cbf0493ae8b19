"""dg_fp8_gemm_nt_noalloc, called through the C ABI: the dense NT GEMM whose split-K
partials live in the library's static per-GPU scratch buffer.  Its output must equal
that of dg_fp8_gemm_nt (same kernels and plan, caller workspace) bit for bit, on calls
in a row that reuse the buffer (a large split call, then a smaller one with C, then a
call that needs no scratch), and a plan needing more than the buffer holds must be
rejected before anything is written."""

import ctypes

import numpy as np
import pytest
import torch

import fp4_gemm_dense_amd as dgm
import synth
from tests.helpers import bits, sentinel_like

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 24 << 20


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(g, d):
    M, K = g["a"].shape
    N = g["b"].shape[0]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return dgm.lib().dg_fp8_gemm_nt_noalloc(_p(g["a"]), _p(g["sfa"]), _p(g["b"]), _p(g["sfb"]), _p(g["c"]), _p(d),
                                            M, N, K, stream)


def _with_workspace(g, d):
    M, K = g["a"].shape
    N = g["b"].shape[0]
    need = dgm.dg_fp8_gemm_workspace_bytes(dgm.FORM_NT, M, N, K)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return dgm.lib().dg_fp8_gemm_nt(_p(g["a"]), _p(g["sfa"]), _p(g["b"]), _p(g["sfb"]), _p(g["c"]), _p(d),
                                    M, N, K, _p(ws), ws.numel(), stream), need


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_the_workspace_entry_point(dg, order):
    cases = [(128, 2112, 7168, False, 11),    # split along K, 7.4 MiB of partials
             (40, 400, 128 * 37, True, 12),   # smaller split call with C: the buffer holds the last call's partials
             (512, 1024, 1024, True, 13)]     # no split: the buffer is not used
    for M, N, K, with_c, seed in cases:
        g = synth.gen_dense(M, N, K, seed=seed, with_c=with_c, backend="torch", device="cuda")
        d_ref = sentinel_like((M, N))
        st, need = _with_workspace(g, d_ref)
        assert st == 0, dgm.dg_status_string(st)
        assert need <= SCRATCH_BYTES
        d = sentinel_like((M, N))
        st = _noalloc(g, d)
        assert st == 0, dgm.dg_status_string(st)
        torch.cuda.synchronize()
        want = bits(d_ref)
        assert not (want == 0xFFFF).any()
        assert np.array_equal(bits(d), want), f"{M}x{N}x{K}: noalloc output differs from dg_fp8_gemm_nt"


def test_noalloc_rejects_plans_beyond_the_scratch(dg):
    M, N, K = 4096, 2112, 7168          # its split tail needs 256 partial 128x256 tiles (32 MiB) on 256 CUs
    need = dgm.dg_fp8_gemm_workspace_bytes(dgm.FORM_NT, M, N, K)
    if need <= SCRATCH_BYTES:
        pytest.skip(f"on this CU count the plan needs only {need} bytes")
    g = synth.gen_dense(M, N, K, seed=14, with_c=False, backend="torch", device="cuda")
    d = sentinel_like((M, N))
    torch.cuda.synchronize()
    assert _noalloc(g, d) == 5          # DG_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert (bits(d) == 0xFFFF).all(), "a rejected call must write nothing"
