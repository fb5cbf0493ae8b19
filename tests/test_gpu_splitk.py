"""Split K (skinny M): the dense GEMM sums K slices into an fp32 workspace and a
second kernel adds them in slice order, then C, then rounds to bf16.  Parity
against the oracle, bit-exact integer cases, uneven slices, C aliased with D and
workspace growth on one stream."""

import numpy as np
import pytest
import torch

import fp4_gemm_dense_amd as dgm
import synth
from oracle import ref as R
from tests.helpers import bits, check_bit_exact, check_parity, sentinel_like
from tests.test_oracle import make_exact_case

pytestmark = pytest.mark.gpu


def _dev(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def _splits(M, N, K):
    return dgm.dg_query_plan(M, N, K, 1, 0)["splits"]


@pytest.mark.parametrize("M,N,K", [(40, 400, 128 * 37), (1, 16, 128 * 40), (64, 2112, 128 * 9),
                                   (100, 1024, 128 * 64)])
def test_splitk_random_parity(dg, M, N, K):
    assert _splits(M, N, K) > 1, "shape must take the split-K path"
    g = synth.gen_dense(M, N, K, seed=M + N + K, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    db = bits(d)
    assert not (db == 0xFFFF).any(), "every output element must be written"
    check_parity(db, R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"split {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,with_c", [(20, 144, 128 * 24, True), (64, 256, 128 * 24, False)])
def test_splitk_exact_integer_case_bit_exact(dg, M, N, K, with_c):
    """Integer-valued products and power-of-two scales: every partial sum is exact
    in fp32, so the sliced sum must equal the oracle bit for bit."""
    assert _splits(M, N, K) > 1
    rng = np.random.default_rng(M * N + K)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, with_c)
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    check_bit_exact(bits(d), exact, f"split exact {M}x{N}x{K}")


def test_splitk_d_aliases_c(dg):
    M, N, K = 48, 528, 128 * 20
    assert _splits(M, N, K) > 1
    g = synth.gen_dense(M, N, K, seed=5, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    cd = _dev(c)
    dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), cd, cd)
    torch.cuda.synchronize()
    check_parity(bits(cd), R.fp8_gemm_nt(a, sfa, b, sfb, c), what="split, d == c")


def test_splitk_workspace_grows_on_one_stream(dg):
    """A small split problem, then a larger one, then the small one again on a
    side stream: the workspace is reallocated and each result stays correct."""
    shapes = [(16, 256, 128 * 16), (128, 2112, 128 * 32), (16, 256, 128 * 16)]
    side = torch.cuda.Stream()
    for i, (M, N, K) in enumerate(shapes):
        assert _splits(M, N, K) > 1
        g = synth.gen_dense(M, N, K, seed=100 + i, with_c=True)
        a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
        ins = [_dev(x) for x in (a, sfa, b, sfb, c)]
        d = sentinel_like((M, N))
        torch.cuda.synchronize()
        if i == 2:
            with torch.cuda.stream(side):
                dg.dg_fp8_gemm_nt(*ins, d)
        else:
            dg.dg_fp8_gemm_nt(*ins, d)
        torch.cuda.synchronize()
        check_parity(bits(d), R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"split ws {M}x{N}x{K}")
