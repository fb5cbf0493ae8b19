"""Parity of the FP8 GEMMs in the NN, TN and TT layouts (dg_fp8_gemm_nn,
dg_m_grouped_fp8_gemm_nn_contiguous: B stored [K, N]; dg_fp8_gemm_tn / _tt: A stored [K, M])
against the oracle on the GPU.

Tolerance: the FP8 GEMM's bar, per element |D - ref| <= 8e-3 * max(|ref|, rms(ref)) and
Frobenius 3e-3; padding rows bit-exact against the bf16 sentinel; an integer case whose
every fp32 partial sum is exact bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import ref as R
from tests.helpers import SENTINEL, bits, check_bit_exact, check_parity, entries_in_chunks, sentinel_like, stratified_entries
from tests.test_oracle import make_exact_case

pytestmark = pytest.mark.gpu


def _dev(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def _run(dg, a, sfa, b_kn, sfb, c):
    d = sentinel_like((a.shape[0], b_kn.shape[1]))
    dg.dg_fp8_gemm_nn(_dev(a), _dev(sfa), _dev(b_kn), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("M,N,K,with_c", [
    (1, 16, 128, False),
    (9, 144, 384, True),        # N: one full and one partial 128-column tile
    (130, 400, 1024, True),
    (256, 256, 512, False),
    (513, 1040, 1152, True),
    (64, 2112, 7168, False),    # skinny: split along K
])
def test_nn_dense_parity(dg, M, N, K, with_c):
    g = synth.gen_dense_nn(M, N, K, seed=M + 3 * N + K, with_c=with_c)
    a, sfa, b, sfb, c = (None if g[k] is None else synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    d = _run(dg, a, sfa, b, sfb, c)
    check_parity(d, R.fp8_gemm_nn(a, sfa, b, sfb, c), what=f"nn {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,with_c", [(9, 144, 384, True), (130, 400, 1024, True), (256, 1024, 2048, False)])
def test_nn_dense_exact_integer_case_bit_exact(dg, M, N, K, with_c):
    rng = np.random.default_rng(M + N + K + 5)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, with_c)
    d = _run(dg, a, sfa, np.ascontiguousarray(b.T), sfb, c)
    check_bit_exact(d, exact, f"nn exact {M}x{N}x{K}")


def test_nn_contiguous_parity_and_padding_rows(dg):
    g = synth.gen_contiguous_nn(4, 700, 400, 1152, seed=33, counts=[130, 0, 1, 569])
    a, sfa, b, sfb, mi = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "m_indices"))
    d = sentinel_like((a.shape[0], b.shape[2]))
    dg.dg_m_grouped_fp8_gemm_nn_contiguous(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(mi), d)
    torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_nn_contiguous(a, sfa, b, sfb, mi)
    assert np.all(db[~written] == SENTINEL) and not np.any(db[written] == SENTINEL)
    check_parity(db[written], ref[written], what="nn contiguous")


def test_nn_dense_full_size_sampled(dg):
    """M 4096, N 7168, K 7168 with C on the device; a random entry and the last-row /
    last-column entry of every 64 x 64 block against the oracle entry by entry (B
    transposed back for the NT entry evaluator)."""
    M, N, K = 4096, 7168, 7168
    g = synth.gen_dense_nn(M, N, K, seed=707, backend="torch", device="cuda")
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nn(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(70)
    rows, cols = stratified_entries(M, N, rng)
    a, sfa, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "sfb", "c"))
    b_nk = synth.to_numpy(g["b"].t().contiguous())
    want = entries_in_chunks(lambda r, q: R.fp8_gemm_nt_entries(a, sfa, b_nk, sfb, c, r, q), rows, cols)
    check_parity(bits(d)[rows, cols], want, what="nn full size sampled")


@pytest.mark.parametrize("kernel_id", [0, 1, 2, 3])
def test_nn_every_tile_shape(dg, kernel_id, monkeypatch):
    """Each compiled tile shape (256x128, 128x256, 128x128, 64x128) on the NN path, with a
    partial last column tile and C."""
    monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    M, N, K = 300, 656, 1024
    g = synth.gen_dense_nn(M, N, K, seed=90 + kernel_id)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    d = _run(dg, a, sfa, b, sfb, c)
    check_parity(d, R.fp8_gemm_nn(a, sfa, b, sfb, c), what=f"nn kernel {kernel_id}")



def _run_t(dg, fn, a_km, sfa, b, sfb, c, N):
    d = sentinel_like((a_km.shape[1], N))
    fn(_dev(a_km), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("b_kn", [True, False], ids=["tn", "tt"])
@pytest.mark.parametrize("M,N,K,with_c,kernel_id", [
    (16, 16, 128, False, None),
    (144, 400, 1024, True, None),     # partial row and column tiles
    (512, 1040, 1152, True, None),
    (64, 2112, 7168, False, None),    # skinny: split along K
    (272, 656, 1024, True, 0),        # each tile shape whose height is a multiple of 128
    (272, 656, 1024, True, 1),
    (272, 656, 1024, True, 2),
])
def test_tn_tt_dense_parity(dg, monkeypatch, b_kn, M, N, K, with_c, kernel_id):
    if kernel_id is not None:
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    g = synth.gen_dense_tn(M, N, K, seed=M + 5 * N + K + b_kn, with_c=with_c, b_kn=b_kn)
    a, sfa, b, sfb, c = (None if g[k] is None else synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    fn = dg.dg_fp8_gemm_tn if b_kn else dg.dg_fp8_gemm_tt
    d = _run_t(dg, fn, a, sfa, b, sfb, c, N)
    ref = (R.fp8_gemm_tn if b_kn else R.fp8_gemm_tt)(a, sfa, b, sfb, c)
    check_parity(d, ref, what=f"{'tn' if b_kn else 'tt'} {M}x{N}x{K} kernel {kernel_id}")


@pytest.mark.parametrize("b_kn", [True, False], ids=["tn", "tt"])
def test_tn_tt_exact_integer_case_bit_exact(dg, b_kn):
    M, N, K = 144, 400, 1024
    rng = np.random.default_rng(31 + b_kn)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, True)
    fn = dg.dg_fp8_gemm_tn if b_kn else dg.dg_fp8_gemm_tt
    d = _run_t(dg, fn, np.ascontiguousarray(a.T), sfa, np.ascontiguousarray(b.T) if b_kn else b, sfb, c, N)
    check_bit_exact(d, exact, f"{'tn' if b_kn else 'tt'} exact")


def test_tn_dense_full_size_sampled(dg):
    M, N, K = 4096, 7168, 7168
    g = synth.gen_dense_tn(M, N, K, seed=808, backend="torch", device="cuda")
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_tn(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(80)
    rows, cols = stratified_entries(M, N, rng)
    sfa, sfb, c = (synth.to_numpy(g[k]) for k in ("sfa", "sfb", "c"))
    a_mk = synth.to_numpy(g["a"].t().contiguous())
    b_nk = synth.to_numpy(g["b"].t().contiguous())
    want = entries_in_chunks(lambda r, q: R.fp8_gemm_nt_entries(a_mk, sfa, b_nk, sfb, c, r, q), rows, cols)
    check_parity(bits(d)[rows, cols], want, what="tn full size sampled")
