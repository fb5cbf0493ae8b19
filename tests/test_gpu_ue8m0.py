"""Parity of the FP8 GEMMs with packed UE8M0 scale factors
(dg_fp8_gemm_nt_ue8m0, dg_m_grouped_fp8_gemm_nt_{contiguous,masked}_ue8m0) against the
oracle on the GPU.

Tolerance: the FP8 GEMM's bar, per element |D - ref| <= 8e-3 * max(|ref|, rms(ref)) and
Frobenius 3e-3.  Row masks are checked bit-exactly against the bf16 sentinel 0xFFFF, and an
integer case whose every fp32 partial sum is exact must match the oracle bit for bit.
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


def _np(g, *keys):
    return [None if g[k] is None else synth.to_numpy(g[k]) for k in keys]


def _pack(exps):
    """exponent bytes [..., S] -> int32 words [..., ceil(S/4)] (byte i of word j: entry 4j+i)."""
    e = np.asarray(exps, np.int64)
    S = e.shape[-1]
    out = np.zeros(e.shape[:-1] + ((S + 3) // 4,), np.int64)
    for j in range(S):
        out[..., j // 4] |= e[..., j] << (8 * (j % 4))
    return out.astype(np.uint32).view(np.int32)


def _run_dense(dg, a, sfa, b, sfb, c):
    d = sentinel_like((a.shape[0], b.shape[0]))
    dg.dg_fp8_gemm_nt_ue8m0(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("M,N,K,with_c", [
    (1, 16, 128, False),
    (9, 144, 640, True),        # five K blocks: the second scale word is partly padding
    (130, 400, 1024, True),     # ragged M and N, two B scale blocks plus a partial one
    (256, 256, 512, False),
    (200, 272, 384, True),
    (64, 2112, 7168, False),    # skinny: split along K with the fp32 partial reduce
    (513, 1040, 1152, True),
])
def test_ue8m0_dense_parity(dg, M, N, K, with_c):
    g = synth.gen_dense_ue8m0(M, N, K, seed=M * 7 + N + K, with_c=with_c)
    a, sfa, b, sfb, c = _np(g, "a", "sfa", "b", "sfb", "c")
    d = _run_dense(dg, a, sfa, b, sfb, c)
    check_parity(d, R.fp8_gemm_nt_ue8m0(a, sfa, b, sfb, c), what=f"ue8m0 {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,with_c", [(9, 144, 384, True), (130, 400, 1024, True), (64, 2112, 7168, False)])
def test_ue8m0_dense_exact_integer_case_bit_exact(dg, M, N, K, with_c):
    """Integer values and power-of-two scales: every fp32 partial sum is exact, so D must
    be bf16(exact) bit for bit (split-K shape included)."""
    rng = np.random.default_rng(M + N + K + 1)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, with_c)
    ea = np.rint(np.log2(sfa.T)).astype(np.int64) + 127      # [M, KB]
    eb = np.rint(np.log2(sfb)).astype(np.int64) + 127        # [NB, KB]
    d = _run_dense(dg, a, _pack(ea), b, _pack(eb), c)
    check_bit_exact(d, exact, f"ue8m0 exact {M}x{N}x{K}")
    assert np.array_equal(R.fp8_gemm_nt_ue8m0(a, _pack(ea), b, _pack(eb), c), exact)


def test_ue8m0_contiguous_parity_and_padding_rows(dg):
    g = synth.gen_contiguous_ue8m0(4, 700, 400, 1152, seed=31, counts=[130, 0, 1, 569])
    a, sfa, b, sfb, mi = _np(g, "a", "sfa", "b", "sfb", "m_indices")
    d = sentinel_like((a.shape[0], b.shape[1]))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(mi), d)
    torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_contiguous_ue8m0(a, sfa, b, sfb, mi)
    assert np.all(db[~written] == SENTINEL) and not np.any(db[written] == SENTINEL)
    check_parity(db[written], ref[written], what="ue8m0 contiguous")


@pytest.mark.parametrize("K", [1152, 4096])   # 4096: long K, split planned on the device
def test_ue8m0_masked_parity_and_masked_rows(dg, K):
    mm = [0, 200, 7, 129, 64]
    g = synth.gen_masked_ue8m0(5, 200, 512, K, seed=41 + K, masked_m=mm)
    a, sfa, b, sfb = _np(g, "a", "sfa", "b", "sfb")
    d = sentinel_like((5, 200, 512))
    dg.dg_m_grouped_fp8_gemm_nt_masked_ue8m0(_dev(a), _dev(sfa), _dev(b), _dev(sfb),
                                             _dev(np.asarray(mm, np.int32)), d, 128)
    torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_masked_ue8m0(a, sfa, b, sfb, mm)
    assert np.all(db[~written] == SENTINEL) and not np.any(db[written] == SENTINEL)
    check_parity(db[written], ref[written], what=f"ue8m0 masked K{K}")


def test_ue8m0_dense_full_size_sampled(dg):
    """M 4096, N 7168, K 16384 with C, on the device; a random entry and the last-row /
    last-column entry of every 64 x 64 block against the oracle entry by entry."""
    M, N, K = 4096, 7168, 16384
    g = synth.gen_dense_ue8m0(M, N, K, seed=606, backend="torch", device="cuda")
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt_ue8m0(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(60)
    rows, cols = stratified_entries(M, N, rng)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    want = entries_in_chunks(lambda r, q: R.fp8_gemm_nt_ue8m0_entries(a, sfa, b, sfb, c, r, q), rows, cols)
    got = bits(d)[rows, cols]
    check_parity(got, want, what="ue8m0 full size sampled")
