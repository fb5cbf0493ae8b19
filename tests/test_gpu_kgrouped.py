"""Parity of the K-grouped FP8 GEMM in the TN layout (dg_k_grouped_fp8_gemm_tn_contiguous)
against the oracle on the GPU.

Tolerance: the FP8 GEMM's bar (per element 8e-3 * max(|ref|, rms(ref)), Frobenius 3e-3) per
group; a group without K rows must come out as exact zeros; an integer case whose every
fp32 partial sum is exact must match bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import ref as R
from tests.helpers import bits, check_bit_exact, check_parity, entries_in_chunks, sentinel_like, stratified_entries
from tests.test_oracle import make_exact_case

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run(dg, a, sfa, b, sfb, ks):
    G = len(ks)
    d = sentinel_like((G, a.shape[1], b.shape[1]))
    dg.dg_k_grouped_fp8_gemm_tn_contiguous(_dev(a), _dev(sfa), _dev(b), _dev(sfb),
                                           _dev(np.asarray(ks, np.int32)), d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("counts,M,N", [
    ([100, 0, 1, 569], 144, 400),     # an empty group; partial row and column tiles
    ([300], 256, 256),
    ([5, 7, 2000, 130, 0, 64], 512, 1040),
])
def test_k_grouped_parity_and_empty_groups(dg, counts, M, N):
    g = synth.gen_kgrouped_tn(len(counts), sum(counts), M, N, seed=sum(counts) + M + N, counts=counts)
    a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    ks = synth.to_numpy(g["ks"]).tolist()
    d = _run(dg, a, sfa, b, sfb, ks)
    ref = R.k_grouped_tn_contiguous(a, sfa, b, sfb, ks)
    for grp, kg in enumerate(ks):
        if kg == 0:
            assert np.all(d[grp] == 0), f"group {grp} without rows is not zero"
        else:
            check_parity(d[grp], ref[grp], what=f"k-grouped group {grp} ({kg} rows)")


def test_k_grouped_exact_integer_case_bit_exact(dg):
    rng = np.random.default_rng(97)
    ks = [256, 0, 128, 512]
    M, N, K = 144, 400, sum(ks)
    a, sfa, b, sfb, _, _ = make_exact_case(rng, M, N, K, False)
    a_km, b_kn = np.ascontiguousarray(a.T), np.ascontiguousarray(b.T)
    exact = R.k_grouped_tn_contiguous(a_km, sfa, b_kn, sfb, ks)   # exact: integers times powers of two
    d = _run(dg, a_km, sfa, b_kn, sfb, ks)
    for grp in range(len(ks)):
        check_bit_exact(d[grp], exact[grp], f"k-grouped exact group {grp}")


def test_k_grouped_counts_are_rounded_and_cut_at_k(dg):
    """Counts that are not multiples of 128, or run past K, are rounded down and cut."""
    g = synth.gen_kgrouped_tn(3, 512, 128, 256, seed=5, counts=[128, 256, 128])
    a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    d = _run(dg, a, sfa, b, sfb, [130, 300, 10000])
    ref = R.k_grouped_tn_contiguous(a, sfa, b, sfb, [128, 256, 128])
    for grp in range(3):
        check_parity(d[grp], ref[grp], what=f"clamped group {grp}")


def test_k_grouped_full_size_sampled(dg):
    """8 groups from 32768 tokens, M 4096, N 7168 on the device; in every group, a random
    entry and the last-row / last-column entry of every 64 x 64 block against the oracle."""
    G, M, N = 8, 4096, 7168
    g = synth.gen_kgrouped_tn(G, 32768, M, N, seed=909, backend="torch", device="cuda")
    d = sentinel_like((G, M, N))
    dg.dg_k_grouped_fp8_gemm_tn_contiguous(g["a"], g["sfa"], g["b"], g["sfb"], g["ks"], d)
    torch.cuda.synchronize()
    db = bits(d)
    ks = synth.to_numpy(g["ks"]).tolist()
    rng = np.random.default_rng(90)
    k0 = 0
    for grp, kg in enumerate(ks):
        rows, cols = stratified_entries(M, N, rng)
        a_mk = synth.to_numpy(g["a"][k0:k0 + kg].t().contiguous())
        b_nk = synth.to_numpy(g["b"][k0:k0 + kg].t().contiguous())
        sfa = synth.to_numpy(g["sfa"][k0 // 128:(k0 + kg) // 128])
        sfb = synth.to_numpy(g["sfb"][:, k0 // 128:(k0 + kg) // 128])
        want = entries_in_chunks(lambda r, q: R.fp8_gemm_nt_entries(a_mk, sfa, b_nk, sfb, None, r, q), rows, cols)
        check_parity(db[grp][rows, cols], want, what=f"k-grouped full size group {grp}")
        k0 += kg
