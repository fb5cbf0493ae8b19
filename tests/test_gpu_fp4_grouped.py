"""Parity of the M-grouped FP8 x FP4 GEMM (dg_m_grouped_fp8_fp4_gemm_nt_{contiguous,masked})
against the oracle on the GPU.

Tolerance: per element |D - ref| <= 8e-3 * max(|ref|, rms(ref)), Frobenius 3e-3 (the
FP8 GEMM's bar: one bf16 rounding of an fp32 sum).  Row masks are checked bit-exactly
(outputs are pre-filled with the bf16 sentinel 0xFFFF), and an integer case whose every
fp32 partial sum is exact must match the oracle bit for bit.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import ref as R
from tests.helpers import SENTINEL, bits, check_bit_exact, check_parity, sentinel_like, stratified_lines

pytestmark = pytest.mark.gpu


def _np(g, *keys):
    return [synth.to_numpy(g[k]) for k in keys]


def _dev(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def _run_contig(dg, a, a_sf, b, b_sf, mi):
    d = sentinel_like((a.shape[0], b.shape[1]))
    dg.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(_dev(a), _dev(a_sf), _dev(b),
                                               dg.dg_transform_fp4_weight_sf(_dev(b_sf)), _dev(mi), d)
    torch.cuda.synchronize()
    return bits(d)


def _run_masked(dg, a, a_sf, b, b_sf, mm):
    G, max_m, _ = a.shape
    d = sentinel_like((G, max_m, b.shape[1]))
    dg.dg_m_grouped_fp8_fp4_gemm_nt_masked(_dev(a), _dev(a_sf), _dev(b), dg.dg_transform_fp4_weight_sf(_dev(b_sf)),
                                           _dev(np.asarray(mm, np.int32)), d, 0)
    torch.cuda.synchronize()
    return bits(d)


def _check(d, ref, written, what):
    assert np.all(d[~written] == SENTINEL), f"{what}: rows outside the groups were written"
    assert not np.any(d[written] == SENTINEL), f"{what}: group rows left unwritten"
    if written.any():
        check_parity(d[written], ref[written], what=what)


@pytest.mark.parametrize("counts,N,K", [
    ([100, 0, 129, 300], 256, 512),
    ([1, 127, 128], 512, 384),        # 3 K blocks: the last weight pair is half used
    ([130], 256, 128),                # one K block
    ([0, 0, 5], 768, 1024),
    ([100, 0, 129, 300], 400, 512),   # N % 256 != 0: a partial last column tile
    ([5, 60], 16, 256),               # N smaller than one column tile
])
def test_fp4_contiguous_parity_and_padding(dg, counts, N, K):
    g = synth.gen_fp4_contiguous(len(counts), sum(counts), N, K, seed=sum(counts) + N + K, counts=counts)
    a, a_sf, b, b_sf, mi = _np(g, "a", "a_sf", "b", "b_sf", "m_indices")
    d = _run_contig(dg, a, a_sf, b, b_sf, mi)
    ref, written = R.m_grouped_fp8_fp4_contiguous(a, a_sf, b, b_sf, mi)
    _check(d, ref, written, f"fp4 contig {counts} N{N} K{K}")


@pytest.mark.parametrize("mm,max_m,N,K", [
    ([0, 1, 127, 128, 129, 256], 256, 256, 640),
    ([300, -5, 40], 128, 512, 256),   # counts outside [0, max_m] are clamped
    ([3], 200, 256, 896),
    ([0, 129, 7], 160, 272, 640),     # partial last column tile
])
def test_fp4_masked_parity_and_clamping(dg, mm, max_m, N, K):
    clamped = [min(max(m, 0), max_m) for m in mm]
    g = synth.gen_fp4_masked(len(mm), max_m, N, K, seed=max_m + N + K, masked_m=clamped)
    a, a_sf, b, b_sf = _np(g, "a", "a_sf", "b", "b_sf")
    d = _run_masked(dg, a, a_sf, b, b_sf, mm)
    ref, written = R.m_grouped_fp8_fp4_masked(a, a_sf, b, b_sf, mm)
    _check(d, ref, written, f"fp4 masked {mm} N{N} K{K}")


def _exact_fp4_case(rng, rows, G, N, K):
    """Integer e4m3 values in [-4, 4], E2M1 codes, power-of-two scales constant over each
    group of 8 K positions: every product and fp32 partial sum is exact."""
    tab = {}
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c, v in zip(codes, vals):
        if np.isfinite(v) and v == np.round(v) and abs(v) <= 4 and v not in tab:
            tab[v] = c
    a = np.vectorize(tab.get)(rng.integers(-4, 5, (rows, K)).astype(np.float64)).astype(np.uint8)
    ea = rng.integers(125, 129, (rows, K // 128))
    ea = np.pad(ea, ((0, 0), (0, (-ea.shape[1]) % 4)))
    a_sf = (ea[:, 0::4] | (ea[:, 1::4] << 8) | (ea[:, 2::4] << 16) | (ea[:, 3::4] << 24)).astype(np.uint32).view(np.int32)
    b = rng.integers(0, 256, (G, N, K // 2)).astype(np.uint8)
    eb = rng.integers(125, 129, (G, N, K // 32))
    b_sf = (eb[..., 0::4] | (eb[..., 1::4] << 8) | (eb[..., 2::4] << 16) | (eb[..., 3::4] << 24)).astype(np.uint32).view(np.int32)
    return a, a_sf, b, b_sf


def test_fp4_contiguous_exact_integer_case_bit_exact(dg):
    rng = np.random.default_rng(12)
    counts, N, K = [100, 0, 200], 256, 512
    mi, _ = synth.padded_group_layout(counts)
    mi = np.array(mi, np.int32)
    a, a_sf, b, b_sf = _exact_fp4_case(rng, mi.size, len(counts), N, K)
    d = _run_contig(dg, a, a_sf, b, b_sf, mi)
    ref, written = R.m_grouped_fp8_fp4_contiguous(a, a_sf, b, b_sf, mi)
    assert np.all(d[~written] == SENTINEL)
    check_bit_exact(d[written], ref[written], "fp4 contig exact")


def test_fp4_masked_exact_integer_case_bit_exact(dg):
    rng = np.random.default_rng(13)
    G, max_m, N, K = 3, 160, 512, 384
    mm = [160, 33, 0]
    a, a_sf, b, b_sf = _exact_fp4_case(rng, G * max_m, G, N, K)
    a, a_sf = a.reshape(G, max_m, K), a_sf.reshape(G, max_m, -1)
    d = _run_masked(dg, a, a_sf, b, b_sf, mm)
    ref, written = R.m_grouped_fp8_fp4_masked(a, a_sf, b, b_sf, mm)
    assert np.all(d[~written] == SENTINEL)
    check_bit_exact(d[written], ref[written], "fp4 masked exact")


def test_fp4_contiguous_full_size_sampled(dg):
    """8 groups, ~32k rows, N 4096, K 7168 on the device; per group, the oracle evaluates
    the rows x columns made of one random and the last index of every 64-row block of the
    group's rows and every 64-column block, so every output tile is checked, its last row
    and column included.  (The weight scales are per row of B, so a column subset of B is
    an exact subproblem.)"""
    G, N, K = 8, 4096, 7168
    g = synth.gen_fp4_contiguous(G, 32768, N, K, seed=515, backend="torch", device="cuda")
    M = int(g["M"])
    d = sentinel_like((M, N))
    dg.dg_m_grouped_fp8_fp4_gemm_nt_contiguous(g["a"], g["a_sf"], g["b"], dg.dg_transform_fp4_weight_sf(g["b_sf"]),
                                               g["m_indices"], d)
    torch.cuda.synchronize()
    db = bits(d)
    mi = synth.to_numpy(g["m_indices"])
    assert np.all(db[mi < 0] == SENTINEL) and not np.any(db[mi >= 0] == SENTINEL)
    rng = np.random.default_rng(51)
    got, want = [], []
    b, b_sf = synth.to_numpy(g["b"]), synth.to_numpy(g["b_sf"])
    for grp in range(G):
        rows = stratified_lines(M, rng, valid=mi == grp)
        if rows.size == 0:
            continue
        cols = stratified_lines(N, rng)
        t_rows = torch.from_numpy(rows).cuda()
        a, a_sf = synth.to_numpy(g["a"][t_rows]), synth.to_numpy(g["a_sf"][t_rows])
        want.append(R.fp8_fp4_gemm_nt(a, a_sf, b[grp][cols], b_sf[grp][cols]).ravel())
        got.append(db[np.ix_(rows, cols)].ravel())
    check_parity(np.concatenate(got), np.concatenate(want), what="fp4 contig full size")


@pytest.mark.parametrize("G,N,K", [(1, 256, 128), (3, 200, 70 * 128), (2, 4096, 7168), (5, 65, 65 * 128)])
def test_transform_fp4_weight_sf_bit_exact(dg, G, N, K):
    """The weight-scale relayout against the oracle's, word for word (sizes straddle the
    64 x 64 transpose tiles in both directions)."""
    rng = np.random.default_rng(G * 1000 + N + K)
    sf = rng.integers(-2**31, 2**31 - 1, size=(G, N, K // 128), dtype=np.int64).astype(np.int32)
    out = torch.full((G, K // 128, N), -1, dtype=torch.int32, device="cuda")
    dg.dg_transform_fp4_weight_sf(_dev(sf), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), R.fp4_weight_sf_k_major(sf))
