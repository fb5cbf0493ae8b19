"""Parity of the M-grouped contiguous and masked GEMMs against the oracle on the GPU.

Group indexing and masks are checked bit-exactly: outputs are pre-filled with
the bf16 sentinel 0xFFFF and every row the layout leaves out must still hold
it, while every row it covers must be written.  Padding / garbage input rows
hold e4m3 NaN codes and NaN scales, so a leak into a valid row shows up as NaN.
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
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def _np(g, *keys):
    return [synth.to_numpy(g[k]) for k in keys]


# ----------------------------------------------------------------------------
# contiguous
# ----------------------------------------------------------------------------

def _run_contig(dg, a, sfa, b, sfb, mi):
    d = sentinel_like((a.shape[0], b.shape[1]))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(mi), d)
    torch.cuda.synchronize()
    return bits(d)


def _check_contig(d, ref, written, what):
    assert np.all(d[~written] == SENTINEL), f"{what}: rows outside the groups were written"
    assert not np.any(d[written] == SENTINEL), f"{what}: group rows left unwritten"
    check_parity(d[written], ref[written], what=what)


@pytest.mark.parametrize("kernel_id", [None, 5], ids=["planned", "128x512"])
@pytest.mark.parametrize("G,total,N,K,counts", [
    (4, 500, 160, 256, None),
    (3, 300, 272, 384, [0, 300, 0]),          # empty groups around a full one
    (5, 700, 2112, 256, [1, 127, 128, 129, 315]),
    (1, 130, 144, 128, None),
])
def test_contiguous_parity_and_padding(dg, monkeypatch, G, total, N, K, counts, kernel_id):
    if kernel_id is not None:
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    g = synth.gen_contiguous(G, total, N, K, seed=G * 31 + N, counts=counts)
    a, sfa, b, sfb, mi = _np(g, "a", "sfa", "b", "sfb", "m_indices")
    d = _run_contig(dg, a, sfa, b, sfb, mi)
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    _check_contig(d, ref, written, f"contig G{G} N{N} K{K}")


@pytest.mark.parametrize("kernel_id", [None, 5], ids=["planned", "128x512"])
def test_contiguous_exact_integer_groups_bit_exact(dg, monkeypatch, kernel_id):
    if kernel_id is not None:
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    rng = np.random.default_rng(5)
    N, K = 160, 384
    counts = [100, 0, 200]
    mi, _ = synth.padded_group_layout(counts)
    mi = np.array(mi, np.int32)
    M = mi.size
    a, sfa, _, _, _, _ = make_exact_case(rng, M, N, K, with_c=False)
    bs, sbs = [], []
    for _ in range(3):
        _, _, b, sfb, _, _ = make_exact_case(rng, 1, N, K, with_c=False)
        bs.append(b)
        sbs.append(sfb)
    b = np.stack(bs)
    sfb = np.stack(sbs)
    d = _run_contig(dg, a, sfa, b, sfb, mi)
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    assert np.all(d[~written] == SENTINEL)
    check_bit_exact(d[written], ref[written], "contig exact")


@pytest.mark.parametrize("kernel_id", [1, 2, 3, 5])
def test_contiguous_many_tiles_per_workgroup(dg, monkeypatch, kernel_id):
    """Two workgroups walk every tile in turn (short K, so many tiles each): the
    rows' group indices are loaded when a tile is set up and tested after its K
    loop, while the next tile's copies are already in flight (kernel 5, the
    128 x 512 tile, skips padding tiles while looking for its next unit)."""
    import fp4_gemm_dense_amd as dgm
    counts = [100, 0, 200, 7, 129]
    g = synth.gen_contiguous(len(counts), sum(counts), 400, 256, seed=77 + kernel_id, counts=counts)
    a, sfa, b, sfb, mi = _np(g, "a", "sfa", "b", "sfb", "m_indices")
    monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    dgm.dg_set_num_cus(2)
    try:
        d = _run_contig(dg, a, sfa, b, sfb, mi)
    finally:
        dgm.dg_set_num_cus(0)
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    _check_contig(d, ref, written, f"contig many tiles per workgroup, kernel {kernel_id}")


@pytest.mark.parametrize("kernel_id", [None, 5], ids=["planned", "128x512"])
def test_contiguous_malformed_indices_are_skipped(dg, monkeypatch, kernel_id):
    if kernel_id is not None:
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    g = synth.gen_contiguous(3, 256, 144, 256, seed=9, counts=[128, 64, 64])
    a, sfa, b, sfb, mi = _np(g, "a", "sfa", "b", "sfb", "m_indices")
    bad = mi.copy()
    bad[5] = 99            # out of range: skipped
    bad[130] = -7          # negative: skipped
    bad[300] = 0           # differs from its block's group (2): not written
    d = _run_contig(dg, a, sfa, b, sfb, bad)
    for r in (5, 130, 300):
        assert np.all(d[r] == SENTINEL), r
    clean = bad.copy()
    clean[[5, 130, 300]] = -1
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, clean)
    _check_contig(d, ref, written, "contig malformed")


@pytest.mark.parametrize("kernel_id", [None, 1], ids=["planned", "128x256"])
@pytest.mark.parametrize("nki", [0, 1])
def test_contiguous_full_size_sampled(dg, monkeypatch, nki, kernel_id):
    """8 experts, 32768 routed rows (multinomial), padded to 128; full size on the
    device, with the planned tile and with the 128 x 256 tile pinned."""
    if kernel_id is not None:
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    N, K = synth.GROUPED_NK[nki]
    g = synth.gen_contiguous(8, 32768, N, K, seed=synth.seed_for(2, nki), backend="torch", device="cuda")
    M = g["M"]
    d = sentinel_like((M, N))
    dg.dg_m_grouped_fp8_gemm_nt_contiguous(g["a"], g["sfa"], g["b"], g["sfb"], g["m_indices"], d)
    torch.cuda.synchronize()
    db = bits(d)
    mi = synth.to_numpy(g["m_indices"])
    valid = mi >= 0
    assert valid.sum() == 32768
    assert np.all(db[~valid] == SENTINEL)
    assert not np.any(db[valid] == SENTINEL)
    a, sfa, b, sfb = _np(g, "a", "sfa", "b", "sfb")
    rng = np.random.default_rng(nki)
    rows, cols = stratified_entries(M, N, rng, valid_rows=valid)   # every tile of valid rows
    got, want = [], []
    for grp in range(8):
        sel = mi[rows] == grp
        if not sel.any():
            continue
        want.append(entries_in_chunks(lambda r, q: R.fp8_gemm_nt_entries(a, sfa, b[grp], sfb[grp], None, r, q),
                                      rows[sel], cols[sel]))
        got.append(db[rows[sel], cols[sel]])
    check_parity(np.concatenate(got), np.concatenate(want), what=f"contig full N{N} K{K}")


# ----------------------------------------------------------------------------
# masked
# ----------------------------------------------------------------------------

def _run_masked(dg, a, sfa, b, sfb, mm, expected_m=0):
    G, max_m, _ = a.shape
    d = sentinel_like((G, max_m, b.shape[1]))
    dg.dg_m_grouped_fp8_gemm_nt_masked(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(np.asarray(mm, np.int32)),
                                       d, expected_m)
    torch.cuda.synchronize()
    return bits(d)


def _check_masked(d, ref, written, what):
    assert np.all(d[~written] == SENTINEL), f"{what}: rows >= masked_m were written"
    assert not np.any(d[written] == SENTINEL), f"{what}: valid rows left unwritten"
    if written.any():
        check_parity(d[written], ref[written], what=what)


@pytest.mark.parametrize("max_m,mm,N,K,expected", [
    (80, [0, 1, 63, 64, 80], 144, 384, 0),
    (300, [0, 1, 127, 128, 129, 255, 256, 257, 300], 160, 256, 0),
    (300, [0, 1, 127, 128, 129, 255, 256, 257, 300], 160, 256, 64),
    (256, [256, 0, 0, 13], 528, 128, 128),
])
def test_masked_parity_edges(dg, max_m, mm, N, K, expected):
    G = len(mm)
    g = synth.gen_masked(G, max_m, N, K, seed=max_m + N, masked_m=mm)
    a, sfa, b, sfb = _np(g, "a", "sfa", "b", "sfb")
    d = _run_masked(dg, a, sfa, b, sfb, mm, expected)
    ref, written = R.m_grouped_masked(a, sfa, b, sfb, mm)
    _check_masked(d, ref, written, f"masked max_m{max_m} N{N}")


def test_masked_out_of_range_counts_are_clamped(dg):
    mm = [-5, 1000, 40]
    g = synth.gen_masked(3, 64, 144, 256, seed=3, masked_m=[0, 64, 40])
    a, sfa, b, sfb = _np(g, "a", "sfa", "b", "sfb")
    d = _run_masked(dg, a, sfa, b, sfb, mm)
    ref, written = R.m_grouped_masked(a, sfa, b, sfb, [0, 64, 40])
    _check_masked(d, ref, written, "masked clamped")


def test_masked_exact_integer_bit_exact(dg):
    rng = np.random.default_rng(8)
    G, max_m, N, K = 3, 70, 144, 256
    mm = [70, 33, 0]
    a = np.zeros((G, max_m, K), np.uint8)
    sfa = np.zeros((G, K // 128, max_m), np.float32)
    b = np.zeros((G, N, K), np.uint8)
    sfb = np.zeros((G, 2, K // 128), np.float32)
    for i in range(G):
        a[i], sfa[i], b[i], sfb[i], _, _ = make_exact_case(rng, max_m, N, K, with_c=False)
    d = _run_masked(dg, a, sfa, b, sfb, mm)
    ref, written = R.m_grouped_masked(a, sfa, b, sfb, mm)
    assert np.all(d[~written] == SENTINEL)
    check_bit_exact(d[written], ref[written], "masked exact")


@pytest.mark.parametrize("nki", [0, 1])
def test_masked_full_size_sampled(dg, nki):
    """32 groups x 256 rows, masked_m ~ U{0..256}; full size on the device."""
    N, K = synth.GROUPED_NK[nki]
    g = synth.gen_masked(32, 256, N, K, seed=synth.seed_for(3, nki), backend="torch", device="cuda")
    mm = synth.to_numpy(g["masked_m"])
    d = sentinel_like((32, 256, N))
    dg.dg_m_grouped_fp8_gemm_nt_masked(g["a"], g["sfa"], g["b"], g["sfb"], g["masked_m"], d, 128)
    torch.cuda.synchronize()
    db = bits(d)
    written = np.arange(256)[None, :] < mm[:, None]
    assert np.all(db[~written] == SENTINEL)
    assert not np.any(db[written] == SENTINEL)
    a, sfa, b, sfb = _np(g, "a", "sfa", "b", "sfb")
    rng = np.random.default_rng(10 + nki)
    got, want = [], []
    for grp in range(32):
        if mm[grp] == 0:
            continue
        rows = rng.integers(0, mm[grp], 128)
        cols = rng.integers(0, N, 128)
        want.append(R.fp8_gemm_nt_entries(a[grp], sfa[grp], b[grp], sfb[grp], None, rows, cols))
        got.append(db[grp, rows, cols])
    check_parity(np.concatenate(got), np.concatenate(want), what=f"masked full N{N} K{K}")
