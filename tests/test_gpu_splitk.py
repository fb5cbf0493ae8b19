"""Split K (skinny M): the dense GEMM sums K slices into fp32 partial tiles in the
caller's workspace and a second kernel adds them in slice order, then C, then
rounds to bf16.  Parity against the oracle, bit-exact integer cases, uneven
slices, C aliased with D, and workspaces of every size on one stream."""

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


@pytest.fixture(params=["skinny", "square"])
def path(request, monkeypatch):
    """Skinny shapes run on the skinny-M kernel by default; "square" pins the
    square-tile kernel's 64 x 128 tile (DG_FORCE_KERNEL), whose split path also
    serves large problems' split tails and the other layouts."""
    if request.param == "square":
        monkeypatch.setenv("DG_FORCE_KERNEL", "3")
    return request.param


@pytest.mark.parametrize("M,N,K", [(40, 400, 128 * 37), (1, 16, 128 * 40), (64, 2112, 128 * 9),
                                   (100, 1024, 128 * 64)])
def test_splitk_random_parity(dg, path, M, N, K):
    if path == "square":
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
def test_splitk_exact_integer_case_bit_exact(dg, path, M, N, K, with_c):
    """Integer-valued products and power-of-two scales: every partial sum is exact
    in fp32, so the sliced sum must equal the oracle bit for bit."""
    assert path == "skinny" or _splits(M, N, K) > 1
    rng = np.random.default_rng(M * N + K)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, with_c)
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    check_bit_exact(bits(d), exact, f"split exact {M}x{N}x{K}")


def test_splitk_d_aliases_c(dg, path):
    M, N, K = 48, 528, 128 * 20
    assert path == "skinny" or _splits(M, N, K) > 1
    g = synth.gen_dense(M, N, K, seed=5, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    cd = _dev(c)
    dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), cd, cd)
    torch.cuda.synchronize()
    check_parity(bits(cd), R.fp8_gemm_nt(a, sfa, b, sfb, c), what="split, d == c")


def test_splitk_caller_workspace(dg, path):
    """The partials live in the caller's workspace: a too-small one is rejected before
    anything is enqueued (D keeps its sentinel), an exact-size one and a larger one
    holding garbage give the same bits, and one workspace serves a small call, a
    larger call and the small call again on a side stream."""
    M, N, K = 128, 2112, 128 * 32
    need = dgm.dg_fp8_gemm_workspace_bytes(dgm.FORM_NT, M, N, K)
    assert need > 0
    g = synth.gen_dense(M, N, K, seed=99, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    ins = [_dev(x) for x in (a, sfa, b, sfb, c)]
    d = sentinel_like((M, N))
    small = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(dgm.DgError) as e:
        dg.dg_fp8_gemm_nt(*ins, d, workspace=small)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert (bits(d) == 0xFFFF).all(), "a rejected call must write nothing"
    exact = torch.empty(need, dtype=torch.uint8, device="cuda")
    dg.dg_fp8_gemm_nt(*ins, d, workspace=exact)
    torch.cuda.synchronize()
    want = bits(d)
    check_parity(want, R.fp8_gemm_nt(a, sfa, b, sfb, c), what="split, exact workspace")
    big = torch.full((need + 4096,), 0xAB, dtype=torch.uint8, device="cuda")
    d2 = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(*ins, d2, workspace=big)
    torch.cuda.synchronize()
    assert np.array_equal(bits(d2), want)
    shapes = [(16, 256, 128 * 16), (128, 2112, 128 * 32), (16, 256, 128 * 16)]
    ws = torch.empty(max(dgm.dg_fp8_gemm_workspace_bytes(dgm.FORM_NT, *s) for s in shapes), dtype=torch.uint8,
                     device="cuda")
    side = torch.cuda.Stream()
    for i, (M, N, K) in enumerate(shapes):
        g = synth.gen_dense(M, N, K, seed=100 + i, with_c=True)
        a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
        ins = [_dev(x) for x in (a, sfa, b, sfb, c)]
        d = sentinel_like((M, N))
        torch.cuda.synchronize()
        if i == 2:
            with torch.cuda.stream(side):
                dg.dg_fp8_gemm_nt(*ins, d, workspace=ws)
        else:
            dg.dg_fp8_gemm_nt(*ins, d, workspace=ws)
        torch.cuda.synchronize()
        check_parity(bits(d), R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"split ws {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# split tail: whole rounds of tiles run unsplit, only the last partial round is
# split along K (a CU cap makes small problems take this path)
# ---------------------------------------------------------------------------
class _cu_cap:
    def __init__(self, n):
        self.n = n

    def __enter__(self):
        dgm.dg_set_num_cus(self.n)

    def __exit__(self, *exc):
        dgm.dg_set_num_cus(0)


def _tail_plan(M, N, K, cus):
    p = dgm.dg_query_plan(M, N, K, 1, cus)
    assert p["splits"] > 1 and 0 < p["full_tiles"] < p["num_tiles"], f"no split tail: {p}"
    return p


@pytest.mark.parametrize("M,N,K,cus,with_c", [(1280, 1024, 128 * 32, 32, True),
                                              (1100, 1040, 128 * 60, 32, True),
                                              (1300, 1040, 128 * 36, 48, False)])
def test_split_tail_random_parity(dg, M, N, K, cus, with_c):
    _tail_plan(M, N, K, cus)
    g = synth.gen_dense(M, N, K, seed=M + N + K + cus, with_c=with_c)
    a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    c = synth.to_numpy(g["c"]) if with_c else None
    d = sentinel_like((M, N))
    with _cu_cap(cus):
        dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
        torch.cuda.synchronize()
    db = bits(d)
    assert not (db == 0xFFFF).any(), "every output element must be written"
    check_parity(db, R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"split tail {M}x{N}x{K} on {cus} CUs")


def test_split_tail_exact_integer_case_bit_exact(dg):
    M, N, K, cus = 512, 640, 128 * 32, 8
    _tail_plan(M, N, K, cus)
    rng = np.random.default_rng(77)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, True)
    d = sentinel_like((M, N))
    with _cu_cap(cus):
        dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
        torch.cuda.synchronize()
    check_bit_exact(bits(d), exact, f"split tail exact {M}x{N}x{K}")


def test_split_tail_full_size_sampled_rows(dg):
    """4096 x 2112 x 7168 on the whole chip: 288 tiles of 128 x 256, of which 256
    run whole and 32 (the last rows of the raster) are split.  Sampled rows from
    both halves are checked against the oracle."""
    M, N, K = 4096, 2112, 7168
    ncu = dgm.dg_get_num_cus()
    p = dgm.dg_query_plan(M, N, K, 1, ncu)
    if not (p["splits"] > 1 and 0 < p["full_tiles"] < p["num_tiles"]):
        pytest.skip(f"no split tail on {ncu} CUs: {p}")
    g = synth.gen_dense(M, N, K, seed=4242, with_c=True, backend="torch", device="cuda")
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.sort(np.concatenate([rng.choice(M // 2, 24, replace=False),
                                   M // 2 + rng.choice(M // 2, 40, replace=False)]))
    db = bits(d)
    assert not (db == 0xFFFF).any(), "every output element must be written"
    t_rows = torch.from_numpy(rows).cuda()
    a = synth.to_numpy(g["a"][t_rows])
    sfa = synth.to_numpy(g["sfa"][:, t_rows])
    c = synth.to_numpy(g["c"][t_rows])
    b, sfb = synth.to_numpy(g["b"]), synth.to_numpy(g["sfb"])
    check_parity(db[rows], R.fp8_gemm_nt(a, sfa, b, sfb, c), what="split tail 4096x2112x7168 sampled rows")


def test_split_tail_then_pure_split_then_whole_on_one_stream(dg):
    """The workspace serves both split forms in turn; results stay correct."""
    cases = [(1280, 1024, 128 * 32, 32), (48, 528, 128 * 20, 0), (1024, 1024, 128 * 8, 0)]
    for i, (M, N, K, cus) in enumerate(cases):
        g = synth.gen_dense(M, N, K, seed=900 + i, with_c=True)
        a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
        d = sentinel_like((M, N))
        with _cu_cap(cus):
            dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
            torch.cuda.synchronize()
        check_parity(bits(d), R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"sequence {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# masked form: the kernel walks only the tiles holding valid rows and, over long
# K, applies the split rule to their count on the device
# ---------------------------------------------------------------------------
def _split_rule(tiles, slots, kb, min_gain=24):
    """Host mirror of the library's split rule (checked against dg_query_plan in
    test_boundary): returns (splits, whole tiles)."""
    if tiles <= 0 or kb < 8:
        return 1, tiles
    every = tiles * 2 <= slots
    rem = tiles if every else tiles % slots
    if rem == 0 or rem * 2 > slots:
        return 1, tiles
    s = min(slots // rem, kb // 4, 16)
    if s < 2:
        return 1, tiles
    per = -(-kb // s)
    s = -(-kb // per)
    if not every and kb - per < min_gain:
        return 1, tiles
    return s, tiles - rem


def _masked_device_plan(mm, max_m, N, K, cus):
    p = dgm.dg_query_plan(max_m, N, K, len(mm), cus)
    bm, bn = p["block_m"], p["block_n"]
    tiles = sum(-(-min(max(m, 0), max_m) // bm) for m in mm) * (-(-N // bn))
    return _split_rule(tiles, cus, K // 128)


@pytest.mark.parametrize("mm,max_m,N,K,cus", [
    ([256, 200, 3, 0], 256, 512, 128 * 48, 8),       # a partial last round, split
    ([256, 200, 3, 0], 256, 512, 128 * 40, 9),
    ([256, 3, 0], 256, 256, 128 * 32, 32),            # too few tiles to fill 32 CUs: every tile split
    ([100, 0, 256, 130, 7, 255], 256, 784, 128 * 40, 10),
    ([0, 0, 0], 128, 256, 128 * 32, 8),               # no valid rows at all
])
def test_masked_device_split_parity(dg, mm, max_m, N, K, cus):
    s, full = _masked_device_plan(mm, max_m, N, K, cus)
    if sum(mm) > 0:
        assert s > 1, f"the case must take the device-side split (plan {s}, {full})"
    g = synth.gen_masked(len(mm), max_m, N, K, seed=sum(mm) + N + cus, masked_m=mm)
    a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    d = sentinel_like((len(mm), max_m, N))
    with _cu_cap(cus):
        dg.dg_m_grouped_fp8_gemm_nt_masked(_dev(a), _dev(sfa), _dev(b), _dev(sfb),
                                           _dev(np.asarray(mm, np.int32)), d, 0)
        torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_masked(a, sfa, b, sfb, mm)
    assert np.all(db[~written] == 0xFFFF), "rows >= masked_m were written"
    assert not np.any(db[written] == 0xFFFF), "valid rows left unwritten"
    if written.any():
        check_parity(db[written], ref[written], what=f"masked device split {mm} on {cus} CUs")


def test_masked_device_split_exact_integer_bit_exact(dg):
    rng = np.random.default_rng(31)
    G, max_m, N, K, cus = 3, 256, 384, 128 * 48, 8
    mm = [256, 129, 40]
    s, _ = _masked_device_plan(mm, max_m, N, K, cus)
    assert s > 1
    a = np.zeros((G, max_m, K), np.uint8)
    sfa = np.zeros((G, K // 128, max_m), np.float32)
    b = np.zeros((G, N, K), np.uint8)
    sfb = np.zeros((G, -(-N // 128), K // 128), np.float32)
    for i in range(G):
        a[i], sfa[i], b[i], sfb[i], _, _ = make_exact_case(rng, max_m, N, K, with_c=False)
    d = sentinel_like((G, max_m, N))
    with _cu_cap(cus):
        dg.dg_m_grouped_fp8_gemm_nt_masked(_dev(a), _dev(sfa), _dev(b), _dev(sfb),
                                           _dev(np.asarray(mm, np.int32)), d, 0)
        torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_masked(a, sfa, b, sfb, mm)
    assert np.all(db[~written] == 0xFFFF)
    check_bit_exact(db[written], ref[written], "masked device split exact")


# ---------------------------------------------------------------------------
# contiguous form: the same split rule over its tiles (padding blocks skipped)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("counts,N,K,cus", [
    ([256, 384, 128, 512], 1024, 128 * 32, 32),       # whole blocks only
    ([300, 0, 100, 500, 380], 768, 128 * 48, 16),     # padding rows inside split tiles
])
def test_contiguous_split_tail_parity(dg, counts, N, K, cus):
    g = synth.gen_contiguous(len(counts), sum(counts), N, K, seed=sum(counts) + N, counts=counts)
    a, sfa, b, sfb, mi = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "m_indices"))
    M = mi.size
    p = dgm.dg_query_plan_contiguous(M, N, K, len(counts), cus)
    assert p["splits"] > 1 and 0 < p["full_tiles"] < p["num_tiles"], f"no split tail: {p}"
    d = sentinel_like((M, N))
    with _cu_cap(cus):
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(mi), d)
        torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    assert np.all(db[~written] == 0xFFFF), "padding rows were written"
    assert not np.any(db[written] == 0xFFFF), "group rows left unwritten"
    check_parity(db[written], ref[written], what=f"contig split tail {counts} on {cus} CUs")


@pytest.mark.parametrize("N", [768, 1024])
@pytest.mark.parametrize("exact", [False, True], ids=["random", "exact"])
def test_contiguous_split_tail_on_the_128x512_tile(dg, monkeypatch, N, exact):
    """The wide 128 x 512 tile's split path in the contiguous form: 16 whole tiles
    and 6 split in two on 16 workgroups, with an empty group and padding rows in
    split tiles (partial tiles summed by the split-K reduce, padding not written)."""
    monkeypatch.setenv("DG_FORCE_KERNEL", "5")
    counts, K, cus = [300, 0, 100, 500, 380], 128 * 48, 16
    mi, _ = synth.padded_group_layout(counts)
    mi = np.array(mi, np.int32)
    M = mi.size
    p = dgm.dg_query_plan_contiguous(M, N, K, len(counts), cus)
    assert p["kernel_id"] == 5 and p["splits"] > 1 and 0 < p["full_tiles"] < p["num_tiles"], p
    if exact:
        rng = np.random.default_rng(N)
        a, sfa, _, _, _, _ = make_exact_case(rng, M, N, K, with_c=False)
        bs, sbs = [], []
        for _ in counts:
            _, _, b1, sfb1, _, _ = make_exact_case(rng, 1, N, K, with_c=False)
            bs.append(b1)
            sbs.append(sfb1)
        b, sfb = np.stack(bs), np.stack(sbs)
    else:
        g = synth.gen_contiguous(len(counts), sum(counts), N, K, seed=N + 5, counts=counts)
        a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    d = sentinel_like((M, N))
    with _cu_cap(cus):
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(mi), d)
        torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    assert np.all(db[~written] == 0xFFFF), "padding rows were written"
    if exact:
        check_bit_exact(db[written], ref[written], "contig 128x512 split tail exact")
    else:
        assert not np.any(db[written] == 0xFFFF), "group rows left unwritten"
        check_parity(db[written], ref[written], what=f"contig 128x512 split tail N{N}")


def test_contiguous_split_tail_exact_integer_bit_exact(dg):
    rng = np.random.default_rng(17)
    counts, N, K, cus = [300, 0, 100, 500, 380], 768, 128 * 48, 16
    mi, _ = synth.padded_group_layout(counts)
    mi = np.array(mi, np.int32)
    M = mi.size
    p = dgm.dg_query_plan_contiguous(M, N, K, len(counts), cus)
    assert p["splits"] > 1 and 0 < p["full_tiles"] < p["num_tiles"]
    a, sfa, _, _, _, _ = make_exact_case(rng, M, N, K, with_c=False)
    bs, sbs = [], []
    for _ in counts:
        _, _, b1, sfb1, _, _ = make_exact_case(rng, 1, N, K, with_c=False)
        bs.append(b1)
        sbs.append(sfb1)
    b, sfb = np.stack(bs), np.stack(sbs)
    d = sentinel_like((M, N))
    with _cu_cap(cus):
        dg.dg_m_grouped_fp8_gemm_nt_contiguous(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(mi), d)
        torch.cuda.synchronize()
    db = bits(d)
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    assert np.all(db[~written] == 0xFFFF)
    check_bit_exact(db[written], ref[written], "contig split tail exact")
