"""Parity of the dense NT GEMM (dg_fp8_gemm_nt) against the oracle on the GPU."""

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import ref as R
from tests.helpers import bits, check_bit_exact, check_parity, entries_in_chunks, sentinel_like, stratified_entries
from tests.test_oracle import make_exact_case

pytestmark = pytest.mark.gpu


def _dev(x):
    """numpy -> device tensor (uint16 bf16 bit patterns travel as int16)."""
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def _run(dg, a, sfa, b, sfb, c):
    M, N = a.shape[0], b.shape[0]
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("M,N,K,with_c", [(9, 144, 384, True), (200, 272, 384, False), (130, 400, 1024, True),
                                          (256, 256, 256, True), (1, 16, 128, False)])
def test_dense_exact_integer_case_bit_exact(dg, M, N, K, with_c):
    rng = np.random.default_rng(M + N + K)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, with_c)
    check_bit_exact(_run(dg, a, sfa, b, sfb, c), exact, f"exact {M}x{N}x{K}")


def test_dense_all_256_e4m3_codes_decode_like_ocp(dg):
    """Row 0 of A holds every finite e4m3 code once; B is the identity, scales 1:
    D[0, n] must be the OCP e4m3fn value of code n (exact in bf16)."""
    K = N = 256
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    a = np.zeros((3, K), np.uint8)
    a[0] = codes
    a[1] = codes[::-1]
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), np.arange(N)] = 0x38
    sfa = np.ones((K // 128, 3), np.float32)
    sfb = np.ones((2, 2), np.float32)
    d = _run(dg, a, sfa, b, sfb, None)
    want = R.fp8_gemm_nt(a, sfa, b, sfb)
    assert np.array_equal(want[0], F.decode_e4m3(codes))
    check_bit_exact(d, want, "256 codes")


def test_dense_identity_b_and_all_ones(dg):
    rng = np.random.default_rng(3)
    M, N, K = 70, 256, 256
    g = synth.gen_dense(M, N, K, seed=77, with_c=False)
    a, sfa = synth.to_numpy(g["a"]), synth.to_numpy(g["sfa"])
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), np.arange(N)] = 0x38
    sfb = rng.uniform(0.5, 2, (2, 2)).astype(np.float32)
    d = _run(dg, a, sfa, b, sfb, None)
    check_bit_exact(d, R.fp8_gemm_nt(a, sfa, b, sfb), "identity-B")
    # all ones with C: D = C + K * sa * sb
    M, N, K = 33, 160, 512
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    sfa = np.full((K // 128, M), 0.5, np.float32)
    sfb = np.full((2, K // 128), 0.25, np.float32)
    c = synth.to_numpy(synth.bf16_bits(torch.full((M, N), 3.0)))
    d = _run(dg, a, sfa, b, sfb, c)
    assert np.all(F.bf16_bits_to_f64(d) == K * 0.5 * 0.25 + 3.0)


@pytest.mark.parametrize("kernel_id", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("K", [128, 256, 384, 640])
@pytest.mark.parametrize("with_c", [True, False], ids=["c", "no_c"])
def test_dense_many_tiles_per_workgroup_bit_exact(dg, monkeypatch, kernel_id, K, with_c):
    """Three workgroups walk every tile in turn, so each runs many tiles back to
    back, with and without C.  A tile starts its LDS ring in the slot of the
    previous tile's last K block and stages C (or D over C) in LDS; one to five K
    blocks per tile cover every step of the ring start (K blocks - 1 modulo the
    slot count).  Kernels 4-6 are the 256 x 256, 128 x 512 and 256 x 224 tiles,
    whose next tile's first stage goes to a different slot with C than without.
    Exact integer inputs: the result is unique."""
    import fp4_gemm_dense_amd as dgm
    rng = np.random.default_rng(kernel_id * 10 + K + (0 if with_c else 5))
    M, N = 520, 784                     # ragged in both dimensions for every tile shape
    a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, with_c)
    monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    dgm.dg_set_num_cus(3)
    try:
        p = dgm.dg_query_plan(M, N, K, 1, 3)
        assert p["splits"] == 1
        got = _run(dg, a, sfa, b, sfb, c)
    finally:
        dgm.dg_set_num_cus(0)
    check_bit_exact(got, exact, f"many tiles per workgroup, kernel {kernel_id}, K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (17, 144, 384), (64, 528, 1024), (130, 2112, 256),
                                   (300, 400, 640), (513, 1040, 384)])
def test_dense_random_parity(dg, M, N, K):
    g = synth.gen_dense(M, N, K, seed=M * 7 + N + K, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    d = _run(dg, a, sfa, b, sfb, c)
    assert not (d == 0xFFFF).any(), "every output element must be written"
    check_parity(d, R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("kernel_id", [0, 1, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("splits_wanted", [False, True])
def test_dense_every_tile_random_parity(dg, monkeypatch, kernel_id, splits_wanted):
    """Every tile shape, pinned, on random inputs with C and ragged M and N:
    per-row and per-block scales that differ everywhere, so a partial promoted with
    another block's scale, or the last row block's partials promoted with the wrong
    K block's scale, fails the tolerance (the exact-integer cases use equal scales).
    With 64 CUs the 12 tiles cannot fill the chip and every tile is split along K,
    which sends the partials through the workspace and the reduce kernel; with 5
    CUs the workgroups walk several tiles each, unsplit."""
    import fp4_gemm_dense_amd as dgm
    bm, bn = {0: (256, 128), 1: (128, 256), 2: (128, 128), 3: (64, 128), 4: (256, 256), 5: (128, 512),
              6: (256, 224)}[kernel_id]
    M, N, K = 2 * bm + bm // 2 + 3, 3 * bn + 48, 128 * 24
    g = synth.gen_dense(M, N, K, seed=500 + kernel_id * 2 + splits_wanted, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    monkeypatch.setenv("DG_FORCE_KERNEL", str(kernel_id))
    cus = 64 if splits_wanted else 5
    dgm.dg_set_num_cus(cus)
    try:
        p = dgm.dg_query_plan(M, N, K, 1, cus)
        assert p["kernel_id"] == kernel_id and (p["splits"] > 1) == splits_wanted, p
        d = _run(dg, a, sfa, b, sfb, c)
    finally:
        dgm.dg_set_num_cus(0)
    assert not (d == 0xFFFF).any(), "every output element must be written"
    check_parity(d, R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"kernel {kernel_id} splits {splits_wanted} {M}x{N}x{K}")


def test_dense_config0_full_parity(dg):
    """M=128, N=2112, K=7168, C = 0 (passed as NULL): the whole output vs the oracle."""
    g = synth.gen_dense(128, 2112, 7168, seed=synth.seed_for(0, 0), with_c=False)
    a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    d = _run(dg, a, sfa, b, sfb, None)
    check_parity(d, R.fp8_gemm_nt(a, sfa, b, sfb), what="config0")


@pytest.mark.parametrize("mi,nki", [(m, j) for m in range(2) for j in range(6)])
def test_dense_sweep_full_size_sampled(dg, mi, nki):
    """The dense sweep shapes at full size, generated on the device; the oracle
    evaluates, one by one, a random entry and the last-row/last-column entry of every
    64 x 64 block of D, so every output tile of the plan is checked."""
    M = synth.DENSE_M[mi]
    N, K = synth.DENSE_NK[nki]
    g = synth.gen_dense(M, N, K, seed=synth.seed_for(1, mi * 6 + nki), backend="torch", device="cuda")
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d)
    torch.cuda.synchronize()
    db = bits(d)
    assert not (db == 0xFFFF).any()
    rng = np.random.default_rng(mi * 6 + nki)
    rows, cols = stratified_entries(M, N, rng)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    ref = entries_in_chunks(lambda r, q: R.fp8_gemm_nt_entries(a, sfa, b, sfb, c, r, q), rows, cols)
    check_parity(db[rows, cols], ref, what=f"sweep M={M} N={N} K={K}")


def test_wide_tile_matches_square_tiles_bitwise(dg, monkeypatch):
    """The 256 x 256, 128 x 512 and 256 x 224 tiles promote each K block's
    partial with the same fused multiply-add, in the same K order, as the
    square-tile template: on random inputs with C their outputs are bit-identical
    to the 128 x 256 and 256 x 128 tiles' (a different accumulation order, or a
    column block promoted with the neighbouring 128-column block's B scale, would
    differ in many elements).  N = 1040 puts 224-wide tile edges at every offset
    into a 128-column scale block that is a multiple of 32."""
    M, N, K = 1000, 1040, 2048
    g = synth.gen_dense(M, N, K, seed=4242, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    outs = {}
    for kid in (0, 1, 4, 5, 6):
        monkeypatch.setenv("DG_FORCE_KERNEL", str(kid))
        outs[kid] = _run(dg, a, sfa, b, sfb, c)
    for wide in (4, 5, 6):
        assert not (outs[wide] == 0xFFFF).any()
        for kid in (0, 1):
            mism = outs[wide] != outs[kid]
            assert not mism.any(), f"{wide} vs {kid}: {mism.sum()} bit mismatches, first at {np.argwhere(mism)[0]}"
    check_parity(outs[4], R.fp8_gemm_nt(a, sfa, b, sfb, c), what="wide tiles 1000x1040x2048")


@pytest.mark.parametrize("kid,M,N,K,with_c", [(4, 4096, 2112, 7168, True), (4, 4096, 7168, 16384, True),
                                               (4, 4096, 4096, 7168, False), (4, 64, 7168, 2048, False),
                                               (4, 3072, 6144, 7168, True), (5, 4096, 7168, 2048, True),
                                               (5, 1000, 4096, 7168, False), (5, 4096, 2112, 7168, True),
                                               (6, 4096, 7168, 16384, True), (6, 4096, 7168, 2048, False),
                                               (6, 3000, 2112, 7168, True)])
def test_wide_tile_full_size_sampled(dg, monkeypatch, kid, M, N, K, with_c):
    """The 256 x 256 (4), 128 x 512 (5) and 256 x 224 (6) tiles, pinned, at full
    size (every output tile sampled as in the sweep test), with and without C;
    the fifth shape's plan splits only its partial last round (32 of 288 tiles,
    in 8 slices each)."""
    monkeypatch.setenv("DG_FORCE_KERNEL", str(kid))
    assert dg.dg_query_plan_form(0, M, N, K)["kernel_id"] == kid
    g = synth.gen_dense(M, N, K, seed=M + N + K + 7, with_c=with_c, backend="torch", device="cuda")
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(g["a"], g["sfa"], g["b"], g["sfb"], g["c"], d)
    torch.cuda.synchronize()
    db = bits(d)
    assert not (db == 0xFFFF).any()
    rng = np.random.default_rng(100 + M + N + K)
    rows, cols = stratified_entries(M, N, rng)
    a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    c = None if g["c"] is None else synth.to_numpy(g["c"])
    ref = entries_in_chunks(lambda r, q: R.fp8_gemm_nt_entries(a, sfa, b, sfb, c, r, q), rows, cols)
    check_parity(db[rows, cols], ref, what=f"kernel {kid} M={M} N={N} K={K} c={with_c}")
