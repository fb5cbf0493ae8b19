"""The skinny-M kernel (all rows of A in one tile, B streamed into registers) on the GPU:
every compiled configuration, pinned with DG_FORCE_SKINNY, against the oracle -- random
inputs with C, ragged N and M, K not a multiple of the prefetch depth, whole tiles and
split K -- and bit for bit on exact-integer inputs."""

import numpy as np
import pytest
import torch

import fp4_gemm_dense_amd as dgm
import synth
from oracle import ref as R
from tests.helpers import bits, check_bit_exact, check_parity, sentinel_like
from tests.test_oracle import make_exact_case

pytestmark = pytest.mark.gpu

# id -> (block_m, block_n, prefetch): must match the library's table
CONFIGS = {0: (16, 128, 8), 1: (32, 128, 8), 2: (64, 128, 8), 3: (128, 128, 4), 4: (64, 64, 8),
           5: (128, 64, 4), 6: (64, 96, 8), 7: (128, 96, 4), 8: (64, 256, 6), 9: (32, 256, 6),
           10: (128, 112, 4), 11: (64, 112, 8), 12: (128, 224, 4)}


def _kblocks(bm, pf, splits):
    """A K length in blocks whose slices end mid-way through a prefetch group (padding
    blocks) after several chunks."""
    return (3 * pf + 5) * splits


def _dev(x):
    if x is None:
        return None
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        x = x.view(np.int16)
    return torch.from_numpy(x).cuda()


def _forced_plan(monkeypatch, sid, splits, M, N, K):
    monkeypatch.setenv("DG_FORCE_SKINNY", f"{sid},{splits}")
    p = dgm.dg_query_plan(M, N, K, 1, 0)
    assert p["kernel_id"] == 100 + sid, f"config {sid} not taken: {p}"
    assert p["block_m"] == CONFIGS[sid][0] and p["block_n"] == CONFIGS[sid][1]
    assert p["splits"] == splits, p
    return p


def _run(dg, a, sfa, b, sfb, c, M, N):
    d = sentinel_like((M, N))
    dg.dg_fp8_gemm_nt(_dev(a), _dev(sfa), _dev(b), _dev(sfb), _dev(c), d)
    torch.cuda.synchronize()
    return bits(d)


@pytest.mark.parametrize("sid", sorted(CONFIGS))
@pytest.mark.parametrize("splits", [1, 3])
def test_skinny_config_random_parity(dg, monkeypatch, sid, splits):
    bm, bn, pf = CONFIGS[sid]
    M = bm - 5 if bm > 16 else 11             # rows past M inside the tile
    if splits == 1:
        M += bm                               # a second row tile, partly filled
    N = 3 * bn + 48                           # a ragged last column tile
    K = 128 * _kblocks(bm, pf, splits)        # slices that end mid-way through a prefetch group
    _forced_plan(monkeypatch, sid, splits, M, N, K)
    g = synth.gen_dense(M, N, K, seed=1000 + 10 * sid + splits, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    d = _run(dg, a, sfa, b, sfb, c, M, N)
    assert not (d == 0xFFFF).any(), "every output element must be written"
    check_parity(d, R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"skinny {sid} splits {splits} {M}x{N}x{K}")


@pytest.mark.parametrize("sid", sorted(CONFIGS))
def test_skinny_config_exact_integer_bit_exact(dg, monkeypatch, sid):
    bm, bn, pf = CONFIGS[sid]
    M, N = bm, 2 * bn
    for splits, with_c in ((1, True), (2, False)):
        K = 128 * _kblocks(bm, pf, splits)
        _forced_plan(monkeypatch, sid, splits, M, N, K)
        rng = np.random.default_rng(77 + sid + splits)
        a, sfa, b, sfb, c, exact = make_exact_case(rng, M, N, K, with_c)
        d = _run(dg, a, sfa, b, sfb, c, M, N)
        check_bit_exact(d, exact, f"skinny {sid} exact, splits {splits}")


@pytest.mark.parametrize("M,N,K", [(1, 4096, 7168), (8, 2112, 1024), (33, 6144, 2048), (100, 1040, 128 * 9),
                                   (128, 7168, 512), (128, 2112, 7168), (192, 7168, 4096)])
def test_skinny_planner_choice_parity(dg, M, N, K):
    """Shapes the planner sends to the skinny kernel (its own choice of configuration and
    K slices), checked in full against the oracle."""
    p = dgm.dg_query_plan(M, N, K, 1, 0)
    assert p["kernel_id"] >= 100, p
    g = synth.gen_dense(M, N, K, seed=M + N + K, with_c=True)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    d = _run(dg, a, sfa, b, sfb, c, M, N)
    assert not (d == 0xFFFF).any()
    check_parity(d, R.fp8_gemm_nt(a, sfa, b, sfb, c), what=f"skinny plan {M}x{N}x{K} {p}")
