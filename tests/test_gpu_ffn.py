"""Parity of the FP8xFP4 expert FFN (dg_fp8_fp4_expert_ffn) against the oracle on the GPU.

Tolerance and the handling of the requantised intermediate (a rounding decision
that legitimately differs at midpoints) are described in tests/ffn_check.py.
"""

import numpy as np
import pytest
import torch

import synth
from tests.ffn_check import check_ffn_output, kernel_intermediate, oracle_ffn
from tests.helpers import bits

pytestmark = pytest.mark.gpu


def _to_dev(g):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in g.items()}


def _run(dg, g, topk_w=None, offset=None, ws_extra=0):
    T, H = g["x"].shape
    E, I2 = g["w1"].shape[0], g["w1"].shape[1]
    k = g["topk_idx"].shape[1]
    nbytes = dg.dg_fp8_fp4_expert_ffn_workspace_bytes(T, k, E, H, I2 // 2)
    ws = torch.zeros(nbytes + ws_extra, dtype=torch.uint8, device="cuda")
    y = torch.full((T, H), -1, dtype=torch.int16, device="cuda")      # sentinel 0xFFFF
    (w1, w1_sf), (w2, w2_sf) = dg.transform_weights_for_expert_ffn((g["w1"], g["w1_sf"]), (g["w2"], g["w2_sf"]))
    dg.dg_fp8_fp4_expert_ffn(g["x"], g["x_sf"], g["topk_idx"], g["topk_w"] if topk_w is None else topk_w,
                             w1, w1_sf, w2, w2_sf, y,
                             g["expert_offset"] if offset is None else offset, ws)
    torch.cuda.synchronize()
    return bits(y), ws


@pytest.mark.parametrize("T,H,I,E,n_exp,topk,offset", [
    (64, 512, 256, 4, 16, 4, 0),
    (100, 1024, 384, 6, 12, 3, 6),
    (1, 512, 128, 1, 1, 1, 0),
    (300, 512, 512, 8, 8, 8, 0),      # every expert local: all T*k pairs computed
])
def test_ffn_small_parity(dg, T, H, I, E, n_exp, topk, offset):
    g = _to_dev(synth.gen_ffn(T=T, H=H, I=I, num_local=E, num_experts=n_exp, topk=topk,
                              seed=T + H + I, expert_offset=offset))
    y, ws = _run(dg, g)
    _, info = oracle_ffn(g)
    hit = check_ffn_output(g, y, kernel_intermediate(g, ws, info), f"ffn T{T} H{H} I{I}")
    assert np.all(y[~hit] == 0), "tokens without a local expert must be exactly zero"
    assert not np.any(y == 0xFFFF), "every row of y must be written"


@pytest.mark.parametrize("T,E,n_exp,topk,offset", [
    (40, 1, 64, 64, 0),     # every token picks every expert: one local pair each, a token spans a wave
    (48, 2, 32, 16, 5),     # 16 entries per token (four tokens per wave), one or two local pairs
    (64, 3, 24, 6, 2),      # 6 does not divide 64: local counts from re-reading the token's entries
])
def test_ffn_tokens_with_one_or_more_local_pairs(dg, T, E, n_exp, topk, offset):
    """A token with exactly one local pair has its row formed by linear2, the
    others go through the combine; both kinds must match the oracle (top-k counts
    whose tokens fill a whole wave, a quarter of one, or do not divide it)."""
    g = _to_dev(synth.gen_ffn(T=T, H=512, I=128, num_local=E, num_experts=n_exp, topk=topk,
                              seed=T * 3 + topk, expert_offset=offset))
    idx = synth.to_numpy(g["topk_idx"])
    nloc = ((idx >= offset) & (idx < offset + E)).sum(axis=1)
    assert (nloc == 1).any()
    y, ws = _run(dg, g)
    _, info = oracle_ffn(g)
    hit = check_ffn_output(g, y, kernel_intermediate(g, ws, info), f"ffn T{T} k{topk}")
    assert np.array_equal(hit, nloc > 0)
    assert np.all(y[nloc == 0] == 0), "tokens without a local expert must be exactly zero"
    assert not np.any(y == 0xFFFF), "every row of y must be written"


def test_ffn_weight_doubling_is_bit_exact(dg):
    g = _to_dev(synth.gen_ffn(T=80, H=512, I=256, num_local=4, num_experts=8, topk=4, seed=5))
    y1, _ = _run(dg, g)
    y2, _ = _run(dg, g, topk_w=(g["topk_w"] * 2).contiguous())
    v1 = torch.from_numpy(y1.view(np.int16)).view(torch.bfloat16).float()
    v2 = torch.from_numpy(y2.view(np.int16)).view(torch.bfloat16).float()
    assert torch.equal(v2, 2 * v1)


def test_ffn_no_local_expert_gives_zero(dg):
    g = _to_dev(synth.gen_ffn(T=50, H=512, I=128, num_local=4, num_experts=16, topk=2, seed=6))
    y, _ = _run(dg, g, offset=1000)
    assert np.all(y == 0)


def test_ffn_repeat_calls_are_deterministic(dg):
    g = _to_dev(synth.gen_ffn(T=120, H=1024, I=256, num_local=4, num_experts=8, topk=4, seed=7))
    y1, _ = _run(dg, g)
    y2, _ = _run(dg, g, ws_extra=4096)
    assert np.array_equal(y1, y2)


def test_ffn_full_size_sampled_tokens(dg):
    """4096 tokens, hidden 7168, intermediate 2048, 32 local experts of 256, top-8;
    generated on the device.  The oracle evaluates 24 tokens that hit local experts."""
    g = synth.gen_ffn(T=4096, H=7168, I=2048, num_local=32, num_experts=256, topk=8, seed=synth.seed_for(4, 0),
                      backend="torch", device="cuda")
    y, ws = _run(dg, g)
    idx = synth.to_numpy(g["topk_idx"])
    hit = (idx < 32).any(1)
    assert np.all(y[~hit] == 0)
    assert not np.any(y == 0xFFFF)
    rng = np.random.default_rng(4)
    toks = np.sort(rng.choice(np.nonzero(hit)[0], 24, replace=False))
    sub = {k: (g[k][toks] if k in ("x", "x_sf", "topk_idx", "topk_w") else g[k]) for k in g}
    # the kernel's codes for the sampled tokens' pairs, in the oracle's pair order
    full_info = {"pairs": []}
    idx_s = synth.to_numpy(sub["topk_idx"])
    for e in range(32):
        tok, slot = np.nonzero(idx_s == e)
        full_info["pairs"].append((toks[tok], slot))
    check_ffn_output(sub, y[toks], kernel_intermediate(g, ws, full_info), "ffn full size")
