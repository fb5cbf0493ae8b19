"""Checks of the FP8xFP4 expert FFN output against the oracle (test infrastructure,
shared by tests/test_gpu_ffn.py and the smoke test).

Tolerance for this path: per element |y - ref| <= 2e-2 * max(|ref|, rms(ref)),
Frobenius relative error <= 8e-3.

The requantised intermediate is a rounding decision taken in fp32 on both sides.
The kernel's linear1 runs on gfx950's matrix cores, which reduce products in
groups of 8 and keep 13 bits below each group's leading bit; the oracle rounds an
exact float64 sum to fp32.  Where a value lies within that accumulation error of
an e4m3 rounding midpoint, either code is a correct result (measured: about one
element in 6000).  One flipped code near the top of a block moves every output of
its token by up to one e4m3 step (1/14 of the block maximum) times one weight, which
at intermediate size 256 reaches several percent of rms(y).  So the intermediate is
not unique and neither is y; following "compare what is unique, check that the
rest is valid":
  1. every differing code must be a rounding of a value within the accumulation
     error bound of the oracle's exact value (and >= 99.9 % of codes agree; every
     block's scale exponent agrees);
  2. tokens whose intermediate codes all equal the oracle's: y within the
     tolerance of the plain oracle, element by element;
  3. tokens with a differing code: y within the tolerance of linear2 + the
     weighted sum evaluated in float64 on the kernel's codes (computed here with
     the oracle's decoders);
  4. all tokens with a local hit: Frobenius bound against the plain oracle.
"""

import numpy as np

import synth
from oracle import ref as R
from tests.helpers import check_parity

ELEM_TOL, FRO_TOL = 2e-2, 8e-3


def oracle_ffn(g, offset=None, topk_w=None):
    n = {k: synth.to_numpy(g[k]) for k in ("x", "x_sf", "topk_idx", "topk_w", "w1", "w1_sf", "w2", "w2_sf")}
    if topk_w is not None:
        n["topk_w"] = topk_w
    return R.expert_ffn(n["x"], n["x_sf"], n["topk_idx"], n["topk_w"], n["w1"], n["w1_sf"], n["w2"], n["w2_sf"],
                        g["expert_offset"] if offset is None else offset, g["E"], return_intermediate=True)


def kernel_intermediate(g, ws, info):
    """The kernel's requantised intermediate (codes, exponents) per local expert, in
    the oracle's pair order, read from the workspace (regions in the order the
    library documents: counts, starts, pair tokens, pair index, codes, exponents)."""
    T, k = g["topk_idx"].shape
    E, I = g["E"], g["I"]
    P = T * k
    sq_stride = ((I // 128) + 3) & ~3

    def a256(v):
        return (v + 255) & ~255
    off = a256(a256(0 + E * 4) + (E + 1) * 4)
    off = a256(off + P * 4)                  # pair tokens
    pair_of_off = off
    off = a256(off + P * 4)
    q_off = off
    sq_off = a256(off + P * I)
    w = ws.cpu().numpy()
    pair_of = w[pair_of_off:pair_of_off + P * 4].view(np.int32).reshape(T, k)
    q = w[q_off:q_off + P * I].reshape(P, I)
    sq = w[sq_off:sq_off + P * sq_stride].reshape(P, sq_stride)
    out = {}
    for e in range(E):
        tok, slot = info["pairs"][e]
        pr = pair_of[tok, slot]
        out[e] = (q[pr], sq[pr, : I // 128].astype(np.int64) - 127)
    return out


def _value_rank():
    """Sorted distinct finite e4m3 values, and each code's rank among them (+0 and -0 share one)."""
    from oracle.formats import E4M3_TABLE
    vals = np.where(np.isnan(E4M3_TABLE), np.inf, E4M3_TABLE)
    distinct = np.unique(vals[np.isfinite(vals)])
    return distinct, np.searchsorted(distinct, vals).astype(np.int64)


_DISTINCT, _RANK = _value_rank()


def _mfma_error_bound(h, w):
    """Bound on |matrix-core dot product - exact| for rows of h . w (elementwise pairs).

    The gfx950 F8F6F4 matrix instructions reduce products in groups of 8
    consecutive K positions aligned to the group's largest product and keep 13
    bits below its leading bit (measured on MI355X: 2^4 + 2^-9 in one group is
    exact, 2^5 + 2^-9 drops the small term; groups are k = 8j .. 8j+7).  Each
    product can therefore lose less than 2^(e_max - 13) with e_max the exponent
    of its group's largest |product|; fp32 accumulation of the group sums adds
    a tree-sum term.
    """
    t = np.abs(h * w)                                     # [n, K]
    n, K = t.shape
    gmax = t.reshape(n, K // 8, 8).max(axis=2)
    _, ex = np.frexp(np.where(gmax > 0, gmax, 1.0))       # gmax < 2^ex
    per_group = np.where(gmax > 0, 8 * np.ldexp(1.0, ex - 1 - 13), 0.0)
    return per_group.sum(axis=1) + (np.ceil(np.log2(K)) + 4) * 2.0 ** -24 * t.sum(axis=1)


def check_codes(kern, info, g):
    """Codes agree with the oracle's except for neighbours at a rounding midpoint;
    returns the tokens (sorted, unique) that have at least one differing code.

    A differing code is accepted only when the oracle's value lies within the
    matrix-core accumulation error of linear1 (see _mfma_error_bound) from the
    midpoint between the two codes, propagated through silu(gate) * up, in the
    block's scaled units.
    """
    n_same = n_all = 0
    flipped = []
    x_deq = None
    n = {k: synth.to_numpy(g[k]) for k in ("x", "x_sf", "w1", "w1_sf")}
    I = g["I"]
    for e, (codes, ex) in kern.items():
        if codes.shape[0] == 0:
            continue
        want, wex = info["codes"][e], info["exps"][e]
        assert np.array_equal(ex, wex), f"expert {e}: requant scale exponents differ"
        same = _RANK[codes] == _RANK[want]                # +0 and -0 are the same value
        n_same += same.sum()
        n_all += same.size
        if same.all():
            continue
        r, c = np.nonzero(~same)
        flipped.append(info["pairs"][e][0][r])
        if x_deq is None:
            x_deq = R.dequant_x_ue8m0(n["x"], n["x_sf"])
        tok = info["pairs"][e][0][r]
        W1 = R.dequant_w_fp4(n["w1"][e], n["w1_sf"][e])
        h = x_deq[tok]
        gate = np.einsum("ik,ik->i", h, W1[c])
        up = np.einsum("ik,ik->i", h, W1[I + c])
        d_gate = _mfma_error_bound(h, W1[c])
        d_up = _mfma_error_bound(h, W1[I + c])
        sig = 1.0 / (1.0 + np.exp(-gate))
        silu = gate * sig
        dsilu = sig * (1.0 + gate * (1.0 - sig))
        s = silu * up
        d_s = np.abs(dsilu * up) * d_gate + np.abs(silu) * d_up + 2.0 ** -21 * np.abs(s)
        scale = np.ldexp(1.0, wex[r, c // 128])
        x = s / scale
        delta = d_s / scale
        # the kernel's code must round some value in [x - delta, x + delta]:
        # its rounding interval (midpoints to its value neighbours) must meet it
        rk = _RANK[codes[r, c]]
        lo = np.where(rk > 0, (_DISTINCT[np.maximum(rk - 1, 0)] + _DISTINCT[rk]) / 2, -np.inf)
        hi = np.where(rk < _DISTINCT.size - 1,
                      (_DISTINCT[np.minimum(rk + 1, _DISTINCT.size - 1)] + _DISTINCT[rk]) / 2, np.inf)
        assert np.all((x + delta >= lo) & (x - delta <= hi)), \
            f"expert {e}: a differing code is not a rounding of any value within the accumulation error bound"
    assert n_same >= 0.999 * n_all, f"only {n_same / n_all:.5f} of intermediate codes agree"
    return np.unique(np.concatenate(flipped)) if flipped else np.zeros(0, np.int64)


def linear2_combine_on_codes(g, kern, info):
    """y in float64 from given intermediate codes: per local expert, (codes x 2^exponent)
    . W2_e^T, weighted by topk_w and summed per token (the oracle's decoders and
    dequantisers; no rounding before the sum)."""
    n = {k: synth.to_numpy(g[k]) for k in ("x", "topk_w", "w2", "w2_sf")}
    T, H = n["x"].shape
    y = np.zeros((T, H))
    for e, (codes, ex) in kern.items():
        tok, slot = info["pairs"][e]
        if tok.size == 0:
            continue
        q = R.decode_e4m3(codes) * np.repeat(np.ldexp(1.0, ex), 128, axis=1)
        o = q @ R.dequant_w_fp4(n["w2"][e], n["w2_sf"][e]).T
        np.add.at(y, tok, n["topk_w"][tok, slot][:, None] * o)
    return y


def check_ffn_output(g, y, kern, what):
    """Steps 1-4 of the module docstring for output bits y [T, H] and the kernel's
    intermediate `kern` (kernel_intermediate).  Returns the bool mask of tokens with
    a local hit."""
    ref, info = oracle_ffn(g)
    idx = synth.to_numpy(g["topk_idx"])
    off, E = g["expert_offset"], g["E"]
    hit = ((idx >= off) & (idx < off + E)).any(1)
    flipped_tok = check_codes(kern, info, g)
    flipped = np.zeros(hit.shape, bool)
    flipped[flipped_tok] = True
    unique = hit & ~flipped
    if hit.any():
        check_parity(y[hit], ref[hit], np.inf, FRO_TOL, what=what + " (plain oracle, Frobenius)")
    if unique.any():
        check_parity(y[unique], ref[unique], ELEM_TOL, np.inf,
                     what=what + " (plain oracle, tokens with the oracle's intermediate)")
    if flipped.any():
        ref_k = linear2_combine_on_codes(g, kern, info)
        check_parity(y[flipped], ref_k[flipped], ELEM_TOL, FRO_TOL,
                     what=what + " (tokens with a differing intermediate code, on the kernel's codes)")
    return hit
