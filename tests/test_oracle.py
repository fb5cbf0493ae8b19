"""Pins for the CPU oracle: every oracle function is checked against something
other than itself -- a library routine, an exact rational brute force, a closed
form, an exact power-of-two case or an invariant -- chosen so that a dropped
term, a wrong sign or index, or a transposed operand fails at least one test.
The ``test_planted_*`` tests plant such mistakes in copies of the oracle and
check that the pins catch them.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import ref as R


# ----------------------------------------------------------------------------
# decoders / encoders
# ----------------------------------------------------------------------------

def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = F.decode_e4m3(codes)
    assert np.array_equal(np.isnan(lib), np.isnan(mine))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], mine[ok])
    assert np.array_equal(np.signbit(lib[ok]), np.signbit(mine[ok]))


def test_e4m3_decoder_closed_form_values():
    assert F.decode_e4m3(0x38) == 1.0
    assert F.decode_e4m3(0x7E) == 448.0
    assert F.decode_e4m3(0xFE) == -448.0
    assert F.decode_e4m3(0x01) == 2.0 ** -9
    assert F.decode_e4m3(0x08) == 2.0 ** -6
    assert F.decode_e4m3(0x40) == 2.0
    assert F.decode_e4m3(0x3C) == 1.5
    assert np.isnan(F.decode_e4m3(0x7F)) and np.isnan(F.decode_e4m3(0xFF))
    # the only NaN codes are 0x7F and 0xFF
    assert np.isnan(F.E4M3_TABLE).sum() == 2


def test_e2m1_table_and_nibble_order():
    assert list(F.E2M1_TABLE[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(F.E2M1_TABLE[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]
    # byte 0x21: low nibble 1 (0.5) is element 0, high nibble 2 (1.0) is element 1
    v = F.unpack_e2m1(np.array([[0x21, 0xF7]], dtype=np.uint8))
    assert list(v[0]) == [0.5, 1.0, 6.0, -6.0]


def test_ue8m0_decode_and_packing():
    assert F.decode_ue8m0(127) == 1.0
    assert F.decode_ue8m0(128) == 2.0
    assert F.decode_ue8m0(120) == 2.0 ** -7
    assert F.decode_ue8m0(0) == 2.0 ** -127
    assert np.isnan(F.decode_ue8m0(255))
    # word 0x8180_7F7E holds bytes 0x7E, 0x7F, 0x80, 0x81 from the least significant end
    w = np.array([[np.int32(np.uint32(0x81807F7E).view(np.int32))]])
    s = F.unpack_ue8m0_int32(w)
    assert list(s[0]) == [0.5, 1.0, 2.0, 4.0]


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, 3.0e38]]).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mine = F.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(lib, mine)


def test_bf16_rounding_ties_to_even():
    one = 1.0
    assert F.round_to_bf16(one + 2.0 ** -8) == 1.0                    # tie, even is 1.0
    assert F.round_to_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6    # tie, even is 1+2^-6
    assert F.round_to_bf16(one + 2.0 ** -8 + 2.0 ** -40) == one + 2.0 ** -7
    assert np.isinf(F.round_to_bf16(3.4e38))


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    v = F.bf16_bits_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = np.isnan(v) == np.isnan(lib)
    assert same.all()
    ok = ~np.isnan(v)
    assert np.array_equal(v[ok], lib[ok])


def _midpoints():
    vals = F.E4M3_TABLE[:0x7F]
    return (vals[:-1] + vals[1:]) / 2


def test_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(50000) * 10.0 ** rng.uniform(-4, 2.7, 50000),
        _midpoints(), -_midpoints(), F.E4M3_TABLE[:0x7F], [500.0, -1000.0, 448.0, 464.0, 0.0],
    ]).astype(np.float32).astype(np.float64)
    clamped = np.clip(x, -448, 448).astype(np.float32)
    assert np.array_equal(clamped.astype(np.float64), np.clip(x, -448, 448)), "test values must be fp32-exact"
    lib = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = F.encode_e4m3_rne(x)
    # torch may keep -0.0 as 0x80; compare decoded values and sign
    assert np.array_equal(F.decode_e4m3(lib), F.decode_e4m3(mine))


def test_e4m3_encoder_ties_go_to_even_code():
    # 1.0 (0x38) and 1.125 (0x39): midpoint 1.0625 -> 0x38 (even)
    assert F.encode_e4m3_rne(1.0625) == 0x38
    # 1.125 (0x39) and 1.25 (0x3A): midpoint 1.1875 -> 0x3A (even)
    assert F.encode_e4m3_rne(1.1875) == 0x3A
    assert F.encode_e4m3_rne(1000.0) == 0x7E
    assert F.encode_e4m3_rne(-1000.0) == 0xFE
    assert F.encode_e4m3_rne(2.0 ** -10) == 0x00            # half of the smallest subnormal -> 0 (even)
    assert F.encode_e4m3_rne(3 * 2.0 ** -10) == 0x02        # 1.5 subnormal steps -> 2 (even)


def test_pow2_scale_exponent_closed_form():
    q = 448.0
    cases = {448.0: 0, 448.0 * (1 + 2 ** -20): 1, 224.0: -1, 224.0 * (1 + 2 ** -20): 0,
             1.0: -8, 0.875: -9, 896.0: 1, 3.0e4: 7}
    for amax, e in cases.items():
        assert F.pow2_scale_exponent(np.array([amax]), q)[0] == e, amax
    assert F.pow2_scale_exponent(np.array([0.0]), q)[0] == 0
    rng = np.random.default_rng(2)
    a = rng.uniform(0, 1, 10000) * 10.0 ** rng.uniform(-8, 8, 10000)
    e = F.pow2_scale_exponent(a, q)
    assert np.all(np.ldexp(q, e) >= a) and np.all(np.ldexp(q, e - 1) < a)
    e6 = F.pow2_scale_exponent(a, 6.0)
    assert np.all(np.ldexp(6.0, e6) >= a) and np.all(np.ldexp(6.0, e6 - 1) < a)


# ----------------------------------------------------------------------------
# dense GEMM
# ----------------------------------------------------------------------------

def _rand_inputs(rng, M, N, K, with_c=True):
    codes = np.arange(256, dtype=np.uint8)
    finite = codes[~np.isnan(F.E4M3_TABLE)]
    a = rng.choice(finite, size=(M, K))
    b = rng.choice(finite, size=(N, K))
    sfa = (rng.uniform(0.5, 2.0, (K // 128, M)) * 2.0 ** rng.integers(-6, 6, (K // 128, M))).astype(np.float32)
    sfb = (rng.uniform(0.5, 2.0, (-(-N // 128), K // 128)) * 2.0 ** rng.integers(-6, 6, (-(-N // 128), K // 128))).astype(np.float32)
    c = synth.to_numpy(synth.bf16_bits(torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32) * 100))) if with_c else None
    return a, sfa, b, sfb, c


def _brute_dense(a, sfa, b, sfb, c):
    """Exact rational triple loop: C + sum_kb sa*sb*sum_{k in kb} a*b."""
    M, K = a.shape
    N = b.shape[0]
    dec = [Fraction(v) if not np.isnan(v) else None for v in F.E4M3_TABLE]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for kb in range(K // 128):
                part = Fraction(0)
                for k in range(128 * kb, 128 * kb + 128):
                    part += dec[a[m, k]] * dec[b[n, k]]
                acc += Fraction(float(sfa[kb, m])) * Fraction(float(sfb[n // 128, kb])) * part
            if c is not None:
                acc += Fraction(float(F.bf16_bits_to_f64(c[m, n])))
            out[m, n] = float(acc)
    return out


@pytest.mark.parametrize("M,N,K", [(3, 5, 128), (4, 2, 256), (2, 3, 384), (1, 1, 128)])
def test_dense_matches_exact_rational_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    a, sfa, b, sfb, c = _rand_inputs(rng, M, N, K)
    exact = _brute_dense(a, sfa, b, sfb, c)
    got = R.fp8_gemm_nt(a, sfa, b, sfb, c)
    scale = np.abs(exact).max() + 1e-300
    assert np.max(np.abs(got - exact)) <= 1e-13 * scale


def test_dense_partial_b_block_brute_force():
    # N = 130 spans two 128-row scale blocks; the last block has 2 rows
    rng = np.random.default_rng(7)
    a, sfa, b, sfb, c = _rand_inputs(rng, 2, 130, 128, with_c=False)
    # evaluate only columns on both sides of the block edge against brute force
    cols = [0, 127, 128, 129]
    got = R.fp8_gemm_nt(a, sfa, b, sfb, None)[:, cols]
    dec = F.E4M3_TABLE
    for j, n in enumerate(cols):
        for m in range(2):
            want = sum(Fraction(dec[a[m, k]]) * Fraction(dec[b[n, k]]) for k in range(128))
            want *= Fraction(float(sfa[0, m])) * Fraction(float(sfb[n // 128, 0]))
            assert abs(got[m, j] - float(want)) <= 1e-13 * max(1.0, abs(float(want)))


def _int_code_table():
    """e4m3 codes whose values are the integers -8..8."""
    out = {}
    for code in range(256):
        v = F.E4M3_TABLE[code]
        if not np.isnan(v) and float(v).is_integer() and -8 <= v <= 8 and not (v == 0 and code != 0):
            out[int(v)] = code
    return out


def make_exact_case(rng, M, N, K, with_c=True):
    """Integer e4m3 values, power-of-two scales and integer C so that every partial
    sum is an integer multiple of a common power of two below 2**24: any fp32
    summation order is then exact and D must equal bf16(exact) bit for bit."""
    tab = _int_code_table()
    ints = rng.integers(-8, 9, (M, K))
    intb = rng.integers(-8, 9, (N, K))
    a = np.vectorize(tab.get)(ints).astype(np.uint8)
    b = np.vectorize(tab.get)(intb).astype(np.uint8)
    sfa = np.ldexp(1.0, rng.integers(-3, 1, (K // 128, M))).astype(np.float32)
    sfb = np.ldexp(1.0, rng.integers(-3, 1, (-(-N // 128), K // 128))).astype(np.float32)
    c = None
    if with_c:
        cv = rng.integers(-128, 129, (M, N)).astype(np.float32)
        c = synth.to_numpy(synth.bf16_bits(torch.from_numpy(cv)))
    exact = np.zeros((M, N))
    for kb in range(K // 128):
        sl = slice(128 * kb, 128 * kb + 128)
        part = ints[:, sl].astype(np.int64) @ intb[:, sl].astype(np.int64).T
        exact += part * sfa[kb][:, None].astype(np.float64) * sfb[np.arange(N) // 128, kb][None, :]
    if with_c:
        exact += F.bf16_bits_to_f64(c)
    return a, sfa, b, sfb, c, exact


def test_dense_exact_integer_case():
    rng = np.random.default_rng(11)
    a, sfa, b, sfb, c, exact = make_exact_case(rng, 9, 140, 384)
    got = R.fp8_gemm_nt(a, sfa, b, sfb, c)
    assert np.array_equal(got, exact)
    # bound that makes every fp32 partial sum exact: |sum| * 2**(6) < 2**24
    assert np.abs(exact).max() * 64 < 2 ** 24


def test_dense_all_ones():
    M, N, K = 5, 200, 512
    a = np.full((M, K), 0x38, np.uint8)
    b = np.full((N, K), 0x38, np.uint8)
    sfa = np.full((K // 128, M), 0.75, np.float32)
    sfb = np.full((2, K // 128), 3.0, np.float32)
    c = synth.to_numpy(synth.bf16_bits(torch.full((M, N), -5.0)))
    got = R.fp8_gemm_nt(a, sfa, b, sfb, c)
    assert np.all(got == K * 0.75 * 3.0 - 5.0)


def test_dense_identity_b_pins_orientation_and_scale_indexing():
    rng = np.random.default_rng(5)
    M, N, K = 6, 256, 256
    a, sfa, _, sfb, _ = _rand_inputs(rng, M, N, K, with_c=False)
    b = np.zeros((N, K), np.uint8)
    b[np.arange(N), np.arange(N)] = 0x38                  # B[n,k] = [k == n]
    got = R.fp8_gemm_nt(a, sfa, b, sfb)
    n = np.arange(N)
    want = F.decode_e4m3(a[:, n]) * sfa[n // 128, :].T * sfb[n // 128, n // 128][None, :]
    assert np.array_equal(got, want)


def test_dense_vs_library_matmul_of_library_dequant():
    """Textbook cross-check: torch decodes the codes, the test applies the scales
    with its own indexing, torch multiplies in fp64 (tight) and bf16 (loose)."""
    rng = np.random.default_rng(9)
    M, N, K = 40, 300, 640
    g = synth.gen_dense(M, N, K, seed=123)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    A = torch.from_numpy(a).view(torch.float8_e4m3fn).double()
    B = torch.from_numpy(b).view(torch.float8_e4m3fn).double()
    for kb in range(K // 128):
        A[:, 128 * kb:128 * kb + 128] *= torch.from_numpy(sfa[kb].astype(np.float64))[:, None]
        for nb in range(-(-N // 128)):
            B[128 * nb:128 * nb + 128, 128 * kb:128 * kb + 128] *= float(sfb[nb, kb])
    C = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).double()
    lib = (C + A @ B.T).numpy()
    got = R.fp8_gemm_nt(a, sfa, b, sfb, c)
    assert np.max(np.abs(got - lib)) <= 1e-12 * np.abs(lib).max()
    lib16 = (C.bfloat16().float() + (A.bfloat16() @ B.bfloat16().T).float()).double().numpy()
    assert np.linalg.norm(got - lib16) / np.linalg.norm(got) <= 1e-2
    del rng


def test_dense_entries_match_full():
    g = synth.gen_dense(50, 270, 384, seed=3)
    a, sfa, b, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    full = R.fp8_gemm_nt(a, sfa, b, sfb, c)
    rows = np.array([0, 49, 17, 3])
    cols = np.array([269, 0, 128, 127])
    got = R.fp8_gemm_nt_entries(a, sfa, b, sfb, c, rows, cols)
    assert np.allclose(got, full[rows, cols], rtol=1e-13, atol=1e-12)


# ----------------------------------------------------------------------------
# grouped forms
# ----------------------------------------------------------------------------

def test_contiguous_one_group_is_dense():
    g = synth.gen_contiguous(1, 300, 144, 256, seed=21)
    a, sfa, b, sfb, mi = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "m_indices"))
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    valid = mi >= 0
    assert written.sum() == 300 and np.array_equal(written, valid)
    dense = R.fp8_gemm_nt(a[valid], sfa[:, valid], b[0], sfb[0])
    assert np.array_equal(ref[valid], dense)
    assert np.isnan(ref[~valid]).all()


def test_contiguous_groups_use_their_own_b_and_padding_never_leaks():
    g = synth.gen_contiguous(4, 500, 160, 256, seed=22)
    a, sfa, b, sfb, mi = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "m_indices"))
    assert (mi == -1).any(), "padding rows must exist for this test"
    assert np.isnan(F.decode_e4m3(a[mi == -1])).all()
    ref, written = R.m_grouped_contiguous(a, sfa, b, sfb, mi)
    assert np.isfinite(ref[written]).all()
    for grp in range(4):
        rows = np.nonzero(mi == grp)[0]
        for r in rows[:3]:
            want = R.fp8_gemm_nt_entries(a, sfa, b[grp], sfb[grp], None, np.full(160, r), np.arange(160))
            assert np.allclose(ref[r], want, rtol=1e-13, atol=1e-10)
    # group boundaries: padded starts are multiples of 128
    starts = [int(np.nonzero(mi == grp)[0][0]) for grp in range(4) if (mi == grp).any()]
    assert all(s % 128 == 0 for s in starts)


def test_masked_full_groups_equal_dense_and_zero_groups_untouched():
    G, max_m, N, K = 3, 40, 144, 256
    g = synth.gen_masked(G, max_m, N, K, seed=31, masked_m=[40, 0, 17])
    a, sfa, b, sfb, mm = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "masked_m"))
    ref, written = R.m_grouped_masked(a, sfa, b, sfb, mm)
    assert np.array_equal(ref[0], R.fp8_gemm_nt(a[0], sfa[0], b[0], sfb[0]))
    assert not written[1].any() and np.isnan(ref[1]).all()
    assert written[2, :17].all() and not written[2, 17:].any()
    assert np.isfinite(ref[2, :17]).all()
    assert np.array_equal(ref[2, :17], R.fp8_gemm_nt(a[2, :17], sfa[2][:, :17], b[2], sfb[2]))


# ----------------------------------------------------------------------------
# FFN
# ----------------------------------------------------------------------------

def _small_ffn(seed=41, T=24, H=256, I=128, E=4, n_exp=16, topk=4, offset=0):
    return synth.gen_ffn(T=T, H=H, I=I, num_local=E, num_experts=n_exp, topk=topk, seed=seed,
                         expert_offset=offset)


def _np(g, *keys):
    return [synth.to_numpy(g[k]) for k in keys]


def _ffn_args(g):
    return _np(g, "x", "x_sf", "topk_idx", "topk_w", "w1", "w1_sf", "w2", "w2_sf")


def test_ffn_textbook_torch_reduction():
    """torch decodes e4m3 (library), the test applies scales with its own indexing and
    bit arithmetic, torch computes silu/matmul in fp32 and requantises with its e4m3 cast."""
    g = _small_ffn(T=40, H=512, I=256, E=6, n_exp=12, topk=3)
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _ffn_args(g)
    T, H = x.shape
    I = w1.shape[1] // 2

    def ue8m0(words, n):
        b = np.stack([(words.astype(np.int64) >> (8 * i)) & 0xFF for i in range(4)], -1)
        return np.exp2(b.reshape(words.shape[0], -1)[:, :n].astype(np.float64) - 127)

    def fp4(packed):
        mags = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], np.float64)
        nib = np.stack([packed & 15, packed >> 4], -1).reshape(packed.shape[0], -1)
        return np.where(nib & 8, -1.0, 1.0) * mags[nib & 7]

    X = torch.from_numpy(x).view(torch.float8_e4m3fn).double().numpy() * np.repeat(ue8m0(x_sf, H // 128), 128, 1)
    y = np.zeros((T, H))
    for e in range(6):
        W1 = fp4(w1[e]) * np.repeat(ue8m0(w1_sf[e], H // 32), 32, 1)
        W2 = fp4(w2[e]) * np.repeat(ue8m0(w2_sf[e], I // 32), 32, 1)
        for t, k in zip(*np.nonzero(idx == e)):
            u = torch.from_numpy(X[t] @ W1.T).float()
            s = torch.nn.functional.silu(u[:I]) * u[I:]
            sb = s.view(-1, 128)
            amax = sb.abs().amax(1).double()
            ex = torch.ceil(torch.log2(amax / 448.0))
            ex = ex + (448.0 * torch.exp2(ex) < amax).double() - (448.0 * torch.exp2(ex - 1) >= amax).double()
            q = (sb.double() / torch.exp2(ex)[:, None]).float().clamp(-448, 448).to(torch.float8_e4m3fn)
            deq = (q.double() * torch.exp2(ex)[:, None]).reshape(-1).numpy()
            y[t] += w[t, k] * (deq @ W2.T)
    got, _ = R.expert_ffn(x, x_sf, idx, w, w1, w1_sf, w2, w2_sf, 0, 6)
    err = np.abs(got - y)
    rms = np.sqrt(np.mean(y ** 2))
    assert np.all(err <= 2e-2 * np.maximum(np.abs(y), rms))
    assert np.linalg.norm(got - y) / np.linalg.norm(y) <= 8e-3
    # tokens with a hit are non-zero
    hit = np.isin(idx, np.arange(6)).any(1)
    assert np.all(np.abs(got[hit]).sum(1) > 0)


def test_ffn_single_pair_brute_force():
    """One token routed to one local expert: linear1 and linear2 evaluated with
    exact rationals, silu in float64, requant decided on float32 values."""
    g = _small_ffn(T=1, H=128, I=128, E=1, n_exp=1, topk=1)
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _ffn_args(g)
    got, info = R.expert_ffn(x, x_sf, idx, w, w1, w1_sf, w2, w2_sf, 0, 1, return_intermediate=True)
    mags = [0, .5, 1, 1.5, 2, 3, 4, 6]

    def fp4v(byte, hi):
        n = (int(byte) >> 4) if hi else (int(byte) & 15)
        return Fraction(mags[n & 7]) * (-1 if n & 8 else 1)

    def sc(words, j):
        return Fraction(2) ** (((int(np.uint32(words[j // 4].view(np.uint32))) >> (8 * (j % 4))) & 0xFF) - 127)

    xs = [Fraction(float(F.E4M3_TABLE[x[0, k]])) * sc(x_sf[0], k // 128) for k in range(128)]
    u = []
    for r in range(256):
        acc = Fraction(0)
        for k in range(128):
            acc += xs[k] * fp4v(w1[0, r, k // 2], k % 2) * sc(w1_sf[0, r], k // 32)
        u.append(acc)
    gate = np.array([np.float32(float(v)) for v in u[:128]], np.float64)
    up = np.array([np.float32(float(v)) for v in u[128:]], np.float64)
    s32 = (gate / (1 + np.exp(-gate)) * up).astype(np.float32)
    amax = float(np.abs(s32).max())
    e = 0
    while 448.0 * 2.0 ** e < amax:
        e += 1
    while 448.0 * 2.0 ** (e - 1) >= amax:
        e -= 1
    codes = F.encode_e4m3_rne(np.ldexp(s32.astype(np.float64), -e))
    assert np.array_equal(codes, info["codes"][0][0])
    q = [Fraction(float(F.E4M3_TABLE[cd])) * Fraction(2) ** e for cd in codes]
    wt = Fraction(float(w[0, 0]))
    for h in range(0, 128, 9):
        acc = Fraction(0)
        for k in range(128):
            acc += q[k] * fp4v(w2[0, h, k // 2], k % 2) * sc(w2_sf[0, h], k // 32)
        assert abs(got[0, h] - float(wt * acc)) <= 1e-13 * max(1.0, abs(float(wt * acc)))


def test_ffn_no_local_hit_gives_exact_zero_and_weights_scale_exactly():
    g = _small_ffn(T=30, E=3, n_exp=16, topk=2, seed=43)
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _ffn_args(g)
    y, _ = R.expert_ffn(x, x_sf, idx, w, w1, w1_sf, w2, w2_sf, 0, 3)
    miss = ~np.isin(idx, np.arange(3)).any(1)
    assert miss.any() and (~miss).any()
    assert np.all(y[miss] == 0.0)
    y2, _ = R.expert_ffn(x, x_sf, idx, 2 * w, w1, w1_sf, w2, w2_sf, 0, 3)
    assert np.array_equal(y2, 2 * y)
    # expert_offset: the same experts addressed with shifted ids give the same result
    y3, _ = R.expert_ffn(x, x_sf, idx + 5, w, w1, w1_sf, w2, w2_sf, 5, 3)
    assert np.array_equal(y3, y)


def test_ffn_slot_permutation_invariance():
    g = _small_ffn(T=20, E=4, n_exp=8, topk=4, seed=44)
    x, x_sf, idx, w, w1, w1_sf, w2, w2_sf = _ffn_args(g)
    y, _ = R.expert_ffn(x, x_sf, idx, w, w1, w1_sf, w2, w2_sf, 0, 4)
    perm = np.array([2, 0, 3, 1])
    yp, _ = R.expert_ffn(x, x_sf, idx[:, perm], w[:, perm], w1, w1_sf, w2, w2_sf, 0, 4)
    assert np.allclose(y, yp, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_ffn_requant_codes_and_range():
    rng = np.random.default_rng(45)
    s = (rng.standard_normal((5, 256)) * 37).astype(np.float32)
    s[3] = 0.0
    codes, e = R.requant_e4m3_pow2(s)
    assert np.all(e[3] == 0) and np.all(codes[3] == 0)
    deq = F.decode_e4m3(codes) * np.repeat(np.ldexp(1.0, e), 128, axis=1)
    blk = np.abs(s.reshape(5, 2, 128)).max(-1)
    # the block amax maps into (224, 448]
    top = blk[:3] / np.ldexp(1.0, e[:3])
    assert np.all((top > 224) & (top <= 448))
    # dequantised values are within half an e4m3 ulp (relative 2**-4) of the inputs
    assert np.all(np.abs(deq - s) <= np.maximum(np.abs(s) * 2.0 ** -4, 2.0 ** -9 * np.repeat(np.ldexp(1.0, e), 128, 1)))


# ----------------------------------------------------------------------------
# planted mistakes: the pins above must fail for plausible oracle bugs
# ----------------------------------------------------------------------------

def _pins_dense(fn):
    """Run the dense pins against ``fn``; return True when all pass."""
    rng = np.random.default_rng(77)
    try:
        a, sfa, b, sfb, c, exact = make_exact_case(rng, 5, 136, 256)
        if not np.array_equal(fn(a, sfa, b, sfb, c), exact):
            return False
        M, N, K = 4, 256, 256
        a, sfa, _, sfb, _ = _rand_inputs(rng, M, N, K, with_c=False)
        b = np.zeros((N, K), np.uint8)
        b[np.arange(N), np.arange(N)] = 0x38
        n = np.arange(N)
        want = F.decode_e4m3(a[:, n]) * sfa[n // 128, :].T * sfb[n // 128, n // 128][None, :]
        return np.array_equal(fn(a, sfa, b, sfb), want)
    except Exception:
        return False


# ----------------------------------------------------------------------------
# FP8 x FP4 M-grouped GEMM
# ----------------------------------------------------------------------------

_FP4_MAGS = [0, .5, 1, 1.5, 2, 3, 4, 6]


def _fp4_frac(byte, hi):
    n = (int(byte) >> 4) if hi else (int(byte) & 15)
    return Fraction(_FP4_MAGS[n & 7]) * (-1 if n & 8 else 1)


def _ue8m0_frac(words, j):
    return Fraction(2) ** (((int(np.uint32(words[j // 4].view(np.uint32))) >> (8 * (j % 4))) & 0xFF) - 127)


@pytest.mark.parametrize("M,N,K", [(3, 5, 128), (2, 3, 384), (4, 2, 640)])
def test_fp8_fp4_gemm_matches_exact_rational_brute_force(M, N, K):
    """Every entry as an exact rational: e4m3 through torch's float8 cast, E2M1 from
    its closed-form magnitudes, UE8M0 as powers of two; 640 = 1.25 scale words."""
    g = synth.gen_fp4_contiguous(1, M, N, K, seed=M * 100 + N + K, align=1, counts=[M])
    a, a_sf, b, b_sf = (synth.to_numpy(g[k]) for k in ("a", "a_sf", "b", "b_sf"))
    got = R.fp8_fp4_gemm_nt(a, a_sf, b[0], b_sf[0])
    av = torch.from_numpy(a.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(av[m, k])) * _ue8m0_frac(a_sf[m], k // 128) *
                        _fp4_frac(b[0, n, k // 2], k % 2) * _ue8m0_frac(b_sf[0, n], k // 32))
            assert got[m, n] == float(acc), (m, n, got[m, n], float(acc))


def test_fp8_fp4_gemm_scale_exponents_shift_exactly():
    """Raising every B exponent byte by one doubles D exactly; raising the A
    exponent of one 1x128 block changes only that block's contribution."""
    g = synth.gen_fp4_contiguous(1, 6, 16, 512, seed=7, align=1, counts=[6])
    a, a_sf, b, b_sf = (synth.to_numpy(g[k]) for k in ("a", "a_sf", "b", "b_sf"))
    base = R.fp8_fp4_gemm_nt(a, a_sf, b[0], b_sf[0])
    bsf2 = (b_sf[0].view(np.uint32) + np.uint32(0x01010101)).view(np.int32)
    assert np.array_equal(R.fp8_fp4_gemm_nt(a, a_sf, b[0], bsf2), 2 * base)
    # A block 2 of every row: one more in byte 2 of word 0
    asf2 = (a_sf.view(np.uint32) + np.uint32(0x00010000) * np.array([1, 0], np.uint32)).view(np.int32)
    part = R.fp8_fp4_gemm_nt(a[:, 256:384], a_sf[:, :1] * 0 + np.int32(0x7F7F7F7F), b[0][:, 128:192],
                             b_sf[0][:, 2:3])
    scale2 = np.ldexp(1.0, ((a_sf[:, 0].view(np.uint32) >> 16) & 0xFF).astype(np.int64) - 127)
    want = base + part * scale2[:, None]
    assert np.allclose(R.fp8_fp4_gemm_nt(a, asf2, b[0], b_sf[0]), want, rtol=0, atol=1e-12 * np.abs(want).max())


def test_fp8_fp4_contiguous_groups_padding_and_relabelling():
    """Each row uses its own group's B; padding rows (-1) are not written; relabelling
    the groups together with B leaves the result unchanged."""
    g = synth.gen_fp4_contiguous(3, 300, 32, 256, seed=3, counts=[100, 0, 200])
    a, a_sf, b, b_sf, mi = (synth.to_numpy(g[k]) for k in ("a", "a_sf", "b", "b_sf", "m_indices"))
    ref, written = R.m_grouped_fp8_fp4_contiguous(a, a_sf, b, b_sf, mi)
    assert written.sum() == 300 and np.all(np.isnan(ref[~written])) and np.all(np.isfinite(ref[written]))
    for r in (0, 99, 100, 128, 327, 383):
        if mi[r] >= 0:
            assert np.array_equal(ref[r], R.fp8_fp4_gemm_nt(a[r:r + 1], a_sf[r:r + 1], b[mi[r]], b_sf[mi[r]])[0])
    perm = np.array([2, 0, 1])                       # new label of old group g: perm[g]
    mi2 = np.where(mi >= 0, perm[np.maximum(mi, 0)], -1).astype(np.int32)
    b2, bsf2 = np.empty_like(b), np.empty_like(b_sf)
    b2[perm], bsf2[perm] = b, b_sf
    ref2, written2 = R.m_grouped_fp8_fp4_contiguous(a, a_sf, b2, bsf2, mi2)
    assert np.array_equal(written, written2) and np.array_equal(ref[written], ref2[written2])


def test_fp8_fp4_masked_equals_contiguous_of_the_same_rows():
    """Masked groups hold the same rows as a contiguous layout of the valid rows;
    rows at or past masked_m (and counts outside [0, max_m]) are not written."""
    mm = [130, 0, 7]
    g = synth.gen_fp4_masked(3, 130, 48, 384, seed=9, masked_m=mm)
    a, a_sf, b, b_sf = (synth.to_numpy(g[k]) for k in ("a", "a_sf", "b", "b_sf"))
    ref, written = R.m_grouped_fp8_fp4_masked(a, a_sf, b, b_sf, mm)
    assert written.sum() == 137
    rows = np.concatenate([a[gi, :m] for gi, m in enumerate(mm)])
    rsf = np.concatenate([a_sf[gi, :m] for gi, m in enumerate(mm)])
    mi = np.concatenate([np.full(m, gi, np.int32) for gi, m in enumerate(mm)])
    cref, _ = R.m_grouped_fp8_fp4_contiguous(rows, rsf, b, b_sf, mi)
    assert np.array_equal(ref[written], cref)
    ref_c, written_c = R.m_grouped_fp8_fp4_masked(a, a_sf, b, b_sf, [500, -3, 7])
    assert np.array_equal(written_c[0], np.ones(130, bool)) and not written_c[1].any()


def test_fp4_weight_sf_k_major_fixture_and_labelled_words():
    """The scale relayout on a hand-written case, and on words that carry their own
    (group, row, K block) label, so a swapped index or group shows as a wrong label."""
    sf = np.array([[[1, 2, 3], [4, 5, 6]]], np.int32)                   # G 1, rows 2, K blocks 3
    assert R.fp4_weight_sf_k_major(sf).tolist() == [[[1, 4], [2, 5], [3, 6]]]
    G, Rr, KB = 3, 70, 5
    g_, r_, k_ = np.meshgrid(np.arange(G), np.arange(Rr), np.arange(KB), indexing="ij")
    lab = ((g_ << 20) | (r_ << 8) | k_).astype(np.int32)
    out = R.fp4_weight_sf_k_major(lab)
    assert out.shape == (G, KB, Rr)
    for g in range(G):
        for kb in range(KB):
            for r in range(Rr):
                w = int(out[g, kb, r])
                assert (w >> 20, (w >> 8) & 0xFFF, w & 0xFF) == (g, r, kb)


# ----------------------------------------------------------------------------
# NN layout (B stored [K, N])
# ----------------------------------------------------------------------------

def test_nn_exact_rational_brute_force():
    """Codes decoded by torch's float8 cast, B indexed as [k][n], scales per (row, K block)
    and (128-column block, K block); N = 130 spans a partial B block."""
    rng = np.random.default_rng(17)
    M, N, K = 2, 130, 256
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    b_kn = rng.integers(0, 256, (K, N), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38
    b_kn[(b_kn & 0x7F) == 0x7F] = 0x40
    sfa = rng.uniform(0.5, 2.0, (K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.5, 2.0, (2, K // 128)).astype(np.float32)
    got = R.fp8_gemm_nn(a, sfa, b_kn, sfb)
    av, bv = _torch_e4m3(a), _torch_e4m3(b_kn)
    for m, n in [(0, 0), (1, 127), (0, 128), (1, 129), (0, 77)]:
        want = sum(Fraction(float(av[m, k])) * Fraction(float(bv[k, n])) * Fraction(float(sfa[k // 128, m])) *
                   Fraction(float(sfb[n // 128, k // 128])) for k in range(K))
        assert abs(got[m, n] - float(want)) <= 1e-13 * max(1.0, abs(float(want)))


@pytest.mark.parametrize("b_kn", [True, False])
def test_tn_tt_exact_rational_brute_force(b_kn):
    """A stored [k][m]; B stored [k][n] (TN) or [n][k] (TT); decoding and indexing here."""
    rng = np.random.default_rng(23 + b_kn)
    M, N, K = 3, 130, 256
    a_km = rng.integers(0, 256, (K, M), dtype=np.uint8)
    b = rng.integers(0, 256, (K, N) if b_kn else (N, K), dtype=np.uint8)
    a_km[(a_km & 0x7F) == 0x7F] = 0x38
    b[(b & 0x7F) == 0x7F] = 0x40
    sfa = rng.uniform(0.5, 2.0, (K // 128, M)).astype(np.float32)
    sfb = rng.uniform(0.5, 2.0, (2, K // 128)).astype(np.float32)
    got = (R.fp8_gemm_tn if b_kn else R.fp8_gemm_tt)(a_km, sfa, b, sfb)
    av, bv = _torch_e4m3(a_km), _torch_e4m3(b)
    for m, n in [(0, 0), (1, 127), (2, 128), (0, 129), (2, 64)]:
        want = sum(Fraction(float(av[k, m])) * Fraction(float(bv[k, n] if b_kn else bv[n, k])) *
                   Fraction(float(sfa[k // 128, m])) * Fraction(float(sfb[n // 128, k // 128])) for k in range(K))
        assert abs(got[m, n] - float(want)) <= 1e-13 * max(1.0, abs(float(want)))


def test_k_grouped_tn_brute_force_and_empty_group():
    """Each group's output is its own K rows only (exact rationals on sampled entries), an
    empty group gives exact zeros, and the groups' sum is the TN GEMM over all rows."""
    g = synth.gen_kgrouped_tn(3, 300, 32, 144, seed=4, counts=[100, 0, 200])
    a, sfa, b, sfb = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb"))
    ks = synth.to_numpy(g["ks"]).tolist()
    assert ks == [128, 0, 256]
    out = R.k_grouped_tn_contiguous(a, sfa, b, sfb, ks)
    assert np.all(out[1] == 0)
    av, bv = _torch_e4m3(a), _torch_e4m3(b)
    for grp, (k0, k1) in ((0, (0, 128)), (2, (128, 384))):
        for m, n in [(0, 0), (31, 129), (7, 64)]:
            want = sum(Fraction(float(av[k, m])) * Fraction(float(bv[k, n])) * Fraction(float(sfa[k // 128, m])) *
                       Fraction(float(sfb[n // 128, k // 128])) for k in range(k0, k1))
            assert abs(out[grp, m, n] - float(want)) <= 1e-13 * max(1.0, abs(float(want)))
    whole = R.fp8_gemm_tn(a, sfa, b, sfb)
    assert np.allclose(out.sum(0), whole, rtol=1e-12, atol=1e-12 * np.abs(whole).max())


def test_nn_equals_nt_of_the_transposed_operand_and_grouped_forms():
    g = synth.gen_dense_nn(5, 144, 384, seed=8)
    a, sfa, b_kn, sfb, c = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "c"))
    x, y = R.fp8_gemm_nn(a, sfa, b_kn, sfb, c), R.fp8_gemm_nt(a, sfa, b_kn.T.copy(), sfb, c)
    assert np.allclose(x, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())   # float64 sums in another order
    gc = synth.gen_contiguous_nn(3, 200, 48, 256, seed=9, counts=[60, 0, 140])
    a, sfa, b_kn, sfb, mi = (synth.to_numpy(gc[k]) for k in ("a", "sfa", "b", "sfb", "m_indices"))
    ref, written = R.m_grouped_nn_contiguous(a, sfa, b_kn, sfb, mi)
    ref_t, written_t = R.m_grouped_contiguous(a, sfa, np.ascontiguousarray(np.swapaxes(b_kn, 1, 2)), sfb, mi)
    assert np.array_equal(written, written_t)
    assert np.allclose(ref[written], ref_t[written], rtol=1e-12, atol=1e-12 * np.abs(ref_t[written]).max())


# ----------------------------------------------------------------------------
# packed UE8M0 scale factors
# ----------------------------------------------------------------------------

def _torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _pack_bytes(e):
    """exponent bytes [..., S] -> int32 words [..., ceil(S/4)], written out byte by byte."""
    e = np.asarray(e, np.int64)
    S = e.shape[-1]
    W = (S + 3) // 4
    out = np.zeros(e.shape[:-1] + (W,), np.int64)
    for j in range(S):
        out[..., j // 4] |= e[..., j] << (8 * (j % 4))
    return out.astype(np.uint32).view(np.int32)


def test_ue8m0_dense_exact_rational_brute_force():
    """Random codes and per-(row, K block) / per-(128-row block, K block) exponents,
    K = 640 (five K blocks: the second word is partly padding), N = 130 (two B blocks);
    sampled entries against exact rationals with decoding done here independently."""
    rng = np.random.default_rng(11)
    M, N, K = 3, 130, 640
    KB = K // 128
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x38                 # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0x40
    ea = rng.integers(118, 136, (M, KB))
    eb = rng.integers(118, 136, ((N + 127) // 128, KB))
    c = synth.to_numpy(synth.bf16_bits(torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32))))
    got = R.fp8_gemm_nt_ue8m0(a, _pack_bytes(ea), b, _pack_bytes(eb), c)
    av, bv = _torch_e4m3(a), _torch_e4m3(b)
    cv = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).double().numpy()
    for m, n in [(0, 0), (1, 127), (2, 128), (0, 129), (1, 64), (2, 5)]:
        want = Fraction(float(cv[m, n]))
        for k in range(K):
            kb = k // 128
            want += (Fraction(float(av[m, k])) * Fraction(float(bv[n, k])) *
                     Fraction(2) ** int(ea[m, kb] - 127) * Fraction(2) ** int(eb[n // 128, kb] - 127))
        assert abs(got[m, n] - float(want)) <= 1e-13 * max(1.0, abs(float(want)))


def test_ue8m0_byte_order_and_block_indexing_closed_form():
    """All-ones operands, A exponents 127 + i + r (K block i, row r), B exponents
    127 + 3 - i (+1 for the second 128-row block): D[r, n] = 128 * 4 * 2**(3 + r) (doubled
    for n >= 128).  Reversed byte order, a transposed exponent table or a wrong B
    block gives a different value."""
    M, N, K = 3, 256, 512
    a = np.full((M, K), 0x38, np.uint8)          # 1.0
    b = np.full((N, K), 0x38, np.uint8)
    ea = np.array([[127 + i + r for i in range(4)] for r in range(M)])
    eb = np.array([[127 + 3 - i + blk for i in range(4)] for blk in range(2)])
    got = R.fp8_gemm_nt_ue8m0(a, _pack_bytes(ea), b, _pack_bytes(eb))
    for r in range(M):
        assert np.all(got[r, :128] == 128 * 4 * 2.0 ** (3 + r))
        assert np.all(got[r, 128:] == 2 * 128 * 4 * 2.0 ** (3 + r))


def test_ue8m0_grouped_forms_agree_with_dense():
    """Contiguous (padding rows skipped) and masked forms equal the dense form on each
    group's rows."""
    g = synth.gen_contiguous_ue8m0(3, 300, 48, 384, seed=5, counts=[100, 0, 200])
    a, sfa, b, sfb, mi = (synth.to_numpy(g[k]) for k in ("a", "sfa", "b", "sfb", "m_indices"))
    ref, written = R.m_grouped_contiguous_ue8m0(a, sfa, b, sfb, mi)
    assert written.sum() == 300 and np.all(mi[written] >= 0)
    for grp in (0, 2):
        rows = np.nonzero(mi == grp)[0]
        assert np.array_equal(ref[rows], R.fp8_gemm_nt_ue8m0(a[rows], sfa[rows], b[grp], sfb[grp]))
    mm = [7, 0, 64]
    gm = synth.gen_masked_ue8m0(3, 64, 48, 384, seed=6, masked_m=mm)
    a, sfa, b, sfb = (synth.to_numpy(gm[k]) for k in ("a", "sfa", "b", "sfb"))
    ref, written = R.m_grouped_masked_ue8m0(a, sfa, b, sfb, mm)
    assert written.sum() == 71
    for grp in (0, 2):
        assert np.array_equal(ref[grp, :mm[grp]],
                              R.fp8_gemm_nt_ue8m0(a[grp, :mm[grp]], sfa[grp, :mm[grp]], b[grp], sfb[grp]))


def test_ue8m0_generator_scales_are_powers_of_two_within_range():
    """The generator's block exponents put every block's amax in (224, 448] (a check of
    the input recipe, not of the oracle)."""
    g = synth.gen_dense_ue8m0(5, 200, 640, seed=3, with_c=False)
    a, sfa, b = synth.to_numpy(g["a"]), synth.to_numpy(g["sfa"]), synth.to_numpy(g["b"])
    av = np.abs(_torch_e4m3(a)).reshape(5, 5, 128).max(axis=-1)
    assert np.all(av <= 448) and np.all(av > 200)
    assert synth.to_numpy(g["sfb"]).shape == (2, 2)


def test_planted_mistakes_fail_dense_pins():
    assert _pins_dense(R.fp8_gemm_nt)

    def no_c(a, sfa, b, sfb, c=None):
        return R.dequant_a(a, sfa) @ R.dequant_b(b, sfb).T

    def sfb_transposed(a, sfa, b, sfb, c=None):
        # reads sfb as if it were stored [K/128][ceil(N/128)]
        s = np.asarray(sfb)
        return R.fp8_gemm_nt(a, sfa, b, s.reshape(s.shape[1], s.shape[0]).T, c)

    def sfa_row_major_misread(a, sfa, b, sfb, c=None):
        # reads sfa as if it were stored [M][K/128]
        s = np.asarray(sfa)
        return R.fp8_gemm_nt(a, s.reshape(s.shape[1], s.shape[0]).T, b, sfb, c)

    def b_not_transposed(a, sfa, b, sfb, c=None):
        # treats B's memory as K x N (an NN product) instead of N x K
        B = np.asarray(b)
        Bd = R.dequant_b(B, sfb)
        out = R.dequant_a(a, sfa) @ Bd.reshape(B.shape[1], B.shape[0])
        return out + (F.bf16_bits_to_f64(c) if c is not None else 0)

    def sign_flip_negative_codes(a, sfa, b, sfb, c=None):
        aa = np.asarray(a) & 0x7F
        return R.fp8_gemm_nt(aa, sfa, b, sfb, c)

    for bad in (no_c, sfb_transposed, sfa_row_major_misread, b_not_transposed, sign_flip_negative_codes):
        assert not _pins_dense(bad), bad.__name__
