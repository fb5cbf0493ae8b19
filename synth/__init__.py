"""Seeded synthetic inputs for the fine-grained-scaled FP8 / FP8xFP4 GEMM workloads.

This module is shared by the tests, the benchmark and the oracle checks.  It
draws random numbers and quantises them into the input formats the library
consumes; it holds none of the GEMM arithmetic (no products, no accumulation,
no requantisation of intermediates).  Quantisation of *inputs* uses torch's
e4m3fn cast (with an explicit clamp, since that cast does not saturate) and a
small E2M1 encoder of its own.

Two backends draw the same distributions:
* ``backend="numpy"`` -- numpy PCG64 ``default_rng(seed)``; draw order A, B, C,
  then metadata, except that the group row counts (which fix A's shape) are
  drawn first.  This is the recipe the parity tests use.
* ``backend="torch"`` with ``device="cuda"`` -- torch's device generator seeded
  with the same seed; used for full-size benchmark inputs, where drawing a GB
  of normals on the host would dominate the run.  The values differ from the
  numpy stream but have the same distribution and quantisation.

Workload recipes (sizes as the workloads state them):
* dense: A [M,K], B [N,K] ~ N(0,1) fp32, A quantised per 1x128 and B per
  128x128 block to e4m3 with fp32 scale amax/448; C = bf16(N(0,1)) or none.
* contiguous: 8 groups, row counts multinomial(32768, 1/8 each), each group
  padded to a multiple of 128; padding rows hold e4m3 NaN (0x7F), NaN scales
  and group index -1.
* masked: 32 groups x 256 rows, masked_m ~ U{0..256}; rows >= masked_m hold
  e4m3 NaN and NaN scales.
* FFN: 4096 bf16 N(0,1) tokens -> e4m3 with a power-of-two (UE8M0) scale per
  1x128; router logits N(0,1) over 256 experts, top-8 by logit (ties to the
  lower id), weights = softmax over the 8 chosen logits; W1 [E, 2I, H] and
  W2 [E, H, I] ~ N(0,1) -> E2M1 with a power-of-two scale per 1x32 (amax/6
  rounded up to a power of two); UE8M0 bytes packed four per int32,
  little-endian; FP4 nibbles packed low nibble first.
"""

import math

import numpy as np
import torch

E4M3_NAN = 0x7F
BF16_SENTINEL = 0xFFFF          # a bf16 NaN pattern used to pre-fill outputs

DENSE_NK = [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168), (7168, 2048)]
DENSE_M = [64, 4096]
GROUPED_NK = [(4096, 7168), (7168, 2048)]


def seed_for(config: int, shape_index: int) -> int:
    return 1000 * config + shape_index


# ----------------------------------------------------------------------------
# drawing
# ----------------------------------------------------------------------------

class _Draw:
    def __init__(self, seed, backend="numpy", device="cpu"):
        self.backend = backend
        self.device = torch.device(device)
        if backend == "numpy":
            self.rng = np.random.default_rng(seed)
        elif backend == "torch":
            self.gen = torch.Generator(device=self.device)
            self.gen.manual_seed(seed)
        else:
            raise ValueError(backend)

    def normal(self, *shape) -> torch.Tensor:
        if self.backend == "numpy":
            return torch.from_numpy(self.rng.standard_normal(shape, dtype=np.float32)).to(self.device)
        return torch.randn(*shape, generator=self.gen, device=self.device, dtype=torch.float32)

    def multinomial_counts(self, total, groups):
        if self.backend == "numpy":
            return [int(v) for v in self.rng.multinomial(total, [1.0 / groups] * groups)]
        draws = torch.randint(0, groups, (total,), generator=self.gen, device=self.device)
        return [int(v) for v in torch.bincount(draws, minlength=groups).cpu()]

    def integers(self, lo, hi_inclusive, n):
        if self.backend == "numpy":
            return [int(v) for v in self.rng.integers(lo, hi_inclusive + 1, n)]
        v = torch.randint(lo, hi_inclusive + 1, (n,), generator=self.gen, device=self.device)
        return [int(t) for t in v.cpu()]


# ----------------------------------------------------------------------------
# input quantisation (input preparation only)
# ----------------------------------------------------------------------------

def e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    """float32 -> e4m3fn codes (uint8), RNE via torch's cast, saturated at +-448."""
    return x.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def quant_rows_1x128(x: torch.Tensor):
    """[M, K] float32 -> (codes uint8 [M, K], scales float32 [K/128, M]); scale = amax/448."""
    M, K = x.shape
    xb = x.view(M, K // 128, 128)
    amax = xb.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = e4m3_codes(xb / s[..., None]).view(M, K)
    return q, s.t().contiguous()


def quant_blocks_128x128(w: torch.Tensor):
    """[N, K] float32 -> (codes uint8 [N, K], scales float32 [ceil(N/128), K/128]).

    The amax of the last (partial) row block is taken over its valid rows.
    """
    N, K = w.shape
    nb = (N + 127) // 128
    wp = torch.zeros(nb * 128, K, dtype=w.dtype, device=w.device)
    wp[:N] = w
    amax = wp.view(nb, 128, K // 128, 128).abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    s_full = s.repeat_interleave(128, 0)[:N].repeat_interleave(128, 1)
    return e4m3_codes(w / s_full), s.contiguous()


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    """float32 -> bf16 bit patterns (uint16 stored as int16 view)."""
    return x.to(torch.bfloat16).view(torch.int16)


def _pow2_exponent(amax: torch.Tensor, qmax: float) -> torch.Tensor:
    """Smallest integer e with qmax * 2**e >= amax (0 where amax == 0)."""
    pos = amax > 0
    safe = torch.where(pos, amax, torch.ones_like(amax)).double()
    e = torch.ceil(torch.log2(safe / qmax))
    e = e + (qmax * torch.exp2(e) < safe).double()
    e = e - (qmax * torch.exp2(e - 1) >= safe).double()
    return torch.where(pos, e, torch.zeros_like(e)).to(torch.int32)


def pack_ue8m0(exps: torch.Tensor) -> torch.Tensor:
    """int exponents [..., S] (S % 4 == 0) -> int32 [..., S/4]; byte i of word j is scale 4j+i."""
    b = (exps + 127).to(torch.int64)
    b = b.view(*b.shape[:-1], b.shape[-1] // 4, 4)
    w = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16) | (b[..., 3] << 24)
    w = torch.where(w >= 2**31, w - 2**32, w)
    return w.to(torch.int32)


def quant_rows_pow2_1x128(x: torch.Tensor):
    """[T, H] float32 -> (e4m3 codes [T, H], packed UE8M0 int32 [T, H/512]); scale 2**ceil(log2(amax/448))."""
    T, H = x.shape
    xb = x.view(T, H // 128, 128)
    e = _pow2_exponent(xb.abs().amax(dim=-1), 448.0)               # [T, H/128]
    q = e4m3_codes(xb * torch.exp2(-e.float())[..., None]).view(T, H)
    nb = H // 128
    pad = (-nb) % 4
    if pad:
        e = torch.cat([e, torch.zeros(T, pad, dtype=e.dtype, device=e.device)], dim=1)
    return q, pack_ue8m0(e)


def _pack_exponent_rows(e: torch.Tensor) -> torch.Tensor:
    """int exponents [..., S] -> packed UE8M0 int32 [..., ceil(S/4)] (zero exponents pad the last word)."""
    pad = (-e.shape[-1]) % 4
    if pad:
        e = torch.cat([e, torch.zeros(*e.shape[:-1], pad, dtype=e.dtype, device=e.device)], dim=-1)
    return pack_ue8m0(e)


def quant_blocks_pow2_128x128(w: torch.Tensor):
    """[N, K] float32 -> (e4m3 codes [N, K], packed UE8M0 int32 [ceil(N/128), ceil(K/512)]);
    one power-of-two scale 2**ceil(log2(amax/448)) per 128x128 block (amax over the valid rows)."""
    N, K = w.shape
    nb = (N + 127) // 128
    wp = torch.zeros(nb * 128, K, dtype=w.dtype, device=w.device)
    wp[:N] = w
    e = _pow2_exponent(wp.view(nb, 128, K // 128, 128).abs().amax(dim=(1, 3)), 448.0)   # [nb, K/128]
    e_full = e.repeat_interleave(128, 0)[:N].repeat_interleave(128, 1)
    return e4m3_codes(w * torch.exp2(-e_full.float())), _pack_exponent_rows(e)


_E2M1_MAGS = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_codes(x: torch.Tensor) -> torch.Tensor:
    """float32 (already scaled, |x| <= 6 after clamp) -> 4-bit codes (uint8), nearest, ties to even code."""
    mags = _E2M1_MAGS.to(x.device)
    a = x.abs().clamp(max=6.0)
    hi = torch.bucketize(a, mags).clamp(max=7)                       # first mag >= a
    lo = (hi - 1).clamp(min=0)
    d_hi = mags[hi] - a
    d_lo = a - mags[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = torch.where(pick_hi, hi, lo).to(torch.uint8)
    return torch.where(torch.signbit(x), code | 8, code)


def quant_fp4_1x32(w: torch.Tensor):
    """[R, C] float32 -> (packed E2M1 bytes [R, C/2], packed UE8M0 int32 [R, C/128]); scale 2**ceil(log2(amax/6))."""
    R, C = w.shape
    wb = w.view(R, C // 32, 32)
    e = _pow2_exponent(wb.abs().amax(dim=-1), 6.0)                  # [R, C/32]
    codes = e2m1_codes(wb * torch.exp2(-e.float())[..., None]).view(R, C)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).to(torch.uint8)
    return packed, pack_ue8m0(e)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

def gen_dense(M, N, K, seed, with_c=True, backend="numpy", device="cpu"):
    """Dense NT GEMM inputs.  Returns dict of tensors on ``device``."""
    d = _Draw(seed, backend, device)
    a, sfa = quant_rows_1x128(d.normal(M, K))
    b, sfb = quant_blocks_128x128(d.normal(N, K))
    c = bf16_bits(d.normal(M, N)) if with_c else None
    return dict(a=a, sfa=sfa, b=b, sfb=sfb, c=c, M=M, N=N, K=K)


def gen_dense_nn(M, N, K, seed, with_c=True, backend="numpy", device="cpu"):
    """gen_dense's inputs with B stored [K, N] (the NN layout; same values and scales)."""
    g = gen_dense(M, N, K, seed, with_c=with_c, backend=backend, device=device)
    g["b"] = g["b"].t().contiguous()
    return g


def gen_dense_tn(M, N, K, seed, with_c=True, b_kn=True, backend="numpy", device="cpu"):
    """gen_dense's inputs with A stored [K, M] and B stored [K, N] (TN; b_kn=False: [N, K], TT)."""
    g = gen_dense(M, N, K, seed, with_c=with_c, backend=backend, device=device)
    g["a"] = g["a"].t().contiguous()
    if b_kn:
        g["b"] = g["b"].t().contiguous()
    return g


def gen_kgrouped_tn(G, total_rows, M, N, seed, align=128, counts=None, backend="numpy", device="cpu"):
    """K-grouped TN inputs: per-group token counts (multinomial unless given), each padded to
    `align` rows of K; A [K, M] and B [K, N] hold N(0,1) values quantised per 1x128 along K
    (A, per output row) and per 128x128 block (B); padding rows hold zeros."""
    d = _Draw(seed, backend, device)
    if counts is None:
        counts = d.multinomial_counts(total_rows, G)
    ks = [((c + align - 1) // align) * align for c in counts]
    K = sum(ks)
    pad = torch.ones(K, dtype=torch.bool, device=device)
    k0 = 0
    for c, kg in zip(counts, ks):
        pad[k0:k0 + c] = False
        k0 += kg
    a_mk, sfa = quant_rows_1x128(torch.where(pad, 0.0, d.normal(M, K)))
    b_nk, sfb = quant_blocks_128x128(torch.where(pad, 0.0, d.normal(N, K)))
    return dict(a=a_mk.t().contiguous(), sfa=sfa, b=b_nk.t().contiguous(), sfb=sfb,
                ks=torch.tensor(ks, dtype=torch.int32, device=device), counts=counts, K=K, M=M, N=N, G=G)


def gen_contiguous_nn(G, total_rows, N, K, seed, align=128, counts=None, backend="numpy", device="cpu"):
    """gen_contiguous's inputs with each group's B stored [K, N]."""
    g = gen_contiguous(G, total_rows, N, K, seed, align=align, counts=counts, backend=backend, device=device)
    g["b"] = g["b"].transpose(1, 2).contiguous()
    return g


def padded_group_layout(counts, align=128):
    """Row counts -> (m_indices list, group start offsets) for the contiguous layout."""
    m_idx = []
    starts = []
    for g, cnt in enumerate(counts):
        starts.append(len(m_idx))
        padded = ((cnt + align - 1) // align) * align
        m_idx += [g] * cnt + [-1] * (padded - cnt)
    return m_idx, starts


def gen_contiguous(G, total_rows, N, K, seed, align=128, counts=None, backend="numpy", device="cpu"):
    d = _Draw(seed, backend, device)
    if counts is None:
        counts = d.multinomial_counts(total_rows, G)
    m_idx, _ = padded_group_layout(counts, align)
    M = len(m_idx)
    m_indices = torch.tensor(m_idx, dtype=torch.int32, device=device)
    a, sfa = quant_rows_1x128(d.normal(M, K)) if M > 0 else (
        torch.zeros(0, K, dtype=torch.uint8, device=device), torch.zeros(K // 128, 0, device=device))
    pad_rows = m_indices < 0
    a[pad_rows] = E4M3_NAN
    sfa[:, pad_rows] = float("nan")
    bs, sbs = zip(*[quant_blocks_128x128(d.normal(N, K)) for _ in range(G)])
    return dict(a=a, sfa=sfa, b=torch.stack(bs), sfb=torch.stack(sbs), m_indices=m_indices,
                counts=counts, M=M, N=N, K=K, G=G)


def gen_fp4_contiguous(G, total_rows, N, K, seed, align=128, counts=None, backend="numpy", device="cpu"):
    """Contiguous-layout FP8 x FP4 grouped GEMM inputs: A e4m3 with UE8M0 1x128 scales
    (packed 4 per int32), B E2M1 with UE8M0 1x32 scales per group."""
    d = _Draw(seed, backend, device)
    if counts is None:
        counts = d.multinomial_counts(total_rows, G)
    m_idx, _ = padded_group_layout(counts, align)
    M = len(m_idx)
    m_indices = torch.tensor(m_idx, dtype=torch.int32, device=device)
    a, a_sf = quant_rows_pow2_1x128(d.normal(M, K))
    pad_rows = m_indices < 0
    a[pad_rows] = E4M3_NAN
    a_sf[pad_rows] = -1                      # exponent bytes 0xFF: NaN scales
    bs, sbs = zip(*[quant_fp4_1x32(d.normal(N, K)) for _ in range(G)])
    return dict(a=a, a_sf=a_sf, b=torch.stack(bs), b_sf=torch.stack(sbs), m_indices=m_indices,
                counts=counts, M=M, N=N, K=K, G=G)


def gen_fp4_masked(G, max_m, N, K, seed, masked_m=None, backend="numpy", device="cpu"):
    """Masked-layout FP8 x FP4 grouped GEMM inputs; rows past masked_m hold NaN codes."""
    d = _Draw(seed, backend, device)
    as_, sas = zip(*[quant_rows_pow2_1x128(d.normal(max_m, K)) for _ in range(G)])
    a = torch.stack(as_)
    a_sf = torch.stack(sas)                                         # [G, max_m, ceil(K/512)]
    bs, sbs = zip(*[quant_fp4_1x32(d.normal(N, K)) for _ in range(G)])
    if masked_m is None:
        masked_m = d.integers(0, max_m, G)
    for g, mg in enumerate(masked_m):
        a[g, max(mg, 0):] = E4M3_NAN
        a_sf[g, max(mg, 0):] = -1
    return dict(a=a, a_sf=a_sf, b=torch.stack(bs), b_sf=torch.stack(sbs),
                masked_m=torch.tensor(masked_m, dtype=torch.int32, device=device),
                G=G, max_m=max_m, N=N, K=K)


def gen_masked(G, max_m, N, K, seed, masked_m=None, backend="numpy", device="cpu"):
    d = _Draw(seed, backend, device)
    as_, sas = zip(*[quant_rows_1x128(d.normal(max_m, K)) for _ in range(G)])
    a = torch.stack(as_)
    sfa = torch.stack(sas)                                          # [G, K/128, max_m]
    bs, sbs = zip(*[quant_blocks_128x128(d.normal(N, K)) for _ in range(G)])
    if masked_m is None:
        masked_m = d.integers(0, max_m, G)
    for g, mg in enumerate(masked_m):
        a[g, mg:] = E4M3_NAN
        sfa[g, :, mg:] = float("nan")
    return dict(a=a, sfa=sfa, b=torch.stack(bs), sfb=torch.stack(sbs),
                masked_m=torch.tensor(masked_m, dtype=torch.int32, device=device),
                G=G, max_m=max_m, N=N, K=K)


def gen_dense_ue8m0(M, N, K, seed, with_c=True, backend="numpy", device="cpu"):
    """Dense NT GEMM inputs with packed UE8M0 scales: A per 1x128 (power-of-two scale),
    B per 128x128 block, C bf16."""
    d = _Draw(seed, backend, device)
    a, sfa = quant_rows_pow2_1x128(d.normal(M, K))
    b, sfb = quant_blocks_pow2_128x128(d.normal(N, K))
    c = bf16_bits(d.normal(M, N)) if with_c else None
    return dict(a=a, sfa=sfa, b=b, sfb=sfb, c=c, M=M, N=N, K=K)


def gen_contiguous_ue8m0(G, total_rows, N, K, seed, align=128, counts=None, backend="numpy", device="cpu"):
    """Contiguous-layout grouped inputs with packed UE8M0 scales; padding rows hold NaN codes and
    exponent bytes 0xFF."""
    d = _Draw(seed, backend, device)
    if counts is None:
        counts = d.multinomial_counts(total_rows, G)
    m_idx, _ = padded_group_layout(counts, align)
    M = len(m_idx)
    m_indices = torch.tensor(m_idx, dtype=torch.int32, device=device)
    a, sfa = quant_rows_pow2_1x128(d.normal(M, K))
    pad_rows = m_indices < 0
    a[pad_rows] = E4M3_NAN
    sfa[pad_rows] = -1
    bs, sbs = zip(*[quant_blocks_pow2_128x128(d.normal(N, K)) for _ in range(G)])
    return dict(a=a, sfa=sfa, b=torch.stack(bs), sfb=torch.stack(sbs), m_indices=m_indices,
                counts=counts, M=M, N=N, K=K, G=G)


def gen_masked_ue8m0(G, max_m, N, K, seed, masked_m=None, backend="numpy", device="cpu"):
    """Masked-layout grouped inputs with packed UE8M0 scales; rows past masked_m are garbage."""
    d = _Draw(seed, backend, device)
    as_, sas = zip(*[quant_rows_pow2_1x128(d.normal(max_m, K)) for _ in range(G)])
    a = torch.stack(as_)
    sfa = torch.stack(sas)                                          # [G, max_m, ceil(K/512)]
    bs, sbs = zip(*[quant_blocks_pow2_128x128(d.normal(N, K)) for _ in range(G)])
    if masked_m is None:
        masked_m = d.integers(0, max_m, G)
    for g, mg in enumerate(masked_m):
        a[g, max(mg, 0):] = E4M3_NAN
        sfa[g, max(mg, 0):] = -1
    return dict(a=a, sfa=sfa, b=torch.stack(bs), sfb=torch.stack(sbs),
                masked_m=torch.tensor(masked_m, dtype=torch.int32, device=device),
                G=G, max_m=max_m, N=N, K=K)


def route_topk(logits: torch.Tensor, k: int):
    """Top-k experts by descending logit (ties: lower id first); weights = softmax of the k chosen logits."""
    T, E = logits.shape
    # stable sort on -logit keeps the lower id first among equal logits
    order = torch.sort(-logits, dim=1, stable=True).indices[:, :k]
    chosen = torch.gather(logits, 1, order)
    w = torch.softmax(chosen, dim=1)
    return order.to(torch.int32), w.to(torch.float32)


def gen_ffn(T=4096, H=7168, I=2048, num_local=32, num_experts=256, topk=8, seed=4000,
            expert_offset=0, backend="numpy", device="cpu"):
    d = _Draw(seed, backend, device)
    xf = d.normal(T, H).to(torch.bfloat16).float()
    x, x_sf = quant_rows_pow2_1x128(xf)
    logits = d.normal(T, num_experts)
    topk_idx, topk_w = route_topk(logits, topk)
    w1s, w1sf, w2s, w2sf = [], [], [], []
    for _ in range(num_local):
        p, s = quant_fp4_1x32(d.normal(2 * I, H))
        w1s.append(p)
        w1sf.append(s)
    for _ in range(num_local):
        p, s = quant_fp4_1x32(d.normal(H, I))
        w2s.append(p)
        w2sf.append(s)
    return dict(x=x, x_sf=x_sf, topk_idx=topk_idx, topk_w=topk_w,
                w1=torch.stack(w1s), w1_sf=torch.stack(w1sf),
                w2=torch.stack(w2s), w2_sf=torch.stack(w2sf),
                T=T, H=H, I=I, E=num_local, topk=topk, expert_offset=expert_offset)


def to_numpy(t):
    """Tensor (any device) -> numpy array with the unsigned view for byte/bf16 data."""
    if t is None:
        return None
    t = t.detach().cpu()
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.numpy()


def ceil_div(a, b):
    return -(-a // b)


def n_blocks(n):
    return math.ceil(n / 128)
