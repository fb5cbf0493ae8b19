"""Comparison helpers for the GPU parity tests (test infrastructure)."""

import numpy as np
import torch

from oracle.formats import bf16_bits_to_f64, f64_to_bf16_bits

SENTINEL = 0xFFFF            # bf16 NaN pattern pre-filled into outputs


def bits(t: torch.Tensor) -> np.ndarray:
    """Device bf16 / int16 tensor -> numpy uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def sentinel_like(shape, device="cuda"):
    return torch.full(shape, -1, dtype=torch.int16, device=device)   # 0xFFFF


def check_parity(d_bits, ref, elem_tol=8e-3, fro_tol=3e-3, what=""):
    """Per element |D - ref| <= elem_tol * max(|ref|, rms(ref)) and
    ||D - ref||_F / ||ref||_F <= fro_tol, over the given (written) elements."""
    d = bf16_bits_to_f64(d_bits).ravel()
    r = np.asarray(ref, dtype=np.float64).ravel()
    assert d.shape == r.shape
    assert np.isfinite(d).all(), f"{what}: non-finite outputs ({np.count_nonzero(~np.isfinite(d))})"
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(d - r)
    bound = elem_tol * np.maximum(np.abs(r), rms)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {r.size} elements out of tolerance; worst "
                           f"err {err.max():.4g} at ref {r[np.argmax(err - bound)]:.4g} (rms {rms:.4g})")
    nrm = np.linalg.norm(r)
    if nrm > 0:
        fro = np.linalg.norm(d - r) / nrm
        assert fro <= fro_tol, f"{what}: Frobenius relative error {fro:.3g} > {fro_tol}"
    return float(err.max()) if r.size else 0.0


def check_bit_exact(d_bits, exact, what=""):
    want = f64_to_bf16_bits(exact)
    mism = d_bits != want
    assert not mism.any(), f"{what}: {mism.sum()} bit mismatches, first at {np.argwhere(mism)[0]}"


def stratified_entries(M, N, rng, valid_rows=None, block=64):
    """(rows, cols) of output entries to check at full size: in every block x block block
    of an M x N output, one element at a random place and the element at the block's
    last (valid) row and last column.  Every tile the library may use is a multiple of 64
    rows and columns, so every output tile -- and every split-K tile -- gets checked,
    its last row and last column included.  valid_rows (bool [M]) restricts the rows to
    the written ones; blocks without a valid row are skipped."""
    nbc = (N + block - 1) // block
    c0 = np.arange(nbc) * block
    c1 = np.minimum(c0 + block, N)
    rows, cols = [], []
    for r0 in range(0, M, block):
        r1 = min(r0 + block, M)
        vr = np.arange(r0, r1) if valid_rows is None else np.nonzero(valid_rows[r0:r1])[0] + r0
        if vr.size == 0:
            continue
        rows.append(rng.choice(vr, nbc))
        cols.append(c0 + (rng.random(nbc) * (c1 - c0)).astype(np.int64))
        rows.append(np.full(nbc, vr[-1]))
        cols.append(c1 - 1)
    return np.concatenate(rows), np.concatenate(cols)


def stratified_lines(n, rng, valid=None, block=64):
    """Indices along one output axis: per block of 64, one random (valid) index and the
    last (valid) one.  The cross product of such row and column sets meets every 64 x 64
    block at a random place and at its last row and column."""
    out = []
    for r0 in range(0, n, block):
        r1 = min(r0 + block, n)
        v = np.arange(r0, r1) if valid is None else np.nonzero(valid[r0:r1])[0] + r0
        if v.size:
            out += sorted({int(rng.choice(v)), int(v[-1])})
    return np.asarray(out, dtype=np.int64)


def entries_in_chunks(fn, rows, cols, chunk=2048):
    """fn(rows, cols) -> values, evaluated over chunks of the entry list (bounds the
    oracle's memory at full size)."""
    return np.concatenate([fn(rows[i:i + chunk], cols[i:i + chunk]) for i in range(0, len(rows), chunk)])
