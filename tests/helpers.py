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
