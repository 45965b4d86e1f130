"""Helpers for GPU parity tests: move synth bf16 bits to and from the device and
compare against the fp64 oracle with the tolerances the tests state."""

import numpy as np

import synth


def torch_mod():
    import torch
    return torch


def to_gpu(bits: np.ndarray, dev="cuda:0"):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(dev).view(torch.bfloat16)


def from_gpu(t) -> np.ndarray:
    """bf16 device tensor -> float64 numpy array (exact)."""
    torch = torch_mod()
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f64(bits)


def mask_to_gpu(bm, dev="cuda:0"):
    if bm is None:
        return None
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(bm, dtype=np.uint8)).to(dev)


def rel_err(got, ref) -> float:
    """max |got - ref| / max |ref| (ref all zero: plain max |got - ref|)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def lse_err(got, ref) -> float:
    """max |got - ref| over rows where ref is finite; rows where ref = -inf must be -inf."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    assert np.all(got[~fin] == -np.inf), "empty rows must have LSE = -inf"
    assert np.all(np.isfinite(got[fin])), "non-empty rows must have a finite LSE"
    return float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0


# Tolerances: O, dQ, dK, dV relative to max |ref|; LSE absolute.
TOL_REL = 1e-2
TOL_LSE = 1e-3
