"""Seeded synthetic inputs for exact attention, shared by the oracle and the GPU path.

This module holds no attention arithmetic.  It only draws random numbers, rounds them
to bfloat16 bit patterns, and builds the boolean block masks that describe which key
blocks a query block may see.  Both sides of every parity check (the fp64 oracle and
the HIP library) receive exactly the bits produced here.

Workloads follow the shapes the pages measure on:
  * the FlashAttention-NeurIPS22 digest, "实验与结果" (attention micro-benchmark on
    B=64, H=16, N=1024, d=64);
  * GPT-style causal training shapes and 16K long context (FlashAttention-2 wiki,
    "性能与效率"; digest "实验与结果", Path-X 16K);
  * the fixed butterfly block-sparsity pattern (digest, "核心方法", Block-sparse 扩展).

Recipe (identical on both sides): numpy ``Generator(PCG64(seed))``; draw
``standard_normal(dtype=float32)`` for Q, K, V, dO in that order, each of shape
(B, H, N, d); round each float32 to bfloat16 with round-to-nearest-even on the bit
pattern; optionally multiply Q and K by an exact power of two.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "bf16_round_bits",
    "bf16_bits_to_f32",
    "bf16_bits_to_f64",
    "butterfly_blockmask",
    "make_blockmask",
    "draw_inputs",
    "draw_inputs_nqk",
    "e4m3_round_codes",
    "draw_inputs_fp8",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    ``mask`` is "dense", "causal" or "butterfly" (block size ``mask_block``).
    ``qk_mult`` multiplies Q and K after bf16 rounding (a power of two, so exact).
    ``backward`` says whether the workload includes the gradient pass.
    """

    name: str
    B: int
    H: int
    N: int
    d: int
    mask: str = "dense"
    mask_block: int = 128
    qk_mult: float = 1.0
    backward: bool = True
    seed: int = 0

    @property
    def causal(self) -> bool:
        return self.mask == "causal"

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(d), as the fp32 value handed to the library."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    def blockmask(self) -> np.ndarray | None:
        if self.mask != "butterfly":
            return None
        return butterfly_blockmask(-(-self.N // self.mask_block))

    def shape(self) -> tuple[int, int, int, int]:
        return (self.B, self.H, self.N, self.d)


CONFIGS: dict[str, Config] = {
    "C1": Config("C1", 1, 2, 128, 64, "dense", backward=False, seed=1001),
    "C2": Config("C2", 64, 16, 1024, 64, "dense", seed=1002),
    "C3": Config("C3", 8, 16, 2048, 128, "causal", seed=1003),
    "C4": Config("C4", 1, 16, 16384, 128, "causal", qk_mult=0.5, seed=1004),
    "C5": Config("C5", 4, 16, 4096, 64, "butterfly", mask_block=128, seed=1005),
}


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest, ties to even.

    Inputs are finite (normal draws); NaN/Inf handling is not needed here.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def _mul_pow2_bits(bits: np.ndarray, mult: float) -> np.ndarray:
    if mult == 1.0:
        return bits
    m, e = math.frexp(mult)
    if m != 0.5:
        raise ValueError("qk_mult must be a power of two so the product stays exact")
    out = bf16_round_bits(bf16_bits_to_f32(bits) * np.float32(mult))
    # exactness check: a power-of-two multiple of a bf16 value is a bf16 value
    assert np.array_equal(bf16_bits_to_f32(out), bf16_bits_to_f32(bits) * np.float32(mult))
    return out


def butterfly_blockmask(nb: int) -> np.ndarray:
    """uint8 [nb, nb]: block (i, j) active iff i == j or i XOR j is a power of two."""
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    x = i ^ j
    pow2 = (x != 0) & ((x & (x - 1)) == 0)
    return ((i == j) | pow2).astype(np.uint8)


def make_blockmask(kind: str, nb: int, rng: np.random.Generator | None = None,
                   density: float = 0.5) -> np.ndarray:
    """Block masks used by tests: "ones", "lower" (block lower-triangular),
    "butterfly", "random" (Bernoulli(density), diagonal forced on) and
    "random_holes" (Bernoulli(density), diagonal not forced, so some block
    rows may be empty)."""
    if kind == "ones":
        return np.ones((nb, nb), np.uint8)
    if kind == "lower":
        return np.tril(np.ones((nb, nb), np.uint8))
    if kind == "butterfly":
        return butterfly_blockmask(nb)
    if kind in ("random", "random_holes"):
        rng = rng if rng is not None else np.random.default_rng(0)
        m = (rng.random((nb, nb)) < density).astype(np.uint8)
        if kind == "random":
            np.fill_diagonal(m, 1)
        return m
    raise ValueError(kind)


def draw_inputs(B: int, H: int, N: int, d: int, seed: int, qk_mult: float = 1.0,
                with_do: bool = True) -> dict[str, np.ndarray]:
    """Seeded Q, K, V, dO as uint16 bf16 bit arrays of shape (B, H, N, d).

    Draw order is fixed (Q, K, V, dO) so every consumer sees the same bits.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    out = {}
    for name in ("q", "k", "v", "do"):
        if name == "do" and not with_do:
            break
        out[name] = bf16_round_bits(rng.standard_normal(shape, dtype=np.float32))
    out["q"] = _mul_pow2_bits(out["q"], qk_mult)
    out["k"] = _mul_pow2_bits(out["k"], qk_mult)
    return out


def config_inputs(cfg: Config) -> dict[str, np.ndarray]:
    return draw_inputs(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed, cfg.qk_mult, with_do=True)


def draw_inputs_nqk(B: int, H: int, Nq: int, Nk: int, d: int, seed: int) -> dict[str, np.ndarray]:
    """Seeded Q, dO of shape (B, H, Nq, d) and K, V of shape (B, H, Nk, d), as uint16
    bf16 bit arrays, drawn in the order Q, K, V, dO from N(0, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, n in (("q", Nq), ("k", Nk), ("v", Nk), ("do", Nq)):
        out[name] = bf16_round_bits(rng.standard_normal((B, H, n, d), dtype=np.float32))
    return out



def draw_inputs_device(B: int, H: int, N: int, d: int, seed: int, device="cuda:0"):
    """Seeded Q, K, V, dO of shape (B, H, N, d) drawn on the device: N(0, 1) from a
    torch generator seeded with ``seed``, rounded to bf16 by torch, in the order
    Q, K, V, dO.  For shapes too large to draw on the host (tensors of several GB);
    a consumer that needs the bits on the host copies them back."""
    import torch
    gen = torch.Generator(device=device).manual_seed(seed)
    out = {}
    for name in ("q", "k", "v", "do"):
        out[name] = torch.randn((B, H, N, d), generator=gen, device=device, dtype=torch.bfloat16)
    return out


# ---------------------------------------------------------------------------
# FP8 (E4M3) inputs.  A tensor is drawn from N(0, 1) in float32 like the bf16
# inputs, given one per-tensor factor ``descale`` = max|x| / 448 (float32, so the
# largest magnitude lands on the largest finite E4M3 value), and stored as the E4M3
# codes of x / descale, rounded to nearest with ties to the even code.
# ---------------------------------------------------------------------------

def _e4m3_table() -> np.ndarray:
    """Magnitudes of the 127 non-negative finite E4M3 codes 0x00 .. 0x7E, in code
    order (which is also increasing order): 2^-9 steps below 2^-6, then three
    mantissa bits per binade up to 448."""
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        vals.append(math.ldexp(m, -9) if e == 0 else math.ldexp(8 + m, e - 10))
    return np.array(vals, dtype=np.float64)


_E4M3 = _e4m3_table()


def e4m3_round_codes(x) -> np.ndarray:
    """float values -> uint8 E4M3 codes, round to nearest, ties to the even code.

    Magnitudes above 448 are an error (the callers scale into range first)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > _E4M3[-1]):
        raise ValueError("value outside the finite E4M3 range")
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x) & (code != 0)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def draw_inputs_fp8(B: int, H: int, N: int, d: int, seed: int,
                    amax: float = 448.0) -> dict[str, np.ndarray]:
    """Seeded Q, K, V as E4M3 codes (uint8, shape (B, H, N, d)) plus their float32
    descales under keys "q_descale", "k_descale", "v_descale".

    Draw order Q, K, V from N(0, 1) float32; descale = float32(max|x| / amax)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name in ("q", "k", "v"):
        x = rng.standard_normal((B, H, N, d), dtype=np.float32)
        ds = np.float32(np.abs(x).max() / amax) if x.size else np.float32(1.0)
        y = x.astype(np.float64) / float(ds)
        out[name] = e4m3_round_codes(np.clip(y, -amax, amax))
        out[name + "_descale"] = float(ds)
    return out
