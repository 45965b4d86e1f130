"""Attention on FP8 (E4M3) inputs with per-tensor scales (TEST INFRASTRUCTURE ONLY).

The FlashAttention-2 wiki ("与后续版本的比较", FlashAttention-3) names 8-bit floating
point as the following generation's way to go faster.  The pages do not say which
8-bit format, how values are scaled, or what the result should be.  This library's
reading, which is what this oracle computes:

* Each of Q, K and V arrives as one byte per element in the OCP 8-bit floating-point
  format E4M3 (the "FN" variant: no infinities), together with one fp32 factor per
  tensor, the "descale": element x stands for ``e4m3_value(x) * descale``.
* The result is exact attention of the real-valued tensors those bytes stand for,
  with the same scale, masks and LSE convention as the bf16 path.  The FP8 kernel
  also rounds P to E4M3 before the P V product, which this definition does not: that
  rounding is the kernel's approximation, bounded separately in the parity tests.

E4M3, per the OCP 8-bit floating point specification: bit 7 is the sign, bits 6..3
an exponent field e with bias 7, bits 2..0 a mantissa field m.  e = 0 encodes the
subnormals m/8 * 2^-6 (and zero); e = 15 with m = 7 is NaN; every other code is
(1 + m/8) * 2^(e - 7).  The largest finite value is 448 (e = 15, m = 6).
"""

from __future__ import annotations

import numpy as np

from .attention import head_forward


def e4m3_value(codes) -> np.ndarray:
    """uint8 codes (any shape) -> float64 values, from the field definition above."""
    c = np.asarray(codes).astype(np.int64)
    if np.any((c < 0) | (c > 255)):
        raise ValueError("E4M3 codes are bytes")
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def dequantize(codes, descale: float) -> np.ndarray:
    """The real values a tensor of codes stands for: e4m3_value(code) * descale.

    ``descale`` is the fp32 factor the caller passes, taken exactly (upcast)."""
    return e4m3_value(codes) * float(np.float32(descale))


def head_forward_fp8(q8, k8, v8, scale: float, q_descale: float, k_descale: float,
                     v_descale: float, allowed: np.ndarray):
    """One head of FP8 attention.  q8 [n_q, d], k8, v8 [n_k, d] uint8 codes.

    Returns (O, LSE, P) of exact attention on the dequantised inputs, float64.
    """
    return head_forward(dequantize(q8, q_descale), dequantize(k8, k_descale),
                        dequantize(v8, v_descale), float(np.float32(scale)), allowed)
