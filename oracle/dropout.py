"""Attention with dropout on the probabilities, in float64 (TEST INFRASTRUCTURE ONLY).

The digest lists dropout among the steps its single kernel fuses between the softmax
and the second product (FlashAttention-NeurIPS22 digest, "核心方法", Kernel fusion:
matmul, mask, softmax, dropout (optional), matmul), and the backward rebuilds
everything it needs on chip from the saved statistics ("核心方法", Backward
recomputation).  The pages say nothing more, so this library reads dropout as the
usual attention dropout, and draws it from a counter-based generator so that the
backward can regenerate the forward's mask instead of storing it:

* P = softmax(S) as in ``attention.head_forward`` (the row sum, and so LSE, is taken
  before dropout).
* keep_ij is a Bernoulli(1 - p) draw; Pd = P * keep / (1 - p); O = Pd V.
* Backward of L = sum(dO * O):  dV = Pd^T dO;  dPd = dO V^T;  dP = dPd * keep / (1 - p);
  D_i = sum_j P_ij dP_ij (which equals sum_k dO_ik O_ik);  dS = P * (dP - D);
  dQ = scale * dS K;  dK = scale * dS^T Q.

One draw of Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
as easy as 1, 2, 3", SC 2011), applied to the counter (j div 4, i div 2, b*H + h,
offset) under the key (seed mod 2^32, seed div 2^32), decides the block of two
queries i and four keys j that share those quotients: its four 32-bit output words
hold eight 16-bit halves, and element (b, h, i, j) takes half number
e = 4 (i mod 2) + (j mod 4), i.e. bits 16 (e mod 2) .. 16 (e mod 2) + 15 of word
e div 2.  The element is dropped iff that 16-bit value is below floor(p * 2^16).
Philox is written here
from its definition in that paper: ten rounds, each multiplying counter words 0 and 2
by two fixed odd constants and mixing the high and low halves of the products with
words 1 and 3 and the round key, the key advancing by two Weyl constants per round.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import head_forward

_M0, _M1 = 0xD2511F53, 0xCD9E8D57        # round multipliers
_W0, _W1 = 0x9E3779B9, 0xBB67AE85        # key increments (Weyl sequence)
_MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of counter words (any shape, values < 2^32).

    Returns the four output words as uint64 arrays holding 32-bit values.
    """
    c0, c1, c2, c3 = (np.asarray(x, dtype=np.uint64) & np.uint64(_MASK32)
                      for x in (c0, c1, c2, c3))
    k0, k1 = int(k0) & _MASK32, int(k1) & _MASK32
    m0, m1, lo32 = np.uint64(_M0), np.uint64(_M1), np.uint64(_MASK32)
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & _MASK32
            k1 = (k1 + _W1) & _MASK32
        p0 = c0 * m0                      # 32 x 32 -> 64 bits, exact in uint64
        p1 = c2 * m1
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ np.uint64(k0), p1 & lo32,
                          (p0 >> np.uint64(32)) ^ c3 ^ np.uint64(k1), p0 & lo32)
    return c0, c1, c2, c3


def drop_threshold(p: float) -> int:
    """floor(p * 2^16), the 16-bit value below which an element is dropped."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(int(math.floor(float(p) * 65536.0)), 0xFFFF)


def draw_halves(n_q: int, n_k: int, bh: int, seed: int, offset: int) -> np.ndarray:
    """uint64 [n_q, n_k]: the 16-bit draw of each element (i, j) of head bh."""
    ig = np.arange((n_q + 1) // 2, dtype=np.uint64)[:, None]
    jg = np.arange((n_k + 3) // 4, dtype=np.uint64)[None, :]
    shape = ((n_q + 1) // 2, (n_k + 3) // 4)
    words = philox4x32_10(np.broadcast_to(jg, shape), np.broadcast_to(ig, shape),
                          np.full(shape, bh, np.uint64), np.full(shape, offset, np.uint64),
                          seed & _MASK32, (seed >> 32) & _MASK32)
    out = np.empty((shape[0], 2, shape[1], 4), np.uint64)   # [i div 2, i mod 2, j div 4, j mod 4]
    for e in range(8):
        half = (words[e // 2] >> np.uint64(16 * (e % 2))) & np.uint64(0xFFFF)
        out[:, e // 4, :, e % 4] = half
    return out.reshape(2 * shape[0], 4 * shape[1])[:n_q, :n_k]


def keep_mask(n_q: int, n_k: int, bh: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean [n_q, n_k]: True where element (i, j) of head bh is kept."""
    return draw_halves(n_q, n_k, bh, seed, offset) >= np.uint64(drop_threshold(p))


def head_forward_dropout(q, k, v, scale: float, allowed: np.ndarray, p: float,
                         keep: np.ndarray):
    """One head with dropout.  Returns (O, LSE, P, Pd); LSE is that of the plain softmax."""
    _, lse, prob = head_forward(q, k, v, scale, allowed)
    pd = prob * keep / (1.0 - p)
    o = pd @ np.asarray(v, dtype=np.float64)
    return o, lse, prob, pd


def head_backward_dropout(q, k, v, do, scale: float, allowed: np.ndarray, p: float,
                          keep: np.ndarray):
    """Gradients of sum(dO * O) for the dropout forward with this keep mask."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _, _, prob, pd = head_forward_dropout(q, k, v, scale, allowed, p, keep)
    dv = pd.T @ do
    dp = (do @ v.T) * keep / (1.0 - p)           # gradient reaching P through the dropout
    dsum = np.einsum("ij,ij->i", prob, dp)
    ds = prob * (dp - dsum[:, None])
    dq = (ds @ k) * float(scale)
    dk = (ds.T @ q) * float(scale)
    return dq, dk, dv


def forward_dropout(q, k, v, scale: float, p: float, seed: int, offset: int,
                    causal: bool = False, blockmask=None, mask_block: int = 128):
    """[B, H, N, d] -> (O, LSE) float64, with dropout drawn as described above."""
    from .attention import allowed_mask
    q, k, v = (np.asarray(x) for x in (q, k, v))
    B, H, N, d = q.shape
    allowed = allowed_mask(N, k.shape[2], causal, blockmask, mask_block)
    o = np.empty((B, H, N, v.shape[3]), np.float64)
    lse = np.empty((B, H, N), np.float64)
    for b in range(B):
        for h in range(H):
            keep = keep_mask(N, k.shape[2], b * H + h, p, seed, offset)
            o[b, h], lse[b, h], _, _ = head_forward_dropout(q[b, h], k[b, h], v[b, h], scale,
                                                            allowed, p, keep)
    return o, lse


def backward_dropout(q, k, v, do, scale: float, p: float, seed: int, offset: int,
                     causal: bool = False, blockmask=None, mask_block: int = 128):
    """[B, H, N, d] -> (dQ, dK, dV) float64 for the dropout forward."""
    from .attention import allowed_mask
    q, k, v, do = (np.asarray(x) for x in (q, k, v, do))
    B, H, N, d = q.shape
    allowed = allowed_mask(N, k.shape[2], causal, blockmask, mask_block)
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(v.shape, np.float64)
    for b in range(B):
        for h in range(H):
            keep = keep_mask(N, k.shape[2], b * H + h, p, seed, offset)
            dq[b, h], dk[b, h], dv[b, h] = head_backward_dropout(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, allowed, p, keep)
    return dq, dk, dv
