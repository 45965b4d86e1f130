"""Plain float64 attention and its analytic gradient (TEST INFRASTRUCTURE ONLY).

What is computed, per (batch, head), for query rows q_i, key rows k_j, value rows v_j:

* Forward, the definition O = softmax(QK^T)V (FlashAttention-NeurIPS22 digest,
  "核心方法", Tiling 与 online softmax; FlashAttention-2 wiki, opening paragraph: the
  result equals standard attention with no loss of precision).  The scores are scaled
  by ``scale`` before masking, and a mask sets a score to -inf, so a masked key gets
  probability exactly 0 (the digest's kernel fuses "mask" into the same pass,
  "核心方法", Kernel fusion).  The standard path materialises S = QK^T and
  P = softmax(S) as N x N matrices (digest, "问题与动机"); so does this oracle.
* The saved softmax statistic is one log-sum-exp per row, in natural log, of the
  scaled and masked scores: LSE_i = m_i + ln sum_j exp(S_ij - m_i).  The digest
  says the forward keeps only O and the softmax normalisers for the backward
  ("核心方法", Backward recomputation); the single-number form is this library's
  reading.
* Backward: the analytic gradient of L = sum(dO * O) with respect to Q, K and V,
  by the chain rule through softmax:
      dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
      dS = P * (dP - D),  dQ = scale * dS K,  dK = scale * dS^T Q.
* Block-sparse masking (digest, "核心方法", Block-sparse 扩展): key block j is
  visible to query block i iff ``blockmask[i // mask_block, j // mask_block]`` is
  nonzero; invisible blocks are masked like any other masked score.
* A row whose keys are all masked has no softmax; by convention its O row is 0, its
  LSE is -inf, and it contributes nothing to any gradient.

Everything runs in float64 with numpy; ``@`` is the only library primitive used.
"""

from __future__ import annotations

import numpy as np


def allowed_mask(n_q: int, n_k: int, causal: bool = False, blockmask=None,
                 mask_block: int = 128) -> np.ndarray:
    """Boolean [n_q, n_k]: True where query i may attend to key j.

    Causal: key j is masked when j > i + (n_k - n_q), i.e. the n_q queries are the
    last n_q positions of the n_k-long key sequence (the decoding case with a KV
    cache, which the pages leave untreated; with n_q == n_k this is j > i).  Rows
    with i + n_k - n_q < 0 see no key.  Block-sparse: masked when the covering
    block of ``blockmask`` ([ceil(n_q / mb), ceil(n_k / mb)]) is zero.  Both may
    apply; a key is visible iff both allow.
    """
    allowed = np.ones((n_q, n_k), dtype=bool)
    if causal:
        allowed &= np.arange(n_k)[None, :] <= np.arange(n_q)[:, None] + (n_k - n_q)
    if blockmask is not None:
        bm = np.asarray(blockmask).astype(bool)
        bi = np.arange(n_q) // mask_block
        bj = np.arange(n_k) // mask_block
        allowed &= bm[bi[:, None], bj[None, :]]
    return allowed


def _softmax_rows(s: np.ndarray, allowed: np.ndarray):
    """Masked row softmax of scaled scores ``s`` (float64, modified in place).

    Returns (P, LSE).  Rows with no visible key get P = 0 and LSE = -inf.
    """
    s[~allowed] = -np.inf
    live = allowed.any(axis=1)
    m = np.where(live, s.max(axis=1, initial=-np.inf), 0.0)
    s -= m[:, None]
    np.exp(s, out=s)                      # exp(-inf) == 0 for masked entries
    denom = s.sum(axis=1)
    safe = np.where(live, denom, 1.0)
    s /= safe[:, None]
    lse = np.where(live, m + np.log(safe), -np.inf)
    return s, lse


def head_forward(q, k, v, scale: float, allowed: np.ndarray):
    """One head.  q [n_q, d], k [n_k, d], v [n_k, d], allowed [n_q, n_k].

    Returns (O [n_q, d], LSE [n_q], P [n_q, n_k]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = q @ k.T
    s *= float(scale)
    p, lse = _softmax_rows(s, allowed)
    o = p @ v
    return o, lse, p


def head_backward(q, k, v, do, scale: float, allowed: np.ndarray):
    """One head: gradients of sum(dO * O) w.r.t. q, k, v, from the definition.

    P is recomputed from Q, K here (the oracle keeps nothing between passes).
    Returns (dQ, dK, dV) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    _, _, p = head_forward(q, k, v, scale, allowed)
    dv = p.T @ do
    dp = do @ v.T
    dsum = np.einsum("ij,ij->i", p, dp)       # D_i = sum_j P_ij dP_ij
    dp -= dsum[:, None]
    dp *= p                                    # dS = P * (dP - D)
    ds = dp
    dq = (ds @ k) * float(scale)
    dk = (ds.T @ q) * float(scale)
    return dq, dk, dv


def _heads(x):
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("expected [B, H, N, d]")
    return x


def forward(q, k, v, scale: float, causal: bool = False, blockmask=None,
            mask_block: int = 128):
    """[B, H, N, d] inputs (any real dtype) -> (O [B,H,N,d], LSE [B,H,N]) float64."""
    q, k, v = _heads(q), _heads(k), _heads(v)
    B, H, N, d = q.shape
    allowed = allowed_mask(N, k.shape[2], causal, blockmask, mask_block)
    o = np.empty((B, H, N, v.shape[3]), np.float64)
    lse = np.empty((B, H, N), np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h], _ = head_forward(q[b, h], k[b, h], v[b, h], scale, allowed)
    return o, lse


def backward(q, k, v, do, scale: float, causal: bool = False, blockmask=None,
             mask_block: int = 128):
    """[B, H, N, d] inputs -> (dQ, dK, dV) float64 of the same shapes."""
    q, k, v, do = _heads(q), _heads(k), _heads(v), _heads(do)
    B, H, N, d = q.shape
    allowed = allowed_mask(N, k.shape[2], causal, blockmask, mask_block)
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(v.shape, np.float64)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = head_backward(
                q[b, h], k[b, h], v[b, h], do[b, h], scale, allowed)
    return dq, dk, dv


def forward_rows(q, k, v, scale: float, rows, causal: bool = False, blockmask=None,
                 mask_block: int = 128):
    """One head, only the query rows listed in ``rows`` (for sampled checks at full size).

    q [n_q, d] (all rows), k, v [n_k, d].  Returns (O [len(rows), d], LSE [len(rows)]).
    Each row's result depends only on that row of S, so this is the same definition
    restricted to a subset of rows.
    """
    rows = np.asarray(rows)
    n_q = np.asarray(q).shape[0]
    n_k = np.asarray(k).shape[0]
    allowed = allowed_mask(n_q, n_k, causal, blockmask, mask_block)[rows]
    o, lse, _ = head_forward(np.asarray(q)[rows], k, v, scale, allowed)
    return o, lse
