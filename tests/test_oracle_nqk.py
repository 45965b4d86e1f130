"""Pins of the oracle for N_q != N_k (cross attention and decoding with a KV
cache), where the causal mask is aligned bottom-right: query i may see key j iff
j <= i + (N_k - N_q).

* scalar brute force with that rule written out here;
* the suffix property: with a causal mask, the N_q queries behave as the last N_q
  rows of a square causal problem over the same keys;
* N_q = 1 under the causal mask sees every key; rows with i + N_k - N_q < 0 see
  none (O = 0, LSE = -inf);
* central finite differences of the gradients; torch's float64 SDPA with an
  explicit boolean mask.
"""

import math

import numpy as np
import pytest

import oracle

from test_oracle import fd_grads


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _brute(q, k, v, scale, causal, bm=None, mb=1):
    nq, nk = len(q), len(k)
    o, lse = [], []
    for i in range(nq):
        sc = []
        for j in range(nk):
            vis = (not causal or j <= i + nk - nq) and (bm is None or bm[i // mb][j // mb])
            sc.append(scale * sum(a * b for a, b in zip(q[i], k[j])) if vis else None)
        vis = [x for x in sc if x is not None]
        if not vis:
            o.append([0.0] * len(v[0]))
            lse.append(-math.inf)
            continue
        mx = max(vis)
        w = [math.exp(x - mx) if x is not None else 0.0 for x in sc]
        t = sum(w)
        o.append([sum(w[j] * v[j][c] for j in range(nk)) / t for c in range(len(v[0]))])
        lse.append(mx + math.log(t))
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("nq,nk", [(1, 1), (1, 5), (2, 7), (3, 4), (5, 3), (6, 2), (4, 9)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(nq, nk, causal):
    q, k, v = _rand((nq, 3), 1), _rand((nk, 3), 2), _rand((nk, 2), 3)
    allowed = oracle.allowed_mask(nq, nk, causal)
    o, lse, _ = oracle.head_forward(q, k, v, 0.7, allowed)
    ro, rl = _brute(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
    assert np.abs(o - ro).max() < 1e-12
    assert np.array_equal(np.isinf(lse), np.isinf(rl))
    fin = np.isfinite(rl)
    assert np.abs(lse[fin] - rl[fin]).max(initial=0) < 1e-12


def test_brute_force_block_sparse():
    nq, nk, mb = 6, 9, 2
    bm = (np.random.default_rng(4).random((3, 5)) < 0.6).astype(np.uint8)
    q, k, v = _rand((nq, 2), 5), _rand((nk, 2), 6), _rand((nk, 3), 7)
    allowed = oracle.allowed_mask(nq, nk, True, bm, mb)
    o, _, _ = oracle.head_forward(q, k, v, 1.1, allowed)
    ro, _ = _brute(q.tolist(), k.tolist(), v.tolist(), 1.1, True, bm.tolist(), mb)
    assert np.abs(o - ro).max() < 1e-12


@pytest.mark.parametrize("nq,nk", [(1, 64), (7, 64), (64, 64), (33, 100)])
def test_suffix_of_square_causal(nq, nk):
    d = 8
    qfull, k, v = _rand((nk, d), 8), _rand((nk, d), 9), _rand((nk, d), 10)
    q = qfull[nk - nq:]
    o, lse, _ = oracle.head_forward(q, k, v, 0.3, oracle.allowed_mask(nq, nk, True))
    of, lf, _ = oracle.head_forward(qfull, k, v, 0.3, oracle.allowed_mask(nk, nk, True))
    assert np.allclose(o, of[nk - nq:], rtol=0, atol=1e-13)
    assert np.allclose(lse, lf[nk - nq:], rtol=0, atol=1e-13)


def test_single_query_sees_all_keys_and_empty_rows():
    k, v = _rand((40, 4), 11), _rand((40, 4), 12)
    q = _rand((1, 4), 13)
    a = oracle.head_forward(q, k, v, 0.5, oracle.allowed_mask(1, 40, True))
    b = oracle.head_forward(q, k, v, 0.5, oracle.allowed_mask(1, 40, False))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # more queries than keys: the first n_q - n_k rows see nothing
    q = _rand((7, 4), 14)
    o, lse, _ = oracle.head_forward(q, k[:3], v[:3], 0.5, oracle.allowed_mask(7, 3, True))
    assert np.all(o[:4] == 0) and np.all(lse[:4] == -np.inf) and np.all(np.isfinite(lse[4:]))
    dq, dk, dv = oracle.head_backward(q, k[:3], v[:3], _rand((7, 4), 15), 0.5,
                                      oracle.allowed_mask(7, 3, True))
    assert np.all(dq[:4] == 0)


@pytest.mark.parametrize("nq,nk,causal", [(3, 5, True), (5, 3, True), (2, 6, False)])
def test_gradients_match_finite_differences(nq, nk, causal):
    q, k, v, do = _rand((nq, 3), 20), _rand((nk, 3), 21), _rand((nk, 3), 22), _rand((nq, 3), 23)
    allowed = oracle.allowed_mask(nq, nk, causal)
    fwd = lambda a, b, c: oracle.head_forward(a, b, c, 0.9, allowed)[0]
    fd = fd_grads(fwd, q, k, v, do)
    an = oracle.head_backward(q, k, v, do, 0.9, allowed)
    for a, b in zip(an, fd):
        assert np.abs(a - b).max() < 1e-7 * max(1.0, np.abs(b).max())


def test_against_torch_sdpa_with_explicit_mask():
    torch = pytest.importorskip("torch")
    nq, nk, d = 9, 21, 8
    q, k, v, do = _rand((nq, d), 30), _rand((nk, d), 31), _rand((nk, d), 32), _rand((nq, d), 33)
    # the bottom-right rule, built here with its own loops
    m = np.array([[j <= i + nk - nq for j in range(nk)] for i in range(nq)])
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq[None], tk[None], tv[None], attn_mask=torch.tensor(m)[None], scale=0.4)[0]
    out.backward(torch.tensor(do))
    o, _, _ = oracle.head_forward(q, k, v, 0.4, oracle.allowed_mask(nq, nk, True))
    dq, dk, dv = oracle.head_backward(q, k, v, do, 0.4, oracle.allowed_mask(nq, nk, True))
    assert np.abs(out.detach().numpy() - o).max() < 1e-10
    for a, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(a - t.grad.numpy()).max() < 1e-10
