"""Pins for the fp64 oracle, each against something other than the oracle itself.

* brute force: scalar Python loops over the attention definition, with the mask
  rules written out independently (tiny sizes);
* a library routine: torch CPU float64 scaled_dot_product_attention plus autograd;
* hand-derived closed forms stored in tests/golden/hand_cases.json;
* closed forms and invariants of softmax attention (N = 1, identical V rows,
  per-row score shift, scale = 0, causal row 0, no future leak, rows of P sum to 1);
* central finite differences of the forward for every gradient;
* mutation checks: plausible mistakes planted into copies of the oracle must fail
  at least one of the pins above.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# ----------------------------------------------------------------------------------
# brute force: plain loops, own mask rules
# ----------------------------------------------------------------------------------

def _visible(i, j, causal, blockmask, mb):
    if causal and j > i:
        return False
    if blockmask is not None and not blockmask[i // mb][j // mb]:
        return False
    return True


def brute_forward(q, k, v, scale, causal=False, blockmask=None, mb=1):
    nq, nk, dv = len(q), len(k), len(v[0])
    O, L = [], []
    for i in range(nq):
        sc = []
        for j in range(nk):
            if _visible(i, j, causal, blockmask, mb):
                sc.append(scale * sum(q[i][t] * k[j][t] for t in range(len(q[i]))))
            else:
                sc.append(None)
        vis = [s for s in sc if s is not None]
        if not vis:
            O.append([0.0] * dv)
            L.append(-math.inf)
            continue
        mx = max(vis)
        w = [math.exp(s - mx) if s is not None else 0.0 for s in sc]
        tot = sum(w)
        O.append([sum(w[j] * v[j][t] for j in range(nk)) / tot for t in range(dv)])
        L.append(mx + math.log(tot))
    return np.array(O), np.array(L)


def fd_grads(fwd, q, k, v, do, h=1e-5):
    """Central differences of L = sum(dO * O) w.r.t. every element of q, k, v."""
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*args[which].shape):
            a = [x.copy() for x in args]
            a[which][idx] += h
            lp = np.sum(do * fwd(*a))
            a[which][idx] -= 2 * h
            lm = np.sum(do * fwd(*a))
            g[idx] = (lp - lm) / (2 * h)
        grads.append(g)
    return grads


def _tiny_cases():
    rng = np.random.default_rng(7)
    cases = []
    for n, d in itertools.product((1, 2, 3, 5, 8), (1, 2, 4)):
        for kind in ("dense", "causal", "block", "block_causal", "holes"):
            mb = 2
            nb = -(-n // mb)
            bm = None
            causal = kind in ("causal", "block_causal")
            if kind in ("block", "block_causal"):
                bm = synth.make_blockmask("random", nb, rng, 0.5)
            if kind == "holes":
                bm = synth.make_blockmask("random_holes", nb, rng, 0.4)
            q = rng.standard_normal((n, d))
            k = rng.standard_normal((n, d))
            v = rng.standard_normal((n, d + 1))
            do = rng.standard_normal((n, d + 1))
            scale = float(rng.uniform(0.2, 1.5))
            cases.append((n, d, kind, q, k, v, do, scale, causal, bm, mb))
    return cases


TINY = _tiny_cases()


@pytest.mark.parametrize("case", TINY, ids=[f"n{c[0]}d{c[1]}{c[2]}" for c in TINY])
def test_forward_matches_brute_force(case):
    n, d, kind, q, k, v, do, scale, causal, bm, mb = case
    allowed = oracle.allowed_mask(n, n, causal, bm, mb)
    o, lse, p = oracle.head_forward(q, k, v, scale, allowed)
    bo, bl = brute_forward(q.tolist(), k.tolist(), v.tolist(), scale, causal, bm, mb)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], bl[fin], rtol=0, atol=1e-12)
    assert np.all(lse[~fin] == -np.inf)


@pytest.mark.parametrize("case", TINY[::3], ids=[f"n{c[0]}d{c[1]}{c[2]}" for c in TINY[::3]])
def test_gradients_match_finite_differences(case):
    n, d, kind, q, k, v, do, scale, causal, bm, mb = case
    allowed = oracle.allowed_mask(n, n, causal, bm, mb)

    def fwd(qq, kk, vv):
        return oracle.head_forward(qq, kk, vv, scale, allowed)[0]

    dq, dk, dv = oracle.head_backward(q, k, v, do, scale, allowed)
    fq, fk, fv = fd_grads(fwd, q, k, v, do)
    for a, b in ((dq, fq), (dk, fk), (dv, fv)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-8 * max(1.0, np.abs(b).max()))


def test_gradients_match_fd_of_brute_force():
    """Backward against finite differences of the *brute-force* forward (not the oracle's)."""
    rng = np.random.default_rng(11)
    n, d, mb = 6, 3, 2
    bm = np.array([[1, 0, 1], [1, 1, 0], [0, 1, 1]], np.uint8)
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    for causal in (False, True):
        def fwd(qq, kk, vv):
            return brute_forward(qq.tolist(), kk.tolist(), vv.tolist(), 0.7, causal, bm, mb)[0]
        allowed = oracle.allowed_mask(n, n, causal, bm, mb)
        got = oracle.head_backward(q, k, v, do, 0.7, allowed)
        ref = fd_grads(fwd, q, k, v, do)
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-8)


# ----------------------------------------------------------------------------------
# library routine: torch float64 SDPA + autograd
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("n,d,mb,mask", [
    (64, 16, 16, "dense"), (80, 8, 32, "causal"), (96, 16, 32, "butterfly"),
    (75, 12, 16, "random"), (128, 32, 32, "random_causal"),
])
def test_against_torch_sdpa_float64(n, d, mb, mask):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(n + d)
    B, H = 2, 3
    q, k, v, do = (rng.standard_normal((B, H, n, d)) for _ in range(4))
    nb = -(-n // mb)
    causal = mask in ("causal", "random_causal")
    bm = None
    if mask == "butterfly":
        bm = synth.butterfly_blockmask(nb)
    elif mask.startswith("random"):
        bm = synth.make_blockmask("random", nb, rng, 0.5)
    scale = 1.0 / math.sqrt(d)
    o, lse = oracle.forward(q, k, v, scale, causal, bm, mb)
    dq, dk, dv = oracle.backward(q, k, v, do, scale, causal, bm, mb)

    vis = np.ones((n, n), bool)
    for i in range(n):
        for j in range(n):
            vis[i, j] = _visible(i, j, causal, bm, mb)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=torch.tensor(vis), scale=scale)
    to.backward(torch.tensor(do))
    np.testing.assert_allclose(o, to.detach().numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-10)
    # LSE against a direct log-sum-exp over the visible scores (brute force per row)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    for i in range(0, n, 7):
        row = s[:, :, i, vis[i]]
        ref = np.log(np.exp(row).sum(-1))
        np.testing.assert_allclose(lse[:, :, i], ref, rtol=0, atol=1e-10)


# ----------------------------------------------------------------------------------
# hand-derived closed forms (golden file)
# ----------------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    q, k, v, do = (np.array(case[x], np.float64) for x in ("q", "k", "v", "do"))
    bm = None if case["blockmask"] is None else np.array(case["blockmask"], np.uint8)
    allowed = oracle.allowed_mask(len(q), len(k), case["causal"], bm, case["mask_block"])
    o, lse, _ = oracle.head_forward(q, k, v, case["scale"], allowed)
    dq, dk, dv = oracle.head_backward(q, k, v, do, case["scale"], allowed)
    np.testing.assert_allclose(o, case["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, case["lse"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dq, case["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk, case["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv, case["dv"], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------------

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_key_closed_form():
    q, k, v, do = (_rand((1, 5), s) for s in range(4))
    allowed = np.ones((1, 1), bool)
    o, lse, p = oracle.head_forward(q, k, v, 0.3, allowed)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, [0.3 * float(q[0] @ k[0])], atol=1e-15)
    dq, dk, dv = oracle.head_backward(q, k, v, do, 0.3, allowed)
    np.testing.assert_array_equal(dq, 0)
    np.testing.assert_array_equal(dk, 0)
    np.testing.assert_allclose(dv, do, atol=1e-15)


def test_rows_of_p_sum_to_one_and_masked_zero():
    n = 40
    q, k, v = (_rand((n, 8), s) for s in range(3))
    bm = synth.make_blockmask("random", 5, np.random.default_rng(3), 0.5)
    allowed = oracle.allowed_mask(n, n, True, bm, 8)
    _, _, p = oracle.head_forward(q, k, v, 0.5, allowed)
    np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
    assert np.all(p[~allowed] == 0.0)
    assert np.all(p[allowed] > 0.0)


def test_identical_value_rows():
    n, d = 33, 6
    q, k, do = (_rand((n, d), s) for s in range(3))
    row = _rand((d,), 9)
    v = np.tile(row, (n, 1))
    for causal in (False, True):
        allowed = oracle.allowed_mask(n, n, causal)
        o, _, _ = oracle.head_forward(q, k, v, 0.9, allowed)
        np.testing.assert_allclose(o, np.tile(row, (n, 1)), atol=1e-13)
        dq, dk, _ = oracle.head_backward(q, k, v, do, 0.9, allowed)
        np.testing.assert_allclose(dq, 0, atol=1e-12)
        np.testing.assert_allclose(dk, 0, atol=1e-12)


def test_per_row_score_shift():
    """K' = K + 1 w^T adds scale*(q_i . w) to row i of S: O and all gradients unchanged."""
    n, d, scale = 30, 5, 0.4
    q, k, v, do = (_rand((n, d), s) for s in range(4))
    w = _rand((d,), 17)
    for causal in (False, True):
        allowed = oracle.allowed_mask(n, n, causal)
        o, lse, _ = oracle.head_forward(q, k, v, scale, allowed)
        o2, lse2, _ = oracle.head_forward(q, k + w, v, scale, allowed)
        np.testing.assert_allclose(o2, o, atol=1e-12)
        np.testing.assert_allclose(lse2 - lse, scale * (q @ w), atol=1e-12)
        g1 = oracle.head_backward(q, k, v, do, scale, allowed)
        g2 = oracle.head_backward(q, k + w, v, do, scale, allowed)
        for a, b in zip(g1, g2):
            np.testing.assert_allclose(a, b, atol=1e-11)


def test_scale_zero_is_uniform_average():
    n, d = 24, 4
    q, k, v = (_rand((n, d), s) for s in range(3))
    bm = synth.make_blockmask("random", 3, np.random.default_rng(5), 0.6)
    allowed = oracle.allowed_mask(n, n, True, bm, 8)
    o, lse, _ = oracle.head_forward(q, k, v, 0.0, allowed)
    cnt = allowed.sum(1)
    np.testing.assert_allclose(o, (allowed @ v) / cnt[:, None], atol=1e-13)
    np.testing.assert_allclose(lse, np.log(cnt), atol=1e-13)


def test_causal_row_zero_and_no_future_leak():
    n, d = 20, 4
    q, k, v = (_rand((n, d), s) for s in range(3))
    allowed = oracle.allowed_mask(n, n, True)
    o, lse, _ = oracle.head_forward(q, k, v, 0.8, allowed)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    np.testing.assert_allclose(lse[0], 0.8 * q[0] @ k[0], atol=1e-15)
    i = 9
    k2, v2 = k.copy(), v.copy()
    k2[i + 1:] += 5.0
    v2[i + 1:] -= 3.0
    o2, _, _ = oracle.head_forward(q, k2, v2, 0.8, allowed)
    np.testing.assert_array_equal(o2[: i + 1], o[: i + 1])


def test_gradient_invariants():
    n, d, scale = 40, 8, 0.35
    q, k, v, do = (_rand((n, d), s + 20) for s in range(4))
    for causal in (False, True):
        allowed = oracle.allowed_mask(n, n, causal)
        o, _, p = oracle.head_forward(q, k, v, scale, allowed)
        dq, dk, dv = oracle.head_backward(q, k, v, do, scale, allowed)
        np.testing.assert_allclose(dv.sum(0), do.sum(0), atol=1e-12)   # columns of P sum... rows sum to 1
        np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)         # rows of dS sum to 0
        dp = do @ v.T
        np.testing.assert_allclose((p * dp).sum(1), (do * o).sum(1), atol=1e-12)


def test_fully_masked_rows_convention():
    n, d = 8, 3
    q, k, v, do = (_rand((n, d), s) for s in range(4))
    bm = np.array([[1, 0], [0, 0]], np.uint8)   # rows 4..7 see nothing
    allowed = oracle.allowed_mask(n, n, False, bm, 4)
    o, lse, p = oracle.head_forward(q, k, v, 1.0, allowed)
    assert np.all(o[4:] == 0) and np.all(lse[4:] == -np.inf) and np.all(p[4:] == 0)
    dq, dk, dv = oracle.head_backward(q, k, v, do, 1.0, allowed)
    assert np.all(dq[4:] == 0)
    # the dead rows must not contribute: same grads as the 4-row live problem
    ref = oracle.head_backward(q[:4], k[:4], v[:4], do[:4], 1.0, np.ones((4, 4), bool))
    np.testing.assert_allclose(dk[:4], ref[1], atol=1e-14)
    np.testing.assert_allclose(dv[:4], ref[2], atol=1e-14)
    assert np.all(dk[4:] == 0) and np.all(dv[4:] == 0)


# ----------------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------------

def test_mask_reductions():
    n, d, mb = 64, 8, 16
    q, k, v = (_rand((2, 2, n, d), s) for s in range(3))
    nb = n // mb
    dense = oracle.forward(q, k, v, 0.5)
    ones = oracle.forward(q, k, v, 0.5, False, synth.make_blockmask("ones", nb), mb)
    np.testing.assert_array_equal(dense[0], ones[0])
    causal = oracle.forward(q, k, v, 0.5, True)
    lower = oracle.forward(q, k, v, 0.5, True, synth.make_blockmask("lower", nb), mb)
    np.testing.assert_array_equal(causal[0], lower[0])


def test_allowed_mask_counts():
    a = oracle.allowed_mask(100, 100, True)
    assert a.sum() == 100 * 101 // 2 and a[3, 3] and not a[3, 4]
    bm = synth.butterfly_blockmask(32)
    assert np.all(bm.sum(1) == 6) and np.array_equal(bm, bm.T)
    a = oracle.allowed_mask(32 * 4, 32 * 4, False, bm, 4)
    assert a.sum() == 32 * 6 * 16
    # ragged: N not a multiple of the block size
    a = oracle.allowed_mask(10, 10, False, np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]]), 4)
    assert a[0, 8] and not a[0, 4] and a[9, 0] and a[9, 9] and not a[5, 9]


def test_forward_rows_matches_full():
    n, d = 50, 6
    q, k, v = (_rand((n, d), s) for s in range(3))
    bm = synth.make_blockmask("random", 4, np.random.default_rng(1), 0.5)
    o, lse, _ = oracle.head_forward(q, k, v, 0.6, oracle.allowed_mask(n, n, True, bm, 16))
    rows = np.array([0, 7, 16, 49])
    o2, lse2 = oracle.forward_rows(q, k, v, 0.6, rows, True, bm, 16)
    np.testing.assert_allclose(o2, o[rows], atol=1e-14)
    np.testing.assert_allclose(lse2, lse[rows], atol=1e-14)


# ----------------------------------------------------------------------------------
# mutation checks: the pins above catch plausible mistakes
# ----------------------------------------------------------------------------------

def _mutant_backward(kind):
    def bwd(q, k, v, do, scale, allowed):
        _, _, p = oatt.head_forward(q, k, v, scale, allowed)
        dv = p.T @ do if kind != "dv_no_transpose" else p @ do
        dp = do @ v.T
        dsum = np.einsum("ij,ij->i", p, dp)
        if kind == "ds_sign":
            ds = p * (dp + dsum[:, None])
        elif kind == "ds_drop_d":
            ds = p * dp
        else:
            ds = p * (dp - dsum[:, None])
        dq = ds @ k * (scale if kind != "dq_no_scale" else 1.0)
        dk = (ds @ q if kind == "dk_transposed" else ds.T @ q) * scale
        return dq, dk, dv
    return bwd


@pytest.mark.parametrize("kind", ["dv_no_transpose", "ds_sign", "ds_drop_d", "dq_no_scale",
                                  "dk_transposed"])
def test_mutants_of_backward_are_caught(kind):
    rng = np.random.default_rng(5)
    n, d = 5, 3
    q, k, v, do = (rng.standard_normal((n, d)) for _ in range(4))
    allowed = oracle.allowed_mask(n, n, True)

    def fwd(qq, kk, vv):
        return brute_forward(qq.tolist(), kk.tolist(), vv.tolist(), 0.7, True)[0]

    ref = fd_grads(fwd, q, k, v, do)
    got = _mutant_backward(kind)(q, k, v, do, 0.7, allowed)
    assert max(np.abs(a - b).max() for a, b in zip(got, ref)) > 1e-4


@pytest.mark.parametrize("kind", ["no_scale", "causal_strict", "mask_after_softmax",
                                  "lse_log2", "v_transposed_rows"])
def test_mutants_of_forward_are_caught(kind):
    rng = np.random.default_rng(6)
    n, d = 6, 6
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    scale = 0.6
    allow = np.array([[j <= i for j in range(n)] for i in range(n)])
    if kind == "causal_strict":
        allow = np.array([[j < i for j in range(n)] for i in range(n)])
        allow[0, 0] = True
    s = (q @ k.T) * (scale if kind != "no_scale" else 1.0)
    if kind == "mask_after_softmax":
        p = np.exp(s - s.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        p = np.where(allow, p, 0.0)
        lse = np.log(np.exp(s).sum(1))
    else:
        s = np.where(allow, s, -np.inf)
        m = s.max(1)
        e = np.exp(s - m[:, None])
        p = e / e.sum(1, keepdims=True)
        lse = m + (np.log2(e.sum(1)) if kind == "lse_log2" else np.log(e.sum(1)))
    o = p @ (v.T if kind == "v_transposed_rows" else v)
    bo, bl = brute_forward(q.tolist(), k.tolist(), v.tolist(), scale, True)
    assert max(np.abs(o - bo).max(), np.abs(lse - bl).max()) > 1e-4


# ----------------------------------------------------------------------------------
# input generator
# ----------------------------------------------------------------------------------

def test_bf16_rounding_is_rne():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5,
                  3.0e-39], np.float32)
    b = synth.bf16_round_bits(f)
    back = synth.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to even (1.0)
    assert back[0] == 1.0 and back[1] == 1.0
    assert back[2] == np.float32(1.0 + 2 ** -6)      # tie 1+3*2^-8 -> even mantissa 1+2^-6
    assert back[3] == np.float32(1.0 + 2 ** -7)      # above the tie rounds up
    assert back[4] == -2.5
    rng = np.random.default_rng(0)
    x = rng.standard_normal(10000).astype(np.float32)
    err = np.abs(synth.bf16_bits_to_f64(synth.bf16_round_bits(x)) - x)
    assert np.all(err <= np.abs(x) * 2.0 ** -8 + 1e-45)


def test_draw_inputs_deterministic_and_shaped():
    a = synth.draw_inputs(1, 2, 16, 8, seed=5)
    b = synth.draw_inputs(1, 2, 16, 8, seed=5)
    for kname in ("q", "k", "v", "do"):
        assert a[kname].shape == (1, 2, 16, 8) and a[kname].dtype == np.uint16
        np.testing.assert_array_equal(a[kname], b[kname])
    c = synth.draw_inputs(1, 2, 16, 8, seed=5, qk_mult=0.5)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(c["q"]),
                                  synth.bf16_bits_to_f32(a["q"]) * np.float32(0.5))
    np.testing.assert_array_equal(c["v"], a["v"])
