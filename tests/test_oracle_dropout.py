"""Pins of the dropout oracle (oracle/dropout.py) that do not re-type its formulas.

What pins what:
* the Philox generator: the published known-answer vectors of Philox4x32-10
  (tests/golden/philox_kat.json: Salmon et al., SC 2011, and the Random123 known-answer
  file), which planted mistakes in the generator (swapped round multipliers, swapped
  key increments, the key advanced before round 0, output words reordered) each fail;
  output statistics (uniform words, balanced bits, no correlation between
  neighbouring counters, keys and streams); the prefix property of the keep mask; and a
  scalar re-implementation on Python integers that checks the vectorised uint64
  arithmetic (consistency only);
* the dropout semantics: p = 0 reduces to the plain oracle exactly; scalar loops over
  the definition for tiny inputs; central finite differences of the dropout forward
  (mask held fixed) against the analytic backward; the mean over many masks of the
  dropout output is the plain output; D = rowsum(dO * O) still holds;
* planted mistakes in the backward and the forward each fail one of these.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import dropout as odrop

from test_oracle import _visible, fd_grads


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- generator ------

def _philox_scalar(c, k):
    """Philox4x32-10 on Python integers (independent of the numpy uint64 version)."""
    c, k = list(c), list(k)
    for r in range(10):
        if r:
            k = [(k[0] + 0x9E3779B9) % 2**32, (k[1] + 0xBB67AE85) % 2**32]
        a = 0xD2511F53 * c[0]
        b = 0xCD9E8D57 * c[2]
        c = [(b // 2**32) ^ c[1] ^ k[0], b % 2**32, (a // 2**32) ^ c[3] ^ k[1], a % 2**32]
    return c


_KAT = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")


def _kat_vectors():
    with open(_KAT) as f:
        data = json.load(f)
    assert data["generator"] == "philox4x32" and data["rounds"] == 10
    out = []
    for vec in data["vectors"]:
        c = [int(x, 16) for x in vec["counter"]]
        k = [int(x, 16) for x in vec["key"]]
        r = [int(x, 16) for x in vec["output"]]
        out.append((vec["name"], c, k, r))
    return out


def _kat_fails(philox) -> bool:
    """True if `philox` (same signature as the oracle's) misses any published vector."""
    for _, c, k, r in _kat_vectors():
        got = [int(np.asarray(w).reshape(-1)[0]) for w in philox(*c, *k)]
        if got != r:
            return True
    return False


def test_philox_matches_published_known_answers():
    """The oracle's generator reproduces the published Philox4x32-10 known-answer
    vectors word for word (an external pin: the values are the generator authors')."""
    for name, c, k, r in _kat_vectors():
        got = [int(np.asarray(w).reshape(-1)[0]) for w in oracle.philox4x32_10(*c, *k)]
        assert got == r, (name, [f"{x:08x}" for x in got])
    assert not _kat_fails(oracle.philox4x32_10)


@pytest.mark.parametrize("kind", ["swap_multipliers", "swap_weyl", "key_bumped_first",
                                  "words_reordered"])
def test_philox_mutants_fail_known_answers(kind, monkeypatch):
    """Plausible misreadings of the generator, planted in the oracle, each miss the
    published vectors."""
    if kind == "swap_multipliers":
        monkeypatch.setattr(odrop, "_M0", odrop._M1)
        monkeypatch.setattr(odrop, "_M1", 0xD2511F53)
        mutant = odrop.philox4x32_10
    elif kind == "swap_weyl":
        monkeypatch.setattr(odrop, "_W0", odrop._W1)
        monkeypatch.setattr(odrop, "_W1", 0x9E3779B9)
        mutant = odrop.philox4x32_10
    elif kind == "key_bumped_first":
        # the key schedule advanced once before round 0 instead of after it
        def mutant(c0, c1, c2, c3, k0, k1):
            return odrop.philox4x32_10(c0, c1, c2, c3, (k0 + 0x9E3779B9) % 2**32,
                                       (k1 + 0xBB67AE85) % 2**32)
    else:
        def mutant(c0, c1, c2, c3, k0, k1):
            w = odrop.philox4x32_10(c0, c1, c2, c3, k0, k1)
            return w[1], w[0], w[3], w[2]
    assert _kat_fails(mutant), kind


def test_vectorised_philox_matches_scalar_integers():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2**32, size=(64, 4), dtype=np.uint64)
    for key in [(0, 0), (0xFFFFFFFF, 0xFFFFFFFF), (123456789, 987654321)]:
        got = np.stack(oracle.philox4x32_10(ctr[:, 0], ctr[:, 1], ctr[:, 2], ctr[:, 3], *key),
                       axis=1)
        for row, out in zip(ctr, got):
            assert [int(x) for x in out] == _philox_scalar([int(x) for x in row], key)


def test_philox_words_uniform_and_bits_balanced():
    n = 1 << 15
    j = np.arange(n, dtype=np.uint64)
    words = np.concatenate(oracle.philox4x32_10(j, 0, 7, 3, 0xDEADBEEF, 0x12345678))
    # 256-bin histogram of the top byte: chi-square with 255 dof, mean 255, sd 22.6
    hist = np.bincount((words >> np.uint64(24)).astype(np.int64), minlength=256)
    expect = len(words) / 256
    chi2 = float(((hist - expect) ** 2 / expect).sum())
    assert 255 - 6 * 22.6 < chi2 < 255 + 6 * 22.6, chi2
    # every bit set with probability 1/2 (6 sigma)
    for bit in range(32):
        frac = float(((words >> np.uint64(bit)) & np.uint64(1)).mean())
        assert abs(frac - 0.5) < 6 * 0.5 / math.sqrt(len(words)), (bit, frac)


def test_philox_avalanche_on_counter_and_key():
    rng = np.random.default_rng(11)
    base = rng.integers(0, 2**32, size=(4096, 4), dtype=np.uint64)
    out0 = np.stack(oracle.philox4x32_10(*base.T, 17, 29), axis=1)
    flips = []
    for word in range(4):
        for bit in (0, 13, 31):
            c = base.copy()
            c[:, word] ^= np.uint64(1 << bit)
            out1 = np.stack(oracle.philox4x32_10(*c.T, 17, 29), axis=1)
            flips.append(np.unpackbits((out0 ^ out1).astype(">u4").view(np.uint8)).mean())
    out_k = np.stack(oracle.philox4x32_10(*base.T, 17 ^ 1, 29), axis=1)
    flips.append(np.unpackbits((out0 ^ out_k).astype(">u4").view(np.uint8)).mean())
    assert all(abs(f - 0.5) < 0.01 for f in flips), flips


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction_is_one_minus_p(p):
    keep = oracle.keep_mask(512, 512, 3, p, 2024, 1)
    n = keep.size
    sd = math.sqrt(n * p * (1 - p))
    assert abs(keep.sum() - n * (1 - p)) < 6 * sd


def test_keep_masks_of_different_streams_are_independent():
    p = 0.5
    a = oracle.keep_mask(256, 256, 0, p, 99, 0)
    for other in (oracle.keep_mask(256, 256, 1, p, 99, 0),     # another head
                  oracle.keep_mask(256, 256, 0, p, 100, 0),    # another seed
                  oracle.keep_mask(256, 256, 0, p, 99, 1),     # another offset
                  oracle.keep_mask(256, 256, 0, p, 99 + (1 << 32), 0)):   # seed high word
        agree = float((a == other).mean())
        assert abs(agree - 0.5) < 6 * 0.5 / 256, agree
    # neighbouring keys and queries are not correlated either
    assert abs(float((a[:, 1:] == a[:, :-1]).mean()) - 0.5) < 6 * 0.5 / 256
    assert abs(float((a[1:, :] == a[:-1, :]).mean()) - 0.5) < 6 * 0.5 / 256


def test_keep_mask_prefix_property_and_threshold():
    big = oracle.keep_mask(300, 301, 5, 0.3, 7, 9)
    assert np.array_equal(oracle.keep_mask(133, 70, 5, 0.3, 7, 9), big[:133, :70])
    assert oracle.keep_mask(64, 64, 0, 0.0, 1, 1).all()
    assert oracle.drop_threshold(0.0) == 0
    assert oracle.drop_threshold(0.5) == 2**15
    assert oracle.drop_threshold(0.99999999) == 0xFFFF
    with pytest.raises(ValueError):
        oracle.drop_threshold(1.0)


def test_draw_halves_take_the_published_zero_counter_output():
    """Queries 0, 1 and keys 0..3 of head 0 with seed 0 and offset 0 form the block of
    the zero counter under the zero key: its eight 16-bit draws are the halves of the
    published output words, element (i, j) taking half (e mod 2) of word (e div 2)
    with e = 4 i + j (low half first)."""
    _, c, k, r = _kat_vectors()[0]
    assert c == [0, 0, 0, 0] and k == [0, 0]
    got = oracle.draw_halves(2, 4, 0, 0, 0)
    for i in range(2):
        for j in range(4):
            e = 4 * i + j
            assert int(got[i, j]) == (r[e // 2] >> (16 * (e % 2))) & 0xFFFF, (i, j)


def test_draw_halves_match_a_scalar_reading_of_the_rule():
    """Every element of a ragged head, from the scalar Philox on its own block counter
    (j div 4, i div 2, bh, offset) and the half e = 4 (i mod 2) + (j mod 4)."""
    n_q, n_k, bh, seed, offset = 7, 10, 3, (5 << 32) + 11, 42
    got = oracle.draw_halves(n_q, n_k, bh, seed, offset)
    for i in range(n_q):
        for j in range(n_k):
            w = _philox_scalar([j // 4, i // 2, bh, offset], [seed % 2**32, seed >> 32])
            e = 4 * (i % 2) + (j % 4)
            assert int(got[i, j]) == (w[e // 2] >> (16 * (e % 2))) & 0xFFFF, (i, j)


# ---------------------------------------------------------------- semantics ------

def test_p_zero_is_the_plain_oracle():
    q, k, v, do = (_rand((40, 8), s) for s in range(4))
    allowed = oracle.allowed_mask(40, 40, True)
    keep = oracle.keep_mask(40, 40, 0, 0.0, 5, 0)
    o, lse, _, _ = oracle.head_forward_dropout(q, k, v, 0.3, allowed, 0.0, keep)
    o0, lse0, _ = oracle.head_forward(q, k, v, 0.3, allowed)
    assert np.array_equal(o, o0) and np.array_equal(lse, lse0)
    g = oracle.head_backward_dropout(q, k, v, do, 0.3, allowed, 0.0, keep)
    g0 = oracle.head_backward(q, k, v, do, 0.3, allowed)
    for a, b in zip(g, g0):
        assert np.allclose(a, b, rtol=0, atol=1e-13)


def _brute_dropout_forward(q, k, v, scale, keep, p, causal):
    nq, nk, dv = len(q), len(k), len(v[0])
    out = []
    for i in range(nq):
        sc = [scale * sum(q[i][t] * k[j][t] for t in range(len(q[i])))
              if _visible(i, j, causal, None, 1) else None for j in range(nk)]
        vis = [s for s in sc if s is not None]
        mx = max(vis)
        w = [math.exp(s - mx) if s is not None else 0.0 for s in sc]
        tot = sum(w)
        out.append([sum((w[j] / tot) * (1.0 if keep[i][j] else 0.0) / (1.0 - p) * v[j][t]
                        for j in range(nk)) for t in range(dv)])
    return np.array(out)


@pytest.mark.parametrize("n,d,causal,p", [(5, 3, False, 0.5), (8, 2, True, 0.25),
                                          (7, 4, True, 0.75)])
def test_dropout_forward_matches_brute_force(n, d, causal, p):
    q, k, v = (_rand((n, d), 10 + s) for s in range(3))
    keep = oracle.keep_mask(n, n, 2, p, 77, 3)
    allowed = oracle.allowed_mask(n, n, causal)
    o, _, _, _ = oracle.head_forward_dropout(q, k, v, 0.7, allowed, p, keep)
    ref = _brute_dropout_forward(q.tolist(), k.tolist(), v.tolist(), 0.7, keep.tolist(), p,
                                 causal)
    assert np.abs(o - ref).max() < 1e-12


def _fd_case(seed=3, n=6, d=3, p=0.4, causal=True):
    q, k, v, do = (_rand((n, d), seed + s) for s in range(4))
    allowed = oracle.allowed_mask(n, n, causal)
    keep = oracle.keep_mask(n, n, 1, p, 555, 2)
    return q, k, v, do, allowed, keep, p


def test_dropout_gradients_match_finite_differences():
    q, k, v, do, allowed, keep, p = _fd_case()
    fwd = lambda a, b, c: oracle.head_forward_dropout(a, b, c, 0.8, allowed, p, keep)[0]
    fd = fd_grads(fwd, q, k, v, do)
    an = oracle.head_backward_dropout(q, k, v, do, 0.8, allowed, p, keep)
    for a, b in zip(an, fd):
        assert np.abs(a - b).max() < 1e-7 * max(1.0, np.abs(b).max())


def test_dropout_is_unbiased_over_masks():
    n, d, p = 24, 4, 0.5
    q, k, v = (_rand((n, d), 40 + s) for s in range(3))
    allowed = oracle.allowed_mask(n, n, False)
    o_plain, _, _ = oracle.head_forward(q, k, v, 0.5, allowed)
    acc = np.zeros_like(o_plain)
    draws = 400
    for seed in range(draws):
        keep = oracle.keep_mask(n, n, 0, p, seed, 0)
        acc += oracle.head_forward_dropout(q, k, v, 0.5, allowed, p, keep)[0]
    mean = acc / draws
    # each output is a sum of n terms with variance below max|v|^2 p/(1-p) / n per term
    sd = np.abs(v).max() * math.sqrt(p / (1 - p)) / math.sqrt(draws)
    assert np.abs(mean - o_plain).max() < 6 * sd


def test_dsum_identity_holds_with_dropout():
    q, k, v, do, allowed, keep, p = _fd_case(seed=8, n=10, d=5)
    o, _, prob, pd = oracle.head_forward_dropout(q, k, v, 0.6, allowed, p, keep)
    dp = (do @ v.T) * keep / (1 - p)
    assert np.allclose(np.einsum("ij,ij->i", prob, dp), np.einsum("ij,ij->i", do, o),
                       rtol=0, atol=1e-12)


# ---------------------------------------------------------------- mutants --------

def _mutant_backward(kind):
    def bwd(q, k, v, do, scale, allowed, p, keep):
        _, _, prob, pd = odrop.head_forward_dropout(q, k, v, scale, allowed, p, keep)
        if kind == "dv_uses_p":
            dv = prob.T @ do
        else:
            dv = pd.T @ do
        dp = do @ v.T
        if kind != "dp_no_mask":
            dp = dp * keep / (1.0 - p) if kind != "dp_no_rescale" else dp * keep
        dsum = np.einsum("ij,ij->i", prob, dp)
        ds = prob * (dp - dsum[:, None])
        return (ds @ k) * scale, (ds.T @ q) * scale, dv
    return bwd


@pytest.mark.parametrize("kind", ["dv_uses_p", "dp_no_mask", "dp_no_rescale"])
def test_backward_mutants_are_caught(kind):
    q, k, v, do, allowed, keep, p = _fd_case(seed=21)
    fwd = lambda a, b, c: oracle.head_forward_dropout(a, b, c, 0.8, allowed, p, keep)[0]
    fd = fd_grads(fwd, q, k, v, do)
    bad = _mutant_backward(kind)(q, k, v, do, 0.8, allowed, p, keep)
    assert max(np.abs(a - b).max() for a, b in zip(bad, fd)) > 1e-3


@pytest.mark.parametrize("kind", ["renormalise_after_drop", "no_rescale", "drop_scores"])
def test_forward_mutants_are_caught(kind):
    n, d, p = 6, 3, 0.5
    q, k, v = (_rand((n, d), 60 + s) for s in range(3))
    keep = oracle.keep_mask(n, n, 0, p, 31, 0)
    allowed = oracle.allowed_mask(n, n, False)
    s = 0.9 * q @ k.T
    e = np.exp(s - s.max(axis=1, keepdims=True))
    if kind == "renormalise_after_drop":
        w = e * keep
        o = (w / w.sum(axis=1, keepdims=True)) @ v
    elif kind == "no_rescale":
        o = (e / e.sum(axis=1, keepdims=True) * keep) @ v
    else:   # dropout applied to the scores (masked to -inf) before the softmax
        e = np.where(keep, e, 0.0)
        o = (e / e.sum(axis=1, keepdims=True)) @ v
    ref = _brute_dropout_forward(q.tolist(), k.tolist(), v.tolist(), 0.9, keep.tolist(), p,
                                 False)
    assert np.abs(o - ref).max() > 1e-3
