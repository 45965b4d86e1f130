"""Pins of the FP8 (E4M3) oracle and of the FP8 input generator.

* e4m3_value against torch's own float8_e4m3fn decoding, for all 256 codes, and
  against closed forms (largest finite value, smallest normal and subnormal, 1, -1);
* the generator's round-to-nearest-even encoder: every finite code round-trips,
  ties go to the even code, and it agrees with torch's float8_e4m3fn conversion;
* head_forward_fp8 against a hand-written closed form with non-trivial descales,
  exact invariants of the descales, and torch's float64 SDPA on the dequantised
  values.
"""

import math

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")


def _torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_value_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_value(codes)
    ref = _torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2            # 0x7F and 0xFF
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0),               # largest finite
    (0xFE, -448.0),
    (0x08, 2.0 ** -6),           # smallest normal
    (0x07, 7 * 2.0 ** -9),       # largest subnormal
    (0x01, 2.0 ** -9),           # smallest subnormal
    (0x38, 1.0),
    (0xB8, -1.0),
    (0x39, 1.125),
    (0x40, 2.0),
    (0x00, 0.0),
])
def test_e4m3_closed_forms(code, value):
    assert oracle.e4m3_value(np.uint8(code)) == value


def test_e4m3_rejects_non_bytes():
    with pytest.raises(ValueError):
        oracle.e4m3_value(np.array([256]))


def test_encoder_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    vals = oracle.e4m3_value(codes)
    assert np.array_equal(synth.e4m3_round_codes(vals), codes)
    # midpoints between neighbouring positive codes go to the even code
    pos = oracle.e4m3_value(np.arange(127, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = synth.e4m3_round_codes(mids)
    lo = np.arange(126)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    with pytest.raises(ValueError):
        synth.e4m3_round_codes([449.0])


def test_encoder_matches_torch_conversion():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.standard_normal(20000) * 40,
                        rng.standard_normal(5000) * 2.0 ** -7]).clip(-448, 448)
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = synth.e4m3_round_codes(x)
    nz = ref != 0x80                 # torch keeps the sign of a zero; the generator does not
    assert np.array_equal(ours[nz], ref[nz])


def test_draw_inputs_fp8_recipe():
    d = synth.draw_inputs_fp8(2, 3, 64, 128, seed=11)
    for name in ("q", "k", "v"):
        assert d[name].dtype == np.uint8 and d[name].shape == (2, 3, 64, 128)
        vals = oracle.e4m3_value(d[name])
        assert np.isfinite(vals).all()
        assert np.abs(vals).max() == 448.0      # the largest magnitude maps to 448
        assert d[name + "_descale"] == float(np.float32(d[name + "_descale"]))
    # the descaled values are the N(0, 1) draws up to E4M3 rounding (3 mantissa bits)
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.standard_normal((2, 3, 64, 128), dtype=np.float32).astype(np.float64)
    deq = oracle.dequantize(d["q"], d["q_descale"])
    big = np.abs(x) > 0.1
    assert np.abs(deq[big] - x[big]).max() <= 2.0 ** -4 * np.abs(x[big]).max()


def test_head_forward_fp8_closed_form():
    # q = [1, 0] * 0.5; keys [2, 0] * 0.25 and [0, 0]; values [1, -1] * 3 and [0.5, 2] * 3
    q8 = np.array([[0x38, 0x00]], np.uint8)
    k8 = np.array([[0x40, 0x00], [0x00, 0x00]], np.uint8)
    v8 = np.array([[0x38, 0xB8], [0x30, 0x40]], np.uint8)
    allowed = np.ones((1, 2), bool)
    o, lse, p = oracle.head_forward_fp8(q8, k8, v8, 0.5, 0.5, 0.25, 3.0, allowed)
    s0 = 0.5 * (1 * 0.5) * (2 * 0.25)           # 0.125; the other score is 0
    w0, w1 = math.exp(s0), 1.0
    t = w0 + w1
    assert abs(lse[0] - math.log(t)) < 1e-15
    assert abs(p[0, 0] - w0 / t) < 1e-15
    assert abs(o[0, 0] - (w0 * 3 + w1 * 1.5) / t) < 1e-14
    assert abs(o[0, 1] - (w0 * -3 + w1 * 6) / t) < 1e-14


def test_head_forward_fp8_descale_invariants():
    rng = np.random.default_rng(2)
    q8, k8, v8 = (synth.e4m3_round_codes(rng.standard_normal((40, 64)) * 50) for _ in range(3))
    allowed = oracle.allowed_mask(40, 40, True)
    o, lse, _ = oracle.head_forward_fp8(q8, k8, v8, 0.125, 0.02, 0.03, 0.05, allowed)
    # V's descale scales O and nothing else (a power of two: exactly)
    o2, lse2, _ = oracle.head_forward_fp8(q8, k8, v8, 0.125, 0.02, 0.03, 0.1, allowed)
    assert np.array_equal(o2, 2 * o) and np.array_equal(lse2, lse)
    # a factor moved between the softmax scale and Q's descale changes nothing
    o3, lse3, _ = oracle.head_forward_fp8(q8, k8, v8, 0.25, 0.01, 0.03, 0.05, allowed)
    assert np.abs(o3 - o).max() < 1e-13 and np.abs(lse3 - lse).max() < 1e-13
    # row 0 under the causal mask sees only key 0: O = V[0] exactly dequantised
    assert np.array_equal(o[0], oracle.dequantize(v8[0], 0.05))


def test_head_forward_fp8_matches_torch_sdpa():
    F = torch.nn.functional
    rng = np.random.default_rng(8)
    q8, k8, v8 = (synth.e4m3_round_codes(rng.standard_normal((70, 32)) * 60) for _ in range(3))
    qd, kd, vd, scale = 0.011, 0.013, 0.017, 0.177
    for causal in (False, True):
        allowed = oracle.allowed_mask(70, 70, causal)
        o, _, _ = oracle.head_forward_fp8(q8, k8, v8, scale, qd, kd, vd, allowed)
        q, k, v = (torch.from_numpy(oracle.e4m3_value(x) * float(np.float32(s)))
                   for x, s in ((q8, qd), (k8, kd), (v8, vd)))
        ref = F.scaled_dot_product_attention(q[None], k[None], v[None],
                                             attn_mask=torch.from_numpy(allowed)[None],
                                             scale=float(np.float32(scale)))[0].numpy()
        assert np.abs(o - ref).max() < 1e-12
