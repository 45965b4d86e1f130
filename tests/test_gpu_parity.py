"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (stated here, applied per tensor): max|gpu - ref| / max|ref| <= 1e-2
for O, dQ, dK and dV; max|gpu - ref| <= 1e-3 (absolute) for LSE.  Both sides get
the same seeded bf16 bits from ``synth``.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL_LSE, TOL_REL, from_gpu, lse_err, mask_to_gpu, rel_err, to_gpu,
                      torch_mod)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_62_amd as fa
    fa.load_library()   # raises if libfa.so is missing: no fallback
    return fa


def run_gpu(fa, bits, scale, causal, bm, mb, backward=True):
    torch = torch_mod()
    q, k, v = (to_gpu(bits[x]) for x in ("q", "k", "v"))
    bmg = mask_to_gpu(bm)
    o, lse = fa.forward(q, k, v, scale, causal, bmg, mb)
    out = {"o": o, "lse": lse}
    if backward:
        do = to_gpu(bits["do"])
        out["dq"], out["dk"], out["dv"] = fa.backward(q, k, v, o, do, lse, scale, causal, bmg, mb)
    torch.cuda.synchronize()
    return out


def check_head(out, bits, b, h, scale, causal, bm, mb, backward=True, tag="", quiet=False):
    q, k, v, do = (synth.bf16_bits_to_f64(bits[x][b, h]) for x in ("q", "k", "v", "do"))
    N = q.shape[0]
    allowed = oracle.allowed_mask(N, N, causal, bm, mb)
    o_ref, lse_ref, _ = oracle.head_forward(q, k, v, scale, allowed)
    errs = {
        "o": rel_err(from_gpu(out["o"][b, h]), o_ref),
        "lse": lse_err(out["lse"][b, h].cpu().numpy(), lse_ref),
    }
    if backward:
        dq, dk, dv = oracle.head_backward(q, k, v, do, scale, allowed)
        errs["dq"] = rel_err(from_gpu(out["dq"][b, h]), dq)
        errs["dk"] = rel_err(from_gpu(out["dk"][b, h]), dk)
        errs["dv"] = rel_err(from_gpu(out["dv"][b, h]), dv)
    if not quiet:
        print(f"{tag} head ({b},{h}) errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
              flush=True)
    for name, e in errs.items():
        assert e <= (TOL_LSE if name == "lse" else TOL_REL), (name, e)
    return errs


# ---------------------------------------------------------------------------
# whole-tensor parity at sizes the oracle finishes in seconds: several tiles,
# ragged tails, every mask kind
# ---------------------------------------------------------------------------

SMALL = [
    # B, H, N, d, mask, mask_block
    (1, 2, 128, 64, "dense", 128),          # C1 shape
    (2, 3, 384, 64, "dense", 128),
    (2, 2, 384, 128, "dense", 128),
    (2, 2, 448, 128, "causal", 128),
    (1, 3, 320, 64, "causal", 128),
    (2, 2, 200, 64, "dense", 128),          # ragged tail
    (1, 2, 333, 128, "causal", 128),        # ragged + causal
    (1, 1, 1, 64, "dense", 128),            # single token
    (1, 1, 65, 128, "causal", 128),
    (1, 2, 130, 64, "butterfly", 128),      # ragged block-sparse
    (2, 2, 512, 64, "butterfly", 128),
    (1, 2, 640, 128, "random_holes", 128),  # empty block rows
    (1, 2, 640, 64, "random_causal", 128),
    (1, 2, 768, 64, "random", 256),         # mask granularity 256
    (1, 1, 512, 128, "random_holes_causal", 128),
]


def _mask_for(kind, N, mb, rng):
    nb = -(-N // mb)
    causal = kind.endswith("causal") or kind == "causal"
    if kind.startswith("random_holes"):
        bm = synth.make_blockmask("random_holes", nb, rng, 0.5)
    elif kind.startswith("random"):
        bm = synth.make_blockmask("random", nb, rng, 0.5)
    elif kind == "butterfly":
        bm = synth.butterfly_blockmask(nb)
    else:
        bm = None
    return causal, bm


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}-{c[4]}-mb{c[5]}"
                                             for c in SMALL])
def test_small_whole_tensor(fa, case):
    B, H, N, d, kind, mb = case
    seed = 77 + N + d
    rng = np.random.default_rng(seed)
    causal, bm = _mask_for(kind, N, mb, rng)
    if kind.startswith("random_holes"):
        bm[min(1, bm.shape[0] - 1)] = 0        # guarantee at least one empty block row
    bits = synth.draw_inputs(B, H, N, d, seed)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    out = run_gpu(fa, bits, scale, causal, bm, mb)
    for b in range(B):
        for h in range(H):
            check_head(out, bits, b, h, scale, causal, bm, mb, tag=str(case))
    if bm is not None:
        # empty rows: O = 0, LSE = -inf, dQ = 0 exactly
        allowed = oracle.allowed_mask(N, N, causal, bm, mb)
        dead = ~allowed.any(1)
        if dead.any():
            assert np.all(from_gpu(out["o"])[:, :, dead] == 0)
            assert np.all(out["lse"].cpu().numpy()[:, :, dead] == -np.inf)
            assert np.all(from_gpu(out["dq"])[:, :, dead] == 0)


# ---------------------------------------------------------------------------
# B*H a multiple of 32: the launches then take the XCD-grouped workgroup order
# (four heads at a time per XCD) in every kernel that uses it (dK/dV always;
# the forward and dQ when not causal).  Every head is compared with the oracle.
# ---------------------------------------------------------------------------

GROUPED = [
    # B, H, N, d, mask
    (2, 16, 384, 128, "dense"),
    (2, 16, 384, 64, "dense"),
    (2, 16, 512, 64, "butterfly"),
    (2, 16, 448, 128, "causal"),
]


@pytest.mark.parametrize("case", GROUPED, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}-{c[4]}"
                                               for c in GROUPED])
def test_grouped_order_every_head(fa, case):
    B, H, N, d, kind = case
    assert (B * H) % 32 == 0
    seed = 300 + N + d
    causal, bm = _mask_for(kind, N, 128, np.random.default_rng(seed))
    bits = synth.draw_inputs(B, H, N, d, seed)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    out = run_gpu(fa, bits, scale, causal, bm, 128)
    for b in range(B):
        for h in range(H):
            check_head(out, bits, b, h, scale, causal, bm, 128, tag=f"grouped {case}")


# ---------------------------------------------------------------------------
# scores that rise along the keys: the running row maximum moves by more than
# the kernels' rescale slack every few tiles, so the rarely taken rescale of the
# accumulated O (and of the row sum) runs many times per row
# ---------------------------------------------------------------------------

RISING = [
    # B, H, N, d, causal
    (1, 2, 704, 128, False),
    (1, 2, 640, 64, True),
    (2, 1, 333, 128, True),
]


@pytest.mark.parametrize("case", RISING, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}-{'causal' if c[4] else 'dense'}"
                                              for c in RISING])
def test_rising_scores_rescale(fa, case):
    B, H, N, d, causal = case
    bits = synth.draw_inputs(B, H, N, d, 600 + N)
    k = synth.bf16_bits_to_f64(bits["k"]).astype(np.float32)
    growth = (1.0 + np.arange(N, dtype=np.float32) / 48.0)[None, None, :, None]
    bits["k"] = synth.bf16_round_bits(k * growth)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    # the scores of the last keys are far above those of the first ones
    qf = synth.bf16_bits_to_f64(bits["q"][0, 0])
    kf = synth.bf16_bits_to_f64(bits["k"][0, 0])
    s = scale * qf @ kf.T * np.log2(np.e)
    assert s[:, -64:].max() - s[:, :64].max() > 16
    out = run_gpu(fa, bits, scale, causal, None, 128)
    for b in range(B):
        for h in range(H):
            check_head(out, bits, b, h, scale, causal, None, 128, tag=f"rising {case}")


# ---------------------------------------------------------------------------
# output rounding: bf16 round-to-nearest-even
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d", [64, 128])
def test_output_rounds_to_nearest_even(fa, d):
    """Q = 0 makes every score 0, so each of the N = 2 rows averages the two value
    rows with weights exactly 1/2.  Value row 1 is value row 0 plus one bf16 ulp (in
    magnitude), so every element of O is exactly the midpoint of two neighbouring bf16
    numbers.  Round-to-nearest-even gives the neighbour with an even last bit;
    truncation would give row 0's value and rounding half away from zero row 1's."""
    torch = torch_mod()
    rng = np.random.default_rng(4000 + d)
    x = rng.standard_normal(4 * d).astype(np.float32)
    x = x[np.abs(x) > 1e-2][:d]
    assert x.size == d
    v0 = synth.bf16_round_bits(x)                       # uint16 bit patterns
    v1 = (v0.astype(np.uint32) + 1).astype(np.uint16)   # one ulp up in magnitude
    even0 = (v0 & 1) == 0
    assert even0.any() and (~even0).any()               # both cases present
    bits = {
        "q": np.zeros((1, 1, 2, d), np.uint16),
        "k": synth.draw_inputs(1, 1, 2, d, 11)["k"],
        "v": np.stack([v0, v1])[None, None],
    }
    o, lse = fa.forward(to_gpu(bits["q"]), to_gpu(bits["k"]), to_gpu(bits["v"]),
                        float(np.float32(d ** -0.5)), False)
    torch.cuda.synchronize()
    got = o.view(torch.int16).cpu().numpy().view(np.uint16)[0, 0]
    want = np.where(even0, v0, v1)
    for row in range(2):
        assert np.array_equal(got[row], want), (row, got[row][got[row] != want])
    assert np.abs(lse.cpu().numpy() - np.log(2.0)).max() <= 1e-6


# ---------------------------------------------------------------------------
# the five workloads at full size, every head compared with the oracle
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_config_full_size(fa, name):
    cfg = synth.CONFIGS[name]
    bits = synth.config_inputs(cfg)
    bm = cfg.blockmask()
    out = run_gpu(fa, bits, cfg.scale, cfg.causal, bm, cfg.mask_block, backward=True)
    BH = cfg.B * cfg.H
    worst = {}
    for hh in range(BH):
        b, h = divmod(hh, cfg.H)
        errs = check_head(out, bits, b, h, cfg.scale, cfg.causal, bm, cfg.mask_block, tag=name,
                          quiet=BH > 16)
        for key, e in errs.items():
            worst[key] = max(worst.get(key, 0.0), e)
    print(f"{name}: all {BH} heads, largest errors: "
          + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)
    # every head: outputs finite, LSE finite (no empty rows in these workloads)
    torch = torch_mod()
    for key in ("o", "dq", "dk", "dv"):
        assert bool(torch.isfinite(out[key].float()).all()), key
    assert bool(torch.isfinite(out["lse"]).all())


# ---------------------------------------------------------------------------
# determinism and mask reductions (bitwise)
# ---------------------------------------------------------------------------

def _same(a, b):
    torch = torch_mod()
    return all(torch.equal(a[k], b[k]) for k in a)


def test_bitwise_deterministic(fa):
    torch = torch_mod()
    cfg = synth.CONFIGS["C3"]
    bits = synth.config_inputs(cfg)
    r1 = run_gpu(fa, bits, cfg.scale, True, None, 128)
    # unrelated work in between
    x = torch.randn(4096, 4096, device="cuda:0")
    (x @ x).sum().item()
    r2 = run_gpu(fa, bits, cfg.scale, True, None, 128)
    assert _same(r1, r2)
    cfg5 = synth.CONFIGS["C5"]
    bits5 = synth.config_inputs(cfg5)
    s1 = run_gpu(fa, bits5, cfg5.scale, False, cfg5.blockmask(), 128)
    s2 = run_gpu(fa, bits5, cfg5.scale, False, cfg5.blockmask(), 128)
    assert _same(s1, s2)


STAGED = [
    # B, H, N, d, mask
    (2, 2, 448, 128, "causal"),
    (2, 2, 200, 64, "dense"),
    (1, 2, 512, 64, "butterfly"),
    (1, 1, 333, 128, "random_holes_causal"),
]


@pytest.mark.parametrize("case", STAGED, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}-{c[4]}"
                                              for c in STAGED])
def test_stage_calls_match_fa_bwd_bitwise(fa, case):
    """fa_bwd (dQ with D formed inside, then dK/dV), fa_bwd_dq_dsum and the
    three separate stage calls all give the same bits."""
    torch = torch_mod()
    B, H, N, d, kind = case
    rng = np.random.default_rng(31)
    causal, bm = _mask_for(kind, N, 128, rng)
    bits = synth.draw_inputs(B, H, N, d, 31)
    s = float(np.float32(d ** -0.5))
    q, k, v, do = (to_gpu(bits[x]) for x in ("q", "k", "v", "do"))
    bmg = mask_to_gpu(bm)
    o, lse = fa.forward(q, k, v, s, causal, bmg, 128)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, s, causal, bmg, 128)
    dsum = fa.bwd_dsum(o, do)
    dk2, dv2 = fa.bwd_dkdv(q, k, v, do, lse, dsum, s, causal, bmg, 128)
    dq2 = fa.bwd_dq(q, k, v, do, lse, dsum, s, causal, bmg, 128)
    dq3, dsum3 = fa.bwd_dq_dsum(q, k, v, o, do, lse, s, causal, bmg, 128)
    torch.cuda.synchronize()
    assert torch.equal(dsum, dsum3)
    assert torch.equal(dq, dq2) and torch.equal(dq, dq3)
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_mask_reductions_bitwise(fa):
    B, H, N, d = 1, 2, 512, 128
    bits = synth.draw_inputs(B, H, N, d, 5)
    s = float(np.float32(d ** -0.5))
    nb = N // 128
    dense = run_gpu(fa, bits, s, False, None, 128)
    ones = run_gpu(fa, bits, s, False, synth.make_blockmask("ones", nb), 128)
    assert _same(dense, ones)
    causal = run_gpu(fa, bits, s, True, None, 128)
    lower = run_gpu(fa, bits, s, True, synth.make_blockmask("lower", nb), 128)
    assert _same(causal, lower)


def test_causal_no_future_leak(fa):
    B, H, N, d = 1, 2, 384, 64
    bits = synth.draw_inputs(B, H, N, d, 9)
    s = 0.125
    base = run_gpu(fa, bits, s, True, None, 128, backward=False)
    i = 200
    bits2 = {k: v.copy() for k, v in bits.items()}
    rng = np.random.default_rng(1)
    for key in ("k", "v"):
        noise = synth.bf16_round_bits(rng.standard_normal((B, H, N - i - 1, d)).astype(np.float32))
        bits2[key][:, :, i + 1:] = noise
    pert = run_gpu(fa, bits2, s, True, None, 128, backward=False)
    torch = torch_mod()
    assert torch.equal(base["o"][:, :, : i + 1], pert["o"][:, :, : i + 1])
    assert torch.equal(base["lse"][:, :, : i + 1], pert["lse"][:, :, : i + 1])
    assert not torch.equal(base["o"][:, :, i + 1:], pert["o"][:, :, i + 1:])


def test_identical_value_rows(fa):
    """V with identical rows gives O = that row for every query."""
    B, H, N, d = 1, 2, 256, 128
    bits = synth.draw_inputs(B, H, N, d, 21)
    bits["v"][:] = bits["v"][:, :, :1, :]
    out = run_gpu(fa, bits, 0.088, True, None, 128)
    o = from_gpu(out["o"])
    row = synth.bf16_bits_to_f64(bits["v"][:, :, :1, :])
    assert np.abs(o - row).max() <= 1e-2 * np.abs(row).max()


# ---------------------------------------------------------------------------
# a tensor of more than 2^31 elements: flat element offsets overflow int32
# ---------------------------------------------------------------------------

def test_offsets_past_2_31_elements(fa):
    """B=1, H=8200, N=2048, d=128, causal: 2.15e9 elements per tensor.  The head
    that starts past element 2^31, the last head and the first one match the oracle
    (fp64, the exact bf16 inputs copied back from the device)."""
    torch = torch_mod()
    B, H, N, d = 1, 8200, 2048, 128
    assert B * H * N * d > 2 ** 31
    scale = float(np.float32(d ** -0.5))
    x = synth.draw_inputs_device(B, H, N, d, 2031)
    o, lse = fa.forward(x["q"], x["k"], x["v"], scale, True)
    dq, dk, dv = fa.backward(x["q"], x["k"], x["v"], o, x["do"], lse, scale, True)
    torch.cuda.synchronize()
    first_past = -(-(2 ** 31) // (N * d))
    allowed = oracle.allowed_mask(N, N, True, None, 128)
    for h in (0, first_past, H - 1):
        qq, kk, vv, dd = (from_gpu(x[n][0, h]) for n in ("q", "k", "v", "do"))
        ro, rl, _ = oracle.head_forward(qq, kk, vv, scale, allowed)
        rq, rk, rv = oracle.head_backward(qq, kk, vv, dd, scale, allowed)
        errs = {"o": rel_err(from_gpu(o[0, h]), ro),
                "lse": lse_err(lse[0, h].cpu().numpy(), rl),
                "dq": rel_err(from_gpu(dq[0, h]), rq),
                "dk": rel_err(from_gpu(dk[0, h]), rk),
                "dv": rel_err(from_gpu(dv[0, h]), rv)}
        print(f"past-2^31 head {h}: " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()),
              flush=True)
        for name, e in errs.items():
            assert e <= (TOL_LSE if name == "lse" else TOL_REL), (h, name, e)
    del x, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
