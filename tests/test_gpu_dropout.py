"""GPU parity of the dropout path (fa_fwd_dropout, fa_bwd_dropout,
fa_dropout_keep_mask) against the fp64 dropout oracle.

The keep mask is integer work and is compared bit for bit.  O, dQ, dK, dV use
the tolerances of the plain path (max|gpu - ref| / max|ref| <= 1e-2; the
probabilities scaled by 1/(1-p) are rounded to bf16 like P); LSE is the plain
softmax's and keeps its 1e-3 absolute bound.
"""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import (TOL_LSE, TOL_REL, from_gpu, lse_err, mask_to_gpu, rel_err, to_gpu,
                      torch_mod)
from test_gpu_parity import _mask_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_62_amd as fa
    fa.load_library()
    return fa


@pytest.mark.parametrize("B,H,N,p,seed,offset", [
    (1, 2, 128, 0.5, 1, 0),
    (2, 3, 130, 0.1, (7 << 32) + 3, 9),       # ragged N, seed with a high word
    (1, 1, 67, 0.9, 123456789, 4294967295),
])
def test_keep_mask_bitwise(fa, B, H, N, p, seed, offset):
    torch = torch_mod()
    keep = fa.dropout_keep_mask(B, H, N, p, seed, offset).cpu().numpy()
    torch.cuda.synchronize()
    for bh in range(B * H):
        ref = oracle.keep_mask(N, N, bh, p, seed, offset)
        assert np.array_equal(keep.reshape(B * H, N, N)[bh].astype(bool), ref), bh


def _p_bracket(h: int):
    """float32 probabilities p_keep, p_drop whose thresholds floor(p * 2^16) are just
    h (keep a 16-bit draw h) and h + 1 (drop it)."""
    lo = np.float32(h / 65536.0)
    hi = np.float32((h + 1) / 65536.0)
    assert int(np.floor(float(lo) * 65536.0)) == h
    assert int(np.floor(float(hi) * 65536.0)) == h + 1
    return float(lo), float(hi)


def test_keep_bits_follow_published_philox_words(fa):
    """Queries 0, 1 and keys 0..3 of head 0 with seed 0 and offset 0 form the block of
    the zero counter under the zero key, whose published output words are in
    tests/golden/philox_kat.json.  Element (i, j) takes 16-bit half e mod 2 of word
    e div 2, e = 4 i + j.  For each element, the threshold equal to its half keeps
    it and the next one drops it: the GPU generator and its half-word layout are
    pinned to the published output independently of the oracle."""
    import json
    import os
    torch = torch_mod()
    with open(os.path.join(os.path.dirname(__file__), "golden", "philox_kat.json")) as f:
        vec = json.load(f)["vectors"][0]
    assert vec["counter"] == ["00000000"] * 4 and vec["key"] == ["00000000"] * 2
    words = [int(x, 16) for x in vec["output"]]
    for i in range(2):
        for j in range(4):
            e = 4 * i + j
            h = (words[e // 2] >> (16 * (e % 2))) & 0xFFFF
            if h == 0xFFFF:
                continue   # no p < 1 drops the largest draw
            p_keep, p_drop = _p_bracket(h)
            kept = fa.dropout_keep_mask(1, 1, 4, p_keep, 0, 0).cpu().numpy().reshape(4, 4)
            dropped = fa.dropout_keep_mask(1, 1, 4, p_drop, 0, 0).cpu().numpy().reshape(4, 4)
            torch.cuda.synchronize()
            assert kept[i, j] == 1, (i, j, hex(h), p_keep)
            assert dropped[i, j] == 0, (i, j, hex(h), p_drop)


CASES = [
    # B, H, N, d, mask, p
    (1, 2, 128, 64, "dense", 0.5),
    (2, 2, 384, 128, "dense", 0.1),
    (2, 2, 448, 128, "causal", 0.2),
    (1, 3, 320, 64, "causal", 0.5),
    (2, 2, 200, 64, "dense", 0.3),          # ragged tail
    (1, 2, 333, 128, "causal", 0.25),       # ragged + causal
    (1, 2, 512, 64, "butterfly", 0.4),
    (1, 2, 640, 128, "random_holes", 0.15),
]


def _check(out, bits, b, h, scale, causal, bm, p, seed, offset, H, tag):
    q, k, v, do = (synth.bf16_bits_to_f64(bits[x][b, h]) for x in ("q", "k", "v", "do"))
    N = q.shape[0]
    allowed = oracle.allowed_mask(N, N, causal, bm, 128)
    keep = oracle.keep_mask(N, N, b * H + h, p, seed, offset)
    o, lse, _, _ = oracle.head_forward_dropout(q, k, v, scale, allowed, p, keep)
    dq, dk, dv = oracle.head_backward_dropout(q, k, v, do, scale, allowed, p, keep)
    errs = {"o": rel_err(from_gpu(out["o"][b, h]), o),
            "lse": lse_err(out["lse"][b, h].cpu().numpy(), lse),
            "dq": rel_err(from_gpu(out["dq"][b, h]), dq),
            "dk": rel_err(from_gpu(out["dk"][b, h]), dk),
            "dv": rel_err(from_gpu(out["dv"][b, h]), dv)}
    print(f"{tag} head ({b},{h}) errors: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for name, e in errs.items():
        assert e <= (TOL_LSE if name == "lse" else TOL_REL), (name, e)


def _run(fa, bits, scale, causal, bm, p, seed, offset):
    torch = torch_mod()
    q, k, v, do = (to_gpu(bits[x]) for x in ("q", "k", "v", "do"))
    bmg = mask_to_gpu(bm)
    o, lse = fa.forward(q, k, v, scale, causal, bmg, 128, dropout_p=p, seed=seed, offset=offset)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, causal, bmg, 128, dropout_p=p,
                             seed=seed, offset=offset)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}N{c[2]}d{c[3]}-{c[4]}-p{c[5]}"
                                             for c in CASES])
def test_dropout_whole_tensor(fa, case):
    B, H, N, d, kind, p = case
    seed, offset = 1000 + N + d, 17
    rng = np.random.default_rng(seed)
    causal, bm = _mask_for(kind, N, 128, rng)
    bits = synth.draw_inputs(B, H, N, d, seed)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    out = _run(fa, bits, scale, causal, bm, p, seed, offset)
    for b in range(B):
        for h in range(H):
            _check(out, bits, b, h, scale, causal, bm, p, seed, offset, H, str(case))


def test_dropout_full_size_c3(fa):
    """C3 with p = 0.1, every head against the dropout oracle."""
    cfg = synth.CONFIGS["C3"]
    bits = synth.config_inputs(cfg)
    p, seed, offset = 0.1, 20261202, 5
    out = _run(fa, bits, cfg.scale, True, None, p, seed, offset)
    for bh in range(cfg.B * cfg.H):
        b, h = divmod(bh, cfg.H)
        _check(out, bits, b, h, cfg.scale, True, None, p, seed, offset, cfg.H, "C3-dropout")


def test_dropout_deterministic_and_stream_dependent(fa):
    torch = torch_mod()
    B, H, N, d = 1, 2, 256, 64
    bits = synth.draw_inputs(B, H, N, d, 3)
    a = _run(fa, bits, 0.125, True, None, 0.3, 5, 1)
    b = _run(fa, bits, 0.125, True, None, 0.3, 5, 1)
    c = _run(fa, bits, 0.125, True, None, 0.3, 5, 2)
    assert all(torch.equal(a[k], b[k]) for k in a)
    assert not torch.equal(a["o"], c["o"])
    assert torch.equal(a["lse"], c["lse"])       # LSE does not see the dropout


def test_dropout_zero_is_the_plain_path(fa):
    """fa_fwd_dropout / fa_bwd_dropout with p = 0 give fa_fwd / fa_bwd's bits."""
    torch = torch_mod()
    B, H, N, d = 1, 2, 200, 128
    bits = synth.draw_inputs(B, H, N, d, 4)
    q, k, v, do = (to_gpu(bits[x]) for x in ("q", "k", "v", "do"))
    lib = fa.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    o0, l0 = fa.forward(q, k, v, 0.1, True)
    g0 = fa.backward(q, k, v, o0, do, l0, 0.1, True)
    o1, l1 = torch.empty_like(q), torch.empty_like(l0)
    assert lib.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, 0.1, 1,
                              None, 128, 0.0, 9, 9, o1.data_ptr(), l1.data_ptr(), stream) == 0
    g1 = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=q.device)
    assert lib.fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(),
                              do.data_ptr(), l1.data_ptr(), B, H, N, d, 0.1, 1, None, 128, 0.0,
                              9, 9, g1[0].data_ptr(), g1[1].data_ptr(), g1[2].data_ptr(),
                              ws.data_ptr(), ws.numel(), stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    assert all(torch.equal(x, y) for x, y in zip(g0, g1))


@pytest.mark.parametrize("d,N,causal", [(128, 256, True), (128, 256, False), (64, 192, True),
                                        (64, 192, False)])
def test_forward_zeroes_exactly_the_dropped_entries(fa, d, N, causal):
    """Element-by-element check of the keep rule as the forward applies it.

    With V rows s..s+d-1 set to the unit vectors and every other row 0,
    O[i, c] = keep(i, s + c) P(i, s + c) / (l_i (1 - p)), which is nonzero
    exactly when key s + c is visible to query i and kept: the zero pattern
    of O is the keep mask of those d keys, with no tolerance involved.
    """
    torch = torch_mod()
    B, H, p, seed, offset = 1, 2, 0.3, 77, 3
    bits = synth.draw_inputs(B, H, N, d, 11)
    q, k = to_gpu(bits["q"]), to_gpu(bits["k"])
    allowed = oracle.allowed_mask(N, N, causal, None, 128)
    for s in range(0, N, d):
        v = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device=q.device)
        v[:, :, s:s + d, :] = torch.eye(d, dtype=torch.bfloat16, device=q.device)
        o, _ = fa.forward(q, k, v, 1.0 / d ** 0.5, causal, None, 128, dropout_p=p, seed=seed,
                          offset=offset)
        torch.cuda.synchronize()
        nz = (o.float() != 0).cpu().numpy()
        for bh in range(B * H):
            b, h = divmod(bh, H)
            keep = oracle.keep_mask(N, N, bh, p, seed, offset)
            want = (allowed & keep)[:, s:s + d]
            bad = np.argwhere(nz[b, h] != want)
            assert bad.size == 0, (s, bh, bad[:5].tolist())
