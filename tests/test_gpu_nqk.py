"""GPU parity for N_q != N_k (fa_fwd_nqk, fa_bwd_nqk) against the fp64 oracle,
causal mask aligned bottom-right.  Same tolerances as the square path."""

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL_LSE, TOL_REL, from_gpu, lse_err, mask_to_gpu, rel_err, to_gpu, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import exact_io_aware_62_amd as fa
    fa.load_library()
    return fa


CASES = [
    # B, H, Nq, Nk, d, mask
    (2, 2, 1, 2048, 128, "causal"),        # one decoding step over a long cache
    (1, 3, 7, 300, 64, "causal"),          # a few new tokens
    (2, 2, 100, 37, 64, "causal"),         # more queries than keys: empty leading rows
    (1, 2, 300, 40, 128, "causal"),        # whole query blocks without a key (no key tile)
    (1, 2, 200, 60, 64, "causal"),
    (1, 2, 256, 512, 128, "dense"),
    (2, 1, 200, 333, 128, "causal"),
    (1, 2, 130, 260, 64, "blocksparse"),
    (1, 2, 333, 130, 128, "dense"),
    # more than 64 mask blocks along the axis a kernel walks: the tile skipping reads
    # the mask 64 blocks at a time and has to move to the next window (keys for the
    # forward and dQ, queries for dK/dV); sparse rows with active blocks on both
    # sides of the window edge and long inactive runs
    (1, 2, 256, 128 * 72, 64, "blocksparse_wide"),
    (1, 2, 128 * 72, 256, 64, "blocksparse_wide"),
    (1, 1, 128 * 70 + 50, 128 * 66 + 7, 128, "blocksparse_wide_causal"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}Nq{c[2]}Nk{c[3]}d{c[4]}-{c[5]}"
                                             for c in CASES])
def test_nqk_parity(fa, case):
    torch = torch_mod()
    B, H, Nq, Nk, d, kind = case
    seed = 500 + Nq + Nk
    bits = synth.draw_inputs_nqk(B, H, Nq, Nk, d, seed)
    causal = kind.endswith("causal")
    bm = None
    if kind == "blocksparse":
        bm = (np.random.default_rng(seed).random((-(-Nq // 128), -(-Nk // 128))) < 0.6)
        bm = bm.astype(np.uint8)
        bm[0, 0] = 1
    elif kind.startswith("blocksparse_wide"):
        nbq, nbk = -(-Nq // 128), -(-Nk // 128)
        bm = (np.random.default_rng(seed).random((nbq, nbk)) < 0.08).astype(np.uint8)
        # blocks just before and after the 64-block window edges, in rows and columns
        for i in range(nbq):
            for j in (0, 63, 64, nbk - 1):
                if j < nbk and (i + j) % 3 == 0:
                    bm[i, j] = 1
        for j in range(nbk):
            for i in (0, 63, 64, nbq - 1):
                if i < nbq and (i + j) % 2 == 0:
                    bm[i, j] = 1
        bm[:, min(nbk - 1, 5):min(nbk, 60)] = 0 if nbk > 66 else bm[:, min(nbk - 1, 5):min(nbk, 60)]
        if nbq > 66:
            bm[5:60, :] = 0         # a long run of inactive query blocks in every column
    scale = float(np.float32(d ** -0.5))
    q, k, v, do = (to_gpu(bits[x]) for x in ("q", "k", "v", "do"))
    bmg = mask_to_gpu(bm)
    o, lse = fa.forward(q, k, v, scale, causal, bmg, 128)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, causal, bmg, 128)
    torch.cuda.synchronize()
    allowed = oracle.allowed_mask(Nq, Nk, causal, bm, 128)
    for b in range(B):
        for h in range(H):
            qq, kk, vv, dd = (synth.bf16_bits_to_f64(bits[x][b, h]) for x in ("q", "k", "v", "do"))
            ro, rl, _ = oracle.head_forward(qq, kk, vv, scale, allowed)
            rq, rk, rv = oracle.head_backward(qq, kk, vv, dd, scale, allowed)
            errs = {"o": rel_err(from_gpu(o[b, h]), ro),
                    "lse": lse_err(lse[b, h].cpu().numpy(), rl),
                    "dq": rel_err(from_gpu(dq[b, h]), rq),
                    "dk": rel_err(from_gpu(dk[b, h]), rk),
                    "dv": rel_err(from_gpu(dv[b, h]), rv)}
            print(f"{case} head ({b},{h}): " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()),
                  flush=True)
            for name, e in errs.items():
                assert e <= (TOL_LSE if name == "lse" else TOL_REL), (name, e)
    dead = ~allowed.any(1)
    if dead.any():
        assert np.all(from_gpu(o)[:, :, dead] == 0)
        assert np.all(lse.cpu().numpy()[:, :, dead] == -np.inf)
        assert np.all(from_gpu(dq)[:, :, dead] == 0)


def test_no_keys_and_no_queries(fa):
    torch = torch_mod()
    B, H, d = 1, 2, 64
    q = torch.randn(B, H, 70, d, device="cuda").bfloat16()
    empty = torch.empty(B, H, 0, d, device="cuda", dtype=torch.bfloat16)
    o, lse = fa.forward(q, empty, empty, 0.125, True)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isinf(lse).all()) and bool((lse < 0).all())
    # no queries: dK = dV = 0 over the keys
    k = torch.randn(B, H, 90, d, device="cuda").bfloat16()
    qe = torch.empty(B, H, 0, d, device="cuda", dtype=torch.bfloat16)
    le = torch.empty(B, H, 0, device="cuda", dtype=torch.float32)
    dq, dk, dv = fa.backward(qe, k, k, qe, qe, le, 0.125, False,
                             dk=torch.full_like(k, 7.0), dv=torch.full_like(k, 7.0))
    torch.cuda.synchronize()
    assert bool((dk == 0).all()) and bool((dv == 0).all())
    # no keys: dQ = 0 over the queries (the dQ kernel runs no key tile)
    for causal in (False, True):
        do = torch.randn_like(q)
        dq, dk, dv = fa.backward(q, empty, empty, o, do, lse, 0.125, causal,
                                 dq=torch.full_like(q, 7.0))
        torch.cuda.synchronize()
        assert bool((dq == 0).all())


def test_suffix_of_square_causal_on_gpu(fa):
    """Decoding the last rows against the cache gives the last rows of the square
    causal result (bitwise: same tiles, same order, same instructions per row)."""
    torch = torch_mod()
    B, H, N, d, n = 1, 2, 384, 128, 5
    bits = synth.draw_inputs(B, H, N, d, 8)
    q, k, v = (to_gpu(bits[x]) for x in ("q", "k", "v"))
    o_full, l_full = fa.forward(q, k, v, 0.09, True)
    o_dec, l_dec = fa.forward(q[:, :, N - n:].contiguous(), k, v, 0.09, True)
    torch.cuda.synchronize()
    e_o = rel_err(from_gpu(o_dec), from_gpu(o_full[:, :, N - n:]))
    e_l = float((l_dec - l_full[:, :, N - n:]).abs().max())
    assert e_o <= 1e-2 and e_l <= 1e-3, (e_o, e_l)
