"""GPU parity of the split-KV forward (fa_fwd_splitkv) against the fp64 oracle
(the plain definition over all keys: the merge of split results is exact up to
rounding) and against the unsplit forward.  Tolerances as the plain path."""

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
    # B, H, Nq, Nk, d, mask, num_splits (0 = automatic)
    (2, 4, 1, 4096, 128, "causal", 0),
    (1, 2, 16, 2000, 64, "causal", 7),       # ragged cache, explicit count
    (1, 2, 130, 1000, 128, "dense", 3),      # two query blocks
    (1, 2, 5, 600, 64, "blocksparse", 0),
    (1, 1, 1, 70, 128, "dense", 1000),       # more splits asked than tiles
    (2, 2, 40, 30, 64, "causal", 2),         # more queries than keys: empty rows
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}Nq{c[2]}Nk{c[3]}d{c[4]}-{c[5]}-s{c[6]}"
                                             for c in CASES])
def test_splitkv_parity(fa, case):
    torch = torch_mod()
    B, H, Nq, Nk, d, kind, splits = case
    seed = 900 + Nq + Nk
    bits = synth.draw_inputs_nqk(B, H, Nq, Nk, d, seed)
    causal = kind == "causal"
    bm = None
    if kind == "blocksparse":
        bm = (np.random.default_rng(seed).random((-(-Nq // 128), -(-Nk // 128))) < 0.5)
        bm = bm.astype(np.uint8)
        bm[:, 0] = 1
    scale = float(np.float32(d ** -0.5))
    q, k, v = (to_gpu(bits[x]) for x in ("q", "k", "v"))
    bmg = mask_to_gpu(bm)
    o, lse = fa.forward_splitkv(q, k, v, scale, causal, bmg, 128, num_splits=splits)
    o1, l1 = fa.forward(q, k, v, scale, causal, bmg, 128)
    torch.cuda.synchronize()
    allowed = oracle.allowed_mask(Nq, Nk, causal, bm, 128)
    for b in range(B):
        for h in range(H):
            qq, kk, vv = (synth.bf16_bits_to_f64(bits[x][b, h]) for x in ("q", "k", "v"))
            ro, rl, _ = oracle.head_forward(qq, kk, vv, scale, allowed)
            e_o = rel_err(from_gpu(o[b, h]), ro)
            e_l = lse_err(lse[b, h].cpu().numpy(), rl)
            print(f"{case} head ({b},{h}): o={e_o:.2e} lse={e_l:.2e}", flush=True)
            assert e_o <= TOL_REL and e_l <= TOL_LSE, (e_o, e_l)
    # against the unsplit kernel (both rounded to bf16 from fp32)
    assert rel_err(from_gpu(o), from_gpu(o1)) <= TOL_REL
    dead = ~allowed.any(1)
    if dead.any():
        assert np.all(from_gpu(o)[:, :, dead] == 0)
        assert np.all(lse.cpu().numpy()[:, :, dead] == -np.inf)


def test_splitkv_one_split_is_the_plain_forward(fa):
    torch = torch_mod()
    bits = synth.draw_inputs_nqk(1, 2, 3, 500, 128, 3)
    q, k, v = (to_gpu(bits[x]) for x in ("q", "k", "v"))
    o, l = fa.forward_splitkv(q, k, v, 0.1, True, num_splits=1)
    o1, l1 = fa.forward(q, k, v, 0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(l, l1)


def test_splitkv_deterministic(fa):
    torch = torch_mod()
    bits = synth.draw_inputs_nqk(2, 2, 1, 3000, 64, 4)
    q, k, v = (to_gpu(bits[x]) for x in ("q", "k", "v"))
    a = fa.forward_splitkv(q, k, v, 0.1, True)
    b = fa.forward_splitkv(q, k, v, 0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
