"""The library can be loaded before the caller imports torch.

torch ships its own HIP runtime under the same soname as the system's, linked
by file name.  If libfa were loaded first, a second runtime would come in with
torch and launches on torch's streams would fail; load_library() therefore
imports torch before it loads libfa.  Checked in a fresh interpreter, since
the order only matters for the first load in a process.
"""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import exact_io_aware_62_amd as fa
fa.load_library()              # before the caller's own torch import
import numpy as np
import torch
import oracle, synth
bits = synth.draw_inputs(1, 2, 200, 64, 7)
dev = lambda x: torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16)
o, lse = fa.forward(dev(bits["q"]), dev(bits["k"]), dev(bits["v"]), 0.125, causal=True)
torch.cuda.synchronize()
f = {x: synth.bf16_bits_to_f64(bits[x]) for x in ("q", "k", "v")}
o_ref, _ = oracle.forward(f["q"], f["k"], f["v"], 0.125, causal=True)
got = synth.bf16_bits_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
err = np.abs(got - o_ref).max() / np.abs(o_ref).max()
print("rel err", err)
assert err <= 1e-2
print("LOAD_ORDER_OK")
"""


def test_library_loaded_before_torch():
    r = subprocess.run([sys.executable, "-c", _SCRIPT, ROOT], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0 and "LOAD_ORDER_OK" in r.stdout, r.stdout + r.stderr
