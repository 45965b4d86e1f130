"""Host-side parts of bench.py that need no GPU: the FLOP accounting's mask
fractions, the source hash that ties stored counters to the code they were
measured on, and the single-GPU guard."""

import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_mask_fractions():
    assert bench.mask_fraction(synth.CONFIGS["C2"]) == 1.0
    assert bench.mask_fraction(synth.CONFIGS["C3"]) == 0.5
    assert bench.mask_fraction(synth.CONFIGS["C4"]) == 0.5
    # butterfly over 32 blocks: the diagonal plus five powers of two per row
    assert bench.mask_fraction(synth.CONFIGS["C5"]) == pytest.approx(6 / 32)


def test_code_only_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles x\n  return 2 * x; /* no overflow\n check */ }\n"
    b = "int f(int x) { return 2 * x; }"
    c = "int f(int x) { return 3 * x; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(b) != bench._code_only(c)


def test_source_hash_is_stable():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
