"""The seeded input generators (synth/): stream identity, ranges, moments."""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import synth


def test_mt19937_standard_value():
    # The C++ standard requires the 10000th draw of a default-seeded
    # (seed 5489) mt19937 to be 4123659995; the first is 3499211612.
    d = synth.mt19937_draws(5489, 10000)
    assert d[0] == 3499211612
    assert d[-1] == 4123659995


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_mt19937_matches_std_mt19937():
    prog = r"""
    #include <random>
    #include <cstdio>
    int main() {
        for (unsigned s = 0; s < 5; ++s) {
            std::mt19937 g(s);
            for (int i = 0; i < 2000; ++i) std::printf("%u\n", (unsigned)g());
        }
    }
    """
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mt.cpp")
        exe = os.path.join(d, "mt")
        open(src, "w").write(prog)
        subprocess.run(["g++", "-O1", src, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    ref = np.array([int(x) for x in out], dtype=np.uint64).reshape(5, 2000)
    for s in range(5):
        assert np.array_equal(synth.mt19937_draws(s, 2000).astype(np.uint64), ref[s])


def test_uniform_exact_and_in_range():
    d = np.array([0, 0xFFFFFFFF, 0x80000000, 0x00000100], dtype=np.uint32)
    v = synth.uniform_values(d)
    assert v.dtype == np.float32
    assert v[0] == -1.0
    assert v[1] == np.float32(1.0 - 2.0**-23)
    assert v[2] == 0.0
    assert v[3] == np.float32(-1.0 + 2.0**-23)
    many = synth.uniform_values(synth.mt19937_draws(0, 100000))
    assert many.min() >= -1.0 and many.max() < 1.0
    assert abs(float(many.mean())) < 0.01
    # every value is a multiple of 2**-23, exactly representable
    assert np.all((many.astype(np.float64) * 2.0**23) % 1.0 == 0.0)


def test_integer_values():
    v = synth.integer_values(synth.mt19937_draws(0, 90000))
    assert set(np.unique(v).tolist()) == set(float(x) for x in range(-4, 5))


def test_normal_moments():
    v = synth.normal_values(synth.mt19937_draws(3, 4 * 200000), 0.5).astype(np.float64)
    assert abs(v.mean()) < 0.005
    assert abs(v.std() - 0.5) < 0.005
    with pytest.raises(ValueError):
        synth.normal_values(np.zeros(3, dtype=np.uint32), 1.0)


def test_eighths_pattern():
    # a[i] = ((17 i) mod 13 - 6) / 8 and b[i] = ((29 i) mod 11 - 5) / 8
    a = synth.eighths_a(30)
    b = synth.eighths_b(30)
    for i in range(30):
        assert a[i] == ((17 * i) % 13 - 6) / 8
        assert b[i] == ((29 * i) % 11 - 5) / 8


def test_make_inputs_layout_and_reproducibility():
    A, B = synth.make_inputs(3, 5, 4, "uniform", seed=7)
    assert A.shape == (3, 5) and B.shape == (5, 4)
    assert A.flags.c_contiguous and B.flags.c_contiguous
    d = synth.uniform_values(synth.mt19937_draws(7, 35))
    assert np.array_equal(A.ravel(), d[:15]) and np.array_equal(B.ravel(), d[15:])
    A2, B2 = synth.make_inputs(3, 5, 4, "uniform", seed=7)
    assert np.array_equal(A, A2) and np.array_equal(B, B2)


def test_workloads_table():
    w = synth.WORKLOADS["leetgpu8192"]
    assert (w.M, w.N, w.K, w.dist, w.seed) == (8192, 6144, 4096, "normal", 3)
    assert w.flops == 412316860416
    assert w.algorithmic_bytes == 436207616
    assert synth.WORKLOADS["ragged1023"].flops == 2153773050
    g = synth.WORKLOADS["gemv8192"]
    assert g.algorithmic_bytes == 268500992
