"""The rotary kernels' sincos (canvas_rope_rotary_amd/csrc/mrope_math.h) compiled for the host and
checked against long-double libm over every angle fl32(fl32(pos) * inv_freq[j]) for pos in
[-1, 65536) and theta = 1e7, plus pseudo-random positions up to 2^24."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_sincos_within_2_double_ulp(tmp_path):
    exe = tmp_path / "sincos_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-o", str(exe),
                    os.path.join(ROOT, "tests", "host", "sincos_check.cpp")], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    worst_s, worst_c = float(out[0]), float(out[1])
    # 2 ulp of 1.0 in double is 4.4e-16
    assert worst_s < 4.4e-16 and worst_c < 4.4e-16, out
