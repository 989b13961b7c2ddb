"""Mutation check of the oracle pins: plant one plausible mistake at a time in a COPY of the oracle
source (CPU only), build it, and require the pin suite to fail on it.  The oracle itself is never
modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mrope_oracle.c")

# (name, text in the oracle source, replacement)
MUTANTS = [
    ("grid row/col swapped", "off[n][1] = k / 8; off[n][2] = k % 8;", "off[n][1] = k % 8; off[n][2] = k / 8;"),
    ("grid row index off by one", "off[n][1] = k / 8; off[n][2] = k % 8;", "off[n][1] = (k + 1) / 8; off[n][2] = (k + 1) % 8;"),
    ("<image> at (O,O,O)", "off[n][0] = 0; off[n][1] = -1; off[n][2] = -1;", "off[n][0] = 0; off[n][1] = 0; off[n][2] = 0;"),
    ("</image> one short", "off[n][0] = 0; off[n][1] = 8; off[n][2] = 8;", "off[n][0] = 0; off[n][1] = 7; off[n][2] = 7;"),
    ("newline dropped from the frame", "#define ORACLE_FRAME_LEN 67", "#define ORACLE_FRAME_LEN 66"),
    ("frame length ignored", "*start = origin + frame_len;", "*start = origin + ORACLE_FRAME_LEN;"),
    ("amount from the frame's own offsets", "int32_t n = canvas_offsets(off);\n    int32_t max_hw = 0;",
     "int32_t n = canvas_offsets(off);\n    if (frame_len < n) n = frame_len;\n    int32_t max_hw = 0;"),
    ("</image> kept in a short frame", "} else if (p >= start) {                        /* everything after the frame */",
     "} else if (p >= start && p - origin != 65) {"),
    ("amount + 1", "*amount = *start - (origin + max_hw + 1);", "*amount = *start - (origin + max_hw);"),
    ("text-only start 2^29", "#define ORACLE_TEXT_ONLY_START (1 << 30)", "#define ORACLE_TEXT_ONLY_START (1 << 29)"),
    ("last marker wins", "for (int32_t p = 0; p < n; ++p)\n        if (ids[p] == marker_id)\n            return p;",
     "int32_t last = -1;\n    for (int32_t p = 0; p < n; ++p)\n        if (ids[p] == marker_id)\n            last = p;\n    if (last >= 0) return last;"),
    ("H and W sections swapped", "if (j % 3 == 1 && j < 33) return 1;", "if (j % 3 == 1 && j < 33) return 2;"),
    ("sections in blocks", "if (j % 3 == 1 && j < 33) return 1;\n    if (j % 3 == 2 && j < 30) return 2;\n    return 0;",
     "return j < 11 ? 0 : (j < 22 ? 1 : 2);"),
    ("sign of sin flipped", "double r1 = x1 * c - x2 * s;", "double r1 = x1 * c + x2 * s;"),
    ("pairing j <-> j+16", "int32_t h = rot_dim / 2;\n    for (int32_t j = 0; j < h; ++j) {",
     "int32_t h = rot_dim / 4;\n    for (int32_t j = 0; j < rot_dim / 2; ++j) {"),
    ("exponent j/d", "(2.0 * j) / (double)rot_dim", "(1.0 * j) / (double)rot_dim"),
    ("angle in double", "float a = pos * inv_freq[j];\n        double c = cos((double)a), s = sin((double)a);",
     "double a = (double)pos * (1.0 / pow(theta_unused_marker, 0.0)) * inv_freq[j];\n        double c = cos(a), s = sin(a);"),
    ("passthrough dims zeroed", "y[d] = x[d];", "y[d] = 0.0f;"),
    ("bf16 rounds half up", "out[i] = (uint16_t)((u + 0x7fffu + lsb) >> 16);", "out[i] = (uint16_t)((u + 0x8000u + 0 * lsb) >> 16);"),
    ("decode ignores amount", "int32_t plane = pos[s] - amount[s];", "int32_t plane = pos[s];"),
    ("pieces ignore the carried origin", "int32_t o = (origin_in && origin_in[s] >= 0) ? origin_in[s] : -1;",
     "int32_t o = -1;"),
    ("per-sequence frame length ignored",
     "oracle_frame_scalars_len(o, oracle_seq_frame_len(frame_len_seq, s, frame_len), &st, &am);",
     "oracle_frame_scalars_len(o, frame_len, &st, &am);"),
    ("per-sequence frame lengths one sequence late",
     "int32_t f = frame_len_seq ? frame_len_seq[s] : 0;",
     "int32_t f = frame_len_seq ? frame_len_seq[s > 0 ? s - 1 : 0] : 0;"),
    ("unusable frame length kept", "if (f == 0 || f < 65 || f > 4096) return frame_len;",
     "if (f == 0) return frame_len;"),
    ("pieces ignore the position offset", "int32_t off = pos_offset ? pos_offset[s] : 0;", "int32_t off = 0;"),
    ("paged block and row swapped", "const int64_t block = slot / block_size, within = slot % block_size;",
     "const int64_t block = slot % block_size, within = slot / block_size;"),
    ("paged slot 0 skipped", "if (slot < 0 || slot >= num_blocks * (int64_t)block_size) continue;\n        const int64_t block",
     "if (slot <= 0 || slot >= num_blocks * (int64_t)block_size) continue;\n        const int64_t block"),
    ("decode V rotated like K", "if (v) memcpy(v_cache + dst, v + src, sizeof(float) * (size_t)head_dim);",
     "if (v) rotate_head(v + src, v_cache + dst, NULL, head_dim, rot_dim, thw, inv_freq);"),
]


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {name}"
    src = src.replace(old, new, 1)
    if "theta_unused_marker" in src:
        src = src.replace("theta_unused_marker", "2.0")
    c = tmp_path / "m.c"
    c.write_text(src)
    so = tmp_path / "libm.so"
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(so), str(c),
                    "-lm"], check=True, capture_output=True)
    return str(so)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    so = _build(tmp_path, name, old, new)
    env = dict(os.environ, MROPE_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant '{name}'\n{r.stdout[-2000:]}"
