"""The comparison gates themselves (CPU): what they accept and what they must reject.

The fp32 gate has a pair-relative part and an element-relative part (tests/parity.py).  The
element part exists to catch a rotation computed with fp32 cos/sin: such errors (~1 fp32 ulp of
cos/sin, a few 1e-8 of the pair norm) stay inside the pair-relative bound but are far above 2e-6 of
an element that cancels to a small fraction of its pair norm.  The red arm below is a textbook
rotate-half written here in numpy float32 (angle, cos, sin, products and sum all fp32).
"""
import numpy as np

import oracle
from canvas_rope_rotary_amd import synth
from parity import check_bf16, check_fp32, elem_rel_err, pair_rel_err


def _batch():
    b = synth.random_batch(71, 24, max_len=600, dtype="f32")
    x, _ = b.qk()
    pl, *_ = oracle.planes(b.ids, b.cu_seqlens, synth.IMAGE_ID)
    return x, pl


def _fp32_rotation(x, planes, theta=1e7):
    """Rotate-half with cos, sin, products and sums in float32 (the red arm).  The angle is the
    oracle's (the same fp32 table and one fp32 multiply), so only the fp32 trigonometry and
    arithmetic differ."""
    inv = oracle.inv_freq(theta)
    sel = np.array([1 if (j % 3 == 1 and j < 33) else 2 if (j % 3 == 2 and j < 30) else 0 for j in range(32)])
    pos = planes[sel].T.astype(np.float32)                 # [T, 32]
    ang = (pos * inv[None, :]).astype(np.float32)
    c, s = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    y = x.copy()
    x1, x2 = x[..., :32], x[..., 32:64]
    y[..., :32] = x1 * c[:, None, :] - x2 * s[:, None, :]
    y[..., 32:64] = x2 * c[:, None, :] + x1 * s[:, None, :]
    return y


def test_fp32_gate_accepts_the_oracle_and_one_ulp_moves():
    x, pl = _batch()
    ref = oracle.rotate(x, pl)
    ok, info = check_fp32(ref, ref)
    assert ok and info["max_elem_rel"] == 0.0
    moved = np.nextafter(ref, np.float32(np.inf)).astype(np.float32)
    moved[..., 64:] = ref[..., 64:]
    ok, info = check_fp32(moved, ref)
    assert ok, info                                   # one fp32 ulp is 2^-23 of the value at most


def test_fp32_rotation_fails_the_element_gate_only():
    x, pl = _batch()
    ref = oracle.rotate(x, pl)
    red = _fp32_rotation(x, pl)
    assert float(pair_rel_err(red, ref).max()) <= 2e-6          # inside the pair-relative bound
    ok, info = check_fp32(red, ref)
    assert not ok and info["max_pair_rel"] <= 2e-6 and info["max_elem_rel"] > 2e-6, info
    assert int((elem_rel_err(red, ref) > 2e-6).sum()) > 100     # not a single stray element


def test_fp32_gate_rejects_a_changed_tail_and_a_nonzero_zero_pair():
    x, pl = _batch()
    ref = oracle.rotate(x, pl)
    bad = ref.copy()
    bad[3, 1, 200] = np.nextafter(bad[3, 1, 200], np.float32(np.inf))
    assert not check_fp32(bad, ref)[0]
    z = np.zeros((1, 1, 64), np.float32)
    zz = z.copy()
    zz[0, 0, 5] = 1e-30
    assert check_fp32(z, z)[0] and not check_fp32(zz, z)[0]


def test_bf16_gate_is_one_ulp_with_signed_zero():
    ref = np.array([[[0x3F80, 0x8000, 0x0000, 0xBF80] + [0] * 60]], np.uint16)
    ok, _ = check_bf16(ref, ref)
    assert ok
    one = ref.copy()
    one[0, 0, 0] += 1                       # next value up
    one[0, 0, 1] = 0x0000                   # -0 and +0 are the same point
    assert check_bf16(one, ref)[0]
    two = ref.copy()
    two[0, 0, 3] += 2
    assert not check_bf16(two, ref)[0]
    cross = ref.copy()
    cross[0, 0, 2] = 0x8001                 # the smallest negative: one step below +0
    assert check_bf16(cross, ref)[0]
