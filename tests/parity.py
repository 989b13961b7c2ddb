"""Comparison gates for rotated Q/K (test helpers; no method arithmetic).

fp32 gate, two parts, both required:
  * pair-relative: for every rotated element, |got - ref| / ||(ref_j, ref_{j+32})||_2 <= 2e-6, the
    pair norm being that of the reference pair (it equals the input pair's norm, a rotation preserves
    it, so the bound never divides by a value near zero; a pair of zeros must come out exactly zero);
  * element-relative: |got - ref| <= 2e-6 * max(|ref|, 1e-6 * pair norm) for every rotated element --
    the maximum relative error of each element itself, with a floor far below any value an fp32
    computation of cos/sin could resolve.  A rotation whose cos/sin carry fp32 errors (~6e-8 of the
    pair norm) passes the first part and fails this one on every element that cancels below a few
    percent of its pair norm.
Dims past the rotary part must be bit-identical.

bf16 / fp16 gate: the ordered-integer distance between the 16-bit patterns of got and of the fp32
oracle rounded to that type is at most 1 (one ulp; -0 and +0 are the same point).  Dims past the
rotary part bit-identical.  Both types are sign-magnitude, so one ordering serves both.
"""
from __future__ import annotations

import numpy as np

ROT = 64
HALF = 32
FP32_TOL = 2e-6
BF16_ULP = 1


def pair_rel_err(got, ref, rot: int = ROT) -> np.ndarray:
    got = np.asarray(got, np.float64)[..., :rot]
    ref = np.asarray(ref, np.float64)[..., :rot]
    h = rot // 2
    norm = np.sqrt(ref[..., :h] ** 2 + ref[..., h:] ** 2)
    norm = np.concatenate([norm, norm], axis=-1)
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        err = np.where(norm > 0, diff / norm, np.where(diff > 0, np.inf, 0.0))
    return err


ELEM_FLOOR = 1e-6


def elem_rel_err(got, ref, rot: int = ROT) -> np.ndarray:
    """|got - ref| / max(|ref|, ELEM_FLOOR * pair norm) per rotated element (0 where both are 0)."""
    got = np.asarray(got, np.float64)[..., :rot]
    ref = np.asarray(ref, np.float64)[..., :rot]
    h = rot // 2
    norm = np.sqrt(ref[..., :h] ** 2 + ref[..., h:] ** 2)
    norm = np.concatenate([norm, norm], axis=-1)
    den = np.maximum(np.abs(ref), ELEM_FLOOR * norm)
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(den > 0, diff / den, np.where(diff > 0, np.inf, 0.0))


def check_fp32(got, ref, tol: float = FP32_TOL, rot: int = ROT):
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    err = pair_rel_err(got, ref, rot)
    worst = float(err.max()) if err.size else 0.0
    elem = elem_rel_err(got, ref, rot)
    worst_elem = float(elem.max()) if elem.size else 0.0
    tail_ok = np.array_equal(got[..., rot:].view(np.uint32), ref[..., rot:].view(np.uint32))
    absmax = float(np.abs(ref[..., :rot]).max()) if err.size else 0.0
    scaled = float(np.abs(got[..., :rot].astype(np.float64) - ref[..., :rot]).max() / absmax) if absmax else 0.0
    return (worst <= tol and worst_elem <= tol and tail_ok), {
        "max_pair_rel": worst, "max_elem_rel": worst_elem, "tail_bit_exact": tail_ok,
        "max_abs_over_absmax": scaled}


def _ordered(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_dist(got_bits, ref_bits) -> np.ndarray:
    return np.abs(_ordered(got_bits) - _ordered(ref_bits))


def check_16bit(got_bits, ref_bits, max_ulp: int = BF16_ULP, rot: int = ROT):
    return check_bf16(got_bits, ref_bits, max_ulp, rot)


def check_bf16(got_bits, ref_bits, max_ulp: int = BF16_ULP, rot: int = ROT):
    got_bits = np.asarray(got_bits, np.uint16)
    ref_bits = np.asarray(ref_bits, np.uint16)
    d = bf16_ulp_dist(got_bits[..., :rot], ref_bits[..., :rot])
    worst = int(d.max()) if d.size else 0
    tail_ok = np.array_equal(got_bits[..., rot:], ref_bits[..., rot:])
    return (worst <= max_ulp and tail_ok), {"max_ulp": worst, "n_off_by_one": int((d == 1).sum()),
                                           "frac_off_by_one": float((d == 1).mean()) if d.size else 0.0,
                                           "tail_bit_exact": tail_ok}
