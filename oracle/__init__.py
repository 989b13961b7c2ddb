"""Canvas M-RoPE oracle -- TEST INFRASTRUCTURE ONLY.

A plain, slow, scalar CPU implementation (``mrope_oracle.c``, C11 + libm) of what the canvas M-RoPE
path computes, with a thin numpy/ctypes wrapper.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never imports, links or
calls it, and the two share no code.

Definitions followed (see the header of ``mrope_oracle.c`` for the full statement):

* canvas rule, start and amount: Hugging Face card "MiniCPM-V-4.7-1B -- Core AI", section "How the
  VLM rides the text-only engine" (canvas table and the start/amount paragraph); Core AI model-zoo
  page "MiniCPM-V-4.7-1B: canvas M-RoPE on the Qwen3.5 hybrid, on Core AI", section "The canvas rule
  and why the gate is on the planes";
* interleaved sections [11, 11, 10]: the same card, section "What it is";
* rotate-half over the first 64 of 256 dims, theta = 1e7, the frequency-to-plane rule: the model
  configuration of the workload (not printed on the pages).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mrope_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# The mutation test points this at a deliberately broken build of a copy of the source.
_LIB_OVERRIDE = os.environ.get("MROPE_ORACLE_LIB")
_lib = None

TEXT_ONLY_START = 1 << 30


def build() -> str:
    """Compile ``liboracle.so`` with gcc (plain C, no fast-math, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _LIB_OVERRIDE or _LIB_PATH
    if not _LIB_OVERRIDE and not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_first_marker.argtypes = [P, i32, i32]
    lib.oracle_first_marker.restype = i32
    lib.oracle_frame_scalars.argtypes = [i32, P, P]
    lib.oracle_frame_scalars.restype = None
    lib.oracle_planes.argtypes = [P, P, i32, i32, P, i64, P, P, P]
    lib.oracle_planes.restype = None
    lib.oracle_planes_chunk.argtypes = [P, P, i32, i32, i32, P, P, P, P, i64, P, P, P]
    lib.oracle_seq_frame_len.argtypes = [P, i32, i32]
    lib.oracle_seq_frame_len.restype = i32
    lib.oracle_frame_scalars_len.argtypes = [i32, i32, P, P]
    lib.oracle_frame_scalars_len.restype = None
    lib.oracle_planes_chunk.restype = None
    lib.oracle_inv_freq.argtypes = [f64, i32, P]
    lib.oracle_inv_freq.restype = None
    lib.oracle_plane_of_freq.argtypes = [i32]
    lib.oracle_plane_of_freq.restype = i32
    lib.oracle_rotate.argtypes = [P, i64, i32, i64, i64, i32, i32, P, i64, f64, P, P]
    lib.oracle_rotate.restype = None
    lib.oracle_decode.argtypes = [P, i32, P, i32, i32, P, P, i32, i32, f64, P, P, P, i32, i64, i64, i64, i64, P, P]
    lib.oracle_scatter_rows.argtypes = [P, i64, i64, P, i32, i64, P]
    lib.oracle_scatter_rows.restype = None
    lib.oracle_decode.restype = None
    lib.oracle_round_bf16.argtypes = [P, P, i64]
    lib.oracle_round_bf16.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def first_marker(ids, marker_id: int) -> int:
    ids = _c(ids, np.int32)
    return int(_load().oracle_first_marker(_ptr(ids), ids.size, marker_id))


def frame_scalars_len(origin: int, frame_len: int) -> tuple[int, int]:
    st, am = ctypes.c_int32(), ctypes.c_int32()
    _load().oracle_frame_scalars_len(int(origin), int(frame_len), ctypes.byref(st), ctypes.byref(am))
    return st.value, am.value


def frame_scalars(origin: int) -> tuple[int, int]:
    st, am = ctypes.c_int32(), ctypes.c_int32()
    _load().oracle_frame_scalars(int(origin), ctypes.byref(st), ctypes.byref(am))
    return st.value, am.value


def planes(ids, cu_seqlens, marker_id: int):
    """Planes [3, L] int32, start [n], amount [n], origin [n] (-1 = no image)."""
    ids = _c(ids, np.int32)
    cu = _c(cu_seqlens, np.int32)
    n = cu.size - 1
    total = int(cu[-1]) if n >= 0 else 0
    if total != ids.size:
        raise ValueError("cu_seqlens[-1] must equal len(ids)")
    pl = np.zeros((3, max(total, 1)), np.int32)[:, :total].copy()
    st = np.zeros(n, np.int32)
    am = np.zeros(n, np.int32)
    og = np.zeros(n, np.int32)
    _load().oracle_planes(_ptr(ids), _ptr(cu), n, int(marker_id), _ptr(pl), total, _ptr(st), _ptr(am),
                          _ptr(og))
    return pl, st, am, og


def planes_chunk(ids, cu_seqlens, marker_id: int, pos_offset=None, origin_in=None, frame_len: int = 67,
                 frame_len_seq=None):
    """Planes of a later piece of each sequence: token i of sequence s sits at pos_offset[s] + i, and
    origin_in[s] (-1 = none) is the origin found in the earlier pieces; frame_len tokens from the
    origin to start, or frame_len_seq[s] for a sequence that gives its own (0: the call's; an entry
    outside [65, 4096] also falls back to the call's).  Returns planes [3, L], start, amount,
    origin (the sequence's origin so far, -1 = none)."""
    ids = _c(ids, np.int32)
    cu = _c(cu_seqlens, np.int32)
    n = cu.size - 1
    total = int(cu[-1])
    po = _c(pos_offset, np.int32) if pos_offset is not None else None
    oi = _c(origin_in, np.int32) if origin_in is not None else None
    fs = _c(frame_len_seq, np.int32) if frame_len_seq is not None else None
    pl = np.zeros((3, max(total, 1)), np.int32)[:, :total].copy()
    st = np.zeros(n, np.int32)
    am = np.zeros(n, np.int32)
    og = np.zeros(n, np.int32)
    _load().oracle_planes_chunk(_ptr(ids), _ptr(cu), n, int(marker_id), int(frame_len),
                                _ptr(fs) if fs is not None else None,
                                _ptr(po) if po is not None else None,
                                _ptr(oi) if oi is not None else None, _ptr(pl), total, _ptr(st), _ptr(am), _ptr(og))
    return pl, st, am, og


def seq_frame_len(frame_len_seq, s: int, frame_len: int = 67) -> int:
    """The frame length the oracle uses for sequence s (see oracle_seq_frame_len)."""
    fs = _c(frame_len_seq, np.int32) if frame_len_seq is not None else None
    return int(_load().oracle_seq_frame_len(_ptr(fs) if fs is not None else None, int(s), int(frame_len)))


def inv_freq(theta: float = 1e7, rot_dim: int = 64) -> np.ndarray:
    out = np.zeros(rot_dim // 2, np.float32)
    _load().oracle_inv_freq(float(theta), rot_dim, _ptr(out))
    return out


def plane_of_freq(j: int) -> int:
    return int(_load().oracle_plane_of_freq(j))


def rotate(x, planes_, theta: float = 1e7, rot_dim: int = 64, want_f64: bool = False):
    """Rotate x [T, H, D] (any float dtype whose values are exact in fp32) with planes [3, T].

    Returns the fp32 result (dense [T, H, D]) and, if ``want_f64``, the unrounded double result.
    """
    x = _c(x, np.float32)
    if x.ndim != 3:
        raise ValueError("x must be [tokens, heads, head_dim]")
    T, H, D = x.shape
    pl = _c(planes_, np.int32)
    if pl.shape != (3, T):
        raise ValueError("planes must be [3, tokens]")
    y = np.empty((T, H, D), np.float32)
    y64 = np.empty((T, H, D), np.float64) if want_f64 else None
    _load().oracle_rotate(_ptr(x), T, H, H * D, D, D, rot_dim, _ptr(pl), T, float(theta), _ptr(y),
                          _ptr(y64) if want_f64 else None)
    return (y, y64) if want_f64 else y


def scatter_paged(rows, slot_mapping, cache):
    """Paged cache write: rows [n, H, D] go to cache[slot // B, slot % B] of a [blocks, B, H, D]
    float32 cache (modified in place); slots < 0 or >= blocks * B are skipped."""
    rows = _c(rows, np.float32)
    slots = _c(slot_mapping, np.int64)
    if not (cache.flags["C_CONTIGUOUS"] and cache.dtype == np.float32):
        raise ValueError("cache must be a C-contiguous float32 array")
    n = rows.shape[0]
    row_elems = int(np.prod(rows.shape[1:])) if rows.ndim > 1 else 1
    if slots.size != n or int(np.prod(cache.shape[2:])) != row_elems:
        raise ValueError("rows, slot_mapping and cache do not match")
    _load().oracle_scatter_rows(_ptr(rows), n, row_elems, _ptr(slots), int(cache.shape[1]), int(cache.shape[0]),
                                _ptr(cache))
    return cache


def decode(q, k, pos, amount, cache, slot_mapping, block_size: int, theta: float = 1e7, rot_dim: int = 64,
           v=None, v_cache=None):
    """Decode step.  q [S, Hq, D], k [S, Hk, D]; returns rotated q (fp32) and writes the rotated k
    heads into ``cache`` ([blocks, block_size, Hk, D] float32, modified in place); v [S, Hk, D]
    (optional) goes unrotated into ``v_cache`` (same shape as cache) at the same slots."""
    q = _c(q, np.float32)
    k = _c(k, np.float32)
    S, Hq, D = q.shape
    Hk = k.shape[1]
    pos = _c(pos, np.int32)
    amount = _c(amount, np.int32)
    slots = _c(slot_mapping, np.int64)
    for c in (cache, v_cache):
        if c is None:
            continue
        if not (c.flags["C_CONTIGUOUS"] and c.dtype == np.float32):
            raise ValueError("caches must be C-contiguous float32 arrays")
        if c.shape[1:] != (block_size, Hk, D):
            raise ValueError("caches must be [blocks, block_size, n_k_heads, head_dim]")
    if (v is None) != (v_cache is None) or (v_cache is not None and v_cache.shape != cache.shape):
        raise ValueError("v and v_cache go together, v_cache shaped like cache")
    vv = _c(v, np.float32) if v is not None else None
    q_out = np.empty_like(q)
    _load().oracle_decode(_ptr(q), Hq, _ptr(k), Hk, S, _ptr(pos), _ptr(amount), D, rot_dim, float(theta),
                          _ptr(q_out), _ptr(cache), _ptr(slots), block_size, int(cache.shape[0]),
                          block_size * Hk * D, D, Hk * D, _ptr(vv) if vv is not None else None,
                          _ptr(v_cache) if v_cache is not None else None)
    return q_out


def round_f16(x) -> np.ndarray:
    """fp32 -> IEEE half bit patterns (uint16), round to nearest even (numpy's IEEE conversion)."""
    return np.ascontiguousarray(x, np.float32).astype(np.float16).view(np.uint16)


def round_bf16(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_bf16(_ptr(x), _ptr(out), x.size)
    return out
