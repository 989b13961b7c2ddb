"""ctypes binding of libmrope.so: argument checks and marshalling only (see include/mrope.h)."""
from __future__ import annotations

import ctypes
import enum
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmrope.so")
_lib = None

MROPE_F32 = 0
MROPE_BF16 = 1
MROPE_F16 = 2
TEXT_ONLY_START = 1 << 30
ROT_DIM = 64

# every symbol include/mrope.h declares
EXPORTS = ("mrope_abi_version", "mrope_status_string", "mrope_last_error", "mrope_set_test_hooks",
           "mrope_workspace_bytes",
           "mrope_workspace_init", "mrope_planes", "mrope_apply", "mrope_apply_ids", "mrope_apply_ids_noalloc",
           "mrope_apply_kv",
           "mrope_apply_ids_kv", "mrope_decode")


HOOK_FUSED_CHUNKED = 1
HOOK_FUSED_SCAN_FIRST = 2
HOOK_SCAN_FALLBACK = 4
HOOK_F32_EIGHT_LANES = 8


def set_test_hooks(flags: int) -> int:
    """Test and tuning hooks of the library (see mrope_set_test_hooks); returns the previous value."""
    return int(load().mrope_set_test_hooks(int(flags)))


class MarkerFlags(enum.IntFlag):
    MULTI_MARKER = 1
    FRAME_OVERRUN = 2
    BAD_FRAME_LEN = 4


class MropeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libmrope.so (built in-tree by canvas_rope_rotary_amd.build).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m canvas_rope_rotary_amd.build` "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, U64, F64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
    lib.mrope_abi_version.argtypes = []
    lib.mrope_abi_version.restype = ctypes.c_int
    lib.mrope_status_string.argtypes = [ctypes.c_int]
    lib.mrope_status_string.restype = ctypes.c_char_p
    lib.mrope_last_error.argtypes = []
    lib.mrope_last_error.restype = ctypes.c_char_p
    lib.mrope_set_test_hooks.argtypes = [ctypes.c_int]
    lib.mrope_set_test_hooks.restype = ctypes.c_int
    lib.mrope_workspace_bytes.argtypes = [I64]
    lib.mrope_workspace_bytes.restype = U64
    lib.mrope_workspace_init.argtypes = [P, U64, P]
    lib.mrope_workspace_init.restype = ctypes.c_int
    U32 = ctypes.c_uint32
    lib.mrope_planes.argtypes = [P, P, I32, I64, I32, I32, P, P, P, P, I64, P, P, P, P, P, U64, U32, P]
    lib.mrope_planes.restype = ctypes.c_int
    lib.mrope_apply.argtypes = [P, I64, I64, I32, P, I64, I64, I32, I64, I32, I32, I32, P, I64, F64, P, P, P]
    lib.mrope_apply.restype = ctypes.c_int
    lib.mrope_apply_ids.argtypes = [P, I64, I64, I32, P, I64, I64, I32, I64, I32, I32, I32, F64, P, P,
                                    P, P, I32, I32, I32, P, P, P, P, I64, P, P, P, P, P, U64, U32, P]
    lib.mrope_apply_ids.restype = ctypes.c_int
    lib.mrope_apply_ids_noalloc.argtypes = [P, I64, I64, I32, P, I64, I64, I32, I64, I32, I32, I32, F64, P, P,
                                            P, P, I32, I32, I32, P, P, P, P, I64, P, P, P, P, P]
    lib.mrope_apply_ids_noalloc.restype = ctypes.c_int
    cache = [P, P, P, I32, I64, I64, I64, I64]  # k_cache, v_cache, slot_mapping, block_size, num_blocks, strides
    lib.mrope_apply_kv.argtypes = [P, I64, I64, I32, P, I64, I64, I32, P, I64, I64, I64, I32, I32, I32, P, I64, F64,
                                   *cache, P]
    lib.mrope_apply_kv.restype = ctypes.c_int
    lib.mrope_apply_ids_kv.argtypes = [P, I64, I64, I32, P, I64, I64, I32, P, I64, I64, I64, I32, I32, I32, F64,
                                       P, P, I32, I32, I32, P, P, P, P, I64, P, P, P, P, P, U64, U32, *cache, P]
    lib.mrope_apply_ids_kv.restype = ctypes.c_int
    lib.mrope_decode.argtypes = [P, I64, I64, I32, P, I64, I64, I32, P, I64, I64, I32, P, P, *cache,
                                 I32, I32, I32, F64, P]
    lib.mrope_decode.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load()
        raise MropeError(status, f"{lib.mrope_status_string(status).decode()}: {lib.mrope_last_error().decode()}")


# While prepare() runs a binding function, the C calls it would make are recorded here instead.
_recording: list | None = None


class _EpochSlot:
    """Stands for a workspace's next epoch in a recorded call: each run of the prepared call takes a
    fresh one."""

    __slots__ = ("ws",)

    def __init__(self, ws):
        self.ws = ws


def _epoch(ws):
    return _EpochSlot(ws) if _recording is not None else ws.next_epoch()


def _invoke(cfunc, *args):
    if _recording is not None:
        _recording.append((cfunc, args))
        return
    _check(cfunc(*args))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class _on_device:
    """Make `device` current for the call, skipping the switch when it already is."""

    __slots__ = ("dev", "prev")

    def __init__(self, dev):
        self.dev = dev
        self.prev = None

    def __enter__(self):
        cur = torch.cuda.current_device()
        if self.dev.index is not None and self.dev.index != cur:
            self.prev = cur
            torch.cuda.set_device(self.dev)

    def __exit__(self, *exc):
        if self.prev is not None:
            torch.cuda.set_device(self.prev)


_DTYPES = {torch.float32: MROPE_F32, torch.bfloat16: MROPE_BF16, torch.float16: MROPE_F16}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)") from None


def _require_cuda(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on a CUDA (HIP) device")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same device")
    return dev


def _heads(t: torch.Tensor, name: str):
    if t.dim() != 3:
        raise ValueError(f"{name} must be [tokens, heads, head_dim]")
    if t.numel() == 0:  # no elements: strides are free, pass those of a contiguous tensor
        return t.shape[1] * t.shape[2], t.shape[2], t.shape[1], t.shape[2]
    if t.stride(2) != 1:
        raise ValueError(f"{name}: head_dim must be contiguous")
    return t.stride(0), t.stride(1), t.shape[1], t.shape[2]


def _i32_vec(t: torch.Tensor, name: str, n: int | None = None):
    if t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous 1-D int32 tensor")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} elements")
    return t


def cu_seqlens_from_lens(lens: torch.Tensor) -> torch.Tensor:
    """Sequence lengths [n] -> cu_seqlens [n + 1] int32 (0, then the running sum)."""
    out = torch.zeros(lens.numel() + 1, dtype=torch.int32, device=lens.device)
    torch.cumsum(lens.to(torch.int32), 0, out=out[1:])
    return out


class Workspace:
    """Device workspace of the plane-deriving calls, zero-filled once, reusable across calls on one
    stream.  It also keeps the call counter that tags each call's status words (the epoch); under
    HIP-graph capture the library's device-side counter is used instead (epoch 0)."""

    def __init__(self, n_tokens: int, device=None):
        self.device = torch.device(device if device is not None else "cuda")
        self.capacity = 0
        self.buf = None
        self.calls = 0
        self.ensure(n_tokens)

    def next_epoch(self) -> int:
        if torch.cuda.is_current_stream_capturing():
            return 0
        self.calls = self.calls % ((1 << 29) - 1) + 1
        return self.calls

    def ensure(self, n_tokens: int):
        need = int(load().mrope_workspace_bytes(int(n_tokens)))
        if self.buf is not None and need <= self.capacity:
            return self
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(f"workspace too small for {n_tokens} tokens; size it before graph capture")
        buf = torch.zeros(need + 256, dtype=torch.uint8, device=self.device)
        off = (-buf.data_ptr()) % 256
        self.buf = buf
        self.view = buf[off:off + need]
        self.capacity = need
        return self

    @property
    def ptr(self):
        return ctypes.c_void_p(self.view.data_ptr())


_default_ws: dict = {}


def _workspace(ws, n_tokens, device):
    """The caller's workspace, else one kept per (device, stream): calls on one stream are ordered,
    so they may share it; calls on different streams never do.  Under graph capture pass one made
    before the capture."""
    if ws is None:
        key = (device, torch.cuda.current_stream(device).cuda_stream)
        ws = _default_ws.get(key)
        if ws is None:
            if torch.cuda.is_current_stream_capturing():
                raise RuntimeError("pass workspace= to calls captured in a graph (a Workspace made before capture)")
            ws = _default_ws[key] = Workspace(n_tokens, device)
    return ws.ensure(n_tokens)


def planes(ids: torch.Tensor, cu_seqlens: torch.Tensor, marker_id: int = 248078, *, out=None, start=None,
           amount=None, origin=None, seq_flags=None, pos_offset=None, origin_in=None, frame_len: int = 67,
           frame_len_seq=None, workspace: Workspace | None = None):
    """Canvas planes from token ids.  Returns (planes [3, L] int32, start [n], amount [n], origin [n],
    seq_flags [n]).  cu_seqlens[-1] must equal len(ids).  For a later piece of each sequence (chunked
    prefill, a second turn) pass pos_offset (position of the piece's first token) and origin_in (the
    previous piece's origin output).  frame_len: tokens from <image> to start (67: this template's
    frame; 66 + k for k marker tokens after </image>; 65: Qwen-VL's rule); frame_len_seq (int32 [n],
    optional): each sequence's own frame length, 0 = frame_len (an entry outside [65, 4096] also takes
    frame_len and sets seq_flags bit 4)."""
    dev = _require_cuda(ids, cu_seqlens, out, start, amount, origin, seq_flags, pos_offset, origin_in,
                        frame_len_seq)
    _i32_vec(ids, "ids")
    _i32_vec(cu_seqlens, "cu_seqlens")
    L = ids.numel()
    n = cu_seqlens.numel() - 1
    for t, name in ((pos_offset, "pos_offset"), (origin_in, "origin_in"), (frame_len_seq, "frame_len_seq")):
        if t is not None:
            _i32_vec(t, name, n)
    if out is None:
        out = torch.empty((3, L), dtype=torch.int32, device=dev)
    if out.dtype != torch.int32 or out.dim() != 2 or out.shape[0] != 3 or out.shape[1] < L or out.stride(1) != 1:
        raise ValueError("out must be an int32 [3, >= L] tensor with unit column stride")
    mk = lambda t, name: _i32_vec(t, name, n) if t is not None else torch.empty(n, dtype=torch.int32, device=dev)
    start, amount, origin, seq_flags = (mk(start, "start"), mk(amount, "amount"), mk(origin, "origin"),
                                        mk(seq_flags, "seq_flags"))
    ws = _workspace(workspace, L, dev)
    with _on_device(dev):
        _invoke(load().mrope_planes, _ptr(ids), _ptr(cu_seqlens), n, L, int(marker_id), int(frame_len),
                                   _ptr(frame_len_seq), _ptr(pos_offset),
                                   _ptr(origin_in), _ptr(out), out.stride(0),
                                   _ptr(start), _ptr(amount), _ptr(origin), _ptr(seq_flags), ws.ptr,
                                   ws.capacity, _epoch(ws), _stream(dev))
    return out, start, amount, origin, seq_flags


def _qk_args(q, k, q_out, k_out):
    dt = _dtype_code(q)
    if k is not None and k.dtype != q.dtype:
        raise TypeError("q and k must have the same dtype")
    qt, qh, nq, D = _heads(q, "q")
    if k is not None:
        kt, kh, nk, Dk = _heads(k, "k")
        if Dk != D or k.shape[0] != q.shape[0]:
            raise ValueError("q and k must have the same tokens and head_dim")
    else:
        kt = kh = nk = 0
    for o, src, name in ((q_out, q, "q_out"), (k_out, k, "k_out")):
        if o is not None:
            if src is None or o.shape != src.shape or o.stride() != src.stride() or o.dtype != src.dtype:
                raise ValueError(f"{name} must match its input's shape, strides and dtype")
    return dt, qt, qh, nq, kt, kh, nk, D


def apply(q: torch.Tensor, k: torch.Tensor | None, planes_: torch.Tensor, theta: float = 1e7, *, q_out=None,
          k_out=None, rot_dim: int = ROT_DIM):
    """Rotate Q and K ([T, heads, head_dim], bf16 / fp16 / fp32) with planes [3, >= T] int32.  In
    place unless q_out / k_out are given (then full heads are written there).  Returns (q, k) as
    written."""
    dev = _require_cuda(q, k, planes_, q_out, k_out)
    dt, qt, qh, nq, kt, kh, nk, D = _qk_args(q, k, q_out, k_out)
    T = q.shape[0]
    if planes_.dtype != torch.int32 or planes_.dim() != 2 or planes_.shape[0] != 3 or planes_.shape[1] < T \
            or planes_.stride(1) != 1:
        raise ValueError("planes must be an int32 [3, >= tokens] tensor with unit column stride")
    with _on_device(dev):
        _invoke(load().mrope_apply, _ptr(q), qt, qh, nq, _ptr(k), kt, kh, nk, T, D, rot_dim, dt, _ptr(planes_),
                                  planes_.stride(0), float(theta), _ptr(q_out), _ptr(k_out), _stream(dev))
    return (q_out if q_out is not None else q), (k_out if k_out is not None else k)


def apply_ids(q: torch.Tensor, k: torch.Tensor | None, ids: torch.Tensor, cu_seqlens: torch.Tensor,
              marker_id: int = 248078, theta: float = 1e7, *, planes_out=None, start=None, amount=None,
              origin=None, seq_flags=None, pos_offset=None, origin_in=None, frame_len: int = 67,
              frame_len_seq=None, q_out=None, k_out=None, workspace: Workspace | None = None,
              rot_dim: int = ROT_DIM):
    """Plane derivation fused with the rotation, one launch.  Returns (start, amount, origin,
    seq_flags, planes_out or None).  pos_offset / origin_in / frame_len / frame_len_seq as in
    planes()."""
    dev = _require_cuda(q, k, ids, cu_seqlens, planes_out, start, amount, origin, seq_flags, q_out, k_out,
                        pos_offset, origin_in, frame_len_seq)
    dt, qt, qh, nq, kt, kh, nk, D = _qk_args(q, k, q_out, k_out)
    _i32_vec(ids, "ids", q.shape[0])
    _i32_vec(cu_seqlens, "cu_seqlens")
    T = q.shape[0]
    n = cu_seqlens.numel() - 1
    for t, name in ((pos_offset, "pos_offset"), (origin_in, "origin_in"), (frame_len_seq, "frame_len_seq")):
        if t is not None:
            _i32_vec(t, name, n)
    ps = 0
    if planes_out is not None:
        if planes_out.dtype != torch.int32 or planes_out.dim() != 2 or planes_out.shape[0] != 3 \
                or planes_out.shape[1] < T or planes_out.stride(1) != 1:
            raise ValueError("planes_out must be an int32 [3, >= tokens] tensor with unit column stride")
        ps = planes_out.stride(0)
    mk = lambda t, name: _i32_vec(t, name, n) if t is not None else torch.empty(n, dtype=torch.int32, device=dev)
    start, amount, origin, seq_flags = (mk(start, "start"), mk(amount, "amount"), mk(origin, "origin"),
                                        mk(seq_flags, "seq_flags"))
    ws = _workspace(workspace, T, dev)
    with _on_device(dev):
        _invoke(load().mrope_apply_ids, _ptr(q), qt, qh, nq, _ptr(k), kt, kh, nk, T, D, rot_dim, dt, float(theta),
                                      _ptr(q_out), _ptr(k_out), _ptr(ids), _ptr(cu_seqlens), n, int(marker_id),
                                      int(frame_len), _ptr(frame_len_seq), _ptr(pos_offset), _ptr(origin_in),
                                      _ptr(planes_out), ps, _ptr(start), _ptr(amount), _ptr(origin),
                                      _ptr(seq_flags), ws.ptr, ws.capacity, _epoch(ws), _stream(dev))
    return start, amount, origin, seq_flags, planes_out


NOALLOC_MAX_TOKENS = 1 << 20


def apply_ids_noalloc(q: torch.Tensor, k: torch.Tensor | None, ids: torch.Tensor, cu_seqlens: torch.Tensor,
                      marker_id: int = 248078, theta: float = 1e7, *, planes_out=None, start=None, amount=None,
                      origin=None, seq_flags=None, pos_offset=None, origin_in=None, frame_len: int = 67,
                      frame_len_seq=None, q_out=None, k_out=None, rot_dim: int = ROT_DIM):
    """apply_ids without a workspace: the library's static per-GPU scratch stands in for it (at most
    NOALLOC_MAX_TOKENS tokens).  Pass every output (start, amount, origin, seq_flags) to allocate
    nothing here either.  The first call on a device must not be captured in a graph."""
    dev = _require_cuda(q, k, ids, cu_seqlens, planes_out, start, amount, origin, seq_flags, q_out, k_out,
                        pos_offset, origin_in, frame_len_seq)
    dt, qt, qh, nq, kt, kh, nk, D = _qk_args(q, k, q_out, k_out)
    _i32_vec(ids, "ids", q.shape[0])
    _i32_vec(cu_seqlens, "cu_seqlens")
    T = q.shape[0]
    n = cu_seqlens.numel() - 1
    for t, name in ((pos_offset, "pos_offset"), (origin_in, "origin_in"), (frame_len_seq, "frame_len_seq")):
        if t is not None:
            _i32_vec(t, name, n)
    ps = 0
    if planes_out is not None:
        if planes_out.dtype != torch.int32 or planes_out.dim() != 2 or planes_out.shape[0] != 3 \
                or planes_out.shape[1] < T or planes_out.stride(1) != 1:
            raise ValueError("planes_out must be an int32 [3, >= tokens] tensor with unit column stride")
        ps = planes_out.stride(0)
    mk = lambda t, name: _i32_vec(t, name, n) if t is not None else torch.empty(n, dtype=torch.int32, device=dev)
    start, amount, origin, seq_flags = (mk(start, "start"), mk(amount, "amount"), mk(origin, "origin"),
                                        mk(seq_flags, "seq_flags"))
    with _on_device(dev):
        _invoke(load().mrope_apply_ids_noalloc, _ptr(q), qt, qh, nq, _ptr(k), kt, kh, nk, T, D, rot_dim, dt,
                                              float(theta), _ptr(q_out), _ptr(k_out), _ptr(ids), _ptr(cu_seqlens), n,
                                              int(marker_id), int(frame_len), _ptr(frame_len_seq),
                                              _ptr(pos_offset), _ptr(origin_in),
                                              _ptr(planes_out), ps, _ptr(start), _ptr(amount), _ptr(origin),
                                              _ptr(seq_flags), _stream(dev))
    return start, amount, origin, seq_flags, planes_out


def check_slots(slot_mapping: torch.Tensor, num_slots: int) -> None:
    """Debug check for a cache write: raise ValueError when two entries of slot_mapping name the
    same slot inside the cache ([0, num_slots)), where which token lands is undefined.  Runs torch
    operations on the mapping's device and waits for them; the cache-writing calls run it when
    given check_slots=True."""
    s = slot_mapping.reshape(-1)
    s = s[(s >= 0) & (s < num_slots)]
    if s.numel() < 2:
        return
    srt = torch.sort(s).values
    dup = srt[1:] == srt[:-1]
    if bool(dup.any()):
        first = int(srt[1:][dup][0])
        raise ValueError(f"slot_mapping names slot {first} (and {int(dup.sum())} repeats in all) more than once")


_slot_check = check_slots  # the cache-writing calls' keyword of the same name shadows it there


def _paged(k_cache, v_cache, slot_mapping, v, n_rows: int, nk: int, D: int, dtype, what: str):
    """Check a paged K/V cache pair and its slots; returns the C arguments (v strides, cache args)."""
    if k_cache is None or slot_mapping is None:
        raise ValueError(f"{what}: k_cache and slot_mapping are required")
    if (v is None) != (v_cache is None):
        raise ValueError(f"{what}: v and v_cache go together")
    for c, name in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if c is None:
            continue
        if c.dim() != 4 or c.shape[2] != nk or c.shape[3] != D or c.stride(3) != 1 or c.dtype != dtype:
            raise ValueError(f"{name} must be [num_blocks, block_size, n_kv_heads, head_dim] of q's dtype")
    if v_cache is not None and (v_cache.shape != k_cache.shape or v_cache.stride() != k_cache.stride()):
        raise ValueError("v_cache must have k_cache's shape and strides")
    if slot_mapping.dtype != torch.int64 or slot_mapping.dim() != 1 or slot_mapping.numel() != n_rows \
            or not slot_mapping.is_contiguous():
        raise ValueError(f"slot_mapping must be a contiguous int64 [{n_rows}] tensor")
    vt = vh = 0
    if v is not None:
        vt, vh, nv, Dv = _heads(v, "v")
        if nv != nk or Dv != D or v.shape[0] != n_rows or v.dtype != dtype:
            raise ValueError("v must match k's shape and dtype")
    return (vt, vh), (_ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), k_cache.shape[1], k_cache.shape[0],
                      k_cache.stride(0), k_cache.stride(1), k_cache.stride(2))


def apply_kv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor | None, planes_: torch.Tensor, k_cache: torch.Tensor,
             v_cache: torch.Tensor | None, slot_mapping: torch.Tensor, theta: float = 1e7, *, rot_dim: int = ROT_DIM,
             check_slots: bool = False):
    """Prefill rotation with the paged K/V cache write: q [T, Hq, D] rotated in place; k [T, Hk, D]
    rotated and written whole into k_cache [num_blocks, block_size, Hk, D] at slot_mapping (int64
    [T]; slots outside the cache are skipped); v [T, Hk, D] copied into v_cache.  k and v are not
    modified.  check_slots: first raise ValueError if two tokens share a slot (see check_slots()).
    Returns (q, k_cache, v_cache)."""
    dev = _require_cuda(q, k, v, planes_, k_cache, v_cache, slot_mapping)
    dt, qt, qh, nq, kt, kh, nk, D = _qk_args(q, k, None, None)
    T = q.shape[0]
    if planes_.dtype != torch.int32 or planes_.dim() != 2 or planes_.shape[0] != 3 or planes_.shape[1] < T \
            or planes_.stride(1) != 1:
        raise ValueError("planes must be an int32 [3, >= tokens] tensor with unit column stride")
    (vt, vh), cache = _paged(k_cache, v_cache, slot_mapping, v, T, nk, D, q.dtype, "apply_kv")
    if check_slots:
        _slot_check(slot_mapping, k_cache.shape[0] * k_cache.shape[1])
    with _on_device(dev):
        _invoke(load().mrope_apply_kv, _ptr(q), qt, qh, nq, _ptr(k), kt, kh, nk, _ptr(v), vt, vh, T, D, rot_dim, dt,
                                     _ptr(planes_), planes_.stride(0), float(theta), *cache, _stream(dev))
    return q, k_cache, v_cache


def apply_ids_kv(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor | None, ids: torch.Tensor, cu_seqlens: torch.Tensor,
                 k_cache: torch.Tensor, v_cache: torch.Tensor | None, slot_mapping: torch.Tensor,
                 marker_id: int = 248078, theta: float = 1e7, *, planes_out=None, start=None, amount=None,
                 origin=None, seq_flags=None, pos_offset=None, origin_in=None, frame_len: int = 67,
                 frame_len_seq=None, workspace: Workspace | None = None, rot_dim: int = ROT_DIM,
                 check_slots: bool = False):
    """apply_ids with the cache write of apply_kv, in one launch: ids -> planes -> q rotated in
    place, k rotated into k_cache, v copied into v_cache.  check_slots as in apply_kv.  Returns
    (start, amount, origin, seq_flags, planes_out or None)."""
    dev = _require_cuda(q, k, v, ids, cu_seqlens, k_cache, v_cache, slot_mapping, planes_out, start, amount, origin,
                        seq_flags, pos_offset, origin_in, frame_len_seq)
    dt, qt, qh, nq, kt, kh, nk, D = _qk_args(q, k, None, None)
    _i32_vec(ids, "ids", q.shape[0])
    _i32_vec(cu_seqlens, "cu_seqlens")
    T = q.shape[0]
    n = cu_seqlens.numel() - 1
    for t, name in ((pos_offset, "pos_offset"), (origin_in, "origin_in"), (frame_len_seq, "frame_len_seq")):
        if t is not None:
            _i32_vec(t, name, n)
    ps = 0
    if planes_out is not None:
        if planes_out.dtype != torch.int32 or planes_out.dim() != 2 or planes_out.shape[0] != 3 \
                or planes_out.shape[1] < T or planes_out.stride(1) != 1:
            raise ValueError("planes_out must be an int32 [3, >= tokens] tensor with unit column stride")
        ps = planes_out.stride(0)
    (vt, vh), cache = _paged(k_cache, v_cache, slot_mapping, v, T, nk, D, q.dtype, "apply_ids_kv")
    if check_slots:
        _slot_check(slot_mapping, k_cache.shape[0] * k_cache.shape[1])
    mk = lambda t, name: _i32_vec(t, name, n) if t is not None else torch.empty(n, dtype=torch.int32, device=dev)
    start, amount, origin, seq_flags = (mk(start, "start"), mk(amount, "amount"), mk(origin, "origin"),
                                        mk(seq_flags, "seq_flags"))
    ws = _workspace(workspace, T, dev)
    with _on_device(dev):
        _invoke(load().mrope_apply_ids_kv, _ptr(q), qt, qh, nq, _ptr(k), kt, kh, nk, _ptr(v), vt, vh, T, D, rot_dim, dt,
                                         float(theta), _ptr(ids), _ptr(cu_seqlens), n, int(marker_id),
                                         int(frame_len), _ptr(frame_len_seq), _ptr(pos_offset), _ptr(origin_in),
                                         _ptr(planes_out), ps, _ptr(start),
                                         _ptr(amount), _ptr(origin), _ptr(seq_flags), ws.ptr, ws.capacity,
                                         _epoch(ws), *cache, _stream(dev))
    return start, amount, origin, seq_flags, planes_out


def decode(q: torch.Tensor, k: torch.Tensor | None, pos: torch.Tensor, amount: torch.Tensor,
           k_cache: torch.Tensor | None, slot_mapping: torch.Tensor | None, theta: float = 1e7, *,
           v: torch.Tensor | None = None, v_cache: torch.Tensor | None = None, rot_dim: int = ROT_DIM,
           check_slots: bool = False):
    """One generated token per sequence: rotate q [S, Hq, D] in place at plane pos - amount; rotate
    k [S, Hk, D] and write it into k_cache [num_blocks, block_size, Hk, D] at slot_mapping (int64,
    slots outside the cache are skipped); copy v [S, Hk, D] (optional) into v_cache at the same
    slots.  check_slots as in apply_kv."""
    dev = _require_cuda(q, k, pos, amount, k_cache, slot_mapping, v, v_cache)
    dt, qt, qh, nq, kt, kh, nk, D = _qk_args(q, k, None, None)
    S = q.shape[0]
    _i32_vec(pos, "pos", S)
    _i32_vec(amount, "amount", S)
    if nk:
        (vt, vh), cache = _paged(k_cache, v_cache, slot_mapping, v, S, nk, D, q.dtype, "decode")
        if check_slots:
            _slot_check(slot_mapping, k_cache.shape[0] * k_cache.shape[1])
    else:
        (vt, vh), cache = (0, 0), (None, None, None, 1, 0, 0, 0, 0)
    with _on_device(dev):
        _invoke(load().mrope_decode, _ptr(q), qt, qh, nq, _ptr(k), kt, kh, nk, _ptr(v), vt, vh, S, _ptr(pos),
                                   _ptr(amount), *cache, D, rot_dim, dt, float(theta), _stream(dev))
    return q, k_cache


class PreparedCall:
    """One binding call with its arguments checked and marshalled once (see prepare()).  Calling it
    launches the same C call again, on the stream and with the tensors bound at preparation; a call
    with a workspace takes a fresh epoch each time.  `result` is what the binding function returned
    (the same output tensors are written by every run)."""

    __slots__ = ("_dev", "_calls", "result")

    def __init__(self, dev, calls, result):
        self._dev = dev
        self._calls = []
        for cfunc, args in calls:
            # arguments as ctypes values of the declared types: ctypes then converts nothing per call
            conv, slots = [], []
            for t, a in zip(cfunc.argtypes, args):
                if isinstance(a, _EpochSlot):
                    slots.append((t(0), a.ws))
                    conv.append(slots[-1][0])
                elif a is None or isinstance(a, ctypes._SimpleCData):
                    conv.append(a)
                else:
                    conv.append(t(a))
            self._calls.append((cfunc, conv, slots))
        self.result = result

    def __call__(self):
        with _on_device(self._dev):
            for cfunc, args, slots in self._calls:
                for cell, ws in slots:
                    ws.calls = ws.calls % ((1 << 29) - 1) + 1
                    cell.value = ws.calls
                _check(cfunc(*args))
        return self.result


def prepare(fn, *args, **kwargs) -> PreparedCall:
    """Check and marshal a call of one of this module's functions (planes, apply, apply_ids,
    apply_ids_noalloc, apply_kv, apply_ids_kv, decode) once, without launching it, and return a
    PreparedCall that launches it each time it is called -- for an eager loop that repeats a call on
    the same buffers (a decode step), where the per-call argument checks would otherwise cost more
    host time than the GPU work.  The stream current now is the one every run launches on.  Output
    tensors the call would allocate are allocated here once.  The prepared call must not be run
    inside HIP-graph capture (capture the plain call instead: its epochs come from the device)."""
    global _recording
    if _recording is not None:
        raise RuntimeError("prepare() does not nest")
    rec = []
    _recording = rec
    try:
        result = fn(*args, **kwargs)
    finally:
        _recording = None
    if not rec:
        raise ValueError(f"{getattr(fn, '__name__', fn)} made no library call to prepare")
    dev = None
    for a in list(args) + list(kwargs.values()):
        if isinstance(a, torch.Tensor) and a.is_cuda:
            dev = a.device
            break
    return PreparedCall(dev, rec, result)
