"""Helpers of the GPU parity tests: move seeded inputs to the device, read results back, and call the
oracle on the same inputs.  No method arithmetic here."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from canvas_rope_rotary_amd import synth
from parity import check_bf16, check_fp32

MARKER = synth.IMAGE_ID


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def dev_heads(x: np.ndarray, dtype: str) -> torch.Tensor:
    """numpy heads (float32 values, or uint16 bit patterns for bf16 / f16) -> cuda tensor of the dtype."""
    if dtype in ("bf16", "f16"):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(TORCH_DT[dtype]).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()


def host_heads(t: torch.Tensor) -> np.ndarray:
    """cuda heads -> numpy (uint16 bit patterns for the 16-bit types, float32 otherwise)."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    return synth.to_f32(x, dtype)


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def compare_heads(got: np.ndarray, x_in: np.ndarray, planes: np.ndarray, dtype: str, theta=1e7, what=""):
    """got: GPU result rows; x_in: the same rows' inputs; planes [3, rows] from the oracle."""
    ref = oracle.rotate(as_f32(x_in, dtype), planes, theta)
    if dtype == "bf16":
        ok, info = check_bf16(got, oracle.round_bf16(ref))
    elif dtype == "f16":
        ok, info = check_bf16(got, oracle.round_f16(ref))
    else:
        ok, info = check_fp32(got, ref)
    assert ok, f"{what}: {info}"
    return info


def host_threads() -> int:
    """Worker threads for host-side checks: the CPUs this process may use, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def compare_heads_all(got: torch.Tensor, x_in: np.ndarray, planes: np.ndarray, dtype: str, theta=1e7, what="",
                      block: int = 8192):
    """Every element of a full-size result against the oracle: `got` is the device result [rows,
    heads, head_dim] (rows in the order of x_in and planes), copied to the host once; the oracle runs
    over blocks of rows in host threads (its C calls release the interpreter lock).  The same gates
    as compare_heads; the worst figures over all blocks are returned."""
    host = host_heads(got)
    n = host.shape[0]
    assert x_in.shape[0] == n and planes.shape[1] == n, what

    def one(lo):
        hi = min(n, lo + block)
        ref = oracle.rotate(as_f32(x_in[lo:hi], dtype), np.ascontiguousarray(planes[:, lo:hi]), theta)
        if dtype == "bf16":
            return check_bf16(host[lo:hi], oracle.round_bf16(ref))
        if dtype == "f16":
            return check_bf16(host[lo:hi], oracle.round_f16(ref))
        return check_fp32(host[lo:hi], ref)

    with ThreadPoolExecutor(host_threads()) as ex:
        results = list(ex.map(one, range(0, n, block)))
    ok = all(r[0] for r in results)
    info = {"rows": n, "blocks": len(results)}
    for key in results[0][1] if results else ():
        vals = [r[1][key] for r in results]
        info[key] = all(vals) if isinstance(vals[0], bool) else (sum(vals) if key.startswith("n_") else max(vals))
    assert ok, f"{what}: {info}"
    return info


def expected_flags(b: synth.Prefill, origin: np.ndarray, frame_len: int = synth.FRAME_TOKENS,
                   frame_len_seq=None) -> np.ndarray:
    """Data-fault bits of whole sequences: 1 = more than one marker in the sequence; 2 = the frame
    (frame_len tokens from the marker, or the sequence's own frame_len_seq entry) runs past the end;
    4 = the sequence's frame_len_seq entry is neither 0 nor in [65, 4096] (frame_len is used)."""
    out = np.zeros(b.n_seqs, np.int32)
    for s in range(b.n_seqs):
        lo, hi = b.cu_seqlens[s], b.cu_seqlens[s + 1]
        f = frame_len
        if frame_len_seq is not None and int(frame_len_seq[s]) != 0:
            e = int(frame_len_seq[s])
            if 65 <= e <= 4096:
                f = e
            else:
                out[s] |= 4
        if int((b.ids[lo:hi] == MARKER).sum()) >= 2:
            out[s] |= 1
        if origin[s] >= 0 and origin[s] + f > hi - lo:
            out[s] |= 2
    return out
