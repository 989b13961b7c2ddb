"""Helpers of the GPU parity tests: move seeded inputs to the device, read results back, and call the
oracle on the same inputs.  No method arithmetic here."""
from __future__ import annotations

import sys

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


def expected_flags(b: synth.Prefill, origin: np.ndarray) -> np.ndarray:
    """Data-fault bits: >1 marker in the sequence; frame (67 tokens from the marker) past the end."""
    out = np.zeros(b.n_seqs, np.int32)
    for s in range(b.n_seqs):
        lo, hi = b.cu_seqlens[s], b.cu_seqlens[s + 1]
        if int((b.ids[lo:hi] == MARKER).sum()) >= 2:
            out[s] |= 1
        if origin[s] >= 0 and origin[s] + synth.FRAME_TOKENS > hi - lo:
            out[s] |= 2
    return out
