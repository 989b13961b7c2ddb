"""canvas_rope_rotary_amd -- canvas M-RoPE for MI355X (gfx950).

Thin Python binding over ``libmrope.so`` (C ABI declared in ``include/mrope.h``): every function here
only checks and marshals arguments -- pointers, strides, sizes and the current HIP stream -- and
calls one C entry point.  All computation happens in the HIP kernels; there is no CPU fallback, and
the functions raise if the library was not built or no GPU is present.

What the path computes (Hugging Face card "MiniCPM-V-4.7-1B -- Core AI", sections "What it is" and
"How the VLM rides the text-only engine"; Core AI model-zoo page "MiniCPM-V-4.7-1B: canvas M-RoPE on
the Qwen3.5 hybrid, on Core AI", section "The canvas rule and why the gate is on the planes"):

* ``planes``    token ids + packed sequences -> per-token (T, H, W) planes, start and amount;
* ``apply``     rotate Q and K heads (first 64 dims, 32 frequencies in interleaved sections
                [11, 11, 10]) with given planes, in place or out of place;
* ``apply_ids`` both in one launch; ``apply_ids_noalloc`` the same with the library's static
                per-GPU scratch in place of a workspace (for callers that cannot allocate);
* ``apply_kv`` / ``apply_ids_kv``  the same with the prefill cache write: Q in place, K rotated and
                V copied into paged K/V caches at each token's slot;
* ``decode``    one new token per sequence at p - amount; Q in place, K (and V) into paged caches.
"""
from __future__ import annotations

from . import _lib
from ._lib import (MROPE_BF16, MROPE_F16, MROPE_F32, MarkerFlags, MropeError, TEXT_ONLY_START, Workspace, apply, apply_ids,
                   apply_ids_kv, apply_ids_noalloc, apply_kv, check_slots, cu_seqlens_from_lens, decode, library_path,
                   planes, prepare, PreparedCall)

IMAGE_ID = 248078
DEFAULT_THETA = 1e7

__all__ = ["planes", "apply", "apply_ids", "apply_ids_noalloc", "apply_kv", "apply_ids_kv", "decode", "Workspace", "MropeError", "MarkerFlags",
           "check_slots", "prepare", "PreparedCall", "cu_seqlens_from_lens", "library_path", "IMAGE_ID", "DEFAULT_THETA", "TEXT_ONLY_START",
           "MROPE_F32", "MROPE_BF16", "MROPE_F16"]
