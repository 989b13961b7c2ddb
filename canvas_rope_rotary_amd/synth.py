"""Seeded synthetic inputs for canvas M-RoPE.

This module builds token ids, sequence lengths and Q/K/cache tensors only.  It holds none of the
method's arithmetic (no planes, no start/amount, no rotation): both the HIP path and the CPU oracle
take their inputs from here.

Prompt layout (Hugging Face card "MiniCPM-V-4.7-1B -- Core AI", sections "Prompt" and "How the VLM
rides the text-only engine"): text, then the frame <image> (248078), 64 x <|image_pad|> (248056),
</image> (248079) and one "\\n" (198), then text.  Text ids are uniform over the vocabulary
(248,094) with the three image ids excluded.

Randomness: numpy PCG64.  Every array comes from its own stream, keyed by (seed, stream tag, chunk),
so large Q/K tensors can be filled by parallel threads and still come out identical.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

IMAGE_ID = 248078        # <image>
IMAGE_END_ID = 248079    # </image>
IMAGE_PAD_ID = 248056    # <|image_pad|>
NEWLINE_ID = 198         # "\n"
VOCAB = 248094
IMAGE_ROWS = 64          # one 448x448 image -> 64 rows
FRAME = [IMAGE_ID] + [IMAGE_PAD_ID] * IMAGE_ROWS + [IMAGE_END_ID, NEWLINE_ID]
FRAME_TOKENS = len(FRAME)

# stream tags
_Q, _K, _LEN, _ORIGIN, _IDS, _POS, _SLOT = range(7)
_CHUNK = 1 << 22


def rng(seed: int, tag: int, chunk: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(entropy=seed, spawn_key=(tag, chunk))))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal(seed: int, tag: int, n: int) -> np.ndarray:
    """n standard-normal float32 values, chunked streams, filled in parallel."""
    out = np.empty(n, np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def fill(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        rng(seed, tag, c).standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even, via torch's conversion."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> IEEE half bit patterns (uint16), round to nearest even (numpy's conversion)."""
    return np.ascontiguousarray(x, np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """IEEE half bit patterns -> the float32 values they represent (exact)."""
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float32)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> the float32 values they represent (exact)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values in the workload's storage form (bit patterns for the 16-bit types)."""
    if dtype == "bf16":
        return to_bf16_bits(x)
    if dtype == "f16":
        return to_f16_bits(x)
    return np.ascontiguousarray(x, np.float32)


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage form back to the float32 values (exact)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype == "f16":
        return f16_bits_to_f32(x)
    return np.asarray(x, np.float32)


def text_ids(g: np.random.Generator, n: int) -> np.ndarray:
    ids = g.integers(0, VOCAB, size=n, dtype=np.int64)
    bad = np.isin(ids, (IMAGE_ID, IMAGE_END_ID, IMAGE_PAD_ID))
    while bad.any():
        ids[bad] = g.integers(0, VOCAB, size=int(bad.sum()), dtype=np.int64)
        bad = np.isin(ids, (IMAGE_ID, IMAGE_END_ID, IMAGE_PAD_ID))
    return ids.astype(np.int32)


def prompt_ids(g: np.random.Generator, n: int, origin: int | None, extra_markers=()) -> np.ndarray:
    """n ids: text, with the image frame placed at `origin` (None = text only).  The frame is cut
    off if it runs past n.  `extra_markers` puts further <image> ids at the given positions."""
    ids = text_ids(g, n)
    if origin is not None:
        m = min(FRAME_TOKENS, n - origin)
        if m > 0:
            ids[origin:origin + m] = FRAME[:m]
    for p in extra_markers:
        ids[p] = IMAGE_ID
    return ids


@dataclass
class Prefill:
    name: str
    ids: np.ndarray            # [L] int32
    cu_seqlens: np.ndarray     # [n+1] int32
    placed: list               # frame position used to build each sequence (None = text only)
    dtype: str                 # "f32" | "bf16" | "f16"
    n_q_heads: int = 8
    n_k_heads: int = 2
    head_dim: int = 256
    rot_dim: int = 64
    theta: float = 1e7
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    def qk(self):
        """(q, k) as numpy arrays [L, H, D]: float32 for "f32", uint16 bit patterns for "bf16" / "f16"."""
        L, D = self.n_tokens, self.head_dim
        q = normal(self.seed, _Q, L * self.n_q_heads * D).reshape(L, self.n_q_heads, D)
        k = normal(self.seed, _K, L * self.n_k_heads * D).reshape(L, self.n_k_heads, D)
        return to_dtype(q, self.dtype), to_dtype(k, self.dtype)


def _batch(name, seed, lengths, placed, dtype, **kw) -> Prefill:
    g = rng(seed, _IDS)
    ids = [prompt_ids(g, n, o) for n, o in zip(lengths, placed)]
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    flat = np.concatenate(ids).astype(np.int32) if ids else np.zeros(0, np.int32)
    return Prefill(name=name, ids=flat, cu_seqlens=cu, placed=list(placed), dtype=dtype, seed=seed, **kw)


def config1() -> Prefill:
    """Single image prompt, fp32: tokens 0..5 text, <image> at 6, 64 rows, </image>, "\\n", then
    text to L = 110.  Q [110, 8, 256], K [110, 2, 256]."""
    return _batch("single-image-L110-f32", 1, [110], [6], "f32")


def config2() -> Prefill:
    """64 image prompts of 4096 tokens, <image> at O ~ U{0..512}, bf16."""
    g = rng(2, _ORIGIN)
    origins = [int(o) for o in g.integers(0, 513, size=64)]
    return _batch("64x4096-image-bf16", 2, [4096] * 64, origins, "bf16")


def config3() -> Prefill:
    """8 sequences of 32768 tokens, one image block each at O ~ U{0..30000}, bf16, ids fused."""
    g = rng(3, _ORIGIN)
    origins = [int(o) for o in g.integers(0, 30001, size=8)]
    return _batch("8x32768-image-bf16-fused", 3, [32768] * 8, origins, "bf16")


def ragged_lengths(seed: int, total: int, hi: int = 16384, lo_image: int = FRAME_TOKENS, lo_text: int = 64):
    """Log-uniform lengths in [lo, hi]; even-indexed sequences are image prompts (lo_image), odd ones
    text only (lo_text); the last one is trimmed to hit `total` (merged into the previous sequence if
    that leaves it below its lower bound)."""
    g = rng(seed, _LEN)
    lengths, kinds = [], []
    acc = 0
    while acc < total:
        image = len(lengths) % 2 == 0
        lo = lo_image if image else lo_text
        n = int(np.floor(np.exp(g.uniform(np.log(lo), np.log(hi + 1)))))
        n = min(max(n, lo), hi)
        lengths.append(n)
        kinds.append(image)
        acc += n
    over = acc - total
    if over:
        lengths[-1] -= over
        lo = lo_image if kinds[-1] else lo_text
        if lengths[-1] < lo:
            lengths[-2] += lengths[-1]
            lengths.pop()
            kinds.pop()
    return lengths, kinds


def config5(total: int = 1 << 20) -> Prefill:
    """Ragged batch via cu_seqlens: `total` tokens, log-uniform lengths in [64, 16384]; half the
    sequences text only, half with one image block at O ~ U{0..n-67}; bf16."""
    lengths, kinds = ragged_lengths(5, total)
    g = rng(5, _ORIGIN)
    placed = [int(g.integers(0, n - FRAME_TOKENS + 1)) if img else None for n, img in zip(lengths, kinds)]
    return _batch(f"ragged-{total}-half-text-bf16", 5, lengths, placed, "bf16")


@dataclass
class Decode:
    name: str
    n_seqs: int
    pos: np.ndarray           # [S] int32
    amount: np.ndarray        # [S] int32
    slot_mapping: np.ndarray  # [S] int64
    num_blocks: int
    block_size: int
    dtype: str
    n_q_heads: int = 8
    n_k_heads: int = 2
    head_dim: int = 256
    rot_dim: int = 64
    theta: float = 1e7
    seed: int = 0
    sentinel_bits: int = 0xFFC1   # a NaN pattern no rotated value can take

    def qk(self):
        D = self.head_dim
        q = normal(self.seed, _Q, self.n_seqs * self.n_q_heads * D).reshape(self.n_seqs, self.n_q_heads, D)
        k = normal(self.seed, _K, self.n_seqs * self.n_k_heads * D).reshape(self.n_seqs, self.n_k_heads, D)
        return to_dtype(q, self.dtype), to_dtype(k, self.dtype)


def config4(n_seqs: int = 4096, num_blocks: int = 65536, block_size: int = 16) -> Decode:
    """Decode step: one new token per sequence at position p ~ U{100..32000}, amount = 58 (the
    shift every image prompt of the pages carries), K scattered into a paged cache of 16-token
    blocks through a random block permutation."""
    g = rng(4, _POS)
    pos = g.integers(100, 32001, size=n_seqs).astype(np.int32)
    amount = np.full(n_seqs, 58, np.int32)
    perm = rng(4, _SLOT).permutation(num_blocks)[:n_seqs].astype(np.int64)
    slots = perm * block_size + (pos.astype(np.int64) % block_size)
    return Decode(name=f"decode-{n_seqs}-paged{block_size}-bf16", n_seqs=n_seqs, pos=pos, amount=amount,
                  slot_mapping=slots, num_blocks=num_blocks, block_size=block_size, dtype="bf16", seed=4)


def random_batch(seed: int, n_seqs: int, max_len: int = 300, min_len: int = 1, text_frac: float = 0.3,
                 dtype: str = "bf16", empty_frac: float = 0.0) -> Prefill:
    """Small ragged batch for fuzzing: lengths in [min_len, max_len], a mix of text-only prompts,
    frames at 0, at n-67, at random places, frames cut off by the end of the sequence, sequences
    with a second marker, and (optionally) empty sequences."""
    g = rng(seed, _LEN)
    lengths, placed, extras = [], [], []
    for _ in range(n_seqs):
        if empty_frac and g.uniform() < empty_frac:
            lengths.append(0)
            placed.append(None)
            extras.append(())
            continue
        n = int(g.integers(min_len, max_len + 1))
        r = g.uniform()
        if r < text_frac:
            o = None
        else:
            c = g.integers(0, 4)
            if c == 0:
                o = 0
            elif c == 1:
                o = max(0, n - FRAME_TOKENS)
            else:
                o = int(g.integers(0, n))
        ex = ()
        if o is not None and n - o > 1 and g.uniform() < 0.15:
            ex = (int(g.integers(o + 1, n)),)
        lengths.append(n)
        placed.append(o)
        extras.append(ex)
    gi = rng(seed, _IDS)
    ids = [prompt_ids(gi, n, o, ex) for n, o, ex in zip(lengths, placed, extras)]
    cu = np.zeros(n_seqs + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    flat = np.concatenate(ids).astype(np.int32) if sum(lengths) else np.zeros(0, np.int32)
    return Prefill(name=f"fuzz-{seed}", ids=flat, cu_seqlens=cu, placed=placed, dtype=dtype, seed=seed)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
