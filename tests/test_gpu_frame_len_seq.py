"""GPU parity of per-sequence frame lengths (frame_len_seq) on every plane-deriving call.

One packed batch mixes prompts whose frames end differently -- 65 tokens (Qwen-VL's rule), 67 (this
template), 75 (a run of marker tokens after </image>) -- with entries of 0 (the call's frame_len)
and entries that describe no frame (64, 4097, -1: the call's frame_len, flagged with bit 4).  The
planes, scalars and flags of mrope_planes, and the planes, scalars and every rotated element of
mrope_apply_ids (each of its kernels), mrope_apply_ids_kv and mrope_apply_ids_noalloc, are compared
with the oracle given the same entries.
"""
import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
import oracle
from canvas_rope_rotary_amd import _lib, synth
from gpu_util import (MARKER, compare_heads, compare_heads_all, dev_heads, expected_flags, host_heads, i32,
                      say)

pytestmark = pytest.mark.gpu

ENTRIES = np.array([65, 67, 75, 0, 64, 4097, -1, 70, 4096, 66], np.int32)
MODES = {"default": 0, "chunked": _lib.HOOK_FUSED_CHUNKED, "scan_first": _lib.HOOK_FUSED_SCAN_FIRST,
         "fallback": _lib.HOOK_SCAN_FALLBACK}


def _entries(seed, n):
    return np.random.default_rng(seed).choice(ENTRIES, size=n).astype(np.int32)


def _long_batch(seed, dtype="bf16", head_dim=256):
    """Long sequences with frames before, across and after 512-token chunk edges, so whole chunks
    lie before a frame, cut it, or lie after it (the fused kernels' per-chunk and per-part
    handovers carry the sequence's frame length), plus short ones packed between them."""
    lens = [3000, 2000, 1300, 40, 700, 1, 0, 2600, 90]
    placed = [1000, 470, 500, 3, 440, 0, None, 2030, None]
    g = synth.rng(seed, 4)
    ids = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed) if n > 0])
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    return synth.Prefill(f"long-{seed}", ids, cu, placed, dtype, seed=seed, head_dim=head_dim)


def _check_scalars(got, want, what):
    for g, w, name in zip(got, want, ("start", "amount", "origin")):
        np.testing.assert_array_equal(g.cpu().numpy(), w, err_msg=f"{what} {name}")


@pytest.mark.parametrize("call_len", [67, 70])
def test_planes_mixed_frame_lengths(call_len):
    b = synth.random_batch(501, 80, max_len=800, dtype="bf16", empty_frac=0.05)
    fls = _entries(501, b.n_seqs)
    say(f"case: planes frame_len_seq, call frame_len {call_len}, {b.n_tokens} tokens")
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len=call_len, frame_len_seq=fls)
    pl, st, am, og, fl = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER, frame_len=call_len,
                                   frame_len_seq=i32(fls))
    np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    _check_scalars((st, am, og), (est, eam, eog), "planes")
    np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog, call_len, fls))


def test_planes_pieces_with_frame_lengths():
    """Later pieces (pos_offset, origin_in) of sequences with their own frame lengths: the pieces,
    fed in order, equal the whole sequences."""
    b = synth.random_batch(503, 40, max_len=900, text_frac=0.1)
    fls = _entries(503, b.n_seqs)
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len_seq=fls)
    lens = np.diff(b.cu_seqlens)
    cut = np.clip(np.where(eog >= 0, eog + 70, lens // 2), 0, lens).astype(np.int64)
    got = np.full_like(epl, -7)
    prev = None
    for part in range(2):
        lo = np.zeros_like(cut) if part == 0 else cut
        hi = cut if part == 0 else lens.astype(np.int64)
        rows = np.concatenate([np.arange(b.cu_seqlens[s] + lo[s], b.cu_seqlens[s] + hi[s])
                               for s in range(b.n_seqs)]).astype(np.int64)
        cu = np.zeros(b.n_seqs + 1, np.int32)
        cu[1:] = np.cumsum(hi - lo)
        say(f"case: planes pieces, part {part}, {rows.size} tokens")
        pl, st, am, og, fl = mr.planes(i32(b.ids[rows]), i32(cu), MARKER, pos_offset=i32(lo.astype(np.int32)),
                                       origin_in=prev, frame_len_seq=i32(fls))
        got[:, rows] = pl.cpu().numpy()
        prev = og
    np.testing.assert_array_equal(got, epl)
    _check_scalars((st, am, og), (est, eam, eog), "last piece")


@pytest.fixture(params=list(MODES))
def mode(request):
    prev = _lib.set_test_hooks(MODES[request.param])
    yield request.param
    _lib.set_test_hooks(prev)


def _apply_ids(b, fls, planes_out, call_len=67, pos_offset=None, origin_in=None, what=""):
    qn, kn = b.qk()
    q, k = dev_heads(qn, b.dtype), dev_heads(kn, b.dtype)
    pl = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda") if planes_out else None
    kw = dict(planes_out=pl, frame_len=call_len, frame_len_seq=i32(fls))
    if pos_offset is not None:
        kw.update(pos_offset=i32(pos_offset), origin_in=i32(origin_in))
    st, am, og, fl, _ = mr.apply_ids(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER, **kw)
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, pos_offset, origin_in, call_len, fls)
    if planes_out:
        np.testing.assert_array_equal(pl.cpu().numpy(), epl, err_msg=f"{what} planes")
    _check_scalars((st, am, og), (est, eam, eog), what)
    if pos_offset is None:
        np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog, call_len, fls), err_msg=f"{what} flags")
    compare_heads(host_heads(q), qn, epl, b.dtype, what=f"{what} q")
    compare_heads(host_heads(k), kn, epl, b.dtype, what=f"{what} k")


@pytest.mark.parametrize("planes_out", [False, True])
def test_apply_ids_mixed_frame_lengths(mode, planes_out):
    b = synth.random_batch(511, 60, max_len=1200, dtype="bf16", empty_frac=0.05)
    fls = _entries(511, b.n_seqs)
    say(f"case: apply_ids {mode} frame_len_seq planes_out={planes_out} {b.n_tokens} tokens")
    _apply_ids(b, fls, planes_out, what=f"{mode} ragged")
    lb = _long_batch(512)
    lfls = np.array([75, 65, 67, 75, 0, 4097, 75, 66, 65], np.int32)
    say(f"case: apply_ids {mode} long sequences, {lb.n_tokens} tokens")
    _apply_ids(lb, lfls, planes_out, call_len=70, what=f"{mode} long")


def test_apply_ids_pieces_with_frame_lengths(mode):
    b = synth.random_batch(513, 24, max_len=1500, dtype="bf16")
    g = np.random.default_rng(513)
    off = g.integers(0, 5000, size=b.n_seqs).astype(np.int32)
    oin = np.where(g.uniform(size=b.n_seqs) < 0.4, g.integers(0, 4000, size=b.n_seqs), -1).astype(np.int32)
    fls = _entries(513, b.n_seqs)
    say(f"case: apply_ids {mode} pieces with frame_len_seq, {b.n_tokens} tokens")
    _apply_ids(b, fls, False, pos_offset=off, origin_in=oin, what=f"{mode} pieces")


def test_apply_ids_kv_mixed_frame_lengths():
    b = _long_batch(521)
    fls = np.array([65, 75, 0, 67, 75, 64, 66, 75, 0], np.int32)
    qn, kn = b.qk()
    vn = synth.to_dtype(synth.normal(521, 77, kn.size).reshape(kn.shape), "bf16")
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len_seq=fls)
    T = b.n_tokens
    slots = np.arange(T, dtype=np.int64)
    nb = (T + 15) // 16
    for planes_out in (False, True):
        say(f"case: apply_ids_kv frame_len_seq planes_out={planes_out}, {T} tokens")
        q, k, v = dev_heads(qn, "bf16"), dev_heads(kn, "bf16"), dev_heads(vn, "bf16")
        kc = torch.full((nb, 16, 2, 256), 3.0, dtype=torch.bfloat16, device="cuda")
        vc = torch.full_like(kc, 3.0)
        pl = torch.full((3, T), -9, dtype=torch.int32, device="cuda") if planes_out else None
        st, am, og, fl, _ = mr.apply_ids_kv(q, k, v, i32(b.ids), i32(b.cu_seqlens), kc, vc,
                                            torch.from_numpy(slots).cuda(), MARKER, planes_out=pl,
                                            frame_len_seq=i32(fls))
        if planes_out:
            np.testing.assert_array_equal(pl.cpu().numpy(), epl)
        _check_scalars((st, am, og), (est, eam, eog), "apply_ids_kv")
        np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog, 67, fls))
        compare_heads(host_heads(q), qn, epl, "bf16", what="kv q")
        kc_rows = host_heads(kc).reshape(nb * 16, 2, 256)[:T]
        compare_heads(kc_rows, kn, epl, "bf16", what="kv k cache")
        np.testing.assert_array_equal(host_heads(vc).reshape(nb * 16, 2, 256)[:T], vn)


def test_apply_ids_noalloc_mixed_frame_lengths():
    b = synth.random_batch(531, 50, max_len=1000, dtype="bf16")
    fls = _entries(531, b.n_seqs)
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    say(f"case: apply_ids_noalloc frame_len_seq, {b.n_tokens} tokens")
    st, am, og, fl, _ = mr.apply_ids_noalloc(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER, frame_len_seq=i32(fls))
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len_seq=fls)
    _check_scalars((st, am, og), (est, eam, eog), "noalloc")
    np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog, 67, fls))
    compare_heads(host_heads(q), qn, epl, "bf16", what="noalloc q")
    compare_heads(host_heads(k), kn, epl, "bf16", what="noalloc k")


@pytest.mark.parametrize("planes_out", [False, True])
def test_apply_ids_mixed_frame_lengths_large(planes_out):
    """524,288 ragged tokens in the launch configuration the library picks at that size: every
    plane, scalar, flag and rotated element."""
    b = synth.config5(1 << 19)
    fls = _entries(541, b.n_seqs)
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    pl = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda") if planes_out else None
    say(f"case: apply_ids frame_len_seq large planes_out={planes_out}, {b.n_tokens} tokens")
    st, am, og, fl, _ = mr.apply_ids(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER, planes_out=pl,
                                     frame_len_seq=i32(fls))
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len_seq=fls)
    if planes_out:
        np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    _check_scalars((st, am, og), (est, eam, eog), "large")
    np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog, 67, fls))
    compare_heads_all(q, qn, epl, "bf16", what="large q")
    compare_heads_all(k, kn, epl, "bf16", what="large k")
