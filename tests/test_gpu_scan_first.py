"""GPU parity of the scan-first fused kernel (mrope_apply_ids for large inputs) at small sizes.

The library picks the scan-first kernel by size; the test hooks force it (and its fallback, in which
every rotation workgroup scans its own chunk instead of reading the scan workgroups' handover) on
inputs the oracle checks in seconds: ragged batches with many tiny and empty sequences, frames on
and across chunk edges, pieces of sequences (pos_offset / origin_in), other frame lengths, planes_out
on and off, in place and out of place.  Every rotated element, every plane and every scalar is
compared with the oracle.
"""
import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
import oracle
from canvas_rope_rotary_amd import _lib, synth
from gpu_util import MARKER, compare_heads, dev_heads, expected_flags, host_heads, i32, say

pytestmark = pytest.mark.gpu

MODES = {"scan_first": _lib.HOOK_FUSED_SCAN_FIRST, "fallback": _lib.HOOK_SCAN_FALLBACK,
         "chunked": _lib.HOOK_FUSED_CHUNKED}


@pytest.fixture(params=list(MODES))
def mode(request):
    prev = _lib.set_test_hooks(MODES[request.param])
    yield request.param
    _lib.set_test_hooks(prev)


def _run(b, mode, planes_out, pos_offset=None, origin_in=None, frame_len=67, out_of_place=False):
    qn, kn = b.qk()
    q, k = dev_heads(qn, b.dtype), dev_heads(kn, b.dtype)
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    pl = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda") if planes_out else None
    kw = dict(planes_out=pl, frame_len=frame_len)
    if pos_offset is not None:
        kw.update(pos_offset=i32(pos_offset), origin_in=i32(origin_in))
    qo = ko = None
    if out_of_place:
        qo, ko = torch.full_like(q, -5.0), torch.full_like(k, -5.0)
        kw.update(q_out=qo, k_out=ko)
    st, am, og, fl, _ = mr.apply_ids(q, k, ids, cu, MARKER, **kw)
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, pos_offset, origin_in, frame_len)
    what = f"{b.name} {mode} planes_out={planes_out}"
    if planes_out:
        np.testing.assert_array_equal(pl.cpu().numpy(), epl, err_msg=f"{what} planes")
    for got, want, name in ((st, est, "start"), (am, eam, "amount"), (og, eog, "origin")):
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"{what} {name}")
    if pos_offset is None and frame_len == 67:
        np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog), err_msg=f"{what} flags")
    rq, rk = (qo, ko) if out_of_place else (q, k)
    compare_heads(host_heads(rq), qn, epl, b.dtype, what=f"{what} q")
    compare_heads(host_heads(rk), kn, epl, b.dtype, what=f"{what} k")
    if out_of_place:
        np.testing.assert_array_equal(host_heads(q), qn, err_msg=f"{what}: q input changed")


@pytest.mark.parametrize("seed,dtype,n_seqs,max_len,empty", [
    (301, "bf16", 40, 900, 0.0), (302, "f32", 30, 700, 0.1), (303, "bf16", 300, 90, 0.2),
    (304, "f16", 12, 3000, 0.0), (305, "bf16", 1, 1, 0.0),
])
@pytest.mark.parametrize("planes_out", [False, True])
def test_ragged_batches(mode, seed, dtype, n_seqs, max_len, empty, planes_out):
    b = synth.random_batch(seed, n_seqs, max_len=max_len, dtype=dtype, empty_frac=empty)
    say(f"case: {mode} fuzz seed={seed} {dtype} seqs={n_seqs} tokens={b.n_tokens} planes_out={planes_out}")
    _run(b, mode, planes_out)


def test_many_tiny_sequences(mode):
    """5000 sequences of 0..3 tokens: hundreds of sequences in a chunk, every 32-token part holds
    several (their planes go over token by token)."""
    g = np.random.default_rng(7)
    lens = g.integers(0, 4, size=5000)
    ids = synth.text_ids(synth.rng(7, 4), int(lens.sum()))
    ids[g.integers(0, ids.size, size=200)] = MARKER
    cu = np.zeros(lens.size + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill("tiny", ids, cu, [None] * lens.size, "bf16", seed=7)
    say(f"case: {mode} tiny sequences, {b.n_tokens} tokens")
    for planes_out in (False, True):
        _run(b, mode, planes_out)


def test_chunk_and_part_edges(mode):
    """Sequences and frames on and across 512-token chunk and 32-token part edges, lengths 31..33
    and 511..513, empties, a long sequence whose look-back crosses many chunks."""
    lens = [512, 31, 33, 1, 511, 513, 32, 0, 0, 1024, 600, 9000, 1700, 3]
    placed = [0, None, 0, 0, 444, 31, None, None, None, 500, 510, 5000, 1023, None]
    g = synth.rng(13, 4)
    ids = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed) if n > 0])
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    for dtype, hd in (("bf16", 256), ("f32", 64)):
        b = synth.Prefill(f"edges-{dtype}", ids, cu, placed, dtype, seed=13, head_dim=hd)
        say(f"case: {mode} edges {dtype} head_dim {hd}")
        for planes_out in (False, True):
            _run(b, mode, planes_out)


def test_pieces_and_frame_lengths(mode):
    """Later pieces of sequences (pos_offset, origin_in carried from an earlier piece, cuts inside
    and after the frame) and longer frames."""
    b = synth.random_batch(311, 24, max_len=1500, dtype="bf16")
    g = np.random.default_rng(311)
    off = g.integers(0, 5000, size=b.n_seqs).astype(np.int32)
    oin = np.where(g.uniform(size=b.n_seqs) < 0.4, g.integers(0, 4000, size=b.n_seqs), -1).astype(np.int32)
    say(f"case: {mode} pieces, {b.n_tokens} tokens")
    _run(b, mode, False, pos_offset=off, origin_in=oin)
    _run(b, mode, True, pos_offset=off, origin_in=oin, frame_len=75)
    _run(b, mode, False, frame_len=65)


def test_out_of_place(mode):
    b = synth.random_batch(321, 16, max_len=2000, dtype="bf16")
    say(f"case: {mode} out of place, {b.n_tokens} tokens")
    _run(b, mode, False, out_of_place=True)


def test_repeated_calls_share_a_workspace(mode):
    """Back-to-back calls on one workspace with different batches: a call never takes a handover
    word of an earlier call (each carries its launch's epoch), with caller epochs and with the
    device counter (graph capture)."""
    ws = mr.Workspace(20000)
    for i, seed in enumerate((331, 332, 333, 331)):
        b = synth.random_batch(seed, 20, max_len=1000, dtype="bf16")
        qn, kn = b.qk()
        q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
        if i % 2:
            g = torch.cuda.CUDAGraph()
            ids, cu = i32(b.ids), i32(b.cu_seqlens)
            with torch.cuda.graph(g):
                mr.apply_ids(q, k, ids, cu, MARKER, workspace=ws)
            q.copy_(dev_heads(qn, "bf16"))
            k.copy_(dev_heads(kn, "bf16"))
            g.replay()
            torch.cuda.synchronize()
        else:
            mr.apply_ids(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER, workspace=ws)
        epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
        compare_heads(host_heads(q), qn, epl, "bf16", what=f"{mode} call {i} q")
        compare_heads(host_heads(k), kn, epl, "bf16", what=f"{mode} call {i} k")


def test_two_level_sequence_search(mode):
    """20,000 sequences of 0..12 tokens: past 8,063 sequences the bracket search takes two levels
    before the window load, and chunks hold dozens of sequences (walked, searched, or counted past
    the window)."""
    g = np.random.default_rng(17)
    lens = g.integers(0, 13, size=20000)
    ids = synth.text_ids(synth.rng(17, 4), int(lens.sum()))
    ids[g.integers(0, ids.size, size=3000)] = MARKER
    cu = np.zeros(lens.size + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill("two-level", ids, cu, [None] * lens.size, "bf16", seed=17)
    say(f"case: {mode} 20000 sequences, {b.n_tokens} tokens")
    _run(b, mode, True)
    fls = g.choice(np.array([65, 67, 75, 0], np.int32), size=lens.size)
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    st, am, og, fl, _ = mr.apply_ids(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER, frame_len_seq=i32(fls))
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len_seq=fls)
    for got, want, name in ((st, est, "start"), (am, eam, "amount"), (og, eog, "origin")):
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"{mode} two-level {name}")
    compare_heads(host_heads(q), qn, epl, "bf16", what=f"{mode} two-level q")
    compare_heads(host_heads(k), kn, epl, "bf16", what=f"{mode} two-level k")
