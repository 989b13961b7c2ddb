"""mrope_apply_ids_noalloc (the library's static per-GPU scratch in place of a workspace) against
mrope_apply_ids with a caller workspace: the same planes, scalars, flags and rotated Q/K bit for
bit, on two calls in a row -- a large ragged batch, then a smaller one -- and when captured in a
graph and replayed with new inputs."""
import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
from canvas_rope_rotary_amd import synth
from gpu_util import MARKER, dev_heads, i32, say

pytestmark = pytest.mark.gpu


def _both(b, planes_out=True, frame_len=67):
    """Run the batch through mrope_apply_ids (workspace) and mrope_apply_ids_noalloc; return both
    results as host arrays."""
    qn, kn = b.qk()
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    out = []
    for noalloc in (False, True):
        q, k = dev_heads(qn, b.dtype), dev_heads(kn, b.dtype)
        pl = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda") if planes_out else None
        n = b.n_seqs
        st, am, og, fl = (torch.full((n,), -9, dtype=torch.int32, device="cuda") for _ in range(4))
        fn = mr.apply_ids_noalloc if noalloc else mr.apply_ids
        fn(q, k, ids, cu, MARKER, planes_out=pl, start=st, amount=am, origin=og, seq_flags=fl, frame_len=frame_len)
        torch.cuda.synchronize()
        out.append([t.cpu() for t in (q.view(torch.int16) if q.dtype != torch.float32 else q,
                                      k.view(torch.int16) if k.dtype != torch.float32 else k, st, am, og, fl)]
                   + ([pl.cpu()] if planes_out else []))
    return out


def _same(a, b, what):
    names = ("q", "k", "start", "amount", "origin", "flags", "planes")
    for x, y, name in zip(a, b, names):
        assert torch.equal(x, y), f"{what}: {name} differs"


def test_noalloc_matches_workspace_call_twice_then_smaller():
    big = synth.config5(1 << 19)          # 524,288 ragged tokens: the scan-first kernel
    small = synth.random_batch(401, 60, max_len=700, dtype="bf16")
    for b in (big, small, big):
        say(f"case: noalloc vs workspace, {b.name}, {b.n_tokens} tokens")
        ref, got = _both(b)
        _same(ref, got, b.name)
    b = synth.random_batch(402, 30, max_len=400, dtype="f32")
    say(f"case: noalloc vs workspace, {b.name} f32, frame_len 75, no planes_out")
    ref, got = _both(b, planes_out=False, frame_len=75)
    _same(ref, got, b.name)


def test_noalloc_rejects_more_tokens_than_its_scratch():
    T = mr._lib.NOALLOC_MAX_TOKENS + 1
    q = torch.empty((T, 1, 64), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    cu = i32([0, T])
    with pytest.raises(mr.MropeError) as e:
        mr.apply_ids_noalloc(q, None, ids, cu, MARKER)
    assert e.value.status == 4


def test_noalloc_in_a_graph_replayed_with_new_inputs():
    """Captured once, replayed three times with new ids and heads copied in between: every replay
    equals a workspace call on the same inputs (the device epoch counter keeps the replays apart)."""
    batches = [synth.random_batch(410 + i, 24, max_len=900, dtype="bf16") for i in range(3)]
    T = max(b.n_tokens for b in batches)
    n = max(b.n_seqs for b in batches)
    q = torch.zeros((T, 8, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((T, 2, 256), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    cu = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    st, am, og, fl = (torch.zeros(n, dtype=torch.int32, device="cuda") for _ in range(4))
    # pad every batch to T tokens and n sequences: trailing empty sequences, filler tokens in the last
    padded = []
    for b in batches:
        cuv = np.concatenate([b.cu_seqlens, np.full(n - b.n_seqs, b.n_tokens, np.int32)])
        cuv[-1] = T
        idv = np.concatenate([b.ids, synth.text_ids(synth.rng(9, 4), T - b.n_tokens)])
        qn, kn = synth.Prefill("pad", idv, cuv, [], "bf16", seed=b.seed).qk()
        padded.append((idv, cuv, qn, kn))
    mr.apply_ids_noalloc(q, k, ids, cu, MARKER)  # first call on the device: not captured
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            mr.apply_ids_noalloc(q, k, ids, cu, MARKER, start=st, amount=am, origin=og, seq_flags=fl)
    torch.cuda.synchronize()
    for i, (idv, cuv, qn, kn) in enumerate(padded):
        ids.copy_(i32(idv))
        cu.copy_(i32(cuv))
        q.copy_(dev_heads(qn, "bf16"))
        k.copy_(dev_heads(kn, "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        q2, k2 = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
        r = mr.apply_ids(q2, k2, i32(idv), i32(cuv), MARKER)
        torch.cuda.synchronize()
        assert torch.equal(q.view(torch.int16), q2.view(torch.int16)), f"replay {i}: q"
        assert torch.equal(k.view(torch.int16), k2.view(torch.int16)), f"replay {i}: k"
        for got, want, name in zip((st, am, og, fl), r[:4], ("start", "amount", "origin", "flags")):
            assert torch.equal(got, want), f"replay {i}: {name}"
