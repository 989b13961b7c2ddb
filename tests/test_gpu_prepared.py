"""prepare(): a binding call checked and marshalled once, then launched repeatedly on new contents
of the same buffers.  Each run must equal the plain call on the same inputs (bit for bit) and the
oracle; calls with a workspace must take a fresh epoch every run (a stale epoch would let a run take
an earlier run's look-back words and derive the wrong planes for the new ids)."""
import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
import oracle
from canvas_rope_rotary_amd import synth
from gpu_util import MARKER, compare_heads, dev_heads, host_heads, i32, say

pytestmark = pytest.mark.gpu


def _batches(seeds):
    """Batches of one token count (the prepared buffers are fixed) with different ids."""
    out = []
    for seed in seeds:
        b = synth.random_batch(seed, 40, max_len=900, dtype="bf16")
        out.append(b)
    L = min(b.n_tokens for b in out)
    fixed = []
    for b in out:
        lens = np.diff(b.cu_seqlens).astype(np.int64)
        cut = np.cumsum(lens)
        keep = cut <= L
        lens = lens[keep]
        lens[-1] += L - int(lens.sum())
        cu = np.zeros(lens.size + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        placed = [p for p, k in zip(b.placed, keep) if k]
        fixed.append(synth.Prefill(b.name, b.ids[:L].copy(), cu, placed, "bf16", seed=b.seed))
    return fixed


def test_prepared_apply_ids_takes_fresh_epochs():
    bs = _batches((701, 702, 703, 701))
    n = max(b.n_seqs for b in bs)
    L = bs[0].n_tokens
    # buffers sized for the largest sequence count: every batch is padded with empty sequences
    ids = torch.zeros(L, dtype=torch.int32, device="cuda")
    cu = torch.full((n + 1,), L, dtype=torch.int32, device="cuda")
    q = torch.empty((L, 8, 256), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((L, 2, 256), dtype=torch.bfloat16, device="cuda")
    ws = mr.Workspace(L)
    call = mr.prepare(mr.apply_ids, q, k, ids, cu, MARKER, workspace=ws)
    st, am, og, fl, _ = call.result
    for i, b in enumerate(bs):
        qn, kn = b.qk()
        cub = np.full(n + 1, L, np.int32)
        cub[:b.n_seqs + 1] = b.cu_seqlens
        ids.copy_(i32(b.ids))
        cu.copy_(i32(cub))
        q.copy_(dev_heads(qn, "bf16"))
        k.copy_(dev_heads(kn, "bf16"))
        say(f"case: prepared apply_ids run {i}, {L} tokens")
        call()
        epl, est, eam, eog = oracle.planes(b.ids, cub, MARKER)
        np.testing.assert_array_equal(st.cpu().numpy(), est, err_msg=f"run {i} start")
        np.testing.assert_array_equal(og.cpu().numpy(), eog, err_msg=f"run {i} origin")
        compare_heads(host_heads(q), qn, epl, "bf16", what=f"run {i} q")
        compare_heads(host_heads(k), kn, epl, "bf16", what=f"run {i} k")


def test_prepared_planes_and_decode_equal_plain_calls():
    b = synth.random_batch(711, 30, max_len=600)
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    call = mr.prepare(mr.planes, ids, cu, MARKER)
    pl, st, am, og, fl = call()
    ref = mr.planes(ids, cu, MARKER)
    for x, y in zip((pl, st, am, og, fl), ref):
        assert torch.equal(x, y)

    d = synth.config4(n_seqs=256, num_blocks=512)
    qn, kn = d.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    q2, k2 = q.clone(), k.clone()
    kc = torch.zeros((d.num_blocks, d.block_size, 2, 256), dtype=torch.bfloat16, device="cuda")
    kc2 = kc.clone()
    pos, amt, slots = (torch.from_numpy(x).cuda() for x in (d.pos, d.amount, d.slot_mapping))
    dec = mr.prepare(mr.decode, q, k, pos, amt, kc, slots)
    say("case: prepared decode, two steps")
    for step in range(2):
        dec()
        mr.decode(q2, k2, pos, amt, kc2, slots)
        torch.cuda.synchronize()
        assert torch.equal(q.view(torch.int16), q2.view(torch.int16)), step
        assert torch.equal(kc.view(torch.int16), kc2.view(torch.int16)), step
        if step == 0:
            planes = np.stack([d.pos - d.amount] * 3).astype(np.int32)
            compare_heads(host_heads(q), qn, planes, "bf16", what="prepared decode q")
        pos += 1


def test_prepare_rejects_a_function_without_a_library_call():
    with pytest.raises(ValueError):
        mr.prepare(lambda: None)
