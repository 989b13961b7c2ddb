"""Element offsets past 2^31: 1,310,720 ragged bf16 tokens, so Q [L, 8, 256] holds 2.68e9 elements and
every token from 1,048,576 on sits past element 2^31 of Q.  mrope_planes, mrope_apply and both fused
routes (the scan-first kernel; the two-launch planes_out route of the cache-writing call) must match
the oracle there: planes on every token, rotated heads on every token past the boundary and the
first ones before it."""
import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
import oracle
from canvas_rope_rotary_amd import synth
from gpu_util import MARKER, compare_heads, dev_heads, host_heads, i32, say

pytestmark = pytest.mark.gpu

L = 1_310_720
BOUNDARY = (1 << 31) // (8 * 256)  # first token whose Q elements lie past 2^31


@pytest.fixture(scope="module")
def batch():
    b = synth.config5(L)
    qn, kn = b.qk()
    epl, est, eam, eog = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    return b, qn, kn, epl, est


def _check(q, k, qn, kn, epl, what):
    rows = np.r_[0:2048, BOUNDARY - 8:L]
    compare_heads(host_heads(q[torch.from_numpy(rows).cuda()]), qn[rows], epl[:, rows], "bf16", what=f"{what} q")
    compare_heads(host_heads(k[torch.from_numpy(rows).cuda()]), kn[rows], epl[:, rows], "bf16", what=f"{what} k")


def test_planes_and_apply_past_2_31_elements(batch):
    b, qn, kn, epl, est = batch
    assert qn.shape[0] * 8 * 256 > (1 << 31) and BOUNDARY < L
    say(f"case: planes + apply, {L} tokens")
    pl, st, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    mr.apply(q, k, pl)
    _check(q, k, qn, kn, epl, "apply")


def test_fused_past_2_31_elements(batch):
    b, qn, kn, epl, est = batch
    say(f"case: apply_ids (scan-first), {L} tokens")
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    pl = torch.full((3, L), -7, dtype=torch.int32, device="cuda")
    st, *_ = mr.apply_ids(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER, planes_out=pl)
    np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    _check(q, k, qn, kn, epl, "apply_ids")


def test_cache_write_past_2_31_elements(batch):
    """The cache-writing call with planes_out past 262,144 tokens: the scan into planes_out, then the
    rotation with the cache write; K and V rows land in a 16-token paged cache in token order."""
    b, qn, kn, epl, est = batch
    say(f"case: apply_ids_kv with planes_out, {L} tokens")
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    v = k.clone()
    nb = L // 16
    kc = torch.zeros((nb, 16, 2, 256), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    slots = torch.arange(L, dtype=torch.int64, device="cuda")
    pl = torch.full((3, L), -7, dtype=torch.int32, device="cuda")
    mr.apply_ids_kv(q, k, v, i32(b.ids), i32(b.cu_seqlens), kc, vc, slots, MARKER, planes_out=pl)
    np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    rows = np.r_[0:2048, BOUNDARY - 8:L]
    ridx = torch.from_numpy(rows).cuda()
    compare_heads(host_heads(q[ridx]), qn[rows], epl[:, rows], "bf16", what="kv q")
    compare_heads(host_heads(kc.view(L, 2, 256)[ridx]), kn[rows], epl[:, rows], "bf16", what="kv k cache")
    np.testing.assert_array_equal(host_heads(vc.view(L, 2, 256)[ridx]), kn[rows])
