"""GPU parity of mrope_apply, of the fused mrope_apply_ids and of the cache-writing calls
(mrope_apply_kv, mrope_apply_ids_kv) in fp32 in both lane layouts: sixteen lanes a token (the default
for 8 Q + 2 K heads) and eight (MROPE_HOOK_F32_EIGHT_LANES; for the cache writes, the generic
kernels).  Each is compared with the oracle (fp32 gate) and with the other bit for bit, in place and
out of place, on strided views, and past the size from which in-place stores take the non-temporal
hint."""
import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
import oracle
from canvas_rope_rotary_amd import _lib, synth
from gpu_util import MARKER, compare_heads, compare_heads_all, dev_heads, host_heads, i32, say

pytestmark = pytest.mark.gpu

LAYOUTS = {"sixteen": 0, "eight": _lib.HOOK_F32_EIGHT_LANES}


def _both_layouts(run, extra_hooks=0):
    out = {}
    for name, hook in LAYOUTS.items():
        prev = _lib.set_test_hooks(hook | extra_hooks)
        try:
            out[name] = run()
        finally:
            _lib.set_test_hooks(prev)
    return out


@pytest.mark.parametrize("seed,n_seqs,max_len", [(601, 1, 110), (602, 30, 700), (603, 7, 5000)])
@pytest.mark.parametrize("out_of_place", [False, True])
def test_f32_layouts_match_oracle_and_each_other(seed, n_seqs, max_len, out_of_place):
    b = synth.random_batch(seed, n_seqs, max_len=max_len, min_len=max_len if n_seqs == 1 else 1, dtype="f32")
    qn, kn = b.qk()
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    say(f"case: fp32 layouts seed={seed} tokens={b.n_tokens} out_of_place={out_of_place}")

    def run():
        q, k = dev_heads(qn, "f32"), dev_heads(kn, "f32")
        if out_of_place:
            qo, ko = torch.full_like(q, -3.0), torch.full_like(k, -3.0)
            mr.apply(q, k, pl, q_out=qo, k_out=ko)
            np.testing.assert_array_equal(host_heads(q), qn)
            return host_heads(qo), host_heads(ko)
        mr.apply(q, k, pl)
        return host_heads(q), host_heads(k)

    res = _both_layouts(run)
    for name, (q, k) in res.items():
        compare_heads(q, qn, epl, "f32", what=f"{name} q")
        compare_heads(k, kn, epl, "f32", what=f"{name} k")
    for a, c in zip(res["sixteen"], res["eight"]):
        np.testing.assert_array_equal(a.view(np.uint32), c.view(np.uint32))


def test_f32_layouts_on_strided_views():
    """Q and K as head-slices of one fused [T, 12, 256] projection buffer."""
    b = synth.random_batch(611, 12, max_len=900, dtype="f32")
    qn, kn = b.qk()
    T = b.n_tokens
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    filler = np.full((T, 2, 256), 7.0, np.float32)
    say(f"case: fp32 layouts on views, {T} tokens")

    def run():
        fused = torch.from_numpy(np.concatenate([qn, kn, filler], axis=1)).cuda()
        mr.apply(fused[:, :8], fused[:, 8:10], pl)
        out = fused.cpu().numpy()
        np.testing.assert_array_equal(out[:, 10:], filler)
        return out[:, :8].copy(), out[:, 8:10].copy()

    res = _both_layouts(run)
    for name, (q, k) in res.items():
        compare_heads(q, qn, epl, "f32", what=f"{name} view q")
        compare_heads(k, kn, epl, "f32", what=f"{name} view k")


@pytest.mark.parametrize("fused", [False, True])
def test_f32_layouts_past_the_store_hint_size(fused):
    """48 x 4,096 fp32 tokens write 402 MB in place: the hinted stores of both layouts, through
    mrope_apply and mrope_apply_ids; the default layout's every element against the oracle, the
    other's bit for bit against it."""
    b = synth.random_batch(621, 48, max_len=4096, min_len=4096, dtype="f32")
    qn, kn = b.qk()
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    say(f"case: fp32 layouts past the hint size, fused={fused}, {b.n_tokens} tokens")

    def run():
        q, k = dev_heads(qn, "f32"), dev_heads(kn, "f32")
        if fused:
            mr.apply_ids(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER)
        else:
            mr.apply(q, k, pl)
        torch.cuda.synchronize()
        return q, k

    res = _both_layouts(run)
    q, k = res["sixteen"]
    compare_heads_all(q, qn, epl, "f32", what="q")
    compare_heads_all(k, kn, epl, "f32", what="k")
    for a, c in zip(res["sixteen"], res["eight"]):
        assert torch.equal(a.view(torch.int32), c.view(torch.int32)), "layouts differ"


@pytest.mark.parametrize("seed,n_seqs,max_len", [(631, 1, 110), (632, 40, 900), (633, 6, 4096)])
@pytest.mark.parametrize("planes_out", [False, True])
@pytest.mark.parametrize("kernel", ["chunked", "scan_first"])
def test_f32_fused_layouts_match_oracle_and_each_other(seed, n_seqs, max_len, planes_out, kernel):
    """The fused kernels -- chunked (up to 262,144 tokens) and scan-first (past it; forced here by its
    test hook) -- in either layout: chunks inside one sequence and shared by several, parts handed
    over whole and token by token."""
    b = synth.random_batch(seed, n_seqs, max_len=max_len, min_len=max_len if n_seqs == 1 else 1, dtype="f32")
    qn, kn = b.qk()
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    say(f"case: fp32 fused {kernel} layouts seed={seed} tokens={b.n_tokens} planes_out={planes_out}")

    def run():
        q, k = dev_heads(qn, "f32"), dev_heads(kn, "f32")
        pl = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda") if planes_out else None
        mr.apply_ids(q, k, i32(b.ids), i32(b.cu_seqlens), MARKER, planes_out=pl)
        if planes_out:
            np.testing.assert_array_equal(pl.cpu().numpy(), epl)
        return host_heads(q), host_heads(k)

    res = _both_layouts(run, _lib.HOOK_FUSED_SCAN_FIRST if kernel == "scan_first" else _lib.HOOK_FUSED_CHUNKED)
    for name, (q, k) in res.items():
        compare_heads(q, qn, epl, "f32", what=f"fused {kernel} {name} q")
        compare_heads(k, kn, epl, "f32", what=f"fused {kernel} {name} k")
    for a, c in zip(res["sixteen"], res["eight"]):
        np.testing.assert_array_equal(a.view(np.uint32), c.view(np.uint32))


def _kv_case(b, slots_seed, block_size, with_v, fused):
    """One fp32 cache-writing call on fresh device copies of seeded inputs: returns the inputs (q, k,
    v, slots, cache blocks) and the device results (q, k cache, v cache or None)."""
    from test_gpu_kv import make_slots, new_cache, v_heads
    qn, kn = b.qk()
    vn = v_heads(b)
    slots, nb = make_slots(slots_seed, b.n_tokens, block_size=block_size)
    q, k, v = dev_heads(qn, "f32"), dev_heads(kn, "f32"), dev_heads(vn, "f32")
    kc = new_cache(nb, block_size, 2, 256, "f32", -7.0)
    vc = new_cache(nb, block_size, 2, 256, "f32", -7.0) if with_v else None
    sl = torch.from_numpy(slots).cuda()
    if fused:
        mr.apply_ids_kv(q, k, v if with_v else None, i32(b.ids), i32(b.cu_seqlens), kc, vc, sl, MARKER)
    else:
        pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
        mr.apply_kv(q, k, v if with_v else None, pl, kc, vc, sl)
    np.testing.assert_array_equal(host_heads(k), kn, err_msg="k input changed")
    np.testing.assert_array_equal(host_heads(v), vn, err_msg="v input changed")
    return (qn, kn, vn, slots, nb), q, kc, vc


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("with_v,block_size", [(True, 16), (False, 5)])
def test_f32_cache_writes_layouts_match_oracle_and_each_other(fused, with_v, block_size):
    """mrope_apply_kv and mrope_apply_ids_kv in fp32: the sixteen-lane kernels (the default for 8 Q +
    2 K heads of 256) and the generic eight-lane path (the hook) against the oracle -- Q in place, K
    rows in the paged cache, V rows bit-exact, rows no valid slot points at untouched, negative slots
    and slots past the cache skipped -- and bit for bit against each other; a block size of 5 takes
    the division path."""
    from test_gpu_kv import check_caches
    b = synth.random_batch(641 + block_size, 40, max_len=700, dtype="f32")
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    say(f"case: fp32 cache writes fused={fused} v={with_v} block={block_size} tokens={b.n_tokens}")
    res = _both_layouts(lambda: _kv_case(b, 642, block_size, with_v, fused))
    for name, ((qn, kn, vn, slots, nb), q, kc, vc) in res.items():
        compare_heads(host_heads(q), qn, epl, "f32", what=f"{name} q")
        n = check_caches(kc, vc, slots, nb, block_size, kn, vn, epl, "f32", -7.0, f"{name} cache")
        assert n > 0.9 * b.n_tokens
    _, q16, kc16, vc16 = res["sixteen"]
    _, q8, kc8, vc8 = res["eight"]
    assert torch.equal(q16.view(torch.int32), q8.view(torch.int32))
    assert torch.equal(kc16.view(torch.int32), kc8.view(torch.int32))
    if with_v:
        assert torch.equal(vc16.view(torch.int32), vc8.view(torch.int32))


@pytest.mark.parametrize("fused", [False, True])
def test_f32_cache_writes_past_the_store_hint_size(fused):
    """48 x 4,096 fp32 tokens with V: Q written in place past the size from which its stores take
    the non-temporal hint; every Q element and every K cache row against the oracle."""
    from test_gpu_kv import check_caches
    b = synth.random_batch(651, 48, max_len=4096, min_len=4096, dtype="f32")
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    say(f"case: fp32 cache writes past the hint size fused={fused} tokens={b.n_tokens}")
    (qn, kn, vn, slots, nb), q, kc, vc = _kv_case(b, 652, 16, True, fused)
    compare_heads_all(q, qn, epl, "f32", what="q")
    check_caches(kc, vc, slots, nb, 16, kn, vn, epl, "f32", -7.0, "cache")
