"""GPU parity of the paged K/V cache writes (mrope_apply_kv, mrope_apply_ids_kv, mrope_decode with V)
against the oracle: planes, rotation and the paged scatter, on the same seeded inputs.

Q rotated in place and K rows in the cache: fp32 within 2e-6 of the oracle (pair-norm relative),
bf16 / fp16 within 1 ulp of the fp32 oracle rounded to the type; dims past the rotary part and every
V row bit-identical.  Cache rows no valid slot points at keep their fill; K and V inputs are left
unchanged.  Slot mappings mix a random permutation of a larger cache with negative slots and slots
past its end, which must write nothing.
"""
import ctypes

import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
import oracle
from canvas_rope_rotary_amd import synth
from gpu_util import MARKER, TORCH_DT, compare_heads, compare_heads_all, dev_heads, host_heads, i32, say

pytestmark = pytest.mark.gpu

_V = 77  # seed tag of the V heads


def v_heads(b: synth.Prefill, n_kv: int = 2, head_dim: int = 256):
    x = synth.normal(b.seed, _V, b.n_tokens * n_kv * head_dim).reshape(b.n_tokens, n_kv, head_dim)
    return synth.to_dtype(x, b.dtype)


def make_slots(seed: int, n: int, block_size: int = 16, room: float = 1.5, neg: float = 0.03, past: float = 0.02):
    """A random permutation of the slots of a cache `room` times larger than needed; a fraction of
    tokens get a negative slot, another fraction a slot past the cache end."""
    g = np.random.default_rng(seed)
    n_blocks = max(1, int(np.ceil(n * room / block_size)))
    slots = g.permutation(n_blocks * block_size)[:n].astype(np.int64)
    r = g.uniform(size=n)
    is_neg = r < neg
    is_past = (r >= neg) & (r < neg + past)
    slots[is_neg] = -1 - g.integers(0, 5, size=int(is_neg.sum()))
    slots[is_past] = n_blocks * block_size + g.integers(0, 100, size=int(is_past.sum()))
    return slots, n_blocks


def new_cache(n_blocks, block_size, heads, head_dim, dtype, fill):
    return torch.full((n_blocks, block_size, heads, head_dim), fill, dtype=TORCH_DT[dtype], device="cuda")


def check_caches(kc, vc, slots, n_blocks, block_size, kn, vn, planes, dtype, fill, what):
    """K rows against the oracle rotation, V rows bit-exact, unreferenced rows untouched."""
    S = n_blocks * block_size
    valid = (slots >= 0) & (slots < S)
    H, D = kn.shape[1], kn.shape[2]
    flat_k = host_heads(kc.view(S, H, D))
    compare_heads(flat_k[slots[valid]], kn[valid], planes[:, valid], dtype, what=f"{what} k cache")
    untouched = np.ones(S, bool)
    untouched[slots[valid]] = False
    fill_bits = host_heads(torch.full((1,), fill, dtype=TORCH_DT[dtype])).reshape(-1)[0]
    assert (flat_k[untouched] == fill_bits).all(), f"{what}: k cache rows written without a slot"
    if vc is not None:
        flat_v = host_heads(vc.view(S, H, D))
        np.testing.assert_array_equal(flat_v[slots[valid]], vn[valid], err_msg=f"{what} v cache")
        assert (flat_v[untouched] == fill_bits).all(), f"{what}: v cache rows written without a slot"
    return int(valid.sum())


@pytest.mark.parametrize("dtype,with_v", [("bf16", True), ("f16", True), ("bf16", False), ("f32", True)])
def test_apply_kv_matches_oracle(dtype, with_v):
    b = synth.random_batch(201, 40, max_len=500, dtype=dtype)
    say(f"case: apply_kv dtype={dtype} v={with_v} tokens={b.n_tokens}")
    qn, kn = b.qk()
    vn = v_heads(b)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    slots, nb = make_slots(202, b.n_tokens)
    q, k, v = dev_heads(qn, dtype), dev_heads(kn, dtype), dev_heads(vn, dtype)
    kc = new_cache(nb, 16, 2, 256, dtype, -7.0)
    vc = new_cache(nb, 16, 2, 256, dtype, -7.0) if with_v else None
    mr.apply_kv(q, k, v if with_v else None, i32(epl), kc, vc, torch.from_numpy(slots).cuda())
    compare_heads(host_heads(q), qn, epl, dtype, what="q")
    np.testing.assert_array_equal(host_heads(k), kn)
    np.testing.assert_array_equal(host_heads(v), vn)
    n = check_caches(kc, vc, slots, nb, 16, kn, vn, epl, dtype, -7.0, "apply_kv")
    assert n > 0.9 * b.n_tokens


@pytest.mark.parametrize("planes_out", [True, False])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_apply_ids_kv_matches_oracle(dtype, planes_out):
    """Planes from ids, rotation and the cache write in one launch; scalars and planes out as in
    mrope_apply_ids.  Without planes_out a chunk inside one sequence takes the kernel's per-chunk
    handover instead of per-token planes."""
    b = synth.random_batch(211, 48, max_len=900 if planes_out else 3000, dtype=dtype, empty_frac=0.05)
    say(f"case: apply_ids_kv dtype={dtype} tokens={b.n_tokens}")
    qn, kn = b.qk()
    vn = v_heads(b)
    epl, est, eam, eog = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    slots, nb = make_slots(212, b.n_tokens, block_size=32)
    q, k, v = dev_heads(qn, dtype), dev_heads(kn, dtype), dev_heads(vn, dtype)
    kc = new_cache(nb, 32, 2, 256, dtype, 3.0)
    vc = new_cache(nb, 32, 2, 256, dtype, 3.0)
    pl = torch.full((3, b.n_tokens), -9, dtype=torch.int32, device="cuda") if planes_out else None
    st, am, og, fl, _ = mr.apply_ids_kv(q, k, v, i32(b.ids), i32(b.cu_seqlens), kc, vc, torch.from_numpy(slots).cuda(),
                                        MARKER, planes_out=pl)
    if planes_out:
        np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    np.testing.assert_array_equal(am.cpu().numpy(), eam)
    np.testing.assert_array_equal(og.cpu().numpy(), eog)
    compare_heads(host_heads(q), qn, epl, dtype, what="q")
    np.testing.assert_array_equal(host_heads(k), kn)
    check_caches(kc, vc, slots, nb, 32, kn, vn, epl, dtype, 3.0, "apply_ids_kv")


@pytest.mark.parametrize("nq,nkv,head_dim,block_size", [(4, 1, 128, 16), (8, 2, 512, 8), (3, 3, 64, 5)])
def test_kv_generic_heads(nq, nkv, head_dim, block_size):
    """Head counts and head dims off the model's shape take the generic kernels; a block size that
    is not a power of two takes the division path."""
    b = synth.random_batch(221 + nq, 20, max_len=300, dtype="bf16")
    say(f"case: kv generic nq={nq} nkv={nkv} head_dim={head_dim} block={block_size} tokens={b.n_tokens}")
    T = b.n_tokens
    g = synth.rng(223, 1)
    qn = synth.to_dtype(g.standard_normal((T, nq, head_dim)).astype(np.float32), "bf16")
    kn = synth.to_dtype(g.standard_normal((T, nkv, head_dim)).astype(np.float32), "bf16")
    vn = synth.to_dtype(g.standard_normal((T, nkv, head_dim)).astype(np.float32), "bf16")
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    slots, nb = make_slots(224, T, block_size=block_size)
    for fused in (False, True):
        q, k, v = dev_heads(qn, "bf16"), dev_heads(kn, "bf16"), dev_heads(vn, "bf16")
        kc = new_cache(nb, block_size, nkv, head_dim, "bf16", 0.5)
        vc = new_cache(nb, block_size, nkv, head_dim, "bf16", 0.5)
        sl = torch.from_numpy(slots).cuda()
        if fused:
            mr.apply_ids_kv(q, k, v, i32(b.ids), i32(b.cu_seqlens), kc, vc, sl, MARKER)
        else:
            mr.apply_kv(q, k, v, i32(epl), kc, vc, sl)
        compare_heads(host_heads(q), qn, epl, "bf16", what=f"q fused={fused}")
        check_caches(kc, vc, slots, nb, block_size, kn, vn, epl, "bf16", 0.5, f"generic fused={fused}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_with_v(dtype):
    d = synth.config4(n_seqs=512, num_blocks=1024)
    say(f"case: decode with V dtype={dtype} seqs={d.n_seqs}")
    qn, kn = d.qk()
    if dtype == "f32":
        qn, kn = synth.to_f32(qn, "bf16"), synth.to_f32(kn, "bf16")
    g = synth.rng(231, 2)
    vn = synth.to_dtype(g.standard_normal(kn.shape).astype(np.float32), dtype)
    slots = d.slot_mapping.copy()
    slots[::37] = -1
    slots[5::41] = d.num_blocks * d.block_size + 3
    q, k, v = dev_heads(qn, dtype), dev_heads(kn, dtype), dev_heads(vn, dtype)
    kc = new_cache(d.num_blocks, d.block_size, 2, 256, dtype, 0.0)
    vc = new_cache(d.num_blocks, d.block_size, 2, 256, dtype, 0.0)
    mr.decode(q, k, torch.from_numpy(d.pos).cuda(), torch.from_numpy(d.amount).cuda(), kc,
              torch.from_numpy(slots).cuda(), v=v, v_cache=vc)
    ref_kc = np.zeros((d.num_blocks, d.block_size, 2, 256), np.float32)
    ref_vc = np.zeros_like(ref_kc)
    oracle.decode(synth.to_f32(qn, dtype), synth.to_f32(kn, dtype), d.pos, d.amount, ref_kc, slots,
                          d.block_size, v=synth.to_f32(vn, dtype), v_cache=ref_vc)
    planes = np.stack([d.pos - d.amount] * 3).astype(np.int32)
    compare_heads(host_heads(q), qn, planes, dtype, what="decode q")
    got_kc = host_heads(kc)
    got_vc = host_heads(vc)
    np.testing.assert_array_equal(synth.to_f32(got_vc, dtype) if dtype != "f32" else got_vc, ref_vc)
    valid = (slots >= 0) & (slots < d.num_blocks * d.block_size)
    flat = got_kc.reshape(-1, 2, 256)
    compare_heads(flat[slots[valid]], kn[valid], planes[:, valid], dtype, what="decode k cache")
    written = np.zeros(flat.shape[0], bool)
    written[slots[valid]] = True
    assert not synth.to_f32(flat[~written], dtype).any() if dtype != "f32" else not flat[~written].any()


def test_apply_ids_kv_full_size():
    """64 x 4096 bf16 prompts with V, caches of 16-token blocks with room for 1.25x the tokens:
    planes, Q, every written K and V cache row in full."""
    b = synth.config2()
    T = b.n_tokens
    say(f"case: apply_ids_kv full size tokens={T}")
    qn, kn = b.qk()
    vn = v_heads(b)
    slots, nb = make_slots(241, T, room=1.25, neg=0.001, past=0.001)
    q, k, v = dev_heads(qn, "bf16"), dev_heads(kn, "bf16"), dev_heads(vn, "bf16")
    kc = new_cache(nb, 16, 2, 256, "bf16", 0.0)
    vc = new_cache(nb, 16, 2, 256, "bf16", 0.0)
    pl = torch.empty((3, T), dtype=torch.int32, device="cuda")
    mr.apply_ids_kv(q, k, v, i32(b.ids), i32(b.cu_seqlens), kc, vc, torch.from_numpy(slots).cuda(), MARKER,
                    planes_out=pl)
    epl, est, eam, eog = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    compare_heads_all(q, qn, epl, "bf16", what="q")
    S = nb * 16
    ok = (slots >= 0) & (slots < S)
    rows = torch.from_numpy(slots[ok]).cuda()
    compare_heads_all(kc.view(S, 2, 256)[rows], kn[ok], epl[:, ok], "bf16", what="k cache")
    np.testing.assert_array_equal(host_heads(vc.view(S, 2, 256)[rows]), vn[ok])
    # every valid slot was written: no zero rows left among them (inputs ~ N(0, 1) are never all zero)
    all_ok = (slots >= 0) & (slots < S)
    written = kc.view(S, 2 * 256)[torch.from_numpy(slots[all_ok]).cuda()].abs().amax(dim=1)
    assert int((written == 0).sum()) == 0


@pytest.mark.parametrize("fused", [False, True, "planes_out"])
def test_kv_past_the_store_hint_size(fused):
    """96 x 4096 bf16 tokens write 403 MB of Q in place, past the size from which the cache-writing
    kernels' Q stores take the non-temporal hint: Q and every written cache row.  With planes_out
    the fused call runs as the scan launch and then mrope_apply_kv's launch."""
    origins = [int(o) for o in np.random.default_rng(251).integers(0, 513, size=96)]
    b = synth._batch("96x4096-image-bf16", 251, [4096] * 96, origins, "bf16")
    T = b.n_tokens
    say(f"case: kv past the store hint size tokens={T} fused={fused}")
    qn, kn = b.qk()
    vn = v_heads(b)
    slots, nb = make_slots(252, T, room=1.1, neg=0.001, past=0.001)
    q, k, v = dev_heads(qn, "bf16"), dev_heads(kn, "bf16"), dev_heads(vn, "bf16")
    kc = new_cache(nb, 16, 2, 256, "bf16", 0.0)
    vc = new_cache(nb, 16, 2, 256, "bf16", 0.0)
    epl, est, eam, eog = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    sl_dev = torch.from_numpy(slots).cuda()
    if fused:
        pl = torch.full((3, T), -9, dtype=torch.int32, device="cuda") if fused == "planes_out" else None
        st, am, og, _, _ = mr.apply_ids_kv(q, k, v, i32(b.ids), i32(b.cu_seqlens), kc, vc, sl_dev, MARKER,
                                           planes_out=pl)
        np.testing.assert_array_equal(st.cpu().numpy(), est)
        np.testing.assert_array_equal(og.cpu().numpy(), eog)
        if pl is not None:
            np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    else:
        mr.apply_kv(q, k, v, i32(epl), kc, vc, sl_dev)
    compare_heads_all(q, qn, epl, "bf16", what="q")
    S = nb * 16
    ok = (slots >= 0) & (slots < S)
    rows = torch.from_numpy(slots[ok]).cuda()
    compare_heads_all(kc.view(S, 2, 256)[rows], kn[ok], epl[:, ok], "bf16", what="k cache")
    np.testing.assert_array_equal(host_heads(vc.view(S, 2, 256)[rows]), vn[ok])


def test_check_slots_option():
    """check_slots=True: distinct slots run as usual; a slot named twice raises before anything is
    launched (q keeps its values)."""
    d = synth.config4(n_seqs=64, num_blocks=128)
    qn, kn = d.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    kc = new_cache(d.num_blocks, d.block_size, 2, 256, "bf16", 0.0)
    pos, am = torch.from_numpy(d.pos).cuda(), torch.from_numpy(d.amount).cuda()
    say("case: decode check_slots")
    mr.decode(q, k, pos, am, kc, torch.from_numpy(d.slot_mapping).cuda(), check_slots=True)
    planes = np.stack([d.pos - d.amount] * 3).astype(np.int32)
    compare_heads(host_heads(q), qn, planes, "bf16", what="decode q")
    dup = d.slot_mapping.copy()
    dup[7] = dup[3]
    before = host_heads(q)
    with pytest.raises(ValueError):
        mr.decode(q, k, pos, am, kc, torch.from_numpy(dup).cuda(), check_slots=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_heads(q), before)
