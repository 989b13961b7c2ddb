"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Planes, start, amount, origin and flags: bit-exact.  Rotated Q/K: fp32 within 2e-6 of the oracle
(pair-norm relative), bf16 within 1 ulp of the fp32 oracle rounded to bf16; the dims past the
rotary part bit-identical.  Small inputs are compared element by element; the full-size workloads
in full, planes and every rotated element (the oracle runs over blocks of tokens in host threads).
"""
import ctypes

import numpy as np
import pytest
import torch

import canvas_rope_rotary_amd as mr
import oracle
from canvas_rope_rotary_amd import synth
from gpu_util import (MARKER, TORCH_DT, as_f32, compare_heads, compare_heads_all, dev_heads, expected_flags, host_heads,
                      i32, say)
from parity import check_bf16, check_fp32

pytestmark = pytest.mark.gpu


def _oracle_planes(b):
    return oracle.planes(b.ids, b.cu_seqlens, MARKER)


def _check_scan(b, pl, st, am, og, fl, what):
    epl, est, eam, eog = _oracle_planes(b)
    np.testing.assert_array_equal(pl.cpu().numpy()[:, :b.n_tokens], epl, err_msg=f"{what} planes")
    np.testing.assert_array_equal(st.cpu().numpy(), est, err_msg=f"{what} start")
    np.testing.assert_array_equal(am.cpu().numpy(), eam, err_msg=f"{what} amount")
    np.testing.assert_array_equal(og.cpu().numpy(), eog, err_msg=f"{what} origin")
    if fl is not None:
        np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog), err_msg=f"{what} flags")
    return epl, est, eam, eog


# ------------------------------------------------------------------ small, element by element ---

def test_config1_fp32_single_image():
    b = synth.config1()
    say("case: single image prompt, fp32, L=110")
    qn, kn = b.qk()
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    pl, st, am, og, fl = mr.planes(ids, cu, MARKER)
    epl, est, eam, eog = _check_scan(b, pl, st, am, og, fl, "config1")
    assert (int(st[0]), int(am[0]), int(og[0])) == (73, 58, 6)
    # in place
    q, k = dev_heads(qn, "f32"), dev_heads(kn, "f32")
    mr.apply(q, k, pl)
    compare_heads(host_heads(q), qn, epl, "f32", what="q in place")
    compare_heads(host_heads(k), kn, epl, "f32", what="k in place")
    # out of place == in place, inputs untouched
    q2, k2 = dev_heads(qn, "f32"), dev_heads(kn, "f32")
    qo, ko = torch.empty_like(q2), torch.empty_like(k2)
    mr.apply(q2, k2, pl, q_out=qo, k_out=ko)
    assert torch.equal(qo, q) and torch.equal(ko, k)
    np.testing.assert_array_equal(host_heads(q2), qn)
    # fused
    q3, k3 = dev_heads(qn, "f32"), dev_heads(kn, "f32")
    pl3 = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda")
    st3, am3, og3, fl3, _ = mr.apply_ids(q3, k3, ids, cu, MARKER, planes_out=pl3)
    _check_scan(b, pl3, st3, am3, og3, fl3, "config1 fused")
    assert torch.equal(q3, q) and torch.equal(k3, k)


def test_config1_prefix_103():
    """Reading of the workload text: 6 + 67 + 30 = 103 tokens; L = 110 is kept, and the 103-token
    prefix must give the same planes."""
    b = synth.config1()
    ids = i32(b.ids[:103])
    pl, st, am, og, fl = mr.planes(ids, i32([0, 103]), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    np.testing.assert_array_equal(pl.cpu().numpy(), epl[:, :103])
    assert (int(st[0]), int(am[0])) == (73, 58)


@pytest.mark.parametrize("seed,dtype,n_seqs,max_len,empty", [
    (101, "bf16", 40, 300, 0.0), (102, "f32", 40, 300, 0.1), (103, "bf16", 300, 90, 0.2),
    (104, "bf16", 12, 3000, 0.0), (105, "f32", 5, 700, 0.0), (106, "bf16", 1, 1, 0.0),
    (107, "f16", 40, 400, 0.05),
])
def test_fuzz_small_batches(seed, dtype, n_seqs, max_len, empty):
    b = synth.random_batch(seed, n_seqs, max_len=max_len, dtype=dtype, empty_frac=empty)
    say(f"case: fuzz seed={seed} dtype={dtype} seqs={n_seqs} tokens={b.n_tokens}")
    qn, kn = b.qk()
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    pl, st, am, og, fl = mr.planes(ids, cu, MARKER)
    epl, *_ = _check_scan(b, pl, st, am, og, fl, f"fuzz {seed}")
    q, k = dev_heads(qn, dtype), dev_heads(kn, dtype)
    mr.apply(q, k, pl)
    compare_heads(host_heads(q), qn, epl, dtype, what="q")
    compare_heads(host_heads(k), kn, epl, dtype, what="k")
    # fused kernel: same bits as planes + apply
    q2, k2 = dev_heads(qn, dtype), dev_heads(kn, dtype)
    pl2 = torch.full_like(pl, -7)
    st2, am2, og2, fl2, _ = mr.apply_ids(q2, k2, ids, cu, MARKER, planes_out=pl2)
    _check_scan(b, pl2, st2, am2, og2, fl2, f"fuzz {seed} fused")
    assert torch.equal(q2, q) and torch.equal(k2, k)
    # fused without planes_out (chunks inside one sequence are handed over per chunk): same bits
    q3, k3 = dev_heads(qn, dtype), dev_heads(kn, dtype)
    st3, am3, og3, fl3, _ = mr.apply_ids(q3, k3, ids, cu, MARKER)
    for a, c in ((st3, st), (am3, am), (og3, og), (fl3, fl)):
        assert torch.equal(a, c)
    assert torch.equal(q3, q) and torch.equal(k3, k)


def test_many_tiny_sequences_and_empties():
    """5000 sequences of 0..3 tokens: many sequences per 64-token tile, empty ones in runs."""
    g = np.random.default_rng(7)
    lens = g.integers(0, 4, size=5000)
    lens[:3] = 0
    lens[-4:] = 0
    ids = synth.text_ids(synth.rng(7, 4), int(lens.sum()))
    ids[g.integers(0, ids.size, size=200)] = MARKER
    cu = np.zeros(lens.size + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill("tiny", ids, cu, [None] * lens.size, "bf16", seed=7)
    pl, st, am, og, fl = mr.planes(i32(ids), i32(cu), MARKER)
    epl, *_ = _check_scan(b, pl, st, am, og, fl, "tiny")
    # fused: hundreds of sequences per 512-token chunk (several sequence windows per chunk)
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    pl2 = torch.full_like(pl, -7)
    st2, am2, og2, fl2, _ = mr.apply_ids(q, k, i32(ids), i32(cu), MARKER, planes_out=pl2)
    _check_scan(b, pl2, st2, am2, og2, fl2, "tiny fused")
    compare_heads(host_heads(q), qn, epl, "bf16", what="tiny fused q")
    compare_heads(host_heads(k), kn, epl, "bf16", what="tiny fused k")


@pytest.mark.parametrize("fused", [False, True])
def test_chunk_boundaries(fused):
    """Sequences and frames on and across the 512-token chunk edges: markers at the first and last
    token of a chunk, frames straddling two and three chunks, lengths 511/512/513, empties."""
    lens = [512, 512, 1, 511, 513, 1024, 0, 0, 512, 600, 1700, 3]
    placed = [0, 511, 0, 444, 0, 500, None, None, None, 510, 1023, None]
    g = synth.rng(13, 4)
    ids = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed) if n > 0])
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill("edges", ids, cu, placed, "bf16", seed=13)
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    if fused:
        pl = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda")
        st, am, og, fl, _ = mr.apply_ids(q, k, i32(ids), i32(cu), MARKER, planes_out=pl)
    else:
        pl, st, am, og, fl = mr.planes(i32(ids), i32(cu), MARKER)
        mr.apply(q, k, pl)
    epl, *_ = _check_scan(b, pl, st, am, og, fl, f"edges fused={fused}")
    compare_heads(host_heads(q), qn, epl, "bf16", what="edges q")
    compare_heads(host_heads(k), kn, epl, "bf16", what="edges k")


@pytest.mark.parametrize("planes_out", [True, False])
@pytest.mark.parametrize("n_chunks", [1, 20, 40, 100, 200, 300])
def test_fused_split_grid_levels(n_chunks, planes_out):
    """The fused call splits each 512-token chunk over up to 16 workgroups when the input is small
    (1 and 20 chunks: 16 parts, 40: 8, 100: 4, 200: 2, 300: 1 on a 256-CU part); only the first
    part of a chunk publishes its look-back word and writes scalars.  A long image sequence whose
    look-back crosses many chunks, image and text sequences around it, a ragged tail."""
    n = n_chunks * 512 - 37
    tail = [300, 0, 70, 1] if n > 600 else []
    lead = 5 if n > 600 else 0
    lens = [lead] + [n - lead - sum(tail)] + tail
    rng = np.random.default_rng(n_chunks)
    placed = [None if lead == 0 else 0, int(rng.integers(0, max(1, lens[1] - 80))), 10, None, 0, None][:len(lens)]
    g = synth.rng(17, n_chunks)
    ids = np.concatenate([synth.prompt_ids(g, m, o) for m, o in zip(lens, placed) if m > 0])
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill(f"split{n_chunks}", ids, cu, placed, "bf16", seed=17, head_dim=64)
    say(f"case: {b.name}, {b.n_tokens} tokens")
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    if planes_out:
        pl = torch.full((3, b.n_tokens), -7, dtype=torch.int32, device="cuda")
        st, am, og, fl, _ = mr.apply_ids(q, k, i32(ids), i32(cu), MARKER, planes_out=pl)
        epl, est, eam, eog = _check_scan(b, pl, st, am, og, fl, b.name)
    else:
        st, am, og, fl, _ = mr.apply_ids(q, k, i32(ids), i32(cu), MARKER)
        epl, est, eam, eog = _oracle_planes(b)
        for got, want in ((st, est), (am, eam), (og, eog)):
            np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=b.name)
    compare_heads_all(q, qn, epl, "bf16", what=f"{b.name} q")
    compare_heads_all(k, kn, epl, "bf16", what=f"{b.name} k")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fused_chunk_classes_without_planes_out(dtype):
    """Without planes_out a chunk inside one sequence is handed over as (sequence begin, offset,
    origin): chunks wholly before the image, wholly after the frame, cutting the frame, inside
    text-only sequences, and chunks shared by several sequences (per-token path).  Frames at and
    around chunk edges; every token compared with the oracle."""
    lens = [3000, 2600, 1536, 700, 5, 1, 0, 1800, 2048, 40, 513]
    placed = [1200, 0, None, 511, 0, None, None, 1022, 2000, None, 446]
    g = synth.rng(23, 4)
    ids = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed) if n > 0])
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill("classes", ids, cu, placed, dtype, seed=23, head_dim=128)
    qn, kn = b.qk()
    q, k = dev_heads(qn, dtype), dev_heads(kn, dtype)
    st, am, og, fl, _ = mr.apply_ids(q, k, i32(ids), i32(cu), MARKER)
    epl, est, eam, eog = _oracle_planes(b)
    for got, want, what in ((st, est, "start"), (am, eam, "amount"), (og, eog, "origin")):
        np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=what)
    np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog), err_msg="flags")
    compare_heads(host_heads(q), qn, epl, dtype, what=f"classes {dtype} q")
    compare_heads(host_heads(k), kn, epl, dtype, what=f"classes {dtype} k")


def test_zero_tokens_text_scalars():
    cu = i32([0, 0, 0])
    ids = torch.zeros(0, dtype=torch.int32, device="cuda")
    pl, st, am, og, fl = mr.planes(ids, cu, MARKER)
    assert st.tolist() == [1 << 30] * 2 and am.tolist() == [0, 0] and og.tolist() == [-1, -1]


def _piece_cuts(b, n_pieces, seed):
    """Per sequence, n_pieces + 1 increasing cut positions from 0 to its length.  Image sequences get
    cuts at the marker and inside the frame (the row tokens, the closing tokens); one whole round
    of pieces is empty for every sequence."""
    g = np.random.default_rng(seed)
    _, _, _, og = _oracle_planes(b)
    cuts = []
    for s in range(b.n_seqs):
        n = int(b.cu_seqlens[s + 1] - b.cu_seqlens[s])
        pts = set(g.integers(0, n + 1, size=n_pieces - 2).tolist())
        if og[s] >= 0:
            o = int(og[s])
            pts.add(min(n, o + int(g.choice([0, 1, 9, 33, 65, 66, 67]))))
        pts = sorted(pts)[: n_pieces - 2]
        pts = pts + [n] * (n_pieces - 2 - len(pts))
        c = [0] + sorted(pts)
        c.insert(2, c[1])  # the empty round
        cuts.append(c + [n])
    return np.array(cuts, np.int64)  # [n_seqs, n_pieces + 1]


@pytest.mark.parametrize("mode", ["planes", "fused", "fused_no_planes_out"])
def test_chunked_pieces_match_whole_sequences(mode):
    """Prefill in pieces (chunked prefill, a second turn): each piece passes the position of its
    first token and the origin the earlier pieces found; planes and rotated Q/K of every piece equal
    the one-call result on the whole sequences, and the last piece's scalars equal the whole
    sequences' scalars.  Without planes_out the fused call hands a single-sequence chunk over per
    chunk, with the piece's offset and carried origin; its planes are then judged by the rotation."""
    fused = mode != "planes"
    b = synth.random_batch(71, 36, max_len=2600, dtype="bf16", empty_frac=0.05)
    n_pieces = 5
    cuts = _piece_cuts(b, n_pieces, 72)
    epl, est, eam, eog = _oracle_planes(b)
    eflags = expected_flags(b, eog)
    qn, kn = b.qk()
    say(f"case: chunked pieces fused={fused} seqs={b.n_seqs} tokens={b.n_tokens} pieces={n_pieces}")
    got_pl = np.full((3, b.n_tokens), -7, np.int32)
    got_q = np.zeros_like(qn)
    got_k = np.zeros_like(kn)
    multi_or = np.zeros(b.n_seqs, np.int32)
    origin_prev = None
    for k in range(n_pieces):
        rows = np.concatenate([np.arange(b.cu_seqlens[s] + cuts[s, k], b.cu_seqlens[s] + cuts[s, k + 1])
                               for s in range(b.n_seqs)]).astype(np.int64)
        lens = cuts[:, k + 1] - cuts[:, k]
        cu = np.zeros(b.n_seqs + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        ids_k = b.ids[rows].astype(np.int32)
        off = cuts[:, k].astype(np.int32)
        oin = None if origin_prev is None else origin_prev
        # the piece alone against the oracle's piece rule
        cpl, cst, cam, cog = oracle.planes_chunk(ids_k, cu, MARKER, off,
                                                 None if oin is None else oin.cpu().numpy())
        if fused:
            q, kk = dev_heads(qn[rows], "bf16"), dev_heads(kn[rows], "bf16")
            pl = torch.full((3, rows.size), -7, dtype=torch.int32, device="cuda") if mode == "fused" else None
            st, am, og, fl, _ = mr.apply_ids(q, kk, i32(ids_k), i32(cu), MARKER, planes_out=pl,
                                             pos_offset=i32(off), origin_in=oin)
            got_q[rows], got_k[rows] = host_heads(q), host_heads(kk)
        else:
            pl, st, am, og, fl = mr.planes(i32(ids_k), i32(cu), MARKER, pos_offset=i32(off), origin_in=oin)
        pl_h = pl.cpu().numpy() if pl is not None else cpl
        got_pl[:, rows] = pl_h[:, :rows.size]
        np.testing.assert_array_equal(pl_h[:, :rows.size], cpl, err_msg=f"piece {k} planes")
        np.testing.assert_array_equal(st.cpu().numpy(), cst, err_msg=f"piece {k} start")
        np.testing.assert_array_equal(am.cpu().numpy(), cam, err_msg=f"piece {k} amount")
        np.testing.assert_array_equal(og.cpu().numpy(), cog, err_msg=f"piece {k} origin")
        multi_or |= fl.cpu().numpy() & 1
        origin_prev = og
    np.testing.assert_array_equal(got_pl, epl, err_msg="pieces vs whole planes")
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    np.testing.assert_array_equal(am.cpu().numpy(), eam)
    np.testing.assert_array_equal(og.cpu().numpy(), eog)
    np.testing.assert_array_equal(multi_or, eflags & 1, err_msg="multi-marker bit over the pieces")
    np.testing.assert_array_equal(fl.cpu().numpy() & 2, eflags & 2, err_msg="overrun bit of the last piece")
    if fused:
        compare_heads(got_q, qn, epl, "bf16", what="pieces q")
        compare_heads(got_k, kn, epl, "bf16", what="pieces k")


def test_second_turn_long_pieces():
    """A second turn after a long first turn.  Sequence 0 (100,000 tokens, marker at 85,000): a
    text-only first piece of 30,000, then 70,000 tokens whose marker sits 55,000 deep (look-back
    across many chunks, with a position offset).  Sequence 1 (60,000 tokens, marker at 45,000): a
    first piece of 50,000 holding the frame, then a text piece that only carries the origin in."""
    lens = [100000, 60000]
    placed = [85000, 45000]
    g = synth.rng(19, 4)
    ids = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed)])
    cu = np.zeros(3, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill("turns", ids, cu, placed, "bf16", seed=19)
    epl, est, eam, eog = _oracle_planes(b)
    say(f"case: two long turns tokens={b.n_tokens}")
    seen = np.zeros(b.n_tokens, bool)
    turns = [[(0, 30000), (int(cu[1]), int(cu[1]) + 50000)],
             [(30000, 100000), (int(cu[1]) + 50000, int(cu[2]))]]
    # the fused call without planes_out on the same pieces (head_dim 64 keeps the inputs small):
    # single-sequence chunks are handed over with the piece's offset and the carried origin
    bq = synth.Prefill("turns-q", ids, cu, placed, "bf16", seed=19, head_dim=64)
    qn, kn = bq.qk()
    og_prev, og_prev_f = None, None
    for k, segs in enumerate(turns):
        rows = np.concatenate([np.arange(a, e) for a, e in segs]).astype(np.int64)
        ccu = np.array([0, segs[0][1] - segs[0][0], rows.size], np.int32)
        off = np.array([segs[0][0], segs[1][0] - int(cu[1])], np.int32)
        pl, st, am, og, fl = mr.planes(i32(b.ids[rows]), i32(ccu), MARKER, pos_offset=i32(off),
                                       origin_in=og_prev)
        np.testing.assert_array_equal(pl.cpu().numpy(), epl[:, rows], err_msg=f"turn {k} planes")
        og_prev = og
        q, kk = dev_heads(qn[rows], "bf16"), dev_heads(kn[rows], "bf16")
        st_f, am_f, og_f, fl_f, _ = mr.apply_ids(q, kk, i32(b.ids[rows]), i32(ccu), MARKER, pos_offset=i32(off),
                                                 origin_in=og_prev_f)
        for a_, c_ in ((st_f, st), (am_f, am), (og_f, og), (fl_f, fl)):
            assert torch.equal(a_, c_), f"turn {k} fused scalars"
        og_prev_f = og_f
        pick = np.unique(np.concatenate([np.random.default_rng(k).integers(0, rows.size, 3000),
                                         np.flatnonzero((epl[0, rows] != epl[1, rows]) | (epl[0, rows] != epl[2, rows]))]))
        compare_heads(host_heads(q)[pick], qn[rows][pick], epl[:, rows][:, pick], "bf16", what=f"turn {k} fused q")
        compare_heads(host_heads(kk)[pick], kn[rows][pick], epl[:, rows][:, pick], "bf16", what=f"turn {k} fused k")
        del q, kk
        seen[rows] = True
    assert seen.all()
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    np.testing.assert_array_equal(am.cpu().numpy(), eam)
    np.testing.assert_array_equal(og.cpu().numpy(), eog)
    assert og.tolist() == [85000, 45000]
    assert fl.tolist() == [0, 0]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_positions_near_the_limit(dtype):
    """Pieces whose positions run up to the supported limit (|plane| < 2^24): a text piece ending
    at 2^24 - 1, an image piece whose frame sits just below it, and a piece after a carried origin
    near it.  Angles reach ~1.7e7 rad; planes, scalars and rotation against the oracle, through
    the two-launch and the fused (no planes_out) calls."""
    top = (1 << 24) - 1
    lens = [1200, 900, 700]
    off = np.array([top + 1 - 1200, top + 1 - 900 - 300, top + 1 - 700], np.int32)
    placed = [None, 500, None]
    g = synth.rng(51, 4)
    ids = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed)])
    cu = np.zeros(4, np.int32)
    cu[1:] = np.cumsum(lens)
    oin = np.array([-1, -1, top - 5000], np.int32)
    b = synth.Prefill("near-limit", ids, cu, placed, dtype, seed=51, head_dim=128)
    epl, est, eam, eog = oracle.planes_chunk(ids, cu, MARKER, off, oin)
    assert np.abs(epl).max() <= top
    say(f"case: positions near 2^24 dtype={dtype} max plane={int(np.abs(epl).max())}")
    qn, kn = b.qk()
    pl, st, am, og, fl = mr.planes(i32(ids), i32(cu), MARKER, pos_offset=i32(off), origin_in=i32(oin))
    np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    np.testing.assert_array_equal(am.cpu().numpy(), eam)
    np.testing.assert_array_equal(og.cpu().numpy(), eog)
    q, k = dev_heads(qn, dtype), dev_heads(kn, dtype)
    mr.apply(q, k, pl)
    compare_heads(host_heads(q), qn, epl, dtype, what=f"near-limit q {dtype}")
    compare_heads(host_heads(k), kn, epl, dtype, what=f"near-limit k {dtype}")
    q2, k2 = dev_heads(qn, dtype), dev_heads(kn, dtype)
    mr.apply_ids(q2, k2, i32(ids), i32(cu), MARKER, pos_offset=i32(off), origin_in=i32(oin))
    assert torch.equal(q2, q) and torch.equal(k2, k)


def test_origin_zero_negative_planes():
    ids = synth.prompt_ids(synth.rng(3, 9), 200, 0)
    b = synth.Prefill("o0", ids, np.array([0, 200], np.int32), [0], "bf16", seed=3)
    pl, st, am, og, fl = mr.planes(i32(ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = _check_scan(b, pl, st, am, og, fl, "O=0")
    assert pl[1, 0].item() == -1 and pl[2, 0].item() == -1
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    mr.apply(q, k, pl)
    compare_heads(host_heads(q), qn, epl, "bf16", what="q O=0")


def test_long_sequence_lookback_chain():
    """One 200,000-token sequence with its marker near the end and one with none: look-back over
    thousands of tiles."""
    lens = [200000, 150000, 70]
    placed = [199000, None, 0]
    g = synth.rng(9, 4)
    ids = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed)])
    cu = np.zeros(4, np.int32)
    cu[1:] = np.cumsum(lens)
    b = synth.Prefill("long", ids, cu, placed, "bf16", seed=9)
    for rep in range(3):
        pl, st, am, og, fl = mr.planes(i32(ids), i32(cu), MARKER)
        _check_scan(b, pl, st, am, og, fl, f"long rep {rep}")


def test_strided_views_equal_contiguous():
    """Q and K as views of one fused QKV projection buffer give the same bits as contiguous copies."""
    b = synth.random_batch(21, 30, max_len=200)
    qn, kn = b.qk()
    T = b.n_tokens
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    qkv = torch.zeros((T, 8 + 2 + 2, 256), dtype=torch.bfloat16, device="cuda")
    qkv[:, :8] = dev_heads(qn, "bf16")
    qkv[:, 8:10] = dev_heads(kn, "bf16")
    qv, kv = qkv[:, :8], qkv[:, 8:10]
    assert not qv.is_contiguous() and qv.stride(0) == 12 * 256
    qc, kc = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    mr.apply(qv, kv, pl)
    mr.apply(qc, kc, pl)
    assert torch.equal(qv, qc) and torch.equal(kv, kc)
    assert torch.equal(qkv[:, 10:], torch.zeros_like(qkv[:, 10:]))


def test_generic_head_counts():
    """Head counts other than 8 + 2 take the generic kernel; same results as the oracle."""
    b = synth.random_batch(31, 10, max_len=300)
    T = b.n_tokens
    xq = synth.to_bf16_bits(synth.normal(31, 60, T * 4 * 128)).reshape(T, 4, 128)
    xk = synth.to_bf16_bits(synth.normal(31, 61, T * 1 * 128)).reshape(T, 1, 128)
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    q, k = dev_heads(xq, "bf16"), dev_heads(xk, "bf16")
    mr.apply(q, k, pl)
    compare_heads(host_heads(q), xq, epl, "bf16", what="q 4x128")
    compare_heads(host_heads(k), xk, epl, "bf16", what="k 1x128")
    q2 = dev_heads(xq, "bf16")
    mr.apply(q2, None, pl)
    assert torch.equal(q2, q)


def test_red_arms_fail_on_gpu_output():
    """amount + 1 and 1-D planes must fail the rotation gate against the GPU output on every image
    prompt with text after the frame (zoo page: gate the planes themselves)."""
    b = synth.random_batch(41, 20, max_len=500, min_len=150, text_frac=0.0, dtype="f32")
    qn, _ = b.qk()
    pl, st, am, og, fl = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    q = dev_heads(qn, "f32")
    mr.apply(q, None, pl)
    got = host_heads(q)
    epl, est, eam, eog = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    n_red = 0
    for s in range(b.n_seqs):
        lo, hi = int(b.cu_seqlens[s]), int(b.cu_seqlens[s + 1])
        if eog[s] < 0 or est[s] >= hi - lo:
            continue
        p = np.arange(hi - lo, dtype=np.int32)
        arm = epl[:, lo:hi].copy()
        arm[:, p >= est[s]] -= 1
        for planes_arm in (arm, np.stack([p, p, p])):
            ok, _ = check_fp32(got[lo:hi], oracle.rotate(qn[lo:hi], planes_arm))
            assert not ok
            n_red += 1
        ok, _ = check_fp32(got[lo:hi], oracle.rotate(qn[lo:hi], epl[:, lo:hi]))
        assert ok
    assert n_red >= 10


# ------------------------------------------------------------------ full-size workloads --------

def _full_prefill(b, fused: bool, planes_out: bool = False):
    """The fused call runs as benchmarked, without planes_out: planes never leave the kernel, so the
    scalars are compared bit for bit and the planes through the rotation.  With planes_out the
    planes are compared in full too.  Every rotated element of Q and K is compared with the oracle
    (host threads over blocks of tokens), and dims 64.. must be untouched."""
    say(f"case: {b.name} tokens={b.n_tokens} seqs={b.n_seqs} fused={fused} planes_out={planes_out}")
    qn, kn = b.qk()
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    q, k = dev_heads(qn, b.dtype), dev_heads(kn, b.dtype)
    q_tail, k_tail = q[..., 64:].clone(), k[..., 64:].clone()
    if fused:
        pl = torch.full((3, b.n_tokens), -9, dtype=torch.int32, device="cuda") if planes_out else None
        st, am, og, fl, _ = mr.apply_ids(q, k, ids, cu, MARKER, planes_out=pl)
        torch.cuda.synchronize()
        epl, est, eam, eog = _oracle_planes(b)
        if planes_out:
            np.testing.assert_array_equal(pl.cpu().numpy(), epl, err_msg=f"{b.name} planes_out")
        for got, want, what in ((st, est, "start"), (am, eam, "amount"), (og, eog, "origin")):
            np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"{b.name} {what}")
        np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog), err_msg=f"{b.name} flags")
    else:
        pl, st, am, og, fl = mr.planes(ids, cu, MARKER)
        mr.apply(q, k, pl)
        torch.cuda.synchronize()
        epl, est, eam, eog = _check_scan(b, pl, st, am, og, fl, b.name)
    assert torch.equal(q[..., 64:], q_tail) and torch.equal(k[..., 64:], k_tail)
    del q_tail, k_tail
    info = compare_heads_all(q, qn, epl, b.dtype, what=f"{b.name} q")
    compare_heads_all(k, kn, epl, b.dtype, what=f"{b.name} k")
    say(f"  every element compared: {info}")
    del q, k
    torch.cuda.empty_cache()
    return eog


def test_config2_full_64x4096():
    _full_prefill(synth.config2(), fused=False)


def test_config2_full_fused():
    _full_prefill(synth.config2(), fused=True)


def test_config3_full_fused_8x32768():
    _full_prefill(synth.config3(), fused=True)


def test_config5_full_ragged():
    b = synth.config5()
    eog = _full_prefill(b, fused=False)
    assert (eog[1::2] == -1).all() and (eog[0::2] >= 0).all()


def test_config5_full_ragged_fused():
    _full_prefill(synth.config5(), fused=True)


def test_config5_full_ragged_fused_planes_out():
    """Past 262,144 tokens with planes_out, mrope_apply_ids runs the scan launch and then the
    rotation launch from planes_out."""
    _full_prefill(synth.config5(), fused=True, planes_out=True)


def _image_batch(name, seed, n_seqs, length, dtype):
    origins = [int(o) for o in np.random.default_rng(seed).integers(0, 513, size=n_seqs)]
    return synth._batch(name, seed, [length] * n_seqs, origins, dtype)


@pytest.mark.parametrize("fused", [False, True])
def test_fp32_past_the_store_hint_size(fused):
    """40 x 4096 fp32 tokens write 419 MB in place, past the size from which the rotation kernels'
    stores take the non-temporal hint: the hinted kernels against the oracle, every element."""
    _full_prefill(_image_batch("40x4096-image-f32", 12, 40, 4096, "f32"), fused=fused)


@pytest.mark.parametrize("seed,total,hi,dtype", [(12, 333333, 3000, "bf16"), (15, 1 << 19, 300, "bf16"),
                                                  (16, 400_001, 2000, "f16")])
def test_ragged_past_the_size_thresholds(seed, total, hi, dtype):
    """Ragged batches past the sizes where mrope_apply takes one-step workgroups and
    mrope_apply_ids the scan-first kernel, where planes_out makes mrope_apply_ids two launches and
    where stores take the non-temporal hint: a total that leaves the last chunk partial (333,333
    tokens, 408 sequences), 3,426 short sequences (more than one 64-sequence window per chunk), and
    the same kernels in fp16 (400,001 tokens).  Scalars, planes and every rotated element in full,
    for the fused call with and without planes_out, out of place (inputs untouched), and for
    planes + apply."""
    lengths, kinds = synth.ragged_lengths(seed, total, hi=hi)
    g = np.random.default_rng(seed)
    placed = [int(g.integers(0, max(1, n - 67))) if k else None for n, k in zip(lengths, kinds)]
    b = synth._batch(f"ragged{seed}-{dtype}", seed, lengths, placed, dtype)
    say(f"case: {b.name} tokens={b.n_tokens} seqs={b.n_seqs}")
    qn, kn = b.qk()
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    epl, est, eam, eog = _oracle_planes(b)
    for mode in ("fused", "fused_planes_out", "fused_out_of_place", "planes_apply"):
        q, k = dev_heads(qn, dtype), dev_heads(kn, dtype)
        pl = torch.full((3, b.n_tokens), -9, dtype=torch.int32, device="cuda")
        if mode == "fused":
            st, am, og, fl, _ = mr.apply_ids(q, k, ids, cu, MARKER)
        elif mode == "fused_out_of_place":
            qo, ko = torch.empty_like(q), torch.empty_like(k)
            st, am, og, fl, _ = mr.apply_ids(q, k, ids, cu, MARKER, q_out=qo, k_out=ko)
            np.testing.assert_array_equal(host_heads(q), qn, err_msg="q input changed")
            np.testing.assert_array_equal(host_heads(k), kn, err_msg="k input changed")
            q, k = qo, ko
        elif mode == "fused_planes_out":
            st, am, og, fl, _ = mr.apply_ids(q, k, ids, cu, MARKER, planes_out=pl)
        else:
            _, st, am, og, fl = mr.planes(ids, cu, MARKER, out=pl)
            mr.apply(q, k, pl)
        for got, want, what in ((st, est, "start"), (am, eam, "amount"), (og, eog, "origin")):
            np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"{mode} {what}")
        np.testing.assert_array_equal(fl.cpu().numpy(), expected_flags(b, eog), err_msg=f"{mode} flags")
        if mode in ("fused_planes_out", "planes_apply"):
            np.testing.assert_array_equal(pl.cpu().numpy(), epl, err_msg=f"{mode} planes")
        compare_heads_all(q, qn, epl, dtype, what=f"{mode} q")
        compare_heads_all(k, kn, epl, dtype, what=f"{mode} k")
        del q, k, pl
        torch.cuda.empty_cache()


def test_config4_decode_paged():
    d = synth.config4()
    say(f"case: {d.name}")
    qn, kn = d.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    cache = torch.full((d.num_blocks, d.block_size, d.n_k_heads, d.head_dim), 0, dtype=torch.int16,
                       device="cuda").fill_(d.sentinel_bits - (1 << 16)).view(torch.bfloat16)
    pos, amount, slots = i32(d.pos), i32(d.amount), torch.from_numpy(d.slot_mapping).cuda()
    mr.decode(q, k, pos, amount, cache, slots)
    torch.cuda.synchronize()
    # Q: every element against the oracle at plane pos - amount
    ref_q = oracle.rotate(as_f32(qn, "bf16"), np.stack([d.pos - d.amount] * 3))
    ok, info = check_bf16(host_heads(q), oracle.round_bf16(ref_q))
    assert ok, info
    # K: the rotated heads at their slots ...
    ref_k = oracle.rotate(as_f32(kn, "bf16"), np.stack([d.pos - d.amount] * 3))
    blk = torch.from_numpy(d.slot_mapping // d.block_size).cuda()
    row = torch.from_numpy(d.slot_mapping % d.block_size).cuda()
    got_k = host_heads(cache[blk, row])
    ok, info = check_bf16(got_k, oracle.round_bf16(ref_k))
    assert ok, info
    # ... and every other slot still holds the sentinel
    untouched = (cache.view(torch.int16) != (d.sentinel_bits - (1 << 16))).sum().item()
    assert untouched == d.n_seqs * d.n_k_heads * d.head_dim
    # decode == prefill rotation of the same token at plane p - amount (oracle cross-check)
    qo = oracle.decode(as_f32(qn[:64], "bf16"), as_f32(kn[:64], "bf16"), d.pos[:64], d.amount[:64],
                       np.zeros((64, d.block_size, 2, 256), np.float32), np.arange(64) * d.block_size, d.block_size)
    np.testing.assert_array_equal(qo, ref_q[:64])


def test_decode_skips_negative_and_out_of_range_slots():
    d = synth.config4(n_seqs=64, num_blocks=64)
    qn, kn = d.qk()
    slots = np.arange(64, dtype=np.int64)
    slots[::3] = -1
    slots[1::7] = 8 * 16 + 5      # past the cache
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    cache = torch.zeros((8, 16, 2, 256), dtype=torch.bfloat16, device="cuda")
    mr.decode(q, k, i32(d.pos), i32(d.amount), cache, torch.from_numpy(slots).cuda())
    ref_k = oracle.round_bf16(oracle.rotate(as_f32(kn, "bf16"), np.stack([d.pos - d.amount] * 3)))
    c = host_heads(cache)
    for s in range(64):
        sl = slots[s]
        if 0 <= sl < 128:
            ok, info = check_bf16(c[sl // 16, sl % 16], ref_k[s])
            assert ok, info
    written = {int(s) for s in slots if 0 <= s < 128}
    for sl in range(128):
        if sl not in written:
            assert (c[sl // 16, sl % 16] == 0).all()


def test_workspace_reuse_across_sizes():
    """Back-to-back calls of different sizes on one workspace: the epoch and counters carry over."""
    ws = mr.Workspace(1 << 16)
    for i, seed in enumerate((51, 52, 53, 54, 55, 56)):
        b = synth.random_batch(seed, 20 + 30 * i, max_len=400 + 200 * i, empty_frac=0.05)
        pl, st, am, og, fl = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER, workspace=ws)
        _check_scan(b, pl, st, am, og, fl, f"reuse {i}")


def test_device_epoch_mode_through_c_abi():
    """epoch = 0: the library tags status words from its device counter and advances it after each
    call (one extra one-thread kernel); back-to-back calls with new inputs stay exact."""

    lib = mr._lib.load()
    ws = mr.Workspace(1 << 15)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i, seed in enumerate((61, 62, 63, 64)):
        b = synth.random_batch(seed, 40, max_len=700)
        ids, cu = i32(b.ids), i32(b.cu_seqlens)
        L, n = b.n_tokens, b.n_seqs
        pl = torch.empty((3, L), dtype=torch.int32, device="cuda")
        st, am, og, fl = (torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(4))
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        ws.ensure(L)
        rc = lib.mrope_planes(p(ids), p(cu), n, L, MARKER, 0, None, None, None, p(pl), L, p(st), p(am), p(og), p(fl), ws.ptr,
                              ws.capacity, 0, stream)
        assert rc == 0
        _check_scan(b, pl, st, am, og, fl, f"device epoch call {i}")
    hdr = ws.view[:4].view(torch.int32).item()
    assert hdr == 4


def _fused_device_epoch(lib, ws, q, k, b, stream):
    """mrope_apply_ids through the C ABI with epoch 0 (the workspace's device counter), in place;
    returns (start, amount, origin, seq_flags)."""
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    n = b.n_seqs
    st, am, og, fl = (torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(4))
    dt = {torch.bfloat16: 1, torch.float16: 2, torch.float32: 0}[q.dtype]
    ws.ensure(b.n_tokens)
    rc = lib.mrope_apply_ids(p(q), q.stride(0), q.stride(1), q.shape[1], p(k), k.stride(0), k.stride(1), k.shape[1],
                             b.n_tokens, q.shape[2], 64, dt, 1e7, None, None, p(ids), p(cu), n, MARKER, 67, None,
                             None, None, None, 0, p(st), p(am), p(og), p(fl), ws.ptr, ws.capacity, 0, stream)
    assert rc == 0, mr._lib.load().mrope_last_error()
    return st, am, og, fl


def test_device_epoch_advances_once_per_call():
    """epoch = 0 on one workspace, a mix of calls -- mrope_planes and the chunked fused kernel on
    small batches, the chunked kernel with other head shapes on 300,000 tokens (1,172 workgroups),
    the scan-first kernel forced on a small batch: each gives the oracle's scalars and rotation, and
    afterwards the device counter has advanced exactly once per call (the header's next word, which
    the library does not use, stays zero)."""
    lib = mr._lib.load()
    ws = mr.Workspace(300_000)  # sized once: a larger workspace would start a new counter
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = 0

    def fused(b, nq=8, nk=2, D=256, hooks=0):
        nonlocal calls
        x = synth.normal(b.seed, 91, b.n_tokens * (nq + nk) * D).reshape(b.n_tokens, nq + nk, D)
        xb = synth.to_dtype(x, "bf16")
        qn, kn = np.ascontiguousarray(xb[:, :nq]), np.ascontiguousarray(xb[:, nq:])
        q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
        prev = mr._lib.set_test_hooks(hooks)
        try:
            st, am, og, fl = _fused_device_epoch(lib, ws, q, k, b, stream)
        finally:
            mr._lib.set_test_hooks(prev)
        calls += 1
        epl, est, eam, eog = _oracle_planes(b)
        for got, want, what in ((st, est, "start"), (am, eam, "amount"), (og, eog, "origin")):
            np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"call {calls} {what}")
        compare_heads_all(q, qn, epl, "bf16", what=f"call {calls} q")
        compare_heads_all(k, kn, epl, "bf16", what=f"call {calls} k")

    def planes(b):
        nonlocal calls
        ids, cu = i32(b.ids), i32(b.cu_seqlens)
        L, n = b.n_tokens, b.n_seqs
        pl = torch.empty((3, L), dtype=torch.int32, device="cuda")
        st, am, og, fl = (torch.empty(n, dtype=torch.int32, device="cuda") for _ in range(4))
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        ws.ensure(L)
        assert lib.mrope_planes(p(ids), p(cu), n, L, MARKER, 0, None, None, None, p(pl), L, p(st), p(am), p(og),
                                p(fl), ws.ptr, ws.capacity, 0, stream) == 0
        calls += 1
        _check_scan(b, pl, st, am, og, fl, f"call {calls} planes")

    say("case: device epochs, small planes and fused calls")
    planes(synth.random_batch(71, 40, max_len=700))
    fused(synth.random_batch(72, 30, max_len=900))
    say("case: device epochs, 300,000 tokens with 4 Q + 1 K heads of 128 (large grid)")
    lengths, kinds = synth.ragged_lengths(73, 300_000, hi=3000)
    g = np.random.default_rng(73)
    placed = [int(g.integers(0, max(1, n - 67))) if kd else None for n, kd in zip(lengths, kinds)]
    fused(synth._batch("ragged73", 73, lengths, placed, "bf16"), nq=4, nk=1, D=128)
    say("case: device epochs, scan-first kernel forced on a small batch")
    fused(synth.random_batch(74, 20, max_len=1500), hooks=mr._lib.HOOK_FUSED_SCAN_FIRST)
    fused(synth.random_batch(75, 1, max_len=110, min_len=110))
    planes(synth.random_batch(76, 3, max_len=300))
    torch.cuda.synchronize()
    hdr = ws.view[:8].view(torch.int32).cpu().numpy()
    assert hdr[0] == calls, f"device epoch {hdr[0]} after {calls} calls"
    assert hdr[1] == 0, f"header word 1 changed to {hdr[1]}"


def test_graph_replays_with_new_inputs():
    """planes + apply captured in a HIP graph; between replays new ids and Q/K are copied into the
    captured buffers (eager work in between); every replay matches the oracle."""
    L, n = 6000, 24
    batches = []
    for seed in (71, 72, 73):
        g = np.random.default_rng(seed)
        cuts = np.sort(g.choice(np.arange(1, L), size=n - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [L]]))
        placed = [int(g.integers(0, max(1, m - 67))) if g.uniform() < 0.7 else None for m in lens]
        gi = synth.rng(seed, 4)
        ids = np.concatenate([synth.prompt_ids(gi, int(m), o) for m, o in zip(lens, placed)])
        cu = np.zeros(n + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        b = synth.Prefill(f"graph{seed}", ids, cu, placed, "bf16", seed=seed)
        batches.append((b,) + b.qk())
    ids_d = torch.zeros(L, dtype=torch.int32, device="cuda")
    cu_d = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    q_d = torch.zeros((L, 8, 256), dtype=torch.bfloat16, device="cuda")
    k_d = torch.zeros((L, 2, 256), dtype=torch.bfloat16, device="cuda")
    pl_d = torch.zeros((3, L), dtype=torch.int32, device="cuda")
    st_d, am_d, og_d, fl_d = (torch.zeros(n, dtype=torch.int32, device="cuda") for _ in range(4))
    ws = mr.Workspace(L)

    def load(bt):
        b, qn, kn = bt
        ids_d.copy_(i32(b.ids))
        cu_d.copy_(i32(b.cu_seqlens))
        q_d.copy_(dev_heads(qn, "bf16"))
        k_d.copy_(dev_heads(kn, "bf16"))

    def body():
        mr.planes(ids_d, cu_d, MARKER, out=pl_d, start=st_d, amount=am_d, origin=og_d, seq_flags=fl_d, workspace=ws)
        mr.apply(q_d, k_d, pl_d)

    load(batches[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()                     # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    for rep in range(6):
        bt = batches[rep % 3]
        load(bt)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        b, qn, kn = bt
        epl, *_ = _check_scan(b, pl_d, st_d, am_d, og_d, fl_d, f"replay {rep}")
        compare_heads(host_heads(q_d), qn, epl, "bf16", what=f"replay {rep} q")
        compare_heads(host_heads(k_d), kn, epl, "bf16", what=f"replay {rep} k")
        _ = torch.randn(1000, device="cuda").sum().item()   # unrelated eager work between replays


def test_graph_replays_fused_and_decode():
    """The fused call (no planes_out, so chunks inside one sequence take the per-chunk handover; the
    device epoch counter and its one-thread kernel under capture), the same call out of place first
    (its copy launch and its rotation launch) and a decode step with V, captured in one HIP graph.
    New prompts, Q/K and decode inputs are copied into the captured buffers between replays, with
    unrelated eager work in between; every replay matches the oracle, and the out-of-place heads
    equal the in-place result."""
    L, n = 6000, 6
    batches = []
    for seed in (81, 82, 83):
        g = np.random.default_rng(seed)
        cuts = np.sort(g.choice(np.arange(600, L - 600), size=n - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [L]]))
        placed = [int(g.integers(0, max(1, m - 67))) if g.uniform() < 0.7 else None for m in lens]
        gi = synth.rng(seed, 4)
        ids = np.concatenate([synth.prompt_ids(gi, int(m), o) for m, o in zip(lens, placed)])
        cu = np.zeros(n + 1, np.int32)
        cu[1:] = np.cumsum(lens)
        b = synth.Prefill(f"graphf{seed}", ids, cu, placed, "bf16", seed=seed)
        gd = np.random.default_rng(seed + 100)
        S = 96
        pos = gd.integers(100, 30000, S).astype(np.int32)
        amount = np.where(gd.uniform(size=S) < 0.5, 58, 0).astype(np.int32)
        slots = gd.permutation(128 * 16)[:S].astype(np.int64)
        dq = synth.to_dtype(gd.standard_normal((S, 8, 256)).astype(np.float32), "bf16")
        dk = synth.to_dtype(gd.standard_normal((S, 2, 256)).astype(np.float32), "bf16")
        dv = synth.to_dtype(gd.standard_normal((S, 2, 256)).astype(np.float32), "bf16")
        batches.append((b,) + b.qk() + (pos, amount, slots, dq, dk, dv))
    S = 96
    ids_d = torch.zeros(L, dtype=torch.int32, device="cuda")
    cu_d = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    q_d = torch.zeros((L, 8, 256), dtype=torch.bfloat16, device="cuda")
    k_d = torch.zeros((L, 2, 256), dtype=torch.bfloat16, device="cuda")
    st_d, am_d, og_d, fl_d = (torch.zeros(n, dtype=torch.int32, device="cuda") for _ in range(4))
    pos_d, amt_d = (torch.zeros(S, dtype=torch.int32, device="cuda") for _ in range(2))
    slots_d = torch.zeros(S, dtype=torch.int64, device="cuda")
    dq_d = torch.zeros((S, 8, 256), dtype=torch.bfloat16, device="cuda")
    dk_d, dv_d = (torch.zeros((S, 2, 256), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    kc = torch.zeros((128, 16, 2, 256), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    qo_d, ko_d = torch.zeros_like(q_d), torch.zeros_like(k_d)
    ws = mr.Workspace(L)

    def load(bt):
        b, qn, kn, pos, amount, slots, dq, dk, dv = bt
        ids_d.copy_(i32(b.ids))
        cu_d.copy_(i32(b.cu_seqlens))
        q_d.copy_(dev_heads(qn, "bf16"))
        k_d.copy_(dev_heads(kn, "bf16"))
        pos_d.copy_(i32(pos))
        amt_d.copy_(i32(amount))
        slots_d.copy_(torch.from_numpy(slots).cuda())
        dq_d.copy_(dev_heads(dq, "bf16"))
        dk_d.copy_(dev_heads(dk, "bf16"))
        dv_d.copy_(dev_heads(dv, "bf16"))

    def body():
        mr.apply_ids(q_d, k_d, ids_d, cu_d, MARKER, q_out=qo_d, k_out=ko_d, workspace=ws)
        mr.apply_ids(q_d, k_d, ids_d, cu_d, MARKER, start=st_d, amount=am_d, origin=og_d, seq_flags=fl_d,
                     workspace=ws)
        mr.decode(dq_d, dk_d, pos_d, amt_d, kc, slots_d, v=dv_d, v_cache=vc)

    load(batches[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()                     # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    for rep in range(6):
        bt = batches[rep % 3]
        b, qn, kn, pos, amount, slots, dq, dk, dv = bt
        load(bt)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        epl, est, eam, eog = _oracle_planes(b)
        for got, want, what in ((st_d, est, "start"), (am_d, eam, "amount"), (og_d, eog, "origin")):
            np.testing.assert_array_equal(got.cpu().numpy(), want, err_msg=f"replay {rep} {what}")
        compare_heads(host_heads(q_d), qn, epl, "bf16", what=f"replay {rep} q")
        compare_heads(host_heads(k_d), kn, epl, "bf16", what=f"replay {rep} k")
        assert torch.equal(qo_d, q_d) and torch.equal(ko_d, k_d), f"replay {rep}: out of place differs from in place"
        plane = np.stack([pos - amount] * 3)
        compare_heads(host_heads(dq_d), dq, plane, "bf16", what=f"replay {rep} decode q")
        rows = torch.from_numpy(slots).cuda()
        compare_heads(host_heads(kc.view(-1, 2, 256)[rows]), dk, plane, "bf16", what=f"replay {rep} decode k cache")
        assert np.array_equal(host_heads(vc.view(-1, 2, 256)[rows]), dv), f"replay {rep} decode v cache"
        _ = torch.randn(1000, device="cuda").sum().item()   # unrelated eager work between replays


def test_bf16_out_of_place_and_wide_plane_stride():
    """bf16 out of place == in place (full heads written, inputs untouched); planes written into a
    wider [3, L + 37] buffer leave the extra columns alone."""
    b = synth.random_batch(81, 25, max_len=500)
    qn, kn = b.qk()
    L = b.n_tokens
    wide = torch.full((3, L + 37), -5, dtype=torch.int32, device="cuda")
    mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER, out=wide)
    assert (wide[:, L:] == -5).all()
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    np.testing.assert_array_equal(wide[:, :L].cpu().numpy(), epl)
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    mr.apply(q, k, wide, q_out=qo, k_out=ko)
    np.testing.assert_array_equal(host_heads(q), qn)
    compare_heads(host_heads(qo), qn, epl, "bf16", what="q out of place")
    compare_heads(host_heads(ko), kn, epl, "bf16", what="k out of place")
    q2, k2 = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    mr.apply(q2, k2, wide)
    assert torch.equal(q2, qo) and torch.equal(k2, ko)
    # fused, out of place, Q only
    q3 = dev_heads(qn, "bf16")
    q3o = torch.empty_like(q3)
    mr.apply_ids(q3, None, i32(b.ids), i32(b.cu_seqlens), MARKER, q_out=q3o)
    assert torch.equal(q3o, qo)
    np.testing.assert_array_equal(host_heads(q3), qn)


def test_out_of_place_generic_shapes_and_padded_strides():
    """Out of place with head counts that are not powers of two, other head dims and padded
    strides: the outputs hold the rotated dims and the rest of every head bit for bit, the inputs
    are untouched, and the padding between the heads and tokens of the outputs is never written."""
    b = synth.random_batch(83, 24, max_len=240)
    T = b.n_tokens
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    sentinel = -3.0

    def padded(nh, D, pad_h, pad_t, tdt):
        """A [T, nh, D] view into a sentinel-filled buffer with padding after every head and token."""
        buf = torch.full((T * (nh * (D + pad_h) + pad_t),), sentinel, dtype=tdt, device="cuda")
        view = buf.as_strided((T, nh, D), (nh * (D + pad_h) + pad_t, D + pad_h, 1))
        outside = torch.ones(buf.shape, dtype=torch.bool, device="cuda")
        outside.as_strided((T, nh, D), view.stride()).fill_(False)
        return buf, view, outside

    for case, (dt, nq, nk, D, pad_h, pad_t) in enumerate((("f16", 3, 1, 136, 8, 16), ("f32", 3, 3, 1024, 4, 0),
                                                          ("bf16", 8, 2, 256, 8, 64), ("bf16", 5, 0, 64, 0, 8),
                                                          ("f32", 8, 2, 256, 0, 4))):
        say(f"case: out of place {dt} {nq}+{nk} heads of {D}, head pad {pad_h}, token pad {pad_t}")
        tdt = TORCH_DT[dt]
        xq = synth.to_dtype(synth.normal(83, 70 + case, T * nq * D), dt).reshape(T, nq, D)
        xk = synth.to_dtype(synth.normal(83, 80 + case, T * nk * D), dt).reshape(T, nk, D) if nk else None
        _, q_in, _ = padded(nq, D, pad_h, pad_t, tdt)
        q_in.copy_(dev_heads(xq, dt))
        qo_buf, q_out, q_pad = padded(nq, D, pad_h, pad_t, tdt)
        k_in = k_out = None
        if nk:
            _, k_in, _ = padded(nk, D, pad_h, pad_t, tdt)
            k_in.copy_(dev_heads(xk, dt))
            ko_buf, k_out, k_pad = padded(nk, D, pad_h, pad_t, tdt)
        for fused in (False, True):
            qo_buf.fill_(sentinel)
            if nk:
                ko_buf.fill_(sentinel)
            if fused:
                mr.apply_ids(q_in, k_in, i32(b.ids), i32(b.cu_seqlens), MARKER, q_out=q_out, k_out=k_out)
            else:
                mr.apply(q_in, k_in, pl, q_out=q_out, k_out=k_out)
            what = f"{dt} {nq}+{nk}x{D} {'fused' if fused else 'apply'}"
            np.testing.assert_array_equal(host_heads(q_in), xq, err_msg=f"{what}: q input changed")
            compare_heads(host_heads(q_out), xq, epl, dt, what=f"{what} q_out")
            assert bool((qo_buf[q_pad] == sentinel).all()), f"{what}: q_out padding written"
            if nk:
                np.testing.assert_array_equal(host_heads(k_in), xk, err_msg=f"{what}: k input changed")
                compare_heads(host_heads(k_out), xk, epl, dt, what=f"{what} k_out")
                assert bool((ko_buf[k_pad] == sentinel).all()), f"{what}: k_out padding written"


def test_out_of_place_one_head_set_only():
    """Out of place with only K heads (no Q heads, k_out alone) and with only Q heads (q_out alone):
    the one output holds every dim of every head -- the rotated dims and, from the copy launch, the
    rest -- and the input is untouched."""
    b = synth.random_batch(84, 16, max_len=200)
    T = b.n_tokens
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    for case, (dt, nh, D, k_side) in enumerate((("bf16", 2, 256, True), ("f32", 3, 128, True),
                                                ("bf16", 8, 256, False), ("f16", 1, 72, False))):
        say(f"case: out of place, {'K' if k_side else 'Q'} heads only: {dt} {nh}x{D}")
        x = synth.to_dtype(synth.normal(84, 90 + case, T * nh * D), dt).reshape(T, nh, D)
        src = dev_heads(x, dt)
        out = torch.full_like(src, -3.0)
        none = torch.empty((T, 0, D), dtype=TORCH_DT[dt], device="cuda")
        for fused in (False, True):
            out.fill_(-3.0)
            q_in, k_in = (none, src) if k_side else (src, None)
            kw = dict(k_out=out) if k_side else dict(q_out=out)
            if fused:
                mr.apply_ids(q_in, k_in, i32(b.ids), i32(b.cu_seqlens), MARKER, **kw)
            else:
                mr.apply(q_in, k_in, pl, **kw)
            what = f"{dt} {nh}x{D} {'K' if k_side else 'Q'} only {'fused' if fused else 'apply'}"
            np.testing.assert_array_equal(host_heads(src), x, err_msg=f"{what}: input changed")
            compare_heads(host_heads(out), x, epl, dt, what=what)


def test_decode_fp32_and_generic_shapes():
    d = synth.config4(n_seqs=300, num_blocks=512)
    g = synth.rng(91, 5)
    for dt, nq, nk, D in (("f32", 8, 2, 256), ("bf16", 4, 1, 128), ("f32", 3, 3, 64), ("f16", 8, 2, 256)):
        qf = synth.normal(91, 70, d.n_seqs * nq * D).reshape(d.n_seqs, nq, D)
        kf = synth.normal(91, 71, d.n_seqs * nk * D).reshape(d.n_seqs, nk, D)
        qn, kn = synth.to_dtype(qf, dt), synth.to_dtype(kf, dt)
        q, k = dev_heads(qn, dt), dev_heads(kn, dt)
        tdt = TORCH_DT[dt]
        cache = torch.zeros((512, 16, nk, D), dtype=tdt, device="cuda")
        pos = g.integers(0, 40000, size=d.n_seqs).astype(np.int32)
        amount = np.where(g.uniform(size=d.n_seqs) < 0.5, 58, 0).astype(np.int32)
        slots = g.permutation(512 * 16)[:d.n_seqs].astype(np.int64)
        mr.decode(q, k, i32(pos), i32(amount), cache, torch.from_numpy(slots).cuda())
        plane = np.stack([pos - amount] * 3)
        compare_heads(host_heads(q), qn, plane, dt, what=f"decode q {dt} {nq}x{D}")
        got_k = host_heads(cache[torch.from_numpy(slots // 16).cuda(), torch.from_numpy(slots % 16).cuda()])
        compare_heads(got_k, kn, plane, dt, what=f"decode k {dt} {nk}x{D}")


def test_binding_raises_library_status():
    q = torch.zeros((4, 8, 256), dtype=torch.bfloat16, device="cuda")
    pl = torch.zeros((3, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(mr.MropeError) as e:
        mr.apply(q, None, pl, rot_dim=32)
    assert e.value.status == 3 and "rot_dim" in str(e.value)
    with pytest.raises(mr.MropeError) as e:
        mr.apply(q, None, pl, theta=-1.0)
    assert e.value.status == 1
    with pytest.raises(mr.MropeError) as e:
        mr.apply(q[:, :, 4:], None, pl)   # head_dim 252: not a multiple of 8
    assert e.value.status == 3


def test_workspace_init_recovers_garbage():
    """A workspace full of garbage words (which can carry any epoch tag) is made safe by
    mrope_workspace_init; results are then exact in both epoch modes."""

    lib = mr._lib.load()
    b = synth.random_batch(95, 30, max_len=2000)
    ws = mr.Workspace(b.n_tokens)
    ws.view.fill_(0xFF)
    rc = lib.mrope_workspace_init(ws.ptr, ws.capacity, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    assert int(ws.view.sum().item()) == 0
    pl, st, am, og, fl = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER, workspace=ws)
    _check_scan(b, pl, st, am, og, fl, "after init")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rounding_is_nearest_even(dtype):
    """The 1-ulp gate alone would pass a kernel that truncates; nearest-even rounding of an accurate
    result leaves only rare 1-ulp differences (results within ~1e-16 of a rounding boundary)."""
    b = synth.random_batch(111, 40, max_len=1000, dtype=dtype)
    qn, kn = b.qk()
    pl, *_ = mr.planes(i32(b.ids), i32(b.cu_seqlens), MARKER)
    epl, *_ = oracle.planes(b.ids, b.cu_seqlens, MARKER)
    q = dev_heads(qn, dtype)
    mr.apply(q, None, pl)
    info = compare_heads(host_heads(q), qn, epl, dtype, what=f"{dtype} rounding")
    assert info["frac_off_by_one"] < 1e-3, info


@pytest.mark.parametrize("frame_len", [65, 66, 68, 75])
def test_frame_len_planes_and_fused(frame_len):
    """Frames of other lengths (marker runs after </image>; Qwen-VL's rule at 65): planes, scalars
    and flags of mrope_planes and the fused call against the oracle's rule for that length."""
    b = synth.random_batch(301 + frame_len, 40, max_len=600, dtype="bf16", empty_frac=0.05)
    say(f"case: frame_len={frame_len} tokens={b.n_tokens}")
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len=frame_len)
    assert (eam[eog >= 0] == frame_len - 9).all()
    want_fl = expected_flags(b, eog) & 1
    lens = np.diff(b.cu_seqlens)
    want_fl |= np.where((eog >= 0) & (eog + frame_len > lens), 2, 0).astype(np.int32)
    ids, cu = i32(b.ids), i32(b.cu_seqlens)
    pl, st, am, og, fl = mr.planes(ids, cu, MARKER, frame_len=frame_len)
    np.testing.assert_array_equal(pl.cpu().numpy(), epl)
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    np.testing.assert_array_equal(am.cpu().numpy(), eam)
    np.testing.assert_array_equal(og.cpu().numpy(), eog)
    np.testing.assert_array_equal(fl.cpu().numpy(), want_fl)
    qn, kn = b.qk()
    q, k = dev_heads(qn, "bf16"), dev_heads(kn, "bf16")
    pl2 = torch.full_like(pl, -7)
    st2, am2, og2, fl2, _ = mr.apply_ids(q, k, ids, cu, MARKER, planes_out=pl2, frame_len=frame_len)
    np.testing.assert_array_equal(pl2.cpu().numpy(), epl)
    np.testing.assert_array_equal(fl2.cpu().numpy(), want_fl)
    compare_heads(host_heads(q), qn, epl, "bf16", what=f"q frame_len={frame_len}")
    compare_heads(host_heads(k), kn, epl, "bf16", what=f"k frame_len={frame_len}")
    # long sequences without planes_out: chunks wholly before the image, cutting the frame, and
    # wholly after it take the per-chunk handover, whose shift depends on the frame length
    lens, placed = [3000, 2000, 1300], [1000, 470, 500]
    g = synth.rng(341 + frame_len, 4)
    ids3 = np.concatenate([synth.prompt_ids(g, n, o) for n, o in zip(lens, placed)])
    cu3 = np.zeros(4, np.int32)
    cu3[1:] = np.cumsum(lens)
    b3 = synth.Prefill(f"long-frame{frame_len}", ids3, cu3, placed, "bf16", seed=341, head_dim=64)
    epl3, est3, eam3, eog3 = oracle.planes_chunk(ids3, cu3, MARKER, frame_len=frame_len)
    qn3, kn3 = b3.qk()
    q3, k3 = dev_heads(qn3, "bf16"), dev_heads(kn3, "bf16")
    st3, am3, og3, _, _ = mr.apply_ids(q3, k3, i32(ids3), i32(cu3), MARKER, frame_len=frame_len)
    np.testing.assert_array_equal(st3.cpu().numpy(), est3)
    np.testing.assert_array_equal(am3.cpu().numpy(), eam3)
    compare_heads(host_heads(q3), qn3, epl3, "bf16", what=f"long q frame_len={frame_len}")
    compare_heads(host_heads(k3), kn3, epl3, "bf16", what=f"long k frame_len={frame_len}")


def test_frame_len_pieces_cut_inside_the_tail():
    """A 75-token frame fed in two pieces cut inside its marker run: the pieces equal the whole."""
    frame_len = 75
    b = synth.random_batch(331, 24, max_len=700, text_frac=0.0)
    epl, est, eam, eog = oracle.planes_chunk(b.ids, b.cu_seqlens, MARKER, frame_len=frame_len)
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
        pl, st, am, og, fl = mr.planes(i32(b.ids[rows]), i32(cu), MARKER, pos_offset=i32(lo.astype(np.int32)),
                                       origin_in=prev, frame_len=frame_len)
        got[:, rows] = pl.cpu().numpy()
        prev = og
    np.testing.assert_array_equal(got, epl)
    np.testing.assert_array_equal(st.cpu().numpy(), est)
    np.testing.assert_array_equal(am.cpu().numpy(), eam)
