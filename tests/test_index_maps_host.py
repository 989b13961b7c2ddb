"""Index arithmetic of the kernels, restated in Python and checked on the CPU over many shapes.

decode_kernel maps (lane, round, item slot) to a chunk of Q, K or V; copy_rest_kernel maps
(workgroup, lane, chunk) to bytes of an out-of-place head; the scan-first grid maps workgroups to
scans and parts; the sixteen-lane fp32 cache write maps (token group, lane, vector) to Q, K and V
elements and cache rows.  They map with arithmetic that a GPU test exercises for a few shapes only,
and a mistake there reads or writes outside a buffer.  These tests restate each mapping as the
kernel source computes it (the two must be changed together) and check that every access stays
inside its buffer and that each output element is written exactly once.
"""
import itertools

import numpy as np

# ------------------------------------------------------------------ decode_kernel ---------------


def _decode_items(nq, nk, D, v):
    return (nq + nk) * 8 + nk * (D - 64) // 8 + (nk * D // 8 if v else 0)


def _decode_item(it, nq, nk, D):
    """Vectorised decode_item: item index -> (kind, head, first element); kinds 0 Q rotation,
    1 K rotation, 2 K pass-through, 3 V."""
    nrq, nrk = nq * 8, nk * 8
    kpass, vch = (D - 64) // 8, D // 8
    n_rot, n_k = nrq + nrk, nrq + nrk + nk * kpass
    kind = np.where(it < nrq, 0, np.where(it < n_rot, 1, np.where(it < n_k, 2, 3)))
    l8 = it & 7
    e_rot = 32 * (l8 & 1) + 8 * (l8 >> 1)
    h_rot = np.where(kind == 0, it, it - nrq) >> 3
    c2 = it - n_rot
    h2 = c2 // max(kpass, 1)
    e2 = 64 + (c2 - h2 * kpass) * 8
    c3 = it - n_k
    h3 = c3 // vch
    e3 = (c3 - h3 * vch) * 8
    h = np.select([kind <= 1, kind == 2], [h_rot, h2], h3)
    e = np.select([kind <= 1, kind == 2], [e_rot, e2], e3)
    return kind, h, e


def _decode_lanes(items, ipl):
    need = (items + ipl - 1) // ipl
    return 1024 if need >= 1024 else (need + 63) // 64 * 64


def _decode_choice(items):
    """The host's items per lane (launch_decode): the most, up to 3, that leave under a wave of
    lanes idle with at most 256 lanes per sequence."""
    for c in (3, 2):
        if _decode_lanes(items, c) <= 256 and _decode_lanes(items, c) * c - items < 64:
            return c
    return 1


def test_decode_item_map_stays_in_bounds_and_pairs_rotation_items():
    bad = []
    for ipl in (1, 2, 3):
        for nq, nk, D, v in itertools.product(range(0, 12), range(0, 5), (64, 136, 256, 512), (False, True)):
            tot = _decode_items(nq, nk, D, v)
            if tot == 0:
                continue
            per = _decode_lanes(tot, ipl)
            li = np.arange(per)[:, None]
            j = np.arange(ipl)[None, :]
            for base in range(0, tot, per * ipl):
                it = base + li + j * per
                live = it < tot
                kind, h, e = _decode_item(np.where(live, it, 0), nq, nk, D)
                heads = np.where(kind == 0, nq, nk)
                ok = (h >= 0) & (h < heads) & (e >= 0) & (e + 8 <= D) & ((kind != 3) | v) & ((kind != 2) | (D > 64))
                # a live rotation item's DPP partner (lane li ^ 1) is live and the other half of its pair
                it2 = base + (li ^ 1) + j * per
                k2, h2, _ = _decode_item(np.where(it2 < tot, it2, 0), nq, nk, D)
                rot = live & (kind <= 1)
                ok &= ~rot | ((it2 < tot) & (k2 == kind) & (h2 == h))
                # every rotation item of a lane sits at the lane's place in its group of eight, so
                # the lane's one sincos serves all of them
                ok &= ~rot | ((it & 7) == (li & 7))
                if not ok.all():
                    bad.append((ipl, nq, nk, D, v, base))
    assert not bad, bad[:5]


def test_decode_items_per_lane_choice():
    for nq, nk, D, v in itertools.product(range(0, 40), range(0, 17), (64, 128, 256, 512), (False, True)):
        tot = _decode_items(nq, nk, D, v)
        if tot == 0:
            continue
        c = _decode_choice(tot)
        per = _decode_lanes(tot, c)
        assert per % 64 == 0 and per <= 1024
        assert c == 1 or per <= 256  # the 2- and 3-item kernels are built for 256 threads
    # the model's shape: 2 items per lane without V, 3 with V, one wave per sequence
    assert (_decode_choice(_decode_items(8, 2, 256, False)), _decode_lanes(128, 2)) == (2, 64)
    assert (_decode_choice(_decode_items(8, 2, 256, True)), _decode_lanes(192, 3)) == (3, 64)


# ------------------------------------------------------------------ copy_rest_kernel ------------

BLOCK, ROWS, BATCH = 256, 1, 3  # threads per workgroup, rows per lane and step, chunks per batch


def _copy_rest_writes(T, nh, D, es, tok_el, head_el, grid_cap=1 << 20):
    """Count how often each byte of the output buffer is stored; assert every load is in a row."""
    n_chunks = (D - 64) * es // 16
    size = (T - 1) * tok_el * es + (nh - 1) * head_el * es + D * es
    written = np.zeros(size, np.int64)
    if n_chunks <= 0:
        return written, n_chunks
    tok_b, head_b, row_from = tok_el * es, head_el * es, 64 * es
    n_rows = T * nh
    shift = (nh - 1).bit_length() if nh & (nh - 1) == 0 else -1
    rows_per_block = BLOCK // 8 * ROWS
    blocks = min((n_rows + rows_per_block - 1) // rows_per_block, grid_cap)
    stride = blocks * rows_per_block
    tid = np.arange(BLOCK)
    l8 = tid & 7
    for blk in range(blocks):
        r0 = blk * rows_per_block + (tid >> 3)
        while (r0 < n_rows).any():
            active = r0 < n_rows
            for jr in range(ROWS):
                row = r0 + jr * (BLOCK // 8)
                row_ok = row < n_rows
                rr = np.where(row_ok, row, n_rows - 1)
                t, h = (rr >> shift, rr & ((1 << shift) - 1)) if shift >= 0 else (rr // nh, rr % nh)
                base = t * tok_b + h * head_b + row_from
                c0 = l8.copy()
                while (active & (c0 - l8 < n_chunks)).any():
                    go = active & (c0 - l8 < n_chunks)
                    for b in range(BATCH):
                        c = c0 + 8 * b
                        a = base + 16 * np.minimum(c, n_chunks - 1)
                        # the load: inside the copied part of a head row
                        assert ((a - (t * tok_b + h * head_b) >= row_from) & (a + 16 - (t * tok_b + h * head_b) <= D * es))[go].all()
                        st = go & row_ok & (c < n_chunks)
                        for off in a[st]:
                            written[off:off + 16] += 1
                    c0 = c0 + 8 * BATCH
            r0 = r0 + stride
    return written, n_chunks


def test_copy_rest_map_copies_each_byte_once():
    cases = [(37, 3, 136, 2, 3 * 144 + 16, 144), (37, 1, 136, 2, 160, 144), (9, 3, 1024, 4, 3084, 1028),
             (50, 8, 256, 2, 8 * 264 + 64, 264), (50, 2, 256, 2, 2 * 264 + 64, 264), (21, 8, 256, 4, 8 * 256 + 4, 256),
             (70, 8, 256, 2, 2048, 256), (5, 5, 72, 2, 5 * 72, 72), (3, 7, 200, 4, 7 * 200, 200), (4, 4, 64, 2, 256, 64)]
    for T, nh, D, es, tok_el, head_el in cases:
        for cap in (1 << 20, 3):  # a capped grid runs the grid-stride loop
            written, n_chunks = _copy_rest_writes(T, nh, D, es, tok_el, head_el, cap)
            want = np.zeros_like(written)
            if n_chunks > 0:
                for t, h in itertools.product(range(T), range(nh)):
                    s = (t * tok_el + h * head_el) * es
                    want[s + 64 * es:s + D * es] = 1
            assert np.array_equal(written, want), (T, nh, D, es, tok_el, head_el, cap)


# ------------------------------------------------------------------ apply_ids_sf_kernel ---------
# Block roles of the scan-first fused kernel (sf_block_role and apply_ids_sf_dispatch): scan
# workgroups of 4 chunks, rotation workgroups of 32 tokens; the first `lead` scan workgroups first,
# then each further one after the 64 rotation workgroups of the chunks `lead` scan workgroups
# behind it; with the fallback hook the rotation workgroups come first.

def _sf_roles(n_tokens, lead_max=32, rot_first=False):
    n_chunks = -(-n_tokens // 512)
    n_scan = -(-n_chunks // 4)
    n_parts = -(-n_tokens // 32)
    lead = min(n_scan, lead_max)
    per = 64
    rot_blocks = n_parts if rot_first else max(n_parts, (n_scan - lead) * per)
    roles = []
    for b in range(n_scan + rot_blocks):
        if rot_first:
            is_scan = b >= n_parts
            idx = b - n_parts if is_scan else b
        elif b < lead:
            is_scan, idx = True, b
        else:
            u, ng, span = b - lead, n_scan - lead, per + 1
            if u < ng * span:
                grp, r = divmod(u, span)
                is_scan = r == per
                idx = lead + grp if is_scan else grp * per + r
            else:
                is_scan, idx = False, ng * per + (u - ng * span)
        roles.append((is_scan, idx))
    return roles, n_scan, n_parts


def test_scan_first_grid_covers_every_chunk_and_part_once():
    for n in (1, 31, 32, 33, 511, 512, 513, 2047, 2048, 2049, 65535, 65536, 65537, 262143, 262144, 300001,
              1 << 20, (1 << 20) + 17):
        for rot_first in (False, True):
            for lead in (1, 32):
                roles, n_scan, n_parts = _sf_roles(n, lead, rot_first)
                scans = sorted(i for s, i in roles if s)
                parts = [i for s, i in roles if not s]
                assert scans == list(range(n_scan)), (n, rot_first, lead)
                assert sorted(p for p in parts if p < n_parts) == list(range(n_parts)), (n, rot_first, lead)
                assert all(p * 32 >= n for p in parts if p >= n_parts), (n, rot_first, lead)


def test_scan_first_scans_run_ahead_of_their_parts():
    """Outside the fallback order, the scan workgroup of a chunk comes before every rotation
    workgroup of that chunk, by at least `lead` scan workgroups' worth of parts when it can."""
    for n in (70000, 300001, 1 << 20):
        roles, n_scan, n_parts = _sf_roles(n)
        pos_scan = {i: b for b, (s, i) in enumerate(roles) if s}
        for b, (s, i) in enumerate(roles):
            if s or i >= n_parts:
                continue
            chunk = i * 32 // 512
            assert pos_scan[chunk // 4] < b, (n, i)


# ------------------------------------------------------------------ fp32 cache writes, sixteen lanes


def _kv_w_lane_elements(l):
    """kv_token_w for lane l of a token's sixteen: (rotated dims of each Q/K head, K pass-through
    dims, V dims), each a list of the first elements of the lane's 4-element vectors."""
    m, half = l >> 1, l & 1
    e0 = 32 * half + 4 * m
    kpass = [64 + 4 * (l + 16 * i) for i in range(3)]
    vdims = [4 * (l + 16 * i) for i in range(4)]
    return [e0], kpass, vdims


def test_f32_cache_write_lane_map_covers_each_head_once():
    """Over a token's sixteen lanes: the rotated vectors tile dims 0..63 of a head, the K
    pass-through vectors dims 64..255 and the V vectors dims 0..255, each element exactly once; a
    lane's rotate-half partner (l ^ 1) holds the dims 32 away (x_j against x_{j+32})."""
    rot = np.zeros(64, int)
    kp = np.zeros(256, int)
    vv = np.zeros(256, int)
    for l in range(16):
        r, k, v = _kv_w_lane_elements(l)
        for e in r:
            rot[e:e + 4] += 1
        for e in k:
            kp[e:e + 4] += 1
        for e in v:
            vv[e:e + 4] += 1
        (rp,), _, _ = _kv_w_lane_elements(l ^ 1)
        assert abs(rp - r[0]) == 32 and (r[0] < 32) == (l % 2 == 0)
    assert (rot == 1).all()
    assert (kp[:64] == 0).all() and (kp[64:] == 1).all()
    assert (vv == 1).all()
    # one instruction (fixed vector index) of the sixteen lanes covers 256 contiguous bytes
    for i in range(3):
        firsts = sorted(64 + 4 * (l + 16 * i) for l in range(16))
        assert firsts == list(range(firsts[0], firsts[0] + 64, 4))


def test_f32_cache_write_grid_covers_every_token_once():
    """apply_kv_f32w_kernel: workgroup b, thread t, step s -> token b * 16 + (t >> 6) * 4 +
    ((t & 63) >> 4) + s * stride; with the host's grid (one step per workgroup) every token is
    taken by exactly one sixteen-lane group and no group reads past the last token."""
    for n in (1, 15, 16, 17, 255, 4096, 100003):
        blocks = (n + 15) // 16
        seen = np.zeros(n, int)
        for b in range(blocks):
            for t in range(0, 256, 16):  # one thread per sixteen-lane group
                G = b * 16 + (t >> 6) * 4
                stride = blocks * 16
                while G < n:
                    g = G + ((t & 63) >> 4)
                    if g < n:
                        seen[g] += 1
                    G += stride
        assert (seen == 1).all(), n
