#!/usr/bin/env python3
"""Benchmark of the canvas M-RoPE hot path on one MI355X.

A step is one pass of the whole prefill path over one batch, in one launch: mrope_apply_ids (token
ids -> first marker per sequence -> (T, H, W) planes, start, amount -> rotate-half of the first 64
dims of Q [L, 8, 256] and K [L, 2, 256], bf16, in place).  Workload: 64 image prompts of 4096 tokens
(262,144 tokens), <image> at O ~ U{0..512}, Q/K ~ N(0, 1) from a fixed seed, inputs resident in HBM
before the timed region.

Prints one JSON line: tokens/s over the timed steps; the roofline of the step's kernel
(mrope_apply_ids: algorithmic bytes / mean time of back-to-back launches from HIP events on its
stream, against 8 TB/s) and, beside it, that of the two-launch form's rotary kernel mrope_apply with
planes given; and the CPU oracle timed on this host over the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "canvas M-RoPE Q+K tokens/sec and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBS = 8000.0
COUNTERS = os.path.join(ROOT, "profiles", "rotary_kernels_64x4096_bf16_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "canvas_rope_rotary_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def algorithmic_bytes_apply(tokens: int, heads: int = 10, rot_dim: int = 64, elem: int = 2) -> int:
    """Bytes mrope_apply must move in place: the rotated dims of every head read and written once,
    plus the three int32 planes of every token read once."""
    return tokens * (heads * rot_dim * elem * 2 + 3 * 4)


def algorithmic_bytes_planes(tokens: int) -> int:
    """ids read (4 B) and three int32 planes written (12 B) per token."""
    return tokens * 16


def algorithmic_bytes_fused(tokens: int, heads: int = 10, rot_dim: int = 64, elem: int = 2) -> int:
    """mrope_apply_ids in place: ids read (4 B) and the rotated dims read and written, per token."""
    return tokens * (heads * rot_dim * elem * 2 + 4)


def algorithmic_bytes_fused_kv(tokens: int, q_heads: int = 8, kv_heads: int = 2, head_dim: int = 256,
                               rot_dim: int = 64, elem: int = 2) -> int:
    """mrope_apply_ids_kv: Q's rotated dims read and written, K and V heads read whole and written
    whole into the caches, one int32 id and one int64 slot, per token."""
    return tokens * (q_heads * rot_dim * elem * 2 + kv_heads * head_dim * elem * 4 + 4 + 8)


def graph_timed(fn, reps, warm=2):
    """Mean GPU time per call of `reps` calls captured in one HIP graph and replayed (no host launch
    overhead: for kernels shorter than the binding's per-call host time)."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(warm):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps / 1e3


def extras(args, dev, timed):
    """Other workloads of the method, one timing each (context; not the headline).  Kernels shorter
    than the host's per-call launch time are also timed from a replayed HIP graph."""
    import numpy as np
    import torch

    import canvas_rope_rotary_amd as mr
    from canvas_rope_rotary_amd import synth

    out = {}

    def heads(x, dt):
        if dt == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    for cfg in (synth.config3(), synth.config5(), synth.config1()):
        log(f"extras: {cfg.name}")
        qn, kn = cfg.qk()
        q, k = heads(qn, cfg.dtype), heads(kn, cfg.dtype)
        ids = torch.from_numpy(cfg.ids).to(dev)
        cu = torch.from_numpy(cfg.cu_seqlens).to(dev)
        ws = mr.Workspace(cfg.n_tokens, dev)
        pl = torch.empty((3, cfg.n_tokens), dtype=torch.int32, device=dev)
        elem = 2 if cfg.dtype == "bf16" else 4
        f_us = timed(lambda: mr.apply_ids(q, k, ids, cu, synth.IMAGE_ID, workspace=ws), args.steps) * 1e6
        p_us = timed(lambda: mr.planes(ids, cu, synth.IMAGE_ID, out=pl, workspace=ws), args.steps) * 1e6
        a_us = timed(lambda: mr.apply(q, k, pl), args.steps) * 1e6
        small = cfg.n_tokens < 65536
        if small:  # launch-bound: GPU time from a graph (scans then use the device epoch counter)
            f_us = graph_timed(lambda: mr.apply_ids(q, k, ids, cu, synth.IMAGE_ID, workspace=ws), args.steps) * 1e6
            p_us = graph_timed(lambda: mr.planes(ids, cu, synth.IMAGE_ID, out=pl, workspace=ws), args.steps) * 1e6
            a_us = graph_timed(lambda: mr.apply(q, k, pl), args.steps) * 1e6
        out[cfg.name] = {"tokens": cfg.n_tokens, "fused_us": f_us, "planes_us": p_us, "apply_us": a_us,
                         "timing": "hip graph replay" if small else "hip events, back-to-back launches",
                         "fused_gbs": algorithmic_bytes_fused(cfg.n_tokens, elem=elem) / f_us / 1e3,
                         "apply_gbs": algorithmic_bytes_apply(cfg.n_tokens, elem=elem) / a_us / 1e3,
                         "tokens_per_s_fused": cfg.n_tokens / (f_us / 1e6)}
        if small:  # out of place: full heads written to new buffers
            qo, ko = torch.empty_like(q), torch.empty_like(k)
            o_us = graph_timed(lambda: mr.apply(q, k, pl, q_out=qo, k_out=ko), args.steps) * 1e6
            out[cfg.name]["apply_out_of_place_us"] = o_us
            del qo, ko
        del q, k, pl
        torch.cuda.empty_cache()
    # fp16 I/O on the default batch shape (same bytes as bf16)
    cfg = synth.config2()
    log("extras: 64x4096 fp16")
    qn, kn = cfg.qk()
    q = torch.from_numpy(synth.to_f16_bits(synth.bf16_bits_to_f32(qn)).view(np.int16)).view(torch.float16).to(dev)
    k = torch.from_numpy(synth.to_f16_bits(synth.bf16_bits_to_f32(kn)).view(np.int16)).view(torch.float16).to(dev)
    ids = torch.from_numpy(cfg.ids).to(dev)
    cu = torch.from_numpy(cfg.cu_seqlens).to(dev)
    pl, *_ = mr.planes(ids, cu, synth.IMAGE_ID)
    a_us = timed(lambda: mr.apply(q, k, pl), args.steps) * 1e6
    out["64x4096-image-f16"] = {"tokens": cfg.n_tokens, "apply_us": a_us,
                                "apply_gbs": algorithmic_bytes_apply(cfg.n_tokens) / a_us / 1e3}
    del q, k, pl
    torch.cuda.empty_cache()

    # out of place on the default batch: full heads read and written (the rotated dims by the
    # rotation kernel, the rest by the copy launch)
    log("extras: 64x4096 bf16 out of place")
    qn, kn = cfg.qk()
    q, k = heads(qn, "bf16"), heads(kn, "bf16")
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    pl, *_ = mr.planes(ids, cu, synth.IMAGE_ID)
    ws = mr.Workspace(cfg.n_tokens, dev)
    oa_us = timed(lambda: mr.apply(q, k, pl, q_out=qo, k_out=ko), args.steps) * 1e6
    of_us = timed(lambda: mr.apply_ids(q, k, ids, cu, synth.IMAGE_ID, q_out=qo, k_out=ko, workspace=ws),
                  args.steps) * 1e6
    oop_bytes = cfg.n_tokens * (10 * 256 * 2 * 2 + 12)
    out["64x4096-image-bf16-out-of-place"] = {
        "tokens": cfg.n_tokens, "apply_us": oa_us, "fused_us": of_us, "apply_gbs": oop_bytes / oa_us / 1e3,
        "note": "10,252 B/token for apply (full Q/K heads read and written, planes read); the fused call "
                "reads 4 B of ids instead of 12 B of planes"}
    del q, k, qo, ko, pl
    torch.cuda.empty_cache()

    # chunked prefill: the 8 x 32,768 prompts fed as 4 pieces of 8,192 tokens per sequence, each piece
    # one fused call carrying pos_offset and the previous piece's origin (all pieces resident)
    cfg = synth.config3()
    log("extras: 8x32768 bf16 in 4 pieces")
    qn, kn = cfg.qk()
    q, k = heads(qn, "bf16"), heads(kn, "bf16")
    n_pc, L = 4, 32768
    piece = L // n_pc
    cu_p = torch.arange(0, 8 * piece + 1, piece, dtype=torch.int32, device=dev)
    rows = [torch.from_numpy(np.concatenate([np.arange(s * L + i * piece, s * L + (i + 1) * piece)
                                             for s in range(8)])).to(dev) for i in range(n_pc)]
    ids_all = torch.from_numpy(cfg.ids).to(dev)
    ids_p = [ids_all[r].contiguous() for r in rows]
    q_p = [q[r].contiguous() for r in rows]
    k_p = [k[r].contiguous() for r in rows]
    offs = [torch.full((8,), i * piece, dtype=torch.int32, device=dev) for i in range(n_pc)]
    origins = [torch.full((8,), -1, dtype=torch.int32, device=dev) for _ in range(n_pc + 1)]
    ws = mr.Workspace(8 * piece, dev)

    def pieces():
        for i in range(n_pc):
            mr.apply_ids(q_p[i], k_p[i], ids_p[i], cu_p, synth.IMAGE_ID, pos_offset=offs[i], origin_in=origins[i],
                         origin=origins[i + 1], workspace=ws)

    # GPU time from a replayed graph: a 65,536-token call is shorter than the binding's host time
    c_us = graph_timed(pieces, max(1, args.steps // n_pc)) * 1e6
    out["8x32768-image-bf16-in-4-pieces"] = {
        "tokens": cfg.n_tokens, "pieces": n_pc, "fused_us_all_pieces": c_us, "fused_us_per_piece": c_us / n_pc,
        "tokens_per_s": cfg.n_tokens / (c_us / 1e6),
        "gbs": algorithmic_bytes_fused(cfg.n_tokens) / c_us / 1e3, "timing": "hip graph replay",
        "note": "mrope_apply_ids per piece of 65,536 tokens with pos_offset and origin_in (chunked prefill)"}
    del q, k, q_p, k_p
    torch.cuda.empty_cache()

    # a longer frame (frame_len 75: a run of 9 marker tokens after </image>) on the default workload
    cfg = synth.config2()
    log("extras: 64x4096 bf16, frame_len 75")
    qn, kn = cfg.qk()
    q, k = heads(qn, "bf16"), heads(kn, "bf16")
    ids = torch.from_numpy(cfg.ids).to(dev)
    cu = torch.from_numpy(cfg.cu_seqlens).to(dev)
    ws = mr.Workspace(cfg.n_tokens, dev)
    f75, f67 = [], []
    for _ in range(3):  # interleaved, median of three
        f67.append(timed(lambda: mr.apply_ids(q, k, ids, cu, synth.IMAGE_ID, workspace=ws), args.steps) * 1e6)
        f75.append(timed(lambda: mr.apply_ids(q, k, ids, cu, synth.IMAGE_ID, frame_len=75, workspace=ws),
                         args.steps) * 1e6)
    f75, f67 = sorted(f75)[1], sorted(f67)[1]
    out["64x4096-image-bf16-frame-len-75"] = {"tokens": cfg.n_tokens, "fused_us": f75, "fused_us_frame_len_67": f67,
                                              "gbs": algorithmic_bytes_fused(cfg.n_tokens) / f75 / 1e3}
    del q, k
    torch.cuda.empty_cache()

    # prefill with the paged K/V cache write fused in (64 x 4096 bf16, V from the same seed stream)
    cfg = synth.config2()
    log("extras: 64x4096 bf16 with the K/V cache write")
    qn, kn = cfg.qk()
    q, k = heads(qn, "bf16"), heads(kn, "bf16")
    v = torch.randn(k.shape, device=dev).to(torch.bfloat16)
    ids = torch.from_numpy(cfg.ids).to(dev)
    cu = torch.from_numpy(cfg.cu_seqlens).to(dev)
    nb = (cfg.n_tokens + 15) // 16
    kc = torch.zeros((nb, 16, 2, 256), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    slots = torch.randperm(nb * 16, device=dev)[:cfg.n_tokens].to(torch.int64)
    ws = mr.Workspace(cfg.n_tokens, dev)
    kv_us = timed(lambda: mr.apply_ids_kv(q, k, v, ids, cu, kc, vc, slots, synth.IMAGE_ID, workspace=ws),
                  args.steps) * 1e6
    out["64x4096-image-bf16-kv-cache"] = {
        "tokens": cfg.n_tokens, "fused_kv_us": kv_us, "tokens_per_s": cfg.n_tokens / (kv_us / 1e6),
        "gbs": algorithmic_bytes_fused_kv(cfg.n_tokens) / kv_us / 1e3,
        "note": "mrope_apply_ids_kv: Q in place, K rotated and V copied into 16-token paged caches at a random "
                "slot permutation"}
    # the same with a serving engine's layout: each 16-token block of a sequence in a random cache block,
    # the tokens in order inside it (so a block's rows are written together)
    blocks = torch.randperm(nb, device=dev).to(torch.int64)
    t = torch.arange(cfg.n_tokens, device=dev, dtype=torch.int64)
    slots_b = blocks[t // 16] * 16 + t % 16
    kvb_us = timed(lambda: mr.apply_ids_kv(q, k, v, ids, cu, kc, vc, slots_b, synth.IMAGE_ID, workspace=ws),
                   args.steps) * 1e6
    out["64x4096-image-bf16-kv-cache-block-order"] = {
        "tokens": cfg.n_tokens, "fused_kv_us": kvb_us, "tokens_per_s": cfg.n_tokens / (kvb_us / 1e6),
        "gbs": algorithmic_bytes_fused_kv(cfg.n_tokens) / kvb_us / 1e3,
        "note": "as above, slots filling randomly placed 16-token blocks in token order"}
    del q, k, v, kc, vc
    torch.cuda.empty_cache()

    d = synth.config4()
    log(f"extras: {d.name}")
    qn, kn = d.qk()
    q, k = heads(qn, "bf16"), heads(kn, "bf16")
    cache = torch.zeros((d.num_blocks, d.block_size, d.n_k_heads, d.head_dim), dtype=torch.bfloat16, device=dev)
    pos, amount = torch.from_numpy(d.pos).to(dev), torch.from_numpy(d.amount).to(dev)
    slots = torch.from_numpy(d.slot_mapping).to(dev)
    d_us = graph_timed(lambda: mr.decode(q, k, pos, amount, cache, slots), args.steps) * 1e6
    dbytes = d.n_seqs * (8 * 64 * 2 * 2 + 2 * 256 * 2 * 2 + 4 + 4 + 8)
    out[d.name] = {"seqs": d.n_seqs, "decode_us": d_us, "tokens_per_s": d.n_seqs / (d_us / 1e6),
                   "gbs": dbytes / d_us / 1e3, "timing": "hip graph replay"}
    v = torch.randn(k.shape, device=dev).to(torch.bfloat16)
    vcache = torch.zeros_like(cache)
    dv_us = graph_timed(lambda: mr.decode(q, k, pos, amount, cache, slots, v=v, v_cache=vcache), args.steps) * 1e6
    dvbytes = dbytes + d.n_seqs * 2 * 256 * 2 * 2
    out[d.name + "-with-v"] = {"seqs": d.n_seqs, "decode_us": dv_us, "tokens_per_s": d.n_seqs / (dv_us / 1e6),
                               "gbs": dvbytes / dv_us / 1e3, "timing": "hip graph replay"}
    del v, vcache
    del q, k, cache
    torch.cuda.empty_cache()
    return out


def traffic_from_counters(kernel: str, launch_tokens: int):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    scaled by the copy-kernel calibration -- only if it was taken on the current kernel sources."""
    try:
        c = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha256") != kernel_source_hash() or c.get("tokens") != launch_tokens:
        return None
    k = c.get("kernels", {}).get(kernel)
    return int(k["hbm_bytes_per_launch"]) if k else None


def cpu_baseline(b, qn, kn, min_seconds: float = 10.0, max_passes: int = 8):
    """The oracle, as it stands, over the whole workload on this host's cores (single-threaded),
    repeated until at least `min_seconds` of work; tokens/s."""
    import numpy as np

    import oracle
    from canvas_rope_rotary_amd import synth

    passes = 0
    t0 = time.perf_counter()
    while True:
        pl, st, am, og = oracle.planes(b.ids, b.cu_seqlens, synth.IMAGE_ID)
        for x in (qn, kn):
            y = oracle.rotate(synth.bf16_bits_to_f32(x), pl)
            oracle.round_bf16(y)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or passes >= max_passes:
            break
    del np
    return {"value": passes * b.n_tokens / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole workload ({b.n_tokens} tokens, planes + Q/K rotation + bf16 rounding), "
                      f"{passes} pass(es), {el:.1f} s, one thread"}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Worker threads for the all-cores oracle timing: the CPUs this process may run on, at most 16
    (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline_threads(b, qn, kn, threads: int, min_seconds: float = 5.0, max_passes: int = 64):
    """The same oracle calls as cpu_baseline, run by `threads` host threads over disjoint groups of
    whole sequences (the oracle's C calls release the interpreter lock); tokens/s."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    from canvas_rope_rotary_amd import synth

    cu = b.cu_seqlens.astype(np.int64)
    # split the sequences into `threads` groups of about equal token counts
    cuts = np.searchsorted(cu, np.linspace(0, cu[-1], threads + 1)[1:-1])
    bounds = [0, *sorted(set(int(c) for c in cuts)), b.n_seqs]
    groups = [(s0, s1) for s0, s1 in zip(bounds[:-1], bounds[1:]) if s1 > s0]

    def work(g):
        s0, s1 = g
        t0, t1 = int(cu[s0]), int(cu[s1])
        pl, *_ = oracle.planes(b.ids[t0:t1], (cu[s0:s1 + 1] - t0).astype(np.int32), synth.IMAGE_ID)
        for x in (qn, kn):
            oracle.round_bf16(oracle.rotate(synth.bf16_bits_to_f32(x[t0:t1]), pl))

    passes = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(work, groups))
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or passes >= max_passes:
                break
    return {"value": passes * b.n_tokens / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu": host_cpu_model(),
            "sample": f"the whole workload ({b.n_tokens} tokens in {len(groups)} sequence groups), {passes} "
                      f"pass(es), {el:.1f} s, {threads} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first: the step time settles only after ~100 back-to-back launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cold", action="store_true", help="also time mrope_apply after a cache-clearing read sweep")
    ap.add_argument("--extras", action="store_true",
                    help="also time the other workloads: 8 x 32768 fused, 1M-token ragged, decode, L=110 fp32")
    ap.add_argument("--mode", choices=("bench", "copy"), default="bench",
                    help="copy: only a plain 1 GiB device copy, repeated (calibrates rocprofv3 HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (the method shards by "
              "sequence or head with no communication); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import canvas_rope_rotary_amd as mr
    from canvas_rope_rotary_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "copy":
        # plain copy of known size: every dispatch reads 1 GiB and writes 1 GiB
        src = torch.ones(1 << 29, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_dispatch": 1 << 30, "bytes_written_per_dispatch": 1 << 30,
                          "dispatches": args.steps}), flush=True)
        return
    mr._lib.load()

    b = synth.config2()
    log(f"workload {b.name}: {b.n_tokens} tokens, {b.n_seqs} sequences; generating inputs")
    qn, kn = b.qk()
    ids = torch.from_numpy(b.ids).to(dev)
    cu = torch.from_numpy(b.cu_seqlens).to(dev)
    q = torch.from_numpy(qn.view(np.int16)).view(torch.bfloat16).to(dev)
    k = torch.from_numpy(kn.view(np.int16)).view(torch.bfloat16).to(dev)
    L = b.n_tokens
    planes = torch.empty((3, L), dtype=torch.int32, device=dev)
    start = torch.empty(b.n_seqs, dtype=torch.int32, device=dev)
    amount = torch.empty_like(start)
    origin = torch.empty_like(start)
    flags = torch.empty_like(start)
    ws = mr.Workspace(L, dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        mr.apply_ids(q, k, ids, cu, synth.IMAGE_ID, start=start, amount=amount, origin=origin, seq_flags=flags,
                     workspace=ws)

    def timed(fn, reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    step_s = timed(step, args.steps)
    wall = time.perf_counter() - w0
    ms_step = step_s * 1e3

    # each kernel alone, `steps` back-to-back launches on the same stream (HIP events): the step's
    # kernel again, and the two-launch form (mrope_planes, then mrope_apply on its planes)
    fused_s = timed(step, args.steps)
    planes_us = timed(lambda: mr.planes(ids, cu, synth.IMAGE_ID, out=planes, start=start, amount=amount,
                                        origin=origin, seq_flags=flags, workspace=ws), args.steps) * 1e6
    apply_mean_s = timed(lambda: mr.apply(q, k, planes), args.steps)
    log(f"timed {args.steps} steps: {ms_step * 1e3:.1f} us/step (wall {wall * 1e6 / args.steps:.1f} us/step); "
        f"mrope_apply_ids {fused_s * 1e6:.1f} us, mrope_planes {planes_us:.1f} us, mrope_apply "
        f"{apply_mean_s * 1e6:.1f} us per launch")

    cold = None
    if args.cold:
        # one launch after streaming 1 GiB through the caches (read only, so no dirty lines are left
        # to write back): the HBM-only figure, without hits in the 256 MB memory-side cache
        sweep = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        ts, tf = [], []
        for _ in range(20):
            sweep.sum()
            torch.cuda.synchronize()
            ts.append(timed(lambda: mr.apply(q, k, planes), 1))
            sweep.sum()
            torch.cuda.synchronize()
            tf.append(timed(step, 1))
        cold = (sorted(ts), sorted(tf))
        del sweep

    # plain device-to-device copy of 1 GiB: the practical streaming ceiling on this machine (context)
    src = torch.empty(1 << 29, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    copy_gbs = 2 * src.numel() * 2 / timed(lambda: dst.copy_(src), 10) / 1e9
    del src, dst

    fb = algorithmic_bytes_fused(L)
    achieved = fb / fused_s / 1e9
    ab = algorithmic_bytes_apply(L)
    a_achieved = ab / apply_mean_s / 1e9
    out = {
        "metric": METRIC,
        "value": L / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "io_dtype": "bf16",
        "angle_dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "64 image prompts x 4096 tokens, bf16: planes from int32 ids + in-place "
                               "rotary of Q[262144,8,256] and K[262144,2,256], one launch",
                   "tokens": L, "seqs": b.n_seqs, "q_heads": 8, "k_heads": 2, "head_dim": 256, "rot_dim": 64,
                   "theta": 1e7, "sections": [11, 11, 10]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_counters("mrope_apply_ids", L),
                     "kernel": "mrope_apply_ids", "algorithmic_bytes_per_launch": fb,
                     "mean_launch_us": fused_s * 1e6},
        "apply_roofline": {"bound": "hbm", "achieved": a_achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": a_achieved / HBM_PEAK_GBS, "traffic": traffic_from_counters("mrope_apply", L),
                           "kernel": "mrope_apply", "algorithmic_bytes_per_launch": ab,
                           "mean_launch_us": apply_mean_s * 1e6},
        "kernels_us": {"mrope_apply_ids": fused_s * 1e6, "mrope_planes": planes_us, "mrope_apply": apply_mean_s * 1e6},
        "two_launch_tokens_per_s": L / (planes_us / 1e6 + apply_mean_s),
        "planes_gbs": algorithmic_bytes_planes(L) / (planes_us / 1e6) / 1e9,
        # torch's own 1 GiB device copy, for context (not a ceiling: hand-written copies with
        # non-temporal loads and stores run faster on the same chip)
        "torch_copy_gbs": copy_gbs,
    }
    if cold is not None:
        pct = lambda v, q: v[min(len(v) - 1, int(round(q * (len(v) - 1))))]
        ma, mf = pct(cold[0], 0.5), pct(cold[1], 0.5)
        out["cold"] = {"mrope_apply_us": ma * 1e6, "mrope_apply_gbs": ab / ma / 1e9,
                       "mrope_apply_ids_us": mf * 1e6, "mrope_apply_ids_gbs": fb / mf / 1e9,
                       "mrope_apply_us_p10_p50_p90": [pct(cold[0], q) * 1e6 for q in (0.1, 0.5, 0.9)],
                       "mrope_apply_ids_us_p10_p50_p90": [pct(cold[1], q) * 1e6 for q in (0.1, 0.5, 0.9)],
                       "reps": len(cold[0]),
                       "note": "single launches, each after a 1 GiB read sweep (no memory-side cache hits)"}
    if args.extras:
        out["extras"] = extras(args, dev, timed)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(b, qn, kn, min_seconds=args.cpu_seconds)
        out["cpu_baseline"]["cpu"] = host_cpu_model()
        nt = cpu_threads()
        if nt > 1:
            log(f"cpu baseline (oracle, {nt} threads)")
            out["cpu_baseline_all_cores"] = cpu_baseline_threads(b, qn, kn, nt)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
