#!/usr/bin/env python3
"""Decode benchmark of the OSCAR INT2-history path on one MI355X.

Workload: Qwen3-8B-shaped batch-1 decode at 100,000 tokens of context -- 36 layers, 32 query
heads and 8 KV heads of dimension 128, 64 BF16 sink + 99,680 INT2 history + 256 BF16 recent
tokens per layer, history in 64-token pages placed through a seeded shuffled page table, keys
and values N(0,1) bf16 with one outlier channel (x16) per layer, head and tensor, U from the QR
of a seeded Gaussian, clip 4.0, group 128.  Inputs are synthetic (no model weights).

One step = oscar_decode_step for each of the 36 layers: write the new token into the BF16 recent
window, demote the displaced token into the INT2 history and rotate the query (one launch), the
INT2 split-KV pass with the BF16 sink/recent pass (one launch), merge and un-rotation (one
launch).  The 36-layer step is captured once in a HIP graph and replayed; 36 distinct layer
pools (2.1 GB) are cycled, so the 256 MB Infinity Cache cannot hold the timed data.

Prints one JSON line: value = effective HBM GB/s of the whole decode step (algorithmic bytes of
all 36 layers / step time); decode_steps_per_s; roofline of the segment-pass kernel (the
dominant one) timed with events on its stream; cpu_baseline = the CPU oracle timed on one KV
head of one layer and scaled; bf16_baseline = the same decode step over a cache that keeps every
token in BF16 pages (the comparison the pages' speedup figures are stated against), with the
INT2 / BF16 step-time ratio.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import bit_rotated_kv_decode_amd as ok  # noqa: E402
import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "decode-attn effective HBM GB/s (% of 8 TB/s peak) + decode steps/s, 100k ctx"


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_8b_100k")
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of a graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the memory probes (plain stream read, INT2-page gather)")
    ap.add_argument("--probe", action="store_true",
                    help="only build the layer pools and run the memory probes, then exit")
    ap.add_argument("--no-bf16-baseline", action="store_true",
                    help="skip the all-BF16 paged cache leg (the comparison the pages quote)")
    ap.add_argument("--levels", default=None, metavar="LO,STEP",
                    help="demote with an equally spaced codebook (lo, step) on every KV head, "
                         "keys and values (default: the plain grid)")
    ap.add_argument("--codebook", default=None, metavar="L0,L1",
                    help="demote with the symmetric codebook (l0, l1, 3 - l1, 3 - l0) on every "
                         "KV head, keys and values, and attend with its levels")
    ap.add_argument("--cascade", action="store_true",
                    help="with a shared prefix, time the shared-prefix cascade step "
                         "(oscar_decode_step_prefix) as the step, the plain step beside it")
    ap.add_argument("--no-cascade", action="store_true",
                    help="with a shared prefix, time the plain step alone (by default the cascade "
                         "step is timed beside it)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times "
                         "(calibration of the HBM byte counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    n = mib << 20
    src = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_kernel_qwen3_8b_100k_hbm_traffic.md")


def recorded_traffic(workload: str):
    """HBM bytes per segment-kernel launch recorded from the FETCH_SIZE / WRITE_SIZE counters for
    ``workload``, or None when they were taken on another workload or the kernel sources changed
    since (their sha256 is stored with the figure)."""
    try:
        fields = {}
        for line in open(TRAFFIC_FILE):
            key, _, val = line.strip().partition(": ")
            fields[key] = val
        if fields["workload"] != workload:
            return None
        h = hashlib.sha256()
        for f in fields["sources"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != fields["source_sha256"]:
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def bytes_per_token_head(group: int) -> int:
    return 2 * 128 // 4 + 2 * (128 // group) * 4


class Layer:
    """One layer's resident cache and per-step inputs for the workload's sequences.  History
    pages inside a shared prefix are built once (from the longest sequence) and aliased by the
    page table; every other page is private."""

    def __init__(self, wl, layer, lengths, spare, levels=None, levels_kind=0):
        dev = "cuda"
        self.lengths = list(lengths)
        B = len(self.lengths)
        hkv = wl.num_kv_heads
        self.table_np, self.num_pages = workloads.page_tables(wl, self.lengths, layer,
                                                              spare_tokens=spare)
        self.lay = ok.make_layout(wl.num_q_heads, hkv, self.num_pages, B,
                                  self.table_np.shape[1], wl.group_size,
                                  levels_kind=levels_kind)
        self.cache = ok.Cache.allocate(self.lay, zero=False)
        self.table = torch.from_numpy(self.table_np).to(dev)
        # a calibrated U (computed offline from query statistics on the CPU) changes code
        # values, not the work: such a workload is timed with seeded orthogonal bases
        uk, uv = workloads.rotation_bases(
            workloads.scaled(wl, rotation="qr") if wl.rotation == "calibrated" else wl, layer)
        self.u_k, self.u_v = uk.to(dev).contiguous(), uv.to(dev).contiguous()
        # the clip threshold changes code values, not the work; a workload without a fixed one
        # (calibrated offline) is timed with 4.0
        clip = wl.clip if wl.clip is not None else 4.0
        self.clip_k = torch.full((hkv,), clip, dtype=torch.float32, device=dev)
        self.clip_v = self.clip_k.clone()
        self.levels = None if levels is None else torch.tensor(
            [levels] * hkv, dtype=torch.float32, device=dev)
        n_hist = [max(0, L - 320) for L in self.lengths]
        longest = int(np.argmax(self.lengths))
        chunk = 16384
        for b in range(B):
            # pages of the shared prefix are built once, from the longest sequence; a sequence
            # still inside the prefix has private copies from the page its next write falls in
            lo0 = 0 if b == longest else 64 * workloads.shared_pages(wl, self.lengths[b], spare)
            for lo in range(lo0, n_hist[b], chunk):
                n = min(chunk, n_hist[b] - lo)
                k, v = workloads.kv_tokens(wl, layer, b, 64 + lo, n, dev)
                ok.demote(self.lay, self.cache.pool, self.table[b:b + 1], self.u_k, self.u_v,
                          self.clip_k, self.clip_v, k.unsqueeze(0), v.unsqueeze(0),
                          torch.full((1,), lo, dtype=torch.int32, device=dev),
                          levels_k=self.levels, levels_v=self.levels)
            L = self.lengths[b]
            k, v = workloads.kv_tokens(wl, layer, b, 0, min(L, 64), dev)
            self.cache.sink_k[b, :, :k.shape[0]] = k.transpose(0, 1)
            self.cache.sink_v[b, :, :k.shape[0]] = v.transpose(0, 1)
            if L > 64:
                pos = torch.arange(max(64, L - 256), L, device=dev)
                k, v = workloads.kv_tokens(wl, layer, b, int(pos[0]), len(pos), dev)
                self.cache.recent_k[b][:, pos % 256] = k.transpose(0, 1)
                self.cache.recent_v[b][:, pos % 256] = v.transpose(0, 1)
        # per-step inputs (the same new token and query every step)
        kn, vn = zip(*[workloads.kv_tokens(wl, layer, b, L, 1, dev)
                       for b, L in enumerate(self.lengths)])
        self.k_new = torch.cat(kn).contiguous()
        self.v_new = torch.cat(vn).contiguous()
        self.q = workloads.queries(wl, layer, 0, dev, batch=B).contiguous()
        self.out = torch.empty((B, wl.num_q_heads, 128), dtype=torch.float32, device=dev)
        # the shared prefix as the cascade takes it: the prefix's page ids and, per sequence, how
        # many leading pages of its row are those
        ids, shared = workloads.shared_prefix(wl, self.table_np, self.lengths, spare)
        ok.check_shared_prefix(self.lay, self.table_np, ids, shared)
        self.prefix_ids = torch.from_numpy(ids).to(dev)
        self.shared_pages = torch.from_numpy(shared).to(dev)


def distribution(xs, digits):
    """Median, 10th and 90th percentile of a list of timings."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), digits),
            "p10": round(float(np.percentile(a, 10)), digits),
            "p90": round(float(np.percentile(a, 90)), digits), "n": int(a.size)}


def timed_graph(fn, reps, per):
    """Capture fn() (``per`` launches) in a HIP graph, replay it ``reps`` times with HIP events
    around each replay on the launch stream; per-launch microseconds of every replay."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    us = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3 / per)
    return us


def probes(wl, layers, steps):
    """Practical HBM ceilings measured in the same run: a plain streaming read of 2 GiB, a plain
    streaming read of one attention launch's INT2 history bytes per launch (36 launches over
    distinct slices, as the attention kernel cycles its layer pools), and the INT2 pages read
    through the page table in the attention kernel's grid order with 2 and 4 pages in flight per
    wave (no arithmetic)."""
    dev = "cuda"
    reps = max(5, min(steps, 20))
    big = 2 << 30
    buf = torch.ones(big, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    us = timed_graph(lambda: ok.probe_read(buf, sink, 2048), reps, 1)
    out = {"stream_read_2GiB": {"GB/s": round(big / (float(np.median(us)) * 1e-6) / 1e9, 1),
                                "us": distribution(us, 2),
                                "kernel": "probe_read_kernel (16-byte non-temporal loads, 2048 "
                                          "workgroups)"}}
    lr0 = layers[0]
    n_pages = [workloads.history_pages(L + 1) for L in lr0.lengths]
    hist = ok.pool_bytes(lr0.lay) // max(1, lr0.num_pages) * sum(n_pages)
    hist = hist // 256 * 256
    n_slices = len(layers)
    if hist * n_slices <= big:
        slices = [buf[i * hist:(i + 1) * hist] for i in range(n_slices)]
        us = timed_graph(lambda: [ok.probe_read(x, sink, 2048) for x in slices], reps, n_slices)
        out["stream_read_int2_launch_bytes"] = {
            "bytes": int(hist), "GB/s": round(hist / (float(np.mean(us)) * 1e-6) / 1e9, 1),
            "us": distribution(us, 2),
            "note": f"{n_slices} launches over distinct slices, per-launch mean"}
    del buf
    if len(lr0.lengths) == 1:
        splits, pps = ok.decode_splits(lr0.lay, 1, lr0.lengths[0] + 1)
        blocks = 4 * splits * wl.num_kv_heads
        # the attention kernel's own access pattern (two register sets of page pairs per wave),
        # bare and with per-pair arithmetic on the waves' paths, then with deeper prefetch
        for sets, work in ((2, 0), (2, 200), (2, 400), (4, 0), (4, 400)):
            us = timed_graph(lambda: [ok.probe_gather(Lr.lay, Lr.cache.pool, Lr.table[0],
                                                      n_pages[0], pps, sets, sink, work)
                                      for Lr in layers], reps, len(layers))
            out[f"int2_page_gather_sets{sets}_work{work}"] = {
                "bytes": int(hist), "GB/s": round(hist / (float(np.mean(us)) * 1e-6) / 1e9, 1),
                "us": distribution(us, 2),
                "note": f"{splits} splits x {wl.num_kv_heads} KV heads of {pps} pages, "
                        f"{blocks} waves, {sets} register sets of page pairs per wave, {work} "
                        f"fp32 FMAs per lane per pair, {len(layers)} layer pools"}
    return out


def history_bytes(wl, lengths, table=None):
    """Cache bytes one attention pass reads for sequences of the given lengths: INT2 history
    (codes + meta), its page-table entries, and the BF16 sink + recent rows.  With the page
    table, a history page shared by several sequences counts once (unique bytes)."""
    hkv = wl.num_kv_heads
    bpt = bytes_per_token_head(wl.group_size)
    total = 0
    page_tokens = {}
    for b, L in enumerate(lengths):
        n_hist = max(0, L - 320)
        n_bf16 = min(L, 64) + min(256, max(0, L - 64))
        total += math.ceil(n_hist / 64) * 4 + hkv * n_bf16 * 128 * 2 * 2
        if table is None:
            total += hkv * n_hist * bpt
        else:
            for p_ in range(math.ceil(n_hist / 64)):
                pid = int(table[b, p_])
                page_tokens[pid] = max(page_tokens.get(pid, 0), min(64, n_hist - 64 * p_))
    return total + hkv * bpt * sum(page_tokens.values())


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (each GPU box here "
              "has one GPU, and this path needs no collectives).", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_mb:
        copy_calibration(args.copy_mb)
        return
    ok.lib()
    wl = workloads.get(args.workload)
    n_layers = args.layers or wl.num_layers
    lengths = workloads.context_lengths(wl)
    B = len(lengths)
    # with a shared prefix both steps are timed (unless --no-cascade): the plain one as the
    # step, or the cascade one with --cascade, and the other beside it
    both = bool(wl.shared_prefix) and not args.no_cascade
    cascade = both and args.cascade
    total_steps = args.warmup + args.steps + 2       # +2: graph capture warm-up and capture
    if both:
        total_steps *= 2                             # the other step is timed after it
    dev = "cuda"

    t0 = time.time()
    if args.levels is not None and args.codebook is not None:
        raise SystemExit("--levels and --codebook exclude each other")
    spec = args.codebook if args.codebook is not None else args.levels
    levels = None if spec is None else tuple(float(x) for x in spec.split(","))
    kind = ok.LEVELS_SYMMETRIC if args.codebook is not None else ok.LEVELS_SPACED
    layers = [Layer(wl, i, lengths, total_steps + 8, levels, kind) for i in range(n_layers)]
    torch.cuda.synchronize()
    setup_s = time.time() - t0
    print(f"[bench] built {n_layers} layer pools in {setup_s:.1f}s", file=sys.stderr, flush=True)
    if args.probe:
        print(json.dumps({"workload": wl.name, "probes": probes(wl, layers, args.steps)}),
              flush=True)
        return

    # position of each sequence's new token
    pos = torch.tensor(lengths, dtype=torch.int32, device=dev)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    max_len = max(lengths) + total_steps + 4
    n_prefix = layers[0].prefix_ids.numel() if both else 0
    ws = torch.zeros(ok.decode_workspace_bytes_prefix(layers[0].lay, B, max_len, n_prefix),
                     dtype=torch.uint8, device=dev)

    def plain_step():
        for Lr in layers:
            c = Lr.cache
            ok.decode_step(Lr.lay, c.pool, Lr.table, c.sink_k, c.sink_v, c.recent_k, c.recent_v,
                           Lr.u_k, Lr.u_v, Lr.clip_k, Lr.clip_v, Lr.k_new, Lr.v_new, slots, pos,
                           Lr.q, Lr.out, ws, max_len, levels_k=Lr.levels, levels_v=Lr.levels)
        pos.add_(1)

    def cascade_step():
        for Lr in layers:
            c = Lr.cache
            ok.decode_step_prefix(Lr.lay, c.pool, Lr.table, c.sink_k, c.sink_v, c.recent_k,
                                  c.recent_v, Lr.u_k, Lr.u_v, Lr.clip_k, Lr.clip_v, Lr.k_new,
                                  Lr.v_new, slots, pos, Lr.q, Lr.prefix_ids, Lr.shared_pages,
                                  Lr.out, ws, max_len)
        pos.add_(1)

    step, other_step = (cascade_step, plain_step) if cascade else (plain_step, cascade_step)

    def capture(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()                                      # warm-up outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    def time_steps(fn):
        """Warm-up, then args.steps whole decode steps (HIP events around each step on the launch
        stream for the distribution; the wall clock between two synchronisations for the mean).
        Returns (ms per step, per-step ms, steps run before the timed ones, graph or None)."""
        graph = None if args.no_graph else capture(fn)
        if graph is None:
            fn()
            fn()

        def run_step():
            if graph is not None:
                graph.replay()
            else:
                fn()

        for _ in range(args.warmup):
            run_step()
        torch.cuda.synchronize()
        before = int(pos[0].item()) - lengths[0]
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t_start = time.perf_counter()
        for e_a, e_b in evs:
            e_a.record()
            run_step()
            e_b.record()
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        return ((t_end - t_start) * 1e3 / args.steps, [a.elapsed_time(b) for a, b in evs],
                before, graph)

    # ---- timed region 1: whole decode steps
    ms_per_step, step_ms, steps_before, graph = time_steps(step)
    if both:
        # the same steps the other way, timed right after on the same pools
        other_ms, other_step_ms, _, other_graph = time_steps(other_step)
        del other_graph

    # ---- timed region 2: the segment-pass kernel (INT2 history + BF16 sink / recent blocks in
    # one launch) exactly as a step launches it -- on the fp8 pass without codebooks or a cascade
    # the launch also appends the token and rotates the query (oscar_decode_step_stages) -- once
    # per layer pool: a graph of n_layers launches (the pools repeated in turn up to at least 8
    # launches, so that one graph launch's overhead is spread) replayed args.steps times, HIP
    # events around each replay on the launch stream.  Each layer gets its own workspace.  The
    # repeated launches append again each time (the caches are not read after this).  Then the
    # same for the segment launch of oscar_decode_attn, which takes an already rotated query.
    lens = pos + 1
    seg = ok.STAGE_INT2 | ok.STAGE_BF16
    wss = [torch.zeros_like(ws) for _ in layers]

    def attn(i, stages):
        Lr = layers[i]
        c = Lr.cache
        a = (Lr.lay, c.pool, Lr.table, c.sink_k, c.sink_v, c.recent_k, c.recent_v, slots, lens,
             Lr.q, Lr.u_k, Lr.u_v, Lr.out, wss[i], max_len)
        if cascade:
            ok.decode_attn_prefix(*a[:12], Lr.prefix_ids, Lr.shared_pages, *a[12:],
                                  stages=stages)
        elif Lr.lay.levels_kind == ok.LEVELS_SYMMETRIC:
            ok.decode_attn_codebook(*a[:12], Lr.levels, Lr.levels, *a[12:], stages=stages)
        else:
            ok.decode_attn(*a, stages=stages)

    def step_part(i, stages):
        Lr = layers[i]
        c = Lr.cache
        ok.decode_step(Lr.lay, c.pool, Lr.table, c.sink_k, c.sink_v, c.recent_k, c.recent_v,
                       Lr.u_k, Lr.u_v, Lr.clip_k, Lr.clip_v, Lr.k_new, Lr.v_new, slots, pos,
                       Lr.q, Lr.out, wss[i], max_len, levels_k=Lr.levels, levels_v=Lr.levels,
                       stages=stages)

    seg_reps = -(-8 // len(layers))

    def time_launches(launch):
        def launches():
            for _ in range(seg_reps):
                for i in range(len(layers)):
                    launch(i, seg)

        g_seg = capture(launches)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        us = []
        for _ in range(args.steps):
            e0.record()
            g_seg.replay()
            e1.record()
            torch.cuda.synchronize()
            us.append(e0.elapsed_time(e1) * 1e3 / (seg_reps * len(layers)))
        return us

    # the step's own segment launch (the cascade step's is oscar_decode_attn_prefix's)
    seg_launch = attn if cascade else step_part
    for i in range(len(layers)):
        seg_launch(i, ok.STAGE_QUERY)
    seg_us = time_launches(seg_launch)
    attn_us = None
    if not cascade:
        for i in range(len(layers)):
            attn(i, ok.STAGE_QUERY)
        attn_us = time_launches(attn)

    # algorithmic bytes of the timed steps: attention (as the segment launch counts them, plus
    # the bf16 query in and the fp32 output) and the append (new K/V rows in, the displaced row
    # read and its codes written)
    hkv, hq = wl.num_kv_heads, wl.num_q_heads
    bpt = bytes_per_token_head(wl.group_size)
    att_bytes = 0
    for s_ in range(args.steps):
        seen = [L + steps_before + s_ + 1 for L in lengths]   # lengths seen by attention
        att = history_bytes(wl, seen, layers[0].table_np) + B * hq * 128 * (2 + 4)
        append = B * (hkv * 128 * 2 * 2 * 3 + hkv * bpt)
        att_bytes += n_layers * (att + append)
    seg_lengths = [int(x) for x in lens.tolist()]
    # the segment launch of oscar_decode_attn also reads the rotated query operand (INT2 blocks)
    # and the bf16 query; pages shared by several sequences count once (logical bytes reported
    # alongside).  The step's own segment launch, when it prepares the step itself, reads the
    # bf16 query, U_k and U_v (once per KV head) and does the append's reads and writes instead
    # of reading a rotated query.
    fused = not cascade and ok.decode_step_launches(layers[0].lay, B, max_len) == 2
    attn_extra = B * hq * (256 + 128 * 2)
    step_extra = (B * hq * 128 * 2 + 2 * hkv * 128 * 128 * 4 +
                  B * (hkv * 128 * 2 * 2 * 3 + hkv * bpt))
    attn_bytes = history_bytes(wl, seg_lengths, layers[0].table_np) + attn_extra
    seg_bytes = attn_bytes - attn_extra + (step_extra if fused else attn_extra)
    seg_logical = history_bytes(wl, seg_lengths) + (step_extra if fused else attn_extra)
    step_bytes = att_bytes / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    seg_us_avg = float(np.mean(seg_us))
    achieved = seg_bytes / (seg_us_avg * 1e-6) / 1e9
    # what the step's segment launch reads besides: the step's preparation (U_k, the new rows,
    # and for a demotion the displaced rows and U_v) -- L2-resident after the first block, so
    # not counted in the algorithmic bytes above

    ctx = (f"context {lengths[0]}" if len(set(lengths)) == 1 else
           f"contexts {min(lengths)}..{max(lengths)}")
    shape = {"qwen3_8b_100k": "Qwen3-8B-shaped decode, batch 1",
             "qwen3_8b_100k_kv1": "one GPU's share (1 of 8 KV heads, tensor-parallel) of "
                                  "Qwen3-8B-shaped decode, batch 1",
             "qwen3_4b_32k": "Qwen3-4B-shaped decode, batch 1 (seeded orthogonal U in place of "
                             "the calibrated one)",
             "tiny_gqa4_1k": "tiny single-layer decode, batch 1",
             "qwen3_32b_131k": "Qwen3-32B-shaped decode, batch 16",
             "qwen3_8b_b64_prefix": "Qwen3-8B-shaped decode, batch 64 with a 32768-token shared "
                                    "prefix"}.get(wl.name, f"decode, batch {B}")
    result = {
        "metric": METRIC if wl.name == "qwen3_8b_100k" else
        f"decode-attn effective HBM GB/s (% of 8 TB/s peak) + decode steps/s, {wl.name}",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: {shape}, {ctx}, "
                               f"{n_layers} layers, Hq {hq}, Hkv {hkv}, head_dim 128, "
                               f"group {wl.group_size}, 64-token shuffled pages",
                   "batch": B, "context": lengths[0] if len(set(lengths)) == 1 else
                   [min(lengths), max(lengths)], "layers": n_layers,
                   "launch": "hip-graph" if graph is not None else "eager",
                   "step_launches": 3 if cascade else ok.decode_step_launches(layers[0].lay, B,
                                                                               max_len),
                   **({} if not levels else
                      {"codebook": {"symmetric_l0_l1": list(levels)}} if kind else
                      {"codebook": {"lo": levels[0], "step": levels[1]}})},
        "decode_steps_per_s": round(1e3 / ms_per_step, 2),
        "step_ms": distribution(step_ms, 4),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step_bytes": int(step_bytes),
        "roofline": {"kernel": ("cascade_kernel + attn_kernel (shared-prefix chunks staged in LDS "
                               "per group of 16 sequences, then the INT2 split-KV items of the "
                               "other pages + BF16 sink/recent blocks; two launches timed as one)"
                               if cascade else
                               "attn_kernel (INT2 split-KV history + BF16 sink/recent blocks)"),
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(wl.name),
                     "bytes_per_launch": int(seg_bytes),
                     **({"logical_bytes_per_launch": int(seg_logical)}
                        if seg_logical != seg_bytes else {}),
                     "avg_launch_us": round(seg_us_avg, 3),
                     "launch_us": distribution(seg_us, 3),
                     "timing": f"HIP events around {args.steps} replays of a graph of "
                               f"{seg_reps * n_layers} launches ({seg_reps} per layer pool), "
                               f"per-launch mean"},
    }
    if fused:
        result["roofline"]["kernel"] = (
            "attn_kernel of the decode step (INT2 split-KV history + BF16 sink/recent blocks; "
            "the INT2 blocks rotate the query, one BF16 block per KV head demotes the displaced "
            "token)")
    if attn_us is not None:
        a_us = float(np.mean(attn_us))
        result["attention_only"] = {
            "kernel": "attn_kernel as oscar_decode_attn launches it (query rotated beforehand)",
            "avg_launch_us": round(a_us, 3), "launch_us": distribution(attn_us, 3),
            "bytes_per_launch": int(attn_bytes),
            "achieved": round(attn_bytes / (a_us * 1e-6) / 1e9, 1),
            "frac": round(attn_bytes / (a_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if both:
        casc_ms, plain_ms = (ms_per_step, other_ms) if cascade else (other_ms, ms_per_step)
        result["cascade"] = {
            "prefix_pages": n_prefix,
            "chunks": n_prefix // 12,
            "timed_as_step": "cascade" if cascade else "plain",
            "cascade_ms_per_step": round(casc_ms, 4),
            "plain_ms_per_step": round(plain_ms, 4),
            "other_step_ms": distribution(other_step_ms, 4),
            "cascade_speedup_vs_plain": round(plain_ms / casc_ms, 3),
            "note": "the same decode steps on the same pools, the other way (oscar_decode_step: "
                    "split-KV items read every page of every sequence; oscar_decode_step_prefix: "
                    "cascade blocks take the shared chunks), timed right after the step"}
    if not args.no_probes:
        result["probes"] = probes(wl, layers, args.steps)
    if not args.no_bf16_baseline:
        int2_layer_bytes = ok.pool_bytes(layers[0].lay) + 2 * (ok.sink_bytes(layers[0].lay) +
                                                               ok.recent_bytes(layers[0].lay))
        result["bf16_baseline"] = bf16_baseline(wl, lengths, n_layers, args, capture, ms_per_step,
                                                int2_layer_bytes)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, layers[0], lengths[0], B)
    print(json.dumps(result), flush=True)


BF16_POOL_BUDGET = 64e9   # bytes of BF16 layer pools a run may hold


def bf16_baseline(wl, lengths, n_layers, args, capture, int2_ms_per_step, int2_layer_bytes):
    """The same decode step over an all-BF16 paged cache: per layer, store the new token
    (oscar_bf16_store) and attend over every cached token (oscar_bf16_decode_attn: split-KV
    kernel + merge), all layers in one HIP graph.  Layers cycle over distinct pools that together
    exceed the Infinity Cache (every layer has its own pool when they fit BF16_POOL_BUDGET)."""
    dev = "cuda"
    B = len(lengths)
    total_steps = args.warmup + args.steps + 2
    spare = total_steps + 8
    hkv, hq = wl.num_kv_heads, wl.num_q_heads
    table_np, num_pages = workloads.page_tables(wl, lengths, 0, spare_tokens=spare, sink=0,
                                                recent=0)
    lay = ok.make_layout(hq, hkv, num_pages, B, table_np.shape[1], wl.group_size)
    layer_bytes = ok.bf16_pool_bytes(lay)
    n_pools = max(1, min(n_layers, int(BF16_POOL_BUDGET // layer_bytes)))
    pools = []
    t0 = time.time()
    longest = int(np.argmax(lengths))
    for i in range(n_pools):
        t_np, _ = workloads.page_tables(wl, lengths, i, spare_tokens=spare, sink=0, recent=0)
        table = torch.from_numpy(t_np).to(dev)
        pool = torch.empty(layer_bytes, dtype=torch.uint8, device=dev)
        for b, L in enumerate(lengths):
            lo0 = 0 if b == longest else 64 * workloads.shared_pages(wl, L, spare, sink=0,
                                                                     recent=0)
            for lo in range(lo0, L, 16384):
                n = min(16384, L - lo)
                k, v = workloads.kv_tokens(wl, i, b, lo, n, dev)
                ok.bf16_store(lay, pool, table[b:b + 1], k.unsqueeze(0), v.unsqueeze(0),
                              torch.full((1,), lo, dtype=torch.int32, device=dev))
        kn, vn = zip(*[workloads.kv_tokens(wl, i, b, L, 1, dev) for b, L in enumerate(lengths)])
        pools.append(dict(table=table, pool=pool,
                          k_new=torch.cat(kn).unsqueeze(1).contiguous(),
                          v_new=torch.cat(vn).unsqueeze(1).contiguous(),
                          q=workloads.queries(wl, i, 0, dev, batch=B).contiguous(),
                          out=torch.empty((B, hq, 128), dtype=torch.float32, device=dev)))
    torch.cuda.synchronize()
    print(f"[bench] built {n_pools} BF16 layer pools ({layer_bytes / 1e9:.2f} GB each) in "
          f"{time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    pos = torch.tensor(lengths, dtype=torch.int32, device=dev)
    lens = pos + 1
    max_len = max(lengths) + total_steps + 4
    ws = torch.empty(ok.bf16_decode_workspace_bytes(lay, B, max_len), dtype=torch.uint8,
                     device=dev)

    def step():
        for i in range(n_layers):
            P = pools[i % n_pools]
            ok.bf16_store(lay, P["pool"], P["table"], P["k_new"], P["v_new"], pos)
            ok.bf16_decode_attn(lay, P["pool"], P["table"], lens, P["q"], P["out"], ws, max_len)
        pos.add_(1)
        lens.add_(1)

    graph = capture(step)
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t_start) * 1e3 / args.steps

    # attention alone (split-KV kernel + merge), one launch pair per layer, as in a step
    wss = [torch.empty_like(ws) for _ in range(n_layers)]

    def attn_launches():
        for i in range(n_layers):
            P = pools[i % n_pools]
            ok.bf16_decode_attn(lay, P["pool"], P["table"], lens, P["q"], P["out"], wss[i],
                                max_len)

    g2 = capture(attn_launches)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    us = []
    for _ in range(args.steps):
        e0.record()
        g2.replay()
        e1.record()
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3 / n_layers)
    seen = [int(x) for x in lens.tolist()]
    # algorithmic bytes per attention launch: K and V rows (512 B per token and KV head, pages
    # shared by several sequences once), page-table entries, the bf16 query and fp32 output
    page_tokens = {}
    for b, L in enumerate(seen):
        for p_ in range(math.ceil(L / 64)):
            pid = int(table_np[b, p_])
            page_tokens[pid] = max(page_tokens.get(pid, 0), min(64, L - 64 * p_))
    att_bytes = (hkv * 512 * sum(page_tokens.values()) +
                 4 * sum(math.ceil(L / 64) for L in seen) + B * hq * 128 * (2 + 4))
    us_avg = float(np.mean(us))
    achieved = att_bytes / (us_avg * 1e-6) / 1e9
    return {"decode_steps_per_s": round(1e3 / ms, 2), "ms_per_step": round(ms, 4),
            "int2_speedup": round(ms / int2_ms_per_step, 3),
            "kernel": "bf16_attn_kernel + bf16_merge_kernel (split-KV over BF16 pages)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "bytes_per_launch": int(att_bytes),
            "avg_launch_us": round(us_avg, 3),
            "kv_bytes_per_layer": {"int2_pool_plus_bf16_segments": int(int2_layer_bytes),
                                   "bf16_pool": int(layer_bytes)},
            "pools": n_pools,
            "timing": f"step: graph of {n_layers} x (bf16_store + bf16_decode_attn) replayed "
                      f"{args.steps} times; attention: HIP events around {args.steps} replays "
                      f"of a graph of {n_layers} bf16_decode_attn calls, per-call mean"}


def host_facts():
    """The host the CPU baseline runs on: model name, logical CPUs, CPUs this process may run
    on, and the BLAS thread pool numpy uses."""
    import threadpoolctl
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0)),
            "blas_threads": blas[0]["num_threads"] if blas else None,
            "blas": blas[0].get("internal_api") if blas else None}


def cpu_baseline(wl, layer0, length, batch):
    """Time the CPU oracle (numpy, fp64) on one KV head of sequence 0 of one layer at full
    context -- demotion of one token and decode attention over the three-segment cache for the
    head's query heads -- with numpy's BLAS pool on every core this process may use; median of
    three runs, scaled to the whole step (every KV head, sequence and layer)."""
    import threadpoolctl

    import oracle

    def bf16_np(t):
        return t.float().cpu().numpy()

    kv = 0
    geom = oracle.Geometry(group=wl.group_size)
    n_hist = length - 320
    table = layer0.table_np
    uk = layer0.u_k.cpu().numpy()
    uv = layer0.u_v.cpu().numpy()
    k, v = workloads.kv_tokens(wl, 0, 0, 0, length, "cuda")
    k = bf16_np(k[:, kv:kv + 1])
    v = bf16_np(v[:, kv:kv + 1])
    pool = oracle.new_pool(layer0.num_pages, wl.num_kv_heads, geom)
    c0 = float(layer0.clip_k[kv])
    kq = oracle.encode(k[64:64 + n_hist, 0], uk[kv], c0, geom.group)[:3]
    vq = oracle.encode(v[64:64 + n_hist, 0], uv[kv], c0, geom.group)[:3]
    oracle.store_history(pool, table[0], np.arange(n_hist), kv, kq, vq, geom)
    sk = np.zeros((1, wl.num_kv_heads, 64, 128), np.float32)
    sv = np.zeros_like(sk)
    rk = np.zeros((1, wl.num_kv_heads, 256, 128), np.float32)
    rv = np.zeros_like(rk)
    sk[0, kv] = k[:64, 0]
    sv[0, kv] = v[:64, 0]
    p = np.arange(length - 256, length)
    rk[0, kv][p % 256] = k[p, 0]
    rv[0, kv][p % 256] = v[p, 0]
    q = bf16_np(layer0.q[:1])
    gq = wl.gqa
    heads = [(0, kv * gq + i) for i in range(gq)]
    clip = layer0.clip_k.cpu().numpy()
    threads = len(os.sched_getaffinity(0))
    times = []
    with threadpoolctl.threadpool_limits(threads, user_api="blas"):
        for _ in range(3):
            t = time.perf_counter()
            oracle.demote(pool, table, uk, uv, clip, clip, k[None, 64:65], v[None, 64:65], [0],
                          geom)
            oracle.decode_attention(pool, table, sk, sv, rk, rv, [0], [length], q, uk, uv, geom,
                                    heads=heads)
            times.append(time.perf_counter() - t)
    per_head = float(np.median(times))
    step_s = per_head * wl.num_kv_heads * wl.num_layers * batch
    head_bytes = n_hist * bytes_per_token_head(wl.group_size) + 320 * 128 * 2 * 2
    step_bytes = head_bytes * wl.num_kv_heads * wl.num_layers * batch
    facts = host_facts()
    return {"value": round(step_bytes / step_s / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "decode_steps_per_s": round(1.0 / step_s, 6), "host": facts,
            "sample": f"numpy fp64 oracle, 1 KV head ({gq} query heads) of 1 layer at context "
                      f"{length}: demotion of 1 token + decode attention over the 3-segment "
                      f"cache ({per_head:.2f}s, median of 3: "
                      f"{', '.join(f'{x:.2f}' for x in times)}), BLAS pool of {threads} threads "
                      f"(the elementwise numpy work runs on one), scaled x{wl.num_kv_heads} heads "
                      f"x{wl.num_layers} layers" + (f" x{batch} sequences" if batch > 1 else "")}


if __name__ == "__main__":
    main()
