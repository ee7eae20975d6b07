"""Throughput of the rolling-window KV decode path on one MI355X.

Default workload: 36 layers x 64 streams, 16 query / 2 KV heads, head_dim 128,
bf16 rings of W = 375 positions (30 s at the 80 ms clock), base re-based in
chunks of 25 positions.  A step is one clock step of every stream through the
whole path: the step plan, re-base, append and GQA decode attention for all
36 layers -- by default one rkv_decode_step_pipelined launch, which also
computes the next step's plan (--path fused: rkv_advance + rkv_decode_step;
--path separate: the individual calls).  Inputs are synthetic N(0, 1) bf16
tensors already resident on the GPU (a pool of steps cycled).

Prints one JSON line: stream-layer decode steps per second (value), the
roofline of the dominant kernel (algorithmic bytes per launch over the
launch's average duration, timed with HIP events on the launch stream on a
sample of the timed launches), and the CPU oracle timed on a bounded sample
on the host cores.

Other workloads (--config): 1 = one layer x one stream, re-base every step
(compensated); 3 = 256 streams of mixed windows 375/250/188 with start
offsets and 1 % x8 outliers; 4 = 26 x 16 streams, window 8192, logical-offset
compaction; 5 = encoder chunks, 32 x 128 streams, 20 heads x 64, 4 frames per
step over a 750-frame window.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0

METRIC = "stream-layer decode steps/sec + achieved HBM GB/s (% of peak), W=375 window"

CONFIGS = {
    1: dict(name="1 layer x 1 stream, 16q/2kv d128 bf16, W=375, re-base every step "
                 "(compensated), 1000 steps",
            mode="rebase", L=1, S=1, W=375, dc=1, comp=True, period=1000, steps=1000, warmup=0),
    2: dict(name="36 layers x 64 streams, 16q/2kv d128 bf16, W=375 rings, re-base chunk 25",
            mode="rebase", L=36, S=64, W=375, dc=25, comp=False, period=64, steps=2000, warmup=100),
    3: dict(name="36 layers x 256 streams, W mix 375/250/188 (86/85/85), re-base chunk 25, "
                 "start offsets U[0,5000], 1% x8 outliers",
            mode="rebase", L=36, S=256, W=(375, 250, 188), dc=25, comp=False, period=16,
            steps=600, warmup=50, outlier=0.01, offsets=5000,
            # staggered starts: a few streams re-base in every step, which the
            # dense update launch handles better than the in-attention write-back
            path="update"),
    4: dict(name="26 layers x 16 streams, 16q/2kv d128 bf16, window 8192, capacity 9216, "
                 "logical-offset compaction",
            mode="compact", L=26, S=16, W=8192, cap=9216, period=16, steps=1024, warmup=16),
    5: dict(name="encoder chunks: 32 layers x 128 streams, 20 heads x d64 bf16, F=4 frames "
                 "per step, 750-frame window (ring 754)",
            mode="enc", L=32, S=128, H=20, d=64, F=4, W=750, period=4, steps=400, warmup=20),
}


def bytes_per_sl_step(c):
    """Algorithmic bytes of one (stream, layer) step: every byte the step must
    move at least once (bf16 = 2 bytes)."""
    if c["mode"] == "rebase":
        Hq, Hkv, d = 16, 2, 128
        Ws = c["W"] if isinstance(c["W"], tuple) else (c["W"],)
        mix = [86, 85, 85] if len(Ws) == 3 else [1]
        total = 0.0
        for W, n in zip(Ws, mix):
            row = Hkv * d * 2                                   # one K (or V) row, all KV heads
            b = W * 2 * row                                     # K and V window read
            b += 2 * Hq * d * 2                                 # q in, out
            b += 2 * row + 2 * row                              # k_new/v_new in, appended K/V
            b += (W - 1) * row / c["dc"]                        # re-based K written
            if c.get("comp"):
                b += 2 * (W - 1) * row / c["dc"] + row          # residual read + written, appended
            total += b * n
        return total / sum(mix)
    if c["mode"] == "compact":
        Hq, Hkv, d = 16, 2, 128
        row = Hkv * d * 2
        E = c["cap"] - c["W"]
        avg_len = (c["W"] + 1 + c["cap"]) / 2.0
        return (avg_len * 2 * row + 2 * Hq * d * 2 + 4 * row
                + 2 * 2 * c["W"] * row / E)                     # compaction read + write, amortised
    H, d, F, W = c["H"], c["d"], c["F"], c["W"]
    row = H * d * 2
    return W * 2 * row + 2 * F * row + 2 * F * row + 2 * F * row  # cached read, q/out, new in, append


def launch_bytes(c, windows, origins, steps):
    """Algorithmic bytes of the attention launches (with the cache updates of
    the step) at the given step numbers (0 = a stream's first step), summed
    over the launches, every layer and stream: the attended K+V rows, q and
    out, the new K/V rows read and appended, and on a re-base step the rotated
    K of the retained rows written (plus, compensated, their residuals read
    and written).  The compaction move runs in its own launch and is not
    charged here."""
    L, S = c["L"], c["S"]
    windows = np.asarray(windows, np.int64)
    origins = np.asarray(origins, np.int64)
    total = 0.0
    if c["mode"] == "enc":
        return float(bytes_per_sl_step(c)) * L * S * len(steps)
    Hq, Hkv, d = 16, 2, 128
    row = Hkv * d * 2
    fixed = 2 * Hq * d * 2 + 2 * row + 2 * row          # q, out; new K/V in; appended K/V
    if c["mode"] == "compact":
        W, cap = c["W"], c["cap"]
        need = max(steps) + 1
        rows = np.empty(need, np.int64)                  # rows attended at each step
        n = 0
        for t in range(need):
            if n >= cap and n >= W:
                n = W
            n += 1
            rows[t] = n
        for t in steps:
            total += S * (rows[t] * 2 * row + fixed)
        return total * L
    dc = c["dc"]
    for t in steps:
        length = np.minimum(t + 1, windows)
        oldest = origins + t - length + 1
        base = dc * (oldest // dc)
        if t == 0:
            prev = dc * (origins // dc)
        else:
            plen = np.minimum(t, windows)
            prev = dc * ((origins + t - 1 - plen + 1) // dc)
        moved = base != prev
        b = length * 2 * row + fixed + moved * (length - 1) * row
        if c.get("comp"):
            b = b + moved * 2 * (length - 1) * row + row
        total += float(b.sum())
    return total * L


ATTN_SOURCES = ("attn.hip", "rkv_device.h", "rkv_internal.h", "rkv_plan.h")


def kernel_source_digest(files=ATTN_SOURCES):
    """Digest of the kernel sources a stored counter figure was taken from."""
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(ROOT, "rolling_window_kv_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    the summary is missing or was taken from a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(f"{kernel}@{workload}")
    files = tuple(ent.get("kernel_src_files", ATTN_SOURCES)) if ent else ATTN_SOURCES
    if not ent or ent.get("kernel_src_digest") != kernel_source_digest(files):
        return None
    return ent.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU oracle baseline
# ---------------------------------------------------------------------------

def _oracle_worker(args):
    seed, stream, c, fill, steps, budget = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):
        from oracle import schedule as sch
        from oracle import storage as stg
        from rolling_window_kv_amd import synth
        W = c["W"][0] if isinstance(c["W"], tuple) else c["W"]
        n = fill + steps
        P = c["period"]                       # the same input pool the GPU run cycles
        if c["mode"] == "enc":
            q, k, v = synth.encoder_pair(seed, 0, stream, P, c["F"], c["H"], c["d"])
            q, k, v = (x.double().numpy()[np.arange(n) % P] for x in (q, k, v))
            ring = stg.EncoderRing(c["H"], c["d"], W, c["F"], 1e6)
        else:
            q, k, v = synth.decoder_pair(seed, 0, stream, P, 16, 2, 128, c.get("outlier", 0.0))
            q, k, v = (x.double().numpy()[np.arange(n) % P] for x in (q, k, v))
            if c["mode"] == "compact":
                ring = stg.CompactBuffer(16, 2, 128, W, c["cap"], 1e6)
            else:
                ring = stg.RebaseRing(16, 2, 128, W, c["dc"], 1e6, compensated=c.get("comp", False))
        if c["mode"] == "compact":
            # Fill the first `fill` rows with the oracle's own append (vectorised)
            # and its schedule, instead of `fill` full attention steps.
            for _ in range(fill):
                sch.step(sch.MODE_COMPACT, ring.state)
            hi, _ = stg.append_k(k[:fill], np.arange(fill)[:, None], 1e6)
            ring.k[:, :fill] = hi.transpose(1, 0, 2)
            ring.v[:, :fill] = v[:fill].transpose(1, 0, 2)
        else:
            for t in range(fill):
                ring.step(q[t], k[t], v[t])
        t0 = time.perf_counter()
        done = 0
        for t in range(fill, n):
            ring.step(q[t], k[t], v[t])
            done += 1
            if time.perf_counter() - t0 > budget:
                break
        return done, time.perf_counter() - t0


def cpu_baseline(c, seed, budget_s=15.0):
    """Storage-faithful oracle (plan, re-base, append and attention per step,
    float64 NumPy) on a bounded sample: one layer of several streams, each
    filled to a full window untimed, then timed for a fixed number of steps."""
    import multiprocessing as mp
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    # one single-threaded process per core, up to one per stream and up to
    # the job's CPU share (OMP_NUM_THREADS where the machine sets it)
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    share = share if share > 0 else cores
    workers = max(1, min(share, cores, c["S"]))
    W = c["W"][0] if isinstance(c["W"], tuple) else c["W"]
    if c["mode"] == "compact":
        fill = (W + c["cap"]) // 2   # mid-way between two compactions
    elif c["mode"] == "enc":
        fill = (W + c["F"] - 1) // c["F"] + 1
    else:
        fill = W
    max_steps = 200000
    ctx = mp.get_context("spawn")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_worker,
                       [(seed, s, c, fill, max_steps, budget_s) for s in range(workers)])
    wall = time.perf_counter() - t0
    total = sum(r[0] for r in res)
    timed = max(r[1] for r in res)
    return {"value": total / timed, "unit": "stream-layer steps/s", "cores": workers,
            "kind": "oracle", "processes": workers, "threads_per_process": 1,
            "host_cores": cores, "cpu_share": share, "cpu_model": cpu_model(),
            "sample": f"storage-faithful float64 oracle, 1 layer x {workers} streams, "
                      f"window pre-filled ({fill} steps untimed), then timed steps for "
                      f"{budget_s:g} s per stream ({total} steps in all), one single-threaded "
                      f"process per stream on {workers} of the {cores} host cores "
                      f"(CPU share {share}) ({wall:.1f} s wall incl. fill)"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
# GPU run
# ---------------------------------------------------------------------------

def build_inputs(c, seed, dev):
    import torch
    from rolling_window_kv_amd import synth
    P = c["period"]
    if c["mode"] == "enc":
        q, k, v = synth.encoder_pool(seed, c["L"], c["S"], P, c["F"], c["H"], c["d"])
    else:
        q, k, v = synth.decoder_pool(seed, c["L"], c["S"], P, 16, 2, 128, c.get("outlier", 0.0))
    return q.to(dev), k.to(dev), v.to(dev)


def state_skip(rkv, cfg, cache, windows, caps, origins, steps):
    """Streams `steps` steps on from their start without launches: states by
    rkv_state_advance_host, every ring row random (normal bfloat16)."""
    import torch
    h = rkv.rkv_state_init_host(cfg, windows, caps, origins)
    rkv.rkv_state_advance_host(cfg, h, steps)
    cache.state.copy_(torch.from_numpy(h.view(np.uint8).copy()))
    for t in (cache.k, cache.v, cache.k_lo):
        if t is not None:
            t.normal_()
    torch.cuda.synchronize()


def run_gpu(c, args):
    import torch
    from rolling_window_kv_amd import rkv, synth
    rkv.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = 1000 + args.config
    L, S = c["L"], c["S"]
    t_setup = time.perf_counter()
    q, k, v = build_inputs(c, seed, dev)
    kv_flags = rkv.RKV_F_KV_FP16 if args.kv_fp16 else 0
    if args.merge_launch:
        kv_flags |= rkv.RKV_F_MERGE_LAUNCH
    if c["mode"] == "rebase":
        flags = (rkv.RKV_F_COMPENSATED if c.get("comp") else 0) | kv_flags
        cfg = rkv.make_cfg(S, L, rebase_chunk=c["dc"], flags=flags, num_splits=args.splits)
        if isinstance(c["W"], tuple):
            counts = [86, 85, 85]
            windows = np.repeat(np.array(c["W"], np.int32), counts)
            from rolling_window_kv_amd import synth
            t0 = synth.start_offsets(seed, S, c["offsets"])
            origins = np.maximum(0, t0 - windows).astype(np.int64)
        else:
            windows = np.full(S, c["W"], np.int32)
            origins = np.zeros(S, np.int64)
        slots = int(windows.max())
        cache = rkv.Cache(cfg, slots, windows, windows, origins, device=dev, zero=False, layout=args.layout)
        caps = windows
        prefill = slots
    elif c["mode"] == "compact":
        cfg = rkv.make_cfg(S, L, mode=rkv.RKV_MODE_COMPACT, flags=kv_flags,
                           num_splits=args.splits)
        cache = rkv.Cache(cfg, c["cap"], c["W"], c["cap"], 0, device=dev, zero=False, layout=args.layout)
        prefill = c["cap"]
        windows, origins = np.full(S, c["W"], np.int32), np.zeros(S, np.int64)
        caps = np.full(S, c["cap"], np.int32)
    else:
        cfg = rkv.make_cfg(S, L, num_q_heads=c["H"], num_kv_heads=c["H"], head_dim=c["d"],
                           mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=c["F"])
        cap = c["W"] + c["F"]
        cache = rkv.Cache(cfg, cap, c["W"], cap, 0, device=dev, zero=False, layout=args.layout)
        prefill = (cap + c["F"] - 1) // c["F"]
        windows, origins = np.full(S, c["W"], np.int32), np.zeros(S, np.int64)
        caps = np.full(S, cap, np.int32)
    out = torch.empty(q.shape[1:], dtype=torch.bfloat16, device=dev)
    P = q.shape[0]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    ws = cache.workspace
    separate = args.path in ("separate", "update")

    pipelined = (args.path in ("pipelined", "update") and c["mode"] != "enc"
                 and not args.per_layer)
    plans = [cache.plan, cache.plan_next]
    per_layer = None
    if args.per_layer:
        # one call per layer and step, as a decoder whose layer l + 1 needs
        # layer l's output would make them; the step plan is shared
        if c["mode"] == "enc":
            cfg1 = rkv.make_cfg(S, 1, num_q_heads=c["H"], num_kv_heads=c["H"], head_dim=c["d"],
                                mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=c["F"],
                                max_cap=cfg.max_cap)
        else:
            cfg1 = rkv.make_cfg(S, 1, mode=cfg.mode, rebase_chunk=cfg.rebase_chunk,
                                flags=cfg.flags, num_splits=args.splits, max_cap=cfg.max_cap)
        views = [rkv.kv_view(cache.k[l:l + 1], cache.v[l:l + 1],
                             None if cache.k_lo is None else cache.k_lo[l:l + 1])
                 for l in range(L)]
        nb = rkv.rkv_workspace_bytes(cfg1, cache.k.shape[3])
        ws1 = torch.zeros((nb + 3) // 4, dtype=torch.float32, device=dev) if nb else None
        slices = [[(q[j][l], k[j][l], v[j][l]) for l in range(L)] for j in range(q.shape[0])]
        outs = [out[l] for l in range(L)]
        per_layer = (cfg1, views, ws1, slices, outs)

    def layer_calls(j, st):
        """One step in per-layer mode: the plan, then one launch per layer."""
        cfg1, views, ws1, slices, outs = per_layer
        rkv.rkv_advance(cfg, cache.state, cache.plan, st)
        if c["mode"] == "compact":
            rkv.rkv_compact(cfg, cache.plan, cache.kv, st)
        for l in range(L):
            ql, kl, vl = slices[j][l]
            if c["mode"] == "enc":
                rkv.rkv_encoder_chunk_attn(cfg1, cache.plan, views[l], ql, kl, vl, outs[l], ws1,
                                           st)
            else:
                rkv.rkv_decode_step(cfg1, cache.plan, views[l], ql, kl, vl, outs[l], ws1, st)

    graphs = None
    tcond = None
    if args.tcond:
        # delay conditioning after each step's attention: the 8 post-trained
        # (clock, delay) settings, streams spread over them
        settings = [(240, 80), (320, 80), (480, 80), (560, 80), (240, 120), (480, 120),
                    (320, 160), (480, 160)]
        conds = [rkv.rkv_tcond_delay_tokens(dl, ck) for dl, ck in settings]
        table, A = synth.tcond_weights(7, L, cfg.num_q_heads * cfg.head_dim, 256)
        tc = rkv.make_tcond_cfg(L, cfg.num_q_heads * cfg.head_dim, dim=256,
                                num_conds=len(conds), max_frame_len=8)
        mod = torch.empty((L, len(conds), 2, tc.hidden), dtype=torch.float32, device=dev)
        rkv.rkv_tcond_prepare(tc, [n for n, _ in conds], [f for _, f in conds], table.to(dev),
                              A.to(dev), mod, sp)
        cond = torch.arange(S, dtype=torch.int32, device=dev) % len(conds)
        tcond = (tc, mod, cond)
    # the pipelined step applies the conditioning as it stores its output
    # (--tcond-pass: a separate rkv_tcond_modulate launch after the step)
    tcond_fused = tcond is not None and pipelined and args.path == "pipelined" and \
        not args.tcond_pass

    def step(i, ev=None):
        j = i % P
        if per_layer is not None:
            if graphs is not None:
                graphs[j].replay()
            else:
                layer_calls(j, sp)
            return
        if pipelined:
            # one launch per step: this step's plan was written by the previous
            # launch (or the priming rkv_advance), the next one is written now
            cur, nxt = plans[i % 2], plans[(i + 1) % 2]
            if c["mode"] == "compact":
                rkv.rkv_compact(cfg, cur, cache.kv, sp)
            if ev is not None:
                ev[0].record(stream)
            if args.path == "update":
                rkv.rkv_update_step(cfg, cur, cache.kv, k[j], v[j], sp)
                rkv.rkv_decode_attn_pipelined(cfg, cache.state, cur, nxt, cache.kv, q[j], out,
                                              ws, sp)
            elif tcond_fused:
                rkv.rkv_decode_step_pipelined_tcond(cfg, tcond[0], tcond[1], tcond[2],
                                                    cache.state, cur, nxt, cache.kv, q[j], k[j],
                                                    v[j], out, ws, sp)
            else:
                rkv.rkv_decode_step_pipelined(cfg, cache.state, cur, nxt, cache.kv, q[j], k[j],
                                              v[j], out, ws, sp)
            if ev is not None:
                ev[1].record(stream)
            if tcond is not None and not tcond_fused:
                rkv.rkv_tcond_modulate(cfg, tcond[0], tcond[1], tcond[2], out, sp)
            return
        rkv.rkv_advance(cfg, cache.state, cache.plan, sp)
        if c["mode"] == "compact":
            rkv.rkv_compact(cfg, cache.plan, cache.kv, sp)
        if ev is not None:
            ev[0].record(stream)
        if c["mode"] == "enc":
            rkv.rkv_encoder_chunk_attn(cfg, cache.plan, cache.kv, q[j], k[j], v[j], out, ws, sp)
        elif separate:
            if c["mode"] == "rebase":
                rkv.rkv_roll_rebase(cfg, cache.plan, cache.kv, sp)
            rkv.rkv_append(cfg, cache.plan, cache.kv, k[j], v[j], sp)
            rkv.rkv_decode_attn(cfg, cache.plan, cache.kv, q[j], out, ws, sp)
        else:
            rkv.rkv_decode_step(cfg, cache.plan, cache.kv, q[j], k[j], v[j], out, ws, sp)
        if ev is not None:
            ev[1].record(stream)
        if tcond is not None:
            rkv.rkv_tcond_modulate(cfg, tcond[0], tcond[1], tcond[2], out, sp)

    def fill(i):
        # Untimed set-up: the same cache updates as a step, without attention
        # (identical ring contents), so every launch of the attention kernel
        # in the run is a full-window one.
        j = i % P
        rkv.rkv_advance(cfg, cache.state, cache.plan, sp)
        if c["mode"] == "compact":
            rkv.rkv_compact(cfg, cache.plan, cache.kv, sp)
        if c["mode"] == "rebase":
            rkv.rkv_roll_rebase(cfg, cache.plan, cache.kv, sp)
        rkv.rkv_append(cfg, cache.plan, cache.kv, k[j], v[j], sp)

    i = 0
    if args.state_fill:
        # (counter runs) the states after `prefill` steps written directly and
        # the rings filled with random values: from here on the same launches
        # over the same rows as a filled run, without its thousands of fill
        # launches; outputs differ
        state_skip(rkv, cfg, cache, windows, caps, origins, prefill)
        i = prefill
    for _ in range(i, prefill):       # fill every window (untimed set-up)
        if c["mode"] == "enc":
            step(i)
        else:
            fill(i)
        i += 1
    if pipelined:                     # the first pipelined step's plan
        rkv.rkv_advance(cfg, cache.state, plans[i % 2], sp)
    if per_layer is not None and args.graph:
        # one HIP graph per pool entry (the inputs differ), each the whole
        # step: the plan and the L per-layer launches.  Capturing runs nothing.
        torch.cuda.synchronize()
        graphs = []
        for j in range(P):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                layer_calls(j, None)
            graphs.append(g)
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step(i)
        i += 1
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    # Live kernel timing inside the timed region.  Pipelined decoder steps are
    # one launch of the attention kernel each: event pairs bracket runs of RUN
    # consecutive launches covering every timed launch (a pair around every
    # launch costs several microseconds per step), and the mean launch
    # duration is their total time / K.  Otherwise other kernels run between
    # attention launches: a pair around the attention launch(es) of every
    # RUN-th step.  Each timed launch is charged its own algorithmic bytes
    # (launch_bytes: a re-base launch also writes the rotated K, a compaction
    # buffer's row count varies), so the fraction follows from the launches
    # actually timed.
    K = args.steps
    RUN = 8
    bracket = (pipelined and args.path == "pipelined" and c["mode"] == "rebase"
               and (tcond is None or tcond_fused))
    if per_layer is not None:
        args.kernel_events = False    # the roofline uses the whole step's time
    runs = []                          # (first, last + 1) timed-step ranges
    if args.kernel_events:
        runs = ([(n, min(n + RUN, K)) for n in range(0, K, RUN)] if bracket
                else [(n, n + 1) for n in range(0, K, RUN)])
    ev = {n: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for n, _ in runs}
    ends = {m - 1: n for n, m in runs}
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    i0 = i
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for n in range(K):
        if bracket and n in ev:
            ev[n][0].record(stream)
        step(i, None if bracket else ev.get(n))
        if bracket and n in ends:
            ev[ends[n]][1].record(stream)
        i += 1
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    elapsed_ms = start.elapsed_time(end)
    kernel_ms = kernel_bytes = None
    kernel_samples = 0
    if runs:
        timed = [i0 + t for n, m in runs for t in range(n, m)]
        kernel_samples = len(timed)
        kernel_ms = sum(ev[n][0].elapsed_time(ev[n][1]) for n, _ in runs) / kernel_samples
        kernel_bytes = launch_bytes(c, windows, origins, timed) / kernel_samples
    copy_gbps = device_copy_gbps()     # after the timed region
    return dict(cfg=cfg, tcond_fused=tcond_fused, elapsed_ms=elapsed_ms, kernel_ms=kernel_ms,
                kernel_bytes=kernel_bytes,
                wall_s=wall, kernel_samples=kernel_samples, copy_gbps=copy_gbps,
                first_timed_step=i0, windows=windows, origins=origins,
                kernel_timing=("event pairs around runs of %d back-to-back launches, every "
                               "timed launch" % RUN) if bracket
                else "event pair around the attention launch(es) of every %d-th step" % RUN,
                setup_s=setup_s, prefill=prefill)


def run_mel(args):
    """The rolling log-mel front end (rkv_mel_step): S streams, one step of
    1280 samples (80 ms at 16 kHz) per call, 8 frames of 128 mel bands each.
    Reported against the float32 vector peak with the direct DFT's flops
    (4 per sample and bin, plus 2 per bin and band)."""
    import torch
    from rolling_window_kv_amd import rkv
    S = args.mel
    steps = args.steps or 200
    warm = args.warmup if args.warmup is not None else 10
    cfg = rkv.make_mel_cfg(S)
    dev = torch.device("cuda:0")
    fe = rkv.MelFrontend(cfg, device=dev)
    gen = torch.Generator().manual_seed(6)
    P = 8
    x = (torch.randn((P, S, cfg.samples_per_step), generator=gen) * 0.1).to(dev)
    out = torch.empty((S, cfg.samples_per_step // cfg.hop, cfg.n_mels), device=dev)
    stream = torch.cuda.current_stream()
    for i in range(warm):
        fe.step(x[i % P], out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        fe.step(x[i % P], out)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    frames = S * (cfg.samples_per_step // cfg.hop)
    bins = cfg.n_fft // 2 + 1
    flops = frames * (4.0 * cfg.n_fft * bins + 2.0 * bins * cfg.n_mels)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"metric": "log-mel frames/s (rolling front end)", "value": round(frames / ms * 1e3, 1),
            "unit": "frames/s", "n_gpus": 1, "steps": steps, "warmup": warm,
            "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"rolling log-mel front end: {S} streams, 1280 samples per "
                                   "step (80 ms at 16 kHz), n_fft 400, hop 160, 128 mel"},
            "roofline": {"bound": "alu", "achieved": round(tflops, 3), "peak": 157.3,
                         "unit": "TFLOP/s", "frac": round(tflops / 157.3, 4), "traffic": None,
                         "kernel": "mel_kernel", "flops_per_step": flops},
            "cpu_baseline": None}


def run_encoder_stack(args):
    """The incremental encoder step through the whole stack (rkv_advance +
    rkv_encoder_step): 32 layers, hidden 1280 (20 heads of 64), MLP 5120,
    S streams x 4 new frames per 80 ms step, 750-frame window (filled by
    untimed steps first); synthetic weights.  The step reads every layer's
    cached window (K and V, 750 x 1280 bfloat16 per stream) and weights once,
    so it is bound by HBM: reported against 8 TB/s with the algorithmic bytes
    of a step (per layer the window read, the appended K/V rows and the
    layer's weights; the float32 residual stream in and out once).  The matrix
    flops (the six projections, 2 x tokens x (4 hidden^2 + 2 hidden ffn), and
    the chunk attention, 4 x frames x (W + F) x hidden per stream) are
    reported beside it: at 0.7 TFLOP per step they need an eighth of the time
    the bytes do."""
    import torch
    from rolling_window_kv_amd import rkv, synth
    S = args.encoder_stack
    L, H, d, F, W, ffn = 32, 20, 64, 4, 750, 5120
    hidden = H * d
    steps = args.steps or 50
    warm = args.warmup if args.warmup is not None else 5
    dev = torch.device("cuda:0")
    cfg = rkv.make_cfg(S, L, num_q_heads=H, num_kv_heads=H, head_dim=d,
                       mode=rkv.RKV_MODE_ENC_CHUNK, new_rows=F)
    ecfg = rkv.make_encoder_cfg(ffn=ffn, norm_eps=1e-5)
    cap = W + F
    cache = rkv.Cache(cfg, cap, W, cap, 0, device=dev)
    wdev = rkv.pack_encoder_weights(synth.encoder_stack_weights(5, L, hidden, ffn)).to(dev)
    ws = torch.empty(rkv.rkv_encoder_step_workspace_bytes(cfg, ecfg, cap), dtype=torch.uint8,
                     device=dev)
    P = 4
    xin = synth.encoder_stack_inputs(5, S, P, F, hidden).to(dev)
    x = torch.empty_like(xin[0])
    stream = torch.cuda.current_stream()

    def step(i):
        x.copy_(xin[i % P])
        rkv.rkv_advance(cfg, cache.state, cache.plan)
        rkv.rkv_encoder_step(cfg, ecfg, cache.plan, cache.kv, wdev, x, ws)

    prefill = (cap + F - 1) // F          # untimed: the window is full from then on
    first = 0
    if args.state_fill:
        state_skip(rkv, cfg, cache, np.full(S, W, np.int32), np.full(S, cap, np.int32),
                   np.zeros(S, np.int64), prefill)
        first = prefill
    for i in range(first, prefill + warm):
        step(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        step(prefill + warm + i)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    tokens = S * F
    flops = L * (2.0 * tokens * (4 * hidden * hidden + 2 * hidden * ffn)
                 + 4.0 * S * F * cap * hidden)
    tflops = flops / (ms * 1e-3) / 1e12
    row = hidden * 2
    nbytes = (L * (S * (W * 2 * row + 2 * F * row)
                   + rkv.rkv_encoder_layer_weight_bytes(cfg, ecfg)) + 2 * tokens * hidden * 4)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"metric": "encoder frames/s (32-layer incremental step)",
            "value": round(tokens / ms * 1e3, 1), "unit": "frames/s", "n_gpus": 1,
            "steps": steps, "warmup": warm, "ms_per_step": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"incremental encoder step: {L} layers, hidden {hidden} "
                                   f"({H}x{d}), MLP {ffn}, {S} streams x {F} frames, "
                                   f"window {W}; synthetic weights",
                       **({"fill": "state written directly, random rings"} if args.state_fill
                          else {})},
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                         "kernel": "rkv_encoder_step (whole step)", "bytes_per_step": nbytes,
                         "matrix_tflops": round(tflops, 2), "flops_per_step": flops},
            "cpu_baseline": None}


def device_copy_gbps(mib=1024, reps=10):
    """Read + write bandwidth of a plain device-to-device copy (torch) on the
    same GPU: the practical ceiling for traffic that reads and writes."""
    import torch
    n = mib * 2 ** 20 // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        y.copy_(x)
    b.record()
    torch.cuda.synchronize()
    gbps = 2 * n * 4 * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return gbps


def _summarize_rocpd(path, root, last, short):
    """The same figures from rocprofv3's SQLite output (the default format):
    per-kernel dispatch statistics, the mean of each kernel's last `last`
    dispatches (in start order), and counter values per dispatch."""
    import sqlite3
    from collections import OrderedDict, defaultdict
    con = sqlite3.connect(path)
    rel = os.path.relpath(path, root)
    lines = []
    dur = defaultdict(list)
    for name, start, end in con.execute("select name, start, end from kernels order by start"):
        dur[name].append(int(end) - int(start))
    if dur:
        total = sum(sum(d) for d in dur.values())
        lines.append(f"# rocprofv3 kernel dispatches: {rel}")
        tail = f" {'last%d_mean_us' % last:>15}" if last else ""
        lines.append(f"{'calls':>7} {'mean_us':>10} {'median_us':>10} {'min_us':>10} {'max_us':>10} "
                     f"{'pct':>6}{tail}  kernel")
        for name, d in sorted(dur.items(), key=lambda x: -sum(x[1])):
            lt = f" {np.mean(d[-last:]) / 1e3:15.2f}" if last else ""
            lines.append(f"{len(d):7d} {np.mean(d) / 1e3:10.2f} {np.median(d) / 1e3:10.2f} "
                         f"{np.min(d) / 1e3:10.2f} {np.max(d) / 1e3:10.2f} "
                         f"{100.0 * sum(d) / total:6.2f}{lt}  {short(name)}")
    per = OrderedDict()
    for name, disp, cname, value in con.execute(
            "select kernel_name, dispatch_id, counter_name, value from counters_collection "
            "order by dispatch_id"):
        per.setdefault((name, disp), defaultdict(float))[cname] += float(value)
    if per:
        agg = defaultdict(lambda: defaultdict(list))
        for (name, _), cnt in per.items():
            for cn, v in cnt.items():
                agg[name][cn].append(v)
        lines.append(f"# counters per dispatch: {rel}")
        tail = f" {'last%d_mean' % last:>16}" if last else ""
        lines.append(f"{'dispatches':>10} {'counter':>12} {'mean':>16} {'min':>16} {'max':>16}{tail}"
                     f"  kernel")
        for name, cs in agg.items():
            for cn, v in cs.items():
                lt = f" {np.mean(v[-last:]):16.1f}" if last else ""
                lines.append(f"{len(v):10d} {cn:>12} {np.mean(v):16.1f} {np.min(v):16.1f} "
                             f"{np.max(v):16.1f}{lt}  {short(name)}")
    con.close()
    return lines


def summarize_rocprof(root, last=0):
    """Per-kernel figures from a rocprofv3 CSV output folder: its own --stats
    table, mean dispatch duration from the kernel trace (and, with last > 0,
    the mean of each kernel's last `last` dispatches, e.g. a bench run's
    warm-up and timed steps without its set-up), and mean counter values per
    dispatch (FETCH_SIZE / WRITE_SIZE are in KiB)."""
    import csv
    import glob
    from collections import OrderedDict, defaultdict

    def short(name):
        return name if len(name) <= 110 else name[:107] + "..."

    lines = []
    for path in sorted(glob.glob(os.path.join(root, "**", "*.db"), recursive=True)):
        lines.extend(_summarize_rocpd(path, root, last, short))
    for path in sorted(glob.glob(os.path.join(root, "**", "*_kernel_stats.csv"), recursive=True)):
        lines.append(f"# rocprofv3 --stats: {os.path.relpath(path, root)}")
        lines.append(f"{'calls':>7} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel")
        for r in csv.DictReader(open(path)):
            lines.append(f"{int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:10.2f} "
                         f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} "
                         f"{float(r['Percentage']):6.2f}  {short(r['Name'])}")
    for path in sorted(glob.glob(os.path.join(root, "**", "*_kernel_trace.csv"), recursive=True)):
        dur = defaultdict(list)
        for r in csv.DictReader(open(path)):
            dur[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines.append(f"# kernel trace: {os.path.relpath(path, root)}")
        tail = f" {'last%d_mean_us' % last:>15}" if last else ""
        lines.append(f"{'calls':>7} {'mean_us':>10} {'median_us':>10}{tail}  kernel")
        for name, d in sorted(dur.items(), key=lambda x: -sum(x[1])):
            lt = f" {np.mean(d[-last:]) / 1e3:15.2f}" if last else ""
            lines.append(f"{len(d):7d} {np.mean(d) / 1e3:10.2f} {np.median(d) / 1e3:10.2f}{lt}  "
                         f"{short(name)}")
    for path in sorted(glob.glob(os.path.join(root, "**", "*_counter_collection.csv"),
                            recursive=True)):
        per = OrderedDict()
        for r in csv.DictReader(open(path)):
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per.setdefault(key, defaultdict(float))[r["Counter_Name"]] += float(r["Counter_Value"])
        agg = defaultdict(lambda: defaultdict(list))
        for (name, _), cnt in per.items():
            for cn, v in cnt.items():
                agg[name][cn].append(v)
        lines.append(f"# counters per dispatch: {os.path.relpath(path, root)}")
        lines.append(f"{'dispatches':>10} {'counter':>12} {'mean':>16} {'min':>16} {'max':>16}  kernel")
        for name, cs in agg.items():
            for cn, v in cs.items():
                lines.append(f"{len(v):10d} {cn:>12} {np.mean(v):16.1f} {np.min(v):16.1f} "
                             f"{np.max(v):16.1f}  {short(name)}")
    return "\n".join(lines)


def bench_config(args):
    """One decoder or encoder-chunk workload (args.config) on the GPU -> (its
    CONFIGS entry, the result line without cpu_baseline)."""
    c = dict(CONFIGS[args.config])
    if args.graph and not args.per_layer:
        print("--graph applies to --per-layer", file=sys.stderr)
        sys.exit(2)
    if args.per_layer and (args.tcond or args.path not in (None, "fused")):
        print("--per-layer runs rkv_advance + one fused step per layer", file=sys.stderr)
        sys.exit(2)
    if args.tcond and c["mode"] == "enc":
        print("--tcond: delay conditioning applies to the decoder workloads", file=sys.stderr)
        sys.exit(2)
    if args.kv_fp16 and c["mode"] == "enc":
        print("--kv-fp16: the encoder cache is bfloat16 only", file=sys.stderr)
        sys.exit(2)
    if args.path is None:
        args.path = "fused" if args.per_layer else c.get("path", "pipelined")
    args.steps = c["steps"] if args.steps is None else args.steps
    args.warmup = c["warmup"] if args.warmup is None else args.warmup

    r = run_gpu(c, args)
    tcond_fused = r["tcond_fused"]
    L, S, K = c["L"], c["S"], args.steps
    secs = r["elapsed_ms"] / 1e3
    sl_steps = L * S * K / secs
    b_sl = bytes_per_sl_step(c)
    step_gbps = b_sl * L * S * K / secs / 1e9
    kernel = {"rebase": "attn_kernel<128,4,decode_fused>",
              "compact": "attn_kernel<128,4,decode_fused>",
              "enc": "attn_kernel<64,2,encoder_fused>"}[c["mode"]]
    if args.path == "separate" and c["mode"] != "enc":
        kernel = "rebase+append+attn_kernel<128,4,decode_read>"
    if args.path == "update" and c["mode"] != "enc":
        kernel = "update+attn_kernel<128,4,decode_read>"
    if args.kv_fp16:
        kernel = kernel.replace(">", ",fp16>")
    roofline = None
    if r["kernel_ms"]:
        per_launch = r["kernel_bytes"]
        achieved = per_launch / (r["kernel_ms"] / 1e3) / 1e9
        # the stored counter figures were taken with the interleaved layout
        traffic = (load_traffic(kernel, f"config{args.config}")
                   if args.layout == "interleaved" else None)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                    "traffic": traffic, "kernel": kernel,
                    "kernel_ms": round(r["kernel_ms"], 5),
                    "kernel_launches_timed": r["kernel_samples"],
                    "kernel_timing": r["kernel_timing"],
                    "first_timed_step": r["first_timed_step"],
                    "alg_bytes_per_launch": round(per_launch, 1)}
    if args.per_layer:
        # L launches per step: the roofline takes the whole step's time and the
        # bytes of the timed steps
        i0 = r["first_timed_step"]
        per_step = launch_bytes(c, r["windows"], r["origins"], list(range(i0, i0 + K))) / K
        gbps = per_step / (r["elapsed_ms"] / K / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(gbps / PEAK_HBM_GBPS, 4),
                    "traffic": None,
                    "kernel": f"{L} per-layer launches per step ({kernel})",
                    "kernel_ms": round(r["elapsed_ms"] / K, 5),
                    "kernel_timing": "whole step (HIP events around the timed steps)",
                    "first_timed_step": i0,
                    "alg_bytes_per_step": round(per_step, 1)}
    res = {
        "metric": METRIC,
        "value": round(sl_steps, 1),
        "unit": "stream-layer steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(r["elapsed_ms"] / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 cache, bf16 i/o" if args.kv_fp16 else "bf16",
        "data": "synthetic",
        "config": {"workload": c["name"], "layers": L, "streams": S,
                   "path": ("per-layer" + (" graph" if args.graph else "")) if args.per_layer
                           else (args.path if c["mode"] != "enc" else "fused"),
                   "alg_bytes_per_stream_layer_step": b_sl,
                   **({"layout": args.layout} if args.layout != "interleaved" else {}),
                   **({"fill": "state written directly, random rings"} if args.state_fill
                      else {}),
                   **({"tcond": ("applied as the attention stores its output "
                                 "(rkv_decode_step_pipelined_tcond)" if tcond_fused else
                                 "rkv_tcond_modulate after each step") + ", 8 settings, dim 256"}
                      if args.tcond else {})},
        "achieved_GBps_step": round(step_gbps, 1),
        "device_copy_GBps": round(r["copy_gbps"], 1),
        "frac_of_device_copy": round(step_gbps / r["copy_gbps"], 4),
        "hbm_frac_step": round(step_gbps / PEAK_HBM_GBPS, 4),
        "clock_steps_per_s": round(K / secs, 1),
        "roofline": roofline,
        "cpu_baseline": None,
    }
    return c, res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", type=int, default=None, choices=sorted(CONFIGS),
                    help="workload (default 2, with short runs of the others reported as "
                         "'secondary' fields of the same line)")
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="default run: skip the short runs of the other workloads")
    ap.add_argument("--path", choices=("pipelined", "fused", "separate", "update"),
                    default=None,
                    help="default: update for workload 3, pipelined otherwise.  "
                         "pipelined: rkv_decode_step_pipelined (the step plan of the next "
                         "step computed in the same launch); fused: rkv_advance + "
                         "rkv_decode_step; separate: rkv_advance + rkv_roll_rebase + "
                         "rkv_append + rkv_decode_attn; update: rkv_update_step (re-base and "
                         "append in one launch) + rkv_decode_attn_pipelined (the read-only "
                         "attention with the next step's plan in the same launch) (encoder "
                         "workloads: always rkv_advance + rkv_encoder_chunk_attn)")
    ap.add_argument("--no-kernel-events", dest="kernel_events", action="store_false")
    ap.add_argument("--mel", type=int, default=0, metavar="STREAMS",
                    help="time the rolling log-mel front end for STREAMS streams instead")
    ap.add_argument("--encoder-stack", type=int, default=0, metavar="STREAMS",
                    help="time the 32-layer incremental encoder step for STREAMS streams "
                         "instead")
    ap.add_argument("--per-layer", action="store_true",
                    help="one launch per layer and step (rkv_decode_step or "
                         "rkv_encoder_chunk_attn with a one-layer view of the cache, after "
                         "one rkv_advance), as a decoder whose layers run in sequence calls "
                         "them")
    ap.add_argument("--state-fill", action="store_true",
                    help="start from the filled-window state written by rkv_state_advance_host "
                         "and random rings instead of running the fill steps (for counter "
                         "runs: the same timed launches, other values)")
    ap.add_argument("--splits", type=int, default=0, metavar="N",
                    help="key-range splits per (layer, stream, head) of the attention "
                         "launches (0: the library's choice)")
    ap.add_argument("--merge-launch", action="store_true",
                    help="merge split key ranges in a second launch (RKV_F_MERGE_LAUNCH) "
                         "instead of inside the attention launch")
    ap.add_argument("--graph", action="store_true",
                    help="with --per-layer: replay each step as a captured HIP graph")
    ap.add_argument("--layout", choices=("interleaved", "separate"), default="interleaved",
                    help="ring layout: K and V rows of a slot side by side (interleaved) or "
                         "K and V in separate buffers")
    ap.add_argument("--tcond", action="store_true",
                    help="apply the delay conditioning (rkv_tcond_modulate) to every step's "
                         "attention output (decoder workloads)")
    ap.add_argument("--tcond-pass", action="store_true",
                    help="with --tcond: modulate in a separate rkv_tcond_modulate launch after "
                         "each step instead of in the attention launch")
    ap.add_argument("--kv-fp16", action="store_true",
                    help="store K and V as fp16 (the fp16 cache variant; decoder workloads)")
    ap.add_argument("--no-cpu-baseline", dest="cpu", action="store_false")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch device-to-device copies of MIB MiB (10 launches): "
                         "the known-size kernel that scales the HBM byte counters")
    ap.add_argument("--summarize-rocprof", metavar="DIR", default=None,
                    help="print per-kernel figures from a rocprofv3 CSV output folder and exit")
    ap.add_argument("--summarize-last", type=int, default=0, metavar="N",
                    help="with --summarize-rocprof: also the mean of each kernel's last N "
                         "dispatches")
    args = ap.parse_args()
    args.path_given = args.path is not None
    if args.summarize_rocprof:
        print(summarize_rocprof(args.summarize_rocprof, args.summarize_last))
        return
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * 2 ** 20
        x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        for _ in range(10):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 10}))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: streams are independent, so N GPUs would each "
              "run the same per-GPU workload on their own streams with no communication; "
              "this benchmark measures the one-GPU share only.", file=sys.stderr)
        sys.exit(2)
    if args.mel:
        print(json.dumps(run_mel(args)), flush=True)
        return
    if args.encoder_stack:
        print(json.dumps(run_encoder_stack(args)), flush=True)
        return
    explicit = args.config is not None
    if args.config is None:
        args.config = 2
    default_run = not (explicit or args.per_layer or args.tcond or args.kv_fp16 or args.graph
                       or args.splits or args.layout != "interleaved" or args.path_given)
    # the other workloads first, so that the headline's timed launches are the
    # last launches of their kernel in a profile of this command
    secondary = secondary_runs(args) if default_run and args.secondary else None
    c, res = bench_config(args)
    if args.cpu and not args.kv_fp16 and not args.tcond and not args.per_layer:
        res["cpu_baseline"] = cpu_baseline(c, 1000 + args.config, args.cpu_budget)
    if secondary is not None:
        res["secondary"] = secondary
    print(json.dumps(res), flush=True)


# Short runs of the other workloads, reported beside the headline line:
# (name, overrides of the command-line arguments).
SECONDARY = (
    ("config1_1x1_every_step_rebase", dict(config=1)),
    ("config2_per_layer", dict(config=2, per_layer=True, steps=200, warmup=20)),
    ("config3_mixed_windows", dict(config=3, steps=200, warmup=20)),
    ("config4_compaction_w8192", dict(config=4, steps=256, warmup=16)),
    ("config5_encoder_chunks", dict(config=5, steps=100, warmup=10)),
)


def secondary_runs(args):
    """Each secondary workload with its own step count; per entry the fields
    of its own bench line that describe the measurement."""
    import copy
    import torch
    out = {}
    for name, over in SECONDARY:
        print(f"bench: secondary workload {name}", file=sys.stderr, flush=True)
        a = copy.copy(args)
        a.steps = a.warmup = a.path = None
        for k, v in over.items():
            setattr(a, k, v)
        _, r = bench_config(a)
        keep = ("value", "unit", "steps", "warmup", "ms_per_step", "hbm_frac_step",
                "achieved_GBps_step", "clock_steps_per_s", "roofline")
        out[name] = {"workload": r["config"]["workload"], "path": r["config"]["path"],
                     **{k: r[k] for k in keep}}
        torch.cuda.empty_cache()
    return out

if __name__ == "__main__":
    main()
