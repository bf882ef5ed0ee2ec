#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV cache on one MI355X.

Workload (default): Llama-3-8B-shaped GQA decode -- 32 layers, batch 16, 32 q heads / 8 KV
heads, head_dim 128, bf16 cache and q, block size 16, every request at 4096 tokens in the
first timed step, 32 per-layer caches (8.6 GB) sharing one seeded-permutation block table;
split-K partitions chosen by the library (partition_tokens 0: one work-group per compute
unit).

One step is one pass of the whole hot path over the batch:
  1. host allocator: append one token to each request (slots; copy-on-write pairs, if any,
     are copied with pa_copy_blocks in every layer),
  2. block-table export: the table rows, lengths and the new tokens' slots staged in one
     pinned host buffer and moved to the device by one pa_upload kernel on the launch stream,
  3. the 32 layers' pa_decode_append launches back to back: each writes its layer's 16 new
     tokens' K/V into the cache and decodes over it in one launch (`--step separate`: the 32
     layers' pa_kv_write first, then the 32 pa_decode launches).
Requests grow by one token per step, as in generation.

Reported (one JSON line): `value` = algorithmic bytes of the whole step (every request's
cached K/V once per KV head, q, out, table entries, lengths; plus the write's rows and
slots) / wall time per step.  `roofline` = the decode kernel (one launch per layer, with the
layer's write in it) measured with HIP events on the launch stream around each step's 32
back-to-back decode launches.  `cpu_baseline` = the float64 oracle
timed on a bounded sample of the same per-request work on the host.  Each run also prints,
on stderr, where a step's time goes: host microseconds per phase and HIP-event microseconds
of the upload, the writes, the decodes and the device's idle time between steps.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--graph]   # --graph: replay each step from HIP graphs
    python bench.py --workload {ragged_prefix,long_context,sweep,mxfp4}   # other workloads' decode rates
    python bench.py --workload swap     # preemption: swap-out / swap-in rates over the host link
    python bench.py --workload prefix_cache   # prompts through the prefix cache vs without it
    python bench.py --workload prefill  # causal paged prefill: TFLOP/s against the bf16 matrix peak
"""

import argparse
import contextlib
import gc
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode attention KV GB/s and % of HBM peak (GQA 32q/8kv d128, bf16)"
HBM_PEAK_GBPS = 8000.0
DECODE_KERNEL = "decode_mfma_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama3_8b_bf16_traffic.md")
TRAFFIC_FILE_FUSED = os.path.join(ROOT, "profiles", "decode_append_llama3_8b_bf16_traffic.md")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_408_amd", "csrc", f) for f in ("pagedkv.hip", "pa_device.h", "pa_layout.h")]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


@contextlib.contextmanager
def gc_held():
    """Python's cyclic garbage collector held off over a timed region, as timeit does.  A full
    collection walks every tracked object (about 170k once torch is imported: 40-55 ms), and
    when one lands inside the region the device idles for that long: a fresh box's first run,
    which also compiles this repository's modules to bytecode, shifted one into the timed steps
    (one step's allocator call took 37.7 ms).  Objects that exist before the region are
    frozen, so a collection after it stays cheap."""
    gc.collect()
    gc.freeze()
    was_enabled = gc.isenabled()
    gc.disable()
    try:
        yield
    finally:
        if was_enabled:
            gc.enable()
        gc.unfreeze()


# ----------------------------------------------------------------------------- byte model

def decode_bytes(seq_lens, Hq, Hkv, d, bs, kv_bytes, q_bytes):
    """Algorithmic bytes of one decode launch: K and V of every cached token once per KV
    head, q in, out, the table entries in use and the lengths."""
    kv = sum(2 * Hkv * int(L) * d * kv_bytes for L in seq_lens)
    qo = len(seq_lens) * Hq * d * 2 * q_bytes
    tab = sum(4 * -(-int(L) // bs) for L in seq_lens)
    return kv + qo + tab + 4 * len(seq_lens)


def kv_write_bytes(T, Hkv, d, e_in, e_cache):
    return 2 * T * Hkv * d * (e_in + e_cache) + 8 * T


def kernel_source_hash():
    """sha256 (first 16 hex digits) of the decode kernel's sources (the kernel file and the
    device helpers it includes) with comments and whitespace removed, so that edits to
    comments alone do not mark the counters as stale."""
    text = ""
    for path in KERNEL_SOURCES:
        with open(path) as f:
            text += f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary `path`, if it
    was taken with the current kernel source; else None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(seconds: float):
    """The float64 oracle (as it stands) on a bounded sample of the benchmark's work: one
    request of one layer at 4096 tokens, all 32 q heads, decoded repeatedly."""
    import numpy as np
    import workloads
    from oracle import attention as OA
    from oracle.allocator import Allocator as OAlloc

    w = workloads.gqa_uniform(B=1, L=4096, layers=1, seed_index=2, name="cpu_sample")
    vals = workloads.host_values(w)
    al = OAlloc(w.num_blocks, w.bs, w.free_order)
    slots = []
    for op in w.ops:
        if op[0] == "add":
            al.add(op[1])
        else:
            slots += al.append(op[1], op[2])[0]
    kc = np.zeros((w.num_blocks, w.Hkv, w.bs, w.d), np.uint16)
    vc = np.zeros_like(kc)
    OA.kv_write(vals["k_pre"], vals["v_pre"], np.array(slots), kc, vc, w.bs, "bf16")
    step = al.append_batch([0], [1])[0]
    OA.kv_write(vals["k_new"], vals["v_new"], np.array(step), kc, vc, w.bs, "bf16")
    t, L = al.block_table([0], w.max_blocks)
    scale = np.float32(1 / math.sqrt(w.d))
    per_call = decode_bytes(L, w.Hq, w.Hkv, w.d, w.bs, 2, 2)
    calls = 0
    c0, t0 = time.process_time(), time.perf_counter()
    while True:
        OA.decode(vals["q"], kc, vc, np.array(t), np.array(L), scale, w.bs, "bf16", "bf16")
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cpu = time.process_time() - c0
    return {
        "value": round(per_call * calls / el / 1e9, 4),
        "unit": "GB/s",
        "cores": max(1, round(cpu / el)),
        "kind": "oracle",
        "sample": f"{calls} float64 decodes of 1 request x 32 q heads x {int(L[0])} tokens (one layer of the "
                  f"benchmark batch's per-request work), {el:.1f} s wall, {cpu:.1f} s CPU, "
                  f"{len(os.sched_getaffinity(0))} host cores visible",
    }


# ----------------------------------------------------------------------------- GPU step

def report_phases(host_marks, evs, t0, t1, layers, phase_evs):
    """Where a timed step's time goes, on stderr: host microseconds per phase (allocator,
    staging the tables and slots, enqueueing the upload, the writes and the decodes) over the
    timed steps, the decodes' HIP-event microseconds over the timed steps, and the upload's, the
    writes' and the gap between one step's last decode and the next step's upload over the
    last warm-up steps, which carry those events (the timed steps carry only the decodes').  A
    gap means the device waited for the host; host enqueue times beyond the device's show where."""
    import statistics as st

    def us(x):
        return f"{st.mean(x):8.1f} {st.median(x):8.1f} {max(x):8.1f}"

    n = len(host_marks)
    ph = [[(m[k + 1] - m[k]) * 1e6 for m in host_marks] for k in range(5)]
    names = ["allocator", "stage tables", "upload enqueue", f"{layers} writes enqueue", f"{layers} decodes enqueue"]
    log(f"phase (us)               mean   median      max   over {n} timed steps")
    for nm, x in zip(names, ph):
        log(f"  host {nm:<18s}{us(x)}")
    g_up = [e[0].elapsed_time(e[1]) * 1e3 for e in phase_evs] or [0.0]
    g_wr = [e[1].elapsed_time(e[2]) * 1e3 for e in phase_evs] or [0.0]
    g_de = [e[2].elapsed_time(e[3]) * 1e3 for e in evs]
    gap = [phase_evs[i][3].elapsed_time(phase_evs[i + 1][0]) * 1e3 for i in range(len(phase_evs) - 1)] or [0.0]
    log(f"  gpu  upload            {us(g_up)}   (last {len(phase_evs)} warm-up steps)")
    log(f"  gpu  {layers} writes         {us(g_wr)}   (last {len(phase_evs)} warm-up steps)")
    log(f"  gpu  {layers} decodes        {us(g_de)}")
    log(f"  gpu  idle between steps{us(gap)}   (last {len(phase_evs)} warm-up steps)")
    busy = len(evs) * (st.mean(g_up) + st.mean(g_wr)) + sum(g_de)
    wall_ms, last_ms = (t1 - t0) * 1e3, (host_marks[-1][5] - t0) * 1e3
    # the host enqueues ahead of the device unless the last step is enqueued near the wall's end
    bound = "host-bound" if last_ms > 0.9 * wall_ms else "device-bound: the host ran ahead"
    log(f"  device busy {busy / 1e3:.3f} ms of {wall_ms:.3f} ms wall ({100 * busy / 1e3 / wall_ms:.1f}%); "
        f"host enqueue per step {st.mean([m[5] - m[0] for m in host_marks]) * 1e6:.1f} us; "
        f"last step enqueued at {last_ms:.3f} ms of the wall ({bound})")



def run(args):
    import numpy as np
    import torch

    from paged_kv_cache_408_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_kv_cache_408_amd as pk
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    steps, warm = args.steps, args.warmup
    L0 = 4096                      # decode length of every request in the first timed step
    grow = steps + warm
    w = workloads.gqa_uniform(B=16, L=L0 - warm, layers=32, spare_blocks=16 * (grow // 16 + 2))
    if args.placement == "identity":
        w.free_order = np.arange(w.num_blocks, dtype=np.int32)
    B, Hq, Hkv, d, bs, layers = w.B, w.Hq, w.Hkv, w.d, w.bs, w.layers
    max_blocks = -(-(L0 + grow) // bs)
    max_seq = max_blocks * bs
    scale = 1.0 / math.sqrt(d)
    log(f"workload {w.name}: {layers} layers x batch {B}, {Hq}q/{Hkv}kv, d {d}, block {bs}, "
        f"{w.num_blocks} blocks per layer")

    # allocator and prefill (L0 - warm - 1 tokens per request: the warmup steps append the next
    # warm tokens, and the first timed step appends token L0)
    alloc = pk.Allocator(w.num_blocks, bs, w.free_order)
    slots = []
    for op in w.ops:
        if op[0] == "add":
            alloc.add(op[1])
        else:
            slots.append(alloc.append(op[1], op[2])[0])
    slots = torch.from_numpy(np.concatenate(slots)).to(dev)
    T = slots.numel()
    kc, vc, q, kn, vn, outs = [], [], [], [], [], []
    for l in range(layers):
        k_cache = torch.empty((w.num_blocks, Hkv, bs, d), dtype=torch.bfloat16, device=dev)
        v_cache = torch.empty_like(k_cache)
        kp = workloads.device_normal(w, "k_pre", (T, Hkv, d), layer=l)
        vp = workloads.device_normal(w, "v_pre", (T, Hkv, d), layer=l)
        pk.pa_kv_write(kp, vp, slots, k_cache, v_cache)
        del kp, vp
        kc.append(k_cache)
        vc.append(v_cache)
        q.append(workloads.device_normal(w, "q", (B, Hq, d), layer=l))
        kn.append(workloads.device_normal(w, "k_new", (B, Hkv, d), layer=l))
        vn.append(workloads.device_normal(w, "v_new", (B, Hkv, d), layer=l))
        outs.append(torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    log(f"caches ready: {2 * layers * kc[0].numel() * 2 / 1e9:.2f} GB")

    # per-step device inputs: the step's table rows, lengths and new-token slots packed into one
    # pinned host buffer per step (no host write can race a copy still in flight) and moved by
    # one pa_upload kernel on the launch stream (no copy engine, no cross-queue wait)
    up16 = lambda x: (x + 15) // 16 * 16
    tab_bytes = B * max_blocks * 4
    len_off = up16(tab_bytes)
    slot_off = up16(len_off + 4 * B)
    pack = up16(slot_off + 8 * B)
    meta_d = torch.zeros(pack, dtype=torch.uint8, device=dev)
    tables_d = meta_d[:tab_bytes].view(torch.int32).view(B, max_blocks)
    lens_d = meta_d[len_off:len_off + 4 * B].view(torch.int32)
    slot_d = meta_d[slot_off:slot_off + 8 * B].view(torch.int64)
    staging = torch.zeros((grow, pack), dtype=torch.uint8).pin_memory()
    stage_np = staging.numpy()
    stage_tab = [stage_np[i, :tab_bytes].view(np.int32).reshape(B, max_blocks) for i in range(grow)]
    stage_len = [stage_np[i, len_off:len_off + 4 * B].view(np.int32) for i in range(grow)]
    stage_slot = [stage_np[i, slot_off:slot_off + 8 * B].view(np.int64) for i in range(grow)]
    nbytes = pk.pa_decode_workspace_bytes(B, Hq, Hkv, d, max_seq, args.partition_tokens, bs)
    part_used = pk.pa_decode_partition_tokens(B, Hkv, max_seq, args.partition_tokens, bs)
    log(f"split-K partitions of {part_used} tokens (requested {args.partition_tokens}; 0 = automatic)")
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    pk.pa_decode_workspace_init(ws)
    fused = args.step == "fused"

    def prepared(stream):
        if fused:   # each layer's write inside its decode launch (pa_decode_append)
            d_ = [pk.PreparedDecodeAppend(outs[l], q[l], kn[l], vn[l], kc[l], vc[l], tables_d, lens_d, scale, bs,
                                          max_seq_len=max_seq, workspace=ws, partition_tokens=args.partition_tokens,
                                          stream=stream) for l in range(layers)]
            return d_, []
        d_ = [pk.PreparedDecode(outs[l], q[l], kc[l], vc[l], tables_d, lens_d, scale, bs, max_seq_len=max_seq,
                                workspace=ws, partition_tokens=args.partition_tokens, stream=stream)
              for l in range(layers)]
        w_ = [pk.PreparedKVWrite(kn[l], vn[l], slot_d, kc[l], vc[l], stream=stream) for l in range(layers)]
        return d_, w_

    dec, wr = prepared(None)             # launches on the current stream
    seq_ids = list(range(B))
    ones = [1] * B

    def write_all():                     # each layer's new K/V first ...
        for l in range(len(wr)):
            wr[l]()

    def decode_all():                    # ... then the 32 decode launches back to back
        for l in range(layers):
            dec[l]()

    # per step: host timestamps [start, allocator done, tables and slots staged, upload enqueued,
    # writes enqueued, decodes enqueued] and, when timing, HIP events on the launch stream
    # [before the upload, after it, after the writes, after the decodes]
    host_marks = []

    def step(i, events=None, launch=(write_all, decode_all)):
        h0 = time.perf_counter()
        s, cow = alloc.batch_append(seq_ids, ones)
        h1 = time.perf_counter()
        alloc.block_tables(seq_ids, max_blocks, stage_tab[i], stage_len[i])
        stage_slot[i][:] = s
        h2 = time.perf_counter()
        if events is not None and events[0] is not None:
            events[0].record()
        pk.pa_upload(meta_d, staging[i])
        if cow:
            pairs = torch.tensor(cow, dtype=torch.int64).to(dev, non_blocking=False)
            for l in range(layers):
                pk.pa_copy_blocks(kc[l], vc[l], pairs)
        if events is not None and events[1] is not None:
            events[1].record()
        h3 = time.perf_counter()
        launch[0]()
        if events is not None and events[2] is not events[1]:
            events[2].record()
        h4 = time.perf_counter()
        launch[1]()
        if events is not None:
            events[3].record()
        h5 = time.perf_counter()
        host_marks.append((h0, h1, h2, h3, h4, h5))
        return stage_len[i].copy()

    # events per step: before the upload, after it, after the writes, after the decodes; with no
    # separate writes (the fused step) the after-upload event stands for the after-writes one.
    # The last warm-up steps carry all of them, for the report of where a step's device time goes;
    # the timed steps only the two around the decodes (the roofline's), so that no other event
    # sits in the timed region.
    def step_events(full):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        if not full:
            return (None, None, e[2], e[3])
        return (e[0], e[1], e[1] if fused else e[2], e[3])

    n_phase = min(3, warm)
    phase_evs = [step_events(True) for _ in range(n_phase)]
    for i in range(warm):
        step(i, phase_evs[i - (warm - n_phase)] if i >= warm - n_phase else None)
    torch.cuda.synchronize()
    launch = (write_all, decode_all)
    if args.graph:
        # the 32 writes and the 32 decodes of a step as two HIP graphs, replayed every step on
        # the same buffers (the step's tables, lengths and slots are uploaded into them first):
        # one launch per graph instead of 64 host calls.  The library's launches on the
        # capture stream are what the graphs hold; nothing in them allocates or clears memory.
        cap = torch.cuda.Stream()
        dec_c, wr_c = prepared(cap)
        g_write, g_decode = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        if wr_c:                         # the fused step has no separate writes
            with torch.cuda.graph(g_write, stream=cap, capture_error_mode="thread_local"):
                for l in range(len(wr_c)):
                    wr_c[l]()
        with torch.cuda.graph(g_decode, stream=cap, capture_error_mode="thread_local"):
            for l in range(layers):
                dec_c[l]()
        torch.cuda.synchronize()
        launch = (g_write.replay if wr_c else (lambda: None), g_decode.replay)
    log(f"warmup done ({warm} steps); timing {steps} steps ({'HIP graphs' if args.graph else 'host launches'})")

    evs = [step_events(False) for _ in range(steps)]
    lens_per_step = []
    host_marks.clear()
    torch.cuda.synchronize()
    with gc_held():
        t0 = time.perf_counter()
        for i in range(steps):
            lens_per_step.append(step(warm + i, evs[i], launch))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    wall = t1 - t0
    log(f"timed {steps} steps in {wall * 1e3:.2f} ms")
    report_phases(host_marks, evs, t0, t1, layers, phase_evs)
    if args.graph:
        # the graphs' last outputs against eager launches on the same inputs: bit for bit
        # (decode is deterministic; the write of the same rows again changes nothing)
        got = [outs[l].clone() for l in (0, layers - 1)]
        write_all()
        decode_all()
        torch.cuda.synchronize()
        for g_out, l in zip(got, (0, layers - 1)):
            if not torch.equal(g_out.view(torch.int16), outs[l].view(torch.int16)):
                raise RuntimeError(f"graph replay of layer {l} differs from an eager decode")
        log("graph outputs of the last step equal eager launches (layers 0 and 31)")

    # HIP events on the launch stream around each step's 32 back-to-back decode launches
    dec_ms = [e[2].elapsed_time(e[3]) / layers for e in evs for _ in range(layers)]
    # a fused launch also moves its layer's write (the new rows read and written; no slots)
    wbytes = 2 * B * Hkv * d * (2 + 2) if fused else 0
    dec_bytes = [decode_bytes(L, Hq, Hkv, d, bs, 2, 2) + wbytes for L in lens_per_step for _ in range(layers)]
    step_bytes = sum(dec_bytes) + (0 if fused else steps * layers * kv_write_bytes(B, Hkv, d, 2, 2))
    value = step_bytes / wall / 1e9
    avg_launch_s = sum(dec_ms) / len(dec_ms) / 1e3
    avg_bytes = sum(dec_bytes) / len(dec_bytes)
    achieved = avg_bytes / avg_launch_s / 1e9
    traffic = measured_traffic(TRAFFIC_FILE_FUSED if fused else TRAFFIC_FILE)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(wall / steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)*0.5 K/V/q drawn on the device; %s)" % (
            "seeded block permutation" if args.placement == "permuted" else "identity block placement"),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "config": {
            "workload": "llama3_8b_gqa_decode: 32 layers x batch 16, 32 q / 8 kv heads, head_dim 128, bf16, "
                        "block 16, 4096 tokens per request at the first timed step (+1 per step), "
                        "split-K partitions of %d tokens" % part_used,
            "layers": layers, "batch": B, "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": d,
            "block_size": bs, "seq_len_start": int(lens_per_step[0][0]), "seq_len_end": int(lens_per_step[-1][0]),
            "partition_tokens": part_used, "placement": args.placement,
            "kv_cache_gb": round(2 * layers * kc[0].numel() * 2 / 1e9, 3),
            "launch": "two HIP graphs per step" if args.graph else "one host launch per kernel",
            "step": "pa_decode_append (each layer's KV write inside its decode launch)" if fused else
                    "pa_kv_write then pa_decode per layer (writes first)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": DECODE_KERNEL + (" (with the layer's KV write: pa_decode_append)" if fused else ""),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": int(round(avg_bytes)),
            "avg_launch_us": round(avg_launch_s * 1e6, 3),
            "launches": len(dec_ms),
        },
    }
    return result


# ----------------------------------------------------------------------------- other workloads

def run_workload(name, args):
    """One decode step of a non-default workload, timed: the step token's pa_kv_write, then
    pa_decode, repeated on the same state (step_gbps from the wall time); then pa_decode alone,
    8 back-to-back launches between HIP events, for the kernel's time.  Prints one JSON line
    per setting (these are measurements for the record, not the benchmark line)."""
    import numpy as np
    import torch

    from paged_kv_cache_408_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_kv_cache_408_amd as pk
    import workloads

    dev = torch.device("cuda:0")
    if name == "ragged_prefix":
        settings = [workloads.ragged_prefix(bs=16)]
    elif name == "long_context":
        settings = [workloads.long_context()]
    elif name == "mxfp4":   # the 4-bit cache on the ragged batch and on one Llama-shaped layer
        settings = [workloads.ragged_prefix(bs=16, fmt="mxfp4"),
                    workloads.gqa_uniform(B=16, L=4096, fmt="mxfp4", layers=1, name="llama3_8b_layer_mxfp4")]
    elif name == "fp8":     # the fp8 cache on the ragged batch and on one Llama-shaped layer
        settings = [workloads.ragged_prefix(bs=16, fmt="fp8"),
                    workloads.gqa_uniform(B=16, L=4096, fmt="fp8", layers=1, name="llama3_8b_layer_fp8")]
    elif name == "llama_layer":   # one layer of the benchmark batch on its own
        settings = [workloads.gqa_uniform(B=16, L=4096, layers=1, name="llama3_8b_layer_bf16")]
    else:  # block-size x KV-dtype sweep on the ragged batch
        settings = [workloads.ragged_prefix(bs=bs, fmt=fmt) for bs, fmt in workloads.sweep_settings()]
    for w in settings:
        if args.placement == "identity":
            w.free_order = np.arange(w.num_blocks, dtype=np.int32)
        alloc = pk.Allocator(w.num_blocks, w.bs, w.free_order)
        slots = []
        for op in w.ops:
            if op[0] == "add":
                alloc.add(op[1])
            elif op[0] == "append":
                slots.append(alloc.append(op[1], op[2])[0])
            elif op[0] == "fork":
                alloc.fork(op[1], op[2])
            elif op[0] == "free":
                alloc.free(op[1])
        slots = torch.from_numpy(np.concatenate(slots)).to(dev)
        if w.fmt == "mxfp4":
            kc = pk.mxfp4_cache(w.num_blocks, w.Hkv, w.bs, w.d, dev)
        else:
            cdt = torch.uint8 if w.fmt == "fp8" else torch.bfloat16
            kc = torch.zeros((w.num_blocks, w.Hkv, w.bs, w.d), dtype=cdt, device=dev)
        vc = torch.zeros_like(kc)
        kp = workloads.device_normal(w, "k_pre", (slots.numel(), w.Hkv, w.d))
        vp = workloads.device_normal(w, "v_pre", (slots.numel(), w.Hkv, w.d))
        kn = workloads.device_normal(w, "k_new", (w.B, w.Hkv, w.d))
        vn = workloads.device_normal(w, "v_new", (w.B, w.Hkv, w.d))
        ks = vs = None
        if w.fmt == "fp8":   # per-head amax / 448 over the head's values
            ks = (torch.maximum(kp.float().abs().amax(dim=(0, 2)), kn.float().abs().amax(dim=(0, 2))) / 448).contiguous()
            vs = (torch.maximum(vp.float().abs().amax(dim=(0, 2)), vn.float().abs().amax(dim=(0, 2))) / 448).contiguous()
        pk.pa_kv_write(kp, vp, slots, kc, vc, k_scale=ks, v_scale=vs)
        del kp, vp
        step_slots, cow = alloc.batch_append(list(range(w.B)), [1] * w.B)
        assert not cow
        step_slots = torch.from_numpy(step_slots).to(dev)
        tab, lens = alloc.block_tables(list(range(w.B)), w.max_blocks)
        tables, lens_d = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
        q = workloads.device_normal(w, "q", (w.B, w.Hq, w.d))
        out = torch.empty_like(q)
        maxL = int(lens.max())
        nbytes = pk.pa_decode_workspace_bytes(w.B, w.Hq, w.Hkv, w.d, maxL, args.partition_tokens, w.bs, kc)
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        dec = pk.PreparedDecode(out, q, kc, vc, tables, lens_d, 1.0 / math.sqrt(w.d), w.bs, max_seq_len=maxL,
                                workspace=ws if nbytes else None, k_scale=ks, v_scale=vs,
                                partition_tokens=args.partition_tokens)
        wr = pk.PreparedKVWrite(kn, vn, step_slots, kc, vc, k_scale=ks, v_scale=vs)
        for _ in range(max(args.warmup, 1)):
            wr()
            dec()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        with gc_held():
            t0 = time.perf_counter()
            for e0, e1 in evs:
                wr()
                e0.record()
                dec()
                e1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
        single_us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
        # the kernel's own time: events around back-to-back launches on the same state (as the
        # headline times its 32 layers); events around one launch also hold its dispatch
        rep = 8
        evb = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for e0, e1 in evb:
            e0.record()
            for _ in range(rep):
                dec()
            e1.record()
        torch.cuda.synchronize()
        dec_us = sorted(e0.elapsed_time(e1) * 1e3 / rep for e0, e1 in evb)
        med = dec_us[len(dec_us) // 2]
        e = {"fp8": 1, "mxfp4": 17 / 32}.get(w.fmt, 2)   # mxfp4: d / 2 code bytes + d / 32 scale bytes per row
        logical = decode_bytes(lens, w.Hq, w.Hkv, w.d, w.bs, e, 2) + (2 * w.Hkv * 4 if w.fmt == "fp8" else 0)
        st = alloc.stats()
        unique_kv = int(st["used_blocks"] * 2 * w.Hkv * w.bs * w.d * e)
        waste = int(sum(-(-int(L) // w.bs) * w.bs - int(L) for L in lens))
        reserved = int(sum(-(-int(L) // w.bs) * w.bs for L in lens))
        step_bytes = logical + kv_write_bytes(w.B, w.Hkv, w.d, 2, e)
        print(json.dumps({
            "workload": w.name, "metric": "decode attention KV GB/s", "unit": "GB/s", "placement": args.placement,
            "decode_us_median": round(med, 3), "decode_us_min": round(dec_us[0], 3),
            "decode_timing": "HIP events around %d back-to-back launches, median over %d" % (rep, args.steps),
            "decode_us_single_launch_median": round(single_us[len(single_us) // 2], 3),
            "logical_gbps": round(logical / med / 1e3, 1),
            "unique_kv_gbps": round(unique_kv / med / 1e3, 1),
            "pct_of_hbm_peak_logical": round(100 * logical / med / 1e3 / HBM_PEAK_GBPS, 2),
            "step_gbps": round(step_bytes * args.steps / wall / 1e9, 1),
            "algorithmic_bytes": int(logical), "unique_kv_bytes": int(unique_kv),
            "batch": w.B, "num_q_heads": w.Hq, "num_kv_heads": w.Hkv, "head_dim": w.d, "block_size": w.bs,
            "kv_dtype": w.fmt, "max_seq_len": maxL, "total_tokens": int(lens.sum()),
            "partition_tokens": pk.pa_decode_partition_tokens(w.B, w.Hkv, maxL, args.partition_tokens, w.bs, kc),
            "final_block_waste_slots": waste, "final_block_waste_pct": round(100 * waste / reserved, 3),
            "contiguous_waste_pct": round(100 * (w.B * max(8192, maxL) - int(lens.sum())) / (w.B * max(8192, maxL)), 2),
            "contiguous_reservation_tokens": max(8192, maxL),
            "steps": args.steps,
        }), flush=True)
        del kc, vc, ws, dec, wr
        torch.cuda.empty_cache()


HOST_LINK_PEAK_GBPS = 64.0   # PCIe 5.0 x16, one direction (32 GT/s x 16 lanes, 128b/130b)


def run_swap(args):
    """Preemption by swapping on the ragged batch (256 requests, bf16, block 16): the 192
    requests without the shared prefix are swapped out to a pinned host pool and back in,
    `steps` times.  Timed with HIP events on the launch stream: each pa_swap_blocks launch
    (device -> host, then host -> device); on the host: the allocator's pa_swap_out /
    pa_swap_in.  For reference, the HIP runtime's own rate for one contiguous buffer of the
    same size in each direction (torch copy_ between device and pinned memory)."""
    import numpy as np
    import torch

    from paged_kv_cache_408_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_kv_cache_408_amd as pk
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.ragged_prefix(bs=16)
    alloc = pk.Allocator(w.num_blocks, w.bs, w.free_order)
    slots = []
    for op in w.ops:
        if op[0] == "add":
            alloc.add(op[1])
        elif op[0] == "append":
            slots.append(alloc.append(op[1], op[2])[0])
        elif op[0] == "fork":
            alloc.fork(op[1], op[2])
        elif op[0] == "free":
            alloc.free(op[1])
    slots = torch.from_numpy(np.concatenate(slots)).to(dev)
    kc = torch.zeros((w.num_blocks, w.Hkv, w.bs, w.d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    pk.pa_kv_write(workloads.device_normal(w, "k_pre", (slots.numel(), w.Hkv, w.d)),
                   workloads.device_normal(w, "v_pre", (slots.numel(), w.Hkv, w.d)), slots, kc, vc)
    victims = list(range(64, w.B))
    nh = sum(-(-int(w.seq_lens[b]) // w.bs) for b in victims) + 16
    alloc.set_host_blocks(nh)
    hk = torch.empty((nh, w.Hkv, w.bs, w.d), dtype=torch.bfloat16).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    block = w.Hkv * w.bs * w.d * 2
    out_us, in_us, host_out_us, host_in_us, npairs = [], [], [], [], 0
    stream = torch.cuda.current_stream()
    for it in range(max(args.warmup, 1) + args.steps):
        t0 = time.perf_counter()
        p_out = alloc.swap_out(victims)
        t1 = time.perf_counter()
        pd_out = torch.from_numpy(p_out).to(dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        pk.pa_swap_blocks(hk, hv, kc, vc, pd_out)
        e[1].record(stream)
        t2 = time.perf_counter()
        p_in = alloc.swap_in(victims)
        t3 = time.perf_counter()
        pd_in = torch.from_numpy(p_in).to(dev)
        e[2].record(stream)
        pk.pa_swap_blocks(kc, vc, hk, hv, pd_in)
        e[3].record(stream)
        torch.cuda.synchronize()
        if it >= max(args.warmup, 1):
            out_us.append(e[0].elapsed_time(e[1]) * 1e3)
            in_us.append(e[2].elapsed_time(e[3]) * 1e3)
            host_out_us.append((t1 - t0) * 1e6)
            host_in_us.append((t3 - t2) * 1e6)
            npairs = len(p_out)
    nbytes = 2 * npairs * block
    # the runtime's copy of one contiguous buffer of the same size, each direction
    dbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    hbuf = torch.empty(nbytes, dtype=torch.uint8).pin_memory()
    ce = {"d2h": [], "h2d": []}
    for it in range(3 + args.steps // 2):
        for name, (dst, src) in (("d2h", (hbuf, dbuf)), ("h2d", (dbuf, hbuf))):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            dst.copy_(src, non_blocking=True)
            b.record(stream)
            torch.cuda.synchronize()
            if it >= 3:
                ce[name].append(a.elapsed_time(b) * 1e3)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    for name, us, hus, cus in (("swap_out_device_to_host", out_us, host_out_us, ce["d2h"]),
                               ("swap_in_host_to_device", in_us, host_in_us, ce["h2d"])):
        m = med(us)
        print(json.dumps({
            "workload": f"{w.name}: {name}", "metric": "swapped KV GB/s", "unit": "GB/s",
            "requests": len(victims), "block_pairs": npairs, "bytes": nbytes,
            "kernel_us_median": round(m, 2), "gbps": round(nbytes / m / 1e3, 2),
            "pct_of_host_link_peak": round(100 * nbytes / m / 1e3 / HOST_LINK_PEAK_GBPS, 1),
            "host_link_peak_gbps": HOST_LINK_PEAK_GBPS,
            "runtime_copy_contiguous_gbps": round(nbytes / med(cus) / 1e3, 2),
            "allocator_us_median": round(med(hus), 1), "steps": args.steps,
        }), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def prefill_flops(ctx_lens, n_new, Hq, d):
    """Algorithmic flops of causal prefill: for every (new token, visible position, q head)
    one d-long dot product (q.k) and one d-long weighted add (p.v), 2 flops per element each."""
    pairs = sum(n * c + n * (n + 1) // 2 for c, n in zip(ctx_lens, n_new))
    return 4 * d * Hq * pairs


def run_prefill(args):
    """Causal paged prefill, Llama-3-8B shape (32 q / 8 KV heads, head_dim 128, bf16, block
    16) on seeded synthetic K/V and q in a seeded-permutation pool: 16 requests x (1024 cached
    + 1024 new tokens) (a chunk after a prefix-cache hit), 4 x 4096 new tokens with no context
    and 1 x 16384; the first shape also over an fp8 cache (random codes, per-head scale 0.01)
    and a 4-bit MXFP4 cache (random codes, block scale 2^-7).  Each case is run warmup + steps
    times; pa_prefill is timed with HIP events on the launch stream (median); flops are the
    algorithmic ones (visible pairs only)."""
    import numpy as np
    import torch

    from paged_kv_cache_408_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_kv_cache_408_amd as pk

    dev = torch.device("cuda:0")
    Hq, Hkv, d, bs = 32, 8, 128, 16
    def cache(fmt, N, g):
        if fmt == "bf16":
            return (torch.randn((N, Hkv, bs, d), generator=g, device=dev) * 0.5).to(torch.bfloat16)
        if fmt == "fp8":        # codes 0x00..0x7D and their negatives: no NaN code
            c = torch.randint(0, 0x7E, (N, Hkv, bs, d), generator=g, device=dev, dtype=torch.int32)
            sign = torch.randint(0, 2, (N, Hkv, bs, d), generator=g, device=dev, dtype=torch.int32) << 7
            return (c | sign).to(torch.uint8)
        c = pk.mxfp4_cache(N, Hkv, bs, d, dev)
        flat = c.view(N, Hkv, -1)
        ncode = bs * d // 2
        flat[:, :, :ncode] = torch.randint(0, 256, (N, Hkv, ncode), generator=g, device=dev,
                                           dtype=torch.int32).to(torch.uint8)
        flat[:, :, ncode:] = 120
        return c

    cases = [(16, 1024, 1024, "bf16"), (4, 0, 4096, "bf16"), (1, 0, 16384, "bf16"),
             (16, 1024, 1024, "fp8"), (16, 1024, 1024, "mxfp4")]
    for B, ctx, n, fmt in cases:
        L = ctx + n
        nb = -(-L // bs)
        N = B * nb + 16
        g = torch.Generator(device=dev)
        g.manual_seed(408_300 + B)
        kc, vc = cache(fmt, N, g), cache(fmt, N, g)
        kw = {}
        if fmt == "fp8":
            kw = dict(k_scale=torch.full((Hkv,), 0.01, device=dev), v_scale=torch.full((Hkv,), 0.01, device=dev))
        perm = torch.from_numpy(np.random.Generator(np.random.PCG64(np.random.SeedSequence(408_301))).permutation(N)[: B * nb])
        tab = perm.reshape(B, nb).to(torch.int32).to(dev)
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        qs = (torch.arange(B + 1, dtype=torch.int32) * n).to(dev)
        q = (torch.randn((B * n, Hq, d), generator=g, device=dev) * 0.5).to(torch.bfloat16)
        out = torch.empty_like(q)
        call = lambda: pk.pa_prefill(out, q, kc, vc, tab, lens, qs, 1 / math.sqrt(d), bs, max_query_len=n, max_seq_len=L, **kw)
        for _ in range(max(args.warmup, 1)):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b2 in ev:
            a.record()
            call()
            b2.record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b2) * 1e3 for a, b2 in ev)
        med = us[len(us) // 2]
        fl = prefill_flops([ctx] * B, [n] * B, Hq, d)
        print(json.dumps({
            "workload": f"prefill {B} x ({ctx} cached + {n} new), 32 q / 8 kv heads, d 128, {fmt} cache, block 16",
            "metric": "causal prefill TFLOP/s", "unit": "TFLOP/s", "kernel": "prefill_kernel",
            "us_median": round(med, 2), "us_min": round(us[0], 2), "algorithmic_flops": int(fl),
            "tflops": round(fl / med / 1e6, 1), "pct_of_bf16_mfma_peak": round(100 * fl / med / 1e6 / MFMA_BF16_PEAK_TFLOPS, 2),
            "steps": args.steps,
        }), flush=True)
        del kc, vc, q, out
        torch.cuda.empty_cache()


def run_prefix_cache(args):
    """The ragged batch's prompts (256 requests, bf16, block 16, 32 q / 8 KV heads, d 128;
    64 of them start with one 1024-token system prompt) arriving one after another, with
    synthetic token ids, through the prefix cache (pa_seq_add_prompt) and without it
    (pa_seq_add + pa_seq_append).  Reported per run: host allocator time per prompt, prompt
    tokens whose K/V the cache already held, K/V bytes written, and the device time of the
    prefill write (one pa_kv_write of every row that has to be written, HIP events)."""
    import numpy as np
    import torch

    from paged_kv_cache_408_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_kv_cache_408_amd as pk
    import workloads

    dev = torch.device("cuda:0")
    w = workloads.ragged_prefix(bs=16)
    lens, _ = workloads.ragged_lengths(w.seed_index)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(408_200)))
    system = g.integers(0, 32000, size=1024).astype(np.int32)
    prompts = []
    for b in range(w.B):
        L = int(lens[b]) - 1                       # the decode token comes later
        own = g.integers(0, 32000, size=L).astype(np.int32)
        prompts.append(np.concatenate([system, own[1024:]]) if b < 64 else own)
    total = int(sum(len(p) for p in prompts))
    row_bytes = 2 * w.Hkv * w.d * 2                # K and V of one token, bf16
    n_blocks = sum(-(-len(p) // w.bs) for p in prompts) + 256   # room for the run without sharing
    order = np.random.Generator(np.random.PCG64(np.random.SeedSequence(408_201))).permutation(n_blocks)
    kc = torch.zeros((n_blocks, w.Hkv, w.bs, w.d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    kv_rows = workloads.device_normal(w, "k_pre", (total, w.Hkv, w.d))
    for cached in (True, False):
        host_us, slots_all, n_hit = [], [], 0
        for rep_i in range(max(args.warmup, 1) + args.steps):
            al = pk.Allocator(n_blocks, w.bs, order)
            slots_all, n_hit, t_total = [], 0, 0.0
            for b, toks in enumerate(prompts):
                t0 = time.perf_counter()
                if cached:
                    nc, sl = al.add_prompt(b, toks)
                else:
                    al.add(b)
                    sl, _ = al.append(b, len(toks))
                    nc = 0
                t_total += time.perf_counter() - t0
                n_hit += nc
                slots_all.append(sl)
            host_us.append(t_total * 1e6 / w.B)
        slots = torch.from_numpy(np.concatenate(slots_all)).to(dev)
        n_write = slots.numel()
        kr, vr = kv_rows[:n_write], kv_rows[:n_write]
        ev = []
        for rep_i in range(max(args.warmup, 1) + args.steps):
            a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            pk.pa_kv_write(kr, vr, slots, kc, vc)
            b2.record()
            ev.append((a, b2))
        torch.cuda.synchronize()
        wr_us = sorted(a.elapsed_time(b2) * 1e3 for a, b2 in ev[max(args.warmup, 1):])
        st = al.stats()
        print(json.dumps({
            "workload": f"{w.name} prompts {'with' if cached else 'without'} the prefix cache",
            "metric": "prefill K/V written", "unit": "bytes",
            "requests": w.B, "prompt_tokens": total, "tokens_from_cache": int(n_hit),
            "tokens_written": int(n_write), "kv_bytes_written": int(n_write * row_bytes),
            "kv_bytes_saved": int(n_hit * row_bytes),
            "used_blocks": st["used_blocks"], "cached_blocks": st["cached_blocks"],
            "allocator_us_per_prompt": round(sorted(host_us)[len(host_us) // 2], 2),
            "prefill_write_us": round(wr_us[len(wr_us) // 2], 2), "steps": args.steps,
        }), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--workload", default="llama3_8b",
                    choices=["llama3_8b", "ragged_prefix", "long_context", "sweep", "mxfp4", "fp8", "llama_layer",
                             "swap", "prefix_cache", "prefill", "read_ceiling"],
                    help="llama3_8b: the benchmark; the others print per-setting measurements instead")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--partition-tokens", type=int, default=0, help="split-K partition size; 0 = automatic")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step", default="fused", choices=["separate", "fused"],
                    help="default workload: each layer's KV write inside its decode launch (pa_decode_append), "
                         "or as its own launch before the decodes (pa_kv_write, then pa_decode)")
    ap.add_argument("--placement", default="permuted", choices=["permuted", "identity"],
                    help="physical block order: a seeded permutation (scattered blocks), or identity (each "
                         "request's blocks contiguous and in logical order: the indirection's cost is the difference)")
    ap.add_argument("--graph", action="store_true",
                    help="default workload: replay each step's writes and decodes from two HIP graphs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run pa_copy_blocks over 1 GiB of blocks (write-counter calibration)")
    ap.add_argument("--calibrate-read", action="store_true",
                    help="only run a reduction that reads 1 GiB (read-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_read:
        calibrate_read()
        return
    if args.workload == "swap":
        run_swap(args)
        return
    if args.workload == "prefix_cache":
        run_prefix_cache(args)
        return
    if args.workload == "prefill":
        run_prefill(args)
        return
    if args.workload == "read_ceiling":
        run_read_ceiling(args)
        return
    if args.workload != "llama3_8b":
        run_workload(args.workload, args)
        return
    result = run(args)
    if not args.no_cpu_baseline:
        log(f"timing the oracle on the host for ~{args.cpu_seconds:.0f} s")
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def decode_tile_order(w, part_tokens):
    """The 4 KiB (block, KV head) tiles the uniform-grid decode reads, per work-group, in pass
    order: work-group j = part + parts * (g + Hkv * b) reads, for each 16-token pass of its
    partition, the K tile then the V tile of block table[b][...] and head g.  Tile indices count
    K tiles from 0 and V tiles from num_blocks * Hkv (the probe's buffer holds the K cache, then
    the V cache).  Every request has the same length and the partitions split it evenly."""
    import numpy as np
    alloc = pk_allocator(w)
    tab, lens = alloc.block_tables(list(range(w.B)), w.max_blocks)
    L = int(lens[0])
    assert (lens == L).all() and L % part_tokens == 0 and part_tokens % w.bs == 0
    parts, per = L // part_tokens, part_tokens // w.bs
    order = []
    for b in range(w.B):
        for g in range(w.Hkv):
            for part in range(parts):
                blocks = tab[b, part * per:(part + 1) * per].astype(np.int64)
                kt = blocks * w.Hkv + g
                order.append(np.stack([kt, kt + w.num_blocks * w.Hkv], 1).reshape(-1))
    # grid order of the work-groups: x = part fastest, then y = g, then z = b
    return np.concatenate(order).astype(np.int32)


def pk_allocator(w):
    import paged_kv_cache_408_amd as pk
    alloc = pk.Allocator(w.num_blocks, w.bs, w.free_order)
    for op in w.ops:
        if op[0] == "add":
            alloc.add(op[1])
        else:
            alloc.append(op[1], op[2])
    alloc.batch_append(list(range(w.B)), [1] * w.B)
    return alloc


def run_read_ceiling(args):
    """The decode's rate beside plain streaming reads of the same memory (pa_probe_read: every
    byte loaded once, nothing written, one four-wave work-group per compute unit).  32 layers of
    the Llama-shaped cache at 4096 tokens, each layer's K and V caches in one allocation (K
    first), the benchmark's seeded block tables; every case runs back to back over the 32
    layers in turn (nothing stays in the last-level cache between launches), timed with HIP
    events:
      - pa_decode of each layer (automatic partitions);
      - tiles, the decode's order: the K and V tiles of every pass the decode reads, split over
        work-groups and waves as the decode splits them, moved to LDS with no arithmetic;
      - ranges: each work-group its own contiguous range of the layer's tiles;
      - grid: a grid-stride sweep of the layer's K and V caches; and of one 4 GiB buffer.
    A reference for the decode's rate, not a benchmark line."""
    import math
    import numpy as np
    import torch
    import paged_kv_cache_408_amd as pk
    import workloads
    dev = torch.device("cuda:0")
    w = workloads.gqa_uniform(B=16, L=4096, layers=1, name="read_ceiling")
    N, Hkv, bs, d = w.num_blocks, w.Hkv, w.bs, w.d
    L = 4096
    pt = pk.pa_decode_partition_tokens(w.B, Hkv, L, 0, bs)
    alloc = pk_allocator(w)
    tab, lens = alloc.block_tables(list(range(w.B)), w.max_blocks)
    tables, lens_d = torch.from_numpy(tab).to(dev), torch.from_numpy(lens).to(dev)
    order = torch.from_numpy(decode_tile_order(w, pt)).to(dev)
    layers = [torch.zeros((2, N, Hkv, bs, d), dtype=torch.bfloat16, device=dev) for _ in range(32)]
    flat = [t.view(-1) for t in layers]
    q = torch.zeros((w.B, w.Hq, d), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(q)
    ws = torch.zeros(max(pk.pa_decode_workspace_bytes(w.B, w.Hq, Hkv, d, L, 0, bs), 256), dtype=torch.uint8, device=dev)
    decs = [pk.PreparedDecode(out, q, t[0], t[1], tables, lens_d, 1 / math.sqrt(d), bs, max_seq_len=L, workspace=ws)
            for t in layers]
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    dec_bytes = decode_bytes([L] * w.B, w.Hq, Hkv, d, bs, 2, 2)
    log(f"32 layers of {2 * N * Hkv * bs * d * 2} bytes; the decode reads {order.numel()} tiles of 4 KiB per layer "
        f"({pt}-token partitions)")

    def timed(fn, n=32, reps=64):
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                fn(i % n)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / reps)
        return sorted(times)[len(times) // 2]

    def report(name, moved, us):
        print(json.dumps({"workload": "read_ceiling", "case": name, "bytes": moved, "us_per_launch": round(us, 2),
                          "GB_s": round(moved / us / 1e3, 1), "pct_of_8000": round(moved / us / 1e3 / 80, 1)}), flush=True)

    report("pa_decode (algorithmic bytes)", dec_bytes, timed(lambda i: decs[i]()))
    report("tiles, the decode's order", order.numel() * 4096,
           timed(lambda i: pk.pa_probe_read(flat[i], sink, pattern=pk.PA_PROBE_TILES, tile_order=order)))
    report("ranges, the layer's K and V", flat[0].numel() * 2,
           timed(lambda i: pk.pa_probe_read(flat[i], sink, pattern=pk.PA_PROBE_RANGES)))
    report("grid, the layer's K and V", flat[0].numel() * 2,
           timed(lambda i: pk.pa_probe_read(flat[i], sink, pattern=pk.PA_PROBE_GRID)))
    report("pa_decode again", dec_bytes, timed(lambda i: decs[i]()))
    del layers, flat, decs
    torch.cuda.empty_cache()
    big = torch.zeros(1 << 30, dtype=torch.float32, device=dev)
    report("grid, one 4 GiB buffer", 4 << 30, timed(lambda i: pk.pa_probe_read(big, sink), n=1, reps=10))


def calibrate_copy():
    """A plain copy of known size for scaling the HBM byte counters: pa_copy_blocks over
    8192 block pairs of 64 KiB in each of K and V (512 MiB read, 512 MiB written per launch),
    5 launches."""
    import torch
    import paged_kv_cache_408_amd as pk
    dev = torch.device("cuda:0")
    N, Hkv, bs, d = 16384, 8, 16, 128
    kc = torch.zeros((N, Hkv, bs, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    src = torch.arange(0, N // 2, dtype=torch.int64)
    pairs = torch.stack([src, src + N // 2], 1).to(dev)
    for _ in range(5):
        pk.pa_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    block = Hkv * bs * d * 2
    print(json.dumps({"copy_read_bytes_per_launch": 2 * (N // 2) * block,
                      "copy_write_bytes_per_launch": 2 * (N // 2) * block, "launches": 5}), flush=True)


def calibrate_read():
    """A plain read of known size for scaling the HBM fetch counter: a float32 sum over 1 GiB
    (read once, a few bytes written), 5 launches."""
    import torch
    dev = torch.device("cuda:0")
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    for _ in range(5):
        x.sum()
    torch.cuda.synchronize()
    print(json.dumps({"read_bytes_per_launch": x.numel() * 4, "launches": 5}), flush=True)


if __name__ == "__main__":
    main()
