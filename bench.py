#!/usr/bin/env python3
"""Benchmark of the indexer top-k path on one MI355X.

A step is one pass of the whole path over one batch: the planning kernel
(topk_plan) followed by the fused selection + page-table kernel
(topk_select_paged). The headline workload is 7 rows x 1,000,000 FP32 scores,
k = 2048, 64-token pages (the 1M-context target-verify batch of the lmsys.org
TopK-V2 section, Figure 4); the 7 x 80,000 batch (its 80K point) is timed in
the same run and reported beside it.

Inputs are resident in HBM before timing starts, and each step reads a
different copy out of a rotation of at least 512 MB (twice the 256 MB
Infinity Cache), so the scores come from HBM rather than cache. Prints one
JSON line (``--sweep`` prints one per workload instead).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TopK latency (µs) at 7×80K and 7×1M, k=2048; HBM GB/s vs peak"
PEAK_HBM_GBS = 8000.0
PAGES_V2_US = {"7x1m": 36.6, "7x80k": 17.5}   # the page's TopK-V2 latencies (B300; context only)
ROTATION_BYTES = 512 << 20
IN_KERNEL_PLAN_ROWS = 512      # batches this small are planned inside topk_select_paged
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "topk_select_kernel_7x1m_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "sparse_attention_indexer_amd", "csrc", f)
                  for f in ("topk_kernels.hip", "topk_device.hpp", "topk_layout.hpp", "topk_plan.hpp")]

DESCRIPTIONS = {
    "7x1m": "7x1M k=2048: 7 rows x 1,000,000 FP32 scores ~N(0,1), 1% in [3.0,3.0005), "
            "64-token pages, shared random page permutation",
    "7x80k": "7x80K k=2048: 7 rows x 80,000 FP32 scores (30% exact zeros, rest 2|N(0,1)|), "
             "valid length 79,994+r, -inf tail, 64-token pages, shared random page permutation",
}


HOST_THREADS_MAX = 16   # CPU share of one GPU on the measurement host, whatever nproc reports


def host_threads(rows: int) -> int:
    """Oracle threads for a batch: one row range each, at most the host share."""
    return max(1, min(rows, HOST_THREADS_MAX, os.cpu_count() or 1))


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def workload(name: str):
    import synth
    table = {"7x1m": 3, "7x80k": 2, "c1": 1, "c2": 2, "c3": 3, "c4": 4, "c5": 5}
    if name == "cp8_7x125k":
        return synth.make_cp_shard()
    if name == "prefill_4096x80k":
        return synth.make_prefill()
    if name == "plan_split_600":
        return synth.make_plan_split()
    if name.startswith("c5_g"):
        # one 64-row group of C5 (0 one value, 1 sixteen values, 2 one FP16
        # bin, 3 sorted descending), run on the full batch's path (one
        # workgroup per row): its share of the C5 time
        g = int(name[4:])
        w = synth.make_config(5)
        rows = slice(64 * g, 64 * (g + 1))
        return synth.Workload(f"c5_group{g}", w.scores[rows], w.lengths[rows], w.block_table[rows],
                              w.bt_row_stride, w.page_size, w.k, w.seed)
    return synth.make_config(table[name])


def path_of(name: str) -> str:
    """The path a workload is timed on: C5's groups alone would be split, so
    they keep the whole batch's one workgroup per row."""
    return "single" if name.startswith("c5_g") else "auto"


def row_sample(w, rows: int):
    """The first `rows` rows of a workload (a bounded sample for the oracle)."""
    import synth
    if rows >= w.rows:
        return w
    bt = w.block_table if w.bt_row_stride == 0 else w.block_table[:rows]
    return synth.Workload(w.name + f"_first{rows}", w.scores[:rows], w.lengths[:rows], bt,
                          w.bt_row_stride, w.page_size, w.k, w.seed)


def algorithmic_bytes(w, slots, with_idx: bool) -> int:
    """Scores read once, lengths, distinct block-table entries touched by the
    selected positions (a shared table counted once), and the outputs."""
    import numpy as np
    n_scores = int(np.minimum(w.lengths, w.stride).astype(np.int64).sum())
    valid = slots >= 0
    pages = slots // w.page_size
    if w.bt_row_stride == 0:
        n_table = int(np.unique(pages[valid]).size)
    else:
        n_table = sum(int(np.unique(pages[r][valid[r]]).size) for r in range(w.rows))
    outputs = w.rows * w.k * (8 if with_idx else 4)
    return 4 * n_scores + 4 * w.rows + 4 * n_table + outputs


EVENT_STEPS_MIN = 200   # event-timed steps (outside the timed region) for percentiles


def measure(w, steps: int, warmup: int, with_idx: bool = True, rotate: bool = True, path: str = "auto"):
    """Time `steps` plan+select steps; returns a dict of timings and the last output.

    Two passes. The first is the timed region proper: exactly `steps` steps
    and nothing else between two synchronisations (wall clock per step). The
    second, max(steps, 200) steps so that the percentiles rest on enough
    launches, records HIP events: stream events around the planning kernel
    and the selection call, on the stream both are launched on (torch's current
    stream, which the binding passes to the library), and the selection
    kernel's own start and end (topk_select_paged_timed), the interval a
    kernel trace reports. Recording events adds work between launches, so
    they stay out of the wall-clock pass."""
    import numpy as np
    import torch
    from sparse_attention_indexer_amd import topk

    dev = torch.device("cuda:0")
    tk = topk.TopK(w.k, w.rows, max(1, w.max_len), force_path=path, device=dev)
    per_copy = max(1, w.scores.nbytes)
    ncopy = max(1, math.ceil(ROTATION_BYTES / per_copy)) if rotate else 1
    base = torch.from_numpy(np.ascontiguousarray(w.scores)).to(dev)
    copies = [base] + [base.clone() for _ in range(ncopy - 1)]
    lengths = torch.from_numpy(w.lengths).to(dev)
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    slots = torch.empty((w.rows, w.k), dtype=torch.int32, device=dev)
    idx = torch.empty_like(slots) if with_idx else None
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        if ev is not None:
            ev[0].record(stream)
        tk.plan(lengths)
        if ev is not None:
            ev[1].record(stream)
        tk.select(copies[i % ncopy], lengths, table, w.bt_row_stride, w.page_size,
                  out_slots=slots, out_indices=idx, with_indices=with_idx,
                  events=None if ev is None else (ev[3], ev[4]))
        if ev is not None:
            ev[2].record(stream)

    for i in range(warmup):
        step(i)
    n_ev = max(steps, EVENT_STEPS_MIN)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(n_ev)]
    for e in evs:   # create the kernel-event pair's HIP events before timing
        e[3].record(stream)
        e[4].record(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(n_ev):
        step(warmup + steps + i, evs[i])
    torch.cuda.synchronize()
    st = tk.status()
    if st != 0:
        raise RuntimeError(f"device status {st}")
    plan_ms = [e[0].elapsed_time(e[1]) for e in evs]
    sel_ms = [e[3].elapsed_time(e[4]) for e in evs]
    sel_stream_ms = [e[1].elapsed_time(e[2]) for e in evs]
    last = (warmup + steps + n_ev - 1) % ncopy
    out = (None if idx is None else idx.cpu().numpy(), slots.cpu().numpy())
    res = {
        "ms_per_step": (t1 - t0) * 1e3 / steps,
        "select_ms": float(np.mean(sel_ms)),
        "select_p50_ms": float(np.median(sel_ms)),
        "select_p10_ms": float(np.percentile(sel_ms, 10)),
        "select_p90_ms": float(np.percentile(sel_ms, 90)),
        "plan_ms": float(np.mean(plan_ms)),
        "plan_p50_ms": float(np.median(plan_ms)),
        "event_steps": n_ev,
        "select_stream_ms": float(np.mean(sel_stream_ms)),
        "copies": ncopy,
        "out": out,
        "last_copy_equal": bool(torch.equal(copies[last], base)),
    }
    del copies, base
    torch.cuda.empty_cache()
    return res


def calibrate_copy(mib: int, reps: int = 3) -> None:
    """A plain device-to-device copy of `mib` MiB, `reps` times: the known-size
    kernel that scales the HBM byte counters."""
    import torch
    n = mib << 18
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    say(f"[bench] copy calibration: {reps} x {mib} MiB device-to-device")


def read_ceiling(headline_bytes: int, reps: int = 20) -> dict:
    """The box's streaming-read ceiling for the selection kernel's load pattern
    (topk_debug_stream_read): the headline's byte count from cold rotated
    copies (>= 512 MB, so none is cache-resident), and one 2 GiB buffer for
    the large-transfer rate. Each launch is timed with HIP events that record
    the kernel's own start and end (as the selection kernel's timing is)."""
    import torch
    from sparse_attention_indexer_amd import topk
    dev = torch.device("cuda:0")
    out = None
    res = {"kernel": "topk_stream_read_kernel (16-byte loads, 256 x 512 lanes, 16 vectors in flight per lane)",
           "timing": "kernel events (the dispatch's own start and end), p50 of %d" % reps}
    for label, nbytes in (("headline_bytes", headline_bytes), ("2gib", 2 << 30)):
        n = nbytes // 16 * 4
        copies = max(1, math.ceil((512 << 20) / (n * 4)))
        bufs = [torch.rand(n, dtype=torch.float32, device=dev) for _ in range(copies)]
        out = topk.topk_debug_stream_read(bufs[0], out)
        torch.cuda.synchronize()
        times = []
        for i in range(reps + 3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            topk.topk_debug_stream_read(bufs[i % copies], out, events=(a, b))
            b.synchronize()
            if i >= 3:
                times.append(a.elapsed_time(b) * 1e3)
        us = statistics.median(times)
        res[label] = {"bytes": n * 4, "us_p50": round(us, 3), "GB/s": round(n * 4 / us / 1e3, 1),
                      "copies": copies}
        del bufs
        torch.cuda.empty_cache()
    say(f"[bench] read ceiling: {res['headline_bytes']['GB/s']} GB/s at {headline_bytes} B, "
        f"{res['2gib']['GB/s']} GB/s at 2 GiB")
    return res


def cpu_baseline(w, seconds: float):
    """The oracle as it stands, over whole batches: with one thread per row
    range (min(rows, nproc) threads) until `seconds` have passed, and with a
    single thread (median of 3 batches). Returns the record and the oracle's
    result on the batch."""
    import oracle
    threads = host_threads(w.rows)
    reps = 0
    t0 = time.perf_counter()
    result = None
    while True:
        result = oracle.topk_workload(w, threads=threads)
        reps += 1
        if time.perf_counter() - t0 >= seconds or reps >= 50:
            break
    dt = time.perf_counter() - t0
    one = []
    for _ in range(3):
        t = time.perf_counter()
        oracle.topk_workload(w, threads=1)
        one.append(time.perf_counter() - t)
    return {"value": round(dt / reps * 1e6, 1), "unit": "µs", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full batches of {w.rows}x{w.stride} (full sort per row, "
                      f"{threads} threads, one row range each); one thread: median of 3 batches",
            "one_thread_value": round(statistics.median(one) * 1e6, 1),
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}, result


def matches(got, want) -> bool:
    import numpy as np
    import oracle
    g, r = oracle.canonical(*got), oracle.canonical(*want)
    return bool(np.array_equal(g[0], r[0]) and np.array_equal(g[1], r[1]))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def key_prologue_bytes(w) -> int:
    """Algorithmic bytes of one key-prologue launch: per live token its BF16
    activations (2 x 128), position and row (8) and its cache row (128 FP8 +
    a 4-byte scale); padding tokens their row index only; once, the LayerNorm
    parameters, the rotary rows of the distinct positions (4 x rope_dim each)
    and the distinct block-table entries the tokens touch."""
    import numpy as np
    live = w.token_row >= 0
    n = int(live.sum())
    pages = set(zip(w.token_row[live].tolist(), (w.positions[live] // w.page_size).tolist()))
    n_pos = int(np.unique(w.positions[live]).size)
    return (n * (2 * w.dim + 8 + w.dim + 4) + 4 * int((~live).sum()) + 8 * w.dim + 4 * len(pages)
            + 4 * w.rope_dim * n_pos)


def measure_key_prologue(w, steps: int, warmup: int) -> dict:
    """Event-timed launches of the key prologue (inputs resident; a fresh
    cache per copy so that writes are not absorbed by a hot cache line);
    returns percentiles and the last cache contents."""
    import numpy as np
    import torch
    from sparse_attention_indexer_amd import prologue as K
    dev = torch.device("cuda:0")
    k_act = torch.from_numpy(w.k_act.view(np.int16)).to(dev)
    weight, bias = torch.from_numpy(w.weight).to(dev), torch.from_numpy(w.bias).to(dev)
    cs = torch.from_numpy(w.cos_sin).to(dev) if w.rope_dim else None
    pos, row = torch.from_numpy(w.positions).to(dev), torch.from_numpy(w.token_row).to(dev)
    table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    per_copy = w.k_act.nbytes + w.cos_sin.nbytes
    ncopy = min(64, max(1, math.ceil(ROTATION_BYTES / max(1, per_copy))))
    acts = [k_act] + [k_act.clone() for _ in range(ncopy - 1)]
    cache = torch.zeros((w.num_slots, w.dim), dtype=torch.uint8, device=dev)
    scale = torch.zeros(w.num_slots, dtype=torch.float32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)

    def launch(i):
        K.indexer_key_prologue(acts[i % ncopy], weight, bias, w.eps, cs, w.rope_dim, pos, row, table,
                               w.bt_row_stride, w.page_size, cache, scale, status)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        launch(i)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) / max(1, steps) * 1e3
    n_ev = max(steps, EVENT_STEPS_MIN)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
    for i, (a, b) in enumerate(evs):
        a.record()
        launch(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"wall_ms": wall_ms, "p50_ms": float(np.percentile(t, 50)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90)), "mean_ms": float(t.mean()), "copies": ncopy,
            "cache": cache.cpu().numpy(), "scale": scale.cpu().numpy(), "status": int(status.item())}


def sweep_key_prologue(name: str, args) -> bool:
    import numpy as np
    import synth
    from oracle import prologue as OP
    tokens = {"key_prologue_128k": 131_072, "key_prologue_7": 7}[name]
    w = synth.make_key_prologue(tokens, seed=12, rows=8 if tokens > 8 else 1)
    say(f"[bench] sweep {name}: {tokens} tokens")
    res = measure_key_prologue(w, args.steps, args.warmup)
    t = time.perf_counter()
    slots, codes, scales, _, scaled = OP.key_prologue(w.k_act[:, :w.dim], w.weight, w.bias, w.eps, w.cos_sin,
                                                      w.rope_dim, w.positions, w.token_row, w.block_table,
                                                      w.bt_row_stride, w.page_size)
    t_oracle = time.perf_counter() - t
    live = slots >= 0
    got = res["cache"][slots[live]]
    exact = int((got != codes[live]).sum())
    srel = float(np.max(np.abs(res["scale"][slots[live]] - scales[live]) / scales[live]))
    parity = res["status"] == 0 and srel <= 1e-5 and exact <= max(4, got.size // 1000)
    nbytes = key_prologue_bytes(w)
    p50 = res["p50_ms"] * 1e-3
    print(json.dumps({
        "workload": name, "tokens": tokens, "dim": w.dim, "rope_dim": w.rope_dim, "page_size": w.page_size,
        "kernel_us": {"p50": round(res["p50_ms"] * 1e3, 3), "p10": round(res["p10_ms"] * 1e3, 3),
                      "p90": round(res["p90_ms"] * 1e3, 3), "mean": round(res["mean_ms"] * 1e3, 3)},
        "timing": "stream events around each launch (one kernel), 200 launches",
        "step_us": round(res["wall_ms"] * 1e3, 3), "tokens_per_s": round(tokens / p50),
        "algorithmic_bytes": nbytes, "gbs": round(nbytes / p50 / 1e9, 1),
        "frac_of_8tbs": round(nbytes / p50 / 1e9 / PEAK_HBM_GBS, 4),
        "cache": f"cold activations ({res['copies']} copies)", "oracle_1thread_s": round(t_oracle, 4),
        "codes_at_rounding_ties": exact, "scale_max_rel_err": srel, "parity": parity,
        "cpu": cpu_model(), "nproc": os.cpu_count(),
    }), flush=True)
    return parity


PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 matrix peak


def sweep_logits(name: str, args) -> bool:
    """MQA logits of 7 verify tokens x 64 heads over a 1M- or 80K-key paged FP8
    cache: kernel events, TFLOP/s against the FP8 matrix peak, algorithmic
    GB/s (key codes and scales read once, FP32 scores written once), and a
    sampled check against the oracle."""
    import numpy as np
    import torch
    import synth
    from oracle import indexer_logits as OL
    from sparse_attention_indexer_amd import logits as G
    keys = {"logits_7x1m": 1_000_000, "logits_7x80k": 80_000}[name]
    w = synth.make_logits(7, keys, seed=22, with_table=False)
    say(f"[bench] sweep {name}: 7 tokens x 64 heads x {keys} keys")
    dev = torch.device("cuda:0")
    qc, wq = torch.from_numpy(w.q_codes).to(dev), torch.from_numpy(w.w).to(dev)
    ks = torch.from_numpy(w.k_scale).to(dev)
    table = torch.from_numpy(np.ascontiguousarray(w.block_table[0])).to(dev)
    lengths = torch.from_numpy(w.lengths).to(dev)
    L_ = int(w.lengths.max())
    per_copy = w.k_fp8.nbytes
    ncopy = min(16, max(1, math.ceil(ROTATION_BYTES / per_copy)))
    kc = [torch.from_numpy(w.k_fp8).to(dev)]
    kc += [kc[0].clone() for _ in range(ncopy - 1)]
    out = torch.empty((7, L_), dtype=torch.float32, device=dev)

    def launch(i):
        G.indexer_mqa_logits(qc, wq, kc[i % ncopy], ks, table, w.page_size, lengths, L_, out)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        launch(i)
    torch.cuda.synchronize()
    wall_us = (time.perf_counter() - t0) / max(1, args.steps) * 1e6
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(max(args.steps, EVENT_STEPS_MIN))]
    for i, (a, b) in enumerate(evs):
        a.record()
        launch(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
    got = out.cpu().numpy()
    ok = True
    rng = np.random.default_rng(1)
    for tok in (0, 6):
        n = int(w.lengths[tok])
        pos = rng.integers(0, n, 5000)
        ref, bound = OL.mqa_logits_at(w.q_codes, w.w, w.k_fp8, w.k_scale, w.block_table, 0, w.page_size, tok, pos)
        ok &= bool(np.all(np.abs(got[tok, pos] - ref) <= 2e-5 * bound + 1e-30))
    n_scores = int(w.lengths.astype(np.int64).sum())
    flops = 2 * 128 * 64 * n_scores
    nbytes = L_ * (128 + 4) + 4 * n_scores + w.q_codes.nbytes + w.w.nbytes + 4 * ((L_ + 63) // 64)
    p50 = float(np.percentile(t, 50))
    print(json.dumps({
        "workload": name, "tokens": 7, "heads": 64, "keys": keys,
        "kernel_us": {"p50": round(p50, 3), "p10": round(float(np.percentile(t, 10)), 3),
                      "p90": round(float(np.percentile(t, 90)), 3), "mean": round(float(t.mean()), 3)},
        "timing": "stream events around each launch (one kernel), 200 launches", "step_us": round(wall_us, 3),
        "flops": flops, "tflops": round(flops / p50 / 1e6, 1),
        "frac_of_fp8_peak": round(flops / p50 / 1e6 / PEAK_FP8_TFLOPS, 4),
        "algorithmic_bytes": nbytes, "gbs": round(nbytes / p50 / 1e3, 1),
        "frac_of_8tbs": round(nbytes / p50 / 1e3 / PEAK_HBM_GBS, 4),
        "cache": f"cold key cache ({ncopy} copies)", "parity_sampled": ok, "parity": ok,
    }), flush=True)
    return ok


def sweep_hisparse(name: str, args) -> bool:
    """HiSparse resolver, one decode step for 64 requests x top-2048 with hot
    buffers of 4096 rows and 656-byte KV rows (an FP8 sparse-MLA row), 60 % of
    each 131,072-token context's pages host-only; every step keeps 90 % of the
    previous step's selection, so about 6 % of the selected tokens miss and
    are copied from pinned host memory. Kernel events per step; the state
    evolves through the timed steps, and the last step is checked against
    the oracle stepped from the same state."""
    import numpy as np
    import torch
    import synth
    from oracle import hisparse as OH
    from sparse_attention_indexer_amd import hisparse as HSB
    R, k, hot, ctx, ps, row_bytes = 64, 2048, 4096, 131_072, 64, 656
    st = synth.Stream(17, 3)
    pages = ctx // ps
    table = np.where(st.uniform(R * pages) < 0.6, -1, st.permutation(R * pages)).astype(np.int32).reshape(R, pages)
    host_pages = 4096
    host_table = st.below(R * pages, host_pages).astype(np.int32).reshape(R, pages)
    hot_rows = st.permutation(R * hot).astype(np.int64).reshape(R, hot)
    host = st.u64(host_pages * ps * row_bytes // 8).view(np.uint8).reshape(host_pages * ps, row_bytes).copy()
    n_steps = args.warmup + max(args.steps, 20)
    sels = []
    cur = np.stack([st.permutation(ctx)[:k] for _ in range(R)]).astype(np.int32)
    for _ in range(n_steps):
        sels.append(cur.copy())
        for r in range(R):
            keep = cur[r][st.permutation(k)[: int(0.9 * k)]]
            fresh = st.permutation(ctx)[: 2 * k]
            fresh = fresh[~np.isin(fresh, keep)][: k - keep.size]
            cur[r] = np.concatenate([keep, fresh])
    say(f"[bench] sweep {name}: {R} requests x top-{k}, hot {hot}, {n_steps} steps")
    dev = torch.device("cuda:0")
    g_table, g_host_table = torch.from_numpy(table).to(dev), torch.from_numpy(host_table).to(dev)
    g_hot = torch.from_numpy(hot_rows).to(dev)
    tag = torch.full((R, hot), -1, dtype=torch.int32, device=dev)
    stamp = torch.zeros((R, hot), dtype=torch.int32, device=dev)
    map_ = torch.full((R, ctx), -1, dtype=torch.int32, device=dev)
    kv = torch.zeros((R * hot, row_bytes), dtype=torch.uint8, device=dev)
    rows = torch.empty((R, k), dtype=torch.int64, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    pool = torch.from_numpy(host).pin_memory()
    g_sels = [torch.from_numpy(x).to(dev) for x in sels]
    times, misses = [], []
    snap = None
    for i in range(n_steps):
        if i == n_steps - 1:
            snap = (tag.cpu().numpy(), stamp.cpu().numpy().view(np.uint32), map_.cpu().numpy(), kv.cpu().numpy())
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        HSB.hisparse_resolve(i + 1, g_sels[i], g_table, g_host_table, ps, g_hot, tag, stamp, map_, kv, pool, rows,
                             status)
        b.record()
        torch.cuda.synchronize()
        if i >= args.warmup:
            times.append(a.elapsed_time(b) * 1e3)
    # the last step against the oracle, from the state before it
    tg, sp, mp, kvh = snap
    ok = int(status.item()) == 0
    got_rows = rows.cpu().numpy()
    n_miss = 0
    for r in range(R):
        hs = OH.HotState(tg[r].copy(), sp[r].copy(), mp[r].copy())
        before = hs.map.copy()
        want, f = OH.resolve(n_steps, sels[-1][r], table[r], host_table[r], ps, hot_rows[r], hs, kvh, host)
        ok &= bool(np.array_equal(got_rows[r], want)) and f == 0
        sel = sels[-1][r]
        n_miss += int(((table[r][sel // ps] < 0) & (before[sel] < 0)).sum())
    ok &= bool(np.array_equal(kv.cpu().numpy(), kvh))
    t = np.array(times)
    p50 = float(np.percentile(t, 50))
    host_bytes = n_miss * row_bytes
    print(json.dumps({
        "workload": name, "requests": R, "k": k, "hot": hot, "context": ctx, "row_bytes": row_bytes,
        "kernel_us": {"p50": round(p50, 3), "p10": round(float(np.percentile(t, 10)), 3),
                      "p90": round(float(np.percentile(t, 90)), 3), "mean": round(float(t.mean()), 3)},
        "timing": "stream events around each launch (one kernel), steps after warmup",
        "misses_last_step": n_miss, "host_bytes_last_step": host_bytes,
        "host_gbs_at_p50": round(host_bytes / p50 / 1e3, 2), "resolved_per_s": round(R * k / p50 * 1e6),
        "parity_last_step": ok, "parity": ok,
    }), flush=True)
    return ok


def sweep(args) -> int:
    """One JSON line per workload: latency percentiles, rows/s, algorithmic GB/s,
    plan time, parity and the oracle's wall time (1 thread and N threads)."""
    import oracle
    ok = True
    names = args.sweep.split(",")
    for name in names:
        if name.startswith("key_prologue"):
            ok &= sweep_key_prologue(name, args)
            continue
        if name.startswith("logits_"):
            ok &= sweep_logits(name, args)
            continue
        if name.startswith("hisparse"):
            ok &= sweep_hisparse(name, args)
            continue
        w = workload(name)
        say(f"[bench] sweep {name}: {w.rows}x{w.stride}")
        res = measure(w, args.steps, args.warmup, rotate=not args.warm_cache, path=path_of(name))
        nthreads = host_threads(w.rows)
        # the oracle's timing on at most 256 rows (scaled to the batch); its
        # parity result on the whole batch
        ws = row_sample(w, 256)
        t1, tn = [], []
        for _ in range(3):
            t = time.perf_counter()
            oracle.topk_workload(ws, threads=1)
            t1.append(time.perf_counter() - t)
            t = time.perf_counter()
            oracle.topk_workload(ws, threads=min(ws.rows, nthreads))
            tn.append(time.perf_counter() - t)
        scale = w.rows / ws.rows
        ref = oracle.topk_workload(w, threads=nthreads) if ws is not w else oracle.topk_workload(w, threads=1)
        parity = matches(res["out"], ref) and res["last_copy_equal"]
        ok &= parity
        nbytes = algorithmic_bytes(w, res["out"][1], True)
        p50 = res["select_p50_ms"] * 1e-3
        print(json.dumps({
            "workload": w.name, "rows": w.rows, "stride": w.stride, "k": w.k, "path": path_of(name),
            "select_us": {"p50": round(res["select_p50_ms"] * 1e3, 3), "p10": round(res["select_p10_ms"] * 1e3, 3),
                          "p90": round(res["select_p90_ms"] * 1e3, 3), "mean": round(res["select_ms"] * 1e3, 3)},
            "plan_us": ({"mean": round(res["plan_ms"] * 1e3, 3), "p50": round(res["plan_p50_ms"] * 1e3, 3)}
                        if w.rows > IN_KERNEL_PLAN_ROWS else "in-kernel"),
            "step_us": round(res["ms_per_step"] * 1e3, 3),
            "rows_per_s": round(w.rows / p50), "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / p50 / 1e9, 1), "frac_of_8tbs": round(nbytes / p50 / 1e9 / PEAK_HBM_GBS, 4),
            "cache": "warm" if args.warm_cache else f"cold ({res['copies']} copies)",
            "oracle_1thread_s": round(statistics.median(t1) * scale, 4),
            f"oracle_{min(ws.rows, nthreads)}threads_s": round(statistics.median(tn) * scale, 4),
            "oracle_sample": (f"first {ws.rows} of {w.rows} rows, scaled by {scale:g}" if ws is not w
                              else "whole batch, median of 3"),
            "cpu": cpu_model(), "nproc": os.cpu_count(), "parity": parity,
        }), flush=True)
    if args.calibrate_copy_mb:
        calibrate_copy(args.calibrate_copy_mb)
    return 0 if ok else 1


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workloads", default="7x1m,7x80k",
                    help="comma list from {7x1m, 7x80k}; the first is the headline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm-cache", action="store_true", help="reuse one input copy (cache-resident)")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after timing, copy this many MiB device-to-device (counter calibration)")
    ap.add_argument("--no-read-ceiling", action="store_true",
                    help="skip the streaming-read ceiling measurement")
    ap.add_argument("--sweep", default="",
                    help="comma list from {c1..c5, c5_g0..c5_g3, cp8_7x125k, prefill_4096x80k, plan_split_600, "
                         "key_prologue_128k, key_prologue_7, logits_7x1m, logits_7x80k, hisparse_64x2048}: "
                         "one JSON line per workload")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: rows are independent, so the path shards by rows with no "
              "exchange; multi-GPU runs are not part of this build (use --gpus 1).", file=sys.stderr)
        return 2
    if args.sweep:
        return sweep(args)

    import oracle

    names = args.workloads.split(",")
    for n in names:
        if n not in DESCRIPTIONS:
            ap.error(f"unknown workload {n}")
    results = {}
    for n in names:
        w = workload(n)
        say(f"[bench] {n}: {args.warmup} warmup + {args.steps} timed steps")
        results[n] = (w, measure(w, args.steps, args.warmup, rotate=not args.warm_cache))
    if args.calibrate_copy_mb:
        calibrate_copy(args.calibrate_copy_mb)
    ceiling = None if args.no_read_ceiling else read_ceiling(int(results[names[0]][0].lengths.sum()) * 4)

    head = names[0]
    w, res = results[head]
    base = None
    if not args.no_cpu_baseline:
        say(f"[bench] oracle CPU baseline on {head} for ~{args.cpu_seconds:g} s")
        base, ref = cpu_baseline(w, args.cpu_seconds)
    else:
        ref = oracle.topk_workload(w, threads=host_threads(w.rows))
    parity = matches(res["out"], ref) and res["last_copy_equal"]

    nbytes = algorithmic_bytes(w, res["out"][1], True)
    achieved = nbytes / (res["select_ms"] * 1e-3) / 1e9
    traffic = None
    if head == "7x1m" and os.path.exists(TRAFFIC_FILE):
        t = json.loads(open(TRAFFIC_FILE).read())
        if t.get("kernel_source_sha") == kernel_source_digest():
            traffic = t.get("bytes_per_launch")
    step_us = res["ms_per_step"] * 1e3
    line = {
        "metric": METRIC,
        "value": round(step_us, 3),
        "unit": "µs",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": DESCRIPTIONS[head],
            "rows": w.rows, "row_len": w.stride, "k": w.k, "page_size": w.page_size,
            "cache": "warm (one input copy)" if args.warm_cache else
                     f"cold: {res['copies']} rotated input copies (>= 512 MB)",
            "step": "topk_plan + topk_select_paged",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": "topk_select_kernel",
            "algorithmic_bytes": nbytes,
            "kernel_us": round(res["select_ms"] * 1e3, 3),
        },
        "cpu_baseline": base,
        "vs_oracle": round(base["value"] / step_us, 1) if base else None,
        "hbm_read_ceiling": ceiling,
        "select_us": {"event_steps": res["event_steps"],
                      "mean": round(res["select_ms"] * 1e3, 3), "p10": round(res["select_p10_ms"] * 1e3, 3),
                      "p50": round(res["select_p50_ms"] * 1e3, 3), "p90": round(res["select_p90_ms"] * 1e3, 3),
                      "stream_events_mean": round(res["select_stream_ms"] * 1e3, 3)},
        "plan_us": round(res["plan_ms"] * 1e3, 3) if w.rows > IN_KERNEL_PLAN_ROWS else None,
        "plan": "in the selection kernel" if w.rows <= IN_KERNEL_PLAN_ROWS else "topk_plan kernel",
        "parity": parity,
        "pages_b300_context_us": {"topk_v2_80k": PAGES_V2_US["7x80k"], "topk_v2_1m": PAGES_V2_US["7x1m"]},
    }
    ok = parity
    for n in names[1:]:
        w2, r2 = results[n]
        p2 = matches(r2["out"], oracle.topk_workload(w2, threads=host_threads(w2.rows)))
        ok &= p2
        line[f"latency_{n}_us"] = {"step": round(r2["ms_per_step"] * 1e3, 3),
                                   "select_mean": round(r2["select_ms"] * 1e3, 3),
                                   "select_stream_events_mean": round(r2["select_stream_ms"] * 1e3, 3),
                                   "select_p50": round(r2["select_p50_ms"] * 1e3, 3),
                                   "select_p10": round(r2["select_p10_ms"] * 1e3, 3),
                                   "select_p90": round(r2["select_p90_ms"] * 1e3, 3),
                                   "event_steps": r2["event_steps"],
                                   "plan": round(r2["plan_ms"] * 1e3, 3) if w2.rows > IN_KERNEL_PLAN_ROWS
                                   else "in the selection kernel", "parity": p2}
    print(json.dumps(line), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
