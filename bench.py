"""Decode-step throughput of the Locks decode path on one MI355X.

One step = lk_decode_step on one layer's cache: append the new token, score
every complete page from its summary, share-average and select, attend over
the selection, merge, and build the summary of a page the append completed.
Workload: Llama-3.1-8B attention shape (32 query / 8 KV heads, d=128), bf16,
page 64, rank 8, budget 2048 tokens, 4 sequences at 131,072 tokens.

Several identical layer copies are rotated so that consecutive steps touch
cold addresses (the per-step working set would otherwise fit the 256 MB
last-level cache).  Inputs (queries, new keys/values) are resident in HBM
before timing.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=512)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--layers", type=int, default=4, help="layer copies rotated across steps")
    p.add_argument("--kernel-reps", type=int, default=200, help="timed launches of the scorer alone")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-steps", type=int, default=3, help="whole oracle steps timed for the CPU baseline")
    p.add_argument("--summary", choices=("kv", "i4"), default="kv",
                   help="page summaries in the KV dtype (bf16, the default) or int4 basis / int8 rows")
    p.add_argument("--workload", type=int, choices=(2, 3, 4), default=2,
                   help="2: 128K x 4 (the headline); 3: one 1M-token sequence; "
                        "4: 64 sequences of 4K..256K tokens (in-stream builds in most steps)")
    p.add_argument("--no-q4", action="store_true", help="skip the int4 / int8 record run of the default line")
    p.add_argument("--no-page16", action="store_true", help="skip the 16-token-page (r8i4) run of the default line")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="also run a plain device copy of this size (counter calibration)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_sparse_page_amd import locks as L
    from long_context_sparse_page_amd import synth
    from long_context_sparse_page_amd.paged import DeviceCache, to_storage

    torch.cuda.set_device(0)
    dev = "cuda"
    total_steps = args.warmup + args.steps
    per_layer = -(-total_steps // args.layers)
    # further steps timed one by one (in-stream build split, below): a page per
    # layer copy, so each copy's sequences complete exactly one page in them
    extra = synth.workload(args.workload).page_size * args.layers
    # the default line also times the same step with int4 / int8 summary
    # records on the same cache (a second summary pool per layer copy)
    with_q4 = args.summary == "kv" and args.workload == 2 and not args.no_q4
    runs = 2 if with_q4 else 1
    w = synth.workload(args.workload, steps=runs * per_layer + 1 + -(-extra // args.layers), summary=args.summary)
    B, d, G, hkv, hq = w.page_size, w.head_dim, w.group, w.num_kv_heads, w.num_q_heads
    e = 2  # bf16
    t0 = time.time()
    base = DeviceCache(w)
    base.fill_from_synth(threads=min(16, os.cpu_count() or 4))
    base.build_all()
    torch.cuda.synchronize()
    print(f"[bench] layer 0 filled and summarized in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    layers = [base]
    for _ in range(1, args.layers):
        c = DeviceCache.__new__(DeviceCache)
        c.__dict__.update(base.__dict__)
        c.k_pool = base.k_pool.clone()
        c.v_pool = base.v_pool.clone()
        c.summary_pool = base.summary_pool.clone()
        c.seq_lens = base.seq_lens.clone()
        c.block_table = base.block_table.clone()
        c.cache = L.make_cache(c.k_pool, c.v_pool, c.summary_pool, c.block_table, c.seq_lens)
        layers.append(c)
    ws, ws_bytes = base.ws, base.ws_bytes

    # resident inputs for every step
    n_var = 16
    qs, kns, vns = [], [], []
    for i in range(n_var):
        lens = [t + 1 + i for t in w.context]
        q = np.zeros((w.batch, hq, d), np.float32)
        for s in range(w.batch):
            for h in range(hkv):
                q[s, h * G:(h + 1) * G] = synth.queries(w, i, s, h, lens[s])[0]
        qs.append(to_storage(q, w.dtype).to(dev))
    rng = np.random.default_rng(7)
    for i in range(n_var):
        kns.append(to_storage(rng.standard_normal((w.batch, hkv, d)).astype(np.float32), w.dtype).to(dev))
        vns.append(to_storage(rng.standard_normal((w.batch, hkv, d)).astype(np.float32), w.dtype).to(dev))
    out = torch.empty((w.batch, hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, hq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(i):
        c = layers[i % len(layers)]
        L.lk_decode_step(c.cfg, c.cache, w.batch, qs[i % n_var], kns[i % n_var], vns[i % n_var], out, lse,
                         None, None, ws, ws_bytes, sp)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.warmup, total_steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / args.steps

    # algorithmic bytes of one step at the lengths reached: per (sequence, KV
    # head) every scored record plus its G page-LSE floats, the selected pages'
    # K and V; per sequence the queries, outputs and the appended k/v
    rec = L.lk_summary_record_bytes(base.cfg)
    k_pages = L.lk_page_budget(base.cfg)
    lens_now = [int(x) for x in layers[0].seq_lens.cpu().tolist()]

    def step_bytes(lens):
        tot = 0
        for T in lens:
            n_mr = (T - 1) // B
            tail = T - n_mr * B
            n_sel = min(k_pages, n_mr + 1)
            toks = (n_sel - 1) * B + tail
            tot += hkv * (n_mr * (rec + 4 * G) + toks * 2 * d * e)
        tot += w.batch * (2 * hq * d * e + 2 * hkv * d * e * 2)  # q + out, k_new/v_new read + write
        return tot

    bytes_step = step_bytes(lens_now)

    # dominant kernel: the scorer, timed alone on the same layers (score-only calls)
    page_lse = torch.empty((w.batch, hq, base.max_pages), dtype=torch.float32, device=dev)
    def score(i):
        c = layers[i % len(layers)]
        L.lk_score_select(c.cfg, c.cache, w.batch, qs[i % n_var], page_lse, None, None, None, ws, ws_bytes, sp)
    for i in range(8):
        score(i)
    torch.cuda.synchronize()
    # back-to-back launches between two events on the launch stream: the
    # average launch duration (launch gaps of a full queue included)
    ev0.record(stream)
    for i in range(args.kernel_reps):
        score(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    score_ms = ev0.elapsed_time(ev1) / args.kernel_reps
    units = sum(hkv * ((T - 1) // B) for T in lens_now)
    score_bytes = units * (rec + 4 * G)
    score_gbs = score_bytes / (score_ms * 1e-3) / 1e9

    # same-GPU dense decode attention over every token
    def dense(i):
        c = layers[i % len(layers)]
        L.lk_dense_decode_attn(c.cfg, c.cache, w.batch, qs[i % n_var], out, lse, ws, ws_bytes, sp)
    for i in range(4):
        dense(i)
    torch.cuda.synchronize()
    reps = 40
    ev0.record(stream)
    for i in range(reps):
        dense(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    dense_ms = ev0.elapsed_time(ev1) / reps
    dense_bytes = sum(hkv * T * 2 * d * e for T in lens_now) + w.batch * 2 * hq * d * e

    # bulk summary build (the pass at the prefill-decode boundary): every page
    # complete at the initial context, all KV heads, one lk_build_page_summary call
    bulk = layers[-1]
    ids = [int(p) for s in range(w.batch) for p in bulk.block_table_host[s, :w.context[s] // B]]
    ids_t = torch.tensor(ids, dtype=torch.int32, device=dev)

    def bulk_build():
        L.lk_build_page_summary(bulk.cfg, bulk.cache, ids_t, len(ids), None, ws, ws_bytes, sp)
    bulk_build()
    torch.cuda.synchronize()
    reps = 3
    ev0.record(stream)
    for _ in range(reps):
        bulk_build()
    ev1.record(stream)
    torch.cuda.synchronize()
    build_ms = ev0.elapsed_time(ev1) / reps

    # the same keys re-paged into 16-token pages, summarized in the int4 basis /
    # int8 row format (r = 8) of the pages' deployment: one bulk call (128K x 4 only)
    page16 = bulk_build_page16(L, w, bulk, reps, stream, ev0, ev1) if args.workload == 2 else None

    # per-step durations over further steps (events between consecutive steps),
    # split by whether the step's append completes a page of some sequence (the
    # step's last launch then also builds that page's summary)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(extra + 1)]
    lens_at = [[int(x) for x in c.seq_lens.cpu().tolist()] for c in layers]
    builds = []
    evs[0].record(stream)
    for j in range(extra):
        i = total_steps + j
        li = i % len(layers)
        builds.append(any(T % B == B - 1 for T in lens_at[li]))
        lens_at[li] = [T + 1 for T in lens_at[li]]
        step(i)
        evs[j + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([evs[j].elapsed_time(evs[j + 1]) * 1e3 for j in range(extra)])
    with_b = np.array(builds)
    step_us = {"median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
               "p90": float(np.percentile(per, 90)), "mean": float(per.mean()), "steps": int(extra),
               "note": "one event pair per step (adds a little per step over the window mean)"}
    in_stream = {"steps": extra, "steps_with_build": int(with_b.sum()),
                 "us_median_without_build": float(np.median(per[~with_b])) if (~with_b).any() else None,
                 "us_median_with_build": float(np.median(per[with_b])) if with_b.any() else None}

    wl = {2: "128K-context decode, batch 4",
          3: "1M-token decode, batch 1",
          4: f"mixed-length decode, batch {w.batch}, lengths log-uniform in [4K, 256K] (seeded, mean "
             f"{int(np.mean(w.context))} tokens)"}[args.workload]
    result = {
        "metric": "decode-attn steps/s and achieved HBM GB/s at 128K ctx, budget 2048 tok" if args.workload == 2
                  else "decode-attn steps/s and achieved HBM GB/s",
        "value": 1e3 / ms_per_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl + ", Llama-3.1-8B attention shape (32 q / 8 KV heads, d=128), "
                        f"bf16 KV, page 64, rank {w.rank}, budget {w.token_budget} tokens; one step = lk_decode_step "
                        "on one layer"
                        + ("; int4 basis / int8 coefficient and centroid summaries" if args.summary == "i4" else ""),
            "summary_records": "bf16" if args.summary == "kv" else "int4 basis, int8 coefficients and centroid",
            "record_bytes": rec,
            "global_batch": w.batch, "seq_len": w.context[0] if len(set(w.context)) == 1 else "mixed",
            "page_size": B, "rank": w.rank,
            "token_budget": w.token_budget, "num_q_heads": hq, "num_kv_heads": hkv, "layers_rotated": args.layers,
            "parallelism": "single GPU",
        },
        "achieved_GBps": bytes_step / (ms_per_step * 1e-3) / 1e9,
        "algorithmic_bytes_per_step": bytes_step,
        "hbm_frac": bytes_step / (ms_per_step * 1e-3) / 8e12,
        "roofline": {
            "bound": "hbm",
            "kernel": ("score_mfma_kernel" if args.summary == "kv" else "score_q4_kernel") + " (reconstructed page LSE)",
            "achieved": score_gbs,
            "peak": 8000.0,
            "unit": "GB/s",
            "frac": score_gbs / 8000.0,
            "traffic": recorded_traffic(TRAFFIC_PROFILE[args.summary]) if args.workload in TRAFFIC_WORKLOADS else None,
            "launch_us": score_ms * 1e3,
            "bytes_per_launch": score_bytes,
        },
        "dense_baseline": {"ms": dense_ms, "GBps": dense_bytes / (dense_ms * 1e-3) / 1e9,
                           "speedup_of_locks_step": dense_ms / ms_per_step},
        "bulk_build": {"pages": len(ids), "page_heads": len(ids) * hkv, "ms": build_ms,
                       "page_heads_per_s": len(ids) * hkv / (build_ms * 1e-3)},
        "step_us": step_us,
        "in_stream_build": in_stream,
    }
    ceil = hbm_ceilings(torch, stream)
    result["hbm_ceilings"] = ceil
    result["step_frac_of_read_ceiling"] = result["achieved_GBps"] / ceil["read_GBps"]
    if with_q4:
        result["int4_records"] = q4_variant(L, w, layers, qs, kns, vns, out, lse, stream, args, ws, ws_bytes)
    if args.workload == 2 and not args.no_page16:
        result["page16_r8i4"] = page16_variant(L, args, stream)
    if page16 is not None:
        result["bulk_build_page16_r8i4"] = page16

    if args.copy_bytes:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters scale
        # the scorer's counters to bytes
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = args.copy_bytes

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = run_cpu_baseline(w, lens_now, args.cpu_steps)
    print(json.dumps(result), flush=True)


def hbm_ceilings(torch, stream):
    """Same-run reference rates: a 2 GiB fp32 sum (reads only) and a 1 GiB
    device copy (read + write), each timed over 10 calls."""
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    x = torch.ones(1 << 29, dtype=torch.float32, device="cuda")
    for _ in range(2):
        x.sum()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(10):
        x.sum()
    ev1.record(stream)
    torch.cuda.synchronize()
    read = x.numel() * 4 / (ev0.elapsed_time(ev1) / 10 * 1e-3) / 1e9
    del x
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    ev1.record(stream)
    torch.cuda.synchronize()
    copy = 2 * src.numel() / (ev0.elapsed_time(ev1) / 10 * 1e-3) / 1e9
    return {"read_GBps": read, "read_kind": "torch.sum over 2 GiB fp32",
            "copy_GBps": copy, "copy_kind": "1 GiB device copy, read + write bytes"}


def q4_variant(L, w, layers, qs, kns, vns, out, lse, stream, args, ws, ws_bytes):
    """The default step with int4 basis / int8 coefficient and centroid
    records: every page complete at the current lengths of each layer copy is
    summarized into a second (uint8) summary pool, then the step and the
    scorer alone are timed as for the bf16 records."""
    import torch

    B, d, G, hkv, hq = w.page_size, w.head_dim, w.group, w.num_kv_heads, w.num_q_heads
    sp = stream.cuda_stream
    cfg = L.make_config(d, B, w.rank, hq, hkv, w.token_budget, L.LK_BF16, w.scale, L.LK_SUMMARY_I4)
    rec = L.lk_summary_record_bytes(cfg)
    need = L.lk_workspace_size(cfg, w.batch, layers[0].max_pages)
    if need > ws_bytes:
        ws, ws_bytes = torch.empty(need, dtype=torch.uint8, device="cuda"), need
    caches = []
    for c in layers:
        pool = torch.empty((c.num_phys, hkv, rec), dtype=torch.uint8, device="cuda")
        lens = [int(x) for x in c.seq_lens.cpu().tolist()]
        ids = torch.tensor([int(p) for s in range(w.batch) for p in c.block_table_host[s, :lens[s] // B]],
                           dtype=torch.int32, device="cuda")
        cache = L.make_cache(c.k_pool, c.v_pool, pool, c.block_table, c.seq_lens)
        L.lk_build_page_summary(cfg, cache, ids, ids.numel(), None, ws, ws_bytes, sp)
        caches.append((cache, pool))
    torch.cuda.synchronize()
    n = len(caches)
    nv = len(qs)

    def step(i):
        L.lk_decode_step(cfg, caches[i % n][0], w.batch, qs[i % nv], kns[i % nv], vns[i % nv], out, lse,
                         None, None, ws, ws_bytes, sp)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    lens_now = [int(x) for x in layers[0].seq_lens.cpu().tolist()]
    k_pages = L.lk_page_budget(cfg)
    e = 2
    step_bytes = w.batch * (2 * hq * d * e + 2 * hkv * d * e * 2)
    for T in lens_now:
        n_mr = (T - 1) // B
        step_bytes += hkv * (n_mr * (rec + 4 * G) + ((min(k_pages, n_mr + 1) - 1) * B + T - n_mr * B) * 2 * d * e)
    page_lse = torch.empty((w.batch, hq, layers[0].max_pages), dtype=torch.float32, device="cuda")

    def score(i):
        L.lk_score_select(cfg, caches[i % n][0], w.batch, qs[i % nv], page_lse, None, None, None, ws, ws_bytes, sp)
    for i in range(8):
        score(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.kernel_reps):
        score(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    score_ms = ev0.elapsed_time(ev1) / args.kernel_reps
    score_bytes = sum(hkv * ((T - 1) // B) for T in lens_now) * (rec + 4 * G)
    return {"records": "int4 basis (per-vector fp16 scales), int8 coefficients (per-token scales) and centroid",
            "record_bytes": rec, "ms_per_step": ms, "steps_per_s": 1e3 / ms,
            "algorithmic_bytes_per_step": step_bytes, "achieved_GBps": step_bytes / (ms * 1e-3) / 1e9,
            "hbm_frac": step_bytes / (ms * 1e-3) / 8e12,
            "scorer": {"kernel": "score_q4_kernel", "launch_us": score_ms * 1e3, "bytes_per_launch": score_bytes,
                       "achieved_GBps": score_bytes / (score_ms * 1e-3) / 1e9,
                       "frac": score_bytes / (score_ms * 1e-3) / 8e12,
                       "traffic": recorded_traffic(TRAFFIC_PROFILE["i4"])}}


def page16_variant(L, args, stream):
    """The same decode step at the pages' deployed page size: 128K x 4 with
    pages of 16 tokens and int4 basis / int8 coefficient and centroid records
    (r = 8), on its own cache (filled from the same key model at 16 tokens,
    bulk-built, layer copies rotated as for the default line)."""
    import torch

    from long_context_sparse_page_amd import synth
    from long_context_sparse_page_amd.paged import DeviceCache, to_storage

    B = 16
    total = args.warmup + args.steps
    n_layers = args.layers
    w = synth.workload(2, steps=-(-total // n_layers) + 2, summary="i4")
    w.page_size = B
    d, G, hkv, hq = w.head_dim, w.group, w.num_kv_heads, w.num_q_heads
    t0 = time.time()
    base = DeviceCache(w)
    base.fill_from_synth(threads=min(16, os.cpu_count() or 4))
    base.build_all()
    torch.cuda.synchronize()
    fill_s = time.time() - t0
    layers = [base]
    for _ in range(1, n_layers):
        c = DeviceCache.__new__(DeviceCache)
        c.__dict__.update(base.__dict__)
        c.k_pool, c.v_pool = base.k_pool.clone(), base.v_pool.clone()
        c.summary_pool, c.seq_lens = base.summary_pool.clone(), base.seq_lens.clone()
        c.block_table = base.block_table.clone()
        c.cache = L.make_cache(c.k_pool, c.v_pool, c.summary_pool, c.block_table, c.seq_lens)
        layers.append(c)
    nv = 16
    qs, kns, vns = [], [], []
    rng = np.random.default_rng(16)
    for i in range(nv):
        lens = [t + 1 + i for t in w.context]
        q = np.zeros((w.batch, hq, d), np.float32)
        for s in range(w.batch):
            for h in range(hkv):
                q[s, h * G:(h + 1) * G] = synth.queries(w, i, s, h, lens[s])[0]
        qs.append(to_storage(q, w.dtype).to("cuda"))
        kns.append(to_storage(rng.standard_normal((w.batch, hkv, d)).astype(np.float32), w.dtype).to("cuda"))
        vns.append(to_storage(rng.standard_normal((w.batch, hkv, d)).astype(np.float32), w.dtype).to("cuda"))
    out = torch.empty((w.batch, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, hq), dtype=torch.float32, device="cuda")
    sp = stream.cuda_stream
    ws, ws_bytes = base.ws, base.ws_bytes

    def step(i):
        c = layers[i % n_layers]
        L.lk_decode_step(c.cfg, c.cache, w.batch, qs[i % nv], kns[i % nv], vns[i % nv], out, lse, None, None,
                         ws, ws_bytes, sp)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.warmup, total):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    lens_now = [int(x) for x in layers[0].seq_lens.cpu().tolist()]
    rec = L.lk_summary_record_bytes(base.cfg)
    k_pages = L.lk_page_budget(base.cfg)
    e = 2
    step_bytes = w.batch * (2 * hq * d * e + 2 * hkv * d * e * 2)
    for T in lens_now:
        n_mr = (T - 1) // B
        step_bytes += hkv * (n_mr * (rec + 4 * G) + ((min(k_pages, n_mr + 1) - 1) * B + T - n_mr * B) * 2 * d * e)
    page_lse = torch.empty((w.batch, hq, base.max_pages), dtype=torch.float32, device="cuda")

    def score(i):
        c = layers[i % n_layers]
        L.lk_score_select(c.cfg, c.cache, w.batch, qs[i % nv], page_lse, None, None, None, ws, ws_bytes, sp)
    for i in range(8):
        score(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(args.kernel_reps):
        score(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    score_ms = ev0.elapsed_time(ev1) / args.kernel_reps
    score_bytes = sum(hkv * ((T - 1) // B) for T in lens_now) * (rec + 4 * G)

    def dense(i):
        c = layers[i % n_layers]
        L.lk_dense_decode_attn(c.cfg, c.cache, w.batch, qs[i % nv], out, lse, ws, ws_bytes, sp)
    for i in range(4):
        dense(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(20):
        dense(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    dense_ms = ev0.elapsed_time(ev1) / 20
    res = {"workload": "128K-context decode, batch 4, pages of 16 tokens, int4 basis / int8 coefficient and "
                       "centroid records, rank 8, budget 2048 tokens (128 pages); one step = lk_decode_step",
           "record_bytes": rec, "ms_per_step": ms, "steps_per_s": 1e3 / ms,
           "algorithmic_bytes_per_step": step_bytes, "achieved_GBps": step_bytes / (ms * 1e-3) / 1e9,
           "hbm_frac": step_bytes / (ms * 1e-3) / 8e12,
           "scorer": {"kernel": "score_q4_kernel (16-token pages)", "launch_us": score_ms * 1e3,
                      "bytes_per_launch": score_bytes, "achieved_GBps": score_bytes / (score_ms * 1e-3) / 1e9,
                      "frac": score_bytes / (score_ms * 1e-3) / 8e12},
           "dense_ms": dense_ms, "speedup_over_dense": dense_ms / ms, "fill_s": fill_s}
    del layers, base
    torch.cuda.empty_cache()
    return res


def bulk_build_page16(L, w, bulk, reps, stream, ev0, ev1):
    """The keys of every complete 64-token page re-paged into 16-token pages
    and summarized in the int4 basis / int8 row format at r = 8, one
    lk_build_page_summary call, timed over ``reps`` calls."""
    import torch

    dev, sp = "cuda", stream.cuda_stream
    B, d, hkv, hq = w.page_size, w.head_dim, w.num_kv_heads, w.num_q_heads
    n_full = [w.context[s] // B for s in range(w.batch)]
    src = torch.cat([bulk.k_pool[torch.from_numpy(bulk.block_table_host[s, :n_full[s]].astype(np.int64)).to(dev)]
                     for s in range(w.batch)])
    k16 = src.view(-1, hkv, B // 16, 16, d).permute(0, 2, 1, 3, 4).reshape(-1, hkv, 16, d).contiguous()
    del src
    cfg16 = L.make_config(d, 16, 8, hq, hkv, w.token_budget, L.LK_BF16, w.scale, L.LK_SUMMARY_I4)
    s16 = torch.zeros((k16.shape[0], hkv, L.lk_summary_record_bytes(cfg16)), dtype=torch.uint8, device=dev)
    cache16 = L.make_cache(k16, None, s16, bulk.block_table, bulk.seq_lens)
    ids16 = torch.arange(k16.shape[0], dtype=torch.int32, device=dev)

    def build16():
        L.lk_build_page_summary(cfg16, cache16, ids16, k16.shape[0], None, None, 0, sp)
    build16()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(reps):
        build16()
    ev1.record(stream)
    torch.cuda.synchronize()
    build16_ms = ev0.elapsed_time(ev1) / reps
    pages16 = int(k16.shape[0])
    del k16, s16
    return {"pages": pages16, "page_heads": pages16 * hkv, "ms": build16_ms,
            "page_heads_per_s": pages16 * hkv / (build16_ms * 1e-3)}


# scorer HBM traffic per launch, from rocprofv3 counters taken on the 128K x 4
# workload: reported for that workload only (other workloads move other bytes)
TRAFFIC_PROFILE = {"kv": "profiles/score_mfma_128K_b4_hbm_traffic.txt",
                   "i4": "profiles/score_q4_128K_b4_hbm_traffic.txt"}
TRAFFIC_WORKLOADS = (2,)


def recorded_traffic(profile):
    """HBM bytes per scorer launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the scorer's
    sources have changed since the counters were taken."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    try:
        fields = dict(line.strip().split("=", 1) for line in open(os.path.join(root, profile))
                      if "=" in line and not line.startswith(" "))
        h = hashlib.sha256()
        for f in fields["kernel_sources"].split():
            with open(os.path.join(root, f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != fields["kernel_sources_sha256"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_worker(conn, wargs, pairs, lens):
    """One process of the CPU baseline: holds its (sequence, KV head) pairs'
    stored K / V, the oracle's own summaries of their complete pages and a
    query, then runs the oracle's decode step on them whenever asked."""
    from threadpoolctl import threadpool_limits

    from long_context_sparse_page_amd import synth
    from oracle import locks_oracle as lo

    w = synth.workload(wargs["wid"], rank=wargs["rank"], budget=wargs["budget"], steps=wargs["steps"],
                       summary=wargs["summary"])
    w.batch, w.context = wargs["batch"], list(wargs["context"])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        data = []
        B, d = w.page_size, w.head_dim
        for (s, h) in pairs:
            T = lens[s]
            k, v = synth.keys_values(w, s, h)
            n_pages = -(-T // B)
            K = np.zeros((n_pages * B, d))
            V = np.zeros((n_pages * B, d))
            K[:T] = lo.storage_round(k[:T], w.dtype)
            V[:T] = lo.storage_round(v[:T], w.dtype)
            K, V = K.reshape(n_pages, B, d), V.reshape(n_pages, B, d)
            n_mr = lo.most_recent_page(T, B)
            if w.summary == "i4":
                summ = lo.dequantize_summary(lo.quantize_summary(lo.build_page_summaries(K[:n_mr], w.rank, "f64")))
            else:
                summ = lo.build_page_summaries(K[:n_mr], w.rank, w.dtype)
            q = lo.storage_round(synth.queries(w, 0, s, h, T)[0], w.dtype)
            data.append((q, K, V, T, summ))
        conn.send(time.perf_counter() - t0)
        while conn.recv() == "step":
            t0 = time.perf_counter()
            for q, K, V, T, summ in data:
                lo.decode_head(q, K, V, T, summ, w.token_budget, w.scale)
            conn.send(time.perf_counter() - t0)


def cpu_baseline(w, lens_now, steps=3, workers=None, max_pairs=64):
    """The fp64 oracle's decode step (score + share + select + attend from its
    own resident summaries, at the lengths the GPU reached) on the host: every
    (sequence, KV head) pair of the batch (a seeded sample of max_pairs pairs
    when there are more, scaled by scored + attended pages), spread over
    ``workers`` processes of one thread each.  Each of ``steps`` whole steps
    is timed twice: with every worker at once (all cores) and with the
    workers one after another (one core).  Medians; the summary build is the
    untimed setup."""
    import multiprocessing as mp

    P = workers or min(16, len(os.sched_getaffinity(0)))
    all_pairs = [(s, h) for s in range(w.batch) for h in range(w.num_kv_heads)]
    B = w.page_size
    k = -(-w.token_budget // B)

    def cost(p):  # scored pages + attended pages of a pair
        return (lens_now[p[0]] - 1) // B + k

    pairs = all_pairs
    if len(all_pairs) > max_pairs:
        idx = np.random.default_rng(20261202).choice(len(all_pairs), size=max_pairs, replace=False)
        pairs = [all_pairs[i] for i in sorted(idx)]
    scale = sum(cost(p) for p in all_pairs) / sum(cost(p) for p in pairs)
    P = min(P, len(pairs))
    wargs = {"wid": w.wid, "rank": w.rank, "budget": w.token_budget, "steps": w.steps, "summary": w.summary,
             "batch": w.batch, "context": list(w.context)}

    def recv(i):  # a worker's reply, or an error if it has died
        while not conns[i].poll(1.0):
            if not procs[i].is_alive():
                raise RuntimeError(f"CPU baseline worker {i} ended (exit code {procs[i].exitcode})")
        return conns[i].recv()

    ctx = mp.get_context("fork")
    conns, procs = [], []
    for i in range(P):
        a, b = ctx.Pipe()
        pr = ctx.Process(target=_oracle_worker, args=(b, wargs, pairs[i::P], list(lens_now)), daemon=True)
        pr.start()
        conns.append(a)
        procs.append(pr)
    try:
        setup = max(recv(i) for i in range(P))
        t_all, t_one = [], []
        for _ in range(steps):
            t0 = time.perf_counter()
            for c in conns:
                c.send("step")
            for i in range(P):
                recv(i)
            t_all.append(time.perf_counter() - t0)
            one = 0.0
            for i, c in enumerate(conns):  # one worker at a time: one core busy
                c.send("step")
                one += recv(i)
            t_one.append(one)
    finally:
        for i, c in enumerate(conns):
            if procs[i].is_alive():
                c.send("quit")
        for pr in procs:
            pr.join(timeout=30)
            if pr.is_alive():
                pr.kill()
    med_all = float(np.median(t_all)) * scale
    med_one = float(np.median(t_one)) * scale
    how = (f"all {len(all_pairs)} (sequence, KV head) pairs" if pairs is all_pairs else
           f"a seeded sample of {len(pairs)} of {len(all_pairs)} pairs, scaled x{scale:.2f} by scored + "
           f"attended pages")
    return {"value": 1.0 / med_all, "unit": "steps/s", "cores": P, "kind": "oracle",
            "sample": f"{how} at the lengths the GPU reached, score + share + select + attend in fp64 from "
                      f"the oracle's own summaries; median of {steps} whole steps on {P} worker processes of "
                      f"one thread; summary build untimed ({setup:.1f}s)",
            "step_s_all_cores": med_all,
            "one_core": {"value": 1.0 / med_one, "unit": "steps/s", "cores": 1, "step_s": med_one},
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}


def cpu_baseline_child(argv):
    """Entry of the CPU-baseline child process (no GPU work in it): prints one
    JSON line."""
    p = argparse.ArgumentParser()
    p.add_argument("--workload", type=int)
    p.add_argument("--rank", type=int)
    p.add_argument("--budget", type=int)
    p.add_argument("--steps-done", type=int)
    p.add_argument("--summary")
    p.add_argument("--lens")
    p.add_argument("--context", default=None, help="initial lengths (default: the workload's)")
    p.add_argument("--cpu-steps", type=int, default=3)
    a = p.parse_args(argv)
    from long_context_sparse_page_amd import synth

    w = synth.workload(a.workload, rank=a.rank, budget=a.budget, steps=a.steps_done, summary=a.summary)
    if a.context:
        w.context = json.loads(a.context)
        w.batch = len(w.context)
    print(json.dumps(cpu_baseline(w, json.loads(a.lens), steps=a.cpu_steps)), flush=True)


def run_cpu_baseline(w, lens_now, cpu_steps):
    """The CPU baseline in a fresh child process (it holds no GPU state)."""
    import subprocess

    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--workload", str(w.wid),
           "--rank", str(w.rank), "--budget", str(w.token_budget), "--steps-done", str(w.steps),
           "--summary", w.summary, "--lens", json.dumps([int(t) for t in lens_now]),
           "--context", json.dumps([int(t) for t in w.context]),
           "--cpu-steps", str(cpu_steps)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    if r.returncode != 0:
        raise RuntimeError(f"CPU baseline failed:\n{r.stderr[-2000:]}")
    return json.loads(r.stdout.strip().splitlines()[-1])


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--cpu-baseline-child":
        cpu_baseline_child(sys.argv[2:])
    else:
        main()
