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
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--summary", choices=("kv", "i4"), default="kv",
                   help="page summaries in the KV dtype (bf16, the default) or int4 basis / int8 rows")
    p.add_argument("--workload", type=int, choices=(2, 3, 4), default=2,
                   help="2: 128K x 4 (the headline); 3: one 1M-token sequence; "
                        "4: 64 sequences of 4K..256K tokens (in-stream builds in most steps)")
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
    w = synth.workload(args.workload, steps=per_layer + 1 + -(-extra // args.layers), summary=args.summary)
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
        "in_stream_build": in_stream,
    }
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
        result["cpu_baseline"] = cpu_baseline(w, lens_now, args.cpu_seconds)
    print(json.dumps(result), flush=True)


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


def cpu_baseline(w, lens_now, seconds):
    """The fp64 oracle, single-threaded, on a bounded sample: one (sequence, KV
    head) pair of the same workload at the same length, its score + share +
    select + attend timed over repeated steps and scaled to a whole step
    (batch x KV heads pairs).  Its summary build is not timed."""
    from threadpoolctl import threadpool_limits

    from long_context_sparse_page_amd import synth
    from oracle import locks_oracle as lo

    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests"))
    import reference as ref

    T = lens_now[0]
    k = lo.page_budget(w.token_budget, w.page_size)
    # per-pair oracle cost grows with the scored and attended pages: other
    # lengths are scaled from the sampled pair by (n_mr + k)
    n0 = lo.most_recent_page(T, w.page_size) + k
    scale = sum(w.num_kv_heads * (lo.most_recent_page(t, w.page_size) + k) / n0 for t in lens_now)
    with threadpool_limits(limits=1):
        K, V = ref.host_pages(w, 0, 0, T)
        n_mr = lo.most_recent_page(T, w.page_size)
        summ = ref.oracle_summaries(w, K, n_mr)
        q64 = ref.stored(synth.queries(w, 0, 0, 0, T)[0], w.dtype)
        n, t0 = 0, time.perf_counter()
        while True:
            lo.decode_head(q64, K, V, T, summ, w.token_budget, w.scale)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    per_pair = el / n
    pairs = w.batch * w.num_kv_heads
    how = (f"scaled x{pairs} to one step" if len(set(lens_now)) == 1 else
           f"scaled x{scale:.1f} to one step's {pairs} pairs by scored + attended pages")
    return {"value": 1.0 / (per_pair * scale), "unit": "steps/s", "cores": 1, "kind": "oracle",
            "sample": f"1 of {pairs} (sequence, KV head) pairs at {T} tokens, {n} steps of score+share+select+"
                      f"attend in fp64 ({el:.1f}s), {how}; host has {os.cpu_count()} cores"}


if __name__ == "__main__":
    main()
