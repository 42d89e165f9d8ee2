"""Diagnostic analogues of [Locks] Table B.1 (selection fidelity of page
scores) and Table D.17 (GQA combine rules) on the seeded synthetic carriers.

Scores compared, each ranked by share-average: the GPU's reconstructed-LSE
scores (lk_score_select on bf16 records and on int4/int8 records, rank 8)
against the oracle's rival scores (rank-8 moment core, envelope, centroid
only) and the exact page log-mass.  Per (sequence, KV head) and budget:
recall = overlap with the exact-mass top-(k-2) candidates; carrier retention
= carriers kept among those the exact selection keeps (the conditional form
of the pages' needle column); coverage = exact group-mean mass captured.
Combine rules (share-average, group-max, group-mass, per head) are compared on
exact scores, so only the rule differs.  The printed tables are the result;
the assertions hold what is proven (Cor. 3) and loose floors."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from long_context_sparse_page_amd import synth
from long_context_sparse_page_amd.paged import DeviceCache
from oracle import locks_oracle as lo

import reference as ref

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def test_rival_scores_and_combine_rules(gpu):
    T = 64 * 256 + 37
    budgets = (256, 512, 1024)
    w = synth.workload(1, batch=2)
    w.context = [T, T]
    w4 = synth.workload(1, batch=2, summary="i4")
    w4.context = [T, T]
    say("rival scores on synthetic carriers: 2 x", T, "tokens, 8 KV heads, G", w.group, "budgets", budgets)
    q64 = ref.host_queries(w, 0, w.context)
    gpu_lse = {}
    for name, wk in (("locks r8 bf16 (GPU)", w), ("locks r8i4 (GPU)", w4)):
        dc = DeviceCache(wk)
        dc.fill_from_synth(threads=16)
        dc.build_all()
        o = dc.outputs()
        dc.score_select(ref.q_device(q64, wk.dtype), o)
        torch.cuda.synchronize()
        gpu_lse[name] = o["page_lse"].cpu().numpy()
        del dc
    B, G, n_mr = w.page_size, w.group, lo.most_recent_page(T, w.page_size)
    scorers = ["locks r8 bf16 (GPU)", "locks r8i4 (GPU)", "moment core r8", "envelope", "centroid only"]
    stats = {(sc, b): {"recall": [], "carrier": [], "cover": []} for sc in scorers for b in budgets}
    rules = ("share_average", "group_max", "group_mass", "per_head")
    cover = {(r, b): [] for r in rules for b in budgets}
    for s in range(w.batch):
        for h in range(w.num_kv_heads):
            K, _ = ref.host_pages(w, s, h, T)
            qg = q64[s, h * G:(h + 1) * G]
            carriers = sorted({p for lst in synth.queries(w, 0, s, h, T)[1] for p in lst})
            exact = lo.exact_page_lse(qg, K[:n_mr], w.scale)
            summ = lo.build_page_summaries(K[:n_mr], w.rank, "f64")
            scores = {
                "locks r8 bf16 (GPU)": gpu_lse["locks r8 bf16 (GPU)"][s, h * G:(h + 1) * G, :n_mr],
                "locks r8i4 (GPU)": gpu_lse["locks r8i4 (GPU)"][s, h * G:(h + 1) * G, :n_mr],
                "moment core r8": lo.moment_core_score(qg, summ, w.scale),
                "envelope": lo.envelope_page_score(qg, K[:n_mr], w.scale),
                "centroid only": lo.centroid_score(qg, summ, w.scale),
            }
            for b in budgets:
                k = lo.page_budget(b, B)
                ex = set(lo.select_by_rule(exact, n_mr, k, "share_average")[0].tolist()) - {0, n_mr}
                kept = [c for c in carriers if c in ex]
                for sc, val in scores.items():
                    sel = lo.select_by_rule(val, n_mr, k, "share_average")[0]
                    got = set(sel.tolist()) - {0, n_mr}
                    st = stats[(sc, b)]
                    st["recall"].append(len(got & ex) / max(len(ex), 1))
                    if kept:
                        st["carrier"].append(sum(c in got for c in kept) / len(kept))
                    st["cover"].append(lo.head_coverage(exact, [sel] * G).mean())
                for r in rules:
                    cover[(r, b)].append(lo.head_coverage(exact, lo.select_by_rule(exact, n_mr, k, r)))
    say("selection fidelity (share-average ranking; mean over 16 (sequence, KV head) pairs)")
    say(f"{'scorer':22s}" + "".join(f" | b={b}: recall carrier cover" for b in budgets))
    for sc in scorers:
        cells = []
        for b in budgets:
            st = stats[(sc, b)]
            cells.append(f" | {np.mean(st['recall']):12.3f} {np.mean(st['carrier']):7.3f} {np.mean(st['cover']):5.3f}")
        say(f"{sc:22s}" + "".join(cells))
    say("GQA combine rules on exact scores (coverage per query head: mean, worst head, p5)")
    for r in rules:
        cells = []
        for b in budgets:
            c = np.stack(cover[(r, b)])      # [pairs, G]
            cells.append(f" | b={b}: {c.mean():.3f} {c.min(axis=1).mean():.3f} {np.quantile(c, 0.05):.3f}")
        say(f"{r:14s}" + "".join(cells))
    for b in budgets:
        sa = np.stack(cover[("share_average", b)]).mean(axis=1)
        for r in ("group_max", "group_mass"):
            assert (sa >= np.stack(cover[(r, b)]).mean(axis=1) - 1e-12).all()   # Cor. 3, per pair
        assert np.mean(stats[("locks r8 bf16 (GPU)", b)]["carrier"]) >= 0.9
        assert np.mean(stats[("locks r8 bf16 (GPU)", b)]["recall"]) >= np.mean(stats[("centroid only", b)]["recall"])
