"""Page LSEs of pages whose deviation logits are extreme (needs an MI355X).

At 64-token pages the scorer forms a page's LSE as its centroid logit plus
log sum_i exp(d_i) over the tokens' deviation logits d_i ([Locks] §4
"Score", Eq. (1), split at the centroid), and takes page maxima only for a
wave in which a sum leaves [2^-64, 2^64]; at 16-token pages it always takes
them.  These cases plant such pages among ordinary ones: one
token far above its centroid (the plain sum overflows), every token far
below it (the sum underflows), one token just past the range, one token
just inside it, one token far below.  The page LSE of every scored page is
compared with the oracle on the same records (1e-3).

Every case prints its name and shapes before touching the GPU."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from long_context_sparse_page_amd import synth
from long_context_sparse_page_amd.paged import DeviceCache, to_storage
from oracle import locks_oracle as lo

import reference as ref

pytestmark = pytest.mark.gpu

# (page, token or None for every token, deviation of the group's first query head in nats)
PLANTS = [(1, 0, 120.0), (2, None, -100.0), (5, 3, 50.0), (7, 1, 38.0), (9, 2, -200.0)]


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def lse_workload(B, summary):
    w = synth.workload(1, rank=8, budget=512, steps=0, summary=summary)
    w.name = "lse-range"
    w.page_size = B
    w.batch = 2
    w.context = [B * 40 + 9, B * 23 + 5]
    w.num_q_heads, w.num_kv_heads = 8, 2
    return w


def planted_summary(w, K, n, q0):
    """The oracle's summary of the first n pages with PLANTS written into the
    coefficients (in fp64, before the records are stored or quantized)."""
    sm = lo.build_page_summaries(K[:n], w.rank, "f64")
    coeffs = sm.coeffs.copy()
    for j, t, x in PLANTS:
        u = sm.basis[j] @ q0                      # V_j^T q
        c = (x / w.scale) * u / float(u @ u)      # scale * u . c = x
        if t is None:
            coeffs[j, :] = c
        else:
            coeffs[j, t] = c
    return lo.PageSummary(centroid=sm.centroid, basis=sm.basis, coeffs=coeffs, eigvals=sm.eigvals, r_eff=sm.r_eff)


@pytest.mark.parametrize("B,summary", [(64, "kv"), (64, "i4"), (16, "kv"), (16, "i4")])
def test_page_lse_extreme_deviations(gpu, B, summary):
    w = lse_workload(B, summary)
    say("page LSE with extreme deviations: B", B, summary, w.context)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth()
    T = w.context
    q64 = ref.host_queries(w, 0, T)
    G = w.group
    seen = {"over": 0, "under": 0, "inside": 0}
    oracle = {}
    for s in range(w.batch):
        n = lo.most_recent_page(T[s], B)
        phys = torch.from_numpy(dc.block_table_host[s, :n].astype(np.int64)).cuda()
        for h in range(w.num_kv_heads):
            K, _ = ref.host_pages(w, s, h, T[s])
            qg = q64[s, h * G:(h + 1) * G]
            sm = planted_summary(w, K, n, qg[0])
            if summary == "i4":
                qs = lo.quantize_summary(sm)
                dc.summary_pool[phys, h] = torch.from_numpy(ref.pack_q4_records(qs)).cuda()
                seen_sm = lo.dequantize_summary(qs)
            else:
                parts = [lo.storage_round(x, w.dtype) for x in (sm.centroid, sm.basis, sm.coeffs)]
                seen_sm = lo.PageSummary(centroid=parts[0], basis=parts[1], coeffs=parts[2], eigvals=sm.eigvals,
                                         r_eff=sm.r_eff)
                recs = np.concatenate([parts[0], parts[1].reshape(n, -1), parts[2].reshape(n, -1)], axis=1)
                dc.summary_pool[phys, h] = to_storage(recs.astype(np.float32), w.dtype).cuda()
            oracle[(s, h)] = lo.reconstructed_page_lse(qg, seen_sm, w.scale)
            # which side of the plain sum's range the planted pages fall on (head 0, log2 units)
            dev = w.scale * np.log2(np.e) * np.einsum("nbr,nr->nb", seen_sm.coeffs, seen_sm.basis @ qg[0])
            for j, _, _ in PLANTS:
                tot = np.log2(np.sum(np.exp2(dev[j] - dev[j].max()))) + dev[j].max()
                seen["over" if tot > 64 else ("under" if tot < -64 else "inside")] += 1
    assert seen["over"] >= w.batch * w.num_kv_heads and seen["under"] >= w.batch * w.num_kv_heads, seen
    assert seen["inside"] >= w.batch * w.num_kv_heads, seen
    o = dc.outputs()
    dc.score_select(ref.q_device(q64, w.dtype), o)
    torch.cuda.synchronize()
    page_lse = o["page_lse"].cpu().numpy()
    worst = 0.0
    for (s, h), want in oracle.items():
        n = want.shape[1]
        got = page_lse[s, h * G:(h + 1) * G, :n]
        assert np.isfinite(got).all(), f"seq {s} head {h}: non-finite page LSE"
        err = np.abs(got - want).max()
        worst = max(worst, err)
        assert err <= 1e-3, f"seq {s} KV head {h}: page LSE error {err:.3g}"
        for j, _, x in PLANTS:
            assert abs(got[0, j] - want[0, j]) <= 1e-3
    say("max page LSE error", worst, "planted pages by side of the range", seen)
