"""Parity at the full workload sizes, in the launch configuration the bench
times (lk_decode_step over the whole batch), with the fp64 oracle run on
sampled (sequence, KV head) pairs and structural checks on every output.

Per workload: fill and bulk-build the cache, run two decode steps; after the
last one
  * every (sequence, KV head): the selection is well formed (ascending,
    unique, sink and most recent page present, size min(k, n_mr + 1), -1
    padding), outputs and LSEs are finite, lengths advanced;
  * sampled pairs, end to end (GPU-built bf16 records): selection within the
    share band of the oracle's cut, attention over the GPU's selection against
    the oracle's attention over the same pages, page LSE against the oracle's;
  * sampled pairs, scorer isolation: the oracle's records are written into
    the summary pool and lk_score_select is compared with the oracle exactly
    (page LSE 1e-3, selection band 1e-4 relative).
Queries and appended tokens of the sampled pairs come from the seeded
generator; the other pairs get seeded Gaussian queries and tokens."""

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


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _pairs(w, n, seed):
    """n distinct (sequence, KV head) pairs: the shortest and the longest
    sequence first, then random ones."""
    rng = np.random.default_rng(seed)
    order = np.argsort(w.context, kind="stable")
    seqs = [int(order[0]), int(order[-1])] + [int(x) for x in rng.integers(w.batch, size=4 * n)]
    out = []
    for s in seqs:
        p = (s, int(rng.integers(w.num_kv_heads)))
        if p not in out:
            out.append(p)
        if len(out) == n:
            break
    return out


def _check_structure(w, sel, cnt, out, lse, lens):
    k = lo.page_budget(w.token_budget, w.page_size)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    for s in range(w.batch):
        n_mr = lo.most_recent_page(lens[s], w.page_size)
        want = min(k, n_mr + 1)
        for h in range(w.num_kv_heads):
            c = int(cnt[s, h])
            g = sel[s, h]
            assert c == want, f"seq {s} head {h}: count {c} != {want}"
            assert (np.diff(g[:c]) > 0).all() and g[0] == 0 and g[c - 1] == n_mr, (s, h, g[:c])
            assert (g[c:] == -1).all()


@pytest.mark.parametrize("wid,rank,budget,summary", [
    (1, None, None, "kv"),    # 32K x 8
    (2, None, None, "kv"),    # 128K x 4 (the bench workload)
    (3, None, None, "kv"),    # one 1M-token sequence
    (4, None, None, "kv"),    # 64 sequences, 4K..256K, r = 8, b = 1024
    (4, 4, 256, "kv"),
    (4, 16, 4096, "kv"),
    (2, None, None, "i4"),    # 128K x 4 with int4 / int8 summary records
    (3, None, None, "i4"),    # one 1M-token sequence with int4 / int8 records (chunked selection)
])
def test_full_size_decode(gpu, wid, rank, budget, summary):
    steps = 2
    w = synth.workload(wid, rank=rank, budget=budget, steps=steps, summary=summary)
    say("full size", w.name, "r", w.rank, "b", w.token_budget, "batch", w.batch,
        "tokens", sum(w.context), "steps", steps, "summary", w.summary)
    dc = DeviceCache(w)
    dc.fill_from_synth(threads=16)
    dc.build_all()
    torch.cuda.synchronize()
    pairs = _pairs(w, 2 if wid in (3, 4) else 3, 1000 + wid)
    say("sampled pairs", pairs)
    hkv, G, d = w.num_kv_heads, w.group, w.head_dim
    rng = np.random.default_rng(77 + wid)
    kvs = {p: synth.keys_values(w, *p) for p in pairs}
    say("cache filled and summarized; sampled keys regenerated")
    lens = list(w.context)
    for step in range(steps):
        new_lens = [t + 1 for t in lens]
        q = rng.standard_normal((w.batch, w.num_q_heads, d)).astype(np.float32)
        kn = rng.standard_normal((w.batch, hkv, d)).astype(np.float32)
        vn = rng.standard_normal((w.batch, hkv, d)).astype(np.float32)
        for (s, h) in pairs:
            q[s, h * G:(h + 1) * G] = synth.queries(w, step, s, h, new_lens[s])[0]
            kn[s, h] = kvs[(s, h)][0][lens[s]]
            vn[s, h] = kvs[(s, h)][1][lens[s]]
        q64 = ref.stored(q, w.dtype)
        qd = ref.q_device(q64, w.dtype)
        o = dc.outputs()
        dc.decode_step(qd, to_storage(kn, w.dtype).cuda(), to_storage(vn, w.dtype).cuda(), o)
        torch.cuda.synchronize()
        assert dc.seq_lens.cpu().tolist() == new_lens
        lens = new_lens
    sel = o["sel"].cpu().numpy()
    cnt = o["cnt"].cpu().numpy()
    out = o["out"].float().cpu().numpy().astype(np.float64)
    lse = o["lse"].cpu().numpy()
    _check_structure(w, sel, cnt, out, lse, lens)
    say("structure ok for", w.batch * hkv, "pairs")

    # page LSE of the same step (the decode step keeps it internal)
    o2 = dc.outputs()
    dc.score_select(qd, o2)
    torch.cuda.synchronize()
    page_lse = o2["page_lse"].cpu().numpy()
    k = lo.page_budget(w.token_budget, w.page_size)
    oracle = {}
    worst_lse, worst_l2 = 0.0, 0.0
    B = w.page_size
    for (s, h) in pairs:
        say("oracle for seq", s, "head", h, "tokens", lens[s])
        n_pages = -(-lens[s] // B)
        K = np.zeros((n_pages * B, d))
        V = np.zeros((n_pages * B, d))
        K[:lens[s]] = ref.stored(kvs[(s, h)][0][:lens[s]], w.dtype)
        V[:lens[s]] = ref.stored(kvs[(s, h)][1][:lens[s]], w.dtype)
        K, V = K.reshape(n_pages, B, d), V.reshape(n_pages, B, d)
        qg = q64[s, h * G:(h + 1) * G]
        hs, summ = ref.oracle_head(w, qg, K, V, lens[s])
        oracle[(s, h)] = (hs, summ if w.summary == "kv" else ref.oracle_quant(w, K, summ.centroid.shape[0]))
        n_mr = lo.most_recent_page(lens[s], w.page_size)
        gsel = sel[s, h, :cnt[s, h]]
        msg = ref.selection_mismatch(gsel, hs.selected, hs.m_bar, n_mr, k, rel=2e-2)
        assert msg is None, f"seq {s} head {h}: {msg}"
        eo, _ = lo.attend(qg, lo.gather_tokens(K, gsel, lens[s], w.page_size),
                          lo.gather_tokens(V, gsel, lens[s], w.page_size), w.scale)
        e = ref.rel_l2(out[s, h * G:(h + 1) * G], eo).max()
        worst_l2 = max(worst_l2, e)
        assert e <= 2e-2, f"seq {s} head {h}: attention rel L2 {e}"
        err = np.abs(page_lse[s, h * G:(h + 1) * G, :n_mr] - hs.page_lse).max()
        worst_lse = max(worst_lse, err)
        assert err < 1e-2, f"seq {s} head {h}: end-to-end page LSE error {err}"
    say("end to end: max page LSE error", worst_lse, "max attention rel L2", worst_l2)

    # scorer isolation: the oracle's records for the sampled pairs
    for (s, h), (hs, summ) in oracle.items():
        if w.summary == "i4":
            n = summ.centroid_q.shape[0]
            phys = torch.from_numpy(dc.block_table_host[s, :n].astype(np.int64)).cuda()
            dc.summary_pool[phys, h] = torch.from_numpy(ref.pack_q4_records(summ)).cuda()
            continue
        n = summ.centroid.shape[0]
        recs = np.concatenate([summ.centroid, summ.basis.reshape(n, -1), summ.coeffs.reshape(n, -1)], axis=1)
        phys = torch.from_numpy(dc.block_table_host[s, :n].astype(np.int64)).cuda()
        dc.summary_pool[phys, h] = to_storage(recs.astype(np.float32), w.dtype).cuda()
    o3 = dc.outputs()
    dc.score_select(qd, o3)
    torch.cuda.synchronize()
    page_lse = o3["page_lse"].cpu().numpy()
    share = o3["share"].cpu().numpy()
    sel3 = o3["sel"].cpu().numpy()
    cnt3 = o3["cnt"].cpu().numpy()
    worst = 0.0
    for (s, h), (hs, summ) in oracle.items():
        n_mr = lo.most_recent_page(lens[s], w.page_size)
        err = np.abs(page_lse[s, h * G:(h + 1) * G, :n_mr] - hs.page_lse).max()
        worst = max(worst, err)
        assert err <= 1e-3, f"seq {s} head {h}: page LSE error {err}"
        np.testing.assert_allclose(share[s, h, :n_mr], hs.m_bar, rtol=5e-3, atol=1e-7)
        msg = ref.selection_mismatch(sel3[s, h, :cnt3[s, h]], hs.selected, hs.m_bar, n_mr, k)
        assert msg is None, f"seq {s} head {h}: {msg}"
    say("scorer isolation: max page LSE error", worst)
