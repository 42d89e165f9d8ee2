"""The decode path at the pages' deployed page size of 16 tokens (needs an
MI355X): scoring, selection, attention and whole decode steps with in-stream
builds, against the fp64 oracle, for bf16 records, int4/int8 records and fp32.

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

B = 16


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def page16(wid=1, batch=2, ctx=(16 * 150 + 5, 16 * 37 + 16), rank=8, budget=512, steps=0, summary="kv",
           hq=32, hkv=8, dtype=None):
    w = synth.workload(wid, rank=rank, budget=budget, steps=steps, summary=summary)
    w.name = "page16"
    w.page_size = B
    w.batch = batch
    w.context = list(ctx)[:batch]
    w.num_q_heads, w.num_kv_heads = hq, hkv
    if dtype:
        w.dtype = dtype
    return w


def upload_oracle_records(dc, w, T):
    """The oracle's records (bf16 mirrored, or int4/int8 codes) for every
    (sequence, KV head); returns their PageSummary views for the oracle."""
    summ = {}
    for s in range(w.batch):
        n_mr = lo.most_recent_page(T[s], B)
        phys = torch.from_numpy(dc.block_table_host[s, :n_mr].astype(np.int64)).cuda()
        for h in range(w.num_kv_heads):
            K, _ = ref.host_pages(w, s, h, T[s])
            if w.summary == "i4":
                qs = ref.oracle_quant(w, K, n_mr)
                dc.summary_pool[phys, h] = torch.from_numpy(ref.pack_q4_records(qs)).cuda()
                summ[(s, h)] = lo.dequantize_summary(qs)
            else:
                sm = lo.build_page_summaries(K[:n_mr], w.rank, w.dtype)
                recs = np.concatenate([sm.centroid, sm.basis.reshape(n_mr, -1), sm.coeffs.reshape(n_mr, -1)], 1)
                dc.summary_pool[phys, h] = to_storage(recs.astype(np.float32), w.dtype).cuda()
                summ[(s, h)] = sm
    return summ


@pytest.mark.parametrize("summary,rank,group,hkv", [("kv", 8, 4, 8), ("i4", 8, 4, 8), ("kv", 4, 4, 8),
                                                    ("i4", 16, 4, 8), ("kv", 8, 1, 8), ("i4", 8, 1, 8),
                                                    ("kv", 16, 8, 2), ("i4", 8, 8, 2), ("i4", 4, 2, 4),
                                                    ("i4", 8, 4, 3)])
def test_page16_scorer_on_oracle_records(gpu, summary, rank, group, hkv):
    """Scorer isolation: the oracle's own records in the pool; page LSE within
    1e-3, shares, the selection at the 1e-4 band and attention over it, for
    GQA groups 1, 2, 4 and 8 and KV head counts 8, 4, 3 and 2 (3: the int4/int8
    scorer's grid split by division instead of a mask)."""
    w = page16(summary=summary, rank=rank, hq=group * hkv, hkv=hkv)
    say("page16 scorer on oracle records:", summary, "r", rank, "G", group, w.context)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth()
    T = w.context
    upload_oracle_records(dc, w, T)
    q64 = ref.host_queries(w, 0, T)
    qd = ref.q_device(q64, w.dtype)
    o = dc.outputs()
    dc.score_select(qd, o)
    dc.sparse_attn(qd, o["sel"], o["cnt"], o)
    torch.cuda.synchronize()
    tot = ref.check_all_pairs(w, dc, o, q64, T, share=True)
    say("page16 scorer isolation:", tot)
    assert tot.lse_own < 1e-4 and tot.lse_e2e < 1e-4


@pytest.mark.parametrize("summary,rank", [("kv", 8), ("i4", 8), ("kv", 16)])
def test_page16_end_to_end(gpu, summary, rank):
    """GPU-built records (the 16-token builder), every matching rule."""
    w = page16(summary=summary, rank=rank)
    say("page16 end to end:", summary, "r", rank, w.context)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth()
    dc.build_all()
    T = w.context
    q64 = ref.host_queries(w, 0, T)
    qd = ref.q_device(q64, w.dtype)
    o = dc.outputs()
    dc.score_select(qd, o)
    dc.sparse_attn(qd, o["sel"], o["cnt"], o)
    torch.cuda.synchronize()
    tot = ref.check_all_pairs(w, dc, o, q64, T, e2e_lse_gate=summary == "kv", share=True)
    say("page16 end to end:", tot)


@pytest.mark.parametrize("group,rank,ctx,budget", [(4, 8, (16 * 60 + 7,), 256), (1, 4, (16 * 33,), 128),
                                                   (8, 2, (16 * 80 + 1,), 512), (2, 16, (5,), 64),
                                                   (4, 8, (16 * 20 + 3,), 4096)])
def test_page16_fp32_variants(gpu, group, rank, ctx, budget):
    """fp32 K/V and records at 16 tokens: G in {1, 2, 4, 8}, ranks 2..16, a
    sequence within one page, a budget covering every page; page LSE,
    selection and attention (fp32 bar) against the oracle on the GPU's own
    records and on its own build."""
    w = page16(wid=0, batch=1, ctx=ctx, rank=rank, budget=budget, hq=group, hkv=1, dtype="f32")
    say("page16 fp32: G", group, "r", rank, "T", ctx, "b", budget)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth()
    dc.build_all()
    T = w.context
    q64 = ref.stored(np.random.default_rng(group * 10 + rank).standard_normal((1, group, 128)).astype(np.float32)
                     * 2, "f32")
    qd = ref.q_device(q64, w.dtype)
    o = dc.outputs()
    dc.score_select(qd, o)
    dc.sparse_attn(qd, o["sel"], o["cnt"], o)
    torch.cuda.synchronize()
    tot = ref.check_all_pairs(w, dc, o, q64, T, share=True)
    say("page16 fp32:", tot)


@pytest.mark.parametrize("summary", ["kv", "i4"])
def test_page16_decode_steps(gpu, summary):
    """lk_decode_step at 16 tokens over 40 steps: pages complete and are built
    in-stream every 16 steps of a sequence; a ragged batch with a one-token
    and an empty sequence; a poisoned workspace.  Checked every 8 steps with
    every matching rule, the page LSE from a score-only call of the same
    step."""
    w = page16(batch=4, ctx=(16 * 30 + 9, 16 * 7 + 15, 1, 0), steps=40, budget=256, summary=summary)
    say("page16 decode steps:", summary, w.context, "steps", w.steps)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth()
    dc.build_all()
    lens = list(w.context)
    kvs = {(s, h): synth.keys_values(w, s, h) for s in range(w.batch) for h in range(w.num_kv_heads)}
    tot = ref.PairCheck()
    for step in range(w.steps):
        new_lens = [t + 1 for t in lens]
        q64 = ref.host_queries(w, step, new_lens)
        kn = np.stack([np.stack([kvs[(s, h)][0][lens[s]] for h in range(w.num_kv_heads)]) for s in range(w.batch)])
        vn = np.stack([np.stack([kvs[(s, h)][1][lens[s]] for h in range(w.num_kv_heads)]) for s in range(w.batch)])
        o = dc.outputs()
        dc.decode_step(ref.q_device(q64, w.dtype), to_storage(kn, w.dtype).cuda(), to_storage(vn, w.dtype).cuda(), o)
        torch.cuda.synchronize()
        assert dc.seq_lens.cpu().tolist() == new_lens
        lens = new_lens
        if step % 8 != 7 and step != 0:
            continue
        o2 = dc.outputs()
        dc.score_select(ref.q_device(q64, w.dtype), o2)
        torch.cuda.synchronize()
        tot.merge(ref.check_all_pairs(w, dc, o, q64, lens, page_lse=o2["page_lse"].cpu().numpy(),
                                      e2e_lse_gate=summary == "kv"))
    say("page16 decode steps:", tot)


@pytest.mark.parametrize("group,dtype", [(1, "f32"), (2, "bf16"), (8, "f32")])
def test_page16_decode_step_groups(gpu, group, dtype):
    """lk_decode_step at 16 tokens for GQA groups 1, 2 and 8 (the builder
    launch merges each (sequence, KV head)'s split partials with one thread
    per output, so a group of 1 leaves most threads idle and a group of 8
    gives each thread two outputs): 18 steps
    over a ragged batch, so both sequences complete pages and build them
    in-stream; every matching rule at the first and the last step."""
    w = page16(wid=0, batch=2, ctx=(16 * 40 + 9, 16 * 12 + 14), steps=18, budget=256, hq=2 * group, hkv=2,
               dtype=dtype)
    say("page16 decode step groups: G", group, dtype, w.context, "steps", w.steps)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth()
    dc.build_all()
    lens = list(w.context)
    kvs = {(s, h): synth.keys_values(w, s, h) for s in range(w.batch) for h in range(w.num_kv_heads)}
    tot = ref.PairCheck()
    for step in range(w.steps):
        new_lens = [t + 1 for t in lens]
        q64 = ref.host_queries(w, step, new_lens)
        kn = np.stack([np.stack([kvs[(s, h)][0][lens[s]] for h in range(w.num_kv_heads)]) for s in range(w.batch)])
        vn = np.stack([np.stack([kvs[(s, h)][1][lens[s]] for h in range(w.num_kv_heads)]) for s in range(w.batch)])
        o = dc.outputs()
        dc.decode_step(ref.q_device(q64, w.dtype), to_storage(kn, w.dtype).cuda(), to_storage(vn, w.dtype).cuda(), o)
        torch.cuda.synchronize()
        assert dc.seq_lens.cpu().tolist() == new_lens
        lens = new_lens
        if step not in (0, w.steps - 1):
            continue
        o2 = dc.outputs()
        dc.score_select(ref.q_device(q64, w.dtype), o2)
        torch.cuda.synchronize()
        tot.merge(ref.check_all_pairs(w, dc, o, q64, lens, page_lse=o2["page_lse"].cpu().numpy()))
    say("page16 decode step groups:", tot)


def test_page16_dense_attention(gpu):
    """The same-GPU dense decode at 16 tokens against the oracle's dense attention."""
    w = page16(ctx=(16 * 300 + 11, 16 * 9 + 2))
    say("page16 dense attention", w.context)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth()
    T = w.context
    q64 = ref.host_queries(w, 0, T)
    o = dc.outputs()
    dc.dense_attn(ref.q_device(q64, w.dtype), o)
    torch.cuda.synchronize()
    out = o["out"].float().cpu().numpy().astype(np.float64)
    lse = o["lse"].cpu().numpy()
    G, d = w.group, w.head_dim
    worst = 0.0
    for s in range(w.batch):
        for h in range(w.num_kv_heads):
            K, V = ref.host_pages(w, s, h, T[s])
            eo, el = lo.attend(q64[s, h * G:(h + 1) * G], K.reshape(-1, d)[:T[s]], V.reshape(-1, d)[:T[s]], w.scale)
            e = ref.rel_l2(out[s, h * G:(h + 1) * G], eo).max()
            worst = max(worst, e)
            assert e <= ref.ATT_REL_BF16
            np.testing.assert_allclose(lse[s, h * G:(h + 1) * G], el, atol=ref.ATT_LSE_ATOL)
    say("page16 dense: max rel L2", worst)


@pytest.mark.parametrize("summary,budget,cap", [("kv", 512, 5000), ("i4", 1024, 5000), ("kv", 2048, 5000),
                                                ("i4", 2048, 9000)])
def test_page16_chunked_selection(gpu, summary, budget, cap):
    """A wide 16-token table (5,000 or 9,000 pages) with one (sequence, KV
    head) pair: the chunked selection with its merge launch, then the split
    attention, in lk_score_select; the decode step selects and attends in one
    launch up to 8,704 pages (lists of 128 or 256 entries at budgets of 32 and
    128 pages), and beyond through the chunk lists."""
    T = 16 * 4500 + 6
    w = page16(wid=1, batch=1, ctx=(T,), budget=budget, summary=summary, hq=4, hkv=1, steps=1)
    say("page16 chunked selection:", summary, "T", T, "budget", budget, "table", cap)
    dc = DeviceCache(w, poison=True, capacity_pages=[cap])
    dc.fill_from_synth()
    dc.build_all()
    q64 = ref.host_queries(w, 0, [T])
    qd = ref.q_device(q64, w.dtype)
    o = dc.outputs()
    dc.score_select(qd, o)
    dc.sparse_attn(qd, o["sel"], o["cnt"], o)
    torch.cuda.synchronize()
    tot = ref.check_all_pairs(w, dc, o, q64, [T], e2e_lse_gate=summary == "kv", share=True)
    say("page16 chunked score/select/attend:", tot)
    # one decode step appending token T (generator's next token)
    k, v = synth.keys_values(w, 0, 0)
    q64 = ref.host_queries(w, 1, [T + 1])
    o = dc.outputs()
    dc.decode_step(ref.q_device(q64, w.dtype), to_storage(k[T:T + 1][None], w.dtype).cuda(),
                   to_storage(v[T:T + 1][None], w.dtype).cuda(), o)
    torch.cuda.synchronize()
    assert dc.seq_lens.cpu().tolist() == [T + 1]
    o2 = dc.outputs()
    dc.score_select(ref.q_device(q64, w.dtype), o2)
    torch.cuda.synchronize()
    tot = ref.check_all_pairs(w, dc, o, q64, [T + 1], page_lse=o2["page_lse"].cpu().numpy(),
                              e2e_lse_gate=summary == "kv")
    say("page16 chunked decode step:", tot)


def test_page16_full_size_r8i4(gpu):
    """128K x 4 at 16 tokens with int4/int8 records (the bench's B = 16 line),
    in the decode step's launch configuration: 16 steps (one page completes per
    sequence), then sampled pairs against the oracle with every rule."""
    w = synth.workload(2, steps=16, summary="i4")
    w.page_size = B
    say("page16 full size r8i4: batch", w.batch, "tokens", w.context[0], "steps", w.steps)
    dc = DeviceCache(w, poison=True)
    dc.fill_from_synth(threads=16)
    dc.build_all()
    torch.cuda.synchronize()
    pairs = [(0, 3), (3, 6)]
    kvs = {p: synth.keys_values(w, *p) for p in pairs}
    hkv, G, d = w.num_kv_heads, w.group, w.head_dim
    lens = list(w.context)
    for step in range(w.steps):
        new_lens = [t + 1 for t in lens]
        rng = np.random.default_rng([16, step])
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
        lens = new_lens
    torch.cuda.synchronize()
    assert dc.seq_lens.cpu().tolist() == lens
    o2 = dc.outputs()
    dc.score_select(qd, o2)
    torch.cuda.synchronize()
    tot = ref.check_all_pairs(w, dc, o, q64, lens, pairs=pairs, page_lse=o2["page_lse"].cpu().numpy(),
                              e2e_lse_gate=False)
    say("page16 full size r8i4:", tot)
