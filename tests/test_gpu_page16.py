"""Pages of 16 tokens on the GPU builder (needs an MI355X).

The summaries of the 16-token builder against the fp64 oracle (fp32 and bf16
records, int4/int8 records), and the isotropic null of the Locks appendix
("Spectral tails": a rank-8 fit of 20,000 flat-spectrum B = 16 pages captures
a median 67.8% of their variance) reproduced from the GPU builder's
eigenvalues.  Every case prints its name and shapes before touching the GPU."""

from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest
import torch

from long_context_sparse_page_amd import locks as L
from long_context_sparse_page_amd import synth
from long_context_sparse_page_amd.paged import to_storage
from oracle import locks_oracle as lo

import reference as ref

pytestmark = pytest.mark.gpu

B, D = 16, 128


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def structured_keys(n, hkv):
    """fp32 [n][Hkv][16][128]: the synthetic key model (page-specific rank 8,
    shared rank 4, noise) on 16-token pages, plus special pages on KV head 0:
    page 0 constant (no nonzero mode), page 1 of rank 2, page 2 with every
    token repeated once (rank <= 7)."""
    w = synth.workload(0)
    w.page_size = B
    w.context = [n * B]
    w.steps = 0
    keys = np.stack([synth.keys_values(w, 0, h)[0].reshape(n, B, D) for h in range(hkv)], axis=1)
    k0 = keys[:, 0]
    k0[0] = k0[0, 3]
    k0[1] = k0[1, :1] + np.outer(np.linspace(-1, 1, B), k0[1, 5] - k0[1, 6]) \
        + np.outer(np.cos(np.arange(B)), k0[1, 7] - k0[1, 8])
    k0[2, 8:] = k0[2, :8]
    return np.ascontiguousarray(keys, dtype=np.float32)


def build16(keys, rank, dtype, fmt=L.LK_SUMMARY_KV, spare=5, seed=0):
    """Place page i of keys [n][Hkv][16][128] at a shuffled physical slot of a
    pool with ``spare`` extra slots, list the pages with -1 entries between
    them, build, and return (records [n][Hkv][...], eigenvalues [n][Hkv][16],
    stored keys as fp64 [n][Hkv][16][128], spare records)."""
    n, hkv = keys.shape[:2]
    cfg = L.make_config(page_size=B, rank=rank, num_q_heads=hkv, num_kv_heads=hkv, token_budget=256,
                        kv_dtype=L.LK_BF16 if dtype == "bf16" else L.LK_F32, summary_format=fmt)
    rb = L.lk_summary_record_bytes(cfg)
    n_phys = n + spare
    phys = np.random.default_rng(seed).permutation(n_phys)
    kstore = to_storage(keys.reshape(n, hkv * B * D), dtype).reshape(n, hkv, B, D)
    kpool = torch.zeros((n_phys, hkv, B, D), dtype=kstore.dtype)
    kpool[torch.from_numpy(phys[:n])] = kstore
    kpool = kpool.cuda()
    if fmt == L.LK_SUMMARY_I4:
        spool = torch.full((n_phys, hkv, rb), 0xAB, dtype=torch.uint8, device="cuda")
    else:
        spool = torch.full((n_phys, hkv, rb // kstore.element_size()), float("nan"), dtype=kstore.dtype,
                           device="cuda")
    ids = np.full(2 * n, -1, dtype=np.int32)
    ids[0::2] = phys[:n]
    ids_t = torch.from_numpy(ids).cuda()
    ev = torch.full((2 * n, hkv, B), -1.0, dtype=torch.float32, device="cuda")
    cache = L.lk_cache(k_pool=kpool.data_ptr(), v_pool=None, summary_pool=spool.data_ptr(), block_table=None,
                       seq_lens=None, max_pages_per_seq=1, num_phys_pages=n_phys)
    L.lk_build_page_summary(cfg, cache, ids_t, 2 * n, ev, None, 0, None)
    torch.cuda.synchronize()
    recs = spool.cpu()
    ev = ev.cpu().numpy()
    assert (ev[1::2] == -1.0).all(), "skipped list entries wrote eigenvalues"
    held = recs[torch.from_numpy(phys[n:])]
    if fmt == L.LK_SUMMARY_I4:
        assert (held == 0xAB).all(), "a page outside the list was written"
    else:
        assert torch.isnan(held.float()).all(), "a page outside the list was written"
    return recs[torch.from_numpy(phys[:n])], ev[0::2], kstore.double().numpy(), rb


@pytest.mark.parametrize("dtype,rank", [("f32", 8), ("f32", 4), ("f32", 16), ("bf16", 8)])
def test_page16_build_matches_oracle(gpu, dtype, rank):
    n, hkv = 96, 2
    say("16-token build", dtype, "pages", n, "KV heads", hkv, "r", rank)
    recs, ev, kst, _ = build16(structured_keys(n, hkv), rank, dtype)
    recs = recs.double().numpy() if dtype == "f32" else recs.float().double().numpy()
    tol = 2e-4 if dtype == "f32" else 2.0 ** -8
    compared = 0
    for h in range(hkv):
        summ = lo.build_page_summaries(kst[:, h], rank, dtype)
        lam1 = summ.eigvals[:, :1]
        assert (np.abs(ev[:, h] - summ.eigvals) <= 1e-5 * np.maximum(lam1, 1e-30) + 1e-6).all()
        cen, bas = recs[:, h, :D], recs[:, h, D:D + rank * D].reshape(n, rank, D)
        co = recs[:, h, D + rank * D:].reshape(n, B, rank)
        np.testing.assert_allclose(cen, summ.centroid, rtol=tol, atol=1e-6)
        # zero modes written as zeros, on every page
        r_eff = summ.r_eff
        for i in range(n):
            assert np.abs(bas[i, r_eff[i]:]).max(initial=0) == 0 and np.abs(co[i, :, r_eff[i]:]).max(initial=0) == 0
        # each basis row and coefficient column whose eigenvalue is isolated
        # (1e-2 lambda_1 from its neighbours; a mode is defined only up to
        # rotations inside a cluster)
        k = np.minimum(r_eff, rank)
        lam = summ.eigvals
        for i in range(n):
            for m in range(k[i]):
                gaps = [abs(lam[i, m] - lam[i, m + 1])] + ([abs(lam[i, m] - lam[i, m - 1])] if m else [])
                if min(gaps) < 1e-2 * lam[i, 0]:
                    continue
                compared += 1
                np.testing.assert_allclose(bas[i, m], summ.basis[i, m], rtol=tol, atol=tol)
                np.testing.assert_allclose(co[i, :, m], summ.coeffs[i, :, m], rtol=tol,
                                           atol=tol * np.abs(summ.coeffs).max())
        # every page: the nonzero basis rows are orthonormal; with every
        # nonzero mode kept, mu + C V gives back the keys
        for i in range(n):
            g = bas[i, :k[i]] @ bas[i, :k[i]].T
            assert np.abs(g - np.eye(k[i])).max(initial=0) < (1e-4 if dtype == "f32" else 2e-2)
            if rank >= B - 1:
                back = cen[i] + co[i] @ bas[i]
                err = np.abs(back - kst[i, h]).max() / np.abs(kst[i, h]).max()
                assert err < (2e-5 if dtype == "f32" else 2e-2), (i, err)
    say("isolated modes compared", compared, "of", n * hkv * rank)
    assert compared >= n * hkv * min(rank, 8) // 2


def test_page16_special_pages(gpu):
    """Constant page: no nonzero mode (all-zero basis and coefficients, centroid
    = the key); rank-2 page: two modes; repeated tokens: rank <= 7."""
    n = 8
    say("16-token build special pages f32, pages", n)
    keys = structured_keys(n, 1)
    recs, ev, kst, _ = build16(keys, 8, "f32")
    recs = recs.double().numpy()[:, 0]
    assert np.abs(recs[0, D:]).max() == 0.0
    np.testing.assert_allclose(recs[0, :D], kst[0, 0, 0], rtol=1e-6, atol=1e-6)
    assert ev[0, 0].max() <= 1e-6 * (kst[0, 0] ** 2).sum()
    summ = lo.build_page_summaries(kst[:, 0], 8, "f32")
    assert summ.r_eff[1] == 2 and summ.r_eff[2] <= 7
    bas1 = recs[1, D:D + 8 * D].reshape(8, D)
    assert np.abs(bas1[2:]).max() == 0.0 and (np.abs(bas1[:2]).max(axis=1) > 0).all()
    bas2 = recs[2, D:D + 8 * D].reshape(8, D)
    assert np.abs(bas2[summ.r_eff[2]:]).max(initial=0) == 0.0


@pytest.mark.parametrize("rank", [4, 8])
def test_page16_q4_build_matches_oracle(gpu, rank):
    n, hkv = 96, 2
    say("16-token int4/int8 build, pages", n, "KV heads", hkv, "r", rank)
    recs, _, kst, rb = build16(structured_keys(n, hkv), rank, "bf16", fmt=L.LK_SUMMARY_I4)
    assert rb == ref.q4_offsets(D, B, rank)["bytes"]
    recs = recs.numpy()
    compared = 0
    for h in range(hkv):
        summ = lo.build_page_summaries(kst[:, h], rank, "f64")
        qs = lo.quantize_summary(summ)
        g = ref.unpack_q4_records(recs[:, h], D, B, rank)
        ref.codes_match(g.centroid_q, qs.centroid_q, g.centroid_s, qs.centroid_s, summ.centroid, 0.01)
        k = np.minimum(summ.r_eff, rank)
        lam = summ.eigvals
        sep = np.array([np.min(np.abs(np.diff(lam[i, :k[i] + 1])), initial=np.inf) / max(lam[i, 0], 1e-30)
                        for i in range(n)])
        ok = (sep >= 1e-2) & (k == rank)
        compared += int(ok.sum())
        if ok.any():
            ref.codes_match(g.basis_q[ok], qs.basis_q[ok], g.basis_s[ok], qs.basis_s[ok], summ.basis[ok], 0.01)
            ref.codes_match(g.coeffs_q[ok], qs.coeffs_q[ok], g.coeffs_s[ok], qs.coeffs_s[ok],
                            summ.coeffs[ok], 0.05)
        # zero-padding bytes after the centroid scale
        o = ref.q4_offsets(D, B, rank)
        assert (recs[:, h, o["mscale"] + 2:] == 0).all()
    say("pages with separated modes", compared, "of", n * hkv)
    assert compared >= n * hkv // 4


def test_page16_isotropic_null(gpu, golden_dir):
    """Median / mean / sd of the rank-8 captured fraction over 20,000 isotropic
    16-token pages from the GPU builder's eigenvalues, against the printed
    statistic, and page by page against the oracle's eigenvalues."""
    g = json.load(open(os.path.join(golden_dir, "isotropic_null.json")))
    n, hkv = g["pages"] // 4, 4
    say("isotropic null on the GPU builder:", g["pages"], "pages of", g["page_size"], "x", g["head_dim"],
        "r", g["rank"])
    keys = synth.isotropic_pages(g["pages"], g["page_size"], g["head_dim"]).reshape(n, hkv, B, D)
    _, ev, kst, _ = build16(keys, g["rank"], "f32", spare=0)
    ev = ev.reshape(-1, B).astype(np.float64)
    fr = ev[:, :g["rank"]].sum(1) / ev.sum(1)
    say("captured fraction: median", np.median(fr), "mean", fr.mean(), "sd", fr.std())
    tol = g["printed_precision"]
    assert abs(np.median(fr) - g["median"]) <= tol["median"] + 3e-4
    assert abs(fr.mean() - g["mean"]) <= tol["mean"] + 3e-4
    assert abs(fr.std() - g["std"]) <= tol["std"] + 3e-4
    # page by page against the oracle (same stored fp32 keys)
    summ = lo.build_page_summaries(kst.reshape(-1, B, D), g["rank"], "f64")
    lam1 = summ.eigvals[:, :1]
    assert (np.abs(ev - summ.eigvals) <= 1e-5 * lam1).all()
    fo = summ.eigvals[:, :g["rank"]].sum(1) / summ.eigvals.sum(1)
    assert np.abs(fr - fo).max() <= 1e-5


def test_page16_full_size_bulk(gpu):
    """The bulk build the bench times: the 128K x 4 keys (32 q / 8 KV heads,
    bf16) re-paged into 32,768 pages of 16 tokens, int4/int8 records at r = 8,
    one lk_build_page_summary call over all 262,144 page-heads; sampled
    page-heads against the oracle (codes and scales), every eigenvalue output
    checked for order and sign."""
    from long_context_sparse_page_amd.paged import DeviceCache

    w = synth.workload(2, steps=0)
    say("16-token bulk build at full size:", w.name, "pages of 16:", sum(w.context) // B, "KV heads", w.num_kv_heads)
    dc = DeviceCache(w)
    dc.fill_from_synth(threads=16)
    torch.cuda.synchronize()
    hkv = w.num_kv_heads
    src = torch.cat([dc.k_pool[torch.from_numpy(dc.block_table_host[s, :w.context[s] // 64].astype(np.int64)).cuda()]
                     for s in range(w.batch)])
    k16 = src.view(-1, hkv, 64 // B, B, D).permute(0, 2, 1, 3, 4).reshape(-1, hkv, B, D).contiguous()
    del src
    n = int(k16.shape[0])
    cfg = L.make_config(D, B, 8, w.num_q_heads, hkv, w.token_budget, L.LK_BF16, w.scale, L.LK_SUMMARY_I4)
    rb = L.lk_summary_record_bytes(cfg)
    spool = torch.full((n, hkv, rb), 0xAB, dtype=torch.uint8, device="cuda")
    ev = torch.full((n, hkv, B), -1.0, dtype=torch.float32, device="cuda")
    cache = L.make_cache(k16, None, spool, dc.block_table, dc.seq_lens)
    ids = torch.arange(n, dtype=torch.int32, device="cuda")
    L.lk_build_page_summary(cfg, cache, ids, n, ev, None, 0, None)
    torch.cuda.synchronize()
    evh = ev.cpu().numpy()
    assert (evh >= 0).all() and (np.diff(evh, axis=2) <= 0).all(), "eigenvalues not sorted descending / negative"
    rng = np.random.default_rng(16)
    pick = rng.choice(n * hkv, size=256, replace=False)
    pg, hd = pick // hkv, pick % hkv
    keys = k16[torch.from_numpy(pg).cuda(), torch.from_numpy(hd).cuda()].double().cpu().numpy()
    recs = spool[torch.from_numpy(pg).cuda(), torch.from_numpy(hd).cuda()].cpu().numpy()
    say("sampled page-heads", len(pick))
    summ = lo.build_page_summaries(keys, 8, "f64")
    lam1 = summ.eigvals[:, :1]
    assert (np.abs(evh[pg, hd] - summ.eigvals) <= 1e-5 * lam1).all()
    qs = lo.quantize_summary(summ)
    g = ref.unpack_q4_records(recs, D, B, 8)
    ref.codes_match(g.centroid_q, qs.centroid_q, g.centroid_s, qs.centroid_s, summ.centroid, 0.01)
    k = np.minimum(summ.r_eff, 8)
    lam = summ.eigvals
    sep = np.array([np.min(np.abs(np.diff(lam[i, :k[i] + 1])), initial=np.inf) / max(lam[i, 0], 1e-30)
                    for i in range(len(pick))])
    ok = (sep >= 1e-2) & (k == 8)
    say("page-heads with separated modes", int(ok.sum()), "of", len(pick))
    assert ok.sum() >= len(pick) // 4
    fb = ref.codes_match(g.basis_q[ok], qs.basis_q[ok], g.basis_s[ok], qs.basis_s[ok], summ.basis[ok], 0.01)
    fc = ref.codes_match(g.coeffs_q[ok], qs.coeffs_q[ok], g.coeffs_s[ok], qs.coeffs_s[ok], summ.coeffs[ok], 0.05)
    say("differing codes: basis", fb, "coefficients", fc)
