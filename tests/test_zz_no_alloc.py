"""lk_decode_step_noalloc (the decode step whose workspace is the library's
static per-GPU buffer) against lk_decode_step with a caller's workspace, on
identical caches: two calls in a row, the second with a smaller batch; every
output, the stored lengths and the caches must be bit-identical (the two
entry points run the same kernels).  Needs an MI355X."""

from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from long_context_sparse_page_amd import locks as L
from long_context_sparse_page_amd import synth
from long_context_sparse_page_amd.paged import DeviceCache, to_storage

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _workload(kind):
    if kind == "fused":  # short tables: selection and attention in one launch
        w = synth.workload(1, budget=512, steps=4)
        w.batch, w.context = 4, [64 * 40 + 7, 64 * 9 + 63, 130, 64 * 25]
    else:  # a wide table and one (sequence, KV head) pair: the chunked selection
        w = synth.workload(0, budget=1024, steps=4)
        w.batch, w.context = 2, [64 * 700 + 40, 64 * 300 + 5]
    return w


def _cache(w, capacity):
    dc = DeviceCache(w, poison=True, capacity_pages=capacity)
    dc.fill_from_synth()
    dc.build_all()
    return dc


@pytest.mark.parametrize("kind", ["fused", "chunked"])
def test_noalloc_decode_step_matches_the_workspace_entry_point(gpu, kind):
    w = _workload(kind)
    cap = None if kind == "fused" else [5000, 5000]
    say("no-alloc decode step vs lk_decode_step:", kind, "lengths", w.context, "batch", w.batch)
    a, b = _cache(w, cap), _cache(w, cap)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    d, hkv, hq = w.head_dim, w.num_kv_heads, w.num_q_heads
    for call, batch in enumerate((w.batch, max(1, w.batch // 2))):
        q = to_storage(rng.standard_normal((batch, hq, d)).astype(np.float32), w.dtype).cuda()
        kn = to_storage(rng.standard_normal((batch, hkv, d)).astype(np.float32), w.dtype).cuda()
        vn = to_storage(rng.standard_normal((batch, hkv, d)).astype(np.float32), w.dtype).cuda()
        oa, ob = a.outputs(), b.outputs()
        say("call", call, "batch", batch)
        L.lk_decode_step(a.cfg, a.cache, batch, q, kn, vn, oa["out"], oa["lse"], oa["sel"], oa["cnt"], a.ws,
                         a.ws_bytes)
        L.lk_decode_step_noalloc(b.cfg, b.cache, batch, q, kn, vn, ob["out"], ob["lse"], ob["sel"], ob["cnt"])
        torch.cuda.synchronize()
        for key in ("out", "lse", "sel", "cnt"):
            x, y = oa[key], ob[key]
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            elif x.dtype == torch.float32:
                x, y = x.view(torch.int32), y.view(torch.int32)
            assert torch.equal(x, y), f"call {call}: {key} differs"
        assert torch.equal(a.seq_lens, b.seq_lens)
        for pool in ("k_pool", "v_pool", "summary_pool"):
            x, y = getattr(a, pool), getattr(b, pool)
            assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"call {call}: {pool} differs"
        got = a.seq_lens.cpu().tolist()
        want = [t + 1 + (call if s < batch else 0) for s, t in enumerate(w.context)]
        assert got == want, (got, want)
        cnt = oa["cnt"].cpu().numpy()
        assert (cnt[:batch] > 0).all()
    say("bit-identical over both calls")
