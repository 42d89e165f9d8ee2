"""Device-memory plumbing for the Locks decode path (torch allocations only).

``DeviceCache`` owns the paged K/V pools, the summary pool, the block table,
the sequence lengths and the workspace of one attention layer, allocated with
torch on the GPU and described to the C ABI by ``lk_cache``.  Physical pages
are handed out in a seeded random order (``perm_seed``; None hands them out in
order) so every kernel exercises the block table.  It performs no step of the method: K/V come from ``synth`` (or the
caller), summaries from ``lk_build_page_summary``.
"""

from __future__ import annotations

import concurrent.futures as cf

import numpy as np
import torch

from . import locks as L
from . import synth

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}
LK_DTYPE = {"f32": L.LK_F32, "bf16": L.LK_BF16}


def to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    """fp32 array -> CPU tensor in the storage dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(TORCH_DTYPE[dtype])


class DeviceCache:
    def __init__(self, w: synth.Workload, device: str = "cuda", perm_seed: int | None = 1,
                 poison: bool = False, capacity_pages: list | None = None, ws_fill: int | None = None):
        self.w = w
        self.device = device
        self.cfg = L.make_config(w.head_dim, w.page_size, w.rank, w.num_q_heads, w.num_kv_heads,
                                 w.token_budget, LK_DTYPE[w.dtype], w.scale,
                                 L.LK_SUMMARY_I4 if w.summary == "i4" else L.LK_SUMMARY_KV)
        B, d, hkv = w.page_size, w.head_dim, w.num_kv_heads
        pages = capacity_pages or [w.pages_needed(s) for s in range(w.batch)]
        self.max_pages = max(pages)
        total = int(sum(pages))
        perm = (np.arange(total) if perm_seed is None
                else np.random.default_rng(perm_seed).permutation(total))
        bt = np.full((w.batch, self.max_pages), -1, dtype=np.int32)
        off = 0
        for s, n in enumerate(pages):
            bt[s, :n] = perm[off:off + n]
            off += n
        self.block_table_host = bt
        self.num_phys = total
        tdt = TORCH_DTYPE[w.dtype]
        fill = float("nan") if poison else 0.0
        self.k_pool = torch.full((total, hkv, B, d), fill, dtype=tdt, device=device)
        self.v_pool = torch.full((total, hkv, B, d), fill, dtype=tdt, device=device)
        if w.summary == "i4":  # byte records; 0xff poison
            rec = L.lk_summary_record_bytes(self.cfg)
            self.summary_pool = torch.full((total, hkv, rec), 255 if poison else 0, dtype=torch.uint8,
                                           device=device)
        else:
            rec = L.lk_summary_record_bytes(self.cfg) // (2 if w.dtype == "bf16" else 4)
            self.summary_pool = torch.full((total, hkv, rec), fill, dtype=tdt, device=device)
        self.record_elems = rec
        self.block_table = torch.from_numpy(bt).to(device)
        self.seq_lens = torch.tensor(w.context, dtype=torch.int32, device=device)
        self.ws_bytes = L.lk_workspace_size(self.cfg, w.batch, self.max_pages)
        # the workspace needs no initialization; ws_fill writes a byte pattern
        # into it (0xFF: NaN floats, -1 integers; the default with poison) for
        # tests that check that
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        if ws_fill is None and poison:
            ws_fill = 0xFF
        if ws_fill is not None:
            self.ws.fill_(ws_fill)
        self.cache = L.make_cache(self.k_pool, self.v_pool, self.summary_pool, self.block_table,
                                  self.seq_lens)

    def set_budget(self, token_budget: int, ws_fill: int | None = 0xFF) -> None:
        """Use another token budget on the same cache; the workspace is
        reallocated (and filled with ws_fill) when the budget needs more."""
        self.w.token_budget = token_budget
        self.cfg.token_budget = token_budget
        need = L.lk_workspace_size(self.cfg, self.w.batch, self.max_pages)
        if need > self.ws_bytes:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            if ws_fill is not None:
                self.ws.fill_(ws_fill)
        self.ws_bytes = max(need, self.ws_bytes)

    # ------------------------------------------------------------- filling
    def fill_from_synth(self, threads: int = 8) -> None:
        """Write the first context[seq] tokens of every (sequence, KV head)."""
        w = self.w
        jobs = [(s, h) for s in range(w.batch) for h in range(w.num_kv_heads)]

        def gen(job):
            s, h = job
            k, v = synth.keys_values(w, s, h)
            T = w.context[s]
            return s, h, to_storage(k[:T], w.dtype), to_storage(v[:T], w.dtype)

        with cf.ThreadPoolExecutor(max_workers=threads) as ex:
            for s, h, k, v in ex.map(gen, jobs):
                self.write_tokens(s, h, 0, k, v)

    def write_tokens(self, seq: int, kvh: int, start: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """Copy tokens start..start+n-1 of one (sequence, KV head) into the pools."""
        B = self.w.page_size
        n = k.shape[0]
        pos = np.arange(start, start + n)
        phys = torch.from_numpy(self.block_table_host[seq, pos // B].astype(np.int64)).to(self.device)
        slot = torch.from_numpy((pos % B).astype(np.int64)).to(self.device)
        self.k_pool[phys, kvh, slot] = k.to(self.device)
        self.v_pool[phys, kvh, slot] = v.to(self.device)

    def complete_pages(self, seq: int, seq_len: int | None = None) -> int:
        T = self.w.context[seq] if seq_len is None else seq_len
        return T // self.w.page_size

    def build_all(self, eigvals: bool = False, stream=None):
        """Summarize every complete page of every sequence (all KV heads)."""
        ids = []
        for s in range(self.w.batch):
            ids.extend(self.block_table_host[s, :self.complete_pages(s)].tolist())
        ids_t = torch.tensor(ids, dtype=torch.int32, device=self.device)
        ev = None
        if eigvals:
            ev = torch.empty((len(ids), self.w.num_kv_heads, self.w.page_size), dtype=torch.float32,
                             device=self.device)
        if ids:
            L.lk_build_page_summary(self.cfg, self.cache, ids_t, len(ids), ev, self.ws, self.ws_bytes, stream)
        return ids, ev

    # ------------------------------------------------------------- inputs
    def queries(self, step: int, seq_lens: list | None = None) -> torch.Tensor:
        """Queries [batch][Hq][d] of decode ``step`` (fp32 draws rounded to the dtype)."""
        w = self.w
        lens = w.context if seq_lens is None else seq_lens
        q = np.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=np.float32)
        for s in range(w.batch):
            for h in range(w.num_kv_heads):
                qq, _ = synth.queries(w, step, s, h, lens[s])
                q[s, h * w.group:(h + 1) * w.group] = qq
        return to_storage(q, w.dtype).to(self.device)

    def outputs(self):
        w = self.w
        tdt = TORCH_DTYPE[w.dtype]
        k = L.lk_page_budget(self.cfg)
        return dict(
            out=torch.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=tdt, device=self.device),
            lse=torch.zeros((w.batch, w.num_q_heads), dtype=torch.float32, device=self.device),
            page_lse=torch.full((w.batch, w.num_q_heads, self.max_pages), float("nan"),
                                dtype=torch.float32, device=self.device),
            share=torch.full((w.batch, w.num_kv_heads, self.max_pages), float("nan"),
                             dtype=torch.float32, device=self.device),
            sel=torch.full((w.batch, w.num_kv_heads, k), -7, dtype=torch.int32, device=self.device),
            cnt=torch.full((w.batch, w.num_kv_heads), -7, dtype=torch.int32, device=self.device),
        )

    # ------------------------------------------------------------- entry points
    def score_select(self, q, o, stream=None):
        L.lk_score_select(self.cfg, self.cache, self.w.batch, q, o["page_lse"], o["share"], o["sel"],
                          o["cnt"], self.ws, self.ws_bytes, stream)

    def sparse_attn(self, q, sel, cnt, o, stream=None):
        L.lk_sparse_decode_attn(self.cfg, self.cache, self.w.batch, q, sel, cnt, o["out"], o["lse"],
                                self.ws, self.ws_bytes, stream)

    def dense_attn(self, q, o, stream=None):
        L.lk_dense_decode_attn(self.cfg, self.cache, self.w.batch, q, o["out"], o["lse"], self.ws,
                               self.ws_bytes, stream)

    def decode_step(self, q, k_new, v_new, o, stream=None, with_sel=True):
        L.lk_decode_step(self.cfg, self.cache, self.w.batch, q, k_new, v_new, o["out"], o["lse"],
                         o["sel"] if with_sel else None, o["cnt"] if with_sel else None, self.ws,
                         self.ws_bytes, stream)
