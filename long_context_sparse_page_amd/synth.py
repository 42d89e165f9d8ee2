"""Seeded synthetic inputs shaped like the Locks decode workloads.

This module draws inputs only: it holds none of the method's arithmetic and
is the one piece both the HIP-path tests and the oracle read.  Every array
comes from numpy's PCG64 seeded by ``SeedSequence([SEED, workload_id,
purpose, seq, head, ...])``, so one (sequence, head) can be regenerated alone.

Key model (per KV head, per page): a page-specific rank-8 component
(N(0,1) coefficients times a Haar-random orthonormal 8 x d basis, scale 1.0),
plus a rank-4 component shared by every page and sequence of that KV head
(N(0,1) coefficients times a Haar 4 x d basis, scale 0.5), plus N(0, 0.05^2)
noise per element.  Values are N(0,1).  A query head's query is 3.0 times the
sum of all eight basis rows of each of its carrier pages, plus N(0, 0.3^2)
noise per element.  Appended tokens follow the basis of the page they land in.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED = 20261202

# purposes (second-level seed word)
_P_PAGE_BASIS = 1
_P_GLOBAL_BASIS = 2
_P_KEYS = 3
_P_VALUES = 4
_P_QUERY = 5
_P_LENGTHS = 6
_P_ISOTROPIC = 7

LOCAL_RANK = 8
GLOBAL_RANK = 4
LOCAL_SCALE = 1.0
GLOBAL_SCALE = 0.5
KEY_NOISE = 0.05
QUERY_SCALE = 3.0
QUERY_NOISE = 0.3


@dataclass
class Workload:
    """One synthetic decode workload."""

    name: str
    wid: int                      # workload id (seed word)
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    rank: int
    token_budget: int
    dtype: str                    # "f32" | "bf16"
    context: list                 # initial sequence lengths, one per sequence
    steps: int                    # decode steps (each appends one token)
    carriers: tuple               # (lo, hi) carriers per query head, inclusive
    scale: float = field(default=0.0)
    summary: str = "kv"           # page summaries in the KV dtype ("kv") or int4/int8 ("i4")

    def __post_init__(self):
        if not self.scale:
            self.scale = 1.0 / math.sqrt(self.head_dim)
        self.context = [int(t) for t in self.context]

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def max_len(self, seq: int) -> int:
        return self.context[seq] + self.steps

    def pages_needed(self, seq: int) -> int:
        return -(-self.max_len(seq) // self.page_size)


def workload(wid: int, *, rank: int | None = None, budget: int | None = None,
             batch: int | None = None, steps: int | None = None, summary: str | None = None) -> Workload:
    """The five decode workloads of the Locks decode path.

    0: tiny fp32 case (1 sequence, 4 query heads on 1 KV head, 4064 tokens:
       63 full pages plus a 32-token page, r=8, b=512);
    1: Llama-3.1-8B attention shape (32 q / 8 KV heads), 32K context, batch 8;
    2: same shape at 128K context, batch 4;
    3: one 1,048,576-token sequence;
    4: mixed batch of 64 with lengths log-uniform in [4K, 256K].
    """
    if wid == 0:
        w = Workload("tiny-4K-fp32", 0, 1, 4, 1, 128, 64, 8, 512, "f32", [63 * 64 + 32], 0, (3, 3))
    elif wid == 1:
        w = Workload("llama8b-32K-b8", 1, 8, 32, 8, 128, 64, 8, 2048, "bf16", [32768] * 8, 64, (1, 5))
    elif wid == 2:
        w = Workload("llama8b-128K-b4", 2, 4, 32, 8, 128, 64, 8, 2048, "bf16", [131072] * 4, 64, (1, 5))
    elif wid == 3:
        w = Workload("llama8b-1M-b1", 3, 1, 32, 8, 128, 64, 8, 2048, "bf16", [1 << 20], 32, (1, 5))
    elif wid == 4:
        n = 64 if batch is None else batch
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, 4, _P_LENGTHS])))
        lens = np.floor(np.exp(rng.uniform(math.log(4096), math.log(262144), size=64))).astype(int)
        w = Workload("mixed-b64-4K..256K", 4, n, 32, 8, 128, 64, 8, 1024, "bf16", list(lens[:n]), 256, (1, 5))
    else:
        raise ValueError(f"unknown workload {wid}")
    if rank is not None:
        w.rank = rank
    if budget is not None:
        w.token_budget = budget
    if batch is not None and wid != 4:
        w.batch = batch
        w.context = (w.context * batch)[:batch]
    if steps is not None:
        w.steps = steps
    if summary is not None:
        w.summary = summary
    return w


def _rng(*words) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED, *words])))


def _haar_rows(rng: np.random.Generator, n: int, rows: int, dim: int) -> np.ndarray:
    """n independent Haar-random orthonormal row sets, [n, rows, dim] (QR of a
    Gaussian with the diagonal of R made positive)."""
    g = rng.standard_normal((n, dim, rows))
    qm, rm = np.linalg.qr(g)
    sign = np.sign(np.diagonal(rm, axis1=1, axis2=2))
    sign[sign == 0] = 1.0
    return np.swapaxes(qm * sign[:, None, :], 1, 2)


def global_basis(w: Workload, kv_head: int) -> np.ndarray:
    """The rank-4 basis shared by all pages and sequences of ``kv_head``: [4, d]."""
    return _haar_rows(_rng(w.wid, _P_GLOBAL_BASIS, kv_head), 1, GLOBAL_RANK, w.head_dim)[0]


def page_bases(w: Workload, seq: int, kv_head: int, n_pages: int | None = None) -> np.ndarray:
    """Page-specific rank-8 bases of one (sequence, KV head): [n_pages, 8, d]."""
    n = w.pages_needed(seq) if n_pages is None else n_pages
    return _haar_rows(_rng(w.wid, _P_PAGE_BASIS, seq, kv_head), n, LOCAL_RANK, w.head_dim)


def keys_values(w: Workload, seq: int, kv_head: int, bases: np.ndarray | None = None):
    """Keys and values of every token position 0..max_len-1 of one
    (sequence, KV head), fp32 [max_len, d] each.  Positions >= context are the
    tokens appended by the decode steps, in order."""
    T = w.max_len(seq)
    B, d = w.page_size, w.head_dim
    if bases is None:
        bases = page_bases(w, seq, kv_head)
    gb = global_basis(w, kv_head)
    n_pages = -(-T // B)
    f32 = np.float32
    rk = _rng(w.wid, _P_KEYS, seq, kv_head)
    a = rk.standard_normal((n_pages * B, LOCAL_RANK), dtype=f32)
    b = rk.standard_normal((n_pages * B, GLOBAL_RANK), dtype=f32)
    keys = rk.standard_normal((n_pages * B, d), dtype=f32)
    keys *= f32(KEY_NOISE)
    # Components as fixed-order elementwise sums (no BLAS): a float32 matrix
    # product may round differently with the library's thread partitioning,
    # and every caller, in any thread, must get the same bits.
    a3 = a.reshape(n_pages, B, LOCAL_RANK)
    b32 = bases[:n_pages].astype(f32)
    acc = np.empty((n_pages, B, d), dtype=f32)
    tmp = np.empty_like(acc)
    np.multiply(a3[:, :, 0, None], b32[:, None, 0, :], out=acc)
    for m in range(1, LOCAL_RANK):
        np.multiply(a3[:, :, m, None], b32[:, None, m, :], out=tmp)
        acc += tmp
    acc *= f32(LOCAL_SCALE)
    keys += acc.reshape(n_pages * B, d)
    g32 = gb.astype(f32)
    acc2 = acc.reshape(n_pages * B, d)
    tmp2 = tmp.reshape(n_pages * B, d)
    np.multiply(b[:, 0, None], g32[0], out=acc2)
    for m in range(1, GLOBAL_RANK):
        np.multiply(b[:, m, None], g32[m], out=tmp2)
        acc2 += tmp2
    acc2 *= f32(GLOBAL_SCALE)
    keys += acc2
    values = _rng(w.wid, _P_VALUES, seq, kv_head).standard_normal((T, d), dtype=f32)
    return keys[:T], values


def queries(w: Workload, step: int, seq: int, kv_head: int, seq_len: int,
            bases: np.ndarray | None = None):
    """Queries of the G query heads of ``kv_head`` at decode ``step``, when the
    sequence holds ``seq_len`` tokens: (q [G, d] fp32, carriers list per head).

    Carrier pages are drawn uniformly without replacement from the candidate
    pages 1..n_mr-1 (n_mr = page of the newest token); the count per query
    head is uniform on ``w.carriers``.
    """
    G, d, B = w.group, w.head_dim, w.page_size
    if bases is None:
        bases = page_bases(w, seq, kv_head)
    n_mr = (seq_len - 1) // B
    rq = _rng(w.wid, _P_QUERY, step, seq, kv_head)
    q = np.zeros((G, d))
    chosen = []
    for g in range(G):
        lo, hi = w.carriers
        cnt = int(rq.integers(lo, hi + 1))
        cand = n_mr - 1
        cnt = min(cnt, max(cand, 0))
        pages = (1 + rq.choice(cand, size=cnt, replace=False)) if cnt > 0 else np.zeros(0, dtype=int)
        chosen.append(sorted(int(p) for p in pages))
        for p in pages:
            q[g] += QUERY_SCALE * bases[p].sum(axis=0)
        q[g] += QUERY_NOISE * rq.standard_normal(d)
    return q.astype(np.float32), chosen


def isotropic_pages(n: int, page_size: int = 16, head_dim: int = 128, stream: int = 0) -> np.ndarray:
    """``n`` pages of i.i.d. N(0, 1) keys, fp32 [n, page_size, head_dim]: the
    flat-spectrum (isotropic) null of the Locks appendix ("Spectral tails").
    ``stream`` selects an independent draw."""
    rng = _rng(_P_ISOTROPIC, page_size, head_dim, stream)
    return rng.standard_normal((n, page_size, head_dim), dtype=np.float32)
