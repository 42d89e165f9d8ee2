"""Oracle-side helpers for the parity tests: regenerate one (sequence, KV head)
from the seeded generator, run the fp64 oracle on it, and the matching rules
of the decode path (selection sets, page LSE, attention output)."""

from __future__ import annotations

import numpy as np
import torch

from long_context_sparse_page_amd import synth
from long_context_sparse_page_amd.paged import to_storage
from oracle import locks_oracle as lo


def stored(x: np.ndarray, dtype: str) -> np.ndarray:
    """What a buffer of ``dtype`` holds for fp32 draws ``x``, widened to fp64."""
    return to_storage(x, dtype).to(torch.float64).numpy()


def host_pages(w: synth.Workload, seq: int, kvh: int, T: int):
    """K, V of one (sequence, KV head) holding T tokens, as stored, in logical
    page order: fp64 [n_pages, B, d] with unwritten slots zero."""
    B, d = w.page_size, w.head_dim
    k, v = synth.keys_values(w, seq, kvh)
    n_pages = w.pages_needed(seq)
    K = np.zeros((n_pages * B, d))
    V = np.zeros((n_pages * B, d))
    K[:T] = stored(k[:T], w.dtype)
    V[:T] = stored(v[:T], w.dtype)
    return K.reshape(n_pages, B, d), V.reshape(n_pages, B, d)


def host_queries(w: synth.Workload, step: int, seq_lens) -> np.ndarray:
    """Queries [batch][Hq][d] as stored (fp64)."""
    q = np.zeros((w.batch, w.num_q_heads, w.head_dim), dtype=np.float32)
    for s in range(w.batch):
        for h in range(w.num_kv_heads):
            qq, _ = synth.queries(w, step, s, h, seq_lens[s])
            q[s, h * w.group:(h + 1) * w.group] = qq
    return stored(q, w.dtype)


def q_device(q64: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(q64)
    return (t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)).to(device)


def oracle_quant(w, K_pages, n_pages) -> lo.QuantSummary:
    """The oracle's int4/int8 summaries (codes and scales) of the first n pages."""
    return lo.quantize_summary(lo.build_page_summaries(K_pages[:n_pages], w.rank, "f64"))


def oracle_summaries(w, K_pages, n_pages):
    """The summaries the scorer reads: rounded to the KV dtype, or quantized
    and dequantized for int4/int8 records."""
    if w.summary == "i4":
        return lo.dequantize_summary(oracle_quant(w, K_pages, n_pages))
    return lo.build_page_summaries(K_pages[:n_pages], w.rank, w.dtype)


# ---- int4/int8 record bytes (the layout documented in include/locks.h) ----
def q4_offsets(d: int, B: int, r: int) -> dict:
    o = {"mu": 0, "basis": d, "coef": d + r * d // 2}
    o["cscale"] = o["coef"] + B * r
    o["bscale"] = o["cscale"] + 2 * B
    o["mscale"] = o["bscale"] + 2 * r
    o["bytes"] = (o["mscale"] + 2 + 15) // 16 * 16
    return o


# int4 basis rows, per group of 8 dims (one 32-bit word): byte b holds dim
# Q4_LO_DIMS[b] in its low nibble and Q4_HI_DIMS[b] in its high nibble, i.e.
# the even dims in the word's low half-word and the odd dims in its high one.
Q4_LO_DIMS = [0, 4, 1, 5]
Q4_HI_DIMS = [2, 6, 3, 7]


def pack_q4_records(qs: lo.QuantSummary) -> np.ndarray:
    """uint8 [n, record bytes] of quantized summaries."""
    n, r, d = qs.basis_q.shape
    B = qs.coeffs_q.shape[1]
    o = q4_offsets(d, B, r)
    out = np.zeros((n, o["bytes"]), dtype=np.uint8)
    out[:, :d] = qs.centroid_q.astype(np.int8).view(np.uint8)
    words = qs.basis_q.reshape(n, r, d // 8, 8)
    lo4 = words[..., Q4_LO_DIMS] & 0xF
    hi4 = words[..., Q4_HI_DIMS] & 0xF
    out[:, o["basis"]:o["coef"]] = (lo4 | (hi4 << 4)).astype(np.uint8).reshape(n, -1)
    out[:, o["coef"]:o["cscale"]] = qs.coeffs_q.astype(np.int8).view(np.uint8).reshape(n, -1)
    out[:, o["cscale"]:o["bscale"]] = qs.coeffs_s.astype(np.float16).view(np.uint8).reshape(n, -1)
    out[:, o["bscale"]:o["mscale"]] = qs.basis_s.astype(np.float16).view(np.uint8).reshape(n, -1)
    out[:, o["mscale"]:o["mscale"] + 2] = qs.centroid_s.astype(np.float16).view(np.uint8).reshape(n, -1)
    return out


def unpack_q4_records(buf: np.ndarray, d: int, B: int, r: int) -> lo.QuantSummary:
    """Codes and scales of uint8 [n, record bytes] records."""
    buf = np.ascontiguousarray(buf, dtype=np.uint8)
    n = buf.shape[0]
    o = q4_offsets(d, B, r)
    mq = buf[:, :d].view(np.int8).astype(np.int64)
    packed = buf[:, o["basis"]:o["coef"]].reshape(n, r, d // 8, 4).astype(np.int64)
    bq = np.zeros((n, r, d // 8, 8), dtype=np.int64)
    bq[..., Q4_LO_DIMS] = ((packed & 0xF) ^ 8) - 8
    bq[..., Q4_HI_DIMS] = ((packed >> 4) ^ 8) - 8
    bq = bq.reshape(n, r, d)
    cq = buf[:, o["coef"]:o["cscale"]].view(np.int8).reshape(n, B, r).astype(np.int64)
    f16 = lambda a, b: np.ascontiguousarray(buf[:, a:b]).view(np.float16).astype(np.float64)
    return lo.QuantSummary(centroid_q=mq, centroid_s=f16(o["mscale"], o["mscale"] + 2)[:, 0],
                           basis_q=bq, basis_s=f16(o["bscale"], o["mscale"]), coeffs_q=cq,
                           coeffs_s=f16(o["cscale"], o["bscale"]), eigvals=np.zeros((n, B)),
                           r_eff=np.full(n, r))


def oracle_head(w, q_g, K_pages, V_pages, T, summary=None):
    n_mr = lo.most_recent_page(T, w.page_size)
    if summary is None:
        summary = oracle_summaries(w, K_pages, max(n_mr, 0))
    return lo.decode_head(q_g, K_pages, V_pages, T, summary, w.token_budget, w.scale), summary


def selection_mismatch(gpu_sel, ora_sel, m_bar, n_mr, k, rel=1e-4):
    """The selection matching rule: same size, sink and most-recent present,
    and every page in the symmetric difference has an oracle share within
    ``rel`` (relative) of the oracle's cut value.  Returns None if matched,
    else a message."""
    g = sorted(int(x) for x in gpu_sel)
    o = sorted(int(x) for x in ora_sel)
    if len(g) != len(o):
        return f"size {len(g)} != {len(o)}: gpu {g} oracle {o}"
    if g != sorted(set(g)):
        return f"duplicate pages {g}"
    if n_mr >= 0 and (0 not in g or n_mr not in g):
        return f"sink/recent missing: {g} (n_mr {n_mr})"
    diff = set(g) ^ set(o)
    if not diff:
        return None
    cand = list(range(1, n_mr))
    n_top = min(k - 2, len(cand))
    if n_top <= 0:
        return f"pages {sorted(diff)} differ with no candidate to rank: gpu {g} oracle {o}"
    ranked = sorted(cand, key=lambda j: (-m_bar[j], j))
    cut = m_bar[ranked[n_top - 1]]
    bad = [j for j in diff if not (1 <= j < n_mr and abs(m_bar[j] - cut) <= rel * cut)]
    if bad:
        return (f"pages {sorted(bad)} differ beyond the near-cut band (cut {cut:.6g}, rel {rel:.3g}, "
                f"shares {[float(m_bar[j]) for j in sorted(bad) if 0 <= j < len(m_bar)]})")
    return None


def record_band(delta: float) -> float:
    """Relative share band within which two selections may differ when every
    page score of one lies within ``delta`` of the other's.

    m_bar_j = (1/G) sum_g exp(s_j(g) - L_g) with L_g = LSE_j s_j(g): moving every
    s by at most delta moves each L_g by at most delta, so each m_bar_j by a
    factor in [e^-2delta, e^2delta].  A page a ranked above b under the
    perturbed scores but not under the reference ones then has
    m_bar_b <= e^{4 delta} m_bar_a, so every page in the symmetric difference
    of the two selections lies within a factor e^{4 delta} of the reference
    cut: |m_bar_j - cut| <= (e^{4 delta} - 1) cut."""
    return float(np.expm1(4.0 * delta))


def rel_l2(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Per-row ||a - b|| / ||b||."""
    return np.linalg.norm(a - b, axis=-1) / np.maximum(np.linalg.norm(b, axis=-1), 1e-30)


def codes_match(gq, oq, gs, os_, x, tol):
    """Scales within one fp16 ulp; codes equal except by one step, and where the
    scales agree only where the oracle's x / s lies within tol of a rounding
    boundary.  Returns the fraction of differing codes."""
    np.testing.assert_allclose(gs, os_, rtol=2.0 ** -10, atol=0)
    assert (np.abs(gq - oq) <= 1).all()
    t = x / np.where(os_ > 0, os_, 1.0)[..., None]
    off = np.abs(t - np.floor(t) - 0.5)
    bad = (gq != oq) & (gs == os_)[..., None] & (off > tol)
    assert not bad.any(), f"{bad.sum()} codes differ away from a rounding boundary"
    return (gq != oq).mean()


# ---- the matching rules on one (sequence, KV head) -------------------------
def gpu_summaries(dc, w, seq: int, kvh: int, n: int) -> lo.PageSummary:
    """The summaries the GPU stored for logical pages 0..n-1 of (seq, kvh),
    read back from the summary pool: records in the KV dtype widened to fp64,
    int4/int8 records dequantized (code x scale)."""
    d, B, r = w.head_dim, w.page_size, w.rank
    if n <= 0:
        return lo.PageSummary(np.zeros((0, d)), np.zeros((0, r, d)), np.zeros((0, B, r)),
                              np.zeros((0, B)), np.zeros(0, dtype=np.int64))
    phys = torch.from_numpy(dc.block_table_host[seq, :n].astype(np.int64)).to(dc.summary_pool.device)
    raw = dc.summary_pool[phys, kvh].cpu()
    if w.summary == "i4":
        return lo.dequantize_summary(unpack_q4_records(raw.numpy(), d, B, r))
    x = raw.to(torch.float64).numpy()
    return lo.PageSummary(centroid=x[:, :d], basis=x[:, d:d + r * d].reshape(n, r, d),
                          coeffs=x[:, d + r * d:].reshape(n, B, r), eigvals=np.zeros((n, B)),
                          r_eff=np.full(n, r))


class PairCheck:
    """Errors of one checked (sequence, KV head), for the test's summary line."""

    def __init__(self):
        self.lse_own = 0.0    # GPU page LSE vs the oracle scoring the GPU's own records
        self.lse_e2e = 0.0    # GPU page LSE vs the oracle's own build (mirrored records)
        self.delta = 0.0      # the oracle's scores of the two record sets
        self.att = 0.0        # attention vs the oracle over the GPU's selection
        self.att_lse = 0.0

    def merge(self, o: "PairCheck") -> "PairCheck":
        for key in vars(self):
            setattr(self, key, max(getattr(self, key), getattr(o, key)))
        return self

    def __str__(self):
        return (f"page LSE vs own records {self.lse_own:.3g}, vs the oracle's build {self.lse_e2e:.3g} "
                f"(record effect {self.delta:.3g}); attention rel L2 {self.att:.3g}, LSE {self.att_lse:.3g}")


LSE_ATOL = 1e-3        # page LSE, absolute
SEL_REL = 1e-4         # selection band at the cut, relative
ATT_REL_BF16 = 2e-2    # attention relative L2, bf16 outputs
ATT_REL_F32 = 1e-5     # attention relative L2, fp32 outputs
ATT_LSE_ATOL = 1e-3    # attention log-sum-exp, absolute


def check_pair(w, qg, K, V, T, gpu_sel, own=None, gpu_page_lse=None, gpu_out=None, gpu_lse=None,
               gpu_share=None, tag="", e2e_lse_gate=True) -> PairCheck:
    """Every matching rule on one (sequence, KV head) holding T tokens.

    qg [G, d], K / V [n_pages, B, d] as stored (fp64).  ``own``: the GPU's
    records read back (gpu_summaries), when the GPU built them; None when the
    records are the oracle's own (then the two oracle runs coincide).
      * selection: the GPU's set against the oracle run on the GPU's records,
        at the 1e-4 band; and the oracle's selections from the two record sets
        against each other at record_band(delta), delta the largest difference
        of their page scores;
      * page LSE (if given): within 1e-3 of the oracle on the GPU's records and
        (e2e_lse_gate, records in the KV dtype) of the oracle's own build;
      * shares m_bar (if given, with the page LSE): within the factor
        e^{2 eps} that page scores within eps of the oracle's allow (eps the
        measured page-LSE error), plus fp32 rounding;
      * attention (if given): the oracle fed the GPU's selection, relative L2
        2e-2 (bf16) or 1e-5 (fp32), log-sum-exp within 1e-3.
    """
    B = w.page_size
    n_mr = lo.most_recent_page(T, B)
    k = lo.page_budget(w.token_budget, B)
    hs_ora, _ = oracle_head(w, qg, K, V, T)
    hs_own = hs_ora if own is None else lo.decode_head(qg, K, V, T, own, w.token_budget, w.scale)
    pc = PairCheck()
    msg = selection_mismatch(gpu_sel, hs_own.selected, hs_own.m_bar, n_mr, k, rel=SEL_REL)
    assert msg is None, f"{tag}: selection vs the oracle on the GPU's records: {msg}"
    if n_mr > 0:
        pc.delta = float(np.abs(hs_own.page_lse - hs_ora.page_lse).max())
    if own is not None:
        band = record_band(pc.delta) + SEL_REL
        msg = selection_mismatch(hs_own.selected, hs_ora.selected, hs_ora.m_bar, n_mr, k, rel=band)
        assert msg is None, f"{tag}: oracle selections of the GPU's and the oracle's records: {msg}"
    if gpu_page_lse is not None and n_mr > 0:
        got = np.asarray(gpu_page_lse)[:, :n_mr]
        pc.lse_own = float(np.abs(got - hs_own.page_lse).max())
        pc.lse_e2e = float(np.abs(got - hs_ora.page_lse).max())
        assert pc.lse_own <= LSE_ATOL, f"{tag}: page LSE vs the oracle on the GPU's records {pc.lse_own:.3g}"
        if e2e_lse_gate:
            assert pc.lse_e2e <= LSE_ATOL, f"{tag}: page LSE vs the oracle's build {pc.lse_e2e:.3g}"
        if gpu_share is not None:
            np.testing.assert_allclose(np.asarray(gpu_share)[:n_mr], hs_own.m_bar,
                                       rtol=float(np.expm1(2 * pc.lse_own)) + 1e-5, atol=1e-30,
                                       err_msg=f"{tag}: shares")
    if gpu_out is not None:
        eo, el = lo.attend(qg, lo.gather_tokens(K, gpu_sel, T, B), lo.gather_tokens(V, gpu_sel, T, B), w.scale)
        pc.att = float(rel_l2(np.asarray(gpu_out, dtype=np.float64), eo).max())
        bar = ATT_REL_BF16 if w.dtype == "bf16" else ATT_REL_F32
        assert pc.att <= bar, f"{tag}: attention rel L2 {pc.att:.3g} > {bar}"
        if gpu_lse is not None:
            gl = np.asarray(gpu_lse, dtype=np.float64)
            fin = np.isfinite(el)
            assert (np.isfinite(gl) == fin).all(), f"{tag}: attention LSE finiteness {gl} vs {el}"
            if fin.any():
                pc.att_lse = float(np.abs(gl[fin] - el[fin]).max())
            assert pc.att_lse <= ATT_LSE_ATOL, f"{tag}: attention LSE {pc.att_lse:.3g}"
    return pc


def bf16_ulps(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between bf16-representable values a and b (steps
    along the ordered bf16 grid; +0 and -0 coincide)."""
    def ordered(x):
        u = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
            .view(torch.int16).to(torch.int32).numpy()
        return np.where(u < 0, -(u & 0x7FFF), u)
    return np.abs(ordered(a) - ordered(b))


def bf16_step_above(x: np.ndarray) -> np.ndarray:
    """The next bf16 value above |x| (bf16-representable x): |x| plus one ulp."""
    u = torch.from_numpy(np.abs(np.ascontiguousarray(x, dtype=np.float32))).to(torch.bfloat16).view(torch.int16)
    return (u + 1).view(torch.bfloat16).to(torch.float64).numpy()


def check_all_pairs(w, dc, o, q64, lens, pairs=None, page_lse=None, e2e_lse_gate=True, share=False):
    """check_pair on every (or the listed) (sequence, KV head) of the outputs
    o, with the GPU's own records read back from the pool (and the shares of
    o when ``share``)."""
    page_lse = o["page_lse"].cpu().numpy() if page_lse is None else page_lse
    sel, cnt = o["sel"].cpu().numpy(), o["cnt"].cpu().numpy()
    out = o["out"].float().cpu().numpy().astype(np.float64)
    lse = o["lse"].cpu().numpy()
    shares = o["share"].cpu().numpy() if share else None
    G = w.group
    tot = PairCheck()
    if pairs is None:
        pairs = [(s, h) for s in range(w.batch) for h in range(w.num_kv_heads)]
    for (s, h) in pairs:
        K, V = host_pages(w, s, h, lens[s])
        n_mr = lo.most_recent_page(lens[s], w.page_size)
        own = gpu_summaries(dc, w, s, h, max(n_mr, 0))
        hs = slice(h * G, (h + 1) * G)
        tot.merge(check_pair(w, q64[s, hs], K, V, lens[s], sel[s, h, :cnt[s, h]], own=own,
                                 gpu_page_lse=page_lse[s, hs], gpu_out=out[s, hs], gpu_lse=lse[s, hs],
                                 gpu_share=None if shares is None else shares[s, h],
                                 tag=f"seq {s} head {h} T {lens[s]}", e2e_lse_gate=e2e_lse_gate))
        assert (sel[s, h, cnt[s, h]:] == -1).all()
    return tot
