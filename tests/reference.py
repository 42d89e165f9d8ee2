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


def pack_q4_records(qs: lo.QuantSummary) -> np.ndarray:
    """uint8 [n, record bytes] of quantized summaries."""
    n, r, d = qs.basis_q.shape
    B = qs.coeffs_q.shape[1]
    o = q4_offsets(d, B, r)
    out = np.zeros((n, o["bytes"]), dtype=np.uint8)
    out[:, :d] = qs.centroid_q.astype(np.int8).view(np.uint8)
    lo4 = qs.basis_q[:, :, 0::2] & 0xF
    hi4 = qs.basis_q[:, :, 1::2] & 0xF
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
    packed = buf[:, o["basis"]:o["coef"]].reshape(n, r, d // 2).astype(np.int64)
    bq = np.zeros((n, r, d), dtype=np.int64)
    bq[:, :, 0::2] = ((packed & 0xF) ^ 8) - 8
    bq[:, :, 1::2] = ((packed >> 4) ^ 8) - 8
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
    ranked = sorted(cand, key=lambda j: (-m_bar[j], j))
    cut = m_bar[ranked[n_top - 1]]
    bad = [j for j in diff if not (1 <= j < n_mr and abs(m_bar[j] - cut) <= rel * cut)]
    if bad:
        return (f"pages {sorted(bad)} differ beyond the near-cut band (cut {cut:.6g}, "
                f"shares {[float(m_bar[j]) for j in sorted(bad) if 0 <= j < len(m_bar)]})")
    return None


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
