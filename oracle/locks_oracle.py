"""Locks decode path, written out plainly in fp64 (numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.  It
shares no code, constants or helpers with the HIP library.

Source: "Locks: Page-Local Compact Key Summaries for Efficient Long-Context
Decoding" (arXiv 2607.24555), cited below as [Locks] with its section,
equation or lemma.  The technical-review blog post of the same paper is cited
as [Review] (its restatement of the method as Algorithms 1-2 and its toy
example in 5.1); where the two differ, [Locks] decides.

Locks is an approximation (reconstructed LSE, then a heuristic shared
selection), so this module runs the method's steps in the paper's order and
notation; beside them sit the plain definitions the method is checked against
(exact page log-mass, exact-mass selection, dense softmax attention).
Library primitives used as steps: ``numpy.linalg.eigh`` (the small symmetric
eigendecomposition of the build), matrix products, sorting.

Readings taken where the pages leave a step open:
  * the most-recent page is the page holding the newest token (possibly
    partial); pages before it are complete, summarized and scored; page 0
    (the sink) is scored but never a candidate;
  * the page-mass share of a query head is normalized over all scored pages,
    the sink included;
  * ties at the top-k cut go to the lower page index;
  * a mode is a zero mode when its Gram eigenvalue is <= ZERO_MODE_RTOL times
    the largest one, or <= ZERO_MODE_FLOOR times the page's uncentred key
    energy sum_i ||k_i||^2 (centering rounding noise of a constant page is not a
    mode); zero modes get a zero basis column and zero coefficients;
  * each basis column is signed so that its largest-magnitude entry is
    positive (scores depend only on V V^T, so this only fixes a representative);
  * the stored summary (centroid, basis, coefficients) is rounded to the
    storage dtype with round-to-nearest-even, because that is what is stored.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "ZERO_MODE_RTOL",
    "ZERO_MODE_FLOOR",
    "bf16_round",
    "storage_round",
    "PageSummary",
    "build_page_summaries",
    "reconstructed_page_lse",
    "exact_page_lse",
    "share_average",
    "select_pages",
    "page_budget",
    "most_recent_page",
    "gather_tokens",
    "attend",
    "decode_head",
    "HeadStep",
    "summary_bytes",
    "record_elements",
    "fp16_round",
    "quantize_symmetric",
    "QuantSummary",
    "quantize_summary",
    "dequantize_summary",
    "QUANT_BASIS_LEVELS",
    "QUANT_ROW_LEVELS",
    "envelope_page_score",
    "moment_core_score",
    "centroid_score",
    "combine_shares",
    "select_by_rule",
    "head_coverage",
]

# Eigenvalue thresholds of the zero-mode rule ([Locks] §4 "Build" states the
# rule, not the constants): relative to the largest eigenvalue, and relative to
# the page's uncentred key energy.
ZERO_MODE_RTOL = 1e-5
ZERO_MODE_FLOOR = 1e-10


# ----------------------------------------------------------------------------
# storage rounding
# ----------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (ties to even), returned as fp64.

    bfloat16 keeps 8 significant bits (7 stored); an fp64 significand has 53,
    so the 45 low bits are rounded away in one step (no double rounding).
    Values beyond the bf16 range are not expected here and are not handled.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    bits = x.view(np.uint64)
    drop = np.uint64(45)
    half = np.uint64((1 << 44) - 1)
    lsb = (bits >> drop) & np.uint64(1)
    rounded = (bits + half + lsb) & ~np.uint64((1 << 45) - 1)
    return rounded.view(np.float64)


def storage_round(x, dtype: str) -> np.ndarray:
    """Round to what a ``dtype`` ("f32" or "bf16") buffer holds, back in fp64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ----------------------------------------------------------------------------
# build: [Locks] §4 "Build (once, when a page completes)"; [Review] Alg. 1
# ----------------------------------------------------------------------------
@dataclass
class PageSummary:
    """Per-page summary arrays for n pages (leading axis)."""

    centroid: np.ndarray  # [n, d]      mu_j
    basis: np.ndarray     # [n, r, d]   row k is the basis vector v_{j,k} (columns of V_j)
    coeffs: np.ndarray    # [n, B, r]   row i is c_i (rows of C_j = U_{j,r} Sigma_{j,r})
    eigvals: np.ndarray   # [n, B]      Gram eigenvalues sigma^2, descending
    r_eff: np.ndarray     # [n]         retained nonzero modes


def build_page_summaries(keys, rank: int, dtype: str = "f64",
                         zero_mode_rtol: float = ZERO_MODE_RTOL,
                         zero_mode_floor: float = ZERO_MODE_FLOOR) -> PageSummary:
    """Build the rank-``rank`` spectral summary of every page in ``keys`` [n, B, d].

    Steps, in [Locks] §4 order: centre the page (k_i = mu + delta_i); stack the
    deviations as rows of D; eigendecompose the B x B Gram D D^T = U Sigma^2 U^T
    with eigenvalues sorted descending; keep r components with
    C = U_r Sigma_r and V = D^T U_r Sigma_r^{-1}; zero modes are dropped (zero
    column, zero coefficients) so Sigma^{-1} only meets nonzero values.
    Centroid, basis and coefficients are then rounded to ``dtype``.
    """
    keys = np.asarray(keys, dtype=np.float64)
    if keys.ndim == 2:
        keys = keys[None]
    n, B, d = keys.shape
    mu = keys.mean(axis=1)                                   # [n, d]
    D = keys - mu[:, None, :]                                # [n, B, d]
    gram = D @ np.swapaxes(D, 1, 2)                          # [n, B, B]
    lam, U = np.linalg.eigh(gram)                            # ascending
    lam = lam[:, ::-1].copy()                                # descending
    U = U[:, :, ::-1].copy()

    kept = min(rank, B)
    lam1 = lam[:, :1]                                        # [n, 1]
    energy = (keys ** 2).sum(axis=(1, 2))[:, None]           # [n, 1]
    thresh = np.maximum(zero_mode_rtol * lam1, zero_mode_floor * energy)
    nonzero = (lam[:, :kept] > thresh) & (lam1 > 0)
    sigma = np.sqrt(np.where(nonzero, lam[:, :kept], 1.0))   # placeholder 1 on zero modes
    Ur = U[:, :, :kept]                                      # [n, B, kept]
    V = np.swapaxes(D, 1, 2) @ Ur / sigma[:, None, :]        # [n, d, kept]
    C = Ur * sigma[:, None, :]                               # [n, B, kept]
    V = np.where(nonzero[:, None, :], V, 0.0)
    C = np.where(nonzero[:, None, :], C, 0.0)

    # sign representative: largest-magnitude entry of each basis column positive
    idx = np.argmax(np.abs(V), axis=1)                       # [n, kept]
    lead = np.take_along_axis(V, idx[:, None, :], axis=1)[:, 0, :]
    flip = np.where(lead < 0, -1.0, 1.0)
    V = V * flip[:, None, :]
    C = C * flip[:, None, :]

    basis = np.zeros((n, rank, d))
    coeffs = np.zeros((n, B, rank))
    basis[:, :kept, :] = np.swapaxes(V, 1, 2)
    coeffs[:, :, :kept] = C
    return PageSummary(
        centroid=storage_round(mu, dtype),
        basis=storage_round(basis, dtype),
        coeffs=storage_round(coeffs, dtype),
        eigvals=np.clip(lam, 0.0, None),
        r_eff=nonzero.sum(axis=1),
    )


# ----------------------------------------------------------------------------
# quantized summary: [Locks] §4 "Build" (int4 basis with per-column scales,
# int8 coefficients and centroid with per-row scales), App. D "State
# accounting"; [Review] Alg. 1 (the quantization follows the build)
#
# The pages name the precisions and where the scales sit, not the scheme.
# Reading taken: symmetric absmax quantization; int4 codes in [-7, 7], int8
# codes in [-127, 127]; each scale is rounded to fp16 (the scale overhead that
# brings the 9.4% payload to "about a tenth" at B = 16) and the codes are
# computed against that stored scale, rounding half to even; an all-zero row
# has scale 0 and codes 0.  Scores use the dequantized values code * scale.
# ----------------------------------------------------------------------------
QUANT_BASIS_LEVELS = 7
QUANT_ROW_LEVELS = 127


def fp16_round(x) -> np.ndarray:
    """Round fp64 values to the nearest IEEE half (ties to even), back in fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def quantize_symmetric(x, levels: int):
    """Symmetric quantization of the last axis of ``x``: one scale per row,
    s = fp16(max |x| / levels), codes = clip(rint(x / s), -levels, levels).
    Returns (codes as int, scales as fp64)."""
    x = np.asarray(x, dtype=np.float64)
    s = fp16_round(np.max(np.abs(x), axis=-1) / levels)
    safe = np.where(s > 0, s, 1.0)[..., None]
    codes = np.clip(np.rint(x / safe), -levels, levels)
    codes = np.where(s[..., None] > 0, codes, 0.0)
    return codes.astype(np.int64), s


@dataclass
class QuantSummary:
    """Quantized page summaries for n pages: integer codes and their scales."""

    centroid_q: np.ndarray  # [n, d]     int8 codes of mu_j
    centroid_s: np.ndarray  # [n]        one scale per centroid
    basis_q: np.ndarray     # [n, r, d]  int4 codes; row k is v_{j,k}
    basis_s: np.ndarray     # [n, r]     one scale per basis vector (column of V_j)
    coeffs_q: np.ndarray    # [n, B, r]  int8 codes; row i is c_i
    coeffs_s: np.ndarray    # [n, B]     one scale per token (row of C_j)
    eigvals: np.ndarray     # [n, B]     carried over from the unquantized build
    r_eff: np.ndarray       # [n]


def quantize_summary(summary: PageSummary) -> QuantSummary:
    """int4 basis (per-column scales), int8 coefficients and centroid (per-row
    scales) of an unrounded (fp64) summary."""
    bq, bs = quantize_symmetric(summary.basis, QUANT_BASIS_LEVELS)
    cq, cs = quantize_symmetric(summary.coeffs, QUANT_ROW_LEVELS)
    mq, ms = quantize_symmetric(summary.centroid, QUANT_ROW_LEVELS)
    return QuantSummary(centroid_q=mq, centroid_s=ms, basis_q=bq, basis_s=bs, coeffs_q=cq, coeffs_s=cs,
                        eigvals=summary.eigvals, r_eff=summary.r_eff)


def dequantize_summary(qs: QuantSummary) -> PageSummary:
    """The summary the scorer sees: every code times its scale."""
    return PageSummary(
        centroid=qs.centroid_q * qs.centroid_s[..., None],
        basis=qs.basis_q * qs.basis_s[..., None],
        coeffs=qs.coeffs_q * qs.coeffs_s[..., None],
        eigvals=qs.eigvals,
        r_eff=qs.r_eff,
    )


# ----------------------------------------------------------------------------
# score: [Locks] §4 "Score", Eq. (1)
# ----------------------------------------------------------------------------
def _logsumexp(z, axis=-1):
    m = np.max(z, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=axis, keepdims=True))).squeeze(axis)


def reconstructed_page_lse(q, summary: PageSummary, scale: float) -> np.ndarray:
    """Eq. (1): s_hat_j(q) = log sum_i exp((q^T mu_j + (V_j^T q)^T c_i) * scale).

    ``q`` is [G, d] (one row per query head of the group); returns [G, n].
    """
    q = np.asarray(q, dtype=np.float64)
    a = q @ summary.centroid.T                               # [G, n]   q^T mu_j
    proj = np.einsum("nrd,gd->gnr", summary.basis, q)        # [G, n, r] V_j^T q
    recon = np.einsum("nbr,gnr->gnb", summary.coeffs, proj)  # [G, n, B] (V_j^T q)^T c_i
    z = scale * (a[:, :, None] + recon)
    return _logsumexp(z, axis=-1)


def exact_page_lse(q, keys, scale: float) -> np.ndarray:
    """Exact page log-mass s_j(q) = log sum_{i in P_j} exp(q^T k_i * scale)
    ([Locks] Lemma 1(ii)); ``keys`` [n, B, d] -> [G, n]."""
    q = np.asarray(q, dtype=np.float64)
    z = scale * np.einsum("gd,nbd->gnb", q, np.asarray(keys, dtype=np.float64))
    return _logsumexp(z, axis=-1)


# ----------------------------------------------------------------------------
# share-average and selection: [Locks] §4 (after Eq. (1)), Cor. 3
# ----------------------------------------------------------------------------
def share_average(page_lse) -> np.ndarray:
    """m_hat_g(j) = exp(s_hat_j(q_g)) / sum_j' exp(s_hat_j'(q_g)); returns the
    group average m_bar_j = (1/G) sum_g m_hat_g(j) over the pages given."""
    s = np.asarray(page_lse, dtype=np.float64)
    norm = _logsumexp(s, axis=1)                             # [G]
    shares = np.exp(s - norm[:, None])                       # [G, n]
    return shares.mean(axis=0)


def page_budget(token_budget: int, page_size: int) -> int:
    """k = ceil(b / B) pages ([Locks] §2)."""
    return -(-token_budget // page_size)


def most_recent_page(seq_len: int, page_size: int) -> int:
    """Index of the page that holds the newest token; -1 for an empty sequence
    (no token, hence no page)."""
    if seq_len <= 0:
        return -1
    return (seq_len - 1) // page_size


def select_pages(m_bar, n_mr: int, k: int) -> np.ndarray:
    """Sink page 0, the most recent page n_mr, and the top-(k-2) candidates
    1..n_mr-1 by m_bar (ties to the lower index); ascending page indices.
    An empty sequence (n_mr < 0) has no page to select."""
    if n_mr < 0:
        return np.zeros(0, dtype=np.int64)
    if n_mr == 0:
        return np.array([0], dtype=np.int64)
    m_bar = np.asarray(m_bar, dtype=np.float64)
    cand = list(range(1, n_mr))
    n_top = min(k - 2, len(cand))
    ranked = sorted(cand, key=lambda j: (-m_bar[j], j))[:n_top]
    return np.array(sorted({0, n_mr, *ranked}), dtype=np.int64)


# ----------------------------------------------------------------------------
# attention: [Locks] §2 "Decode-time attention"
# ----------------------------------------------------------------------------
def gather_tokens(pages_kv, pages, seq_len: int, page_size: int) -> np.ndarray:
    """Tokens of the listed logical pages, in page order; the page holding the
    newest token contributes only its filled slots.  ``pages_kv`` [n, B, d].
    No page gives an empty [0, d] array."""
    if len(pages) == 0:
        return np.zeros((0, pages_kv.shape[-1]))
    out = []
    for j in pages:
        filled = min(page_size, seq_len - j * page_size)
        out.append(np.asarray(pages_kv[j, :filled], dtype=np.float64))
    return np.concatenate(out, axis=0)


def attend(q, keys, values, scale: float):
    """o = sum_i alpha_i v_i with alpha = softmax(q^T k * scale); also the
    log-sum-exp of the logits.  ``q`` [G, d], ``keys``/``values`` [T, d].
    With no token (an empty sequence) the sum is empty: o = 0 and the
    log-sum-exp is log 0 = -inf."""
    q = np.asarray(q, dtype=np.float64)
    if np.asarray(keys).shape[0] == 0:
        return np.zeros((q.shape[0], np.asarray(values).shape[-1])), np.full(q.shape[0], -np.inf)
    z = scale * (q @ np.asarray(keys, dtype=np.float64).T)   # [G, T]
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    l = w.sum(axis=1, keepdims=True)
    o = (w @ np.asarray(values, dtype=np.float64)) / l
    return o, (m + np.log(l))[:, 0]


# ----------------------------------------------------------------------------
# one decode step for one (sequence, KV head)
# ----------------------------------------------------------------------------
@dataclass
class HeadStep:
    page_lse: np.ndarray   # [G, n_mr] reconstructed scores of the scored pages
    m_bar: np.ndarray      # [n_mr] group-averaged shares
    selected: np.ndarray   # ascending logical page indices
    out: np.ndarray        # [G, d]
    lse: np.ndarray        # [G]


def decode_head(q, keys_pages, values_pages, seq_len: int, summary: PageSummary,
                token_budget: int, scale: float) -> HeadStep:
    """Score -> share-average -> select -> attend for one KV head's group.

    ``keys_pages``/``values_pages`` [n_pages, B, d] hold the head's cache in
    logical page order; ``summary`` covers at least pages 0..n_mr-1.
    """
    B = keys_pages.shape[1]
    n_mr = most_recent_page(seq_len, B)
    k = page_budget(token_budget, B)
    if n_mr > 0:
        sub = PageSummary(summary.centroid[:n_mr], summary.basis[:n_mr],
                          summary.coeffs[:n_mr], summary.eigvals[:n_mr], summary.r_eff[:n_mr])
        s_hat = reconstructed_page_lse(q, sub, scale)
        m_bar = share_average(s_hat)
    else:
        s_hat = np.zeros((np.asarray(q).shape[0], 0))
        m_bar = np.zeros(0)
    sel = select_pages(m_bar, n_mr, k)
    K = gather_tokens(keys_pages, sel, seq_len, B)
    Vv = gather_tokens(values_pages, sel, seq_len, B)
    out, lse = attend(q, K, Vv, scale)
    return HeadStep(s_hat, m_bar, sel, out, lse)


# ----------------------------------------------------------------------------
# rival page scores and GQA combine rules (diagnostics: [Locks] §3 Lemma 2,
# App. A.5 Prop. 3 / Eq. (A.2), Table B.1, Table D.17)
# ----------------------------------------------------------------------------
def envelope_page_score(q, keys, scale: float) -> np.ndarray:
    """Envelope score of [Locks] Lemma 2: e_j(q) = sum_c max(q_c u_jc, q_c l_jc)
    with u, l the page's per-dimension key maxima and minima, times the logit
    scale (an upper bound of every within-page logit).  keys [n, B, d] -> [G, n]."""
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    u, lo = keys.max(axis=1), keys.min(axis=1)                       # [n, d]
    e = np.maximum(q[:, None, :] * u[None], q[:, None, :] * lo[None])  # [G, n, d]
    return scale * e.sum(axis=-1)


def moment_core_score(q, summary: PageSummary, scale: float) -> np.ndarray:
    """Rank-r moment core of [Locks] Eq. (A.2), the second-cumulant truncation
    of the page log-mass: scale q.mu + (scale^2 / 2B) sum_{k<=r} sigma_k^2 (v_k.q)^2,
    plus log B so it estimates s_j like Eq. (1) (log B is page-independent).
    sigma_k^2 are the kept Gram eigenvalues (zero modes have zero basis rows)."""
    q = np.asarray(q, dtype=np.float64)
    n, r, d = summary.basis.shape
    B = summary.coeffs.shape[1]
    a = scale * (q @ summary.centroid.T)                              # [G, n]
    proj = np.einsum("nrd,gd->gnr", summary.basis, q)                 # [G, n, r]
    lam = summary.eigvals[:, :r]                                      # [n, r]
    quad = (scale ** 2 / (2 * B)) * np.einsum("nr,gnr->gn", lam, proj ** 2)
    return a + quad + np.log(B)


def centroid_score(q, summary: PageSummary, scale: float) -> np.ndarray:
    """Centroid-only score: Eq. (1) at r = 0, scale q.mu + log B."""
    q = np.asarray(q, dtype=np.float64)
    B = summary.coeffs.shape[1]
    return scale * (q @ summary.centroid.T) + np.log(B)


def combine_shares(page_scores, rule: str) -> np.ndarray:
    """One ranking value per page from per-head log-mass estimates [G, n]:
    "share_average" (the shipped rule, [Locks] §4): mean over heads of the
    normalized shares; "group_max": their maximum; "group_mass": the summed
    unnormalized mass sum_g e^{s_g} (as its log).  The pages name group-max
    and group-mass without formulas; these are the plain readings."""
    s = np.asarray(page_scores, dtype=np.float64)
    if rule == "group_mass":
        return _logsumexp(s, axis=0)
    shares = np.exp(s - _logsumexp(s, axis=-1)[:, None])
    if rule == "share_average":
        return shares.mean(axis=0)
    if rule == "group_max":
        return shares.max(axis=0)
    raise ValueError(f"unknown combine rule {rule!r}")


def select_by_rule(page_scores, n_mr: int, k: int, rule: str) -> list:
    """Selections of one GQA group: one shared set for "share_average",
    "group_max" and "group_mass", one set per head for "per_head" (each head's
    own top-(k-2) by its share).  Returns a list of G page-index arrays."""
    s = np.asarray(page_scores, dtype=np.float64)
    G = s.shape[0]
    if rule == "per_head":
        return [select_pages(np.exp(s[g] - _logsumexp(s[g])), n_mr, k) for g in range(G)]
    return [select_pages(combine_shares(s, rule), n_mr, k)] * G


def head_coverage(exact_page_lse, selections) -> np.ndarray:
    """Per-head coverage gamma_S(q_g) = sum_{j in S_g} m_g(j) of the exact
    page-mass shares over the scored pages ([Locks] Lemma 1); [G]."""
    s = np.asarray(exact_page_lse, dtype=np.float64)
    m = np.exp(s - _logsumexp(s, axis=-1)[:, None])
    n = s.shape[1]
    return np.array([m[g, [j for j in sel if j < n]].sum() for g, sel in enumerate(selections)])


# ----------------------------------------------------------------------------
# byte accounting: [Locks] App. D "State accounting", Table D.10
# ----------------------------------------------------------------------------
def record_elements(head_dim: int, page_size: int, rank: int) -> dict:
    """Elements of one page summary: basis d*r, coefficients B*r, centroid d."""
    return {"basis": head_dim * rank, "coeffs": page_size * rank, "centroid": head_dim}


def summary_bytes(head_dim: int, page_size: int, rank: int,
                  basis_bits: float, coeff_bits: float, centroid_bits: float) -> float:
    """Logical payload bytes of one page summary (quantization scales excluded)."""
    e = record_elements(head_dim, page_size, rank)
    return (e["basis"] * basis_bits + e["coeffs"] * coeff_bits
            + e["centroid"] * centroid_bits) / 8.0
