"""Pins of the fp64 oracle to facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, a value the pages print, an identity or bound the paper proves, a
library routine for a special case, or brute force on tiny inputs.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import locks_oracle as lo

RNG = np.random.default_rng(1234)


def _rand_pages(rng, n, B, d, rank=None, offset=0.0):
    if rank is None:
        return rng.standard_normal((n, B, d)) + offset
    coef = rng.standard_normal((n, B, rank))
    basis = rng.standard_normal((n, rank, d))
    return coef @ basis + offset * rng.standard_normal((n, 1, d))


# ---------------------------------------------------------------- rounding
def test_bf16_round_ties_and_torch_agreement():
    # explicit ties: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 -> even (1)
    assert lo.bf16_round(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert lo.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert lo.bf16_round(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert lo.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    # fp32-exact inputs: a single rounding, so torch's fp32->bf16 (RNE) agrees
    x = RNG.standard_normal(20000).astype(np.float32) * 10.0
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(lo.bf16_round(x.astype(np.float64)), ref)


# ---------------------------------------------------------------- build
def test_review_toy_example_closed_form(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "review_toy_example.json")))
    delta = np.array(g["deviations"])
    mu = np.array(g["centroid_used_in_test"])
    keys = (delta + mu)[None]
    s = lo.build_page_summaries(keys, 1)
    lam1 = 1.82 + math.sqrt(3.2724)
    lam2 = 1.82 - math.sqrt(3.2724)
    np.testing.assert_allclose(s.eigvals[0, :2], [lam1, lam2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(s.eigvals[0, 2:], 0.0, atol=1e-12)
    np.testing.assert_allclose(s.centroid[0], mu, atol=1e-15)
    # tau_{j,1} = sum_{k>1} sigma_k^2
    assert abs(s.eigvals[0, 1:].sum() - lam2) < 1e-12
    # basis = unit eigenvector of [[3.62, .18], [.18, .02]] for lambda_1
    v = np.array([0.18, lam1 - 3.62])
    v /= np.linalg.norm(v)
    np.testing.assert_allclose(s.basis[0, 0], [v[0], v[1], 0, 0], atol=1e-12)
    # coefficients c_i = v^T delta_i
    np.testing.assert_allclose(s.coeffs[0, :, 0], delta @ s.basis[0, 0], atol=1e-12)


@pytest.mark.parametrize("rho,r", [(3, 3), (5, 8), (8, 8), (1, 4)])
def test_exact_reconstruction_when_rank_covers_page(rho, r):
    """delta_i = V c_i exactly when r >= rank(D) ([Locks] §4 "Build")."""
    keys = _rand_pages(RNG, 6, 64, 128, rank=rho, offset=2.0)
    s = lo.build_page_summaries(keys, r)
    D = keys - keys.mean(axis=1, keepdims=True)
    recon = s.coeffs @ s.basis
    assert np.abs(recon - D).max() <= 1e-12 * np.abs(D).max()
    assert (s.r_eff <= rho).all()


def test_basis_orthonormal_coeffs_are_projections_and_residual():
    """V^T V = I, c_i = V^T delta_i, and ||D - D V V^T||_F^2 = sum_{k>r} sigma_k^2
    ([Locks] Cor. 1)."""
    keys = _rand_pages(RNG, 8, 64, 128)
    for r in (4, 8, 16):
        s = lo.build_page_summaries(keys, r)
        D = keys - keys.mean(axis=1, keepdims=True)
        gram_v = s.basis @ np.swapaxes(s.basis, 1, 2)
        np.testing.assert_allclose(gram_v, np.broadcast_to(np.eye(r), gram_v.shape), atol=1e-12)
        np.testing.assert_allclose(s.coeffs, D @ np.swapaxes(s.basis, 1, 2), atol=1e-10)
        resid = D - (D @ np.swapaxes(s.basis, 1, 2)) @ s.basis
        tau = (resid ** 2).sum(axis=(1, 2))
        np.testing.assert_allclose(tau, s.eigvals[:, r:].sum(axis=1), rtol=1e-10)
        # eigenvalues agree with the singular values of D (an independent routine)
        sv = np.linalg.svd(D, compute_uv=False)
        np.testing.assert_allclose(s.eigvals[:, :64], sv ** 2, rtol=1e-9, atol=1e-9)


def test_basis_sign_and_order_conventions():
    keys = _rand_pages(RNG, 5, 64, 128)
    s = lo.build_page_summaries(keys, 8)
    assert (np.diff(s.eigvals, axis=1) <= 1e-12).all()
    lead = np.take_along_axis(s.basis, np.argmax(np.abs(s.basis), axis=2)[..., None], axis=2)
    assert (lead > 0).all()


def test_zero_modes_dropped_and_constant_page():
    # a page of rank 2: modes 3.. are zero modes -> zero basis rows and coefficients
    keys = _rand_pages(RNG, 1, 64, 128, rank=2, offset=1.0)
    s = lo.build_page_summaries(keys, 8)
    assert s.r_eff[0] == 2
    assert np.abs(s.basis[0, 2:]).max() == 0.0 and np.abs(s.coeffs[0, :, 2:]).max() == 0.0
    # a constant page has no nonzero mode: s_hat = q.mu * scale + log B exactly
    const = np.tile(RNG.standard_normal(128), (1, 64, 1))
    s = lo.build_page_summaries(const, 8)
    assert s.r_eff[0] == 0
    q = RNG.standard_normal((3, 128))
    scale = 1 / math.sqrt(128)
    got = lo.reconstructed_page_lse(q, s, scale)[:, 0]
    np.testing.assert_allclose(got, q @ const[0, 0] * scale + math.log(64), rtol=0, atol=1e-12)
    np.testing.assert_allclose(got, lo.exact_page_lse(q, const, scale)[:, 0], atol=1e-12)


def test_isotropic_null_matches_printed_statistic(golden_dir):
    """Rank-8 fit of 20,000 isotropic B=16, d=128 pages captures a median 67.8%
    (mean 0.679, sd 0.009) of the variance ([Locks] App. D "Spectral tails")."""
    g = json.load(open(os.path.join(golden_dir, "isotropic_null.json")))
    rng = np.random.default_rng(7)
    fr = []
    for chunk in range(10):
        keys = rng.standard_normal((g["pages"] // 10, g["page_size"], g["head_dim"]))
        s = lo.build_page_summaries(keys, g["rank"])
        fr.append(s.eigvals[:, :g["rank"]].sum(1) / s.eigvals.sum(1))
    fr = np.concatenate(fr)
    tol = g["printed_precision"]
    assert abs(np.median(fr) - g["median"]) <= tol["median"] + 3e-4
    assert abs(fr.mean() - g["mean"]) <= tol["mean"] + 3e-4
    assert abs(fr.std() - g["std"]) <= tol["std"] + 3e-4


# ---------------------------------------------------------------- score
def test_score_equals_exact_lse_when_rank_covers_page():
    """s_hat_j = s_j whenever r >= rank(D_j) (Prop. 2); also at r = d (clamped)."""
    scale = 1 / math.sqrt(128)
    q = RNG.standard_normal((4, 128)) * 2
    keys = _rand_pages(RNG, 10, 64, 128, rank=6, offset=1.0)
    s = lo.build_page_summaries(keys, 8)
    np.testing.assert_allclose(lo.reconstructed_page_lse(q, s, scale),
                               lo.exact_page_lse(q, keys, scale), atol=1e-12)
    full = _rand_pages(RNG, 4, 64, 128)
    s = lo.build_page_summaries(full, 128)
    np.testing.assert_allclose(lo.reconstructed_page_lse(q, s, scale),
                               lo.exact_page_lse(q, full, scale), atol=1e-10)


def test_rank_zero_is_centroid_only_row():
    """With r = 0 Eq. (1) reduces to q^T mu / sqrt(d) + log B."""
    scale = 1 / math.sqrt(128)
    keys = _rand_pages(RNG, 7, 64, 128)
    q = RNG.standard_normal((2, 128))
    s = lo.build_page_summaries(keys, 0)
    np.testing.assert_allclose(lo.reconstructed_page_lse(q, s, scale),
                               scale * q @ keys.mean(axis=1).T + math.log(64), atol=1e-12)


def test_score_error_bound_prop2():
    """|s_hat - s| <= max_i |q_perp^T delta_perp_i| / sqrt(d) <= ||q_perp|| sqrt(tau) / sqrt(d)."""
    d = 128
    scale = 1 / math.sqrt(d)
    keys = _rand_pages(RNG, 40, 64, d) + 0.7 * _rand_pages(RNG, 40, 64, d, rank=5)
    q = RNG.standard_normal((4, d)) * 3
    for r in (2, 8):
        s = lo.build_page_summaries(keys, r)
        err = np.abs(lo.reconstructed_page_lse(q, s, scale) - lo.exact_page_lse(q, keys, scale))
        D = keys - keys.mean(axis=1, keepdims=True)
        P = np.swapaxes(s.basis, 1, 2) @ s.basis            # [n, d, d] projector
        dperp = D - D @ P
        qperp = q[None] - q[None] @ P                        # [n, G, d]
        first = np.abs(np.einsum("ngd,nbd->gnb", qperp, dperp)).max(axis=2) * scale
        tau = s.eigvals[:, r:].sum(1)
        second = np.linalg.norm(qperp, axis=2).T * np.sqrt(tau)[None] * scale
        assert (err <= first + 1e-12).all()
        assert (first <= second + 1e-12).all()
        assert err.max() > 1e-6  # the bound is exercised, not vacuous


def test_lemma3_outlier_capture():
    d, r = 128, 8
    keys = _rand_pages(RNG, 20, 64, d)
    keys[:, 5] += 6.0 * RNG.standard_normal((20, d))  # one dominant key per page
    s = lo.build_page_summaries(keys, r)
    D = keys - keys.mean(axis=1, keepdims=True)
    q = RNG.standard_normal(d)
    captured = (s.eigvals[:, :r] * (s.basis @ q) ** 2).sum(1)
    for i_star in range(64):
        rhs = (D[:, i_star] @ q) ** 2 - s.eigvals[:, r] * (q @ q)
        assert (captured >= rhs - 1e-9).all()


# ---------------------------------------------------------------- share + select
def test_share_average_is_shift_invariant_and_a_distribution():
    s = RNG.standard_normal((4, 30)) * 5
    m = lo.share_average(s)
    np.testing.assert_allclose(m.sum(), 1.0, atol=1e-14)
    np.testing.assert_allclose(lo.share_average(s + np.array([[3.0], [-7.0], [100.0], [0.5]])), m, atol=1e-14)
    # G = 1: the share is the softmax of the scores
    sm = torch.softmax(torch.from_numpy(s[:1]), dim=1).numpy()[0]
    np.testing.assert_allclose(lo.share_average(s[:1]), sm, atol=1e-15)


def test_selection_brute_force_cor3():
    """Top-(k-2) by m_bar maximizes sum_{j in S} m_bar_j over sets holding the
    sink and the most recent page ([Locks] Cor. 3): brute force on tiny inputs."""
    rng = np.random.default_rng(99)
    for trial in range(60):
        n_mr = int(rng.integers(1, 13))
        k = int(rng.integers(2, 8))
        m_bar = rng.random(n_mr)
        sel = lo.select_pages(m_bar, n_mr, k)
        assert sel[0] == 0 and sel[-1] == n_mr and (np.diff(sel) > 0).all()
        cand = list(range(1, n_mr))
        n_top = min(k - 2, len(cand))
        assert len(sel) == 2 + n_top
        best = max(sum(m_bar[j] for j in c) for c in itertools.combinations(cand, n_top))
        got = sum(m_bar[j] for j in sel if j not in (0, n_mr))
        assert abs(got - best) < 1e-12
    assert list(lo.select_pages(np.zeros(0), 0, 8)) == [0]
    # ties at the cut go to the lower index
    assert list(lo.select_pages(np.array([9.0, 1.0, 1.0, 1.0, 0.5]), 5, 4)) == [0, 1, 2, 5]


def test_retention_guarantee_thm1():
    """Group-share sandwich |log m_bar_hat - log m_bar| <= 2 eta and Thm. 1(ii):
    coverage of the estimated selection >= e^{-4 eta} x exact-selection coverage."""
    d, B, G, scale = 64, 16, 4, 1 / 8.0
    rng = np.random.default_rng(5)
    for trial in range(25):
        n = int(rng.integers(6, 14))
        keys = rng.standard_normal((n, B, d)) * 0.8 + rng.standard_normal((n, B, 3)) @ rng.standard_normal((n, 3, d))
        q = rng.standard_normal((G, d)) * 2
        r = int(rng.integers(1, 4))
        s = lo.build_page_summaries(keys, r)
        sh = lo.reconstructed_page_lse(q, s, scale)
        se = lo.exact_page_lse(q, keys, scale)
        eta = np.abs(sh - se).max()
        mh, me = lo.share_average(sh), lo.share_average(se)
        assert np.abs(np.log(mh) - np.log(me)).max() <= 2 * eta + 1e-12
        n_mr = n - 1
        k = int(rng.integers(3, 7))
        cov = lambda S: me[[j for j in S if j < n_mr]].sum()  # noqa: E731
        S_hat = lo.select_pages(mh[:n_mr], n_mr, k)
        S_ex = lo.select_pages(me[:n_mr], n_mr, k)
        assert cov(S_hat) >= math.exp(-4 * eta) * cov(S_ex) - 1e-12


def test_exact_mass_topk_maximizes_coverage_lemma1ii():
    rng = np.random.default_rng(3)
    for _ in range(20):
        n, B, d = 9, 8, 16
        keys = rng.standard_normal((n, B, d))
        q = rng.standard_normal((1, d)) * 2
        s = lo.exact_page_lse(q, keys, 0.25)[0]
        w = np.exp(s - s.max()); w /= w.sum()
        k = 3
        top = np.argsort(-s)[:k]
        best = max(w[list(c)].sum() for c in itertools.combinations(range(n), k))
        assert abs(w[top].sum() - best) < 1e-12


# ---------------------------------------------------------------- attention
def test_dense_attention_matches_sdpa_fp64():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((4, 128))
    K = rng.standard_normal((300, 128))
    V = rng.standard_normal((300, 128))
    o, lse = lo.attend(q, K, V, 1 / math.sqrt(128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(K)[None, None].expand(1, 4, 300, 128),
        torch.from_numpy(V)[None, None].expand(1, 4, 300, 128))[0, :, 0].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    ref_lse = torch.logsumexp(torch.from_numpy(q @ K.T / math.sqrt(128)), dim=1).numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_lemma1_exact_deficit_identity():
    """o - o_S = eps (v_bar_{S^c} - v_bar_S) and ||o_S - o|| <= 2R(1 - gamma_S)."""
    rng = np.random.default_rng(12)
    B, d, n = 16, 32, 10
    keys = rng.standard_normal((n, B, d))
    vals = rng.standard_normal((n, B, d))
    q = rng.standard_normal((1, d)) * 1.5
    scale = 1 / math.sqrt(d)
    T = n * B
    o, _ = lo.attend(q, keys.reshape(T, d), vals.reshape(T, d), scale)
    for S in ([0, 3, 9], [1, 2], [0, 4, 5, 6, 7]):
        Sc = [j for j in range(n) if j not in S]
        oS, _ = lo.attend(q, lo.gather_tokens(keys, S, T, B), lo.gather_tokens(vals, S, T, B), scale)
        oC, _ = lo.attend(q, lo.gather_tokens(keys, Sc, T, B), lo.gather_tokens(vals, Sc, T, B), scale)
        mass = np.exp(lo.exact_page_lse(q, keys, scale)[0])
        gamma = mass[S].sum() / mass.sum()
        np.testing.assert_allclose(o - oS, (1 - gamma) * (oC - oS), atol=1e-12)
        R = np.linalg.norm(vals.reshape(T, d), axis=1).max()
        assert np.linalg.norm(oS - o) <= 2 * R * (1 - gamma) + 1e-12


def test_gather_tokens_partial_tail_and_decode_head_dense_limit():
    rng = np.random.default_rng(13)
    B, d, G = 8, 16, 2
    T = 5 * B + 3
    keys = rng.standard_normal((6, B, d))
    vals = rng.standard_normal((6, B, d))
    toks = lo.gather_tokens(keys, [0, 5], T, B)
    assert toks.shape == (B + 3, d)
    np.testing.assert_array_equal(toks[B:], keys[5, :3])
    # full-rank summaries and a budget covering every page: the step is dense attention
    q = rng.standard_normal((G, d))
    s = lo.build_page_summaries(keys[:5], B)
    hs = lo.decode_head(q, keys, vals, T, s, token_budget=6 * B, scale=0.25)
    assert list(hs.selected) == [0, 1, 2, 3, 4, 5]
    o, lse = lo.attend(q, keys.reshape(-1, d)[:T], vals.reshape(-1, d)[:T], 0.25)
    np.testing.assert_allclose(hs.out, o, atol=1e-12)
    np.testing.assert_allclose(hs.page_lse, lo.exact_page_lse(q, keys[:5], 0.25), atol=1e-12)
    # a sequence that fits in one page attends page 0 only
    hs = lo.decode_head(q, keys, vals, 5, s, token_budget=2 * B, scale=0.25)
    assert list(hs.selected) == [0]


def test_empty_sequence_selects_nothing_and_attends_to_nothing():
    """A sequence with no token holds no page: the selection is empty (its size
    min(k, n_mr + 1) is 0), and attention is an empty sum, whose log-sum-exp is
    log 0 = -inf (as torch.logsumexp gives over an empty axis) and whose output
    is the zero vector."""
    rng = np.random.default_rng(17)
    B, d, G, k = 8, 16, 2, 4
    keys = rng.standard_normal((3, B, d))
    vals = rng.standard_normal((3, B, d))
    q = rng.standard_normal((G, d))
    for T in range(0, 3 * B + 1):
        n_mr = lo.most_recent_page(T, B)
        assert n_mr == (-1 if T == 0 else (T - 1) // B)
        s = lo.build_page_summaries(keys[:max(n_mr, 0)], 4)
        hs = lo.decode_head(q, keys, vals, T, s, token_budget=k * B, scale=0.25)
        assert len(hs.selected) == min(k, n_mr + 1)
        assert hs.page_lse.shape == (G, max(n_mr, 0))
    hs = lo.decode_head(q, keys, vals, 0, lo.build_page_summaries(keys[:0], 4), token_budget=k * B, scale=0.25)
    assert hs.selected.size == 0 and hs.m_bar.size == 0
    empty_lse = torch.logsumexp(torch.empty((G, 0), dtype=torch.float64), dim=1).numpy()
    np.testing.assert_array_equal(hs.lse, empty_lse)
    np.testing.assert_array_equal(hs.out, np.zeros((G, d)))


# ---------------------------------------------------------------- byte model
def test_table_d10_byte_accounting(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "table_d10_bytes.json")))
    for row in g["rows"]:
        b = lo.summary_bytes(g["head_dim"], g["page_size"], row["rank"], row["basis_bits"], 8, 8)
        assert b == row["bytes"], row
        assert abs(100 * b / g["kv_bytes"] - row["pct"]) < 0.06


# ----------------------------------------------------------------------------
# quantized summary ([Locks] §4 "Build": int4 basis with per-column scales,
# int8 coefficients and centroid with per-row scales; App. D)
# ----------------------------------------------------------------------------
def test_quantize_symmetric_properties():
    """Every entry comes back within half a step (the row maximum may lose the
    sliver by which the fp16 scale was rounded down), the row maximum sits on
    +-levels, codes are integers in range, the scale is an fp16 value within
    half an fp16 ulp of max|x| / levels, and a power-of-two rescale of a row
    only rescales its scale."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((200, 128)) * rng.uniform(0.01, 10.0, (200, 1))
    for levels in (lo.QUANT_BASIS_LEVELS, lo.QUANT_ROW_LEVELS):
        q, s = lo.quantize_symmetric(x, levels)
        assert q.dtype.kind == "i" and np.abs(q).max() <= levels
        amax = np.abs(x).max(axis=1)
        slack = np.maximum(amax - levels * s, 0.0)
        assert (np.abs(x - q * s[:, None]) <= (s / 2 + slack)[:, None] + 1e-12).all()
        big = np.argmax(np.abs(x), axis=1)
        assert (np.abs(q[np.arange(len(x)), big]) == levels).all()
        assert (s.astype(np.float16).astype(np.float64) == s).all()
        assert (np.abs(s - amax / levels) <= (amax / levels) * 2.0 ** -11).all()
        q8, s8 = lo.quantize_symmetric(x * 8.0, levels)
        assert (q8 == q).all() and (s8 == 8.0 * s).all()
    zq, zs = lo.quantize_symmetric(np.zeros((2, 16)), 7)
    assert (zq == 0).all() and (zs == 0).all()


def test_quantized_summary_lossless_case_and_score():
    """Rows that are exact multiples k * s of an fp16 scale with max |k| = levels
    are reproduced exactly (codes, scales and dequantized values), so Eq. (1) on
    the dequantized summary equals Eq. (1) on the original."""
    rng = np.random.default_rng(22)
    n, B, d, r = 5, 64, 128, 8

    def exact(shape, levels):
        k = rng.integers(-levels, levels + 1, size=shape)
        k[..., 3] = -levels
        s = lo.fp16_round(rng.uniform(1e-3, 2.0, size=shape[:-1]))
        return k * s[..., None], k, s

    basis, bk, bsc = exact((n, r, d), lo.QUANT_BASIS_LEVELS)
    coeffs, ck, csc = exact((n, B, r), lo.QUANT_ROW_LEVELS)
    mu, mk, msc = exact((n, d), lo.QUANT_ROW_LEVELS)
    summ = lo.PageSummary(centroid=mu, basis=basis, coeffs=coeffs, eigvals=np.zeros((n, B)),
                          r_eff=np.full(n, r))
    qs = lo.quantize_summary(summ)
    assert (qs.basis_q == bk).all() and (qs.coeffs_q == ck).all() and (qs.centroid_q == mk).all()
    assert (qs.basis_s == bsc).all() and (qs.coeffs_s == csc).all() and (qs.centroid_s == msc).all()
    back = lo.dequantize_summary(qs)
    assert (back.basis == basis).all() and (back.coeffs == coeffs).all() and (back.centroid == mu).all()
    q = rng.standard_normal((4, d))
    np.testing.assert_allclose(lo.reconstructed_page_lse(q, back, 0.0884),
                               lo.reconstructed_page_lse(q, summ, 0.0884), rtol=0, atol=1e-12)


def test_quantized_build_zero_modes_and_score_perturbation():
    """On built pages: zero modes (a page of rank 3 at r = 8) quantize to zero
    scales and codes; the quantized score moves by at most the largest change of
    a reconstructed logit (log-sum-exp is 1-Lipschitz in the sup norm, [Locks]
    Prop. 2 proof), and every dequantized entry is within half a step."""
    rng = np.random.default_rng(23)
    d, B, r = 128, 64, 8
    low = rng.standard_normal((2, B, 3)) @ rng.standard_normal((2, 3, d)) + 0.3
    pages = np.concatenate([low, rng.standard_normal((4, B, d))], axis=0)
    summ = lo.build_page_summaries(pages, r, dtype="f64")
    qs = lo.quantize_summary(summ)
    assert (qs.basis_s[:2, 3:] == 0).all() and (qs.basis_q[:2, 3:] == 0).all()
    assert (qs.coeffs_q[:2, :, 3:] == 0).all()
    back = lo.dequantize_summary(qs)
    for a, b, sc in ((summ.basis, back.basis, qs.basis_s), (summ.coeffs, back.coeffs, qs.coeffs_s),
                     (summ.centroid, back.centroid, qs.centroid_s)):
        assert (np.abs(a - b) <= sc[..., None] / 2 + 1e-12).all()
    q = rng.standard_normal((4, d)) * 2.0
    scale = 1 / np.sqrt(d)

    def logits(sm):
        a = q @ sm.centroid.T
        proj = np.einsum("nrd,gd->gnr", sm.basis, q)
        return scale * (a[:, :, None] + np.einsum("nbr,gnr->gnb", sm.coeffs, proj))

    dz = np.abs(logits(back) - logits(summ)).max(axis=-1)
    ds = np.abs(lo.reconstructed_page_lse(q, back, scale) - lo.reconstructed_page_lse(q, summ, scale))
    assert (ds <= dz + 1e-12).all() and dz.max() > 0


# ----------------------------------------------------------------------------
# rival scores and GQA combine rules (diagnostics)
# ----------------------------------------------------------------------------
def test_envelope_bounds_every_logit_and_is_content_blind():
    """[Locks] Lemma 2: the envelope score upper-bounds every within-page logit
    (so s_j <= e_j + log B), and depends on a page only through its
    per-dimension extremes: a page whose columns are permuted independently
    (same extremes, other keys) gets the same envelope score but another mass."""
    rng = np.random.default_rng(31)
    d, B = 128, 64
    keys = rng.standard_normal((6, B, d))
    q = rng.standard_normal((4, d)) * 2.0
    scale = 1 / np.sqrt(d)
    env = lo.envelope_page_score(q, keys, scale)
    logits = scale * np.einsum("gd,nbd->gnb", q, keys)
    assert (logits.max(axis=-1) <= env + 1e-12).all()
    assert (lo.exact_page_lse(q, keys, scale) <= env + np.log(B) + 1e-12).all()
    shuffled = np.stack([rng.permutation(keys[0][:, c]) for c in range(d)], axis=1)[None]
    np.testing.assert_allclose(lo.envelope_page_score(q, shuffled, scale), env[:, :1], rtol=0, atol=1e-12)
    assert np.abs(lo.exact_page_lse(q, shuffled, scale) - lo.exact_page_lse(q, keys[:1], scale)).max() > 1e-3


def test_moment_core_is_the_second_order_truncation():
    """[Locks] Eq. (A.2): with keys mu + eps * delta, the exact page log-mass
    minus the moment core shrinks like eps^3 (the truncation drops the third
    and higher cumulants; a wrong second-order coefficient would leave eps^2);
    at r >= rank the rank-r form equals (1/(2Bd)) q^T D^T D q directly."""
    rng = np.random.default_rng(32)
    d, B, rho = 128, 64, 6
    dev = rng.standard_normal((3, B, rho)) @ rng.standard_normal((3, rho, d))
    dev -= dev.mean(axis=1, keepdims=True)
    mu = rng.standard_normal((3, 1, d))
    q = rng.standard_normal((2, d)) * 3.0
    scale = 1 / np.sqrt(d)
    errs = []
    for eps in (0.02, 0.01):
        keys = mu + eps * dev
        summ = lo.build_page_summaries(keys, 8, "f64")
        errs.append(np.abs(lo.exact_page_lse(q, keys, scale) - lo.moment_core_score(q, summ, scale)).max())
        D = keys - keys.mean(axis=1, keepdims=True)
        direct = scale * (q @ keys.mean(axis=1).T) + np.log(B) + np.einsum(
            "gd,nbd,nbe,ge->gn", q, D, D, q) / (2 * B * d)
        np.testing.assert_allclose(lo.moment_core_score(q, summ, scale), direct, rtol=0, atol=1e-10)
    assert errs[0] / errs[1] > 6.0, errs


def test_centroid_score_is_rank_zero():
    rng = np.random.default_rng(33)
    keys = rng.standard_normal((4, 64, 128))
    summ = lo.build_page_summaries(keys, 8, "f64")
    q = rng.standard_normal((3, 128))
    zeroed = lo.PageSummary(centroid=summ.centroid, basis=summ.basis, coeffs=np.zeros_like(summ.coeffs),
                            eigvals=summ.eigvals, r_eff=summ.r_eff)
    np.testing.assert_allclose(lo.centroid_score(q, summ, 0.088), lo.reconstructed_page_lse(q, zeroed, 0.088),
                               rtol=0, atol=1e-12)


def test_combine_rules_coverage_orderings():
    """On exact shares: share-average has the largest group-mean coverage of
    every shared rule ([Locks] Cor. 3), each head's own selection covers that
    head at least as well as any shared one, and with G = 1 every rule is the
    same selection."""
    rng = np.random.default_rng(34)
    for trial in range(40):
        G, n = 4, int(rng.integers(20, 80))
        s = rng.standard_normal((G, n)) * rng.uniform(0.5, 4.0)
        n_mr, k = n, int(rng.integers(3, 12))
        cov = {r: lo.head_coverage(s, lo.select_by_rule(s, n_mr, k, r))
               for r in ("share_average", "group_max", "group_mass", "per_head")}
        assert cov["share_average"].mean() >= cov["group_max"].mean() - 1e-12
        assert cov["share_average"].mean() >= cov["group_mass"].mean() - 1e-12
        for r in ("share_average", "group_max", "group_mass"):
            assert (cov["per_head"] >= cov[r] - 1e-12).all()
        one = s[:1]
        sels = [lo.select_by_rule(one, n_mr, k, r)[0].tolist() for r in ("share_average", "group_max", "group_mass", "per_head")]
        assert all(x == sels[0] for x in sels)
