"""Pins of the oracle's top-p deterministic stratum (no GPU).

"Stratified Sparse Attention speeds up decoding 2.96x at 1M context",
"Where sparse attention loses quality": top-p is one of the deterministic
options -- the highest-estimate tokens up to a probability mass p.  The
oracle counts mass in integer units of 2^-38 of the largest weight.  The pins
below check it against what the definition fixes without those units: closed
forms for uniform and two-level scores, the float64 softmax (libm exp) of the
scores within the quantisation error, and the estimator's unbiasedness by
enumeration with a top-p stratum.  The last test plants plausible slips.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import ssa_oracle as orc

P_VALUES = (0.0, 2.0 ** -30, 0.1, 0.25, 0.5, 0.7, 0.9, 0.95, 0.999, 1.0)


def exact_ceil(p, n):
    """ceil(p * n) for the float32 p, by exact rational arithmetic."""
    x = Fraction(float(np.float32(p))) * n
    return -((-x.numerator) // x.denominator)


def uniform_case_error():
    """Uniform scores: every token holds 1/L of the mass, so the prefix is the
    ceil(p L) lowest indices (ties go to the lower index)."""
    bad = 0
    for L in (1, 7, 1000, 4099):
        s = np.full(L, np.float32(0.37))
        for p in P_VALUES:
            n = orc.topp_count(s, p)
            bad += n != exact_ceil(p, L)
            st = orc.tail_stratum(s, L, 0, top_p=p)
            if not st["dense"]:
                bad += not np.array_equal(st["S"], np.arange(exact_ceil(p, L)))
    return bad


def test_uniform_scores_closed_form():
    assert uniform_case_error() == 0


def two_level_error():
    """a tokens at the maximum, the rest far below (exp underflows to 0): the
    prefix is ceil(p a) of the high tokens, never a zero-mass one."""
    rng = np.random.default_rng(3)
    bad = 0
    for L, a in ((500, 37), (4096, 1), (4096, 300)):
        s = np.full(L, np.float32(-150.0))
        hi = rng.choice(L, a, replace=False)
        s[hi] = np.float32(2.5)
        for p in P_VALUES:
            n = orc.topp_count(s, p)
            bad += n != exact_ceil(p, a)
            st = orc.tail_stratum(s, L, 0, top_p=p)
            bad += not np.array_equal(st["S"], np.sort(hi)[:n])
    return bad


def test_two_level_scores_closed_form():
    assert two_level_error() == 0


def softmax_case_error(nseeds=6):
    """Random scores: with P the float64 softmax (libm exp), the prefix reaches
    p and the prefix one shorter does not, up to the quantisation error
    (L * 2^-38 of the top weight, plus a few ulp of float32 exp)."""
    worst = 0.0
    for seed in range(nseeds):
        rng = np.random.default_rng(100 + seed)
        L = int(rng.integers(200, 5000))
        s = (rng.standard_normal(L) * rng.uniform(0.5, 4.0)).astype(np.float32)
        s64 = s.astype(np.float64)
        P = np.exp(s64 - s64.max())
        P /= P.sum()
        order = sorted(range(L), key=lambda j: (-s64[j], j))
        cum = np.cumsum(P[order])
        eps = 1e-6
        for p in rng.uniform(0.05, 0.999, 12):
            p32 = np.float32(p)
            n = orc.topp_count(s, p32)
            assert 1 <= n <= L
            reach = float(cum[n - 1]) - float(p32)                      # must be >= -eps
            short = float(p32) - (float(cum[n - 2]) if n > 1 else 0.0)  # must be > -eps
            worst = max(worst, -reach, -short)
            st = orc.tail_stratum(s, L, 0, top_p=p32)
            assert np.array_equal(st["S"], np.sort(order[:n]))
    return worst


def test_prefix_matches_float64_softmax():
    assert softmax_case_error() < 1e-6


def units_boundary_error():
    """Integer units at the target: one token at the maximum (2^38 units) and
    32768 tokens at e^-26 of it (1.4 units each, floored to 1).  With
    p = 1 - 2^-24, p * Q = 2^38 + 16384 - 2^-9, so the target is 2^38 + 16384
    units and the prefix holds the top token and the first 16384 others."""
    x = np.float32(-26.0)
    assert orc.mass_units(orc.sexp(x)) == 1
    s = np.concatenate([[np.float32(0.0)], np.full(32768, x)]).astype(np.float32)
    p = np.float32(1.0 - 2.0 ** -24)
    return abs(orc.topp_count(s, p) - (1 + 16384))


def test_integer_units_at_the_target():
    assert units_boundary_error() == 0


def test_top_p_and_top_k_cap_each_other():
    rng = np.random.default_rng(9)
    s = rng.standard_normal(3000).astype(np.float32)
    n = orc.topp_count(s, np.float32(0.8))
    for topk in (0, 1, n - 1, n, n + 1, 3000):
        st = orc.tail_stratum(s, topk, 10, top_p=np.float32(0.8))
        k = min(topk, n)
        assert st["S"].size == k
        assert np.array_equal(st["S"], orc.topk_indices(s, k))
    # monotone in p; p = 0 and NaN leave no deterministic set; p >= 1 saturates
    ns = [orc.topp_count(s, p) for p in np.linspace(0, 1, 41, dtype=np.float32)]
    assert ns == sorted(ns) and ns[0] == 0
    assert orc.topp_count(s, np.float32("nan")) == 0
    assert orc.topp_count(s, np.float32(3.0)) == orc.topp_count(s, np.float32(1.0))
    # dense rule on the actual stratum size: k + m >= L
    st = orc.tail_stratum(s, 3000, 3000 - n, top_p=np.float32(0.8))
    assert st["dense"]
    st = orc.tail_stratum(s, 3000, 3000 - n - 1, top_p=np.float32(0.8))
    assert not st["dense"] and st["S"].size == n


def top_p_enumeration_error(p):
    """E[N_hat], E[D_hat] over every sample outcome with a top-p stratum, against
    the exact sums from torch's float64 SDPA and logsumexp."""
    rng = np.random.default_rng(21)
    G, d, L = 2, 8, 17
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    scale = 0.7
    s32 = orc.approx_scores(q, K, 0, d // 2, scale).astype(np.float32)
    st = orc.tail_stratum(s32, L, 4, top_p=np.float32(p))
    assert 0 < st["S"].size < L - 4
    T, pi = st["T"], st["pi"].astype(np.float64)
    shift = np.zeros(G)
    EN = np.zeros((G, d))
    ED = np.zeros(G)
    for mask in range(1 << T.size):
        x = np.array([(mask >> i) & 1 for i in range(T.size)], bool)
        P = float(np.prod(np.where(x, pi, 1 - pi)))
        if P == 0.0:
            continue
        N, D = orc.ht_terms(q, K, V, st["S"], T[x], st["pi"][x], scale, shift)
        EN += P * N
        ED += P * D
    l = torch.from_numpy(scale * (q @ K.T))
    Dt = torch.exp(torch.logsumexp(l, dim=1)).numpy()
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :],
        torch.from_numpy(K)[None, None].expand(1, G, L, d),
        torch.from_numpy(V)[None, None].expand(1, G, L, d), scale=scale)[0, :, 0, :].numpy()
    Nt = o * Dt[:, None]
    return max(np.abs(EN - Nt).max() / np.abs(Nt).max(), np.abs(ED - Dt).max() / Dt.max())


def test_estimator_unbiased_with_top_p_stratum():
    assert top_p_enumeration_error(0.6) < 1e-12


def test_pins_catch_planted_top_p_mistakes(monkeypatch):
    """Each mutation is a plausible slip in the top-p count; a pin must fail."""
    real = orc.topp_count
    # 1. one token too many (searching past the target)
    monkeypatch.setattr(orc, "topp_count", lambda s, p: min(real(s, p) + 1, np.asarray(s).size)
                        if real(s, p) > 0 else 0)
    assert uniform_case_error() > 0 and softmax_case_error(2) > 1e-6
    monkeypatch.undo()
    # 2. one token too few
    monkeypatch.setattr(orc, "topp_count", lambda s, p: max(real(s, p) - 1, 0))
    assert two_level_error() > 0 and softmax_case_error(2) > 1e-6
    monkeypatch.undo()
    # 3. target taken as floor(p * Q) instead of the ceiling
    real_target = orc.mass_target

    def floor_target(p, Q):
        t = real_target(p, Q)
        return t - 1 if 0 < t < Q and Fraction(float(np.float32(p))) * Q != t else t
    monkeypatch.setattr(orc, "mass_target", floor_target)
    assert units_boundary_error() > 0
    monkeypatch.undo()
    # 4. mass of the lowest tokens first (ascending order)
    def ascending(s, p):
        s = np.asarray(s, np.float32)
        return real(-s, p)
    monkeypatch.setattr(orc, "topp_count", ascending)
    assert softmax_case_error(2) > 1e-6
    monkeypatch.undo()
