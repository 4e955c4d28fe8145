"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something the pages or mathematics fix:
a special case that reduces to a library routine (torch's scaled-dot-product
attention, a full sort), an independent implementation called rather than
copied (rocRAND's Philox engine, libm's exp via numpy float64), an exact
expectation by enumeration, or a Monte-Carlo bound.  The mutation tests at the
end plant plausible mistakes in the oracle and check that a pin catches each.
"""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

from oracle import ssa_oracle as orc
from long_context_sparse_approx_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))


# ---------------------------------------------------------------- helpers

def sdpa_f64(qg, K, V, scale, mask=None):
    """torch's SDPA in float64 for one group: qg [G, d], K/V [L, d]."""
    q = torch.from_numpy(qg)[None, :, None, :]          # [1, G, 1, d]
    k = torch.from_numpy(K)[None, None].expand(1, qg.shape[0], *K.shape)
    v = torch.from_numpy(V)[None, None].expand(1, qg.shape[0], *V.shape)
    am = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=am, scale=scale)
    return o[0, :, 0, :].numpy()


def true_terms(qg, K, V, scale, shift):
    """N = sum_j e^{l_j - shift} v_j and D = sum_j e^{l_j - shift} via SDPA and logsumexp."""
    l = torch.from_numpy(scale * (qg @ K.T))
    D = torch.exp(torch.logsumexp(l, dim=1) - torch.from_numpy(shift)).numpy()
    N = sdpa_f64(qg, K, V, scale) * D[:, None]
    return N, D


def tiny_unit(L=4096, data_seed=1, **kw):
    wl = synth.make_workload("tiny", "cpu", L=L, data_seed=data_seed, **kw)
    hs = wl.host()
    b, h = 0, 0
    qg = hs["q"][0]
    K = orc.gather_rows(hs["k_cache"], hs["block_table"][b], h, L)
    V = orc.gather_rows(hs["v_cache"], hs["block_table"][b], h, L)
    return wl, hs, qg, K, V


# ---------------------------------------------------------------- sexp

def check_sexp_ulp(bound=2.0):
    x = np.concatenate([np.linspace(-87.0, 0.0, 400001, dtype=np.float32),
                        -np.abs(np.random.default_rng(0).standard_normal(200000) * 4)
                        .astype(np.float32)])
    x = x[x >= -87.0]
    y = orc.sexp(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.abs(y - ref) / np.spacing(ref.astype(np.float32)).astype(np.float64)
    return float(ulp.max())


def test_sexp_within_two_ulp_of_libm():
    assert check_sexp_ulp() <= 2.0


def test_sexp_special_points():
    assert orc.sexp(np.float32(0.0)) == np.float32(1.0)
    assert orc.sexp(np.float32(-87.5)) == 0.0
    assert orc.sexp(np.float32(-np.inf)) == 0.0
    y = orc.sexp(np.float32(-87.0))
    assert y > 0 and y >= np.finfo(np.float32).tiny  # a normal float
    k = np.arange(0, 125)
    x = (-k * math.log(2.0)).astype(np.float32)
    y = orc.sexp(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    assert np.all(np.abs(y - ref) <= 2 * np.spacing(ref.astype(np.float32)))


# ---------------------------------------------------------------- Philox

def _build_rocrand_helper(tmpdir):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND helper")
    exe = os.path.join(tmpdir, "rocrand_philox_words")
    subprocess.run([hipcc, "-O1", os.path.join(HERE, "helpers", "rocrand_philox_words.cpp"),
                    "-o", exe], check=True, capture_output=True)
    return exe


def rocrand_words(exe, queries):
    inp = "".join(f"{s} {b} {h} {j}\n" for s, b, h, j in queries)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [int(x) for x in out.split()]


PHILOX_QUERIES = [(0, 0, 0, j) for j in range(12)] + [
    (0x0123456789ABCDEF, 3, 5, 7), (0xFFFFFFFFFFFFFFFF, 31, 7, 1048575),
    (1000, 17, 2, 65536), (2**32 + 5, 1, 0, 4095), (12345, 0, 7, 3), (1, 2, 3, 4),
    (0xDEADBEEF00000000, 255, 15, 1 << 25), (7, 31, 1, 131071)]


def oracle_words(queries):
    return [int(orc.philox_word(s, b, h, np.array([j]))[0]) for s, b, h, j in queries]


def test_philox_matches_rocrand(tmp_path):
    exe = _build_rocrand_helper(str(tmp_path))
    assert oracle_words(PHILOX_QUERIES) == rocrand_words(exe, PHILOX_QUERIES)


def test_uniforms_are_uniform():
    j = np.arange(200000)
    u = orc.uniforms(42, 1, 2, j).astype(np.float64)
    assert u.min() >= 0.0 and u.max() < 1.0
    counts, _ = np.histogram(u, bins=100, range=(0, 1))
    chi2 = ((counts - 2000.0) ** 2 / 2000.0).sum()
    assert chi2 < 160  # 99 dof; P(chi2 > 160) ~ 1e-4
    # the 24-bit grid: u * 2^24 is an integer
    assert np.all(np.floor(u * 2**24) == u * 2**24)


# ---------------------------------------------------------------- paging

def test_gather_rows_follows_the_block_table():
    """Brute force: write each token's own position into its paged slot with
    plain loops, then gather it back."""
    rng = np.random.default_rng(4)
    L, Hkv, d = 77, 3, 4
    nblk = (L + 15) // 16
    phys = rng.permutation(nblk + 5)[:nblk]
    cache = np.full((nblk + 5, Hkv, 16, d), -1.0)
    for j in range(L):
        for h in range(Hkv):
            cache[phys[j // 16], h, j % 16, :] = [j, h, j % 16, phys[j // 16]]
    for h in range(Hkv):
        rows = orc.gather_rows(cache, phys, h, L)
        assert rows.shape == (L, d)
        assert np.array_equal(rows[:, 0], np.arange(L)) and np.all(rows[:, 1] == h)


# ---------------------------------------------------------------- ranking

def test_order_key_is_monotone():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-40, 38, 5000),
                        [0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38]]).astype(np.float32)
    v = v[np.isfinite(v)]
    key = orc.order_key(v)
    by_key = v[np.argsort(key, kind="stable")]
    assert np.all(np.diff(by_key.astype(np.float64)) >= 0)
    assert orc.order_key(np.float32(-0.0)) < orc.order_key(np.float32(0.0))


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(5)
    s = rng.standard_normal(300).astype(np.float32)
    s[rng.integers(0, 300, 60)] = s[rng.integers(0, 300, 60)]  # forced duplicates
    s[10] = s[20] = s[30] = np.float32(s.max())
    s[40], s[41] = np.float32(-0.0), np.float32(0.0)
    for k in (0, 1, 3, 17, 150, 299, 300):
        # -0.0 == +0.0 as floats; the brute force ranks -0.0 below +0.0 explicitly
        brute = sorted(range(300), key=lambda j: (-float(s[j]), 0 if math.copysign(1, s[j]) > 0 else 1, j))[:k]
        assert list(orc.topk_indices(s, k)) == sorted(brute), k


# ---------------------------------------------------------------- scores

def scores_error():
    rng = np.random.default_rng(7)
    d, L = 64, 50
    q = rng.standard_normal((1, d))
    K = rng.standard_normal((L, d))
    scale = 1 / 8.0
    full = (torch.from_numpy(q) @ torch.from_numpy(K).T).numpy()[0] * scale
    err = np.abs(orc.approx_scores(q, K, 0, d // 2, scale) - full).max()
    # a pair subset equals the exact logit of vectors with the other dims zeroed
    pb, pc = 8, 16
    qz = q.copy()
    keep = np.zeros(d, bool)
    keep[2 * pb:2 * (pb + pc)] = True
    qz[:, ~keep] = 0.0
    part = (torch.from_numpy(qz) @ torch.from_numpy(K).T).numpy()[0] * scale
    return max(err, np.abs(orc.approx_scores(q, K, pb, pc, scale) - part).max())


def test_scores_reduce_to_exact_logits():
    assert scores_error() < 1e-12


def test_scores_average_the_group():
    rng = np.random.default_rng(8)
    G, d, L = 4, 64, 40
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    per_head = np.stack([orc.approx_scores(q[g:g + 1], K, 16, 16, 0.125) for g in range(G)])
    assert np.allclose(orc.approx_scores(q, K, 16, 16, 0.125), per_head.mean(0), rtol=1e-13)
    proxy = q.mean(0, keepdims=True)  # PIVOT's mean proxy query
    assert np.allclose(orc.approx_scores(q, K, 16, 16, 0.125),
                       orc.approx_scores(proxy, K, 16, 16, 0.125), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- special cases

def test_dense_rule_equals_sdpa():
    wl, hs, qg, K, V = tiny_unit(L=300)
    scale = 1 / math.sqrt(wl.d)
    for topk, m in ((300, 0), (200, 100), (0, 300), (250, 80)):
        out, info = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                               hs["seq_lens"], [topk], [m], [0], hs["pair_begin"],
                               hs["pair_count"])
        assert info[(0, 0)]["dense"]
        assert np.allclose(out[0], sdpa_f64(qg, K, V, scale), rtol=0, atol=1e-12)


def test_sample_budget_zero_is_exact_topk():
    wl, hs, qg, K, V = tiny_unit(L=1000)
    scale = 1 / math.sqrt(wl.d)
    out, info = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                           hs["seq_lens"], [64], [0], [0], hs["pair_begin"], hs["pair_count"])
    s32 = info[(0, 0)]["scores"].astype(np.float32)
    brute = sorted(range(1000), key=lambda j: (-float(s32[j]), j))[:64]
    assert list(info[(0, 0)]["S"]) == sorted(brute)
    assert info[(0, 0)]["R"].size == 0
    mask = np.zeros(1000, bool)
    mask[brute] = True
    assert np.allclose(out[0], sdpa_f64(qg, K, V, scale, mask), rtol=0, atol=1e-12)


def uniform_case_z(nseeds=2000):
    """topk = 0 and constant scores: max |z| of per-token hit counts and of
    the mean sample size against textbook uniform Poisson sampling, pi = m/L."""
    L, m = 512, 40
    st = orc.tail_stratum(np.zeros(L, np.float32), 0, m)
    assert st["W"] == np.float32(L)
    assert np.all(st["pi"] == np.float32(m / L))
    hits = np.zeros(L)
    sizes = []
    for seed in range(nseeds):
        R, pi = orc.sample_tail(st, m, seed, 0, 0)
        hits[R] += 1
        sizes.append(R.size)
    p = m / L
    z_size = abs(np.mean(sizes) - m) / math.sqrt(L * p * (1 - p) / nseeds)
    z = (hits - nseeds * p) / math.sqrt(nseeds * p * (1 - p))
    return max(z_size, np.abs(z).max())


def test_uniform_sampling_special_case():
    assert uniform_case_z() < 5.0


def test_budget_equal_to_length_is_dense():
    wl, hs, qg, K, V = tiny_unit(L=200)
    out, info = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                           hs["seq_lens"], [100], [100], [3], hs["pair_begin"], hs["pair_count"])
    assert info[(0, 0)]["dense"] and info[(0, 0)]["S"].size == 200


def test_inclusion_probabilities_sum_to_budget():
    wl, hs, qg, K, V = tiny_unit(L=4096)
    s32 = orc.approx_scores(qg, K, hs["pair_begin"], hs["pair_count"], 1 / 8.0).astype(np.float32)
    st = orc.tail_stratum(s32, 64, 32)
    assert st["pi"].max() <= 1.0 and st["pi"].min() > 0
    assert st["pi"].astype(np.float64).sum() <= 32 * (1 + 1e-5)
    if st["pi"].max() < 1.0:
        assert abs(st["pi"].astype(np.float64).sum() - 32) < 1e-3


def test_injected_normaliser_is_used():
    s32 = np.random.default_rng(1).standard_normal(400).astype(np.float32)
    st = orc.tail_stratum(s32, 10, 20, W_in=np.float32(123.5))
    assert st["W"] == np.float32(123.5)
    assert np.array_equal(st["pi"], np.minimum(np.float32(1), st["mw"] / np.float32(123.5)))


# ---------------------------------------------------------------- unbiasedness

def enumeration_error(q, K, V, topk, m, scale):
    """max relative error of E[N_hat], E[D_hat] computed over every outcome."""
    s32 = orc.approx_scores(q, K, 0, q.shape[1] // 2, scale).astype(np.float32)
    st = orc.tail_stratum(s32, topk, m)
    T, pi = st["T"], st["pi"].astype(np.float64)
    shift = np.zeros(q.shape[0])
    EN = np.zeros((q.shape[0], K.shape[1]))
    ED = np.zeros(q.shape[0])
    Ptot = 0.0
    for mask in range(1 << T.size):
        x = np.array([(mask >> i) & 1 for i in range(T.size)], bool)
        P = float(np.prod(np.where(x, pi, 1 - pi)))
        if P == 0.0:
            continue
        N, D = orc.ht_terms(q, K, V, st["S"], T[x], st["pi"][x], scale, shift)
        EN += P * N
        ED += P * D
        Ptot += P
    Nt, Dt = true_terms(q, K, V, scale, shift)
    return max(np.abs(EN - Nt).max() / np.abs(Nt).max(), np.abs(ED - Dt).max() / Dt.max(),
               abs(Ptot - 1.0))


def test_estimator_unbiased_by_enumeration():
    rng = np.random.default_rng(11)
    G, d, L = 2, 8, 18
    q = rng.standard_normal((G, d))
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d))
    assert enumeration_error(q, K, V, topk=4, m=5, scale=0.5) < 1e-12  # |T| = 14
    # no deterministic stratum at all: pure sampling, |T| = 13
    assert enumeration_error(q[:, :], K[:13], V[:13], topk=0, m=3, scale=0.3) < 1e-12
    # a budget large enough to cap some pi at 1
    assert enumeration_error(q, K[:14], V[:14], topk=2, m=9, scale=2.0) < 1e-12


def test_estimator_unbiased_monte_carlo():
    """10^4 seeds on the tiny config: every component of E[N_hat], E[D_hat]
    lies within 4.5 standard errors of the truth (HT variance)."""
    wl, hs, qg, K, V = tiny_unit(L=4096)
    scale = 1 / math.sqrt(wl.d)
    s32 = orc.approx_scores(qg, K, hs["pair_begin"], hs["pair_count"], scale).astype(np.float32)
    st = orc.tail_stratum(s32, 64, 32)
    logits = scale * (qg @ K.T)
    shift = logits.max(axis=1)
    Nt, Dt = true_terms(qg, K, V, scale, shift)
    n = 10000
    sumN = np.zeros_like(Nt)
    sumD = np.zeros_like(Dt)
    sizes = np.zeros(n)
    for seed in range(n):
        R, pi_R = orc.sample_tail(st, 32, seed, 0, 0)
        N, D = orc.ht_terms(qg, K, V, st["S"], R, pi_R, scale, shift)
        sumN += N
        sumD += D
        sizes[seed] = R.size
    T, pi = st["T"], st["pi"].astype(np.float64)
    e = np.exp(logits[:, T] - shift[:, None])                     # [G, |T|]
    varN = ((1 - pi) / pi)[None, :, None] * (e[:, :, None] * V[T][None]) ** 2
    varD = ((1 - pi) / pi)[None, :] * e ** 2
    seN = np.sqrt(varN.sum(1) / n)
    seD = np.sqrt(varD.sum(1) / n)
    zN = np.abs(sumN / n - Nt) / np.maximum(seN, 1e-300)
    zD = np.abs(sumD / n - Dt) / np.maximum(seD, 1e-300)
    assert zN.max() < 4.5 and zD.max() < 4.5, (zN.max(), zD.max())
    se_size = math.sqrt((pi * (1 - pi)).sum() / n)
    assert abs(sizes.mean() - pi.sum()) < 4.5 * se_size


# ---------------------------------------------------------------- workload recipe

def test_budget_rule_reproduces_configs():
    assert synth.budget_rule(32768) == (328, 327)
    assert synth.budget_rule(131072) == (1311, 1310)
    assert synth.budget_rule(1048576) == (10486, 10486)


def test_rope_depends_on_relative_position():
    d, theta = 64, 1e4
    rng = np.random.default_rng(2)
    a = torch.from_numpy(rng.standard_normal((1, 1, d)).astype(np.float32))
    b = torch.from_numpy(rng.standard_normal((1, 1, d)).astype(np.float32))

    def rot(x, pos):
        c, s = synth.rope_tables(torch.tensor([pos]), d, theta)
        return synth.apply_rope(x, c, s)
    d1 = float((rot(a, 100) * rot(b, 40)).sum())
    d2 = float((rot(a, 1060) * rot(b, 1000)).sum())
    assert abs(d1 - d2) < 1e-3
    assert abs(float(rot(a, 77).norm()) - float(a.norm())) < 1e-4


def test_planted_keys_score_high():
    wl, hs, qg, K, V = tiny_unit(L=4096)
    full = (qg.mean(0) @ K.T)
    z = (full - full.mean()) / full.std()
    assert (z > 4.5).sum() >= 8


# ---------------------------------------------------------------- planted mistakes

def test_pins_catch_planted_mistakes(monkeypatch, tmp_path):
    """Each mutation below is a plausible slip; some pin above must fail."""
    # 1. a wrong Taylor coefficient in sexp -> ulp pin fails
    bad = list(orc._TAYLOR)
    bad[3] = np.float32(1 / 5.0)
    monkeypatch.setattr(orc, "_TAYLOR", bad)
    assert check_sexp_ulp() > 2.0
    monkeypatch.undo()
    # 2. Philox key words swapped -> rocRAND pin fails
    exe = _build_rocrand_helper(str(tmp_path))
    real = orc.philox4x32_10
    monkeypatch.setattr(orc, "philox4x32_10", lambda c0, c1, c2, c3, k0, k1: real(c0, c1, c2, c3, k1, k0))
    assert oracle_words(PHILOX_QUERIES) != rocrand_words(exe, PHILOX_QUERIES)
    monkeypatch.undo()
    # 3. HT weight pi instead of 1/pi -> enumeration pin fails
    rng = np.random.default_rng(11)
    q, K, V = rng.standard_normal((2, 8)), rng.standard_normal((18, 8)), rng.standard_normal((18, 8))
    real_terms = orc.ht_terms

    def ht_wrong(q_, K_, V_, S, R, pi_R, scale, shift):
        return real_terms(q_, K_, V_, S, R, 1.0 / np.asarray(pi_R, np.float64), scale, shift)
    monkeypatch.setattr(orc, "ht_terms", ht_wrong)
    assert enumeration_error(q, K, V, topk=4, m=5, scale=0.5) > 1e-3
    monkeypatch.undo()
    # 4. inclusion decision flipped (include iff u*W >= m*w) -> uniform pin fails
    def sample_flipped(strata, m, seed, b, h):
        T = strata["T"]
        u = orc.uniforms(seed, b, h, T)
        keep = np.multiply(u, strata["W"], dtype=np.float32) >= strata["mw"]
        return T[keep], strata["pi"][keep]
    monkeypatch.setattr(orc, "sample_tail", sample_flipped)
    assert uniform_case_z(200) > 5.0
    monkeypatch.undo()
    # 5. pair range off by one pair -> score pin fails
    real_scores = orc.approx_scores
    monkeypatch.setattr(orc, "approx_scores",
                        lambda q_, K_, pb, pc, sc: real_scores(q_, K_, pb + 1, pc - 1, sc))
    assert scores_error() > 1e-3
    monkeypatch.undo()
    # 6. ties broken towards the higher index -> brute-force ranking pin fails
    real_topk = orc.topk_indices

    def topk_high(s32, k):
        key = orc.order_key(s32)
        idx = np.arange(key.size)
        return np.sort(np.lexsort((-idx, ~key))[:k])
    s = np.array([1, 2, 2, 2, 0], np.float32)
    assert list(real_topk(s, 2)) == [1, 2] and list(topk_high(s, 2)) != [1, 2]
