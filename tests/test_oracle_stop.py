"""Pins of the oracle's early stopping over the deterministic stratum (no GPU).

"S2O: Early Stopping for Sparse Attention via Online Permutation",
methodology part 2: blocks are visited in descending estimated importance and
the visit ends once a block's marginal gain in the online-softmax l falls
below a threshold relative to the accumulated score; part 3: the state
(m, l, acc) is carried through the visit.  The oracle visits the stratum's
64-token blocks in its order; each query row's gain is the block's exact
attention mass.  The pins check the exact logits against float64 dots,
closed forms, the same rule with float64 libm exp and real arithmetic, a row
that holds the visit back, a stratum far above any kernel capacity, the
attention result against torch's masked SDPA, and plant plausible slips.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from long_context_sparse_approx_amd import synth
from oracle import ssa_oracle as orc

from test_oracle_pins import sdpa_f64

TAUS = (np.float32(0.05), np.float32(0.1), np.float32(0.25), np.float32(0.3), np.float32(0.5),
        np.float32(1.0))


def bf16(x):
    """float32 values rounded to bf16 (round to nearest even), as float32."""
    b = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def keep(q_rows, K_ordered, tau, spans=None, scale=1.0):
    """Tokens kept for a stratum already in its order (positions 0..n-1)."""
    n = K_ordered.shape[0]
    spans = [n] * len(q_rows) if spans is None else spans
    lg = orc.stop_logits(q_rows, K_ordered, scale)
    vis = np.arange(n)[None, :] < np.asarray(spans)[:, None]
    return orc.stop_count(orc.stop_gains(lg, vis), n, tau)


def logit_keys(values, d=64):
    """Keys whose logit against q = e_0 (scale 1) is exactly each value."""
    K = np.zeros((len(values), d), np.float32)
    K[:, 0] = bf16(np.asarray(values, np.float32))
    return K


E0 = np.eye(1, 64, dtype=np.float32)


def logits_error():
    """The decision logits are float32 roundings of the exact dot: within the
    float32 summation bound of the float64 dot, on random bf16 data."""
    rng = np.random.default_rng(7)
    worst = 0.0
    for d in (64, 128):
        q = bf16(rng.standard_normal((4, d)).astype(np.float32))
        K = bf16(rng.standard_normal((500, d)).astype(np.float32))
        scale = 1 / math.sqrt(d)
        ref = (q.astype(np.float64) @ K.astype(np.float64).T) * scale
        bound = d * 2.0 ** -23 * (np.abs(q).astype(np.float64) @ np.abs(K).T.astype(np.float64))
        bound = bound * scale + np.abs(ref) * 2.0 ** -23
        got = orc.stop_logits(q, K, scale).astype(np.float64)
        worst = max(worst, float((np.abs(got - ref) / bound).max()))
    return worst


def test_logits_are_the_exact_dot():
    assert logits_error() <= 1.0


def order_error():
    """The specified summation order, on a worked case: a slice [1, 2^-24 x 7]
    summed in dim order stays 1 (each addend rounds away, to even), and the
    second slice's 2^-22 then joins it pairwise."""
    q = np.ones((1, 16), np.float32)
    k = np.zeros((1, 16), np.float32)
    k[0, 0] = 1.0
    k[0, 1:8] = 2.0 ** -24
    k[0, 8] = 2.0 ** -22
    got = float(orc.stop_logits(q, k, 1.0)[0, 0])
    return got != 1.0 + 2.0 ** -22


def test_specified_summation_order():
    assert not order_error()


def uniform_case_error():
    """Equal logits, whole blocks: every block has the same gain, so the visit
    stops after the first block i with (i + 1) tau > 1 (or never, if the
    stratum ends first)."""
    bad = 0
    for n in (64, 640, 1280, 5120):
        K = logit_keys(np.full(n, 0.7))
        for tau in TAUS:
            i = 0
            while not (i + 1) * Fraction(float(tau)) > 1:
                i += 1
            bad += keep(E0, K, tau) != min(64 * (i + 1), n)
    return bad


def test_uniform_logits_closed_form():
    assert uniform_case_error() == 0


def two_level_error():
    """a tokens at the top, the rest of the stratum 20 nats lower: with tau
    above the top tokens' share of the first mixed block the visit ends
    there, otherwise at the first all-low block."""
    bad = 0
    for a, tau, want in ((100, 0.5, 128), (100, 0.3, 192), (64, 0.5, 128), (64, 0.01, 128),
                         (200, 0.2, 256)):
        K = logit_keys(np.concatenate([np.full(a, 1.0), np.full(600, -19.0)]))
        bad += keep(E0, K, np.float32(tau)) != want
    return bad


def test_two_level_logits_closed_form():
    assert two_level_error() == 0


def libm_rule_error(nseeds=8):
    """The same rule with float64 exact logits, libm exp and real arithmetic
    stops at the same block on random strata (the decision logits round at
    2^-24 and the integer units at 2^-38 of the top token)."""
    bad = 0
    for seed in range(nseeds):
        rng = np.random.default_rng(200 + seed)
        n = int(rng.integers(100, 3000))
        R = int(rng.integers(1, 5))
        d = 64
        q = bf16(rng.standard_normal((R, d)).astype(np.float32))
        K = bf16(rng.standard_normal((n, d)).astype(np.float32) * rng.uniform(0.3, 2.0))
        scale = 1 / math.sqrt(d)
        ex = (q.astype(np.float64) @ K.astype(np.float64).T) * scale  # [R, n]
        w = np.exp(ex - ex.max(axis=1, keepdims=True))
        for tau in rng.uniform(0.01, 0.6, 6).astype(np.float32):
            acc, ref = np.zeros(R), n
            for i in range(-(-n // 64)):
                g = w[:, i * 64:(i + 1) * 64].sum(axis=1)
                acc += g
                if np.all(g < float(tau) * acc):
                    ref = min((i + 1) * 64, n)
                    break
            bad += keep(q, K, tau, scale=scale) != ref
    return bad


def test_rule_matches_real_valued_gains():
    assert libm_rule_error() == 0


def veto_error():
    """Two rows: row 0's logits fall by 2 nats per block (alone it stops
    after block 1: e^-2 < 0.25 (1 + e^-2)), row 1's are equal (alone it stops
    after block 4 at tau = 0.25: the first i with (i + 1) tau > 1).  The visit
    ends at the first block where both agree: 4."""
    n = 1024
    r0 = -2.0 * (np.arange(n) // 64)
    r1 = np.full(n, 0.5)
    K = np.zeros((n, 64), np.float32)
    K[:, 0] = bf16(r0.astype(np.float32))
    K[:, 1] = bf16(r1.astype(np.float32))
    q = np.zeros((2, 64), np.float32)
    q[0, 0] = 1.0
    q[1, 1] = 1.0
    tau = np.float32(0.25)
    alone0 = keep(q[:1], K, tau)
    alone1 = keep(q[1:], K, tau)
    both = keep(q, K, tau)
    return (alone0, alone1, both) != (128, 320, 320)


def test_every_row_must_agree():
    assert not veto_error()


def test_invisible_tokens_do_not_hold_back():
    """A row whose span excludes the stratum's tokens adds nothing and never
    holds the visit back; the other row decides."""
    n = 640
    K = logit_keys(np.full(n, 0.7))
    q = np.concatenate([E0, E0])
    tau = np.float32(0.5)
    assert keep(q, K, tau, spans=[n, 0]) == keep(E0, K, tau) == 192


def test_large_stratum_is_cut():
    """No capacity limit: a 20000-token stratum of equal logits stops after
    block 2 at tau = 0.5 (the first i with (i + 1) tau > 1) like a short one."""
    K = logit_keys(np.full(20000, 0.1))
    assert keep(E0, K, np.float32(0.5)) == 192


def test_no_stopping_cases():
    K = logit_keys(np.linspace(0, -8, 3000))
    for tau in (0.0, -1.0, float("nan")):
        assert keep(E0, K, np.float32(tau)) == 3000
    assert keep(E0, K, np.float32(3.0)) == keep(E0, K, np.float32(1.0))
    ks = [keep(E0, K, t) for t in np.linspace(0.01, 1, 30, dtype=np.float32)]
    assert ks == sorted(ks, reverse=True)
    assert orc.stop_count(np.zeros((1, 0), np.uint64), 0, np.float32(0.5)) == 0


def proxy_blind_error():
    """The gain is exact attention, not the proxy score: keys whose scored
    pairs are zero (equal proxy scores, so the stratum is in index order)
    while dim 0 makes the exact logits fall by 1 nat per 64-token block
    (scale 1/8).  At tau = 0.25 block 1 gains e^-1 / (1 + e^-1) = 0.27 of the
    mass so far and block 2 gains 0.09: the visit ends after block 2 (192
    tokens).  Equal proxy masses would run to block 4; unscaled logits
    (8 nats per block) would stop after block 1."""
    wl = synth.make_workload(dict(B=1, Hq=4, Hkv=1, d=64, L=[1024], theta=1e4,
                                  kdist="normal", planted=0, pair_count=16, topk=1024 - 40,
                                  m=0, seeds=[3], data_seed=9), "cpu")
    hs = wl.host()
    pb, pc = hs["pair_begin"], hs["pair_count"]
    kc = np.zeros_like(hs["k_cache"])
    bt = hs["block_table"][0]
    q = np.zeros_like(hs["q"])
    q[0, :, 0] = 1.0  # dim 0 is below the scored pairs
    for j in range(1024):
        kc[bt[j // 16], 0, j % 16, 0] = bf16(np.float32([-1.0 * (j // 64) * 8.0]))[0]
    _, info = orc.decode(q, kc, hs["v_cache"], hs["block_table"], hs["seq_lens"], [984], [0],
                         [3], pb, pc, stop_tau=np.float32(0.25))
    return info[(0, 0)]["S"].size != 192


def test_gain_is_exact_attention_not_the_proxy():
    assert not proxy_blind_error()


def stopped_attention_error():
    """No sampling: the output is float64 SDPA masked to the first k' tokens of
    the stratum's order, k' from the rule on brute-force ordered gains with
    float64 logits and libm exp."""
    wl = synth.make_workload("tiny", "cpu", L=3000, data_seed=4)
    hs = wl.host()
    scale = 1 / math.sqrt(wl.d)
    qg = hs["q"][0]
    K = orc.gather_rows(hs["k_cache"], hs["block_table"][0], 0, 3000)
    V = orc.gather_rows(hs["v_cache"], hs["block_table"][0], 0, 3000)
    worst = 0.0
    for tau in (np.float32(0.15), np.float32(0.3)):
        out, info = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                               hs["seq_lens"], [600], [0], [0], hs["pair_begin"],
                               hs["pair_count"], stop_tau=tau)
        s32 = orc.approx_scores(qg, K, hs["pair_begin"], hs["pair_count"], scale).astype(np.float32)
        order = sorted(range(3000), key=lambda j: (-float(s32[j]), j))[:600]
        ex = scale * (qg @ K[order].T)  # [G, 600]
        w = np.exp(ex - ex.max(axis=1, keepdims=True))
        acc, kk = np.zeros(qg.shape[0]), 600
        for i in range(0, 600, 64):
            g = w[:, i:i + 64].sum(axis=1)
            acc += g
            if np.all(g < float(tau) * acc):
                kk = min(i + 64, 600)
                break
        assert info[(0, 0)]["S"].size == kk < 600, (info[(0, 0)]["S"].size, kk)
        mask = np.zeros(3000, bool)
        mask[order[:kk]] = True
        worst = max(worst, float(np.abs(out[0] - sdpa_f64(qg, K, V, scale, mask)).max()))
    return worst


def test_stopped_stratum_attention_equals_masked_sdpa():
    assert stopped_attention_error() < 1e-12


def test_tail_sample_is_unchanged():
    wl = synth.make_workload("tiny", "cpu", L=3000, data_seed=5)
    hs = wl.host()
    args = (hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"], hs["seq_lens"], [500],
            [200], [3], hs["pair_begin"], hs["pair_count"])
    _, a = orc.decode(*args)
    _, b = orc.decode(*args, stop_tau=np.float32(0.2))
    assert np.array_equal(a[(0, 0)]["R"], b[(0, 0)]["R"]) and a[(0, 0)]["W"] == b[(0, 0)]["W"]
    assert b[(0, 0)]["S"].size < a[(0, 0)]["S"].size
    assert np.isin(b[(0, 0)]["S"], a[(0, 0)]["S"]).all()


def test_pins_catch_planted_stop_mistakes(monkeypatch):
    real_count, real_logits = orc.stop_count, orc.stop_logits
    # 1. 32-token blocks instead of 64
    monkeypatch.setattr(orc, "STOP_BLOCK", 32)
    assert uniform_case_error() > 0 or two_level_error() > 0
    monkeypatch.undo()
    # 2. stopping before the low-gain block instead of after it
    monkeypatch.setattr(orc, "stop_count",
                        lambda g, n, tau: (max(real_count(g, n, tau) - 64, 0)
                                           if real_count(g, n, tau) < n else n))
    assert two_level_error() > 0 and libm_rule_error(2) > 0
    monkeypatch.undo()
    # 3. gain compared with the accumulated mass before the block
    def before(g, n, tau):
        tau = Fraction(min(float(np.float32(tau)), 1.0))
        g = np.atleast_2d(g)
        acc = [0] * g.shape[0]
        for i in range(g.shape[1]):
            ok = all(acc[r] and int(g[r, i]) < tau * acc[r] for r in range(g.shape[0]))
            for r in range(g.shape[0]):
                acc[r] += int(g[r, i])
            if ok:
                return min((i + 1) * 64, n)
        return n
    monkeypatch.setattr(orc, "stop_count", before)
    assert uniform_case_error() > 0 or two_level_error() > 0
    monkeypatch.undo()
    # 4. only the first row decides
    monkeypatch.setattr(orc, "stop_count", lambda g, n, tau: real_count(np.atleast_2d(g)[:1], n, tau))
    assert veto_error()
    monkeypatch.undo()
    # 5. the logits without the softmax scale
    monkeypatch.setattr(orc, "stop_logits", lambda q, K, scale: real_logits(q, K, 1.0))
    assert logits_error() > 1.0 and proxy_blind_error()
    monkeypatch.undo()
    # 6. the slices summed pairwise inside (not in dim order)
    def pairwise(q, K, scale):
        p = np.asarray(q, np.float32)[:, None, :] * np.asarray(K, np.float32)[None, :, :]
        while p.shape[-1] > 1:
            p = np.add(p[..., 0::2], p[..., 1::2], dtype=np.float32)
        return np.multiply(p[..., 0], np.float32(scale), dtype=np.float32)
    monkeypatch.setattr(orc, "stop_logits", pairwise)
    assert order_error()
    monkeypatch.undo()
    # 7. the gain taken from the proxy score instead of the exact logits
    def proxy(q, K, scale):
        d = K.shape[1]
        pb, pc = d // 2 - d // 4, d // 4
        dims = np.arange(2 * pb, 2 * (pb + pc))
        qq = np.zeros_like(np.asarray(q, np.float32))
        qq[:, dims] = np.asarray(q, np.float32)[:, dims]
        return real_logits(qq, K, scale)
    monkeypatch.setattr(orc, "stop_logits", proxy)
    assert proxy_blind_error()
    monkeypatch.undo()
