"""Pins of the oracle's refine mode of query groups (no GPU).

"PIVOT slashes sparse-attention indexer cost", "The two observations behind
PIVOT" (the proxy's candidate list is refined for each member of the group)
and "Two operating modes" (refine keeps the dense indexer's accuracy).  The
group's proxy selection runs with a candidate list of r * k tokens; each
member ranks the candidates inside its span by its own score, keeps k of
them, and samples the rest of the group's span with the proxy's weights and
its own normaliser.  The pins check the member's score against float64
logits, reductions to plain decode and to the reuse mode, a member-specific
stratum built by hand, brute-force ranking with ties, the normaliser against
a brute-force tail sum, exact unbiasedness by enumeration, and planted slips.
"""

import itertools
import math

import numpy as np
import pytest

from long_context_sparse_approx_amd import synth
from oracle import ssa_oracle as orc

from test_oracle_pins import sdpa_f64


def case(L, T, data_seed=3, **kw):
    wl = synth.make_workload("tiny", "cpu", L=L, num_queries=T, data_seed=data_seed, **kw)
    return wl, wl.host()


def run(hs, g, topk, m, r, seeds=(0,)):
    return orc.decode_multi(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                            hs["seq_lens"], [topk], [m], list(seeds), hs["pair_begin"],
                            hs["pair_count"], g, refine=r)


def rows(hs, L):
    return (orc.gather_rows(hs["k_cache"], hs["block_table"][0], 0, L),
            orc.gather_rows(hs["v_cache"], hs["block_table"][0], 0, L))


def member_score_error():
    """The member's own score is its G heads' mean partial logit over the
    scored pairs: within the float32 summation bound of float64."""
    wl, hs = case(700, 3)
    K, _ = rows(hs, 700)
    scale = 1 / math.sqrt(wl.d)
    pb, pc = hs["pair_begin"], hs["pair_count"]
    dims = np.arange(2 * pb, 2 * (pb + pc))
    worst = 0.0
    for t in range(3):
        qg = hs["q"][0, t]
        ref = orc.approx_scores(qg, K, pb, pc, scale)
        G = qg.shape[0]
        bound = (2 * pc + G + 2) * 2.0 ** -24 * scale / G * (np.abs(qg[:, dims]) @ np.abs(K[:, dims]).T).sum(0)
        got = orc.member_scores(qg, K, pb, pc, scale).astype(np.float64)
        worst = max(worst, float((np.abs(got - ref) / (bound + 1e-300)).max()))
    return worst


def test_member_score_is_its_mean_partial_logit():
    assert member_score_error() <= 1.0


def test_refine_r1_single_query_is_plain_decode():
    """One query, r = 1: the candidate list is the stratum itself, so the
    member keeps it and its tail normaliser is the stratum's complement's."""
    wl = synth.make_workload("tiny", "cpu", L=900)
    hs = wl.host()
    ref, info = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                           hs["seq_lens"], [40], [30], [5], hs["pair_begin"], hs["pair_count"])
    out, minfo = orc.decode_multi(hs["q"][:, None], hs["k_cache"], hs["v_cache"],
                                  hs["block_table"], hs["seq_lens"], [40], [30], [5],
                                  hs["pair_begin"], hs["pair_count"], 1, refine=1)
    assert np.array_equal(out[:, 0], ref)
    mem = minfo[(0, 0, 0)]["members"][0]
    assert np.array_equal(mem["S"], info[(0, 0)]["S"]) and np.array_equal(mem["R"], info[(0, 0)]["R"])


def test_refine_r1_last_member_is_reuse():
    """r = 1: the group's last member (whose span is the group's) keeps the
    whole candidate list and draws exactly the reuse mode's sample."""
    wl, hs = case(800, 4)
    _, reuse = orc.decode_multi(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                                hs["seq_lens"], [40], [30], [7], hs["pair_begin"],
                                hs["pair_count"], 4)
    _, ref = run(hs, 4, 40, 30, 1, seeds=(7,))
    last = ref[(0, 0, 0)]["members"][3]
    assert np.array_equal(last["S"], reuse[(0, 0, 0)]["S"])
    assert np.array_equal(last["R"], reuse[(0, 0, 0)]["R"])
    for t in range(3):  # earlier members keep the candidates inside their spans
        Lt = orc.member_span(800, 4, t)
        C = reuse[(0, 0, 0)]["S"]
        assert np.array_equal(ref[(0, 0, 0)]["members"][t]["S"], C[C < Lt])


def full_list_error():
    """r k >= the span, no sampling: each member reads the brute-force top-k
    of its own scores over its span (ties to the lower index); output =
    float64 SDPA on that set.  Duplicated keys force ties."""
    wl, hs = case(640, 3, data_seed=5)
    bt = hs["block_table"][0]
    for j in range(100, 160):  # tokens 100..159 copy token 40's key (equal own scores)
        hs["k_cache"][bt[j // 16], 0, j % 16] = hs["k_cache"][bt[40 // 16], 0, 40 % 16]
    P, T, topk = 640, 3, 60
    out, info = run(hs, 3, topk, 0, 20)
    scale = 1 / math.sqrt(wl.d)
    worst = 0.0
    for t in range(T):
        Lt = P - T + t + 1
        K, V = rows(hs, Lt)
        qg = hs["q"][0, t]
        s32 = orc.approx_scores(qg, K, hs["pair_begin"], hs["pair_count"], scale).astype(np.float32)
        brute = sorted(range(Lt), key=lambda j: (-float(s32[j]), j))[:topk]
        mask = np.zeros(Lt, bool)
        mask[brute] = True
        if not np.array_equal(info[(0, 0, 0)]["members"][t]["S"], np.sort(brute)):
            return float("inf")
        worst = max(worst, float(np.abs(out[0, t] - sdpa_f64(qg, K, V, scale, mask)).max()))
    return worst


def test_full_candidate_list_is_per_member_topk():
    assert full_list_error() < 1e-12


def own_strata_error():
    """Two members with different interests: 30 keys planted along member
    0's query and 30 along member 1's (orthogonalised), in one group.  The
    proxy (their mean) ranks all 60 on top, so with r = 4 both sets are
    candidates, and each member keeps exactly its own 30."""
    wl, hs = case(1000, 2, data_seed=9)
    pb, pc = hs["pair_begin"], hs["pair_count"]
    dims = np.arange(2 * pb, 2 * (pb + pc))
    q0 = hs["q"][0, 0].mean(0)[dims]
    q1 = hs["q"][0, 1].mean(0)[dims]
    q1 = q1 - (q1 @ q0) / (q0 @ q0) * q0
    u0, u1 = q0 / np.linalg.norm(q0), q1 / np.linalg.norm(q1)
    rng = np.random.default_rng(1)
    pos = rng.choice(990, 60, replace=False)
    bt = hs["block_table"][0]
    for i, j in enumerate(pos):
        row = np.zeros(wl.d)
        row[dims] = (u0 if i < 30 else u1) * 12.0
        hs["k_cache"][bt[j // 16], 0, j % 16] = np.asarray(row, np.float32).astype(np.float64)
    _, info = run(hs, 2, 30, 0, 4)
    mem = info[(0, 0, 0)]["members"]
    return (set(map(int, mem[0]["S"])) != set(map(int, pos[:30])) or
            set(map(int, mem[1]["S"])) != set(map(int, pos[30:])))


def test_members_take_their_own_strata():
    assert not own_strata_error()


def normaliser_error():
    """W_t = the proxy weight over the group's span minus the member's
    stratum, tail built by brute force (sets) and summed exactly."""
    wl, hs = case(900, 4, data_seed=11)
    _, info = run(hs, 4, 40, 50, 2, seeds=(3,))
    unit = info[(0, 0, 0)]
    s32 = unit["scores"].astype(np.float32)
    M = float(unit["M"])
    worst = 0.0
    for t, mem in unit["members"].items():
        tail = sorted(set(range(s32.size)) - set(map(int, mem["S"])))
        w = orc.sexp(np.asarray([float(s32[j]) - M for j in tail], np.float32))
        ref = math.fsum(float(x) for x in w)
        worst = max(worst, abs(float(mem["W"]) - ref) / ref)
    return worst


def test_member_normaliser_is_its_tail_mass():
    assert normaliser_error() < 1e-6


def enumeration_error():
    """Exact expectation over every sample outcome of each member: E[N_hat]
    = N and E[D_hat] = D over the member's span (Horvitz-Thompson with the
    member's inclusion probabilities)."""
    wl, hs = case(18, 2, data_seed=13)
    scale = 1 / math.sqrt(wl.d)
    _, info = run(hs, 2, 4, 3, 2, seeds=(1,))
    unit = info[(0, 0, 0)]
    s32 = unit["scores"].astype(np.float32)
    worst = 0.0
    for t, mem in unit["members"].items():
        Lt = orc.member_span(18, 2, t)
        K, V = rows(hs, Lt)
        qg = hs["q"][0, t]
        W = mem["W"]
        S = set(map(int, mem["S"]))
        T = [j for j in range(s32.size) if j not in S and j < Lt]
        w = orc.sexp(np.subtract(s32[T], unit["M"], dtype=np.float32))
        pi = np.minimum(np.float32(1), np.divide(np.multiply(np.float32(3), w, dtype=np.float32),
                                                 W, dtype=np.float32)).astype(np.float64)
        logits = scale * (qg @ K.T)
        shift = logits.max(axis=1)
        e = np.exp(logits - shift[:, None])  # [G, Lt]
        N = e @ V
        D = e.sum(1)
        EN, ED = np.zeros_like(N), np.zeros_like(D)
        Sl = sorted(S)
        for bits in itertools.product((0, 1), repeat=len(T)):
            p = np.prod([pi[i] if b else 1 - pi[i] for i, b in enumerate(bits)])
            if p == 0:
                continue
            R = [T[i] for i, b in enumerate(bits) if b]
            c = np.array([1.0] * len(Sl) + [1 / pi[T.index(j)] for j in R])
            A = Sl + R
            EN += p * (c[None, :] * e[:, A]) @ V[A]
            ED += p * (c[None, :] * e[:, A]).sum(1)
        worst = max(worst, float(np.abs(EN - N).max() / np.abs(N).max()),
                    float(np.abs(ED - D).max() / D.max()))
    return worst


def test_member_estimator_is_unbiased_by_enumeration():
    assert enumeration_error() < 1e-12


def sampling_frame_error(nseeds=400):
    """The realised samples over 400 seeds: every tail token inside the
    member's span with pi >= 0.2 -- the candidates the member dropped among
    them -- is drawn at least once, and the mean sample size matches the sum
    of the inclusion probabilities within 5 standard errors."""
    wl, hs = case(18, 2, data_seed=13)
    bad = 0
    counts, sizes = {}, {}
    for seed in range(nseeds):
        _, info = run(hs, 2, 4, 3, 2, seeds=(seed,))
        for t, mem in info[(0, 0, 0)]["members"].items():
            for j in mem["R"]:
                counts[(t, int(j))] = counts.get((t, int(j)), 0) + 1
            sizes.setdefault(t, []).append(len(mem["R"]))
    _, info = run(hs, 2, 4, 3, 2, seeds=(0,))
    unit = info[(0, 0, 0)]
    s32 = unit["scores"].astype(np.float32)
    for t, mem in unit["members"].items():
        Lt = orc.member_span(18, 2, t)
        S = set(map(int, mem["S"]))
        T = [j for j in range(s32.size) if j not in S and j < Lt]
        w = orc.sexp(np.subtract(s32[T], unit["M"], dtype=np.float32))
        pi = np.minimum(1.0, 3.0 * w.astype(np.float64) / float(mem["W"]))
        for j, p in zip(T, pi):
            bad += p >= 0.2 and counts.get((t, j), 0) == 0
        se = math.sqrt(float((pi * (1 - pi)).sum()) / nseeds) + 1e-9
        bad += abs(np.mean(sizes[t]) - pi.sum()) > 5 * se
    return bad


def test_member_samples_cover_its_tail():
    assert sampling_frame_error() == 0


def test_pins_catch_planted_refine_mistakes(monkeypatch):
    real = orc.refine_member
    # 1. the member keeps the proxy's top-k instead of ranking by its own score
    def proxy_rank(sel, s32, q, K, Lt, topk, m, *a, **k):
        out = real(sel, s32, q, K, Lt, topk, m, *a, **k)
        C = np.asarray(sel["S"])
        C = C[C < Lt]
        order = np.lexsort((C, ~orc.order_key(np.asarray(s32, np.float32)[C])))
        out["S"] = np.sort(C[order[:min(topk, C.size)]])
        return out
    monkeypatch.setattr(orc, "refine_member", proxy_rank)
    assert own_strata_error() or full_list_error() > 1e-12
    monkeypatch.undo()
    # 2. the member's normaliser is the group's (the candidates it drops left out)
    def group_w(sel, *a, **k):
        k = dict(k)
        k["W_in"] = sel["W"]
        return real(sel, *a, **k)
    monkeypatch.setattr(orc, "refine_member", group_w)
    assert normaliser_error() > 1e-6
    monkeypatch.undo()
    # 3. the dropped candidates are never sampled (frame = the span minus C)
    def no_dropped(sel, s32, q, K, Lt, topk, m, *a, **k):
        out = real(sel, s32, q, K, Lt, topk, m, *a, **k)
        keep = ~np.isin(out["R"], sel["S"])
        out["R"], out["pi_R"] = out["R"][keep], out["pi_R"][keep]
        return out
    monkeypatch.setattr(orc, "refine_member", no_dropped)
    assert sampling_frame_error(100) > 0
    monkeypatch.undo()
    # 4. one head left out of the member's score
    real_scores = orc.member_scores
    monkeypatch.setattr(orc, "member_scores",
                        lambda q, K, pb, pc, scale: real_scores(q[:-1], K, pb, pc, scale))
    assert member_score_error() > 1.0
    monkeypatch.undo()
