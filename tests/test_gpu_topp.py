"""GPU parity of the top-p deterministic stratum, through the C ABI.

"Stratified Sparse Attention speeds up decoding 2.96x at 1M context",
"Where sparse attention loses quality": top-p is a deterministic option.  The
library ends the stratum at min(top-k, top-p prefix); mass is counted in
integer units, so the prefix is bit-exact against the oracle given the same
float32 scores.  Sampling decisions are compared with the oracle's
normaliser injected (its float64 sum order differs from the kernels').
"""


import numpy as np
import pytest
import torch

from long_context_sparse_approx_amd import ssa, synth
from oracle import ssa_oracle as orc

from gpu_helpers import (default_scale, gpu_sets, group, oracle_scores, say, selection_arrays,
                         unit_rows, vmax_unit)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def select_params(B, Hkv, Lmax):
    return ssa.make_params(batch=B, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=128,
                           max_blocks_per_seq=(Lmax + 15) // 16, num_blocks=1, max_seq_len=Lmax)


def check_select(s32, lens, topk, top_p, m, seeds, label, inject=True):
    """Selection parity for score arrays s32 [B, Hkv, Lmax] (float32).

    Returns {(b, h): oracle selection}."""
    B, Hkv, Lmax = s32.shape
    p = select_params(B, Hkv, Lmax)
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device=DEV)
    tp = torch.tensor(np.asarray(top_p, np.float32), device=DEV)
    seed_t = torch.tensor([int(s) for s in seeds], dtype=torch.int64, device=DEV)
    sels, w_in = {}, np.zeros((B, Hkv), np.float32)
    for b in range(B):
        for h in range(Hkv):
            sel = orc.select_unit(s32[b, h, :lens[b]], int(topk[b]), int(m[b]), int(seeds[b]),
                                  b, h, top_p=np.float32(top_p[b]))
            sels[(b, h)] = sel
            w_in[b, h] = sel["W"]
    si, sl, sn, nm = ssa.select(p, torch.from_numpy(s32).to(DEV), i32(lens), i32(topk), i32(m),
                                seed_t, w_in=torch.from_numpy(w_in).to(DEV) if inject else None,
                                top_p=tp)
    torch.cuda.synchronize()
    si, sl, sn, nm = (t.cpu().numpy() for t in (si, sl, sn, nm))
    nS = nR = 0
    for (b, h), sel in sels.items():
        S, R, lR = gpu_sets(si, sl, sn, b, h)
        assert np.array_equal(S, sel["S"]), (
            f"{label}: stratum differs at {(b, h)}: gpu {S.size} oracle {sel['S'].size}")
        if lens[b] > 0:
            assert nm[b, h, 0] == sel["M"]
        if inject:
            assert np.array_equal(R, sel["R"]), f"{label}: sample differs at {(b, h)}"
            assert np.allclose(lR, -np.log(sel["pi_R"].astype(np.float64)), rtol=1e-5, atol=1e-5)
        elif not sel["dense"] and sel["W"] > 0:
            assert abs(float(nm[b, h, 1]) - float(sel["W"])) <= 1e-5 * float(sel["W"])
        nS += S.size
        nR += R.size
    say(f"[topp] {label}: selection bit-exact (|S|={nS}, |R|={nR})")
    return sels


def model_scores(wl):
    hs = wl.host()
    ref = oracle_scores(wl, hs, default_scale(wl.d))
    s32 = np.zeros((wl.B, wl.Hkv, wl.max_seq_len), np.float32)
    for (b, h), s64 in ref.items():
        s32[b, h, :s64.size] = s64.astype(np.float32)
    return s32


RAGGED = dict(B=2, Hq=8, Hkv=2, d=128, L=[9000, 4097], theta=1e6, kdist="normal", planted=16,
              pair_count=32, topk=0, m=40, seeds=[5, 6], data_seed=11)


def test_mass_bound_on_model_scores():
    wl = synth.make_workload(dict(RAGGED), "cpu")
    s32 = model_scores(wl)
    L = wl.lens
    for tp in ([0.2, 0.05], [0.5, 0.01], [0.9, 0.3]):
        check_select(s32, L, L, tp, [40, 40], [5, 6], f"mass p={tp}")
        check_select(s32, L, L, tp, [40, 40], [5, 6], f"mass p={tp} own W", inject=False)


def test_count_and_mass_bounds_meet():
    """topk around the top-p count n_p: the count bound binds (n_p - 1), both
    bounds end on the same token (n_p), the mass bound binds (n_p + 1)."""
    wl = synth.make_workload("tiny", "cpu")
    s = model_scores(wl)[0, 0]
    for p in (0.05, 0.3, 0.77):
        n = orc.topp_count(s, np.float32(p))
        s32 = np.stack([s, s, s, s])[:, None, :]
        check_select(s32, [s.size] * 4, [n - 1, n, n + 1, 3], [p] * 4, [32] * 4, [1, 2, 3, 4],
                     f"meet p={p} n_p={n}")


def test_ties_on_the_last_key():
    """Coarse scores (many equal keys, across chunks): the mass bound takes
    ceil(remaining units / units per token) of the tied tokens, in index order."""
    rng = np.random.default_rng(31)
    L = 13000
    s = (np.round(rng.standard_normal((2, 1, L)) * 2) / 2).astype(np.float32)
    for tp in ([0.1, 0.37], [0.8, 0.55], [0.013, 0.999]):
        check_select(s, [L, L - 1234], [L, L], tp, [50, 50], [7, 8], f"ties p={tp}")


def test_uniform_scores_take_the_lowest_positions():
    L = 20000
    s = np.full((1, 1, L), np.float32(0.25))
    sels = check_select(s, [L], [L], [0.25], [100], [9], "uniform p=0.25")  # 0.25 is exact
    assert np.array_equal(sels[(0, 0)]["S"], np.arange(5000))


def test_edges():
    rng = np.random.default_rng(41)
    Lmax = 9000
    s = (rng.standard_normal((7, 1, Lmax)) * 1.5).astype(np.float32)
    lens = [9000, 9000, 9000, 9000, 1, 0, 5000]
    # p = 0 (empty stratum), NaN (as 0), above 1 (as 1), a tiny p (one token),
    # L = 1, L = 0, p = 1 with no budget (every token with mass)
    tp = [0.0, float("nan"), 3.0, 1e-30, 0.5, 0.5, 1.0]
    topk = [Lmax] * 7
    m = [30, 30, 30, 30, 30, 30, 0]
    check_select(s, lens, topk, tp, m, list(range(7)), "edges")


def test_dense_rule_on_the_resolved_stratum():
    """k + m >= L makes the unit dense only once k is known."""
    wl = synth.make_workload("tiny", "cpu")
    s = model_scores(wl)[0, 0]
    n = orc.topp_count(s, np.float32(0.4))
    L = s.size
    s32 = np.stack([s, s])[:, None, :]
    sels = check_select(s32, [L, L], [L, L], [0.4, 0.4], [L - n, L - n - 1], [1, 2], "late dense")
    assert sels[(0, 0)]["dense"] and not sels[(1, 0)]["dense"]


def test_end_to_end_top_p():
    wl = synth.make_workload(dict(RAGGED), DEV)
    wl.topk = torch.tensor(wl.lens, dtype=torch.int32, device=DEV)
    top_p = np.array([0.2, 0.05], np.float32)
    p = ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                       pair_begin=wl.pair_begin, pair_count=wl.pair_count)
    tp = torch.from_numpy(top_p).to(DEV)
    out = ssa.decode(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.topk,
                     wl.sample_budget, wl.seed, top_p=tp).clone()
    out2 = ssa.decode(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.topk,
                      wl.sample_budget, wl.seed, top_p=tp)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    hs = wl.host()
    ref, info = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                           hs["seq_lens"], hs["topk"], hs["sample_budget"], hs["seed"],
                           wl.pair_begin, wl.pair_count, default_scale(wl.d), top_p=top_p)
    got = out.double().cpu().numpy()
    G = wl.Hq // wl.Hkv
    for (b, h), inf in info.items():
        _, V = unit_rows(hs, b, h, wl.lens[b])
        err = float(np.abs(got[b, h * G:(h + 1) * G] - ref[b, h * G:(h + 1) * G]).max())
        bound = 2e-3 * vmax_unit(V)
        assert err <= bound, f"top-p e2e out of tolerance at {(b, h)}: {err} > {bound}"
        say(f"[topp] e2e unit {(b, h)} |S|={inf['S'].size} err/bound {err / bound:.3g}")
    # attention on the oracle's top-p selection
    sels = {k: v for k, v in info.items()}
    ai, al, ac = selection_arrays(p, sels, DEV)
    att = ssa.attend(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, ai, al, ac)
    torch.cuda.synchronize()
    att = att.double().cpu().numpy()
    for (b, h), inf in info.items():
        K, V = unit_rows(hs, b, h, wl.lens[b])
        o = orc.attend_unit(group(hs, b, h, G), K, V, inf["S"], inf["R"], inf["pi_R"],
                            default_scale(wl.d))
        assert float(np.abs(att[b, h * G:(h + 1) * G] - o).max()) <= 2e-3 * vmax_unit(V)
