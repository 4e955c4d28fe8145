"""GPU parity of early stopping over the deterministic stratum, through the
C ABI.

"S2O: Early Stopping for Sparse Attention via Online Permutation",
methodology part 2: the stratum is visited in 64-token blocks of its order and
the visit ends after the first block whose gain is below tau times the mass
visited so far.  Gains are integer mass units, so the cut is bit-exact against
the oracle given the same float32 scores; sampling is compared with the
oracle's normaliser injected.
"""

import math

import numpy as np
import pytest
import torch

from long_context_sparse_approx_amd import ssa, synth
from oracle import ssa_oracle as orc

from gpu_helpers import default_scale, gpu_sets, oracle_scores, say, unit_rows, vmax_unit

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def check_select(s32, lens, topk, m, seeds, tau, label, top_p=None, T=1, g=1, Hkv=None):
    """Stratum cut and sample bit-exact for scores s32 [B, units per sequence, Lmax]."""
    B, UH, Lmax = s32.shape
    Hkv = Hkv or UH
    p = ssa.make_params(batch=B, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=128,
                        max_blocks_per_seq=(Lmax + 15) // 16, num_blocks=1, max_seq_len=Lmax,
                        num_queries=T, query_group=g, early_stop=float(tau))
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device=DEV)
    seed_t = torch.tensor([int(x) for x in seeds], dtype=torch.int64, device=DEV)
    tp = None if top_p is None else torch.tensor(np.asarray(top_p, np.float32), device=DEV)
    sels, w_in = {}, np.zeros((B, UH), np.float32)
    ng = UH // Hkv
    for b in range(B):
        for r in range(UH):
            c, h = divmod(r, Hkv)
            span = orc.group_span(lens[b], T, min(g, T), c)
            sel = orc.select_unit(s32[b, r, :span], int(topk[b]), int(m[b]), int(seeds[b]), b, h,
                                  top_p=None if top_p is None else np.float32(top_p[b]), grp=c,
                                  stop_tau=np.float32(tau))
            sels[(b, r)] = sel
            w_in[b, r] = sel["W"]
    si, sl, sn, _ = ssa.select(p, torch.from_numpy(s32).to(DEV), i32(lens), i32(topk), i32(m),
                               seed_t, w_in=torch.from_numpy(w_in).to(DEV), top_p=tp)
    torch.cuda.synchronize()
    si, sl, sn = (t.cpu().numpy() for t in (si, sl, sn))
    cut = 0
    for (b, r), sel in sels.items():
        S, R, _ = gpu_sets(si, sl, sn, b, r)
        assert np.array_equal(S, sel["S"]), (
            f"{label}: stratum differs at {(b, r)}: gpu {S.size} oracle {sel['S'].size} "
            f"(uncut {sel['S_full'].size})")
        assert np.array_equal(R, sel["R"]), f"{label}: sample differs at {(b, r)}"
        cut += sel["S_full"].size - sel["S"].size
    say(f"[stop] {label}: stratum cut and sample bit-exact ({cut} tokens cut)")
    return sels, cut


def model_scores(wl):
    hs = wl.host()
    ref = oracle_scores(wl, hs, default_scale(wl.d))
    s32 = np.zeros((wl.B, wl.Hkv, wl.max_seq_len), np.float32)
    for (b, h), s64 in ref.items():
        s32[b, h, :s64.size] = s64.astype(np.float32)
    return s32


RAGGED = dict(B=2, Hq=8, Hkv=2, d=128, L=[9000, 4097], theta=1e6, kdist="normal", planted=16,
              pair_count=32, topk=700, m=40, seeds=[5, 6], data_seed=11)


def test_cut_on_model_scores():
    wl = synth.make_workload(dict(RAGGED), "cpu")
    s32 = model_scores(wl)
    total = 0
    for tau in (0.02, 0.1, 0.3, 1.0):
        _, cut = check_select(s32, wl.lens, [700, 700], [40, 40], [5, 6], tau, f"tau={tau}")
        total += cut
    assert total > 0


def test_cut_among_equal_keys():
    """Coarse scores: the cut falls inside runs of equal keys, ordered by position."""
    rng = np.random.default_rng(7)
    L = 12000
    s = (np.round(rng.standard_normal((2, 1, L)) * 3) / 3).astype(np.float32)
    for tau in (0.05, 0.2):
        check_select(s, [L, L - 777], [3000, 5000], [60, 60], [1, 2], tau, f"ties tau={tau}")


def test_stratum_limits():
    """At most 64 tokens: nothing to cut; more than 16384: visited whole; dense."""
    rng = np.random.default_rng(8)
    L = 40000
    s = (rng.standard_normal((3, 1, L)) * 2).astype(np.float32)
    sels, cut = check_select(s, [L, L, 600], [60, 16385, 500], [30, 30, 300], [1, 2, 3], 0.5,
                             "limits")
    assert cut == 0


def test_cut_with_top_p_and_groups():
    wl = synth.make_workload(dict(RAGGED), "cpu")
    s32 = model_scores(wl)
    check_select(s32, wl.lens, [4000, 4000], [40, 40], [5, 6], 0.05, "top-p", top_p=[0.5, 0.3])
    # two query groups per sequence: rows are (group, head)
    rng = np.random.default_rng(9)
    s = (rng.standard_normal((2, 4, 9000)) * 1.5).astype(np.float32)
    check_select(s, [9000, 7000], [900, 900], [50, 50], [3, 4], 0.1, "groups", T=4, g=2, Hkv=2)


def test_end_to_end_with_early_stopping():
    cfg = dict(RAGGED)
    wl = synth.make_workload(cfg, DEV)
    tau = 0.05
    p = ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                       pair_begin=wl.pair_begin, pair_count=wl.pair_count, early_stop=tau)
    out = ssa.decode(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.topk,
                     wl.sample_budget, wl.seed).clone()
    out2 = ssa.decode(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.topk,
                      wl.sample_budget, wl.seed)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    hs = wl.host()
    ref, info = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                           hs["seq_lens"], hs["topk"], hs["sample_budget"], hs["seed"],
                           wl.pair_begin, wl.pair_count, default_scale(wl.d),
                           stop_tau=np.float32(tau))
    got = out.double().cpu().numpy()
    G = wl.Hq // wl.Hkv
    for (b, h), inf in info.items():
        _, V = unit_rows(hs, b, h, wl.lens[b])
        err = float(np.abs(got[b, h * G:(h + 1) * G] - ref[b, h * G:(h + 1) * G]).max())
        assert err <= 2e-3 * vmax_unit(V), f"early-stop e2e out of tolerance at {(b, h)}"
        say(f"[stop] e2e unit {(b, h)}: |S| {inf['S'].size} of {inf['S_full'].size}")


def test_cut_inside_the_threshold_ties():
    """The stop falls among the tokens tied on the stratum's last key, whose
    order is by position across chunks: 100 high scores, then 5000 equal ones
    spread over several chunks; top-k 3000 ends the stratum inside the tie run
    and the stop lands a few blocks later, still inside it."""
    rng = np.random.default_rng(10)
    L = 20000
    s = (rng.standard_normal((2, 1, L)) * 0.3 - 2.0).astype(np.float32)
    for b in range(2):
        pos = rng.permutation(L)
        s[b, 0, pos[:100]] = np.float32(5.0)
        s[b, 0, pos[100:5100]] = np.float32(1.0)
    sels, cut = check_select(s, [L, L - 3001], [3000, 2500], [40, 40], [3, 4], 0.05, "tie cut")
    for sel in sels.values():
        S, full = sel["S"], sel["S_full"]
        assert 100 < S.size < full.size, (S.size, full.size)  # the cut is inside the ties
    assert cut > 0
