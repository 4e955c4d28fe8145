"""GPU parity of the refine mode of query groups, through the C ABI.

"PIVOT slashes sparse-attention indexer cost", "The two observations behind
PIVOT" and "Two operating modes": the group is scored once through its proxy
query; its selection, with a candidate list of r * k tokens, is refined by
every member with its own score.  Member selections are compared bit-exact
with the oracle's, given the oracle's float32 group scores and the members'
normalisers; the library's own member normalisers within 1e-6 relative;
outputs within 2e-3 max|V|.
"""

import math

import numpy as np
import pytest
import torch

from long_context_sparse_approx_amd import ssa, synth
from oracle import ssa_oracle as orc

from gpu_helpers import default_scale, gpu_sets, say, unit_rows, vmax_unit

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def params(wl, g, r, **kw):
    return ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                          pair_begin=wl.pair_begin, pair_count=wl.pair_count, query_group=g,
                          refine=r, **kw)


def oracle_members(wl, g, r):
    """The oracle's group scores, group selections and member selections:
    (s32 [B, NG*Hkv, Lmax], members {(b, t, h): sel})."""
    hs = wl.host()
    q = hs["q"]
    T = q.shape[1]
    g = min(g, T)
    NG = -(-T // g)
    G = wl.Hq // wl.Hkv
    scale = default_scale(wl.d)
    s32 = np.zeros((wl.B, NG * wl.Hkv, wl.max_seq_len), np.float32)
    members = {}
    for b in range(wl.B):
        P = wl.lens[b]
        k, m, seed = int(hs["topk"][b]), int(hs["sample_budget"][b]), int(hs["seed"][b])
        for c in range(NG):
            mem = list(range(c * g, min((c + 1) * g, T)))
            Lg = orc.group_span(P, T, g, c)
            for h in range(wl.Hkv):
                K, _ = unit_rows(hs, b, h, Lg)
                qs = np.concatenate([q[b, t, h * G:(h + 1) * G] for t in mem])
                s = orc.approx_scores(qs, K, wl.pair_begin, wl.pair_count, scale).astype(np.float32)
                s32[b, c * wl.Hkv + h, :s.size] = s
                sel = orc.select_unit(s, r * k, m, seed, b, h, grp=c)
                for t in mem:
                    members[(b, t, h)] = orc.refine_member(
                        sel, s, q[b, t, h * G:(h + 1) * G], K, orc.member_span(P, T, t), k, m,
                        seed, b, h, c, wl.pair_begin, wl.pair_count, scale)
    return s32, members


def check_staged(wl, g, r, label, split=False):
    T = wl.q.shape[1]
    s32, members = oracle_members(wl, g, r)
    kw = dict(key_layout=ssa.SSA_KEYS_SPLIT) if split else {}
    p = params(wl, g, r, **kw)
    w_in = np.zeros((wl.B, T * wl.Hkv), np.float32)
    for (b, t, h), ms in members.items():
        w_in[b, t * wl.Hkv + h] = ms["W"]
    keys = dict(k_cache=wl.k_cache)
    if split:
        lo, hi = 2 * wl.pair_begin, 2 * (wl.pair_begin + wl.pair_count)
        keys = dict(k_cache=wl.k_cache[..., lo:hi].contiguous(),
                    k_rest=torch.cat([wl.k_cache[..., :lo], wl.k_cache[..., hi:]],
                                     dim=-1).contiguous())
    sd = torch.from_numpy(s32).to(DEV)
    si, sl, sn, _ = ssa.select(p, sd, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed,
                               w_in=torch.from_numpy(w_in).to(DEV), q=wl.q,
                               block_table=wl.block_table, **keys)
    torch.cuda.synchronize()
    si, sl, sn = (x.cpu().numpy() for x in (si, sl, sn))
    nS = nR = 0
    for (b, t, h), ms in members.items():
        S, R, lR = gpu_sets(si, sl, sn, b, t * wl.Hkv + h)
        assert np.array_equal(S, ms["S"]), f"{label}: member stratum differs at {(b, t, h)}"
        assert np.array_equal(R, ms["R"]), f"{label}: member sample differs at {(b, t, h)}"
        assert np.allclose(lR, -np.log(ms["pi_R"].astype(np.float64)), rtol=1e-5, atol=1e-5)
        nS, nR = nS + S.size, nR + R.size
    # the library's own member normalisers
    _, _, _, nm = ssa.select(p, sd, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed, q=wl.q,
                             block_table=wl.block_table, **keys)
    torch.cuda.synchronize()
    nm = nm.cpu().numpy()
    worst = 0.0
    for (b, t, h), ms in members.items():
        W = float(ms["W"])
        got = float(nm[b, t * wl.Hkv + h, 1])
        rel = abs(got - W) / W if W > 0 else abs(got)
        worst = max(worst, rel)
        assert rel <= 1e-6, f"{label}: member normaliser at {(b, t, h)}: {got} vs {W}"
    say(f"[refine] {label}: member selections bit-exact (|S|={nS}, |R|={nR}); own W worst "
        f"rel err {worst:.3g}")
    return members


def check_end_to_end(wl, g, r, label):
    p = params(wl, g, r)
    args = (wl.block_table, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    out = ssa.decode(p, wl.q, wl.k_cache, wl.v_cache, *args).clone()
    out2 = ssa.decode(p, wl.q, wl.k_cache, wl.v_cache, *args)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), f"{label}: not bitwise reproducible"
    hs = wl.host()
    ref, _ = orc.decode_multi(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                              hs["seq_lens"], hs["topk"], hs["sample_budget"], hs["seed"],
                              wl.pair_begin, wl.pair_count, g, refine=r)
    got = out.double().cpu().numpy()
    G = wl.Hq // wl.Hkv
    worst = 0.0
    for b in range(wl.B):
        for h in range(wl.Hkv):
            _, V = unit_rows(hs, b, h, wl.lens[b])
            bound = 2e-3 * vmax_unit(V)
            err = float(np.abs(got[b, :, h * G:(h + 1) * G] - ref[b, :, h * G:(h + 1) * G]).max())
            worst = max(worst, err / bound if bound else 0.0)
            assert err <= bound, f"{label}: output out of tolerance at {(b, h)}: {err} > {bound}"
    say(f"[refine] {label}: end to end within bound (worst err/bound {worst:.3g})")


CFG = dict(B=2, Hq=8, Hkv=2, d=128, L=[9000, 4097], theta=1e6, kdist="normal", planted=16,
           pair_count=32, topk=300, m=200, seeds=[5, 6], data_seed=41)


@pytest.mark.parametrize("T,g,r", [(4, 4, 2), (4, 2, 3), (3, 4, 2), (5, 2, 1)])
def test_refine_staged_and_end_to_end(T, g, r):
    wl = synth.make_workload(dict(CFG), DEV, num_queries=T)
    check_staged(wl, g, r, f"T={T} g={g} r={r}")
    check_end_to_end(wl, g, r, f"T={T} g={g} r={r}")


def test_refine_head_dim_64_many_heads():
    wl = synth.make_workload(dict(B=1, Hq=16, Hkv=1, d=64, L=[12289], theta=1e4,
                                  kdist="normal", planted=8, pair_count=16, topk=100, m=50,
                                  seeds=[7], data_seed=12), DEV, num_queries=2)
    check_staged(wl, 2, 4, "d=64, 16 heads")
    check_end_to_end(wl, 2, 4, "d=64, 16 heads")


def test_refine_edges():
    """Dense members (k + m reaches the span), pure sampling (topk 0), a
    3-token cache, and split keys."""
    wl = synth.make_workload(dict(CFG, L=[700, 300], topk=[100, 150], m=[120, 200]), DEV,
                             num_queries=4)
    check_staged(wl, 4, 2, "dense members")
    check_end_to_end(wl, 4, 2, "dense members")
    wl = synth.make_workload(dict(CFG, topk=0, m=150), DEV, num_queries=4)
    check_staged(wl, 4, 2, "pure sampling")
    wl = synth.make_workload(dict(CFG, L=[3, 9000]), DEV, num_queries=4)
    check_staged(wl, 4, 2, "3-token cache")
    check_end_to_end(wl, 4, 2, "3-token cache")
    wl = synth.make_workload(dict(CFG), DEV, num_queries=4)
    check_staged(wl, 4, 2, "split keys", split=True)
    p_w, p_s = params(wl, 4, 2), params(wl, 4, 2, key_layout=ssa.SSA_KEYS_SPLIT)
    args = (wl.block_table, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    a = ssa.decode(p_w, wl.q, wl.k_cache, wl.v_cache, *args).clone()
    lo, hi = 2 * wl.pair_begin, 2 * (wl.pair_begin + wl.pair_count)
    b = ssa.decode_split(p_s, wl.q, wl.k_cache[..., lo:hi].contiguous(),
                         torch.cat([wl.k_cache[..., :lo], wl.k_cache[..., hi:]], dim=-1).contiguous(),
                         wl.v_cache, *args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_refine_r1_single_query_equals_decode():
    """One query, r = 1: the member keeps the group's stratum and sample, so
    the step is bitwise plain decode."""
    wl = synth.make_workload(dict(CFG), DEV)
    args = (wl.block_table, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    a = ssa.decode(params(wl, 1, 0), wl.q, wl.k_cache, wl.v_cache, *args).clone()
    b = ssa.decode(params(wl, 1, 1), wl.q, wl.k_cache, wl.v_cache, *args)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_refine_rejects_top_p():
    wl = synth.make_workload(dict(CFG), DEV, num_queries=2)
    tp = torch.full((wl.B,), 0.5, dtype=torch.float32, device=DEV)
    with pytest.raises(ssa.SsaError):
        ssa.decode(params(wl, 2, 2), wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens,
                   wl.topk, wl.sample_budget, wl.seed, top_p=tp)
