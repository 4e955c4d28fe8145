"""The decode step with one query per sequence takes the sample stage's
decisions inside the attention kernel ("Stratified Sparse Attention speeds up
decoding 2.96x at 1M context", "How SSA stratifies the cache").  Its output
must equal attention over the staged selection (ssa_select on the step's own
scores, then ssa_attend) bit for bit, in every mode of that in-kernel
selection:

* sparse chunks, whose lists (at most 128 entries each) are held in
  registers;
* crowded chunks, whose lists are read in rounds with the sampled tokens'
  biases passed through a scratch row;
* tie quotas on a threshold key shared by thousands of tokens across chunks;
* dense units (every valid position), empty and ragged sequences, pure
  sampling, top-k only, top-p, split keys.

The staged path itself is held to the oracle by the parity tests; this file
checks that the fused step computes exactly what it computes.
"""

import pytest
import torch

from long_context_sparse_approx_amd import ssa, synth

from gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def cfg(**kw):
    base = dict(B=1, Hq=8, Hkv=2, d=128, theta=1e6, kdist="normal", planted=4, pair_count=32,
                data_seed=40)
    base.update(kw)
    return base


def staged(wl, p, ws, top_p=None):
    """Attention over ssa_select's selection of the step's own scores."""
    sc = ssa.score(p, wl.q, wl.k_cache, wl.block_table, wl.seq_lens, workspace=ws)
    si, sl, sn, _ = ssa.select(p, sc, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed,
                               workspace=ws, top_p=top_p)
    out = ssa.attend(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, si, sl, sn,
                     workspace=ws)
    return out, sn


def check_equal(wl, label, top_p=None, **kw):
    p = ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                       pair_begin=wl.pair_begin, pair_count=wl.pair_count, **kw)
    ws = ssa.alloc_workspace(p, DEV)
    fused = ssa.decode(p, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, wl.topk,
                       wl.sample_budget, wl.seed, workspace=ws, top_p=top_p).clone()
    ref, sn = staged(wl, p, ws, top_p=top_p)
    torch.cuda.synchronize()
    per_chunk = sn.sum(dim=-1)
    say(f"[fused] {label}: selected {int(per_chunk.sum())} tokens, at most "
        f"{int(per_chunk.max())} in a chunk; max |diff| "
        f"{float((fused.double() - ref.double()).abs().max()):.3g}")
    assert torch.equal(fused, ref), f"{label}: fused step differs from the staged path"
    return per_chunk


def tie_rows(wl, frac, seed):
    """Give a fraction of the cached tokens one shared key row: their scores
    are equal, so the threshold key is shared by thousands of tokens."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    kc = wl.k_cache
    mask = torch.rand(kc.shape[:3], generator=g, device=DEV) < frac
    kc[mask] = kc[0, 0, 0].clone()
    return wl


def test_sparse_chunks_in_registers():
    wl = synth.make_workload(cfg(L=[30000, 12289], topk=[300, 150], m=[300, 100],
                                 seeds=[3, 4], B=2), DEV)
    per_chunk = check_equal(wl, "sparse")
    assert int(per_chunk.max()) <= 256


def test_crowded_chunks_read_in_rounds():
    wl = synth.make_workload(cfg(L=[20000, 13001], topk=[3000, 2500], m=[2000, 1500],
                                 seeds=[5, 6], B=2), DEV)
    per_chunk = check_equal(wl, "crowded")
    assert int(per_chunk.max()) > 256


@pytest.mark.parametrize("frac", [1.0, 0.4])
def test_shared_threshold_key(frac):
    wl = tie_rows(synth.make_workload(cfg(L=[18000, 9000], topk=[2000, 700], m=[500, 400],
                                          seeds=[7, 8], B=2), DEV), frac, 41)
    check_equal(wl, f"ties {frac}")


def test_dense_empty_ragged_and_limits():
    wl = synth.make_workload(cfg(B=5, L=[600, 0, 5000, 1, 4097], topk=[4000, 5, 3000, 1, 20],
                                 m=[1000, 5, 2500, 0, 30], seeds=[9, 10, 11, 12, 13], d=64,
                                 pair_count=16, theta=1e4), DEV)
    check_equal(wl, "dense/empty/ragged")


@pytest.mark.parametrize("topk,m", [(0, 64), (90, 0)])
def test_pure_sampling_and_topk_only(topk, m):
    wl = synth.make_workload(cfg(L=[7000], topk=topk, m=m, seeds=[14]), DEV)
    check_equal(wl, f"topk {topk} m {m}")


def test_top_p():
    wl = synth.make_workload(cfg(B=2, L=[15000, 9000], topk=[400, 300], m=[200, 100],
                                 seeds=[15, 16]), DEV)
    top_p = torch.tensor([0.6, 0.95], dtype=torch.float32, device=DEV)
    check_equal(wl, "top-p", top_p=top_p)


def test_split_keys_fused_equals_staged():
    wl = synth.make_workload(cfg(B=2, L=[20000, 6000], topk=[2500, 60], m=[1500, 40],
                                 seeds=[17, 18]), DEV, pair_begin=16)
    p = ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                       pair_begin=wl.pair_begin, pair_count=wl.pair_count)
    ws = ssa.alloc_workspace(p, DEV)
    ref, _ = staged(wl, p, ws)
    ps = ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                        pair_begin=wl.pair_begin, pair_count=wl.pair_count,
                        key_layout=ssa.SSA_KEYS_SPLIT)
    lo, hi = 2 * wl.pair_begin, 2 * (wl.pair_begin + wl.pair_count)
    k_dom = wl.k_cache[..., lo:hi].contiguous()
    k_rest = torch.cat([wl.k_cache[..., :lo], wl.k_cache[..., hi:]], dim=-1).contiguous()
    out = ssa.decode_split(ps, wl.q, k_dom, k_rest, wl.v_cache, wl.block_table, wl.seq_lens,
                           wl.topk, wl.sample_budget, wl.seed,
                           workspace=ssa.alloc_workspace(ps, DEV))
    torch.cuda.synchronize()
    say(f"[fused] split keys: max |diff| {float((out.double() - ref.double()).abs().max()):.3g}")
    assert torch.equal(out, ref)


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_splits_spanning_several_chunks(splits):
    """A split that spans several chunks takes each chunk's decisions in turn
    (only the first can use the lists read with the query)."""
    wl = synth.make_workload(cfg(B=3, L=[40000, 17000, 4097], topk=[400, 2500, 60],
                                 m=[400, 1500, 40], seeds=[19, 20, 21]), DEV)
    check_equal(wl, f"{splits} splits", num_splits=splits)


def test_batched_mixed_lengths():
    """Sequences of log-uniform lengths (8K-128K), the 50x budget rule: the
    split whose guessed first chunk is past a short sequence's range."""
    wl = synth.make_workload("batched", DEV, B=6)
    check_equal(wl, "batched")


@pytest.mark.parametrize("T,g,L,topk,m", [
    (4, 4, [9000], 60, 40),          # one group of four queries
    (5, 2, [6000, 4100], 50, 30),    # a ragged last group
    (3, 1, [5000], 40, 20),          # one selection per query
    (4, 2, [700], 600, 200),         # dense units
    (5, 2, [3, 4099], 20, 10),       # caches shorter than the step
    (3, 8, [8200], 30, 30),          # a group wider than the step
    (4, 4, [20000], 3000, 2000),     # crowded chunks, lists read in rounds
])
def test_query_groups(T, g, L, topk, m):
    """Several query positions per step, groups of g sharing one selection
    (PIVOT reuse): the decisions are the group's, placed with their positions
    so that every member keeps its own causal span."""
    B = len(L)
    wl = synth.make_workload(cfg(B=B, L=L, topk=topk, m=m, seeds=list(range(30, 30 + B))),
                             DEV, num_queries=T)
    check_equal(wl, f"T={T} g={g}", query_group=g)
