"""GPU parity of split keys and cache append, through the C ABI.

"FASA: Frequency-aware Sparse Attention", section 3, variants: FASA-M keeps
the dominant key components on the GPU and moves the other key components and
the values to host memory.  Append is byte work: bit-exact against the
oracle.  A decode over split keys runs the same arithmetic in the same order
as over whole keys, so its output is compared bitwise with the whole-key
decode (itself parity-tested against the oracle), and once directly against
the oracle within 2e-3 max|V|.  Split arrays handed to the library are cut
from the whole cache with torch slicing (the caller's layout), never by the
library under test.
"""

import math

import numpy as np
import pytest
import torch

from long_context_sparse_approx_amd import ssa, synth
from oracle import ssa_oracle as orc

from gpu_helpers import say, unit_rows, vmax_unit

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def split_dev(k_cache, pb, pc):
    """(k_dom, k_rest) of a whole-key cache by torch slicing; k_rest None when
    the scored pairs cover the head."""
    d = k_cache.shape[-1]
    lo, hi = 2 * pb, 2 * (pb + pc)
    k_dom = k_cache[..., lo:hi].contiguous()
    if hi - lo == d:
        return k_dom, None
    return k_dom, torch.cat([k_cache[..., :lo], k_cache[..., hi:]], dim=-1).contiguous()


def bits(t):
    return None if t is None else t.view(torch.int16).cpu().numpy().view(np.uint16)


APPEND_CASES = {
    "one_token": dict(d=128, Hkv=8, pb=32, pc=32, T=1, lens=[1000, 37]),
    "short_sequences": dict(d=64, Hkv=3, pb=0, pc=16, T=5, lens=[3, 700, 64]),
    "middle_pairs": dict(d=128, Hkv=2, pb=4, pc=8, T=7, lens=[16, 4099]),
    "whole_head_scored": dict(d=128, Hkv=4, pb=0, pc=64, T=3, lens=[50]),
    "many_heads": dict(d=64, Hkv=16, pb=8, pc=4, T=2, lens=[33, 1]),
    "bulk": dict(d=128, Hkv=8, pb=32, pc=32, T=5000, lens=[5000, 6000]),
}


def append_setup(c, seed):
    g = torch.Generator().manual_seed(seed)
    B, T, Hkv, d = len(c["lens"]), c["T"], c["Hkv"], c["d"]
    per = [(L + 15) // 16 for L in c["lens"]]
    nblk = sum(per) + 3
    perm = torch.randperm(nblk, generator=g)
    mb = max(per)
    bt = torch.zeros((B, mb), dtype=torch.int32)
    at = 0
    for b, n in enumerate(per):  # disjoint blocks per sequence
        bt[b, :n] = perm[at:at + n]
        at += n
    rnd = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16)
    return (bt, rnd(nblk, Hkv, 16, d), rnd(nblk, Hkv, 16, d), rnd(B, T, Hkv, d),
            rnd(B, T, Hkv, d), max(c["lens"]))


@pytest.mark.parametrize("layout", ["whole", "split"])
@pytest.mark.parametrize("name", list(APPEND_CASES))
def test_append_bit_exact(name, layout):
    c = APPEND_CASES[name]
    bt, k0, v0, kn, vn, Lmax = append_setup(c, 100 + len(name))
    B, d = len(c["lens"]), c["d"]
    say(f"[split] append case={name} layout={layout} T={c['T']} lens={c['lens']}")
    split = layout == "split"
    p = ssa.make_params(batch=B, num_q_heads=c["Hkv"], num_kv_heads=c["Hkv"], head_dim=d,
                        max_blocks_per_seq=bt.shape[1], num_blocks=k0.shape[0],
                        max_seq_len=Lmax, pair_begin=c["pb"], pair_count=c["pc"],
                        key_layout=ssa.SSA_KEYS_SPLIT if split else ssa.SSA_KEYS_WHOLE)
    dev = lambda t: t.to(DEV)
    kd, kr = (split_dev(dev(k0), c["pb"], c["pc"]) if split else (dev(k0).clone(), None))
    vd = dev(v0).clone()
    lens = torch.tensor(c["lens"], dtype=torch.int32)
    ssa.append_kv(p, dev(kn), dev(vn), dev(bt), dev(lens), kd, kr, vd)
    torch.cuda.synchronize()
    u16 = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    k_ref, v_ref = orc.append_kv(u16(k0), u16(v0), bt.numpy(), c["lens"], u16(kn), u16(vn))
    assert np.array_equal(bits(vd), v_ref)
    if split:
        dom_ref, rest_ref = orc.split_keys(k_ref, c["pb"], c["pc"])
        assert np.array_equal(bits(kd), dom_ref)
        if kr is not None:
            assert np.array_equal(bits(kr), rest_ref)
        else:
            assert rest_ref.shape[-1] == 0
    else:
        assert np.array_equal(bits(kd), k_ref)


DECODE_CASES = {
    "ragged": dict(cfg=dict(B=2, Hq=8, Hkv=2, d=128, L=[9000, 4097], theta=1e6,
                            kdist="normal", planted=16, pair_count=32, topk=300, m=200,
                            seeds=[5, 6], data_seed=41), pb=32),
    "low_pairs": dict(cfg=dict(B=1, Hq=4, Hkv=1, d=64, L=[5000], theta=1e4, kdist="normal",
                               planted=8, pair_count=16, topk=60, m=40, seeds=[7],
                               data_seed=42), pb=0),
    "middle_pairs": dict(cfg=dict(B=1, Hq=16, Hkv=2, d=128, L=[12289], theta=1e6,
                                  kdist="mixture", planted=8, pair_count=8, topk=100, m=100,
                                  seeds=[8], data_seed=43), pb=20),
    "whole_head_scored": dict(cfg=dict(B=1, Hq=8, Hkv=8, d=64, L=[3000], theta=1e4,
                                       kdist="normal", planted=0, pair_count=32, topk=50,
                                       m=50, seeds=[9], data_seed=44), pb=0),
}


def decode_case(name, **kw):
    spec = DECODE_CASES[name]
    cfg = dict(spec["cfg"])
    wl = synth.make_workload(cfg, DEV, pair_begin=spec["pb"], **kw)
    return wl


def params(wl, split, **kw):
    return ssa.params_for(wl.q, wl.k_cache, wl.block_table, wl.max_seq_len,
                          pair_begin=wl.pair_begin, pair_count=wl.pair_count,
                          key_layout=ssa.SSA_KEYS_SPLIT if split else ssa.SSA_KEYS_WHOLE, **kw)


def both(wl, k_rest_dev=True, **kw):
    """(whole-key output, split-key output) of one decode step."""
    pw, ps = params(wl, False, **kw), params(wl, True, **kw)
    args = (wl.block_table, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    out_w = ssa.decode(pw, wl.q, wl.k_cache, wl.v_cache, *args).clone()
    k_dom, k_rest = split_dev(wl.k_cache, wl.pair_begin, wl.pair_count)
    v = wl.v_cache
    if not k_rest_dev:  # FASA-M: the rest of the keys and the values in pinned host memory
        k_rest = None if k_rest is None else k_rest.cpu().pin_memory()
        v = wl.v_cache.cpu().pin_memory()
    out_s = ssa.decode_split(ps, wl.q, k_dom, k_rest, v, *args)
    torch.cuda.synchronize()
    return out_w, out_s


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_split_equals_whole_keys(name):
    wl = decode_case(name)
    say(f"[split] decode case={name} pairs=[{wl.pair_begin}, +{wl.pair_count})")
    out_w, out_s = both(wl)
    assert torch.equal(out_w, out_s)


def test_decode_split_against_oracle():
    wl = decode_case("ragged")
    _, out_s = both(wl)
    hs = wl.host()
    ref, _ = orc.decode(hs["q"], hs["k_cache"], hs["v_cache"], hs["block_table"],
                        hs["seq_lens"], hs["topk"], hs["sample_budget"], hs["seed"],
                        wl.pair_begin, wl.pair_count, 1.0 / math.sqrt(wl.d))
    got = out_s.double().cpu().numpy()
    G = wl.Hq // wl.Hkv
    for b in range(wl.B):
        for h in range(wl.Hkv):
            _, V = unit_rows(hs, b, h, wl.lens[b])
            err = float(np.abs(got[b, h * G:(h + 1) * G] - ref[b, h * G:(h + 1) * G]).max())
            assert err <= 2e-3 * vmax_unit(V), (b, h, err)


def test_decode_split_with_options():
    """Multi-query groups, top-p and early stopping over split keys."""
    wl = decode_case("ragged", num_queries=4)
    out_w, out_s = both(wl, query_group=2)
    assert torch.equal(out_w, out_s)
    wl = decode_case("ragged")
    for kw in (dict(early_stop=0.05),):
        out_w, out_s = both(wl, **kw)
        assert torch.equal(out_w, out_s), kw
    tp = torch.tensor([0.3, 0.5], dtype=torch.float32, device=DEV)
    pw, ps = params(wl, False), params(wl, True)
    args = (wl.block_table, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    a = ssa.decode(pw, wl.q, wl.k_cache, wl.v_cache, *args, top_p=tp).clone()
    k_dom, k_rest = split_dev(wl.k_cache, wl.pair_begin, wl.pair_count)
    b = ssa.decode_split(ps, wl.q, k_dom, k_rest, wl.v_cache, *args, top_p=tp)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_scores_and_attention_split_equal_whole_keys():
    wl = decode_case("middle_pairs")
    pw, ps = params(wl, False), params(wl, True)
    k_dom, k_rest = split_dev(wl.k_cache, wl.pair_begin, wl.pair_count)
    sw = ssa.score(pw, wl.q, wl.k_cache, wl.block_table, wl.seq_lens)
    ss = ssa.score(ps, wl.q, k_dom, wl.block_table, wl.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(sw, ss)
    si, sl, sn, _ = ssa.select(pw, sw, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    aw = ssa.attend(pw, wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.seq_lens, si, sl, sn)
    aw = aw.clone()
    as_ = ssa.attend_split(ps, wl.q, k_dom, k_rest, wl.v_cache, wl.block_table, wl.seq_lens,
                           si, sl, sn)
    torch.cuda.synchronize()
    assert torch.equal(aw, as_)


@pytest.mark.parametrize("name", ["ragged", "whole_head_scored"])
def test_offloaded_rest_and_values(name):
    """k_rest and v_cache in pinned host memory, read by the kernels in place."""
    wl = decode_case(name)
    say(f"[split] host-offloaded rest and values, case={name}")
    out_w, out_s = both(wl, k_rest_dev=False)
    assert torch.equal(out_w, out_s)


def test_cache_built_by_append_decodes_like_the_original():
    """Bulk append of every token into empty split caches rebuilds the cache;
    the decode over it equals the whole-key decode of the original cache."""
    wl = decode_case("ragged")
    B, Hkv, d = wl.B, wl.Hkv, wl.d
    T = max(wl.lens)
    pos = torch.arange(T, device=DEV)
    k_new = torch.zeros((B, T, Hkv, d), dtype=torch.bfloat16, device=DEV)
    v_new = torch.zeros_like(k_new)
    for b in range(B):  # token t of sequence b lands at position L_b - T + t
        L = wl.lens[b]
        p = pos[:L]
        rows = wl.block_table[b, (p // 16).long()].long()
        k_new[b, T - L:] = wl.k_cache[rows, :, (p % 16).long(), :]
        v_new[b, T - L:] = wl.v_cache[rows, :, (p % 16).long(), :]
    ps = params(wl, True)
    pc2 = 2 * wl.pair_count
    k_dom = torch.zeros((wl.k_cache.shape[0], Hkv, 16, pc2), dtype=torch.bfloat16, device=DEV)
    k_rest = torch.zeros((wl.k_cache.shape[0], Hkv, 16, d - pc2), dtype=torch.bfloat16,
                         device=DEV)
    v = torch.zeros_like(wl.v_cache)
    ssa.append_kv(ps, k_new, v_new, wl.block_table, wl.seq_lens, k_dom, k_rest, v)
    args = (wl.block_table, wl.seq_lens, wl.topk, wl.sample_budget, wl.seed)
    out_s = ssa.decode_split(ps, wl.q, k_dom, k_rest, v, *args).clone()
    out_w = ssa.decode(params(wl, False), wl.q, wl.k_cache, wl.v_cache, *args)
    torch.cuda.synchronize()
    assert torch.equal(out_w, out_s)
