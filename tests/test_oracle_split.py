"""Pins of the oracle's split keys and cache append (no GPU).

"FASA: Frequency-aware Sparse Attention", section 3, variants: FASA-M keeps
the dominant key components resident and moves the rest of each key (and the
values) elsewhere.  The oracle's reading: the scored RoPE pairs of a key row
in one array, the remaining dims in dim order in another, under the same row
number; new tokens land at positions seq_lens[b] - T + t.  The pins check the
two parts against torch's exact logits over the dims they hold, the dim order
against rows that carry their own dim index, placement against the
brute-force-pinned paging, and plant plausible slips.
"""

import numpy as np
import torch

from oracle import ssa_oracle as orc

CASES = ((128, 32, 32), (128, 0, 16), (128, 4, 8), (64, 0, 32), (64, 16, 16), (64, 8, 4))


def pair_mask(d, pb, pc):
    """Dims 2p and 2p + 1 of every scored pair p (built pair by pair)."""
    m = np.zeros(d, bool)
    for p in range(pb, pb + pc):
        m[2 * p] = m[2 * p + 1] = True
    return m


def logits(q, K, keep):
    """torch's exact logits q . k over the dims in keep (the others zeroed)."""
    qz, kz = q.copy(), K.copy()
    qz[:, ~keep] = 0.0
    kz[:, ~keep] = 0.0
    return (torch.from_numpy(qz) @ torch.from_numpy(kz).T).numpy()


def split_error():
    """Scores from the scored part alone, and the rest's share of the logit,
    against torch over the dims each should hold."""
    rng = np.random.default_rng(21)
    worst = 0.0
    for d, pb, pc in CASES:
        q = rng.standard_normal((3, d))
        K = rng.standard_normal((50, d))
        k_dom, k_rest = orc.split_keys(K, pb, pc)
        q_dom, q_rest = orc.split_keys(q, pb, pc)
        keep = pair_mask(d, pb, pc)
        worst = max(worst, np.abs(q_dom @ k_dom.T - logits(q, K, keep)).max())
        worst = max(worst, np.abs(q_rest @ k_rest.T - logits(q, K, ~keep)).max() if pc < d // 2
                    else 0.0)
        # the indexer's score needs nothing but the scored part
        s_full = orc.approx_scores(q, K, pb, pc, 0.125)
        s_dom = orc.approx_scores(q_dom, k_dom, 0, pc, 0.125)
        worst = max(worst, np.abs(s_full - s_dom).max())
    return worst


def test_parts_hold_the_scored_and_other_dims():
    assert split_error() < 1e-12


def order_error():
    """Rows that carry their dim index: the scored part is the dims of the
    pair range in order, the rest the dims below it then the dims above it."""
    bad = 0
    for d, pb, pc in CASES:
        row = np.arange(d, dtype=np.float64)[None, None, :].repeat(2, 0).repeat(3, 1)
        k_dom, k_rest = orc.split_keys(row, pb, pc)
        lo, hi = 2 * pb, 2 * (pb + pc)
        bad += not np.array_equal(k_dom[0, 0], np.arange(lo, hi))
        bad += not np.array_equal(k_rest[1, 2], np.r_[np.arange(0, lo), np.arange(hi, d)])
        bad += not np.array_equal(orc.join_keys(k_dom, k_rest, pb), row)
    return bad


def test_dim_order_and_round_trip():
    assert order_error() == 0


def append_case():
    rng = np.random.default_rng(22)
    B, T, Hkv, d = 2, 40, 3, 8
    nblk = 8
    perm = rng.permutation(nblk)
    bt = np.stack([perm[:4], perm[4:]])  # the sequences own disjoint blocks
    kc = np.full((nblk, Hkv, 16, d), -7.0)
    vc = np.full((nblk, Hkv, 16, d), -9.0)
    k_new = rng.standard_normal((B, T, Hkv, d))
    v_new = rng.standard_normal((B, T, Hkv, d))
    seq_lens = [40, 25]  # sequence 1: only its last 25 new tokens have a position
    return bt, kc, vc, k_new, v_new, seq_lens


def append_error():
    bt, kc, vc, k_new, v_new, seq_lens = append_case()
    k, v = orc.append_kv(kc, vc, bt, seq_lens, k_new, v_new)
    bad = 0
    for h in range(3):
        bad += not np.array_equal(orc.gather_rows(k, bt[0], h, 40), k_new[0, :, h])
        bad += not np.array_equal(orc.gather_rows(v, bt[0], h, 40), v_new[0, :, h])
        bad += not np.array_equal(orc.gather_rows(k, bt[1], h, 25), k_new[1, 15:, h])
        bad += not np.array_equal(orc.gather_rows(v, bt[1], h, 25), v_new[1, 15:, h])
    # every other slot keeps its old contents: 40 + 25 tokens per head written
    bad += int(np.sum(k != -7.0)) != 65 * 3 * 8 or int(np.sum(v != -9.0)) != 65 * 3 * 8
    return bad


def test_append_places_tokens_at_their_positions():
    assert append_error() == 0


def test_append_of_one_step_extends_the_cache():
    """T new tokens after P - T cached ones: the cache then holds the old
    prefix followed by the new tokens."""
    rng = np.random.default_rng(23)
    P, T, Hkv, d = 37, 3, 2, 8
    bt = np.array([[5, 1, 3]])
    old = rng.standard_normal((P - T, Hkv, d))
    kc = np.zeros((6, Hkv, 16, d))
    kc, _ = orc.append_kv(kc, kc.copy(), bt, [P - T], old[None], old[None])
    k_new = rng.standard_normal((1, T, Hkv, d))
    k, _ = orc.append_kv(kc, kc.copy(), bt, [P], k_new, k_new)
    for h in range(Hkv):
        assert np.array_equal(orc.gather_rows(k, bt[0], h, P),
                              np.concatenate([old[:, h], k_new[0, :, h]]))


def test_pins_catch_planted_split_mistakes(monkeypatch):
    real_split, real_append = orc.split_keys, orc.append_kv
    # 1. the scored range one pair too high
    def shifted(K, pb, pc):
        if pb + pc < K.shape[-1] // 2:
            return real_split(K, pb + 1, pc)
        return real_split(K, pb - 1, pc) if pb > 0 else real_split(K, pb, pc)
    monkeypatch.setattr(orc, "split_keys", shifted)
    assert split_error() > 1e-6
    monkeypatch.undo()
    # 2. the rest with the dims above the range first
    def above_first(K, pb, pc):
        lo, hi = 2 * pb, 2 * (pb + pc)
        return K[..., lo:hi].copy(), np.concatenate([K[..., hi:], K[..., :lo]], axis=-1)
    monkeypatch.setattr(orc, "split_keys", above_first)
    assert order_error() > 0
    monkeypatch.undo()
    # 3. new tokens written after seq_lens instead of ending at it
    monkeypatch.setattr(orc, "append_kv", lambda kc, vc, bt, sl, kn, vn: real_append(
        kc, vc, bt, [s - 1 for s in sl], kn, vn))
    assert append_error() > 0
