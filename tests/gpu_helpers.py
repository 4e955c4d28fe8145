"""Shared helpers of the GPU parity tests (not collected as tests).

They convert between the library's chunk-segmented selection layout and the
oracle's per-unit sets, and compute the parity bounds.  Every expected value
comes from the oracle, fed with the same seeded inputs as the HIP path.
"""

import math
import sys

import numpy as np
import torch

from long_context_sparse_approx_amd import ssa
from oracle import ssa_oracle as orc

CHUNK = ssa.CHUNK_TOKENS


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def unit_rows(hs, b, h, L):
    K = orc.gather_rows(hs["k_cache"], hs["block_table"][b], h, L)
    V = orc.gather_rows(hs["v_cache"], hs["block_table"][b], h, L)
    return K, V


def group(hs, b, h, G):
    return hs["q"][b, h * G:(h + 1) * G, :]


def oracle_scores(wl, hs, scale):
    """float64 scores per unit {(b, h): [L]}."""
    G = wl.Hq // wl.Hkv
    out = {}
    for b in range(wl.B):
        L = wl.lens[b]
        for h in range(wl.Hkv):
            K, _ = unit_rows(hs, b, h, L)
            out[(b, h)] = orc.approx_scores(group(hs, b, h, G), K, wl.pair_begin, wl.pair_count,
                                            scale)
    return out


def gpu_sets(sel_idx, sel_logw, sel_count, b, h):
    """(S, R, logw_R) of one unit from the segment layout (numpy)."""
    idx = sel_idx[b, h]
    lw = sel_logw[b, h]
    cnt = sel_count[b, h]
    S, R, LR = [], [], []
    for c in range(cnt.shape[0]):
        nS, nR = int(cnt[c, 0]), int(cnt[c, 1])
        base = c * CHUNK
        S.append(idx[base:base + nS])
        R.append(idx[base + nS:base + nS + nR])
        LR.append(lw[base + nS:base + nS + nR])
        assert np.all(lw[base:base + nS] == 0.0)
    return (np.concatenate(S).astype(np.int64), np.concatenate(R).astype(np.int64),
            np.concatenate(LR))


def selection_arrays(p, sels, device):
    """The library's segment layout built from oracle selections {(b, h): sel}."""
    nc = ssa.num_chunks(p)
    B, Hkv = p.batch, p.num_kv_heads
    idx = np.zeros((B, Hkv, nc * CHUNK), np.int32)
    lw = np.zeros((B, Hkv, nc * CHUNK), np.float32)
    cnt = np.zeros((B, Hkv, nc, 2), np.int32)
    for (b, h), sel in sels.items():
        S, R = np.asarray(sel["S"]), np.asarray(sel["R"])
        lR = (-np.log(np.asarray(sel["pi_R"], np.float64))).astype(np.float32)
        for c in range(nc):
            lo, hi = c * CHUNK, (c + 1) * CHUNK
            s_c = S[(S >= lo) & (S < hi)]
            mR = (R >= lo) & (R < hi)
            r_c = R[mR]
            idx[b, h, lo:lo + s_c.size] = s_c
            idx[b, h, lo + s_c.size:lo + s_c.size + r_c.size] = r_c
            lw[b, h, lo + s_c.size:lo + s_c.size + r_c.size] = lR[mR]
            cnt[b, h, c] = (s_c.size, r_c.size)
    t = lambda a: torch.from_numpy(a).to(device)
    return t(idx), t(lw), t(cnt)


def vmax_unit(V):
    return float(np.abs(V).max()) if V.size else 0.0


def jaccard(a, b):
    a, b = set(map(int, a)), set(map(int, b))
    return 1.0 if not a and not b else len(a & b) / len(a | b)


def score_tolerance_ok(gpu, ref):
    """|gpu - ref| <= 1e-3 * max(|ref|, 1e-2 * rms(ref)) for every token: 1e-3
    relative, with a floor at a hundredth of the unit's typical score (a pure
    relative bound is ill-posed at a score of 0).  Returns (ok, worst
    error / bound)."""
    if ref.size == 0:
        return True, 0.0
    err = np.abs(gpu.astype(np.float64) - ref)
    rms = float(np.sqrt(np.mean(np.square(ref))))
    bound = 1e-3 * np.maximum(np.abs(ref), 1e-2 * rms)
    return bool(np.all(err <= bound)), float((err / bound).max())


def default_scale(d):
    return 1.0 / math.sqrt(d)
