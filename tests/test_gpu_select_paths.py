"""GPU parity of the top-k selection on score arrays built to reach the
kernels' less common paths, through the C ABI.

"Stratified Sparse Attention speeds up decoding 2.96x at 1M context", "How
SSA stratifies the cache": the top-k stratum is read deterministically (ties
to the lower position) and the rest is Poisson-sampled with inclusion
probability min(1, m w / W).  The resolve kernel keeps each chunk's first 64
threshold-digit candidates of the first 256 chunks in registers and reads
the rest again from memory; the sample kernel ranks the ties on the
threshold key by block scans in the chunks that hold them.  These cases put
candidates and ties past those limits:

* sequences longer than 256 chunks (1M tokens), so the resolve's
  memory-read path serves the chunks beyond;
* coarse scores (many equal keys), so chunks hold thousands of candidates
  and the threshold key is shared by many tokens across chunks.

Selections must be bit-exact against the oracle given the same float32
scores; the tail sample is compared with the oracle's normaliser injected,
and the library's own normaliser within 1e-6 relative.
"""

import numpy as np
import pytest
import torch

from long_context_sparse_approx_amd import ssa
from oracle import ssa_oracle as orc

from gpu_helpers import gpu_sets, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def select_topk(s32, lens, topk, m, seeds, label):
    """Top-k selection parity for score arrays s32 [B, Hkv, Lmax]: once with
    the oracle's W injected (stratum and sample bit-exact), once with the
    library's own W (stratum bit-exact, M exact, W within 1e-6)."""
    B, Hkv, Lmax = s32.shape
    p = ssa.make_params(batch=B, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=128,
                        max_blocks_per_seq=(Lmax + 15) // 16, num_blocks=1, max_seq_len=Lmax)
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device=DEV)
    seed_t = torch.tensor([int(s) for s in seeds], dtype=torch.int64, device=DEV)
    sels, w_in = {}, np.zeros((B, Hkv), np.float32)
    for b in range(B):
        for h in range(Hkv):
            sel = orc.select_unit(s32[b, h, :lens[b]], int(topk[b]), int(m[b]), int(seeds[b]),
                                  b, h)
            sels[(b, h)] = sel
            w_in[b, h] = sel["W"]
    scores = torch.from_numpy(s32).to(DEV)
    for inject in (True, False):
        si, sl, sn, nm = ssa.select(p, scores, i32(lens), i32(topk), i32(m), seed_t,
                                    w_in=torch.from_numpy(w_in).to(DEV) if inject else None)
        torch.cuda.synchronize()
        si, sl, sn, nm = (t.cpu().numpy() for t in (si, sl, sn, nm))
        nS = nR = 0
        for (b, h), sel in sels.items():
            S, R, lR = gpu_sets(si, sl, sn, b, h)
            assert np.array_equal(S, sel["S"]), (
                f"{label}: stratum differs at {(b, h)}: gpu {S.size} oracle {sel['S'].size}")
            if lens[b] > 0:
                assert nm[b, h, 0] == sel["M"], f"{label}: M differs at {(b, h)}"
            if inject:
                assert np.array_equal(R, sel["R"]), f"{label}: sample differs at {(b, h)}"
                assert np.allclose(lR, -np.log(sel["pi_R"].astype(np.float64)), rtol=1e-5,
                                   atol=1e-5)
            elif not sel["dense"] and sel["W"] > 0:
                rel = abs(float(nm[b, h, 1]) - float(sel["W"])) / float(sel["W"])
                assert rel <= 1e-6, f"{label}: own W differs at {(b, h)} by {rel:.2e}"
            nS += S.size
            nR += R.size
        say(f"[select] {label} ({'oracle' if inject else 'own'} W): bit-exact "
            f"(|S|={nS}, |R|={nR})")
    return sels


def test_sequences_past_256_chunks():
    """1,248,576 and 1,050,000 tokens: 305 and 257 chunks, so the resolve
    reads the candidates of chunks 256 and beyond from memory in each pass."""
    rng = np.random.default_rng(71)
    Lmax = 1_248_576
    s = (rng.standard_normal((2, 2, Lmax)) * 0.4).astype(np.float32)
    lens = [Lmax, 1_050_000]
    topk = [12_000, 20_000]
    m = [12_000, 9_000]
    select_topk(s, lens, topk, m, [3, 4], "past 256 chunks")


def test_crowded_chunks_and_shared_threshold_key():
    """Scores on grids of 1/2 and 1/8: a first-digit bin is one or two keys,
    so chunks hold hundreds to thousands of candidates (beyond the 64 kept in
    registers and the 256 a sample workgroup takes per round) and the
    threshold key is shared by hundreds to thousands of tokens across
    chunks."""
    rng = np.random.default_rng(72)
    Lmax = 40_000
    s = rng.standard_normal((3, 1, Lmax))
    s[0] = np.round(s[0] * 2) / 2
    s[1:] = np.round(s[1:] * 8) / 8
    s = s.astype(np.float32)
    lens = [Lmax, 33_333, 9_001]
    topk = [16_000, 7_777, 4_500]
    m = [800, 3_000, 100]
    sels = select_topk(s, lens, topk, m, [5, 6, 7], "crowded")
    for b in range(3):
        keys = orc.order_key(s[b, 0, :lens[b]])
        S = sels[(b, 0)]["S"]
        # the quota on the threshold key (the stratum's smallest) went to
        # that key's lowest positions
        tied = np.nonzero(keys == keys[S].min())[0]
        taken = np.intersect1d(S, tied)
        assert 0 < taken.size < tied.size
        assert np.array_equal(taken, tied[:taken.size])
