"""Seeded synthetic decode workloads (inputs only; none of the method's arithmetic).

Both the HIP path and the CPU oracle are fed from here.  A workload is one
decode step of one GQA attention layer over a paged KV cache:

* q ~ N(0, 1) per element, K and V ~ N(0, 1) (or a per-token scale mixture for
  K), drawn in float32 from a seeded ``torch.Generator`` and rounded to bf16
  (round to nearest even);
* RoPE with interleaved pairs (2p, 2p+1) and frequency theta^(-2p/d) rotates
  q at position L and the keys at positions 0..L-1, so the cache holds
  post-RoPE keys, as a decoder's cache does;
* optional planted keys: at uniformly drawn positions the (post-RoPE) key z is
  replaced by z - (u.z) u + 6 u with u the unit vector of the group's mean
  query, so that its dot with the mean query is 6 standard deviations;
* 16-token blocks, shuffled over the whole cache (the block table is a random
  permutation), so every run exercises the paged gather;
* per-sequence budgets: the 50x rule budget = round(L / 50) (half up),
  topk = ceil(budget / 2), sample_budget = floor(budget / 2).

The named configurations mirror the decode workloads the pages discuss
(32K, 128K and 1M contexts, an 8B-class 32/8-head layer, 50x sparsity).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK = 16


def budget_rule(L: int) -> tuple[int, int]:
    """(topk, sample_budget) for a 50x budget round(L/50), split ceil/floor."""
    budget = (L + 25) // 50
    return (budget + 1) // 2, budget // 2


CONFIGS = {
    # Tiny CPU-checkable decode.
    "tiny": dict(B=1, Hq=4, Hkv=1, d=64, L=[4096], theta=1e4, kdist="normal", planted=8,
                 pair_count=16, topk=64, m=32, seeds=[0], data_seed=1),
    # One 8B-class GQA layer at 32K.
    "32k": dict(B=1, Hq=32, Hkv=8, d=128, L=[32768], theta=1e6, kdist="normal", planted=64,
                pair_count=32, topk="rule", m="rule", seeds=[0], data_seed=2),
    # Same layer at 128K, batch 4, heavy-tailed keys.
    "128k": dict(B=4, Hq=32, Hkv=8, d=128, L=[131072] * 4, theta=1e6, kdist="mixture",
                 planted=0, pair_count=32, topk="rule", m="rule", seeds=[0] * 4, data_seed=3),
    # Million-token decode.
    "1m": dict(B=1, Hq=32, Hkv=8, d=128, L=[1048576], theta=1e6, kdist="normal", planted=256,
               pair_count=32, topk="rule", m="rule", seeds=[0], data_seed=4),
    # Batched paged decode, lengths log-uniform in [8192, 131072].
    "batched": dict(B=32, Hq=32, Hkv=8, d=128, L="loguniform", theta=1e6, kdist="normal",
                    planted=0, pair_count=32, topk="rule", m="rule",
                    seeds=[1000 + b for b in range(32)], data_seed=5),
}


@dataclass
class Workload:
    name: str
    q: torch.Tensor            # [B, Hq, d] bf16
    k_cache: torch.Tensor      # [num_blocks, Hkv, 16, d] bf16
    v_cache: torch.Tensor      # [num_blocks, Hkv, 16, d] bf16
    block_table: torch.Tensor  # [B, max_blocks] int32
    seq_lens: torch.Tensor     # [B] int32
    topk: torch.Tensor         # [B] int32
    sample_budget: torch.Tensor  # [B] int32
    seed: torch.Tensor         # [B] int64 holding uint64 bit patterns
    pair_begin: int
    pair_count: int
    theta: float
    lens: list = field(default_factory=list)

    @property
    def B(self):
        return self.q.shape[0]

    @property
    def T(self):
        """Query positions per sequence (q is [B, Hq, d] when 1, else [B, T, Hq, d])."""
        return 1 if self.q.dim() == 3 else self.q.shape[1]

    @property
    def Hq(self):
        return self.q.shape[-2]

    @property
    def Hkv(self):
        return self.k_cache.shape[1]

    @property
    def d(self):
        return self.q.shape[-1]

    @property
    def max_seq_len(self):
        return max(self.lens)

    def host(self):
        """float64 / int64 numpy copies for the oracle (exact bf16 values)."""
        f = lambda t: t.detach().to("cpu", torch.float32).numpy().astype("float64")
        i = lambda t: t.detach().to("cpu").numpy().astype("int64")
        return dict(q=f(self.q), k_cache=f(self.k_cache), v_cache=f(self.v_cache),
                    block_table=i(self.block_table), seq_lens=i(self.seq_lens),
                    topk=i(self.topk), sample_budget=i(self.sample_budget),
                    seed=[int(s) & 0xFFFFFFFFFFFFFFFF for s in self.seed.tolist()],
                    pair_begin=self.pair_begin, pair_count=self.pair_count)


def rope_tables(positions: torch.Tensor, d: int, theta: float):
    """cos, sin [len(positions), d/2] (float32) for interleaved pairs."""
    p = torch.arange(d // 2, dtype=torch.float64, device=positions.device)
    inv = theta ** (-2.0 * p / d)
    ang = positions.to(torch.float64)[:, None] * inv[None, :]
    return torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)


def apply_rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor) -> torch.Tensor:
    """Rotate interleaved pairs of x [..., T, H, d] by (cos, sin) [T, d/2]."""
    x0, x1 = x[..., 0::2], x[..., 1::2]
    c, s = cos[:, None, :], sin[:, None, :]
    out = torch.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def _lens(cfg, gen, device):
    if cfg["L"] == "loguniform":
        u = torch.rand(cfg["B"], generator=gen, device=device, dtype=torch.float64).cpu()
        lo, hi = math.log(8192), math.log(131072)
        return [int(round(math.exp(lo + (hi - lo) * float(x)))) for x in u]
    return list(cfg["L"])


def make_workload(name_or_cfg, device="cpu", *, L=None, B=None, topk=None, m=None,
                  seeds=None, data_seed=None, chunk_tokens=1 << 16, num_queries=1,
                  **overrides) -> Workload:
    """Build a workload from a named config (or a config dict) with overrides.

    ``L`` may be an int (all sequences) or a list; ``topk``/``m`` may be ints or
    "rule".  Generation is chunked over tokens to bound temporary memory.
    With ``num_queries`` T > 1 the step carries T query positions per sequence
    (the last T cache positions, their keys already cached): q is
    [B, T, Hq, d] and the planted keys follow the mean of all T queries.
    """
    if isinstance(name_or_cfg, str):
        name, cfg = name_or_cfg, dict(CONFIGS[name_or_cfg])
    else:
        name, cfg = "custom", dict(name_or_cfg)
    cfg.update(overrides)
    if B is not None:
        cfg["B"] = B
    if L is not None:
        cfg["L"] = [L] * cfg["B"] if isinstance(L, int) else list(L)
    if topk is not None:
        cfg["topk"] = topk
    if m is not None:
        cfg["m"] = m
    if seeds is not None:
        cfg["seeds"] = list(seeds)
    if data_seed is not None:
        cfg["data_seed"] = data_seed
    B, Hq, Hkv, d = cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["d"]
    G = Hq // Hkv
    gen = torch.Generator(device=device)
    gen.manual_seed(int(cfg["data_seed"]))
    lens = _lens(cfg, gen, device)
    assert len(lens) == B
    nblk = [(L_ + BLOCK - 1) // BLOCK for L_ in lens]
    total = sum(nblk)
    max_blocks = max(nblk)
    perm = torch.randperm(total, generator=gen, device=device).to(torch.int32)
    block_table = torch.zeros((B, max_blocks), dtype=torch.int32, device=device)
    k_cache = torch.zeros((total, Hkv, BLOCK, d), dtype=torch.bfloat16, device=device)
    v_cache = torch.zeros_like(k_cache)
    nq = int(num_queries)
    q_all = torch.empty((B, Hq, d) if nq == 1 else (B, nq, Hq, d), dtype=torch.bfloat16,
                        device=device)
    off = 0
    for b in range(B):
        L_ = lens[b]
        phys = perm[off:off + nblk[b]]
        off += nblk[b]
        block_table[b, :nblk[b]] = phys
        if nq == 1:
            qb = torch.randn((1, Hq, d), generator=gen, device=device, dtype=torch.float32)
            cq, sq = rope_tables(torch.tensor([L_], device=device), d, cfg["theta"])
            qb = apply_rope(qb, cq, sq)[0].to(torch.bfloat16)
            q_all[b] = qb
            qbar = qb.float().view(Hkv, G, d).mean(dim=1)  # [Hkv, d]
        else:
            qb = torch.randn((nq, Hq, d), generator=gen, device=device, dtype=torch.float32)
            pos = torch.arange(L_ - nq, L_, device=device)
            cq, sq = rope_tables(pos, d, cfg["theta"])
            qb = apply_rope(qb, cq, sq).to(torch.bfloat16)
            q_all[b] = qb
            qbar = qb.float().view(nq, Hkv, G, d).mean(dim=(0, 2))  # [Hkv, d]
        uhat = qbar / qbar.norm(dim=-1, keepdim=True)
        planted = int(cfg["planted"])
        plant_pos = []
        for h in range(Hkv):
            if planted > 0:
                plant_pos.append(torch.randperm(L_, generator=gen, device=device)[:planted])
        # Keys and values, generated in token chunks (whole blocks).
        step = max(BLOCK, (chunk_tokens // BLOCK) * BLOCK)
        for t0 in range(0, L_, step):
            t1 = min(L_, t0 + step)
            T = t1 - t0
            kz = torch.randn((T, Hkv, d), generator=gen, device=device, dtype=torch.float32)
            if cfg["kdist"] == "mixture":
                wide = torch.rand((T, 1, 1), generator=gen, device=device) < 0.1
                kz = torch.where(wide, kz * 3.0, kz)
            vz = torch.randn((T, Hkv, d), generator=gen, device=device, dtype=torch.float32)
            ck, sk = rope_tables(torch.arange(t0, t1, device=device), d, cfg["theta"])
            kz = apply_rope(kz, ck, sk)
            for h in range(planted and Hkv):
                pos = plant_pos[h]
                pos = pos[(pos >= t0) & (pos < t1)] - t0
                if pos.numel():
                    z = kz[pos, h, :]
                    u = uhat[h][None, :]
                    kz[pos, h, :] = z - (z * u).sum(-1, keepdim=True) * u + 6.0 * u
            tok = torch.arange(t0, t1, device=device)
            blk = phys[(tok // BLOCK).long()].long()
            slot = (tok % BLOCK).long()
            k_cache[blk, :, slot, :] = kz.to(torch.bfloat16)
            v_cache[blk, :, slot, :] = vz.to(torch.bfloat16)
    rule = [budget_rule(L_) for L_ in lens]
    def per_seq(v, i):  # "rule", one value for every sequence, or one per sequence
        if isinstance(v, str):
            return [r[i] for r in rule]
        return [int(x) for x in v] if isinstance(v, (list, tuple)) else [int(v)] * B

    tk, mm = per_seq(cfg["topk"], 0), per_seq(cfg["m"], 1)
    seeds_ = list(cfg["seeds"])
    if len(seeds_) == 1 and B > 1:
        seeds_ = seeds_ * B
    seed_t = torch.tensor([int(s) if s < (1 << 63) else int(s) - (1 << 64) for s in seeds_],
                          dtype=torch.int64, device=device)
    pc = int(cfg["pair_count"])
    pb = int(cfg.get("pair_begin", d // 2 - pc))
    i32 = lambda xs: torch.tensor(xs, dtype=torch.int32, device=device)
    return Workload(name=name, q=q_all, k_cache=k_cache, v_cache=v_cache,
                    block_table=block_table, seq_lens=i32(lens), topk=i32(tk),
                    sample_budget=i32(mm), seed=seed_t, pair_begin=pb, pair_count=pc,
                    theta=float(cfg["theta"]), lens=lens)
