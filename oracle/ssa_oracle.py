"""Plain CPU oracle for stratified sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of the
benchmark call it.  It shares no code with the HIP library and imports nothing
from it.

Sources (web pages; cited by title and section):

* [SSA] "Stratified Sparse Attention speeds up decoding 2.96x at 1M context"
  (news.hamidun.com).  Sections "Where sparse attention loses quality" (top-k /
  top-p read deterministically, sampling covers the tail) and "How SSA
  stratifies the cache" (the high-estimate tokens are read deterministically;
  the rest of the cache is sampled with probability proportional to an
  approximate attention estimate; each sampled token is corrected by its
  inclusion probability so the mass outside the selected set is recovered;
  top-k, top-p and top-k + sampling are special cases).
* [FASA] "FASA: Frequency-aware Sparse Attention" (gist.science summary of
  arXiv 2602.03152).  Section 2 (RoPE splits a head into 2-D frequency chunks;
  low-frequency chunks carry contextual attention), section 3 stage 1 "TIP"
  (online score = sum of the contributions of a fixed chunk subset; keep the
  highest-scoring tokens) and stage 2 "FAC" (full-precision attention on the
  selected tokens at their original positions); section 3, variants (FASA-M
  keeps only the dominant key components on the GPU and moves the other key
  components and the values to host memory).
* [PIVOT] "PIVOT slashes sparse-attention indexer cost" (gyaansetu.com),
  section "The two observations behind PIVOT": one proxy query, the mean of a
  group of consecutive queries, is scored instead of each member, and the
  group's candidate set serves its members (section "Two operating modes":
  reusing it as is is the faster mode).
* [S2O] "S2O: Early Stopping for Sparse Attention via Online Permutation"
  (gist.science summary of arXiv 2602.22575), methodology part 2 "Early-
  stopping rule" (blocks visited in descending estimated importance stop once
  a block's marginal gain falls below a threshold relative to the
  accumulated score) and part 3 "Kernel implementation" (the online-softmax
  state (m, l, acc) is stored and resumed).

Readings of points the pages leave open (each one is also listed in the design
notes of the repository):

R1  GQA aggregation: the score of a kv head is the mean over its query group of
    the per-head partial logits (PIVOT's averaged proxy query).
R2  Score scale: the partial dot product times the softmax scale (1/sqrt(d) by
    default); "approximate attention estimate" is exp(score - max score).
R3  Pairs: interleaved RoPE pairs (2p, 2p+1); the scored subset is a contiguous
    pair range [pair_begin, pair_begin + pair_count), the same for every head.
R4  Ranking is done on the float32 rounding of the score, ordered by the
    float's bits (-0.0 below +0.0); ties go to the lower token index.
R5  Dense rule: when k + m >= L every token is read with weight 1, k being
    the size of the deterministic stratum (min(topk, L), further capped by the
    top-p prefix of R15 when a top-p mass is given).
R6  Tail design: Poisson sampling.  w_j = sexp(s_j - M) with M the maximum
    score over the whole sequence, W = sum of w_j over the tail, inclusion
    probability pi_j = min(1, m * w_j / W); m is the expected sample size.
R7  The inclusion decision is made in float32: include j iff
    fl(u_j * W) < fl(m * w_j), with u_j a 24-bit uniform; pi_j (for the
    weight) is min(1, fl(fl(m * w_j) / W)).
R8  u_j comes from Philox4x32-10 (Salmon et al., SC'11) keyed by the 64-bit
    seed (low word first) with counter (j >> 2, h, b, 0); word (j & 3) of the
    output block, u_j = (word >> 8) * 2^-24.  This is element h * 2^34 + j of
    subsequence b of the seed's stream in rocRAND's Philox4x32-10 layout.
R9  sexp is a specified float32 exp (Cody-Waite reduction, degree-7 Taylor
    polynomial, one rounding per operation, no fused multiply-add):
    0 for x < -87.
R10 Horvitz-Thompson weights: c_j = 1 on the deterministic set S and 1/pi_j on
    the sample R; output = sum c e^l v / sum c e^l over S u R.
R15 Top-p stratum: the approximate probability mass of token j is counted in
    integer units, q_j = floor(w_j * 2^38) with w_j = sexp(s_j - M) (so the
    top token holds exactly 2^38 units); Q = sum of q_j over the sequence and
    the target is tau = ceil(p * Q), evaluated exactly.  n_p is the length of
    the shortest prefix of the order (key descending, index ascending) whose
    units reach tau (0 when tau = 0).  The deterministic stratum is the first
    min(topk, n_p) tokens of that order.  Integer mass makes the prefix
    independent of summation order.  p is clamped to [0, 1]; NaN counts as 0.
R16 Multi-query decode (PIVOT reuse): a step may carry T query positions per
    sequence; with P the cache length (the T new tokens included), query t sits
    at position P - T + t and attends to tokens [0, P - T + t].  Queries are
    grouped g consecutive at a time (the last group may be smaller); a group's
    proxy score of token j is the mean over its members and their query heads
    of the partial logits (R1 over the group), over the group's span (the
    last member's causal length).  One selection per (sequence, group, kv
    head), drawn with Philox counter (j >> 2, h, b, group); every member
    attends over it restricted to its own span, with the group's inclusion
    probabilities (the restriction of a Horvitz-Thompson sum to a subset of
    the population stays unbiased for that subset).
R17 Early stopping (S2O): with a gain threshold tau > 0 the deterministic
    stratum S, in its order (key descending, index ascending), is visited in
    blocks of 64 consecutive tokens while the online-softmax state of every
    query row of the unit (each query head of each member; a row only sees
    tokens inside its member's span) accumulates the block's exact attention
    mass.  Block i's marginal gain for row r is D_i^r = the increment of that
    row's l, and C_i^r = the row's l after the block; the visit stops after
    the first block at which every row has D_i^r < tau * C_i^r or D_i^r = 0,
    and S's later blocks are skipped: neither read nor sampled.  The tail
    sample (over the complement of the whole S, normaliser W over it) is
    unchanged.  The decision is taken in the kernel's precision: the exact
    logit is l = fl32(scale * dot), the dot of bf16 values summed in float32
    (each 8-dim slice in dim order, then the slices pairwise); the gain is
    counted in R15's integer units of sexp(l - M_r), M_r the row's largest
    logit over S, so the sums and the comparison are exact.  tau is clamped
    to 1 (NaN and tau <= 0: no stopping).  The rule applies at every
    stratum size.
R18 Split keys (FASA-M): a key row is held as two rows under the same row
    number: the scored dims [2 pair_begin, 2 (pair_begin + pair_count)) in
    one array and the remaining dims, in their order ([0, 2 pair_begin) then
    the dims above the scored range), in another; values are unchanged.
    Appending T new tokens per sequence writes token t of sequence b at
    position seq_lens[b] - T + t (seq_lens counting the new tokens), row
    pos mod 16 of block block_table[b][pos // 16]; negative positions are
    skipped.  A step over split keys computes what it computes over the
    whole keys they hold.
R19 Query groups, refine mode (PIVOT "Two operating modes": each member
    refines the proxy's candidate list): with a refine factor r >= 1 the
    group's proxy selection (R16) runs with a deterministic stratum of r * k
    tokens -- the candidate list C -- and each member t then scores C's
    tokens inside its span with its own query (the mean of its G heads'
    partial logits over the scored pairs) and takes the first
    k_t = min(k, |C inside its span|) of them in the order (own score
    descending, index ascending) as its own deterministic stratum S_t
    (dense when k_t + m >= its span).  Its tail is the group's span minus
    S_t, sampled with the proxy's weights w_j = sexp(s_j - M) (M the group's
    maximum proxy score) and its own normaliser W_t = sum of w_j over that
    tail (float64 sum rounded to float32), with the group's uniforms (Philox
    counter (j >> 2, h, b, group)); pi_j = min(1, fl(fl(m w_j) / W_t)).  The
    member attends over S_t and its samples inside its span.  The own score
    is ranked in the decision precision: per head the float32 dot over the
    scored dims (8-dim slices in dim order, then the slices pairwise, as in
    R17), the heads summed in head order, times fl32(fl32(scale) / G).
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "BLOCK_TOKENS",
    "gather_rows",
    "approx_scores",
    "order_key",
    "topk_indices",
    "sexp",
    "MASS_FRAC_BITS",
    "mass_units",
    "mass_target",
    "topp_count",
    "philox4x32_10",
    "philox_word",
    "uniforms",
    "tail_stratum",
    "sample_tail",
    "select_unit",
    "ht_terms",
    "attend_unit",
    "decode",
    "STOP_BLOCK",
    "stop_logits",
    "stop_gains",
    "stop_count",
    "member_span",
    "group_span",
    "decode_multi",
    "member_scores",
    "refine_member",
    "split_keys",
    "join_keys",
    "append_kv",
]

# Inputs arrive as a paged cache of 16-token blocks (layout, not arithmetic).
BLOCK_TOKENS = 16

_F32 = np.float32


# ---------------------------------------------------------------------------
# Inputs: paged rows
# ---------------------------------------------------------------------------

def gather_rows(cache: np.ndarray, block_row: np.ndarray, h: int, L: int) -> np.ndarray:
    """Rows 0..L-1 of kv head ``h`` of one sequence, as float64 [L, d].

    ``cache`` is [num_blocks, Hkv, 16, d] (values exactly representable in
    bf16, any float dtype); token j lives in block ``block_row[j // 16]`` at
    offset ``j % 16``.  [S2O] methodology part 1 (index arrays drive the loads;
    the physical layout is left in place).
    """
    j = np.arange(L)
    return cache[block_row[j // BLOCK_TOKENS], h, j % BLOCK_TOKENS, :].astype(np.float64)


# ---------------------------------------------------------------------------
# Step 1: approximate scores ([FASA] stage 1 TIP; [PIVOT] proxy query)
# ---------------------------------------------------------------------------

def approx_scores(q_group: np.ndarray, K: np.ndarray, pair_begin: int, pair_count: int,
                  scale: float) -> np.ndarray:
    """Approximate score of every token for one (batch, kv head), float64 [L].

    s_j = (1/G) * sum_g scale * sum_{p in I} (q_g[2p] k_j[2p] + q_g[2p+1] k_j[2p+1])
    with I = [pair_begin, pair_begin + pair_count) (readings R1-R3).
    ``q_group`` is [G, d], ``K`` is [L, d] (post-RoPE keys).
    """
    dims = np.arange(2 * pair_begin, 2 * (pair_begin + pair_count))
    partial = scale * (q_group[:, dims].astype(np.float64) @ K[:, dims].T)  # [G, L]
    return partial.mean(axis=0)


# ---------------------------------------------------------------------------
# Step 2: deterministic stratum ([SSA] "Where sparse attention loses quality",
# top-k; [FASA] TIP selection of the highest-scoring tokens)
# ---------------------------------------------------------------------------

def order_key(s32: np.ndarray) -> np.ndarray:
    """Monotone map of float32 scores to uint32 (larger float -> larger key).

    Negative floats have all bits flipped, non-negative ones get the sign bit
    set, so -0.0 (0x7fffffff) ranks just below +0.0 (0x80000000) (reading R4).
    """
    bits = np.ascontiguousarray(s32, dtype=_F32).view(np.uint32)
    neg = (bits >> np.uint32(31)) == 1
    return np.where(neg, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)


def topk_indices(s32: np.ndarray, k: int) -> np.ndarray:
    """The k tokens first in the order (key descending, index ascending),
    returned in ascending index order.  A full sort, no partial selection."""
    key = order_key(s32)
    idx = np.arange(key.size, dtype=np.int64)
    order = np.lexsort((idx, ~key))  # primary: ~key ascending == key descending
    return np.sort(order[:k])


# ---------------------------------------------------------------------------
# Step 3: tail weights -- the specified float32 exp (reading R9)
# ---------------------------------------------------------------------------

# Cody & Waite, "Software Manual for the Elementary Functions" (1980): reduce
# x = n ln2 + r with ln2 split into a short head (so n * head is exact for
# |n| < 2^9) and a float32 tail.  The head keeps 16 fractional bits of ln2.
_LOG2E = _F32(1.0 / math.log(2.0))
_LN2_HI = _F32(math.floor(math.log(2.0) * 2.0 ** 16) / 2.0 ** 16)
_LN2_LO = _F32(math.log(2.0) - float(_LN2_HI))
# Taylor coefficients 1/k!, k = 0..7, each rounded to float32.
_TAYLOR = [_F32(1.0 / math.factorial(k)) for k in range(8)]
_SEXP_MIN = _F32(-87.0)


def sexp(x) -> np.ndarray:
    """Specified float32 exp for x <= 0 (reading R9).

    n = rint(fl(x * log2e)); r = fl(fl(x - fl(n * ln2_hi)) - fl(n * ln2_lo));
    p = Horner over 1/k!, k = 7..0, one multiply then one add per step, each
    rounded to float32; result = p * 2^n (exact); 0 when x < -87, which keeps
    every non-zero result a normal float.
    """
    x = np.asarray(x, dtype=_F32)
    low = x < _SEXP_MIN
    x = np.where(low, _F32(0.0), x)  # keep the (discarded) lanes finite
    t = np.multiply(x, _LOG2E, dtype=_F32)
    n = np.rint(t).astype(_F32)
    r = np.subtract(x, np.multiply(n, _LN2_HI, dtype=_F32), dtype=_F32)
    r = np.subtract(r, np.multiply(n, _LN2_LO, dtype=_F32), dtype=_F32)
    p = _TAYLOR[7]
    for k in range(6, -1, -1):
        p = np.multiply(p, r, dtype=_F32)
        p = np.add(p, _TAYLOR[k], dtype=_F32)
    y = np.ldexp(p, n.astype(np.int32)).astype(_F32)
    return np.where(low, _F32(0.0), y).astype(_F32)


# ---------------------------------------------------------------------------
# Step 2 alternative: the top-p deterministic stratum ([SSA] "Where sparse
# attention loses quality", top-p as a deterministic option; "How SSA
# stratifies the cache", top-p as a special case) -- reading R15
# ---------------------------------------------------------------------------

MASS_FRAC_BITS = 38


def mass_units(w32) -> np.ndarray:
    """floor(w * 2^38) of float32 weights in [0, 1], as uint64 (exact: the
    scaling by a power of two and the floor are both exact in float64)."""
    w = np.asarray(w32, dtype=_F32).astype(np.float64)
    return np.floor(w * 2.0 ** MASS_FRAC_BITS).astype(np.uint64)


def mass_target(p, Q: int) -> int:
    """tau = ceil(p * Q) as an exact rational, p a float32 clamped to [0, 1]."""
    p = float(np.float32(p))
    if not p > 0.0:  # also NaN
        return 0
    if p >= 1.0:
        return int(Q)
    prod = Fraction(p) * int(Q)
    return -((-prod.numerator) // prod.denominator)


def topp_count(s32: np.ndarray, p) -> int:
    """n_p of reading R15: length of the shortest prefix of the order whose
    mass units reach tau = ceil(p * Q)."""
    s32 = np.asarray(s32, dtype=_F32)
    if s32.size == 0:
        return 0
    key = order_key(s32)
    M = _F32(s32[key.argmax()])
    q = mass_units(sexp(np.subtract(s32, M, dtype=_F32)))
    order = np.lexsort((np.arange(key.size), ~key))
    cum = np.cumsum(q[order], dtype=np.uint64)  # Q < 2^24 * 2^38: no overflow
    tau = mass_target(p, int(cum[-1]))
    if tau == 0:
        return 0
    return int(np.searchsorted(cum, np.uint64(tau), side="left")) + 1


# ---------------------------------------------------------------------------
# Early stopping over the deterministic stratum ([S2O] methodology parts 2
# and 3) -- reading R17
# ---------------------------------------------------------------------------

STOP_BLOCK = 64


def stop_logits(q_rows: np.ndarray, K: np.ndarray, scale: float) -> np.ndarray:
    """Exact logits l = fl32(scale * dot) in the decision precision of R17,
    float32 [R, n] for query rows q_rows [R, d] and keys K [n, d] (both
    holding bf16 values): products of bf16 values are exact in float32; each
    8-dim slice is summed in dim order, then the d/8 slice sums pairwise
    (neighbours first), all in float32."""
    q = np.asarray(q_rows, dtype=_F32)
    k = np.asarray(K, dtype=_F32)
    R, d = q.shape
    n = k.shape[0]
    prod = q[:, None, :] * k[None, :, :]  # exact
    prod = prod.reshape(R, n, d // 8, 8)
    acc = prod[..., 0]
    for i in range(1, 8):
        acc = np.add(acc, prod[..., i], dtype=_F32)
    while acc.shape[-1] > 1:
        acc = np.add(acc[..., 0::2], acc[..., 1::2], dtype=_F32)
    return np.multiply(acc[..., 0], _F32(scale), dtype=_F32)


def stop_gains(logits: np.ndarray, visible: np.ndarray) -> np.ndarray:
    """Per-row block gains in integer units, uint64 [R, nblocks]: the stratum's
    logits [R, n] in stratum order, visible [R, n] = the token lies in the
    row's span.  A row's units are floor(2^38 sexp(l - M_r)) with M_r its
    largest visible logit; invisible tokens add nothing."""
    R, n = logits.shape
    nb = -(-n // STOP_BLOCK)
    gains = np.zeros((R, nb), np.uint64)
    for r in range(R):
        vis = np.asarray(visible[r], bool)
        if not vis.any():
            continue
        M = _F32(logits[r][vis].max())
        units = mass_units(sexp(np.subtract(logits[r], M, dtype=_F32)))
        units[~vis] = 0
        for i in range(nb):
            gains[r, i] = sum(int(x) for x in units[i * STOP_BLOCK:(i + 1) * STOP_BLOCK])
    return gains


def stop_count(gains: np.ndarray, n: int, tau) -> int:
    """Tokens of the stratum (n of them) kept by the rule: the visit stops
    after the first block at which every row's gain D is 0 or below tau times
    the row's mass C of blocks 0..i (exact rationals)."""
    tau = float(np.float32(tau))
    if not tau > 0.0 or n == 0:
        return n
    tau = Fraction(min(tau, 1.0))
    gains = np.atleast_2d(gains)
    acc = [0] * gains.shape[0]
    for i in range(gains.shape[1]):
        agree = True
        for r in range(gains.shape[0]):
            g = int(gains[r, i])
            acc[r] += g
            if g != 0 and not g < tau * acc[r]:
                agree = False
        if agree:
            return min((i + 1) * STOP_BLOCK, n)
    return n


# ---------------------------------------------------------------------------
# Step 4: counter-based uniforms (reading R8)
# ---------------------------------------------------------------------------

_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = 0x9E3779B9
_PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
    numbers: as easy as 1, 2, 3", SC'11).  Vectorised over counters.

    One round: (hi0, lo0) = M0 * c0 and (hi1, lo1) = M1 * c2 as 64-bit
    products; the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0).
    Between rounds the key is bumped by the Weyl constants (W0, W1).
    Returns four uint32 arrays.
    """
    x = [np.asarray(c, dtype=np.uint64) & _MASK32 for c in (c0, c1, c2, c3)]
    x = np.broadcast_arrays(*x)
    x = [a.copy() for a in x]
    ka, kb = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for rnd in range(10):
        p0 = _PHILOX_M0 * x[0]
        p1 = _PHILOX_M1 * x[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x = [hi1 ^ x[1] ^ np.uint64(ka), lo1, hi0 ^ x[3] ^ np.uint64(kb), lo0]
        ka = (ka + _PHILOX_W0) & 0xFFFFFFFF
        kb = (kb + _PHILOX_W1) & 0xFFFFFFFF
    return [a.astype(np.uint32) for a in x]


def philox_word(seed: int, b: int, h: int, j, grp: int = 0) -> np.ndarray:
    """The 32-bit random word of token(s) j of (batch b, kv head h, query
    group grp): counter (j >> 2, h, b, grp) (R8, R16)."""
    j = np.asarray(j, dtype=np.int64)
    words = philox4x32_10(j >> 2, np.full_like(j, h), np.full_like(j, b), np.full_like(j, grp),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    sel = (j & 3).astype(np.int64)
    stacked = np.stack(words, axis=0)
    return np.take_along_axis(stacked, sel[None, ...], axis=0)[0]


def uniforms(seed: int, b: int, h: int, j, grp: int = 0) -> np.ndarray:
    """u_j = (word >> 8) * 2^-24 as float32, in [0, 1)."""
    w = philox_word(seed, b, h, j, grp)
    return ((w >> np.uint32(8)).astype(np.float64) * 2.0 ** -24).astype(_F32)


# ---------------------------------------------------------------------------
# Steps 2-4 together: the strata of one (batch, kv head)
# ---------------------------------------------------------------------------

def tail_stratum(s32: np.ndarray, topk: int, m: int, W_in=None, top_p=None):
    """Deterministic set S, tail T and inclusion probabilities of T.

    Returns a dict with S, T (ascending int64), dense (bool), M, W (float32),
    w (float32 tail weights), mw = fl(m * w) and pi = min(1, fl(mw / W)).
    ``W_in`` replaces the computed normaliser (used to feed both
    implementations the same normaliser).  ``top_p`` (a float, or None for
    top-k alone) caps the deterministic stratum at the top-p prefix (R15).
    """
    s32 = np.asarray(s32, dtype=_F32)
    L = s32.size
    if L == 0:
        e = np.zeros(0, np.int64)
        return dict(S=e, T=e, dense=False, M=_F32(0), W=_F32(0), w=np.zeros(0, _F32),
                    mw=np.zeros(0, _F32), pi=np.zeros(0, _F32))
    M = _F32(s32[order_key(s32).argmax()])
    k = min(topk, L)
    if top_p is not None:
        k = min(k, topp_count(s32, top_p))
    if k + m >= L:  # reading R5
        e = np.zeros(0, np.int64)
        return dict(S=np.arange(L, dtype=np.int64), T=e, dense=True, M=M, W=_F32(0),
                    w=np.zeros(0, _F32), mw=np.zeros(0, _F32), pi=np.zeros(0, _F32))
    S = topk_indices(s32, k)
    in_s = np.zeros(L, bool)
    in_s[S] = True
    T = np.nonzero(~in_s)[0].astype(np.int64)
    w = sexp(np.subtract(s32[T], M, dtype=_F32))
    W = _F32(w.astype(np.float64).sum()) if W_in is None else _F32(W_in)
    mw = np.multiply(_F32(m), w, dtype=_F32)
    if W > 0:
        pi = np.minimum(_F32(1.0), np.divide(mw, W, dtype=_F32)).astype(_F32)
    else:
        pi = np.zeros_like(w)
    return dict(S=S, T=T, dense=False, M=M, W=W, w=w, mw=mw, pi=pi)


def sample_tail(strata: dict, m: int, seed: int, b: int, h: int, grp: int = 0):
    """Poisson sample of the tail (reading R7): returns (R, pi_R)."""
    T, W = strata["T"], strata["W"]
    if strata["dense"] or m == 0 or T.size == 0 or not (W > 0):
        return np.zeros(0, np.int64), np.zeros(0, _F32)
    u = uniforms(seed, b, h, T, grp)
    keep = np.multiply(u, W, dtype=_F32) < strata["mw"]
    return T[keep], strata["pi"][keep]


def select_unit(s32: np.ndarray, topk: int, m: int, seed: int, b: int, h: int, W_in=None,
                top_p=None, grp: int = 0, stop_tau=None, stop_rows=None):
    """Full selection of one (batch, [query group,] kv head): dict with S, R,
    pi_R, M, W, dense (and S_full, the stratum before early stopping).

    Early stopping (R17) needs ``stop_tau`` and ``stop_rows`` = (q_rows
    [R, d], K [L, d], spans [R], scale): the unit's query rows, its key rows
    and each row's causal length."""
    st = tail_stratum(s32, topk, m, W_in, top_p)
    R, pi_R = sample_tail(st, m, seed, b, h, grp)
    S = st["S"]
    S_full = S
    if stop_tau is not None and not st["dense"] and S.size:
        s32 = np.asarray(s32, dtype=_F32)
        order = S[np.lexsort((S, ~order_key(s32[S])))]  # key descending, index ascending
        q_rows, K, spans, scale = stop_rows
        logits = stop_logits(q_rows, K[order], scale)
        visible = order[None, :] < np.asarray(spans)[:, None]
        kept = stop_count(stop_gains(logits, visible), order.size, stop_tau)
        S = np.sort(order[:kept])
    return dict(S=S, R=R, pi_R=pi_R, M=st["M"], W=st["W"], dense=st["dense"], S_full=S_full)


# ---------------------------------------------------------------------------
# Step 5: attention over S u R with Horvitz-Thompson weights
# ([FASA] stage 2 FAC; [SSA] "How SSA stratifies the cache", correction by
# inclusion probability)
# ---------------------------------------------------------------------------

def ht_terms(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, S, R, pi_R, scale: float,
             shift):
    """Unnormalised estimator terms with a caller-given per-head shift.

    N_hat[g] = sum_{j in S} e^{l_gj - shift_g} v_j + sum_{j in R} e^{l_gj - shift_g} v_j / pi_j
    D_hat[g] = the same sums without v_j, with l_gj = scale * q_g . k_j.
    Returns (N_hat [G, d], D_hat [G]) in float64.
    """
    S = np.asarray(S, np.int64)
    R = np.asarray(R, np.int64)
    A = np.concatenate([S, R])
    c = np.concatenate([np.ones(S.size), 1.0 / np.asarray(pi_R, np.float64)])
    q = q_group.astype(np.float64)
    logits = scale * (q @ K[A].T)  # [G, |A|]
    e = c[None, :] * np.exp(logits - np.asarray(shift, np.float64)[:, None])
    return e @ V[A], e.sum(axis=1)


def attend_unit(q_group: np.ndarray, K: np.ndarray, V: np.ndarray, S, R, pi_R,
                scale: float) -> np.ndarray:
    """Normalised HT attention output of one (batch, kv head), float64 [G, d]."""
    G, d = q_group.shape
    A = np.concatenate([np.asarray(S, np.int64), np.asarray(R, np.int64)])
    if A.size == 0:
        return np.zeros((G, d))
    logits = scale * (q_group.astype(np.float64) @ K[A].T)
    shift = logits.max(axis=1)
    N, D = ht_terms(q_group, K, V, S, R, pi_R, scale, shift)
    return N / D[:, None]


# ---------------------------------------------------------------------------
# The whole decode step
# ---------------------------------------------------------------------------

def decode(q, k_cache, v_cache, block_table, seq_lens, topk, sample_budget, seed,
           pair_begin: int, pair_count: int, scale: float | None = None, units=None,
           top_p=None, stop_tau=None):
    """Stratified sparse decode attention for every (batch, kv head).

    q [B, Hq, d]; caches [num_blocks, Hkv, 16, d]; block_table [B, max_blocks];
    seq_lens, topk, sample_budget, seed: [B] integers; top_p: [B] float32 or
    None.  ``units`` optionally restricts the work to a list of (b, h) pairs
    (other outputs stay zero).
    Returns (out [B, Hq, d] float64, info dict keyed by (b, h)).
    """
    q = np.asarray(q)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, d))
    info = {}
    todo = units if units is not None else [(b, h) for b in range(B) for h in range(Hkv)]
    for b, h in todo:
        L = int(seq_lens[b])
        qg = q[b, h * G:(h + 1) * G, :].astype(np.float64)
        K = gather_rows(k_cache, block_table[b], h, L)
        V = gather_rows(v_cache, block_table[b], h, L)
        s64 = approx_scores(qg, K, pair_begin, pair_count, scale)
        s32 = s64.astype(_F32)
        tp = None if top_p is None else np.float32(top_p[b])
        sel = select_unit(s32, int(topk[b]), int(sample_budget[b]), int(seed[b]), b, h,
                          top_p=tp, stop_tau=stop_tau, stop_rows=(qg, K, [L] * G, scale))
        out[b, h * G:(h + 1) * G, :] = attend_unit(qg, K, V, sel["S"], sel["R"], sel["pi_R"], scale)
        info[(b, h)] = dict(scores=s64, **sel)
    return out, info


# ---------------------------------------------------------------------------
# Multi-query decode with a shared proxy per query group (reading R16;
# [PIVOT] "The two observations behind PIVOT", reuse mode)
# ---------------------------------------------------------------------------

def member_span(P: int, T: int, t: int) -> int:
    """Causal length of query t of T: it sits at position P - T + t (R16)."""
    return max(P - T + t + 1, 0)


def group_span(P: int, T: int, g: int, grp: int) -> int:
    """Causal length of group grp's last member: P - T + min((grp+1) g, T), >= 0."""
    return max(P - T + min((grp + 1) * g, T), 0)


def member_scores(q_member: np.ndarray, K: np.ndarray, pair_begin: int, pair_count: int,
                  scale: float) -> np.ndarray:
    """A member's own approximate score of each key row, float32 [n], in the
    decision precision of R19: per head the float32 dot over the scored dims
    (R17's summation order), summed over the G heads in head order, times
    fl32(fl32(scale) / G)."""
    dims = np.arange(2 * pair_begin, 2 * (pair_begin + pair_count))
    q = np.asarray(q_member)[:, dims]
    dots = stop_logits(q, np.asarray(K)[:, dims], 1.0)  # [G, n]
    acc = dots[0]
    for g in range(1, dots.shape[0]):
        acc = np.add(acc, dots[g], dtype=_F32)
    c = np.divide(_F32(scale), _F32(dots.shape[0]), dtype=_F32)
    return np.multiply(acc, c, dtype=_F32)


def refine_member(sel_group: dict, s32_group: np.ndarray, q_member: np.ndarray, K: np.ndarray,
                  Lt: int, topk: int, m: int, seed: int, b: int, h: int, grp: int,
                  pair_begin: int, pair_count: int, scale: float, W_in=None) -> dict:
    """Refine mode (R19): member t's own selection from the group's
    selection with candidate list C = sel_group["S"] (r * k tokens of the
    proxy order).  K holds the group span's key rows.  Returns a dict with
    S, R (samples inside the member's span), pi_R, W, dense."""
    Lg = s32_group.size
    C = np.asarray(sel_group["S"], np.int64)
    cand = C[C < Lt]
    own = member_scores(q_member, K[cand], pair_begin, pair_count, scale)
    kt = min(topk, cand.size)
    e = np.zeros(0, np.int64)
    if kt + m >= Lt:  # reading R5 for the member
        return dict(S=np.arange(Lt, dtype=np.int64), R=e, pi_R=np.zeros(0, _F32), W=_F32(0),
                    dense=True)
    order = np.lexsort((cand, ~order_key(own)))  # own score descending, index ascending
    S = np.sort(cand[order[:kt]])
    in_s = np.zeros(Lg, bool)
    in_s[S] = True
    T = np.nonzero(~in_s)[0].astype(np.int64)  # the group's span minus S_t
    w = sexp(np.subtract(np.asarray(s32_group, _F32)[T], sel_group["M"], dtype=_F32))
    W = _F32(w.astype(np.float64).sum()) if W_in is None else _F32(W_in)
    if m == 0 or T.size == 0 or not W > 0:
        return dict(S=S, R=e, pi_R=np.zeros(0, _F32), W=W, dense=False)
    mw = np.multiply(_F32(m), w, dtype=_F32)
    pi = np.minimum(_F32(1.0), np.divide(mw, W, dtype=_F32)).astype(_F32)
    u = uniforms(seed, b, h, T, grp)
    keep = (np.multiply(u, W, dtype=_F32) < mw) & (T < Lt)
    return dict(S=S, R=T[keep], pi_R=pi[keep], W=W, dense=False)


def decode_multi(q, k_cache, v_cache, block_table, seq_lens, topk, sample_budget, seed,
                 pair_begin: int, pair_count: int, query_group: int,
                 scale: float | None = None, units=None, top_p=None, stop_tau=None,
                 refine: int = 0):
    """T query positions per sequence, g = query_group per shared selection.

    q [B, T, Hq, d]; seq_lens are the cache lengths P_b (the T new tokens
    included).  ``units`` optionally restricts the work to (b, grp, h)
    triples.  With ``refine`` = r >= 1 every member refines the group's
    candidate list of r * k tokens (R19) instead of reusing its selection.
    Returns (out [B, T, Hq, d] float64, info keyed by (b, grp, h) with the
    group's scores and selection, and with refine a "members" dict keyed by
    t with each member's selection).
    """
    q = np.asarray(q)
    B, T, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    g = int(query_group)
    NG = -(-T // g)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, T, Hq, d))
    info = {}
    todo = units if units is not None else [(b, c, h) for b in range(B) for c in range(NG)
                                            for h in range(Hkv)]
    for b, c, h in todo:
        P = int(seq_lens[b])
        members = list(range(c * g, min((c + 1) * g, T)))
        Lg = group_span(P, T, g, c)
        K = gather_rows(k_cache, block_table[b], h, Lg)
        V = gather_rows(v_cache, block_table[b], h, Lg)
        # every member's query heads of this kv head, stacked: their mean is the proxy
        qstack = np.concatenate([q[b, t, h * G:(h + 1) * G, :] for t in members]).astype(np.float64)
        s64 = approx_scores(qstack, K, pair_begin, pair_count, scale)
        tp = None if top_p is None else np.float32(top_p[b])
        if refine:
            s32 = s64.astype(_F32)
            k, m = int(topk[b]), int(sample_budget[b])
            sel = select_unit(s32, int(refine) * k, m, int(seed[b]), b, h, grp=c)
            mem = {}
            for t in members:
                Lt = member_span(P, T, t)
                qg = q[b, t, h * G:(h + 1) * G, :].astype(np.float64)
                ms = refine_member(sel, s32, qg, K, Lt, k, m, int(seed[b]), b, h, c,
                                   pair_begin, pair_count, scale)
                mem[t] = ms
                out[b, t, h * G:(h + 1) * G, :] = attend_unit(qg, K[:Lt], V[:Lt], ms["S"],
                                                              ms["R"], ms["pi_R"], scale)
            info[(b, c, h)] = dict(scores=s64, span=Lg, members=mem, **sel)
            continue
        spans = [member_span(P, T, t) for t in members for _ in range(G)]
        sel = select_unit(s64.astype(_F32), int(topk[b]), int(sample_budget[b]), int(seed[b]),
                          b, h, top_p=tp, grp=c, stop_tau=stop_tau,
                          stop_rows=(qstack, K, spans, scale))
        for t in members:
            Lt = member_span(P, T, t)
            S = sel["S"][sel["S"] < Lt]
            keep = sel["R"] < Lt
            qg = q[b, t, h * G:(h + 1) * G, :].astype(np.float64)
            out[b, t, h * G:(h + 1) * G, :] = attend_unit(qg, K[:Lt], V[:Lt], S, sel["R"][keep],
                                                          sel["pi_R"][keep], scale)
        info[(b, c, h)] = dict(scores=s64, span=Lg, **sel)
    return out, info


# ---------------------------------------------------------------------------
# reading R18: split keys and appending to the cache
# ---------------------------------------------------------------------------

def split_keys(k_cache: np.ndarray, pair_begin: int, pair_count: int):
    """[FASA] section 3, variants (FASA-M: the dominant key components stay
    resident, the other components move): (k_dom, k_rest) of whole keys
    [..., d], k_dom the scored dims, k_rest the others in dim order."""
    lo, hi = 2 * pair_begin, 2 * (pair_begin + pair_count)
    k_dom = k_cache[..., lo:hi].copy()
    k_rest = np.concatenate([k_cache[..., :lo], k_cache[..., hi:]], axis=-1)
    return k_dom, k_rest


def join_keys(k_dom: np.ndarray, k_rest: np.ndarray, pair_begin: int) -> np.ndarray:
    """Whole keys from (k_dom, k_rest): the inverse of split_keys."""
    lo = 2 * pair_begin
    return np.concatenate([k_rest[..., :lo], k_dom, k_rest[..., lo:]], axis=-1)


def append_kv(k_cache: np.ndarray, v_cache: np.ndarray, block_table, seq_lens,
              k_new: np.ndarray, v_new: np.ndarray):
    """Copies of the paged caches [nblk, Hkv, 16, d] with the new tokens
    k_new, v_new [B, T, Hkv, d] written at positions seq_lens[b] - T + t
    (negative positions skipped)."""
    k, v = k_cache.copy(), v_cache.copy()
    B, T = k_new.shape[:2]
    for b in range(B):
        pos = int(seq_lens[b]) - T + np.arange(T)
        keep = pos >= 0
        blk = np.asarray(block_table[b])[pos[keep] // BLOCK_TOKENS]
        slot = pos[keep] % BLOCK_TOKENS
        k[blk, :, slot, :] = k_new[b, keep]
        v[blk, :, slot, :] = v_new[b, keep]
    return k, v
