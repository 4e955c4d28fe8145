"""Host check of the indexer's tile indexing (no GPU).

The indexer stages a tile's block ids in LDS (at most 8192 tokens = 512
ids) and each lane group of a wave iteration reads the id of the 16-token
block holding its first token.  This walks the kernel's iteration scheme
(waves of 64 lanes, LPT lanes per token, 8 tokens per lane group, four waves
per workgroup, full iterations then one ragged one) over every ragged tile
length and checks that every LDS index a lane forms lies inside the tile's
ids, including lane groups that start past the tile's end.
"""

import pytest

MAX_TILE = 8192
BLOCK = 16
WAVES = 4


def lds_indices(n, lpt):
    """Every block-id index a lane group forms for a tile of n tokens."""
    tpi = 64 // lpt
    wave_tok = tpi * 8
    wg_tok = WAVES * wave_tok
    t0, t_end = 0, n
    out = []
    for wave in range(WAVES):
        base = t0 + wave * wave_tok
        n_full = (t_end - wave_tok - base) // wg_tok + 1 if base + wave_tok <= t_end else 0
        for _ in range(n_full):
            for grp in range(tpi):
                tg = base + 8 * grp
                assert tg + 7 < t_end
                out.append((tg - t0) >> 4)
            base += wg_tok
        if base < t_end:
            for grp in range(tpi):
                tg = base + 8 * grp
                out.append((tg - t0) >> 4 if tg < t_end else 0)
    return out


@pytest.mark.parametrize("lpt", [1, 2, 4, 8, 16])
def test_block_id_index_in_tile(lpt):
    for n in list(range(1, 700)) + list(range(MAX_TILE - 700, MAX_TILE + 1)):
        nblk = (n + BLOCK - 1) // BLOCK
        idx = lds_indices(n, lpt)
        assert min(idx) >= 0 and max(idx) < nblk <= MAX_TILE // BLOCK, (lpt, n)


def test_unclamped_index_would_read_stale_ids():
    """Without the clamp, lane groups past a ragged tile's end would read ids
    beyond those staged for the tile (left over from an earlier tile; still
    inside the 512-entry array, since tiles hold at most 8192 tokens)."""
    stale = False
    for n in range(1, MAX_TILE + 1):
        nblk = (n + BLOCK - 1) // BLOCK
        tpi = 64 // 8
        wave_tok = tpi * 8
        for wave in range(WAVES):
            base = wave * wave_tok
            n_full = (n - wave_tok - base) // (WAVES * wave_tok) + 1 if base + wave_tok <= n else 0
            base += n_full * WAVES * wave_tok
            if base < n:
                top = (base + 8 * (tpi - 1)) >> 4
                assert top < MAX_TILE // BLOCK
                stale |= top >= nblk
    assert stale
