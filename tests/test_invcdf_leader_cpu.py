"""The inverse-CDF leader's chunk search, emulated in fp32 on the CPU.

The leader wave of a row holds KPL consecutive chunk weights per lane.  It
forms an inclusive prefix of the lanes' totals with a DPP scan (shifts by 1,
2, 4 and 8 within each 16-lane row, then the two row broadcasts), and each
lane walks its chunks from its exclusive prefix.  The chosen chunk is the
first one whose running sum exceeds t = u * total (fused_markov page, module
docstring: inverse CDF in vocabulary order).  Because the lane sums and the
scan round differently, a lane whose chunks all lie past the last real chunk
(or whose chunks carry no weight) can start above t.  Such a chunk must never
be chosen: the search takes only chunks with weight, and falls back to the
last chunk with weight when rounding leaves none above t.

These tests mirror the kernel's operations in numpy float32, in the same
order, and check the rule on draws with u close to 1, where the rounding
matters.  They also show that the rule without the weight test (the old
search) picks a chunk with no weight on the same draws.
"""

import numpy as np
import pytest

F = np.float32


def dpp_incl_scan(x: np.ndarray) -> np.ndarray:
    """Inclusive scan of 64 fp32 lane values in the kernel's order."""
    x = x.astype(F).copy()
    lane = np.arange(64)
    for s in (1, 2, 4, 8):  # row_shr: lanes shifted in from outside the row add 0
        sh = np.where(lane % 16 >= s, np.roll(x, s), F(0))
        x = (x + sh).astype(F)
    row = lane // 16
    # row_bcast:15 into rows 1 and 3, then row_bcast:31 into rows 2 and 3
    add = np.zeros(64, F)
    add[row == 1] = x[15]
    add[row == 3] = x[47]
    x = (x + add).astype(F)
    add = np.zeros(64, F)
    add[row >= 2] = x[31]
    return (x + add).astype(F)


def leader_pick(w: np.ndarray, KPL: int, u: float, need_weight: bool) -> int:
    """The chunk the leader decides for weights w[NC] (zeros beyond NC)."""
    NC = len(w)
    wl = np.zeros(64 * KPL, F)
    wl[:NC] = w
    wl = wl.reshape(64, KPL)
    lsum = np.zeros(64, F)
    for k in range(KPL):  # serial per-lane sum, chunk order
        lsum = (lsum + wl[:, k]).astype(F)
    incl = dpp_incl_scan(lsum)
    total = incl[63]
    t = F(F(u) * total)
    found = np.full(64, -1)
    last = np.full(64, -1)
    run = (incl - lsum).astype(F)
    for k in range(KPL):
        wk = wl[:, k]
        hit = (found < 0) & ((run + wk).astype(F) > t)
        if need_weight:
            hit &= wk > 0
        found = np.where(hit, np.arange(64) * KPL + k, found)
        last = np.where(wk > 0, np.arange(64) * KPL + k, last)
        run = (run + wk).astype(F)
    if (found >= 0).any():
        return int(found[np.flatnonzero(found >= 0)[0]])
    return int(last[np.flatnonzero(last >= 0)[-1]])


def draws(n, seed):
    """Chunk-weight vectors and uniforms near 1 (the top of (0, 1))."""
    rng = np.random.default_rng(seed)
    for _ in range(n):
        KPL = int(rng.integers(1, 5))
        NC = int(rng.integers(2, 63 * KPL + 1))
        # chunk weights: sums of exp over a chunk rescaled to the row maximum,
        # spread over a few decades, with some chunks of -inf logits (weight 0)
        w = np.exp(rng.uniform(-6, 0, NC)).astype(F) * F(rng.uniform(1, 512))
        w[rng.random(NC) < 0.05] = 0
        w[int(rng.integers(0, NC))] = F(1 + rng.uniform(0, 511))  # the maximum's chunk
        k = int(rng.integers(0, 32))
        u = float(F((2 * ((1 << 23) - 1 - k) + 1) * 2.0**-24))
        yield w, KPL, u


def test_chosen_chunk_always_has_weight():
    picks = 0
    for w, KPL, u in draws(15000, 7):
        c = leader_pick(w, KPL, u, need_weight=True)
        assert 0 <= c < len(w) and w[c] > 0, (len(w), KPL, u, c)
        picks += 1
    assert picks == 15000


def test_old_search_picks_chunks_without_weight():
    """The same draws without the weight test: some picks land past the last
    chunk or on a chunk with no weight (this is what the weight test fixes)."""
    bad = 0
    for w, KPL, u in draws(15000, 7):
        c = leader_pick(w, KPL, u, need_weight=False)
        bad += not (c < len(w) and w[c] > 0)
    assert bad > 0


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_pick_is_the_fp64_bin_or_an_edge_neighbour(seed):
    """Away from rounding, the pick is the exact inverse-CDF bin of the
    chunk weights; any disagreement lies at a bin edge within 2^-16 of the
    total."""
    rng = np.random.default_rng(seed)
    for w, KPL, _ in draws(3000, seed):
        u = float(F((2 * int(rng.integers(0, 1 << 23)) + 1) * 2.0**-24))
        c = leader_pick(w, KPL, u, need_weight=True)
        cdf = np.cumsum(w.astype(np.float64))
        t = u * cdf[-1]
        k = int(np.searchsorted(cdf, t, side="right"))
        k = min(k, len(w) - 1)
        while w[k] == 0:  # the exact rule's last chunk with weight
            k -= 1
        if c != k:
            lo, hi = min(c, k), max(c, k)
            assert np.all(np.abs(cdf[lo:hi] - t) <= 2.0**-16 * cdf[-1])
