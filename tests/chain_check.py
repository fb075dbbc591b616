"""Comparison of a chain call's outputs with the CPU oracle.

The walk follows each row position by position with the oracle's own
tokens.  At every position it checks:
  * cache: the same NaN-ness, and every value within the bound the bias
    tolerance implies.  The device bias is an fp32 sum rounded to bf16, the
    oracle's the exact sum rounded once; `bias_tolerance` bounds their
    difference (one bf16 spacing, plus the fp32 accumulation error, which
    only matters where the sum nearly cancels).  x = base + bias then moves
    by at most that times |multiplier| (the soft cap's slope is at most 1),
    and each side rounds x to bf16 once:
    |c_dev - c_orc| <= tol(bias) |mult| + ulp(c).  Where base and bias nearly
    cancel this exceeds one ulp of the tiny c, so "one bf16 ulp" alone would
    be the wrong test.  Exact and within-one-ulp counts are reported;
  * token: equal to the oracle's.  A different token is accepted only when
    the device's own cache explains it (the device token is what the
    sampling rule gives on the device cache, evaluated here in the same fp32
    precision), the two caches differ, and the oracle's decision margin is
    within what those cache differences can move.  The walk then goes on
    teacher-forced: the oracle's next position starts from the device's
    token, as the device's did, so every later position is still compared.
For the inverse CDF, a draw whose u * S falls within WINDOW * S of a bin
edge may also land in the neighbouring bin (fp32 partial sums on the device,
fp64 on the oracle).
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np

import oracle

# fp32 blockwise sums of exp: a few dozen roundings of 2^-24 relative to S,
# bounded well inside 2^-16 (see the derivation in the design notes).
WINDOW = 2.0**-16


def f32(bits):
    return oracle.bf16_to_f32(bits)


def ordinal(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns on a monotone integer line (+0 and -0 both 0)."""
    b = bits.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_spacing(x: np.ndarray) -> np.ndarray:
    """Gap from |x| to the next larger bf16 value (2^-133 at least)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, -126.0), -126.0)
    return np.exp2(e - 7)


def bias_tolerance(bias_o_bits: np.ndarray, abs_dot: np.ndarray, r: int) -> np.ndarray:
    """Largest |bias_dev - bias_orc| allowed per element.

    bias_orc = bf16(S) for the exact sum S; bias_dev = bf16(S_dev) for an fp32
    accumulation of the r exact products, |S_dev - S| <= E = r 2^-24 sum|h e|
    (the recursive-summation bound; abs_dot = sum_k |h_vk e_k|).  The two
    roundings add at most half a bf16 spacing each at magnitude
    max(|S|, |S_dev|) <= |bias_orc| + spacing/2 + E, so the difference is at
    most spacing(|bias_orc| + spacing(bias_orc)/2 + E) + E: one bf16 ulp
    unless the sum nearly cancels."""
    b = np.abs(f32(bias_o_bits).astype(np.float64))
    E = r * 2.0**-24 * np.asarray(abs_dot, dtype=np.float64)
    return bf16_spacing(b + 0.5 * bf16_spacing(b) + E) + E


class AbsDot:
    """sum_k |head[v, k] * embed[p, k]| for every v (the scale of the fp32
    accumulation error), with |head| converted once."""

    def __init__(self, w):
        self.abs_head = np.abs(f32(w.head[:w.V]))
        self.abs_embed = np.abs(f32(w.embed))

    def __call__(self, p: int) -> np.ndarray:
        # an fp32 sum of r <= 512 positive terms is within r 2^-24 < 2^-10 of
        # its exact value, so the inflated result is an upper bound
        return (self.abs_head @ self.abs_embed[p]).astype(np.float64) * (1.0 + 2.0**-10)


def is_nan_bits(bits: np.ndarray) -> np.ndarray:
    return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)


def cache_values(c: np.ndarray) -> np.ndarray:
    """Cache values as float32: bf16 bit patterns (uint16) widened, fp32
    caches as they are."""
    return f32(c) if c.dtype == np.uint16 else np.asarray(c, dtype=np.float32)


def cache_ordinal(c: np.ndarray) -> np.ndarray:
    """Cache values on a monotone integer line in units of the cache type's
    ulp (+0 and -0 both 0)."""
    if c.dtype == np.uint16:
        return ordinal(c)
    b = np.asarray(c, dtype=np.float32).view(np.int32).astype(np.int64)
    mag = b & 0x7FFFFFFF
    return np.where(b < 0, -mag, mag)


def cache_spacing(c: np.ndarray, mag: np.ndarray) -> np.ndarray:
    """One ulp of the cache type at magnitude mag: a bf16 spacing, or for an
    fp32 cache four fp32 spacings (its roundings of x, x * mult and the soft
    cap, and the two libraries' tanhf, each within an ulp or two)."""
    if c.dtype == np.uint16:
        return bf16_spacing(mag)
    return 4.0 * np.spacing(np.asarray(mag, dtype=np.float32)).astype(np.float64)


def pick_max(s: np.ndarray) -> int:
    """Lowest NaN index, else lowest index of the maximum (numpy argmax
    returns the first NaN or the first maximum)."""
    return int(np.argmax(s))


def scores(c_bits, T, g):
    cf = cache_values(c_bits)
    if T > 0:
        s = cf / np.float32(T)
        if g is not None:
            s = s + g
        return s.astype(np.float32)
    return cf.astype(np.float32)


def inv_cdf_bin(c_bits, T, u):
    """(bin, cdf, t) of the fp64 inverse CDF of softmax(f32(c) / T)."""
    z = (cache_values(c_bits) / np.float32(T)).astype(np.float64)
    e = np.exp(z - z.max())
    cdf = np.cumsum(e)
    t = float(u) * cdf[-1]
    k = int(np.searchsorted(cdf, t, side="right"))
    return min(k, len(cdf) - 1), cdf, t


@dataclasses.dataclass
class Stats:
    pairs: int = 0
    token_match: int = 0
    mismatches: list = dataclasses.field(default_factory=list)
    cache_elems: int = 0
    cache_exact: int = 0
    cache_one_ulp: int = 0
    walked_rows: int = 0

    @property
    def cache_beyond_1ulp(self) -> int:
        return self.cache_elems - self.cache_one_ulp

    def merge(self, o: "Stats") -> None:
        self.pairs += o.pairs
        self.token_match += o.token_match
        self.mismatches += o.mismatches
        self.cache_elems += o.cache_elems
        self.cache_exact += o.cache_exact
        self.cache_one_ulp += o.cache_one_ulp
        self.walked_rows += o.walked_rows

    def summary(self) -> str:
        return (f"pairs={self.pairs} token_match={self.token_match} "
                f"mismatch={len(self.mismatches)} cache_exact={self.cache_exact}/{self.cache_elems} "
                f"within_1ulp={self.cache_one_ulp} beyond_1ulp={self.cache_beyond_1ulp}")


def record(name: str, st: "Stats | None", **extra) -> None:
    """Append the counts of a parity check as one JSON line to the file named
    by MARKOV_PARITY_LOG, if set (the parity figures quoted in the design
    notes come from these lines)."""
    path = os.environ.get("MARKOV_PARITY_LOG")
    if not path:
        return
    import json
    line = {"check": name}
    if st is not None:
        line.update(pairs=st.pairs, token_match=st.token_match, mismatches=len(st.mismatches),
                    cache_elems=st.cache_elems, cache_exact=st.cache_exact,
                    cache_beyond_1ulp=st.cache_beyond_1ulp, walked_rows=st.walked_rows)
    line.update(extra)
    with open(path, "a") as f:
        f.write(json.dumps(line) + "\n")


def walk(w, tok_gpu, cache_gpu, gumbel, rows=None, exact=False, workers=None, absdot=None) -> Stats:
    """Walk `rows` (default: all) of workload w; gumbel[rows, N, V] is the
    noise both sides used (mode 0).  exact=True demands bit-identical caches
    and tokens.  Rows are walked in parallel threads (the oracle's C calls
    release the interpreter lock)."""
    sidx = np.arange(w.rows) if w.state_idx is None else w.state_idx
    rows = [b for b in (range(w.rows) if rows is None else rows) if int(sidx[b]) >= 0]
    if absdot is None and not exact:
        absdot = AbsDot(w)
    st = Stats()
    if workers is None:
        workers = min(16, os.cpu_count() or 1, max(1, len(rows)))
    if workers <= 1:
        for b in rows:
            st.merge(_walk_row(w, b, int(sidx[b]), tok_gpu, cache_gpu, gumbel, exact, absdot))
        return st
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(_walk_row, w, b, int(sidx[b]), tok_gpu, cache_gpu, gumbel, exact, absdot)
                for b in rows]
        for f in futs:
            st.merge(f.result())
    return st


def _walk_row(w, b, s, tok_gpu, cache_gpu, gumbel, exact, absdot) -> Stats:
    """One row of `walk` (state index s >= 0)."""
    st = Stats()
    V = w.V
    st.walked_rows += 1
    p = int(w.prev[b])
    T = float(w.temperature[b])
    for i in range(w.N):
        g = gumbel[b, i] if (w.mode == 0 and gumbel is not None) else None
        u = oracle.uniform(oracle.hash_step(int(w.seeds[b]), b, i)) if w.mode == 1 else 0.0
        tok_o, c_o, diag, bias_o = oracle.step(w.base[b, i], w.head, w.embed, p, T, g, u=u,
                                               mult=w.mult, cap=w.cap, mode=w.mode,
                                               with_diag=True, with_bias=True,
                                               cache_f32=w.cache_f32)
        c_g = cache_gpu[s, i, :V]
        nan_o, nan_g = np.isnan(cache_values(c_o)), np.isnan(cache_values(c_g))
        assert np.array_equal(nan_o, nan_g), f"row {b} step {i}: NaN positions differ"
        d = np.abs(cache_ordinal(c_o) - cache_ordinal(c_g))
        d[nan_o] = 0
        st.cache_elems += V
        same = (d == 0)
        st.cache_exact += int(same.sum())
        st.cache_one_ulp += int((d <= 1).sum())
        if exact:
            assert same.all(), f"row {b} step {i}: {int((~same).sum())} cache elements differ"
        else:
            fo = cache_values(c_o).astype(np.float64)
            fg = cache_values(c_g).astype(np.float64)
            fin = ~nan_o & np.isfinite(fo) & np.isfinite(fg)
            assert np.array_equal(fo[~nan_o & ~fin], fg[~nan_o & ~fin]), f"row {b} step {i}: infinities differ"
            tol_bias = bias_tolerance(bias_o, absdot(p), w.r)
            bound = (tol_bias * abs(w.mult)
                     + cache_spacing(c_o, np.maximum(np.abs(fo), np.abs(fg))))
            bad = fin & (np.abs(fo - fg) > bound)
            assert not bad.any(), (f"row {b} step {i}: {int(bad.sum())} cache values beyond the "
                                   f"bias-implied bound, e.g. v={int(np.flatnonzero(bad)[0])}")
        t_g = int(tok_gpu[b, i])
        st.pairs += 1
        if t_g == tok_o:
            st.token_match += 1
            p = tok_o
            continue
        assert not exact, f"row {b} step {i}: token {t_g} != oracle {tok_o}"
        assert 0 <= t_g < V, f"row {b} step {i}: token {t_g} out of range"
        caches_differ = not same.all()
        if w.mode == 0 or T <= 0 or diag[3] == 1.0:
            # Argmax-type decision: the device token must be the rule's
            # pick on the device cache (+ the same noise), and the oracle's
            # margin must be within the score change the cache moved.
            s_g = scores(c_g, T, g if w.mode == 0 else None)
            s_o = scores(c_o, T, g if w.mode == 0 else None)
            assert t_g == pick_max(s_g), f"row {b} step {i}: device token is not its own argmax"
            assert caches_differ, f"row {b} step {i}: identical caches but tokens differ"
            moved = abs(float(s_o[tok_o]) - float(s_g[tok_o])) + abs(float(s_o[t_g]) - float(s_g[t_g]))
            margin = float(diag[0]) - float(s_o[t_g])
            assert margin <= moved + 1e-12, f"row {b} step {i}: margin {margin} > moved {moved}"
        else:
            k_g, cdf, t = inv_cdf_bin(c_g, T, u)
            if t_g != k_g:
                # every edge between the two bins lies within the window of u*S
                lo, hi = min(t_g, k_g), max(t_g, k_g)
                edges = cdf[lo:hi]
                assert np.all(np.abs(t - edges) <= WINDOW * cdf[-1]), \
                    f"row {b} step {i}: device bin {t_g} vs its own cache's {k_g}"
            assert caches_differ or diag[2] <= WINDOW, \
                f"row {b} step {i}: identical caches, bin {t_g} vs {tok_o}, edge distance {diag[2]}"
        st.mismatches.append((b, i, tok_o, t_g))
        # teacher-forced: the device's next position started from its
        # own token, so the oracle's does too
        p = t_g
    return st
