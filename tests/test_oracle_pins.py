"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a library routine, a published test
vector, a closed form, an invariant of the method or brute force, chosen so
that a plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a rounding done twice) fails at least one of them.
All of these run on the CPU.
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from markov_bias_chain_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def bf16(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float32))


def f32(bits):
    return oracle.bf16_to_f32(bits)


# --------------------------------------------------------------- bfloat16 --

def test_bf16_round_f32_exhaustive_vs_torch():
    """Every fp32 bit pattern rounds like torch's float32 -> bfloat16 cast
    (NaN: only NaN-ness is compared)."""
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        ours = oracle.bf16_round_f32(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(x)
        assert np.array_equal(ours[~nan], ref[~nan]), hex(start)
        assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


@pytest.mark.parametrize("x,bits", [
    (1.0 + 2.0**-8, 0x3F80),                 # halfway: ties to even (down)
    (1.0 + 3 * 2.0**-8, 0x3F82),             # halfway: ties to even (up)
    (1.0 + 2.0**-8 + 2.0**-30, 0x3F81),      # just above halfway: one rounding, not via fp32
    (1.0 + 2.0**-8 - 2.0**-60, 0x3F80),      # just below halfway
    (-(1.0 + 2.0**-8 + 2.0**-30), 0xBF81),
    (2.0**-133, 0x0001),                     # smallest subnormal
    (2.0**-134, 0x0000),                     # halfway to zero: even
    (3 * 2.0**-134, 0x0002),                 # halfway between 1 and 2 quanta: even
    (2.0**-126, 0x0080),                     # smallest normal
    ((2 - 2.0**-7) * 2.0**127, 0x7F7F),      # largest finite
    ((2 - 2.0**-8) * 2.0**127, 0x7F80),      # halfway to 2^128: overflows
    (-0.0, 0x8000),
    (0.0, 0x0000),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
    (float("nan"), 0x7FC0),
])
def test_bf16_round_f64_one_step(x, bits):
    assert oracle.bf16_round_f64(x) == bits


# ----------------------------------------------------------- SplitMix64 ---

def _golden_splitmix():
    rows = []
    with open(os.path.join(GOLDEN, "splitmix64.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            seed, outs = line.split(":")
            rows.append((int(seed), [int(o, 0) for o in outs.split()]))
    return rows


def test_splitmix64_published_vectors():
    for seed, outs in _golden_splitmix():
        for n, expect in enumerate(outs, start=1):
            assert oracle.splitmix64((seed + (n - 1) * GAMMA) & M64) == expect


def test_splitmix64_mix_is_a_bijection():
    """Undo the finaliser with its algebraic inverse (xor-shift inverses and
    the modular inverses of the odd multipliers): a collision-free map, so
    distinct vocab ids never share a hash for one (seed, row, step)."""
    c1, c2 = 0xBF58476D1CE4E5B9, 0x94D049BB133111EB
    i1, i2 = pow(c1, -1, 1 << 64), pow(c2, -1, 1 << 64)

    def unxorshift(z, s):
        x = z
        for _ in range(64 // s + 1):
            x = z ^ (x >> s)
        return x & M64

    rng = np.random.default_rng(1)
    for z in [0, 1, M64, GAMMA] + [int(v) for v in rng.integers(0, 2**63, 200)]:
        y = oracle.splitmix64_mix(z)
        x = unxorshift(y, 31)
        x = (x * i2) & M64
        x = unxorshift(x, 27)
        x = (x * i1) & M64
        x = unxorshift(x, 30)
        assert x == z


def test_hash_is_keyed_by_every_counter():
    """Changing any of seed, row, step or the vocab id changes the draw."""
    base = oracle.hash_vocab(oracle.hash_step(7, 3, 2), 11)
    assert oracle.hash_vocab(oracle.hash_step(8, 3, 2), 11) != base
    assert oracle.hash_vocab(oracle.hash_step(7, 4, 2), 11) != base
    assert oracle.hash_vocab(oracle.hash_step(7, 3, 1), 11) != base
    assert oracle.hash_vocab(oracle.hash_step(7, 3, 2), 12) != base
    # negative seeds use the int64 bits as uint64
    assert oracle.hash_step(-1, 0, 0) == oracle.hash_step(-1, 0, 0)


# -------------------------------------------------------------- uniforms --

def test_uniform_exact_form_and_open_interval():
    rng = np.random.default_rng(2)
    hs = [0, M64, 1 << 41, (1 << 41) - 1] + [int(v) for v in rng.integers(0, 2**63, 500)]
    for h in hs:
        u = oracle.uniform(h)
        assert Fraction(u) == Fraction(2 * (h >> 41) + 1, 1 << 24)
        assert 0.0 < u < 1.0
    assert oracle.uniform(0) == 2.0**-24
    assert oracle.uniform(M64) == 1.0 - 2.0**-24


def test_uniform_chi_square_2pow16_bins():
    n = 10_000_000
    u = oracle.uniform_range(12345, 0, 0, 0, n).astype(np.float64)
    counts = np.bincount((u * 65536).astype(np.int64), minlength=65536)
    exp = n / 65536
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    df = 65535
    assert abs(chi2 - df) < 5 * math.sqrt(2 * df), chi2


def test_gumbel_moments_closed_form():
    """Mean of a standard Gumbel is the Euler-Mascheroni constant, variance
    pi^2/6 (5 standard errors at 10^7 draws)."""
    g = oracle.noise_fill(np.array([99], dtype=np.int64), 1, 10_000_000).astype(np.float64).ravel()
    n = g.size
    euler_gamma = 0.5772156649015329
    var = math.pi**2 / 6
    assert abs(g.mean() - euler_gamma) < 5 * math.sqrt(var / n)
    # Var(s^2) = sigma^4 (excess kurtosis + 2) / n, excess kurtosis 12/5
    assert abs(g.var() - var) < 5 * math.sqrt(var**2 * (2.4 + 2) / n)


def test_noise_fill_matches_per_element_hash():
    seeds = np.array([5, -3], dtype=np.int64)
    g = oracle.noise_fill(seeds, 3, 40)
    for row in range(2):
        for i in range(3):
            p = oracle.hash_step(int(seeds[row]), row, i)
            for v in (0, 1, 17, 39):
                u = oracle.uniform(oracle.hash_vocab(p, v))
                # each fp32 log is the correctly rounded one (fp64 log, one rounding)
                inner = np.float32(math.log(u))
                assert g[row, i, v] == -np.float32(math.log(-inner))


# ------------------------------------------------------------------ bias --

def test_bias_exact_on_integer_weights():
    """With head = k*2^-6 integers, base = 0 and no transform the cache holds
    bf16(exact integer dot product * 2^-12): checked with numpy int64 matmul
    and torch's cast."""
    w = synth.make("t", 512, 256, 1, 1, seed=11, weights="int", base_std=0.0)
    kh = (f32(w.head) * 64).astype(np.int64)
    ke = (f32(w.embed) * 64).astype(np.int64)
    base0 = np.zeros(512, dtype=np.uint16)
    for prev in (0, 7, 511):
        _, cache = oracle.step(base0, w.head, w.embed, prev, 1.0, np.zeros(512, np.float32))
        exact = (kh @ ke[prev]).astype(np.float32) * np.float32(2.0**-12)  # exact in fp32
        assert np.array_equal(cache, bf16(exact + np.float32(0.0)))


def test_bias_random_weights_vs_blas():
    """Random N(0, 0.02) weights: the oracle's bias (exact sum, one rounding)
    agrees with a BLAS fp64 product rounded through fp32, to within one bf16
    ulp everywhere and exactly almost everywhere."""
    w = synth.make("t", 4096, 256, 1, 1, seed=12, base_std=0.0)
    H = f32(w.head).astype(np.float64)
    E = f32(w.embed).astype(np.float64)
    base0 = np.zeros(4096, dtype=np.uint16)
    prev = 123
    _, cache = oracle.step(base0, w.head, w.embed, prev, 1.0, np.zeros(4096, np.float32))
    ref = bf16((H @ E[prev]).astype(np.float32))
    ours = cache.astype(np.int32)
    diff = np.abs(ours - ref.astype(np.int32))
    # +0 / -0 for exactly cancelling sums are equal values
    same_value = f32(cache) == f32(ref)
    assert np.all(same_value | (diff <= 1))
    assert same_value.mean() > 0.999


def test_transform_matches_torch_fp32_ops():
    """Multiplier then soft cap, in fp32 as torch orders it, with one bf16
    rounding at the end (base = value, head = 0 so bias = 0)."""
    V = 4096
    rng = np.random.default_rng(3)
    base = bf16(rng.standard_normal(V).astype(np.float32) * 40)
    head = np.zeros((V, 16), dtype=np.uint16)
    embed = bf16(rng.standard_normal((V, 16)).astype(np.float32))
    mult, cap = np.float32(0.5), np.float32(30.0)
    _, cache = oracle.step(base, head, embed, 0, 1.0, np.zeros(V, np.float32),
                           mult=float(mult), cap=float(cap))
    x = torch.from_numpy(f32(base).copy()) * float(mult)
    inv = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(float(cap), dtype=torch.float32)
    x = torch.tanh(x * inv) * float(cap)
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    d = np.abs(cache.astype(np.int32) - ref.astype(np.int32))
    assert d.max() <= 1  # tanhf of two libms may differ in the last fp32 bit
    assert (d == 0).mean() > 0.999
    # no cap and no multiplier: the cache is base + bias exactly
    _, c2 = oracle.step(base, head, embed, 0, 1.0, np.zeros(V, np.float32))
    assert np.array_equal(c2, base)


# -------------------------------------------------------- argmax and ties --

def _flat_step(values, T=0.0, gumbel=None, mode=0, u=0.5):
    """One step with head = 0, so the cache is the given bf16 values."""
    vals = np.asarray(values, dtype=np.float32)
    V = vals.size
    base = bf16(vals)
    head = np.zeros((V, 16), dtype=np.uint16)
    embed = np.zeros((V, 16), dtype=np.uint16)
    g = np.zeros(V, np.float32) if gumbel is None else np.asarray(gumbel, np.float32)
    return oracle.step(base, head, embed, 0, T, g, u=u, mode=mode)[0]


nan, inf = float("nan"), float("inf")


@pytest.mark.parametrize("vals,expect", [
    ([1, 3, 2, 3], 1),            # two equal maxima: the lower id
    ([1, nan, 9, nan], 1),        # NaN at j < k: j
    ([9, 1, nan], 2),             # a NaN beats a larger value
    ([-0.0, 0.0, -1], 0),         # -0 and +0 are equal: the lower id
    ([0.0, -0.0, -1], 0),
    ([inf, 1, inf], 0),           # +inf ties: the lowest
    ([-inf, -inf, -inf], 0),      # all -inf: the lowest
])
@pytest.mark.parametrize("mode", [0, 1])
def test_tie_and_nan_rules(vals, expect, mode):
    assert _flat_step(vals, T=0.0, mode=mode) == expect


@pytest.mark.parametrize("vals,expect", [
    ([1, nan, 9, nan], 1),
    ([inf, 1, inf], 0),
])
def test_nan_and_inf_rules_under_temperature(vals, expect):
    # mode 0 with noise, and mode 1: NaN / +inf decide before any sampling
    assert _flat_step(vals, T=0.7, gumbel=[0.3, -2, 5, 1][: len(vals)]) == expect
    assert _flat_step(vals, T=0.7, mode=1, u=0.999) == expect


def test_greedy_is_argmax_of_cache():
    w = synth.make("t", 2048, 256, 3, 5, seed=13, temperature=0.0)
    toks, cache = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds)
    ref = torch.argmax(torch.from_numpy(f32(cache)), dim=-1).numpy()
    assert np.array_equal(toks, ref)


def test_zero_head_reduces_to_per_step_argmax():
    """head = 0 makes the bias 0: every step is torch.argmax of its base
    logits, whatever the previous token."""
    w = synth.make("t", 3000, 256, 2, 6, seed=14, weights="zero", temperature=0.0)
    toks, _ = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds)
    ref = torch.argmax(torch.from_numpy(f32(w.base)), dim=-1).numpy()
    assert np.array_equal(toks, ref)


def test_gumbel_max_with_given_noise_is_argmax_of_scores():
    """Mode 0 draws argmax(cache / T + gumbel) with fp32 division."""
    w = synth.make("t", 1024, 256, 1, 1, seed=15, temperature=0.7)
    g = oracle.noise_fill(w.seeds, 1, 1024)
    tok, cache = oracle.step(w.base[0, 0], w.head, w.embed, int(w.prev[0]), 0.7, g[0, 0])
    s = torch.from_numpy(f32(cache)) / torch.tensor(0.7, dtype=torch.float32) + torch.from_numpy(g[0, 0])
    assert tok == int(torch.argmax(s))


# ------------------------------------------------------- sampling laws ---

def _chi2(counts, probs):
    n = counts.sum()
    exp = n * probs
    return float(((counts - exp) ** 2 / exp).sum())


def _softmax64(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max())
    return e / e.sum()


@pytest.mark.parametrize("mode", [0, 1])
def test_sampling_law_chi_square_v16(mode):
    """V=16, head = 0 (independent steps), logits 0.25 j - 2, T = 1:
    10^5 draws against the exact softmax (df 15, p = 1e-3 critical 37.70)."""
    V, rows, N = 16, 100, 1000
    logits = (0.25 * np.arange(V) - 2).astype(np.float32)
    base = np.broadcast_to(bf16(logits), (rows, N, V)).copy()
    head = np.zeros((V, 16), dtype=np.uint16)
    embed = np.zeros((V, 16), dtype=np.uint16)
    seeds = np.arange(rows, dtype=np.int64) * 7919 + 1
    toks, _ = oracle.chain(base, head, embed, np.zeros(rows, np.int64),
                           np.ones(rows, np.float32), seeds, mode=mode)
    counts = np.bincount(toks.ravel(), minlength=V).astype(np.float64)
    assert _chi2(counts, _softmax64(logits)) < 37.70


def test_inverse_cdf_bin_vs_numpy_searchsorted():
    """Mode 1's bin is numpy's searchsorted (side='right') of u*S in the fp64
    cumulative sum of exp(z - max z), z = cache / T."""
    rng = np.random.default_rng(4)
    for trial in range(200):
        V = int(rng.integers(2, 17))
        vals = rng.standard_normal(V).astype(np.float32) * 3
        T = np.float32(rng.choice([0.6, 1.0, 1.5]))
        u = float(rng.integers(1, 2**23) * 2 - 1) * 2.0**-24
        tok = _flat_step(vals, T=float(T), mode=1, u=u)
        z = (torch.from_numpy(f32(bf16(vals)).copy()) / torch.tensor(float(T))).numpy().astype(np.float64)
        cdf = np.cumsum(np.exp(z - z.max()))
        k = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
        assert tok == min(k, V - 1)


def test_inverse_cdf_small_temperature_is_argmax():
    rng = np.random.default_rng(5)
    for _ in range(50):
        vals = rng.permutation(np.arange(16, dtype=np.float32) * 0.5)
        for u in (2.0**-24, 0.5, 1 - 2.0**-24):
            assert _flat_step(vals, T=1e-3, mode=1, u=u) == int(np.argmax(vals))


def test_chain_property_no_look_ahead():
    """Perturbing base logits or noise at steps > i leaves tokens and cache
    of steps <= i unchanged."""
    w = synth.make("t", 1024, 256, 2, 6, seed=16, temperature=1.0)
    g = oracle.noise_fill(w.seeds, 6, 1024)
    t0, c0 = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    for i in range(5):
        b2, g2 = w.base.copy(), g.copy()
        b2[:, i + 1:] = bf16(np.random.default_rng(i).standard_normal(b2[:, i + 1:].shape).astype(np.float32))
        g2[:, i + 1:] = -g2[:, i + 1:]
        t1, c1 = oracle.chain(b2, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g2)
        assert np.array_equal(t0[:, : i + 1], t1[:, : i + 1])
        assert np.array_equal(c0[:, : i + 1], c1[:, : i + 1])


def test_free_running_noise_equals_noise_fill():
    w = synth.make("t", 777, 256, 3, 4, seed=17, temperature=[0.6, 1.0, 1.5])
    g = oracle.noise_fill(w.seeds, 4, 777)
    a = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds)
    b = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _brute_force_law(w, T, prev0):
    """Exact joint law of all V^N paths from independently computed cache
    rows: integer weights make bias and cache exact in numpy/torch."""
    V, N = w.V, w.N
    kh = (f32(w.head) * 64).astype(np.int64)
    ke = (f32(w.embed) * 64).astype(np.int64)

    def cache_row(i, p):
        bias = bf16((kh @ ke[p]).astype(np.float32) * np.float32(2.0**-12))
        x = f32(w.base[0, i]) + f32(bias)
        return f32(bf16(x))

    law = {}

    def walk(i, p, prob, path):
        if i == N:
            law[tuple(path)] = prob
            return
        c = (torch.from_numpy(cache_row(i, p).copy()) / torch.tensor(T, dtype=torch.float32)).numpy()
        pr = _softmax64(c)
        for q in range(V):
            walk(i + 1, q, prob * pr[q], path + [q])

    walk(0, prev0, 1.0, [])
    return law


@pytest.mark.parametrize("mode", [0, 1])
def test_brute_force_joint_law_of_paths(mode):
    """V=4, N=3: the oracle's path frequencies over 10^5 seeds follow the
    exact product of per-step softmaxes (chi-square over the 64 paths)."""
    V, N, r = 4, 3, 16
    w = synth.make("t", V, r, 1, N, seed=18, weights="int", base_std=1.0)
    # larger integer weights so the bias matters: k * 2^-6 scaled by 16
    w.head = bf16(f32(w.head) * 16)
    w.embed = bf16(f32(w.embed) * 16)
    law = _brute_force_law(w, 1.0, 2)
    draws = 100_000
    base = np.broadcast_to(w.base, (draws, N, V)).copy()
    seeds = np.arange(draws, dtype=np.int64) * 104729 + 3
    toks, _ = oracle.chain(base, w.head, w.embed, np.full(draws, 2, np.int64),
                           np.ones(draws, np.float32), seeds, mode=mode)
    idx = toks[:, 0] * 16 + toks[:, 1] * 4 + toks[:, 2]
    counts = np.bincount(idx, minlength=64).astype(np.float64)
    probs = np.array([law[(a, b, c)] for a in range(4) for b in range(4) for c in range(4)])
    assert abs(probs.sum() - 1) < 1e-12
    # df = 63: p = 1e-3 critical value 103.44
    assert _chi2(counts, probs) < 103.44


def test_textbook_markov_chain_identity_weights():
    """r = V, head = a*I, embed = b*I, base = 0: bias = ab * onehot(prev), so
    the chain stays with probability e^(ab)/(e^(ab) + V - 1)."""
    V = 8
    a = b = 1.0
    head = bf16(np.eye(V, dtype=np.float32) * a)
    embed = bf16(np.eye(V, dtype=np.float32) * b)
    rows, N = 2000, 50
    base = np.zeros((rows, N, V), dtype=np.uint16)
    seeds = np.arange(rows, dtype=np.int64) + 1000
    prev = np.arange(rows, dtype=np.int64) % V
    toks, _ = oracle.chain(base, head, embed, prev, np.ones(rows, np.float32), seeds)
    path = np.concatenate([prev[:, None], toks], axis=1)
    stay = (path[:, 1:] == path[:, :-1]).mean()
    p_stay = math.e / (math.e + V - 1)
    n = rows * N
    assert abs(stay - p_stay) < 5 * math.sqrt(p_stay * (1 - p_stay) / n)


# ------------------------------------------------------------ row rules --

def test_padding_row_is_inert_and_states_map_cache_rows():
    w = synth.make("t", 1500, 256, 4, 3, seed=19, temperature=[0.0, 1.0, 0.6, 1.5])
    g = oracle.noise_fill(w.seeds, 3, 1500)
    sidx = np.array([2, -1, 0, 3], dtype=np.int64)
    toks = np.full((4, 3), -7, dtype=np.int64)
    cache = np.full((4, 3, 1500), 0xABCD, dtype=np.uint16)
    oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g,
                 state_idx=sidx, tokens=toks, cache=cache)
    assert np.all(toks[1] == -7)           # untouched
    assert np.all(cache[1] == 0xABCD)      # state 1 is nobody's
    ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    for row, st in ((0, 2), (2, 0), (3, 3)):
        assert np.array_equal(toks[row], ref_t[row])
        assert np.array_equal(cache[st], ref_c[row])


def test_bad_previous_token_is_reported():
    w = synth.make("t", 64, 256, 1, 1, seed=20)
    with pytest.raises(ValueError):
        oracle.chain(w.base, w.head, w.embed, np.array([64]), w.temperature, w.seeds)


# ------------------------------------------------------- element types ---
# The pages' sampler takes bf16 or fp32 base logits and a bf16 or fp32
# draft-logits cache; cache_round rounds to the cache's type, so an fp32
# cache holds x itself.

def test_fp32_base_of_bf16_values_equals_bf16_base():
    """fp32 base logits that are bf16 values give the bf16 chain exactly."""
    w = synth.make("dt", 3000, 256, 3, 4, seed=61, temperature=[0.7, 0.0, 1.0], mult=0.5, cap=30.0)
    t1, c1 = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, mult=w.mult, cap=w.cap)
    t2, c2 = oracle.chain(f32(w.base), w.head, w.embed, w.prev, w.temperature, w.seeds, mult=w.mult, cap=w.cap)
    assert np.array_equal(t1, t2) and np.array_equal(c1, c2)


def test_fp32_cache_is_base_plus_bias_and_tokens_are_argmax():
    """Closed form: with an fp32 cache and no transform, cache = fp32(base +
    f32(bias)) (numpy fp32 add) for the oracle's own bias (pinned above), and
    each token is numpy's first argmax of cache / T + gumbel (fp32 ops)."""
    V, N = 2048, 3
    w = synth.make("dt2", V, 256, 1, N, seed=62, temperature=0.6)
    rng = np.random.default_rng(63)
    base = (rng.standard_normal((1, N, V)) * 3).astype(np.float32)  # not bf16 values
    g = oracle.noise_fill(w.seeds, N, V)
    toks, cache = oracle.chain(base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g,
                               cache_f32=True)
    assert cache.dtype == np.float32
    p = int(w.prev[0])
    for i in range(N):
        _, _, bias = oracle.step(base[0, i], w.head, w.embed, p, 0.6, g[0, i], with_bias=True)
        expect = (base[0, i] + f32(bias)).astype(np.float32)
        assert np.array_equal(cache[0, i], expect)
        s = (cache[0, i] / np.float32(0.6)).astype(np.float32) + g[0, i]
        assert toks[0, i] == int(np.argmax(s))
        p = int(toks[0, i])


def test_fp32_cache_inverse_cdf_vs_searchsorted():
    """Mode 1 on an fp32 cache: numpy's searchsorted of u*S in the fp64
    cumulative exp(z - max z), z = cache / T (no bf16 rounding anywhere)."""
    V, N = 512, 4
    w = synth.make("dt3", V, 256, 1, N, seed=64, temperature=1.5, mode=1)
    rng = np.random.default_rng(65)
    base = (rng.standard_normal((1, N, V)) * 2).astype(np.float32)
    toks, cache = oracle.chain(base, w.head, w.embed, w.prev, w.temperature, w.seeds, mode=1,
                               cache_f32=True)
    for i in range(N):
        z = (cache[0, i] / np.float32(1.5)).astype(np.float32).astype(np.float64)
        cdf = np.cumsum(np.exp(z - z.max()))
        u = oracle.uniform(oracle.hash_step(int(w.seeds[0]), 0, i))
        k = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
        assert toks[0, i] == min(k, V - 1)


# ------------------------------------------- the fp32 log, correctly rounded --
# The noise's fp32 logs are defined as ln(x) correctly rounded to fp32
# (sharded_markov page, _shard_noise_kernel: fp32 noise; the reading takes
# the correctly rounded log so that two libraries agree).  These pins compute
# that value with Python's decimal module at 50 digits, independently of any
# libm, and compare the oracle's log with it bit for bit.

def _ln_rn32(x) -> np.float32:
    """ln(x) for an fp32 x > 0, correctly rounded to fp32, from a 50-digit
    decimal logarithm: the nearest of the three fp32 values around it (a
    logarithm of an fp32 value other than 1 is never an fp32 midpoint)."""
    from decimal import Decimal, localcontext
    x = np.float32(x)
    with localcontext() as ctx:
        ctx.prec = 50
        d = Decimal(float(x)).ln()
        f = np.float32(float(d))
        cands = (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf)))
        errs = [abs(Decimal(float(c)) - d) for c in cands]
    return cands[int(np.argmin(errs))]


def test_log_f32_correctly_rounded_on_sampled_noise_inputs():
    """10^5 uniforms u of the noise and their -ln u: both fp32 logs of the
    Gumbel draw equal the decimal log correctly rounded to fp32."""
    rng = np.random.default_rng(21)
    ks = rng.integers(0, 1 << 23, 100_000)
    ks[:4] = [0, 1, (1 << 23) - 1, 1 << 22]  # the extremes of u and u = 1/2 + 2^-24
    for k in ks:
        u = np.float32((2 * int(k) + 1) * 2.0**-24)
        inner = np.float32(oracle.log_f32(float(u)))
        assert inner == _ln_rn32(u), (hex(int(k)), float(u))
        y = np.float32(-inner)
        outer = np.float32(oracle.log_f32(float(y)))
        assert outer == _ln_rn32(y), (hex(int(k)), float(y))
        assert np.float32(oracle.gumbel(float(u))) == np.float32(-outer)


def test_log_f32_correctly_rounded_on_hard_inputs(tmp_path):
    """The noise inputs whose fp64 logarithm lies so close to an fp32
    rounding midpoint that the device's table-driven log leaves them to the
    library (listed by tests/noise_log_check.cpp --list over all 2^24 noise
    inputs): the oracle's log is the correctly rounded one there too."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    exe = str(tmp_path / "noise_log_check")
    subprocess.run(["g++", "-O2", "-ffp-contract=off", "-std=c++17",
                    os.path.join(os.path.dirname(__file__), "noise_log_check.cpp"), "-o", exe],
                   check=True)
    out = subprocess.run([exe, "--list"], check=True, capture_output=True, text=True).stdout.split()
    xs = np.array([int(h, 16) for h in out], dtype=np.uint32).view(np.float32)
    assert len(xs) > 50
    for x in xs:
        assert np.float32(oracle.log_f32(float(x))) == _ln_rn32(x), float(x)


# --------------------------------------------------- the hash, restated --
# DESIGN's reading of the noise hash, restated here in plain Python integers:
# sm(x) is one SplitMix64 output for state x (Steele, Lea and Flood, OOPSLA
# 2014; its finaliser constants are pinned by the published vectors above),
# the prefix absorbs seed, row and step in that order, then the global vocab
# id; the uniform is (2k + 1) 2^-24 with k the top 23 bits.

def _sm(x: int) -> int:
    z = (x + GAMMA) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _prefix(seed: int, row: int, step: int) -> int:
    h = _sm(seed & M64)
    h = _sm(h ^ (row & M64))
    return _sm(h ^ (step & M64))


@pytest.mark.parametrize("seed,row,step", [
    (0, 0, 0), (1, 0, 0), (-1, 0, 0), (-(2**63), 5, 7), (2**63 - 1, 63, 255),
    (0x4D41524B02, 3, 1), (-123456789, 4095, 15), (42, 1, 2), (42, 2, 1),
])
def test_hash_and_uniform_restated_in_python_integers(seed, row, step):
    h2 = _prefix(seed, row, step)
    assert oracle.hash_step(seed, row, step) == h2
    assert Fraction(oracle.uniform(h2)) == Fraction(2 * (h2 >> 41) + 1, 1 << 24)
    for v in (0, 1, 15, 16, 4095, 129279, 262143, (1 << 24) - 1):
        h3 = _sm(h2 ^ v)
        assert oracle.hash_vocab(h2, v) == h3
        assert Fraction(oracle.uniform(h3)) == Fraction(2 * (h3 >> 41) + 1, 1 << 24)
    # the noise of a small row, element by element
    g = oracle.noise_fill(np.array([seed], dtype=np.int64), step + 1, 16)[0, step]
    for v in range(16):
        u = np.float32((2 * (_sm(_prefix(seed, 0, step) ^ v) >> 41) + 1) * 2.0**-24)
        assert g[v] == -_ln_rn32(-_ln_rn32(u))


# ------------------------------------------------------ diagnostics pins --
# The oracle's diagnostics (used by the parity walk to explain a device token
# that differs from the oracle's) on hand-built vectors whose answers are
# exact: a zero head makes the bias 0, so the cache holds the base logits.

def _step_diag(vals, T, mode, u=0.0):
    V = len(vals)
    base = bf16(np.asarray(vals, dtype=np.float32))
    head = np.zeros((V, 16), dtype=np.uint16)
    embed = np.zeros((V, 16), dtype=np.uint16)
    g = np.zeros(V, dtype=np.float32) if mode == 0 else None
    tok, _, diag = oracle.step(base, head, embed, 0, T, g, u=u, mode=mode, with_diag=True)
    return tok, diag


@pytest.mark.parametrize("vals,tok,best,second,second_at,nan", [
    ([1, 5, 3, 5, 2], 1, 5, 5, 3, 0),          # tie: the lower id wins, the other is runner-up
    ([1, 5, 3, 4, 2], 1, 5, 4, 3, 0),
    ([-3, -1, -2, -7], 1, -1, -2, 2, 0),
    ([2, np.nan, 9, np.nan], 1, None, 9, 2, 1),  # NaN decides; runner-up ignores NaNs
    ([0.0, -0.0, -1.0], 0, 0, 0, 1, 0),        # -0 equals +0
    ([np.inf, 3, np.inf], 0, np.inf, np.inf, 2, 0),
])
def test_diag_of_the_argmax_rule(vals, tok, best, second, second_at, nan):
    t, d = _step_diag(vals, 0.0, 0)
    assert t == tok
    if best is None:
        assert np.isnan(d[0])
    else:
        assert d[0] == best
    assert d[1] == second and d[2] == second_at and d[3] == nan


@pytest.mark.parametrize("u,tok,dist,across", [
    (0.625, 2, 0.125, 1),    # t = 2.5: midway in bin 2 (cdf 2 .. 3); ties go to the lower edge
    (0.5625, 2, 0.0625, 1),  # t = 2.25: nearer the lower edge, id 1 across it
    (0.6875, 2, 0.0625, 3),  # t = 2.75: nearer the upper edge, id 3 across it
    (0.125, 0, 0.125, -1),   # t = 0.5 in bin 0: the lower edge has nothing across
    (0.9375, 3, 0.0625, -1), # t = 3.75: the top edge has nothing across
])
def test_diag_of_the_inverse_cdf(u, tok, dist, across):
    """Four equal weights (all logits 0): cdf = 1, 2, 3, 4, S = 4, t = 4u,
    all exact in fp64."""
    t, d = _step_diag([0, 0, 0, 0], 1.0, 1, u=u)
    assert t == tok
    assert d[0] == 4 * u and d[1] == 4.0 and d[2] == dist and d[3] == 0 and d[4] == across


def test_inverse_cdf_nan_diag_and_trailing_zero_weights():
    t, d = _step_diag([0, np.nan, 0], 1.0, 1, u=0.5)
    assert t == 1 and d[3] == 1 and d[4] == -1
    # -inf logits carry no weight: t = 3.75 lies in bin 3 (cdf 3 .. 4); the
    # id across the nearer (upper) edge is 4, though it has no weight
    t, d = _step_diag([0, 0, 0, 0, -np.inf, -np.inf], 1.0, 1, u=0.9375)
    assert t == 3 and d[1] == 4.0 and d[2] == 0.0625 and d[4] == 4


def test_inverse_cdf_no_bin_fallback():
    """The hash's u is at most 1 - 2^-24, so t = u S stays below the total and
    some bin always exceeds it; u = 1 (reachable through the step call
    only) leaves none, and the rule then takes the last id with weight, not
    a trailing id of weight 0."""
    vals = [0, -1, 0, 0, 0, -np.inf, -np.inf, -np.inf]
    assert _step_diag(vals, 1.0, 1, u=1.0)[0] == 4
    assert _step_diag(vals, 1.0, 1, u=1.0 - 2.0**-24)[0] == 4
    assert _step_diag([0, 0, 0, 0], 1.0, 1, u=1.0)[0] == 3
