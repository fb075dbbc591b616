"""Seeded synthetic inputs for the Markov draft-sampling chain.

This module draws input data only; it holds none of the chain's arithmetic.
Both the tests (for the CPU oracle and the HIP path alike) and the bench take
their inputs from here, so the two sides see identical bytes.

Random draws come from numpy's PCG64 (a different generator from the chain's
SplitMix64 noise hash); bf16 values are torch's round-to-nearest-even cast of
fp32 draws.  "N(0, s)" means a normal draw with standard deviation s.

The five named workloads follow the chain's use in DeepSeek-V4.1 drafting:
a [V, r] bf16 Markov head and embedding, [rows, N, V] bf16 base logits, one
anchor token and one seed per request row.  No model weights exist here; the
shapes, value ranges and structure (peaked tokens, padding rows, injected NaN
and exact ties) stand in for them.
"""

from __future__ import annotations

import dataclasses
import functools

import numpy as np
import torch

MASTER_SEED = 0x4D41524B00


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 values -> bf16 bit patterns (uint16), torch's RNE cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class Workload:
    name: str
    V: int
    r: int
    rows: int
    N: int
    mode: int
    head: np.ndarray          # uint16 [V, r] bf16 bits
    embed: np.ndarray         # uint16 [V, r] bf16 bits
    base: np.ndarray          # uint16 [rows, N, V] bf16 bits, or float32 values
    prev: np.ndarray          # int64 [rows] anchor tokens
    seeds: np.ndarray         # int64 [rows]
    temperature: np.ndarray   # float32 [rows]
    state_idx: np.ndarray | None  # int64 [rows], negative = padding; None = identity
    mult: float = 1.0         # fp32 output multiplier (1 = none)
    cap: float = 0.0          # fp32 soft cap (0 = none)
    exact: bool = False       # integer-valued weights: fp32 sums are order-exact
    cache_f32: bool = False   # an fp32 draft-logits cache (else bf16)

    @property
    def states(self) -> int:
        if self.state_idx is None:
            return self.rows
        return max(int(self.state_idx.max()) + 1, 1)

    @property
    def real_rows(self) -> int:
        if self.state_idx is None:
            return self.rows
        return int((self.state_idx >= 0).sum())


def _rngs(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng, shape, std):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _seeds(rng, rows):
    return rng.integers(0, 2**64, size=rows, dtype=np.uint64).view(np.int64)


def _peaks(rng, base_f32, count, value):
    """Add `value` at `count` distinct random ids of every (row, step)."""
    rows, N, V = base_f32.shape
    for b in range(rows):
        for i in range(N):
            ids = rng.choice(V, size=count, replace=False)
            base_f32[b, i, ids] += np.float32(value)


def make(name: str, V: int, r: int, rows: int, N: int, *, seed: int,
         weights: str = "normal", weight_std: float = 0.02,
         base_std: float = 3.0, peaks: int = 0, peak_value: float = 12.0,
         temperature=1.0, state_idx=None, mult: float = 1.0, cap: float = 0.0,
         mode: int = 0, base_f32: bool = False, cache_f32: bool = False) -> Workload:
    """A generic workload.  weights: "normal" (N(0, weight_std)), "int"
    (k * 2^-6 with k uniform in [-4, 4]) or "zero" (head = 0).  base_f32
    keeps the base logits as fp32 draws (else their bf16 rounding);
    cache_f32 asks for an fp32 draft-logits cache."""
    r_head, r_embed, r_base, r_peak, r_prev, r_seed = _rngs(seed, 6)
    if weights == "int":
        head = to_bf16_bits(r_head.integers(-4, 5, size=(V, r)).astype(np.float32) * 2.0**-6)
        embed = to_bf16_bits(r_embed.integers(-4, 5, size=(V, r)).astype(np.float32) * 2.0**-6)
    elif weights == "zero":
        head = np.zeros((V, r), dtype=np.uint16)
        embed = to_bf16_bits(_normal(r_embed, (V, r), weight_std))
    else:
        head = to_bf16_bits(_normal(r_head, (V, r), weight_std))
        embed = to_bf16_bits(_normal(r_embed, (V, r), weight_std))
    base_f32_out = base_f32
    base_f32 = _normal(r_base, (rows, N, V), base_std)
    if peaks:
        _peaks(r_peak, base_f32, peaks, peak_value)
    base = base_f32 if base_f32_out else to_bf16_bits(base_f32)
    prev = r_prev.integers(0, V, size=rows, dtype=np.int64)
    seeds = _seeds(r_seed, rows)
    temp = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (rows,)).copy()
    sidx = None if state_idx is None else np.asarray(state_idx, dtype=np.int64)
    return Workload(name, V, r, rows, N, mode, head, embed, base, prev, seeds,
                    temp, sidx, float(np.float32(mult)), float(np.float32(cap)),
                    exact=(weights == "int"), cache_f32=bool(cache_f32))


# The five named workloads.  Each has its own master seed.

def tiny_exact() -> Workload:
    """V=8192, r=256, one row, N=4, T=1: integer-valued weights k*2^-6,
    base N(0, 2); bit-exact on every output."""
    return make("tiny_exact_V8192_r256_rows1_N4", 8192, 256, 1, 4,
                seed=MASTER_SEED + 1, weights="int", base_std=2.0, temperature=1.0)


def dsv41_single_row() -> Workload:
    """V=129280, r=256 (a 66 MB bf16 head), one row, N=8, T=0.7: weights
    N(0, 0.02), base N(0, 3) with 32 peaked ids at +12 per step."""
    return make("dsv41_V129280_r256_rows1_N8", 129280, 256, 1, 8,
                seed=MASTER_SEED + 2, peaks=32, temperature=0.7)


def dsv41_eight_rows() -> Workload:
    """The 8-row batch: row 7 is padding; T per row cycles through
    {0, 0.6, 1.0, 1.5}; output multiplier 0.5 and soft cap 30."""
    temps = np.array([0.0, 0.6, 1.0, 1.5] * 2, dtype=np.float32)
    return make("dsv41_V129280_r256_rows8_N8_capped", 129280, 256, 8, 8,
                seed=MASTER_SEED + 3, peaks=32, temperature=temps,
                state_idx=[0, 1, 2, 3, 4, 5, 6, -1], mult=0.5, cap=30.0)


def dsv41_invcdf_64rows() -> Workload:
    """Inverse-CDF mode over 64 rows, N=8, T=1 (base as the 1-row case)."""
    return make("dsv41_V129280_r256_rows64_N8_invcdf", 129280, 256, 64, 8,
                seed=MASTER_SEED + 4, peaks=32, temperature=1.0, mode=1)


def large_vocab_stress() -> Workload:
    """V=262144, r=512 (a 256 MB head), 8 rows, N=16, T=1 except row 5 (T=0).
    Row 2: NaN at two ids a < b on even steps.  Row 5: exactly 40.0 at three
    ids on every step (exact ties) and a NaN on odd steps."""
    temps = np.ones(8, dtype=np.float32)
    temps[5] = 0.0
    w = make("stress_V262144_r512_rows8_N16", 262144, 512, 8, 16,
             seed=MASTER_SEED + 5, temperature=temps)
    rng = _rngs(MASTER_SEED + 50, 1)[0]
    nan_bits = np.uint16(0x7FC0)
    forty = to_bf16_bits(np.array([40.0], dtype=np.float32))[0]
    for i in range(w.N):
        if i % 2 == 0:
            a, b = sorted(rng.choice(w.V, size=2, replace=False))
            w.base[2, i, a] = nan_bits
            w.base[2, i, b] = nan_bits
        ties = rng.choice(w.V, size=3, replace=False)
        w.base[5, i, ties] = forty
        if i % 2 == 1:
            w.base[5, i, rng.integers(0, w.V)] = nan_bits
    return w


def dsv41_rank_shard() -> Workload:
    """One rank's share of the DeepSeek row when the vocabulary is split over
    8 GPUs: V = 129280 / 8 = 16160 ids (an 8.3 MB head), r=256, one row,
    N=8, T=0.7, base as the 1-row case with 4 peaked ids per step (the 32
    of the whole vocabulary spread over 8 shards)."""
    return make("dsv41_shard8_V16160_r256_rows1_N8", 16160, 256, 1, 8,
                seed=MASTER_SEED + 9, peaks=4, temperature=0.7)


def dsv41_batch(rows: int, mode: int = 0) -> Workload:
    """Beyond the five named workloads: a DeepSeek-sized batch of `rows`
    rows (N=8, T=1, base as the 1-row case), Gumbel or inverse CDF, for the
    > 64-row path (per-position step kernels)."""
    return make(f"dsv41_V129280_r256_rows{rows}_N8" + ("_invcdf" if mode == 1 else ""), 129280, 256, rows, 8,
                seed=MASTER_SEED + 6 + rows, peaks=32, temperature=1.0, mode=mode)


WORKLOADS = {
    "tiny_exact": tiny_exact,
    "dsv41_single_row": dsv41_single_row,
    "dsv41_eight_rows": dsv41_eight_rows,
    "dsv41_invcdf_64rows": dsv41_invcdf_64rows,
    "large_vocab_stress": large_vocab_stress,
    "dsv41_rank_shard": dsv41_rank_shard,
    "dsv41_64rows": functools.partial(dsv41_batch, 64),
    "dsv41_256rows": functools.partial(dsv41_batch, 256),
    "dsv41_invcdf_256rows": functools.partial(dsv41_batch, 256, 1),
}


@functools.lru_cache(maxsize=2)
def workload(name: str) -> Workload:
    return WORKLOADS[name]()
