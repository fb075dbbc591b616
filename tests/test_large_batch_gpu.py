"""Batches beyond one launch's 64 rows (consecutive launches of at most 64
rows): sampled rows on both sides of the launch boundaries must equal the
CPU oracle bit for bit (integer-valued weights), with the call's own row
indices in the mode-1 hash and in the identity state map, padding rows
inert and the noise kernel covering every row."""

import sys

import numpy as np
import pytest
import torch

import oracle
from markov_bias_chain_amd import binding as lm
from markov_bias_chain_amd import synth
from markov_bias_chain_amd.device import DeviceChain

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


SAMPLED = [0, 1, 63, 64, 65, 127, 128, 150, 191, 199]


def _check(w, g, rows):
    d = DeviceChain(w)
    say(f"  device call: {w.name} V={w.V} r={w.r} rows={w.rows} N={w.N} mode={w.mode}")
    if w.mode == 0:
        d.set_gumbel(g)
    d.chain()
    lm.markov_status(d.workspace)
    t, c = d.results()
    mask = np.zeros(w.rows, dtype=np.uint8)
    mask[[b for b in rows if b < w.rows]] = 1
    tokens = np.full((w.rows, w.N), -7, dtype=np.int64)
    cache = c.copy()  # the oracle overwrites the sampled rows' states only
    ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds,
                                gumbel=g, state_idx=w.state_idx, mode=w.mode, row_mask=mask,
                                tokens=tokens, cache=cache)
    sidx = np.arange(w.rows) if w.state_idx is None else w.state_idx
    for b in rows:
        if b >= w.rows:
            continue
        if sidx[b] < 0:
            assert np.all(t[b] == -7), f"padding row {b} written"
            continue
        assert np.array_equal(t[b], ref_t[b]), f"row {b}: tokens differ"
        assert np.array_equal(c[sidx[b]], ref_c[sidx[b]]), f"row {b}: cache differs"
    return t


def test_mode0_200_rows_identity_states():
    w = synth.make("big0", 4096 + 16, 256, 200, 3, seed=81, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.7, 0.0, 1.5] * 50, dtype=np.float32))
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    _check(w, g, SAMPLED)


def test_mode1_150_rows_permuted_states_and_padding():
    rows = 150
    rng = np.random.default_rng(82)
    sidx = rng.permutation(rows + 10)[:rows].astype(np.int64)
    sidx[[5, 70, 149]] = -1
    w = synth.make("big1", 2048 + 32, 512, rows, 4, seed=83, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.6, 0.0] * 50, dtype=np.float32), mode=1,
                   state_idx=sidx)
    _check(w, None, SAMPLED + [5, 70, 149])


def test_noise_fill_100_rows():
    rows, N, V = 100, 3, 1024
    seeds = np.random.default_rng(84).integers(-2**63, 2**63 - 1, size=rows, dtype=np.int64)
    g = torch.empty((rows, N, V), dtype=torch.float32, device="cuda")
    lm.markov_noise_fill(g, torch.from_numpy(seeds).cuda())
    dev = g.cpu().numpy()
    ref = oracle.noise_fill(seeds, N, V)
    assert (dev.view(np.int32) == ref.view(np.int32)).mean() > 1 - 1e-5
