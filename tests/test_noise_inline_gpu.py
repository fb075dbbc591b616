"""Inline noise (MARKOV_NOISE_INLINE): the chain kernel draws the Gumbel
noise itself from the seeds.  On every kernel variant (one row with a
resident or streamed head, prefetched batches, more than 8 rows, r = 512,
calls of several launches) its tokens and cache must equal, bit for bit,
those of the same call reading the noise markov_noise_fill wrote; and on
integer-valued weights the oracle's, given the oracle's noise."""

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


def _run(w, inline, grid=0):
    old = lm.markov_set_grid(grid)
    try:
        d = DeviceChain(w, noise_inline=inline)
        say(f"  device call: {w.name} V={w.V} r={w.r} rows={w.rows} N={w.N} inline={inline} grid={grid}")
        d.step()
        lm.markov_status(d.workspace)
        return d.results()
    finally:
        lm.markov_set_grid(old)


def _same(w, grid=0):
    t0, c0 = _run(w, False, grid)
    t1, c1 = _run(w, True, grid)
    assert np.array_equal(t0, t1), "tokens differ between inline and markov_noise_fill noise"
    assert np.array_equal(c0, c1), "cache differs between inline and markov_noise_fill noise"
    return t1, c1


@pytest.mark.parametrize("grid", [0, 5])  # resident head (one-row kernel) / streamed
def test_inline_tiny_exact_matches_oracle(grid):
    w = synth.tiny_exact()
    t, c = _same(w, grid)
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    assert np.array_equal(t, ref_t)
    assert np.array_equal(c, ref_c)


@pytest.mark.parametrize("name", ["dsv41_single_row", "dsv41_eight_rows", "large_vocab_stress", "dsv41_64rows"])
def test_inline_named_workloads(name):
    _same(synth.workload(name))


def test_inline_small_batches_and_argmax_rows():
    # 3 rows (prefetched batch), T = 0 on one row: no noise drawn for it
    w = synth.make("inl3", 8192 + 16, 256, 3, 5, seed=91, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.0, 0.6], dtype=np.float32))
    _same(w)


def test_inline_two_launches_with_padding():
    # 100 rows: launches of 64 and 36 rows; the hash uses the call's row index
    rows = 100
    sidx = np.arange(rows, dtype=np.int64)
    sidx[[3, 64, 99]] = -1
    w = synth.make("inl100", 4096 + 16, 256, rows, 3, seed=92, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.7, 0.0, 1.5] * 25, dtype=np.float32),
                   state_idx=sidx)
    t, c = _same(w)
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    mask = np.zeros(rows, dtype=np.uint8)
    picked = [0, 1, 3, 63, 64, 65, 98, 99]
    mask[picked] = 1
    ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g,
                                state_idx=sidx, row_mask=mask,
                                tokens=np.full((rows, w.N), -7, dtype=np.int64), cache=c.copy())
    for b in picked:
        if sidx[b] < 0:
            assert np.all(t[b] == -7)
        else:
            assert np.array_equal(t[b], ref_t[b]), f"row {b}"
            assert np.array_equal(c[sidx[b]], ref_c[sidx[b]]), f"row {b}"


def test_inline_r512_rows9():
    # r = 512, more than 8 rows (the many-row exchange, noise in the epilogue)
    w = synth.make("inl9", 8192 + 16, 512, 9, 4, seed=93, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.5, 0.0, 2.0, 1.0, 1.0, 0.7, 1.0, 1.0], dtype=np.float32))
    _same(w)


@pytest.mark.parametrize("V,r,rows,N,T,grid", [
    (16, 256, 1, 5, 1.0, 0),          # the smallest vocabulary: one group of one chunk
    (4096 + 16, 512, 1, 6, 0.8, 0),   # r = 512, one row, ragged last group
    (4096 + 16, 512, 1, 6, 0.8, 3),   # the same on a streamed head
    (2048, 256, 1, 256, 1.3, 0),      # the most steps a call takes
    (2048, 256, 2, 3, 0.0, 0),        # argmax rows draw no noise
])
def test_inline_edge_shapes(V, r, rows, N, T, grid):
    w = synth.make(f"inl_edge_{V}_{r}_{rows}_{N}", V, r, rows, N, seed=96 + N, weights="int",
                   base_std=2.0, temperature=np.full(rows, T, dtype=np.float32))
    t, c = _same(w, grid)
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    assert np.array_equal(t, ref_t)
    assert np.array_equal(c, ref_c)


@pytest.mark.parametrize("V,r,rows,N", [
    (8192 + 16, 256, 8, 10),   # 8 rows (one T = 0), more steps than the named workload
    (8192 + 16, 512, 3, 14),   # r = 512, a prefetched batch of 3 rows
    (4096 + 16, 256, 1, 53),   # one row, many steps
])
def test_inline_noise_batches_and_steps(V, r, rows, N):
    # Inline draws must give the side-stream kernel's values and, on
    # integer weights, the oracle's tokens and cache.
    w = synth.make(f"inl_ahead_{r}_{rows}_{N}", V, r, rows, N, seed=97 + N, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.6, 0.0, 1.5, 1.0, 0.8, 1.2, 0.9][:rows], dtype=np.float32))
    t, c = _same(w)
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    assert np.array_equal(t, ref_t)
    assert np.array_equal(c, ref_c)


@pytest.mark.parametrize("rows", [1, 3])
def test_inline_noise_fp32_dtypes(rows):
    # The flag-reading kernels (fp32 base logits and cache) draw inline too.
    w = synth.make(f"inl_f32_{rows}", 8192 + 16, 256, rows, 9, seed=98 + rows, base_f32=True, cache_f32=True,
                   temperature=np.array([0.9, 1.1, 0.0][:rows], dtype=np.float32))
    _same(w)


def test_inline_graph_replays():
    w = synth.make("inlg", 8192 + 16, 256, 1, 5, seed=94, weights="int", base_std=2.0)
    d = DeviceChain(w, noise_inline=True)
    eager = DeviceChain(w, noise_inline=True)
    g = d.capture_step()
    rng = np.random.default_rng(95)
    for k in range(3):
        prev = rng.integers(0, w.V, size=1, dtype=np.int64)
        seeds = rng.integers(-2**63, 2**63 - 1, size=1, dtype=np.int64)
        for x in (d, eager):
            x.prev.copy_(torch.from_numpy(prev))
            x.seeds.copy_(torch.from_numpy(seeds))
        g.replay()
        torch.ones(1 << 20, device=d.device).sum().item()
        eager.step()
        lm.markov_status(d.workspace)
        lm.markov_status(eager.workspace)
        t_g, c_g = d.results()
        t_e, c_e = eager.results()
        assert np.array_equal(t_g, t_e), f"replay {k}"
        assert np.array_equal(c_g, c_e), f"replay {k}"
