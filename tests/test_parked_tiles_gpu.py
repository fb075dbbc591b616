"""Streamed head with part of one chunk kept in LDS across steps.

When a workgroup streams its chunks (more chunks than workgroups), the first
tiles of each wave's group in its chunk 1 are written to LDS at step 0 and
read from there at later steps, as long as they fit beside the embeddings
(up to 13 rows at r = 512, 10 at r = 256).  Small vocabularies with a
reduced grid force the streamed kernel with 2, 3 and 4 chunks per workgroup
(chunk 1 is then streamed every other step, or every step); N = 5 covers
both visiting orders and several reads of the parked tiles.  Integer-valued
weights: tokens and cache must equal the CPU oracle bit for bit, with the
tiles parked and without (more rows than fit).
"""

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


@pytest.fixture(autouse=True)
def _gpu_and_grid():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lm.load()
    old = lm.markov_set_grid(0)
    yield
    lm.markov_set_grid(old)
    torch.cuda.synchronize()


def chunks(V, r):
    return -(-V // (8 * (16384 // r)))


def check(w, grid, inline=False, calls=2):
    lm.markov_set_grid(grid)
    G = lm.markov_grid(w.rows, w.N, w.V, w.r, w.mode)
    NC = chunks(w.V, w.r)
    assert G == grid and G < NC, (G, NC)
    say(f"  {w.name}: V={w.V} r={w.r} rows={w.rows} N={w.N} mode={w.mode} grid={G} "
        f"chunks per workgroup {NC // G}..{-(-NC // G)} inline={inline}")
    g = oracle.noise_fill(w.seeds, w.N, w.V) if w.mode == 0 and not inline else None
    d = DeviceChain(w, noise_inline=inline)
    if g is not None:
        d.set_gumbel(g)
    t_o, c_o = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g, mode=w.mode)
    for k in range(calls):  # a second call on the same workspace reads what the first parked anew
        d.tokens.fill_(-7)
        d.chain()
        lm.markov_status(d.workspace)
        t, c = d.results()
        assert np.array_equal(t, t_o), f"call {k}: tokens differ from the oracle"
        assert np.array_equal(c, c_o), f"call {k}: cache differs from the oracle"


TEMPS = np.array([1.0, 0.7, 0.0, 1.5, 0.6], dtype=np.float32)


@pytest.mark.parametrize("r,V,grid", [
    (512, 8192, 8),    # 32 chunks: 4 per workgroup
    (512, 8192, 11),   # 2 or 3 per workgroup
    (512, 8192, 16),   # 2 per workgroup: chunk 1 streamed on even steps only
    (256, 8192 + 16, 4),  # 17 chunks, ragged vocabulary: 4 or 5 per workgroup
    (256, 8192, 6),    # 2 or 3 per workgroup
])
@pytest.mark.parametrize("rows", [1, 3, 9])
def test_parked_tiles_exact(r, V, grid, rows):
    w = synth.make(f"park_r{r}_rows{rows}", V, r, rows, 5, seed=V + r + rows + grid, weights="int",
                   base_std=2.0, temperature=TEMPS[np.arange(rows) % 5])
    check(w, grid)


@pytest.mark.parametrize("r,V,grid", [(512, 8192, 8), (256, 8192, 6)])
def test_parked_tiles_inline_noise_and_inverse_cdf(r, V, grid):
    w = synth.make(f"park_nz_r{r}", V, r, 4, 5, seed=31 + r, weights="int", base_std=2.0,
                   temperature=TEMPS[np.arange(4) % 5])
    check(w, grid, inline=True)
    w = synth.make(f"park_cdf_r{r}", V, r, 6, 5, seed=37 + r, weights="int", base_std=2.0,
                   temperature=TEMPS[np.arange(6) % 5], mode=1)
    check(w, grid)


@pytest.mark.parametrize("r,rows", [(512, 13), (512, 20), (256, 10), (256, 24)])
def test_parked_tiles_row_limits(r, rows):
    """The largest row counts with parked tiles, and counts beyond them
    (the tiles are then streamed every step, as without parking)."""
    w = synth.make(f"park_lim_r{r}_rows{rows}", 8192, r, rows, 4, seed=41 + rows, weights="int",
                   base_std=2.0, temperature=TEMPS[np.arange(rows) % 5])
    check(w, 4 if r == 512 else 5, calls=1)
    wm = synth.make(f"park_lim_cdf_r{r}_rows{rows}", 8192, r, rows, 3, seed=43 + rows, weights="int",
                    base_std=2.0, temperature=1.0, mode=1)
    check(wm, 4 if r == 512 else 5, calls=1)
