"""Token-match rate of the DeepSeek-sized chain on random weights.

The device runs the chain kernel that draws its Gumbel noise inline (the
kernel the bench times), free-running from the seeds.  The oracle draws its
own noise from the same seeds and walks every (row, position) pair: the
cache within the bias-implied bound, the token equal to the oracle's or, where
it differs, explained by the device's own cache (the device token is the
sampling rule's pick on the device cache, the caches differ, and the oracle's
top-2 margin is within what that difference moves).  The walk continues from
the device's token after a mismatch.  Over about a thousand pairs per shape
the tokens must match on at least 99.9% of the pairs.

Anchors and seeds vary call by call; head, embedding and base logits are
those of the named DeepSeek-sized workloads (N(0, 0.02) weights, N(0, 3) base
logits with 32 peaked ids at +12 per position).
"""

import concurrent.futures
import dataclasses
import os
import sys

import numpy as np
import pytest
import torch

import chain_check
import oracle
from markov_bias_chain_amd import binding as lm
from markov_bias_chain_amd import synth
from markov_bias_chain_amd.device import DeviceChain

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lm.load()
    old = lm.markov_set_grid(0)
    yield
    lm.markov_set_grid(old)
    torch.cuda.synchronize()


def rate_walk(name, calls, rng):
    """`calls` device calls of workload `name` with fresh anchors and seeds,
    inline noise; every call walked against the oracle with its own noise."""
    w = synth.workload(name)
    d = DeviceChain(w, noise_inline=True)
    say(f"  {name}: {calls} calls, grid {lm.markov_grid(w.rows, w.N, w.V, w.r, w.mode)}")
    runs = []
    for _ in range(calls):
        prev = rng.integers(0, w.V, size=w.rows, dtype=np.int64)
        seeds = rng.integers(0, 2**64, size=w.rows, dtype=np.uint64).view(np.int64)
        d.prev.copy_(torch.from_numpy(prev))
        d.seeds.copy_(torch.from_numpy(seeds))
        d.tokens.fill_(-7)
        d.chain()
        t, c = d.results()
        runs.append((dataclasses.replace(w, prev=prev, seeds=seeds), t, c))
    lm.markov_status(d.workspace)
    del d
    absdot = chain_check.AbsDot(w)

    def one(run):
        wk, t, c = run
        g = oracle.noise_fill(wk.seeds, wk.N, wk.V)
        return chain_check.walk(wk, t, c, g, workers=1, absdot=absdot)

    st = chain_check.Stats()
    with concurrent.futures.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for s in ex.map(one, runs):
            st.merge(s)
    say("  " + st.summary())
    for m in st.mismatches:
        say(f"  explained mismatch (row, step, oracle, device): {m}")
    chain_check.record(f"rate_{name}_inline", st, calls=calls)
    return st


def test_token_match_rate_one_row_inline_noise():
    st = rate_walk("dsv41_single_row", 128, np.random.default_rng(0x5EED1))
    assert st.pairs == 128 * 8
    assert st.token_match >= 0.999 * st.pairs


def test_token_match_rate_eight_rows_inline_noise():
    """Seven real rows (one padding row), per-row temperatures 0 / 0.6 / 1 /
    1.5, output multiplier 0.5 and soft cap 30."""
    st = rate_walk("dsv41_eight_rows", 18, np.random.default_rng(0x5EED8))
    assert st.pairs == 18 * 7 * 8
    assert st.token_match >= 0.999 * st.pairs
