"""The chain's bounded cross-workgroup waits, driven to give up from the host.

Every wait of the chain kernel is bounded (sharded_markov page,
DSparkShardedMarkovSampler: timeout_ms bounds every cross-rank wait).  With
the bound set to 0 (markov_set_wait_limit), a wait gives up as soon as one
poll finds a slot still empty, so every workgroup still runs to its end and
exits normally; no kernel is broken and nothing faults.  markov_status must
then report MARKOV_DEVERR_TIMEOUT, and after the workspace is zeroed again the
next call must be exact again.
"""

import sys
import time

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
    yield
    lm.markov_set_wait_limit(-1)
    lm.markov_set_batch_path(0)
    torch.cuda.synchronize()


@pytest.mark.parametrize("V,rows,mode,inline", [
    (129280, 1, 0, False),  # one row: the two-level exchange through reducer workgroups
    (129280, 1, 0, True),   # the same with inline noise (the bench's kernel)
    (20000, 3, 0, False),   # a batch: the all-to-all exchange
    (12288, 5, 1, False),   # inverse CDF: leader, decision and token waits
    (8192, 100, 0, False),  # two persistent launches of up to 64 rows
])
def test_wait_limit_zero_times_out_then_recovers(V, rows, mode, inline):
    w = synth.make(f"timeout_V{V}_rows{rows}", V, 256, rows, 3, seed=V + rows, weights="int",
                   base_std=2.0, temperature=1.0, mode=mode)
    g = oracle.noise_fill(w.seeds, w.N, w.V) if mode == 0 and not inline else None
    d = DeviceChain(w, noise_inline=inline)
    if g is not None:
        d.set_gumbel(g)
    lm.markov_set_batch_path(1)  # the persistent kernels (the only ones that wait)
    say(f"  V={V} rows={rows} mode={mode} inline={inline}: wait limit 0")
    assert lm.markov_set_wait_limit(0) == 2_000_000
    t0 = time.perf_counter()
    d.chain()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    lm.markov_set_wait_limit(-1)
    with pytest.raises(lm.MarkovError) as err:
        lm.markov_status(d.workspace)
    assert err.value.code == lm.MARKOV_E_DEVICE and "timed out" in str(err.value)
    assert elapsed < 1.0, f"a call with a zero wait limit took {elapsed:.3f} s"
    # the documented recovery: zero the workspace, call again
    d.workspace.zero_()
    d.tokens.fill_(-7)
    d.chain()
    lm.markov_status(d.workspace)
    t, c = d.results()
    ref = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g,
                       mode=mode)
    assert np.array_equal(t, ref[0])
    assert np.array_equal(c, ref[1])
    # and a later call on the same workspace is still exact
    d.chain()
    lm.markov_status(d.workspace)
    t2, c2 = d.results()
    assert np.array_equal(t2, ref[0]) and np.array_equal(c2, ref[1])


def test_persistent_step_kernel_times_out_then_recovers():
    """The persistent step kernel (mode 0, large batches) waits for each
    position's tokens: with a zero wait limit the workgroups that arrive
    before the last one give up at once (every wait is bounded, every
    workgroup runs to its end), MARKOV_DEVERR_TIMEOUT is reported, and after
    the workspace is zeroed again the next call is exact."""
    w = synth.make("timeout_pers", 8192, 256, 100, 3, seed=8293, weights="int", base_std=2.0, temperature=1.0)
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    d = DeviceChain(w)
    d.set_gumbel(g)
    lm.markov_set_batch_path(3)
    say("  persistent step kernel, rows=100: wait limit 0")
    lm.markov_set_wait_limit(0)
    d.chain()
    torch.cuda.synchronize()
    lm.markov_set_wait_limit(-1)
    with pytest.raises(lm.MarkovError) as err:
        lm.markov_status(d.workspace)
    assert err.value.code == lm.MARKOV_E_DEVICE and "timed out" in str(err.value)
    d.workspace.zero_()
    d.tokens.fill_(-7)
    d.chain()
    lm.markov_status(d.workspace)
    t, c = d.results()
    ref = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    assert np.array_equal(t, ref[0]) and np.array_equal(c, ref[1])


def test_step_kernels_never_wait():
    """The per-position launches (large batches) have no cross-workgroup
    wait: with a zero wait limit they still complete without an error and
    exactly."""
    w = synth.make("timeout_step", 8192, 256, 100, 3, seed=8292, weights="int", base_std=2.0, temperature=1.0)
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    d = DeviceChain(w)
    d.set_gumbel(g)
    lm.markov_set_batch_path(2)
    lm.markov_set_wait_limit(0)
    d.chain()
    lm.markov_status(d.workspace)
    lm.markov_set_wait_limit(-1)
    t, c = d.results()
    ref = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    assert np.array_equal(t, ref[0]) and np.array_equal(c, ref[1])
