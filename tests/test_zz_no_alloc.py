"""markov_chain_sample_noalloc, the entry point that allocates nothing.

Its outputs must equal markov_chain_sample's on the same inputs bit for bit
(the same kernels run; only the exchange state lives in the library's static
scratch instead of a caller's workspace), call after call, with the second
call of a pair on a smaller input, and match the oracle exactly on
integer-valued weights.
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
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lm.load()
    yield
    lm.markov_set_wait_limit(-1)
    torch.cuda.synchronize()


def both(w, inline=False):
    """(tokens, cache) from markov_chain_sample and from the allocation-free
    entry point, on the same device inputs."""
    d = DeviceChain(w, noise_inline=inline)
    if w.mode == 0 and not inline:
        d.set_gumbel(oracle.noise_fill(w.seeds, w.N, w.V))
    d.chain()
    lm.markov_status(d.workspace)
    ref = d.results()
    d.tokens.fill_(-7)
    d.cache.zero_()
    say(f"  noalloc call: {w.name} V={w.V} rows={w.rows} N={w.N} mode={w.mode} inline={inline}")
    lm.markov_chain_sample_noalloc(
        d.base, d.head, d.embed, d.prev, d.temperature, d.tokens, d.cache, gumbel=d.gumbel,
        seeds=d.seeds, state_idx=d.state_idx, output_multiplier=w.mult, soft_cap=w.cap,
        mode=w.mode | (lm.MARKOV_NOISE_INLINE if inline else 0))
    lm.markov_status(None)
    return ref, d.results()


def same(a, b):
    return np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("pair", ["mode0", "inline_one_row", "invcdf", "step_paths", "step_inline"])
def test_noalloc_matches_the_workspace_entry_point_twice(pair):
    """Two calls in a row, the second on a smaller input; each equals the
    workspace entry point's result, and the oracle's on integer weights."""
    if pair == "mode0":
        big = synth.make("na_big", 20000, 256, 5, 6, seed=61, weights="int", base_std=2.0,
                         temperature=[1.0, 0.0, 0.6, 1.5, 1.0], state_idx=[3, 0, -1, 1, 2])
        small = synth.make("na_small", 4096, 256, 2, 3, seed=62, weights="int", base_std=2.0,
                           temperature=0.8)
        inline = False
    elif pair == "inline_one_row":
        big = synth.workload("dsv41_single_row")
        small = synth.make("na_small1", 8192, 256, 1, 4, seed=63, weights="int", base_std=2.0,
                           temperature=1.0)
        inline = True
    elif pair == "invcdf":
        big = synth.make("na_big1", 12288, 256, 9, 4, seed=64, weights="int", base_std=2.0,
                         temperature=[1.0, 0.0, 0.5, 2.0, 1.0, 1.0, 0.7, 1.0, 1.3], mode=1)
        small = synth.make("na_small2", 2048, 256, 3, 2, seed=65, weights="int", base_std=2.0,
                           temperature=1.0, mode=1)
        inline = False
    elif pair == "step_paths":
        # more than 64 rows: the per-position kernels (a step kernel in mode
        # 0; a step and a pick kernel in mode 1), then a smaller such call
        big = synth.make("na_step0", 8192, 256, 100, 3, seed=66, weights="int", base_std=2.0,
                         temperature=np.array([1.0, 0.0, 0.7, 1.5] * 25, dtype=np.float32))
        small = synth.make("na_step1", 4096, 256, 70, 3, seed=67, weights="int", base_std=2.0,
                           temperature=np.array([1.0, 0.0, 0.6, 1.3, 2.0] * 14, dtype=np.float32), mode=1)
        inline = False
    else:
        # more than 64 rows with the noise drawn inside the step kernel
        big = synth.make("na_stepnz0", 8192, 256, 100, 3, seed=68, weights="int", base_std=2.0,
                         temperature=np.array([1.0, 0.0, 0.7, 1.5] * 25, dtype=np.float32))
        small = synth.make("na_stepnz1", 4096, 256, 70, 2, seed=69, weights="int", base_std=2.0,
                           temperature=np.array([1.0, 0.0, 0.6, 1.3, 2.0] * 14, dtype=np.float32))
        inline = True
    for w in (big, small):
        ref, got = both(w, inline)
        assert same(ref, got), w.name
        if w.exact:
            g = None if (w.mode == 1 or inline) else oracle.noise_fill(w.seeds, w.N, w.V)
            t_o, c_o = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds,
                                    gumbel=g, state_idx=w.state_idx, mode=w.mode)
            padded = np.flatnonzero(w.state_idx < 0) if w.state_idx is not None else []
            real = [b for b in range(w.rows) if b not in set(padded)]
            assert np.array_equal(got[0][real], t_o[real])
            for b in real:
                s = b if w.state_idx is None else int(w.state_idx[b])
                assert np.array_equal(got[1][s], c_o[s])


def test_noalloc_many_calls_alternating_shapes():
    """Thirty calls alternating a larger and a smaller shape on the one
    static scratch: every result equals the first of its shape."""
    a = synth.make("na_a", 8192, 256, 4, 5, seed=66, temperature=0.9)
    b = synth.make("na_b", 2048, 256, 1, 3, seed=67, temperature=1.2)
    ref = {}
    for k in range(30):
        w = a if k % 2 == 0 else b
        r, got = both(w)
        assert same(r, got)
        if w.name in ref:
            assert same(ref[w.name], got)
        ref[w.name] = got


def test_noalloc_timeout_is_reported_and_cleared():
    """A zero wait limit makes the waits give up; markov_status(NULL) reports
    it and zeroes the scratch, and the next call is exact again."""
    w = synth.make("na_to", 129280, 256, 1, 3, seed=69, weights="int", base_std=2.0,
                   temperature=1.0)
    d = DeviceChain(w, noise_inline=True)
    lm.markov_set_wait_limit(0)
    lm.markov_chain_sample_noalloc(d.base, d.head, d.embed, d.prev, d.temperature, d.tokens,
                                   d.cache, seeds=d.seeds, mode=lm.MARKOV_NOISE_INLINE)
    torch.cuda.synchronize()
    lm.markov_set_wait_limit(-1)
    with pytest.raises(lm.MarkovError) as e:
        lm.markov_status(None)
    assert "timed out" in str(e.value)
    lm.markov_status(None)  # cleared
    ref, got = both(w, inline=True)
    assert same(ref, got)
    t_o, c_o = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds)
    assert np.array_equal(got[0], t_o) and np.array_equal(got[1], c_o)
