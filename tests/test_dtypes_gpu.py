"""The element-type variants through the C ABI: base logits bf16 or fp32 and
the draft-logits cache bf16 or fp32 (the pages' sampler takes either; an
fp32 cache keeps x unrounded).  Integer-valued weights make every fp32 sum
order-exact, so those cases are bit-exact against the CPU oracle; random
weights are walked with the bias-implied tolerance."""

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


def run(w, gumbel):
    d = DeviceChain(w)
    say(f"  device call: {w.name} V={w.V} r={w.r} rows={w.rows} N={w.N} mode={w.mode} "
        f"base={w.base.dtype} cache_f32={w.cache_f32}")
    if w.mode == 0:
        d.set_gumbel(gumbel)
    d.chain()
    lm.markov_status(d.workspace)
    return d.results()


@pytest.mark.parametrize("base_f32,cache_f32", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("V,r,rows,mode", [
    (8192 + 16, 256, 1, 0),    # one row (lane = vocab id)
    (4096, 256, 5, 0),         # batches of rows
    (2048 + 32, 512, 3, 1),    # inverse CDF, r = 512
    (3072, 256, 12, 1),        # inverse CDF over more than 8 rows
])
def test_dtype_variants_bit_exact(base_f32, cache_f32, V, r, rows, mode):
    temps = np.array([1.0, 0.0, 0.7, 1.5] * 4, dtype=np.float32)[:rows]
    w = synth.make(f"dt_{int(base_f32)}{int(cache_f32)}_V{V}", V, r, rows, 4, seed=V + rows + r,
                   weights="int", base_std=2.0, temperature=temps, mode=mode,
                   base_f32=base_f32, cache_f32=cache_f32)
    g = oracle.noise_fill(w.seeds, w.N, w.V) if mode == 0 else None
    t, c = run(w, g)
    ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds,
                                gumbel=g, mode=mode, cache_f32=cache_f32)
    assert c.dtype == ref_c.dtype
    assert np.array_equal(t, ref_t)
    assert np.array_equal(c.view(np.uint32) if cache_f32 else c,
                          ref_c.view(np.uint32) if cache_f32 else ref_c)


@pytest.mark.parametrize("base_f32,cache_f32", [(True, False), (True, True)])
def test_dtype_variants_random_weights(base_f32, cache_f32):
    """DeepSeek-sized rows with fp32 base logits (as an LM head produces them)
    and either cache: the bias-tolerance walk over sampled rows."""
    w = synth.make(f"dt_rand_{int(cache_f32)}", 129280, 256, 3, 8, seed=71, peaks=32,
                   temperature=[0.7, 0.0, 1.0], mult=0.5, cap=30.0,
                   base_f32=base_f32, cache_f32=cache_f32)
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    t, c = run(w, g)
    st = chain_check.walk(w, t, c, g)
    say("  " + st.summary())
    assert len(st.mismatches) <= 1
