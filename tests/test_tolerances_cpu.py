"""The parity tolerances themselves, checked on the CPU.

The bias tolerance in chain_check must (a) admit every fp32 accumulation of
the exact bf16 products, whatever the summation order, and (b) stay one bf16
ulp wherever the sum does not nearly cancel, so that it still rejects a
plausible device mistake (a two-ulp error on an ordinary element).  The fp32
sums here are numpy float32 recursive sums in three different orders,
independent of both the oracle's arithmetic and the device's.
"""

import numpy as np

import chain_check
import oracle
from markov_bias_chain_amd import synth


def _fp32_sums(head_f, e_f, order):
    """Recursive fp32 sums of the exact products (bf16 x bf16 products are
    exact in fp32) in the given k order."""
    prods = (head_f[:, order] * e_f[order]).astype(np.float32)
    acc = np.zeros(head_f.shape[0], dtype=np.float32)
    for k in range(prods.shape[1]):
        acc = (acc + prods[:, k]).astype(np.float32)
    return acc


def test_bias_tolerance_admits_fp32_accumulation_and_is_one_ulp_otherwise():
    w = synth.make("tol", 6000, 256, 1, 1, seed=91)
    p = int(w.prev[0])
    head_f = chain_check.f32(w.head)
    e_f = chain_check.f32(w.embed[p])
    _, _, bias_o = oracle.step(np.zeros(w.V, np.uint16), w.head, w.embed, p, 0.0, None,
                               with_bias=True)
    absdot = chain_check.AbsDot(w)(p)
    tol = chain_check.bias_tolerance(bias_o, absdot, w.r)
    bo = chain_check.f32(bias_o).astype(np.float64)
    rng = np.random.default_rng(92)
    for order in (np.arange(w.r), np.arange(w.r)[::-1], rng.permutation(w.r)):
        dev = oracle.bf16_round_f32(_fp32_sums(head_f, e_f, order))
        diff = np.abs(chain_check.f32(dev).astype(np.float64) - bo)
        assert np.all(diff <= tol)
    # Away from cancellation E is a few percent of a bf16 spacing (r 2^-24
    # sum|h e| against |bias| 2^-8 with sum|h e| ~ 10 |bias|), so the
    # tolerance is one ulp plus a sliver, and a two-ulp error is rejected.
    spacing = chain_check.bf16_spacing(bo)
    ordinary = tol < 1.5 * spacing
    assert ordinary.mean() > 0.95
    two_ulp = bo + 2.0 * spacing
    assert np.all(np.abs(two_ulp - bo)[ordinary] > tol[ordinary])


def test_bias_tolerance_special_values():
    # zero bias, zero products: only the smallest spacing is allowed
    t = chain_check.bias_tolerance(np.array([0], np.uint16), np.array([0.0]), 256)
    assert t[0] == 2.0**-133
    # a power of two: spacing of its own binade, not the next one
    one = synth.to_bf16_bits(np.array([1.0], np.float32))
    t = chain_check.bias_tolerance(one, np.array([0.0]), 256)
    assert t[0] == 2.0**-7


# ------------------------------------------------------------ the walk --
# The parity walk run on the oracle's own outputs, with mistakes planted in
# copies of them on the CPU: it must accept the oracle, reject a token its
# cache does not explain, and accept (and walk past) one its cache does.

def _oracle_run(w):
    import oracle
    g = oracle.noise_fill(w.seeds, w.N, w.V)
    t, c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g)
    return g, t, c


def test_walk_accepts_the_oracle_and_rejects_an_unexplained_token():
    import pytest
    from markov_bias_chain_amd import synth
    w = synth.make("walk", 512, 256, 2, 4, seed=3, temperature=[1.0, 0.0])
    g, t, c = _oracle_run(w)
    st = chain_check.walk(w, t, c, g)
    assert st.token_match == st.pairs == 8 and not st.mismatches
    assert chain_check.walk(w, t, c, g, exact=True).token_match == 8
    bad = t.copy()
    bad[0, 1] = (bad[0, 1] + 1) % w.V
    with pytest.raises(AssertionError):
        chain_check.walk(w, bad, c, g)


def test_walk_accepts_an_explained_flip_and_continues_from_the_device_token():
    """Zero head (bias 0), greedy rows: the cache is the base logits.  At
    step 1 ids 10 and 5 are one bf16 ulp apart (2 and 2 - 2^-7).  A 'device'
    whose cache holds id 10 one ulp lower ties the two and takes id 5: the
    walk must accept it (one-ulp cache difference, device token = its own
    argmax, margin = the move) and compare the later steps too."""
    from markov_bias_chain_amd import synth
    w = synth.make("flip", 256, 256, 1, 4, seed=4, weights="zero", base_std=0.5, temperature=0.0)
    w.base[0, 1, 10] = synth.to_bf16_bits(np.array([2.0], np.float32))[0]
    w.base[0, 1, 5] = synth.to_bf16_bits(np.array([2.0 - 2.0**-7], np.float32))[0]
    g, t, c = _oracle_run(w)
    assert t[0, 1] == 10
    dev_t, dev_c = t.copy(), c.copy()
    dev_c[0, 1, 10] = w.base[0, 1, 5]
    dev_t[0, 1] = 5
    st = chain_check.walk(w, dev_t, dev_c, g)
    assert st.pairs == 4 and st.token_match == 3 and st.mismatches == [(0, 1, 10, 5)]
    assert st.cache_beyond_1ulp == 0
