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
