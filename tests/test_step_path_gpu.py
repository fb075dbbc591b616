"""The step-kernel path for large batches: per draft position one step
kernel over all rows (mode 0: the last workgroup to arrive picks the
winners) or a step kernel and a pick kernel (mode 1: one wave per row draws
by inverse CDF from the chunks' partials).

It must give exactly the outputs of the persistent path (both compute the
bias with the same MFMA passes and, in mode 1, combine the partials and
scan the chosen chunk with the same arithmetic, so even random weights
agree bit for bit), and sampled rows must equal the CPU oracle (bit for bit
on integer-valued weights, within the derived tolerances on random ones).
Covered, in both modes: padding rows, permuted state indices, greedy rows,
the output transform, fp32 base logits and cache, r = 512, ragged
vocabularies, the largest row count, repeated calls on one workspace shared
with persistent calls, and the DeepSeek-sized 256-row batch; in mode 0 also
the noise drawn inside the step kernels (bit-identical to the noise in
memory), and more positions than the persistent step kernel's first
layout held.
"""

import dataclasses
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
    old = lm.markov_set_batch_path(0)
    yield
    lm.markov_set_batch_path(old)
    torch.cuda.synchronize()


def noise_for(w):
    return oracle.noise_fill(w.seeds, w.N, w.V) if w.mode == 0 else None


def run_path(w, g, path, d=None):
    """(tokens, cache) of one call on the given path (1 persistent chain
    launches, 2 per-position launches, 3 the persistent step kernel); the
    documented workspace size covers every path."""
    if d is None:
        d = DeviceChain(w)
        if g is not None:
            d.set_gumbel(g)
    lm.markov_set_batch_path(path)
    say(f"  path {path}: {w.name} V={w.V} r={w.r} rows={w.rows} N={w.N}")
    d.tokens.fill_(-7)
    d.chain()
    lm.markov_status(d.workspace)
    lm.markov_set_batch_path(0)
    return d.results(), d


def oracle_rows(w, g, rows, c_dev):
    mask = np.zeros(w.rows, dtype=np.uint8)
    mask[rows] = 1
    tokens = np.full((w.rows, w.N), -7, dtype=np.int64)
    return oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g,
                        state_idx=w.state_idx, mult=w.mult, cap=w.cap, mode=w.mode, row_mask=mask,
                        tokens=tokens, cache=c_dev.copy(), cache_f32=w.cache_f32)


def check_exact(w, rows):
    rows = [b for b in rows if b < w.rows]
    g = noise_for(w)
    (t2, c2), _ = run_path(w, g, 2)
    (t1, c1), _ = run_path(w, g, 1)
    assert np.array_equal(t1, t2), "step path tokens differ from the persistent path's"
    assert np.array_equal(c1, c2), "step path cache differs from the persistent path's"
    if w.mode == 0:
        (t3, c3), _ = run_path(w, g, 3)
        assert np.array_equal(t3, t2), "persistent step kernel tokens differ from the per-position launches'"
        assert np.array_equal(c3, c2), "persistent step kernel cache differs from the per-position launches'"
    ref_t, ref_c = oracle_rows(w, g, rows, c2)
    sidx = np.arange(w.rows) if w.state_idx is None else w.state_idx
    for b in rows:
        if sidx[b] < 0:
            assert np.all(t2[b] == -7), f"padding row {b} written"
            continue
        assert np.array_equal(t2[b], ref_t[b]), f"row {b}: tokens differ from the oracle"
        assert np.array_equal(c2[sidx[b]], ref_c[sidx[b]]), f"row {b}: cache differs from the oracle"


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("V,r,rows,N", [
    (4096 + 16, 256, 200, 3),   # ragged vocabulary, four row blocks (the last partial)
    (2048 + 32, 512, 130, 4),   # r = 512
    (16, 256, 65, 2),           # the smallest vocabulary, one row past a block
])
def test_step_path_exact_integer_weights(V, r, rows, N, mode):
    rng = np.random.default_rng(V + rows)
    sidx = rng.permutation(rows + 7)[:rows].astype(np.int64)
    sidx[[1, rows // 2, rows - 1]] = -1
    temps = np.array([1.0, 0.7, 0.0, 1.5, 0.6], dtype=np.float32)[np.arange(rows) % 5]
    w = synth.make(f"step_V{V}_r{r}_m{mode}", V, r, rows, N, seed=V + r + rows, weights="int", base_std=2.0,
                   temperature=temps, state_idx=sidx, mode=mode)
    check_exact(w, sorted({0, 1, 2, 63, 64, 65, rows // 2, rows - 2, rows - 1}))


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("base_f32,cache_f32", [(True, False), (False, True), (True, True)])
def test_step_path_fp32_types(base_f32, cache_f32, mode):
    rows = 96
    w = synth.make(f"step_fl_m{mode}", 3000 - 8, 256, rows, 3, seed=91, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.0, 1.3] * 32, dtype=np.float32), mult=0.5,
                   base_f32=base_f32, cache_f32=cache_f32, mode=mode)
    check_exact(w, [0, 1, 2, 64, 95])


@pytest.mark.parametrize("V,r,rows,N", [
    (4096 + 16, 256, 200, 3),   # ragged vocabulary, four row blocks
    (2048 + 32, 512, 130, 4),   # r = 512
])
def test_step_path_inline_noise(V, r, rows, N):
    """Mode 0 with the noise drawn inside the step kernels (the persistent
    one, the per-position one, and the default path beyond 64 rows): the
    noise fill kernel's function, so the outputs equal those of the same
    path with the device's noise in memory bit for bit; sampled rows equal
    the oracle drawing its own noise."""
    rng = np.random.default_rng(V + rows + 1)
    sidx = rng.permutation(rows + 5)[:rows].astype(np.int64)
    sidx[[2, rows // 3, rows - 1]] = -1
    temps = np.array([1.0, 0.7, 0.0, 1.5, 0.6], dtype=np.float32)[np.arange(rows) % 5]
    w = synth.make(f"step_nz_V{V}_r{r}", V, r, rows, N, seed=V + r + rows + 1, weights="int", base_std=2.0,
                   temperature=temps, state_idx=sidx)
    d = DeviceChain(w)
    d.noise()  # the device's noise fill kernel
    (ts, cs), _ = run_path(w, None, 2, d)
    for path in (2, 3, 0):
        (t, c), _ = run_path(w, None, path, DeviceChain(w, noise_inline=True))
        assert np.array_equal(t, ts), f"path {path}: inline-noise tokens differ from the noise in memory"
        assert np.array_equal(c, cs), f"path {path}: inline-noise cache differs from the noise in memory"
    rows_chk = [b for b in (0, 1, 3, 63, 64, 65, rows // 2, rows - 2) if b < rows]
    g = noise_for(w)
    ref_t, ref_c = oracle_rows(w, g, rows_chk, cs)
    for b in rows_chk:
        if sidx[b] < 0:
            assert np.all(ts[b] == -7), f"padding row {b} written"
            continue
        assert np.array_equal(ts[b], ref_t[b]), f"row {b}: tokens differ from the oracle"
        assert np.array_equal(cs[sidx[b]], ref_c[sidx[b]]), f"row {b}: cache differs from the oracle"


@pytest.mark.parametrize("base_f32,cache_f32", [(True, False), (False, True), (True, True)])
def test_step_path_inline_noise_fp32_types(base_f32, cache_f32):
    """The inline-noise step kernels with fp32 base logits and/or an fp32
    cache equal the same paths with the device's noise in memory, and
    sampled rows equal the oracle."""
    rows = 96
    w = synth.make(f"step_nz_fl_{int(base_f32)}{int(cache_f32)}", 3000 - 8, 256, rows, 3, seed=191,
                   weights="int", base_std=2.0, temperature=np.array([1.0, 0.0, 1.3] * 32, dtype=np.float32),
                   mult=0.5, base_f32=base_f32, cache_f32=cache_f32)
    d = DeviceChain(w)
    d.noise()
    (ts, cs), _ = run_path(w, None, 2, d)
    for path in (2, 3):
        (t, c), _ = run_path(w, None, path, DeviceChain(w, noise_inline=True))
        assert np.array_equal(t, ts) and np.array_equal(c, cs), f"path {path}"
    sample = [0, 1, 2, 64, 95]
    ref_t, ref_c = oracle_rows(w, noise_for(w), sample, cs)
    for b in sample:
        assert np.array_equal(ts[b], ref_t[b]) and np.array_equal(cs[b], ref_c[b]), b


def test_persistent_step_kernel_many_positions():
    """72 positions of 130 rows (three row blocks, the last of two rows):
    the persistent step kernel keeps an arrival counter per position, more
    than fit in the 256 bytes before its best keys; all paths agree and
    sampled rows equal the oracle; drawing the noise inline gives the same
    outputs."""
    rows = 130
    w = synth.make("step_many_positions", 4096 + 16, 256, rows, 72, seed=101, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.0, 0.7, 1.5, 0.6] * 26, dtype=np.float32))
    check_exact(w, [0, 64, 128, 129])
    d = DeviceChain(w)
    d.noise()
    (ts, cs), _ = run_path(w, None, 3, d)
    (t, c), _ = run_path(w, None, 3, DeviceChain(w, noise_inline=True))
    assert np.array_equal(t, ts) and np.array_equal(c, cs)


def test_step_path_inline_noise_soft_cap():
    """Random weights with the output transform (multiplier 0.5, soft cap
    30): the inline-noise step kernels equal the same paths with the
    device's noise in memory bit for bit."""
    rows = 80
    w = synth.make("step_nz_cap", 8192, 256, rows, 3, seed=196, peaks=8,
                   temperature=np.array([1.0, 0.0, 0.6, 1.5] * 20, dtype=np.float32), mult=0.5, cap=30.0)
    d = DeviceChain(w)
    d.noise()
    (ts, cs), _ = run_path(w, None, 2, d)
    for path in (2, 3):
        (t, c), _ = run_path(w, None, path, DeviceChain(w, noise_inline=True))
        assert np.array_equal(t, ts) and np.array_equal(c, cs), f"path {path}"


@pytest.mark.parametrize("mode", [0, 1])
def test_step_path_more_chunks_than_compute_units(mode):
    """513 chunks (V = 262160 at r = 256): more workgroups than CUs, so the
    persistent step kernel does not apply and mode 0 runs one launch per
    position on every path; sampled rows equal the oracle."""
    rows = 70
    w = synth.make(f"step_wide_m{mode}", 262144 + 16, 256, rows, 2, seed=99 + mode, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.0, 0.7, 1.5, 0.6] * 14, dtype=np.float32), mode=mode)
    check_exact(w, [0, 1, 69])


def test_step_path_invcdf_nan_inf_and_ties():
    """Inverse CDF on the step path: rows whose logits hold NaN or +inf take
    the argmax rule, exact ties keep the lowest id, and the last chunk and
    ids past V are never drawn."""
    rows = 70
    w = synth.make("step_cdf_edges", 4096 + 48, 256, rows, 3, seed=97, weights="int", base_std=2.0,
                   temperature=np.array([1.0, 0.8, 0.0, 2.5, 1.0] * 14, dtype=np.float32), mode=1)
    base = w.base.copy()
    base[3, 1, [17, 4000]] = 0x7FC0   # NaN: argmax rule, lowest NaN id
    base[66, 0, [100, 2000]] = 0x7F80  # +inf: argmax rule, lowest id of the maximum
    base[10, 2, [5, 700, 3000]] = 0x4220  # an exact tie at 40.0
    base[69, :, -48:] = 0x42C8          # 100.0 on the ragged tail's ids
    w = dataclasses.replace(w, base=base)
    check_exact(w, [0, 3, 10, 64, 66, 69])


@pytest.mark.parametrize("mode", [0, 1])
def test_step_path_soft_cap(mode):
    """With the soft cap the two libraries' tanhf may differ in the last fp32
    bit, so the oracle comparison uses the tolerance walk; the two paths
    still agree bit for bit."""
    rows = 80
    w = synth.make(f"step_cap_m{mode}", 8192, 256, rows, 3, seed=96, peaks=8, temperature=np.array(
        [1.0, 0.0, 0.6, 1.5] * 20, dtype=np.float32), mult=0.5, cap=30.0, mode=mode)
    g = noise_for(w)
    (t2, c2), _ = run_path(w, g, 2)
    (t1, c1), _ = run_path(w, g, 1)
    assert np.array_equal(t1, t2) and np.array_equal(c1, c2)
    if mode == 0:
        (t3, c3), _ = run_path(w, g, 3)
        assert np.array_equal(t3, t2) and np.array_equal(c3, c2)
    st = chain_check.walk(w, t2, c2, g, rows=[0, 1, 2, 3, 64, 79])
    say("  " + st.summary())
    assert st.token_match >= st.pairs - 1


@pytest.mark.parametrize("mode", [0, 1])
def test_step_path_forced_for_small_batches(mode):
    """The knob runs 1, 3 and 64 rows through the step kernels too; outputs
    equal the persistent kernels' (one row, small batch and 64-row
    variants)."""
    for rows in (1, 3, 64):
        w = synth.make(f"step_small{rows}_m{mode}", 20000, 256, rows, 4, seed=92 + rows, weights="int",
                       base_std=2.0, temperature=0.9, mode=mode)
        check_exact(w, list(range(min(rows, 4))))


@pytest.mark.parametrize("mode", [0, 1])
def test_step_path_most_rows(mode):
    rows = lm.MARKOV_MAX_ROWS
    w = synth.make(f"step_max_m{mode}", 1024, 256, rows, 2, seed=93, weights="int", base_std=2.0,
                   temperature=1.0, mode=mode)
    g = noise_for(w)
    (t, c), _ = run_path(w, g, 0)  # the default path for this size
    sample = [0, 63, 64, 1000, 2048, 4095]
    ref_t, ref_c = oracle_rows(w, g, sample, c)
    for b in sample:
        assert np.array_equal(t[b], ref_t[b]) and np.array_equal(c[b], ref_c[b]), b


def test_step_path_repeat_calls_share_a_workspace_with_persistent_calls():
    """Step-path calls of both modes and persistent calls take turns on one
    workspace (all use its parity halves); every result equals the first of
    its kind."""
    big = synth.make("rep_big", 8192, 256, 100, 3, seed=94, temperature=0.8)
    bigc = synth.make("rep_big_cdf", 8192, 256, 90, 3, seed=98, temperature=1.0, mode=1)
    small = synth.make("rep_small", 8192, 256, 5, 3, seed=95, temperature=1.1)
    gb, gs = oracle.noise_fill(big.seeds, big.N, big.V), oracle.noise_fill(small.seeds, small.N, small.V)
    db, dc, ds = DeviceChain(big), DeviceChain(bigc), DeviceChain(small)
    ws = max((d.workspace for d in (db, dc, ds)), key=lambda t: t.numel())
    for d in (db, dc, ds):
        d.workspace = ws
    db.set_gumbel(gb)
    ds.set_gumbel(gs)
    ref = {}
    for k in range(30):
        d = (db, dc, ds)[k % 3]
        d.tokens.fill_(-7)
        d.chain()
        out = d.results()
        name = d.w.name
        if name in ref:
            assert np.array_equal(out[0], ref[name][0]) and np.array_equal(out[1], ref[name][1]), (k, name)
        else:
            ref[name] = (out[0].copy(), out[1].copy())
    lm.markov_status(ws)
    chain_check.walk(big, ref["rep_big"][0], ref["rep_big"][1], gb, rows=[0, 50, 99])
    chain_check.walk(bigc, ref["rep_big_cdf"][0], ref["rep_big_cdf"][1], None, rows=[0, 45, 89])
    chain_check.walk(small, ref["rep_small"][0], ref["rep_small"][1], gs)


@pytest.mark.parametrize("mode", [0, 1])
def test_step_path_dsv41_256_rows(mode):
    """The DeepSeek-sized 256-row batch on random weights: the step path
    equals the persistent path bit for bit, and sampled rows pass the
    oracle walk."""
    w = synth.workload("dsv41_256rows")
    if mode == 1:
        w = dataclasses.replace(w, name=w.name + "_invcdf", mode=1)
    g = noise_for(w)
    (t2, c2), _ = run_path(w, g, 2)
    (t1, c1), _ = run_path(w, g, 1)
    assert np.array_equal(t1, t2) and np.array_equal(c1, c2)
    if mode == 0:
        (t3, c3), _ = run_path(w, g, 3)
        assert np.array_equal(t3, t2) and np.array_equal(c3, c2)
    st = chain_check.walk(w, t2, c2, g, rows=[0, 1, 63, 64, 127, 128, 200, 255])
    say("  " + st.summary())
    chain_check.record(f"step_path_dsv41_256rows{'_invcdf' if mode else ''}_sampled", st)
    assert st.token_match >= 0.999 * st.pairs
