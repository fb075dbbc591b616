"""The C-ABI library loads, exports every symbol include/markov.h declares,
and rejects bad arguments on the host before any GPU work (CPU only)."""

import ctypes
import os
import re

import pytest

from markov_bias_chain_amd import binding as lm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "markov.h")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(markov_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_symbols() == sorted(lm.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lm.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name


def _round256(x):
    return -(-x // 256) * 256


def _step_halves(rows, N, chunks, mode):
    """The per-position paths' halves: mode 0 keeps each row's best key on a
    128-byte line for two positions and 4-byte tokens, or (the persistent
    step kernel) a 4-byte arrival counter per position, a line per
    (position, row) and 8-byte tagged tokens; mode 1 keeps an 8-byte key and
    a 4-byte sum per (row, chunk) and 4-byte tokens."""
    if mode == 0:
        arrive = _round256(N * 4)
        return max(_round256(256 + 2 * rows * 128 + rows * 4), _round256(arrive + N * rows * 128 + rows * 8))
    return _round256(256 + rows * chunks * 12 + rows * 4)


def test_workspace_bytes():
    # header + two halves, each the largest layout a call may use.  The
    # persistent kernel, mode 0: an 8-byte key per (step, row, chunk) and an
    # 8-byte reducer partial per (step, row, 64 chunks) (512-id chunks at
    # r=256); up to 8 rows keep 16 copies of each step's partials, 512 bytes apart
    chunks = -(-129280 // 512)
    red = -(-chunks // 64)
    half = max(_round256(8 * 1 * chunks * 8 + 8 * 16 * 64 * 8), _step_halves(1, 8, chunks, 0))
    assert lm.markov_workspace_bytes(1, 8, 129280, 256, 0) == 256 + 2 * half
    # one row without reducers (at most 64 chunks): one partial word per step, no copies
    assert lm.markov_workspace_bytes(1, 8, 4096, 256, 0) == 256 + 2 * max(
        _round256(8 * 8 * 8 + 8 * 8), _step_halves(1, 8, 8, 0))
    # more than 64 rows: launches of 64 rows and of the rest share the workspace
    assert lm.markov_workspace_bytes(65, 8, 129280, 256, 0) == 256 + 2 * max(
        _round256(8 * 64 * chunks * 8 + 8 * 64 * red * 8), _step_halves(65, 8, chunks, 0))
    half9 = max(_round256(8 * 9 * chunks * 8 + 8 * 9 * red * 8), _step_halves(9, 8, chunks, 0))
    assert lm.markov_workspace_bytes(9, 8, 129280, 256, 0) == 256 + 2 * half9
    # mode 1 adds 4-byte sums and one 8-byte token word per (step, row) in 16
    # copies, no partials
    half1 = max(_round256(8 * 64 * chunks * 12 + 8 * 16 * 64 * 8), _step_halves(64, 8, chunks, 1))
    assert lm.markov_workspace_bytes(64, 8, 129280, 256, 1) == 256 + 2 * half1
    # 256 rows: the per-position layouts are the larger
    assert lm.markov_workspace_bytes(256, 8, 129280, 256, 1) == 256 + 2 * max(
        half1, _step_halves(256, 8, chunks, 1))
    # the persistent step kernel's arrival counters outgrow 256 bytes at
    # more than 64 positions
    assert lm.markov_workspace_bytes(65, 256, 4096, 256, 0) >= 256 + 2 * _step_halves(65, 256, 16, 0)
    assert _step_halves(65, 256, 16, 0) == _round256(_round256(256 * 4) + 256 * 65 * 128 + 65 * 8)
    # r=512 chunks hold 256 ids
    c5 = 262144 // 256
    half5 = max(_round256(16 * 8 * c5 * 8 + 16 * 8 * 16 * 64 * 8), _step_halves(8, 16, c5, 0))  # <= 8 rows: partial copies
    assert lm.markov_workspace_bytes(8, 16, 262144, 512, 0) == 256 + 2 * half5


@pytest.mark.parametrize("args", [
    (0, 8, 1024, 256, 0),      # rows
    (4097, 8, 1024, 256, 0),
    (1, 0, 1024, 256, 0),      # steps
    (1, 257, 1024, 256, 0),
    (1, 8, 1000, 256, 0),      # vocab % 16
    (1, 8, 0, 256, 0),
    (1, 8, 1024, 128, 0),      # rank
    (1, 8, 1024, 384, 0),
    (1, 8, 1024, 256, 2),      # mode
])
def test_unsupported_shapes(args):
    lib = lm.load()
    assert lib.markov_workspace_bytes(*args) == 0
    assert lib.markov_grid(*args) == lm.MARKOV_E_UNSUPPORTED
    assert lm.markov_last_error() != ""


def _sample(**kw):
    """markov_chain_sample with fake (never dereferenced) aligned pointers:
    argument checks run on the host before any HIP call."""
    lib = lm.load()
    P = 1 << 20  # a 256-byte aligned dummy address
    a = dict(base=P, brs=8 * 1024, bss=1024, head=P, embed=P, prev=P, temp=P, seeds=P,
             gumbel=P, sidx=None, mult=1.0, cap=0.0, rows=1, steps=8, vocab=1024, rank=256,
             mode=0, tok=P, trs=8, cache=P, states=1, crs=8 * 1024, css=1024, ws=P,
             wsb=lm.markov_workspace_bytes(1, 8, 1024, 256, 0), stream=None)
    a.update(kw)
    return lib.markov_chain_sample(
        a["base"], a["brs"], a["bss"], a["head"], a["embed"], a["prev"], a["temp"], a["seeds"],
        a["gumbel"], a["sidx"], a["mult"], a["cap"], a["rows"], a["steps"], a["vocab"],
        a["rank"], a["mode"], a["tok"], a["trs"], a["cache"], a["states"], a["crs"], a["css"], a["ws"],
        a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(base=None), lm.MARKOV_E_INVAL),
    (dict(head=None), lm.MARKOV_E_INVAL),
    (dict(gumbel=None), lm.MARKOV_E_INVAL),                     # mode 0 needs noise
    (dict(mode=1, seeds=None, gumbel=None), lm.MARKOV_E_INVAL),  # mode 1 needs seeds
    (dict(cache=(1 << 20) + 2), lm.MARKOV_E_INVAL),             # unaligned
    (dict(ws=(1 << 20) + 16), lm.MARKOV_E_INVAL),               # workspace alignment
    (dict(bss=1000), lm.MARKOV_E_INVAL),                        # step stride < vocab
    (dict(css=1028), lm.MARKOV_E_INVAL),                        # stride % 8
    (dict(wsb=64), lm.MARKOV_E_INVAL),                          # workspace too small
    (dict(cap=-1.0), lm.MARKOV_E_INVAL),
    (dict(mult=float("inf")), lm.MARKOV_E_INVAL),
    (dict(states=0), lm.MARKOV_E_INVAL),
    (dict(rows=2, states=1, trs=8), lm.MARKOV_E_INVAL),          # no state_idx: states >= rows
    (dict(rank=384), lm.MARKOV_E_UNSUPPORTED),
    (dict(rows=4097), lm.MARKOV_E_UNSUPPORTED),
    (dict(mode=2 | lm.MARKOV_CACHE_F32), lm.MARKOV_E_UNSUPPORTED),  # a bad mode with a dtype flag
    (dict(mode=lm.MARKOV_BASE_F32, bss=1000), lm.MARKOV_E_INVAL),  # flags do not skip the checks
    (dict(mode=lm.MARKOV_CACHE_F32, cache=(1 << 20) + 8), lm.MARKOV_E_INVAL),
    (dict(mode=1 | lm.MARKOV_NOISE_INLINE), lm.MARKOV_E_INVAL),          # inline noise is mode 0's
    (dict(mode=lm.MARKOV_NOISE_INLINE, seeds=None), lm.MARKOV_E_INVAL),  # it needs seeds
    (dict(mode=lm.MARKOV_NOISE_INLINE, gumbel=None, wsb=64), lm.MARKOV_E_INVAL),  # gumbel may be NULL
])
def test_invalid_arguments_rejected_on_host(kw, code):
    assert _sample(**kw) == code
    assert lm.markov_last_error()


def test_inline_noise_needs_no_gumbel():
    # the checks pass the missing noise and stop at the (too small) workspace
    assert _sample(mode=lm.MARKOV_NOISE_INLINE, gumbel=None, wsb=64) == lm.MARKOV_E_INVAL
    assert "workspace" in lm.markov_last_error()
    assert _sample(mode=0, gumbel=None, wsb=64) == lm.MARKOV_E_INVAL
    assert "gumbel" in lm.markov_last_error()


def test_noise_fill_rejects_bad_arguments():
    lib = lm.load()
    P = 1 << 20
    assert lib.markov_noise_fill(None, P, 1, 1, 16, None) == lm.MARKOV_E_INVAL
    assert lib.markov_noise_fill(P + 4, P, 1, 1, 16, None) == lm.MARKOV_E_INVAL
    assert lib.markov_noise_fill(P, P, 1, 1, 20, None) == lm.MARKOV_E_UNSUPPORTED
    assert lib.markov_noise_fill(P, P, 0, 1, 16, None) == lm.MARKOV_E_UNSUPPORTED


def test_set_grid_roundtrip():
    old = lm.markov_set_grid(7)
    assert lm.markov_set_grid(old) == 7


def test_binding_refuses_cpu_tensors():
    import torch
    w = torch.zeros(4, dtype=torch.float32)
    s = torch.zeros(1, dtype=torch.int64)
    with pytest.raises(ValueError):
        lm.markov_noise_fill(w.view(1, 1, 4), s)


def test_dtype_flags_do_not_change_shape_queries():
    for f in (0, lm.MARKOV_BASE_F32, lm.MARKOV_CACHE_F32, lm.MARKOV_BASE_F32 | lm.MARKOV_CACHE_F32,
              lm.MARKOV_NOISE_INLINE):
        assert lm.markov_workspace_bytes(3, 8, 4096, 256, f) == lm.markov_workspace_bytes(3, 8, 4096, 256, 0)
        assert lm.markov_workspace_bytes(3, 8, 4096, 512, 1 | f) == lm.markov_workspace_bytes(3, 8, 4096, 512, 1)


def test_binding_refuses_other_element_types():
    import torch
    base = torch.zeros(1, 1, 16, dtype=torch.float16)
    with pytest.raises(TypeError):
        lm.markov_chain_sample(base, base, base, base, base, base, base, base)


def test_noalloc_refuses_shapes_beyond_its_scratch():
    """markov_chain_sample_noalloc takes the shapes whose workspace fits its
    static scratch and refuses larger ones on the host (fake, never
    dereferenced pointers; no HIP call is made before the refusal)."""
    lib = lm.load()
    P = 1 << 20
    rows, steps, vocab = 64, 256, 129280
    assert lm.markov_workspace_bytes(rows, steps, vocab, 256, 0) > 8 << 20
    rc = lib.markov_chain_sample_noalloc(
        P, steps * vocab, vocab, P, P, P, P, P, P, None, 1.0, 0.0, rows, steps, vocab, 256,
        lm.MARKOV_NOISE_INLINE, P, steps, P, rows, steps * vocab, vocab, None)
    assert rc == lm.MARKOV_E_UNSUPPORTED
    assert "workspace" in lm.markov_last_error()
    # the argument checks are those of markov_chain_sample
    rc = lib.markov_chain_sample_noalloc(
        None, 8 * 1024, 1024, P, P, P, P, P, P, None, 1.0, 0.0, 1, 8, 1024, 256, 0, P, 8, P, 1,
        8 * 1024, 1024, None)
    assert rc == lm.MARKOV_E_INVAL
