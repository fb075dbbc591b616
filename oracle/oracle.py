"""ctypes marshalling for ``markov_oracle.c`` (test infrastructure only).

Every function here converts numpy arrays to pointers and calls the C oracle;
none of the method's arithmetic is in this file.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "markov_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DIAG = 8  # doubles of diagnostics per step (see markov_oracle.c)

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)


def build() -> str:
    """Compile the oracle with gcc (plain C11, no fp contraction)."""
    cmd = [
        "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
        "-fPIC", "-shared", _SRC, "-o", _LIB + ".tmp", "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        sig = {
            "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "orc_bf16_round": (ctypes.c_uint16, [ctypes.c_double]),
            "orc_bf16_round_f32_array": (None, [_f32p, _u16p, ctypes.c_size_t]),
            "orc_splitmix64_mix": (ctypes.c_uint64, [ctypes.c_uint64]),
            "orc_splitmix64": (ctypes.c_uint64, [ctypes.c_uint64]),
            "orc_hash_step": (ctypes.c_uint64, [ctypes.c_int64] * 3),
            "orc_hash_vocab": (ctypes.c_uint64, [ctypes.c_uint64, ctypes.c_int64]),
            "orc_uniform": (ctypes.c_float, [ctypes.c_uint64]),
            "orc_log_f32": (ctypes.c_float, [ctypes.c_float]),
            "orc_gumbel": (ctypes.c_float, [ctypes.c_float]),
            "orc_noise_fill": (None, [_f32p, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int]),
            "orc_uniform_range": (None, [_f32p] + [ctypes.c_int64] * 5),
            "orc_step": (
                ctypes.c_int64,
                [_u16p, _u16p, _u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                 ctypes.c_float, _f32p, ctypes.c_float, ctypes.c_float,
                 ctypes.c_float, ctypes.c_int, _u16p, _f64p, _u16p],
            ),
            "orc_step_t": (
                ctypes.c_int64,
                [ctypes.c_void_p, ctypes.c_int, _u16p, _u16p, ctypes.c_int, ctypes.c_int,
                 ctypes.c_int64, ctypes.c_float, _f32p, ctypes.c_float, ctypes.c_float,
                 ctypes.c_float, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, _f64p, _u16p],
            ),
            "orc_chain_t": (
                ctypes.c_int,
                [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p,
                 ctypes.c_int, ctypes.c_int, _i64p, _f32p, _i64p, _f32p, _i64p, ctypes.c_float,
                 ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p,
                 _i64p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64],
            ),
            "orc_chain": (
                ctypes.c_int,
                [_u16p, ctypes.c_int64, ctypes.c_int64, _u16p, _u16p, ctypes.c_int,
                 ctypes.c_int, _i64p, _f32p, _i64p, _f32p, _i64p, ctypes.c_float,
                 ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, _u8p,
                 _i64p, _u16p, ctypes.c_int64, ctypes.c_int64],
            ),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a, typ):
    if a is None:
        return None
    return a.ctypes.data_as(typ)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- scalars --

def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (a bit placement only)."""
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def bf16_round_f64(x: float) -> int:
    return int(_load().orc_bf16_round(float(x)))


def bf16_round_f32(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().orc_bf16_round_f32_array(_ptr(x, _f32p), _ptr(out, _u16p), x.size)
    return out


def splitmix64_mix(z: int) -> int:
    return int(_load().orc_splitmix64_mix(z & 0xFFFFFFFFFFFFFFFF))


def splitmix64(x: int) -> int:
    return int(_load().orc_splitmix64(x & 0xFFFFFFFFFFFFFFFF))


def hash_step(seed: int, row: int, step: int) -> int:
    return int(_load().orc_hash_step(seed, row, step))


def hash_vocab(prefix: int, v: int) -> int:
    return int(_load().orc_hash_vocab(prefix & 0xFFFFFFFFFFFFFFFF, v))


def uniform(h: int) -> float:
    return float(_load().orc_uniform(h & 0xFFFFFFFFFFFFFFFF))


def log_f32(x: float) -> float:
    """The oracle's fp32 natural log (the one inside the Gumbel draw)."""
    return float(_load().orc_log_f32(x))


def gumbel(u: float) -> float:
    return float(_load().orc_gumbel(u))


def uniform_range(seed: int, row: int, step: int, v0: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.float32)
    _load().orc_uniform_range(_ptr(out, _f32p), seed, row, step, v0, count)
    return out


# ----------------------------------------------------------------- arrays --

def noise_fill(seeds: np.ndarray, steps: int, vocab: int) -> np.ndarray:
    """gumbel[rows, steps, vocab] float32 drawn from seeds[rows]."""
    seeds = _c(seeds, np.int64)
    rows = seeds.shape[0]
    out = np.empty((rows, steps, vocab), dtype=np.float32)
    _load().orc_noise_fill(_ptr(out, _f32p), _ptr(seeds, _i64p), rows, steps, vocab)
    return out


def _base_array(a):
    """bf16 bits (uint16) stay as they are; float32 values select fp32 base
    logits."""
    a = np.asarray(a)
    if a.dtype == np.float32:
        return np.ascontiguousarray(a), 1
    return _c(a, np.uint16), 0


def step(base_row, head, embed, prev, temperature, gumbel_row=None, u=0.0,
         mult=1.0, cap=0.0, mode=0, with_diag=False, with_bias=False, cache_f32=False):
    """One position of one row: returns (token, cache_row[, diag][, bias]).
    base_row is bf16 bits (uint16) or fp32 values; the cache row is bf16 bits,
    or fp32 values with cache_f32."""
    base_row, base_f32 = _base_array(base_row)
    head = _c(head, np.uint16)
    embed = _c(embed, np.uint16)
    V, r = head.shape
    assert base_row.shape == (V,) and embed.shape[1] == r
    g = None if gumbel_row is None else _c(gumbel_row, np.float32)
    cache = np.empty(V, dtype=np.float32 if cache_f32 else np.uint16)
    diag = np.zeros(DIAG, dtype=np.float64)
    bias = np.empty(V, dtype=np.uint16) if with_bias else None
    tok = _load().orc_step_t(
        base_row.ctypes.data, base_f32, _ptr(head, _u16p), _ptr(embed, _u16p), V, r,
        int(prev), float(temperature), _ptr(g, _f32p), float(u), float(mult),
        float(cap), int(mode), cache.ctypes.data, int(bool(cache_f32)), _ptr(diag, _f64p),
        _ptr(bias, _u16p))
    out = (int(tok), cache)
    if with_diag:
        out += (diag,)
    if with_bias:
        out += (bias,)
    return out


def chain(base, head, embed, prev_tokens, temperature, seeds, gumbel=None,
          state_idx=None, mult=1.0, cap=0.0, mode=0, row_mask=None,
          tokens=None, cache=None, cache_f32=False):
    """The whole chain.  base [rows, N, V] bf16 bits (uint16) or fp32 values;
    head/embed [V, r]; returns (tokens [rows, N] int64, cache [states, N, V]
    uint16 bf16 bits, or float32 with cache_f32).  Rows that are masked out or
    inert keep what ``tokens``/``cache`` held."""
    base, base_f32 = _base_array(base)
    head = _c(head, np.uint16)
    embed = _c(embed, np.uint16)
    rows, N, V = base.shape
    r = head.shape[1]
    assert head.shape[0] >= V and embed.shape[0] >= V and embed.shape[1] == r
    prev = _c(prev_tokens, np.int64)
    temp = _c(temperature, np.float32)
    seeds = _c(seeds, np.int64)
    g = None if gumbel is None else _c(gumbel, np.float32)
    if g is not None:
        assert g.shape == (rows, N, V)
    sidx = None if state_idx is None else _c(state_idx, np.int64)
    states = rows if sidx is None else max(int(sidx.max()) + 1, 1)
    if tokens is None:
        tokens = np.full((rows, N), -7, dtype=np.int64)
    cdt = np.float32 if cache_f32 else np.uint16
    if cache is None:
        cache = np.zeros((states, N, V), dtype=cdt)
    assert tokens.flags.c_contiguous and tokens.dtype == np.int64
    assert cache.flags.c_contiguous and cache.dtype == cdt
    mask = None if row_mask is None else _c(row_mask, np.uint8)
    rc = _load().orc_chain_t(
        base.ctypes.data, base_f32, N * V, V, _ptr(head, _u16p), _ptr(embed, _u16p), V, r,
        _ptr(prev, _i64p), _ptr(temp, _f32p), _ptr(seeds, _i64p), _ptr(g, _f32p),
        _ptr(sidx, _i64p), float(mult), float(cap), rows, N, int(mode),
        _ptr(mask, _u8p), _ptr(tokens, _i64p), cache.ctypes.data, int(bool(cache_f32)),
        cache.shape[1] * cache.shape[2], cache.shape[2])
    if rc != 0:
        raise ValueError("oracle: a previous token outside [0, V)")
    return tokens, cache
