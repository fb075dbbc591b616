"""Python binding of libmarkov (include/markov.h): argument marshalling only.

Each function takes torch tensors (device memory and streams come from
PyTorch), checks dtypes, devices and shapes, and calls the C entry point of
the same name; every step of the chain runs in the HIP kernels of
libmarkov.so.  There is no fallback: if the library is missing or a call
fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmarkov.so")

MARKOV_OK = 0
MARKOV_E_INVAL = -1
MARKOV_E_UNSUPPORTED = -2
MARKOV_E_HIP = -3
MARKOV_E_DEVICE = -4
MARKOV_MODE_GUMBEL = 0
MARKOV_MODE_INVCDF = 1
MARKOV_BASE_F32 = 0x10
MARKOV_CACHE_F32 = 0x20
MARKOV_NOISE_INLINE = 0x40  # mode 0: the chain draws the noise from seeds
MARKOV_MAX_ROWS = 4096
MARKOV_MAX_STEPS = 256

# every symbol include/markov.h declares
EXPORTS = (
    "markov_workspace_bytes",
    "markov_noise_fill",
    "markov_chain_sample",
    "markov_chain_sample_noalloc",
    "markov_status",
    "markov_last_error",
    "markov_set_grid",
    "markov_set_batch_path",
    "markov_set_wait_limit",
    "markov_grid",
)

_lock = threading.Lock()
_lib = None


class MarkovError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmarkov error {code}: {msg}")
        self.code = code


def load():
    """Load libmarkov.so (built in-tree by markov_bias_chain_amd.build)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m markov_bias_chain_amd.build` (there is no CPU fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        lib.markov_workspace_bytes.restype = sz
        lib.markov_workspace_bytes.argtypes = [i32] * 5
        lib.markov_noise_fill.restype = i32
        lib.markov_noise_fill.argtypes = [vp, vp, i32, i32, i32, vp]
        lib.markov_chain_sample.restype = i32
        lib.markov_chain_sample.argtypes = [
            vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, f32, f32,
            i32, i32, i32, i32, i32, vp, i64, vp, i64, i64, i64, vp, sz, vp]
        lib.markov_chain_sample_noalloc.restype = i32
        lib.markov_chain_sample_noalloc.argtypes = [
            vp, i64, i64, vp, vp, vp, vp, vp, vp, vp, f32, f32,
            i32, i32, i32, i32, i32, vp, i64, vp, i64, i64, i64, vp]
        lib.markov_status.restype = i32
        lib.markov_status.argtypes = [vp, vp]
        lib.markov_last_error.restype = ctypes.c_char_p
        lib.markov_last_error.argtypes = []
        lib.markov_set_grid.restype = i32
        lib.markov_set_grid.argtypes = [i32]
        lib.markov_set_batch_path.restype = i32
        lib.markov_set_batch_path.argtypes = [i32]
        lib.markov_set_wait_limit.restype = ctypes.c_longlong
        lib.markov_set_wait_limit.argtypes = [ctypes.c_longlong]
        lib.markov_grid.restype = i32
        lib.markov_grid.argtypes = [i32] * 5
        _lib = lib
        return lib


def _check(rc: int) -> int:
    if rc < 0:
        msg = load().markov_last_error().decode(errors="replace")
        raise MarkovError(rc, msg)
    return rc


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, dtype, name, device=None, contiguous=False):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    allowed = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in allowed:
        raise TypeError(f"{name} must be {' or '.join(map(str, allowed))}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ------------------------------------------------------------- entry points --

def markov_workspace_bytes(rows: int, steps: int, vocab: int, rank: int, mode: int = 0) -> int:
    n = load().markov_workspace_bytes(rows, steps, vocab, rank, mode)
    if n == 0:
        raise MarkovError(MARKOV_E_UNSUPPORTED, "unsupported shape for a workspace")
    return int(n)


def markov_workspace(rows: int, steps: int, vocab: int, rank: int, mode: int = 0,
                     device=None) -> torch.Tensor:
    """A zeroed workspace tensor (uint8) sized for this shape."""
    n = markov_workspace_bytes(rows, steps, vocab, rank, mode)
    return torch.zeros(n, dtype=torch.uint8, device=device or "cuda")


def markov_noise_fill(gumbel: torch.Tensor, seeds: torch.Tensor, stream=None) -> None:
    """Fill gumbel[rows, steps, vocab] (fp32) from seeds[rows] (int64)."""
    _need(gumbel, torch.float32, "gumbel", contiguous=True)
    _need(seeds, torch.int64, "seeds", gumbel.device, contiguous=True)
    if gumbel.dim() != 3 or seeds.shape != (gumbel.shape[0],):
        raise ValueError("gumbel must be [rows, steps, vocab] and seeds [rows]")
    rows, steps, vocab = gumbel.shape
    _check(load().markov_noise_fill(_ptr(gumbel), _ptr(seeds), rows, steps, vocab, _stream(stream)))


def markov_chain_sample(base_logits: torch.Tensor, head: torch.Tensor, embed: torch.Tensor,
                        prev_tokens: torch.Tensor, temperature: torch.Tensor,
                        draft_tokens: torch.Tensor, cache: torch.Tensor,
                        workspace: torch.Tensor | None, *, gumbel: torch.Tensor | None = None,
                        seeds: torch.Tensor | None = None,
                        state_idx: torch.Tensor | None = None,
                        output_multiplier: float = 1.0, soft_cap: float = 0.0,
                        mode: int = MARKOV_MODE_GUMBEL, stream=None) -> None:
    """Run the whole chain: draft_tokens[rows, >=N] (int64) and
    cache[states, N, >=V] (bf16 or fp32) are written in place.  base_logits
    are bf16 or fp32; the element types are passed to the library as flags
    of `mode`.  workspace None calls markov_chain_sample_noalloc (the
    library's own static scratch; no device memory is allocated)."""
    dev = base_logits.device
    _need(base_logits, (torch.bfloat16, torch.float32), "base_logits", dev)
    _need(head, torch.bfloat16, "head", dev, contiguous=True)
    _need(embed, torch.bfloat16, "embed", dev, contiguous=True)
    _need(prev_tokens, torch.int64, "prev_tokens", dev, contiguous=True)
    _need(temperature, torch.float32, "temperature", dev, contiguous=True)
    _need(draft_tokens, torch.int64, "draft_tokens", dev)
    _need(cache, (torch.bfloat16, torch.float32), "cache", dev)
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace", dev, contiguous=True)
    if base_logits.dim() != 3 or base_logits.stride(2) != 1:
        raise ValueError("base_logits must be [rows, N, V] with unit last stride")
    rows, steps, vocab = base_logits.shape
    if head.dim() != 2 or embed.dim() != 2 or head.shape[1] != embed.shape[1]:
        raise ValueError("head and embed must be [V, r] with the same r")
    if head.shape[0] < vocab or embed.shape[0] < vocab:
        raise ValueError("head and embed need at least V rows")
    rank = head.shape[1]
    if prev_tokens.shape != (rows,) or temperature.shape != (rows,):
        raise ValueError("prev_tokens and temperature must be [rows]")
    if draft_tokens.dim() != 2 or draft_tokens.shape[0] != rows or draft_tokens.shape[1] < steps \
            or draft_tokens.stride(1) != 1:
        raise ValueError("draft_tokens must be [rows, >=N] with unit last stride")
    if cache.dim() != 3 or cache.shape[1] < steps or cache.shape[2] < vocab or cache.stride(2) != 1:
        raise ValueError("cache must be [states, >=N, >=V] with unit last stride")
    if gumbel is not None:
        _need(gumbel, torch.float32, "gumbel", dev, contiguous=True)
        if gumbel.shape != (rows, steps, vocab):
            raise ValueError("gumbel must be [rows, N, V]")
    if seeds is not None:
        _need(seeds, torch.int64, "seeds", dev, contiguous=True)
        if seeds.shape != (rows,):
            raise ValueError("seeds must be [rows]")
    if state_idx is not None:
        _need(state_idx, torch.int64, "state_idx", dev, contiguous=True)
        if state_idx.shape != (rows,):
            raise ValueError("state_idx must be [rows]")
    args = (_ptr(base_logits), base_logits.stride(0), base_logits.stride(1),
            _ptr(head), _ptr(embed), _ptr(prev_tokens), _ptr(temperature), _ptr(seeds),
            _ptr(gumbel), _ptr(state_idx), float(output_multiplier), float(soft_cap),
            rows, steps, vocab, rank,
            int(mode) | (MARKOV_BASE_F32 if base_logits.dtype == torch.float32 else 0)
            | (MARKOV_CACHE_F32 if cache.dtype == torch.float32 else 0),
            _ptr(draft_tokens), draft_tokens.stride(0),
            _ptr(cache), cache.shape[0], cache.stride(0), cache.stride(1))
    if workspace is None:
        _check(load().markov_chain_sample_noalloc(*args, _stream(stream)))
    else:
        _check(load().markov_chain_sample(*args, _ptr(workspace), workspace.numel(), _stream(stream)))


def markov_chain_sample_noalloc(base_logits: torch.Tensor, head: torch.Tensor, embed: torch.Tensor,
                                prev_tokens: torch.Tensor, temperature: torch.Tensor,
                                draft_tokens: torch.Tensor, cache: torch.Tensor, **kw) -> None:
    """markov_chain_sample without a workspace: the library's static scratch
    holds the exchange state and no device memory is allocated."""
    markov_chain_sample(base_logits, head, embed, prev_tokens, temperature, draft_tokens, cache,
                        None, **kw)


def markov_status(workspace: torch.Tensor | None, stream=None) -> None:
    """Synchronise the stream and raise if the kernel reported an error
    (workspace None: the scratch of markov_chain_sample_noalloc on the
    current device)."""
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
    _check(load().markov_status(_ptr(workspace), _stream(stream)))


def markov_last_error() -> str:
    return load().markov_last_error().decode(errors="replace")


def markov_set_grid(g: int) -> int:
    return int(load().markov_set_grid(int(g)))


def markov_set_batch_path(path: int) -> int:
    """0 auto, 1 persistent launches, 2 step kernels (mode 0, noise in
    memory).  Returns the previous value."""
    return int(load().markov_set_batch_path(int(path)))


def markov_set_wait_limit(us: int) -> int:
    """Bound (microseconds) of the chain's cross-workgroup waits; negative
    restores the default.  Returns the previous bound."""
    return int(load().markov_set_wait_limit(int(us)))


def markov_grid(rows: int, steps: int, vocab: int, rank: int, mode: int = 0) -> int:
    return _check(load().markov_grid(rows, steps, vocab, rank, mode))
