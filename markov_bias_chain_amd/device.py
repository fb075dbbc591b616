"""Device buffers for one chain call: upload a synthetic workload, allocate
the outputs and the workspace, and run the two C-ABI calls on torch streams.
Marshalling only; the arithmetic is in libmarkov.so."""

from __future__ import annotations

import numpy as np
import torch

from . import binding as lm
from .synth import Workload


def to_device_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceChain:
    """All device tensors of one workload, allocated once (so a HIP graph or
    a timing loop sees fixed addresses)."""

    def __init__(self, w: Workload, device="cuda", token_fill: int = -7, cache_fill: int = 0xABCD,
                 noise_inline: bool = False):
        """noise_inline (mode 0): the chain kernel draws the Gumbel noise
        itself from the seeds; no noise buffer is allocated."""
        self.w = w
        self.noise_inline = bool(noise_inline) and w.mode == 0
        dev = torch.device(device)
        self.device = dev
        self.head = to_device_bf16(w.head, dev)
        self.embed = to_device_bf16(w.embed, dev)
        self.base = (torch.from_numpy(np.ascontiguousarray(w.base)).to(dev) if w.base.dtype == np.float32
                     else to_device_bf16(w.base, dev))
        self.prev = torch.from_numpy(w.prev).to(dev)
        self.seeds = torch.from_numpy(w.seeds).to(dev)
        self.temperature = torch.from_numpy(w.temperature).to(dev)
        self.state_idx = None if w.state_idx is None else torch.from_numpy(w.state_idx).to(dev)
        self.gumbel = torch.empty((w.rows, w.N, w.V), dtype=torch.float32, device=dev) \
            if w.mode == 0 and not self.noise_inline else None
        self.tokens = torch.full((w.rows, w.N), token_fill, dtype=torch.int64, device=dev)
        if w.cache_f32:
            self.cache = torch.full((w.states, w.N, w.V), float("nan"), dtype=torch.float32, device=dev)
        else:
            fill = cache_fill - 0x10000 if cache_fill >= 0x8000 else cache_fill  # as int16 bits
            self.cache = torch.full((w.states, w.N, w.V), fill, dtype=torch.int16,
                                    device=dev).view(torch.bfloat16)
        self.workspace = lm.markov_workspace(w.rows, w.N, w.V, w.r, w.mode, device=dev)
        self.side = torch.cuda.Stream(dev)

    def set_gumbel(self, g: np.ndarray) -> None:
        """Use the given noise (e.g. drawn by another implementation)."""
        self.gumbel.copy_(torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)))

    def noise(self, stream=None) -> None:
        lm.markov_noise_fill(self.gumbel, self.seeds, stream=stream)

    def chain(self, stream=None) -> None:
        w = self.w
        lm.markov_chain_sample(
            self.base, self.head, self.embed, self.prev, self.temperature, self.tokens,
            self.cache, self.workspace, gumbel=self.gumbel, seeds=self.seeds,
            state_idx=self.state_idx, output_multiplier=w.mult, soft_cap=w.cap,
            mode=w.mode | (lm.MARKOV_NOISE_INLINE if self.noise_inline else 0), stream=stream)

    def step(self) -> None:
        """One pass of the hot path: the noise on a side stream forked after
        the current stream's work and joined before the chain, then the chain
        (with inline noise, the chain alone)."""
        cur = torch.cuda.current_stream(self.device)
        if self.w.mode == 0 and not self.noise_inline:
            self.side.wait_stream(cur)
            self.noise(stream=self.side)
            cur.wait_stream(self.side)
        self.chain(stream=cur)

    def capture_step(self) -> torch.cuda.CUDAGraph:
        """A HIP graph of one step(): the noise fork on the side stream, the
        join and the chain, replayable with g.replay() on fixed buffers (the
        workspace needs no reset between calls, and no memset is recorded).
        One eager step runs first so that every one-time set-up (kernel
        attributes, library loading) happens outside the capture."""
        self.step()
        torch.cuda.synchronize(self.device)
        lm.markov_status(self.workspace)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize(self.device)
        return g

    def results(self):
        """(tokens int64 [rows, N], cache [states, N, V]: uint16 bf16 bits, or
        float32 values for an fp32 cache) on the host."""
        torch.cuda.synchronize(self.device)
        c = self.cache.cpu().numpy() if self.cache.dtype == torch.float32 else bf16_bits(self.cache)
        return self.tokens.cpu().numpy(), c
