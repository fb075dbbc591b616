"""HIP-graph capture of the hot path (noise fork on a side stream, join,
chain) through the C ABI: every replay must equal an eager step on the same
inputs, bit for bit, with the program's own eager work and synchronisations
between replays; the first replay is also checked against the CPU oracle
(integer-valued weights make every fp32 sum order-exact)."""

import numpy as np
import pytest
import torch

import oracle
from markov_bias_chain_amd import binding, synth
from markov_bias_chain_amd.device import DeviceChain

pytestmark = pytest.mark.gpu


def _set_inputs(d: DeviceChain, prev: np.ndarray, seeds: np.ndarray) -> None:
    d.prev.copy_(torch.from_numpy(prev))
    d.seeds.copy_(torch.from_numpy(seeds))


@pytest.mark.parametrize("mode,rows", [(0, 1), (0, 3), (1, 2)])
def test_graph_replays_match_eager(mode, rows):
    V, r, N = 8192 + 16, 256, 5
    w = synth.make(f"graph_m{mode}_b{rows}", V, r, rows, N, seed=77 + rows, weights="int",
                   base_std=2.0, temperature=[1.0, 0.0, 0.7][:rows], mode=mode)
    d = DeviceChain(w)
    eager = DeviceChain(w)
    g = d.capture_step()
    rng = np.random.default_rng(78 + rows)
    for k in range(4):
        prev = rng.integers(0, V, size=rows, dtype=np.int64)
        seeds = rng.integers(-2**63, 2**63 - 1, size=rows, dtype=np.int64)
        _set_inputs(d, prev, seeds)
        _set_inputs(eager, prev, seeds)
        g.replay()
        # eager work of the program's own between the replay and the check
        torch.ones(1 << 20, device=d.device).sum().item()
        eager.step()
        binding.markov_status(d.workspace)
        binding.markov_status(eager.workspace)
        t_g, c_g = d.results()
        t_e, c_e = eager.results()
        assert np.array_equal(t_g, t_e), f"replay {k}: tokens differ from the eager step"
        assert np.array_equal(c_g, c_e), f"replay {k}: cache differs from the eager step"
        if k == 0:
            w.prev[:] = prev
            w.seeds[:] = seeds
            # the chain given the device's own noise (the noise kernel has its
            # own parity test)
            gum = d.gumbel.cpu().numpy() if mode == 0 else None
            ref_t, ref_c = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds,
                                        gumbel=gum, mode=mode)
            assert np.array_equal(t_g, ref_t)
            assert np.array_equal(c_g, ref_c)
