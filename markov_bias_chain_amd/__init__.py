"""MI355X (gfx950) DSpark sequential Markov draft-sampling chain.

The hot path is libmarkov.so (HIP kernels behind the C ABI of
include/markov.h); ``binding`` is its Python binding and ``device`` holds
per-call device buffers.  ``synth`` draws seeded synthetic inputs.
"""

from .binding import (  # noqa: F401
    MARKOV_MODE_GUMBEL,
    MARKOV_MODE_INVCDF,
    MarkovError,
    markov_chain_sample,
    markov_grid,
    markov_last_error,
    markov_noise_fill,
    markov_set_grid,
    markov_status,
    markov_workspace,
    markov_workspace_bytes,
)
