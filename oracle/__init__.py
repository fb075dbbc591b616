"""CPU oracle of the DSpark sequential Markov draft-sampling chain.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg may import this package; the product path
(``markov_bias_chain_amd``) never does.  The arithmetic lives in
``markov_oracle.c`` (plain single-threaded C); this module only builds it with
gcc and marshals numpy arrays through ctypes.
"""

from .oracle import (  # noqa: F401
    DIAG,
    bf16_round_f32,
    bf16_round_f64,
    bf16_to_f32,
    build,
    chain,
    gumbel,
    hash_step,
    hash_vocab,
    log_f32,
    noise_fill,
    splitmix64,
    splitmix64_mix,
    step,
    uniform,
    uniform_range,
)
