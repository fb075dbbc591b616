"""The noise kernel's log table is what its generator writes, and its entries
are the logarithms they claim to be (CPU only)."""

import importlib.util
import math
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "markov_bias_chain_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_log_table", os.path.join(CSRC, "gen_log_table.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _arrays(text):
    body = re.search(r"g_log_tab\[kLogTable\] = \{(.*?)\n\};", text, re.S).group(1)
    pairs = re.findall(r"\{([^,{}]+), ([^,{}]+)\}", body)
    return [float.fromhex(c) for c, _ in pairs], [float.fromhex(v) for _, v in pairs]


def test_committed_table_matches_generator():
    with open(os.path.join(CSRC, "log_table.inc")) as f:
        assert f.read() == _gen().table_text()


def test_table_entries():
    c, nlc = _arrays(_gen().table_text())
    assert len(c) == len(nlc) == 92
    for k, (cj, v) in enumerate(zip(c, nlc)):
        j = k - 38
        # c_j is the fp32 value nearest 1 / (1 + j/128), held exactly
        assert float(np.float32(cj)) == cj
        assert abs(cj * (1 + j / 128) - 1) <= 2 ** -24
        # nlc_j = -ln(c_j) to within an ulp of fp64 (libm's log is not exact)
        assert abs(v + math.log(cj)) <= 2 ** -52 * max(abs(v), 2 ** -60)
    assert nlc[38] == 0.0 and c[38] == 1.0
