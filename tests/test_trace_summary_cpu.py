"""The tracing tool's summaries on synthetic clock stamps with known answers
(CPU only; no library is loaded)."""

import numpy as np

from markov_bias_chain_amd import trace


def test_exchange_probe_summary():
    # 20 rounds of 8 workgroups: publications 10 ticks apart from each
    # round's start (1000 ticks apart), the maximum known 100 + g ticks after
    # the last publication
    R, G = 20, 8
    st = np.zeros((R, G, 2), dtype=np.uint64)
    for r in range(R):
        st[r, :, 0] = 1000 * r + 10 * np.arange(G)
        st[r, :, 1] = 1000 * r + 70 + 100 + np.arange(G)
    s = trace.summarize_probe(st, skip=2)
    assert s["rounds"] == 18
    assert abs(s["spread"] - 0.70) < 1e-9          # 70 ticks of 10 ns
    assert abs(s["known_med"] - 1.035) < 1e-9      # median of 100 .. 107 ticks
    assert abs(s["known_last"] - 1.07) < 1e-9
    assert abs(s["period"] - 10.0) < 1e-9


def test_chain_summary_last_step_counts_only_the_waiting_workgroups():
    # 3 workgroups, 2 steps; at the last step only workgroup 0 stamps the
    # winner (phase 4), as the chain kernel does for mode 0 with at most 8 rows
    G, N = 3, 2
    t = np.zeros((G, N, trace.TRACE_PHASES), dtype=np.int64)
    for g in range(G):
        t[g, 0, 6] = 100 + g          # entry
        t[g, 0, 7] = 200 + g          # prologue done
        for i in range(N):
            base = 1000 * (i + 1)
            t[g, i, 0] = base + g     # step start
            t[g, i, 1] = base + 50    # local work done
            t[g, i, 2] = base + 60 + g  # published
            t[g, i, 5] = base + 500   # step end
    t[:, 0, 4] = [300 + 1000 + 62, 1000 + 400 + 62, 1000 + 500 + 62]  # after the last publication (1062)
    t[0, 1, 4] = 2000 + 62 + 80
    s = trace.summarize([t], G, N, mode=0)["steps"]
    assert abs(s["win_med"][0] - 4.0) < 1e-9 and abs(s["win_max"][0] - 5.0) < 1e-9
    assert abs(s["win_med"][1] - 0.8) < 1e-9 and abs(s["win_max"][1] - 0.8) < 1e-9
    assert abs(s["spread"][0] - 0.02) < 1e-9
