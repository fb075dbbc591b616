"""Per-step time breakdown of the chain kernel, from its tracing build.

    python -m markov_bias_chain_amd.build --trace     # libmarkov_trace.so
    python -m markov_bias_chain_amd.trace --workload dsv41_single_row --noise inline

The tracing build (MARKOV_TRACE) is the same kernel source with clock stamps
at fixed points of every step, one thread per workgroup (the phases are
listed in markov.hip next to trace_buf).  This tool runs warm (back to back)
or cold (a 1 GiB read before each call) calls of a workload through that
library, reads the stamps after each call and prints a markdown summary:
per step, medians over the calls of

  * local work: bias and epilogue of wave 0 (median over workgroups);
  * last key out: the last workgroup's publication, from the step's first
    start;
  * winner known: when wave 0 of a workgroup knows the winner, after the last
    publication (median and slowest workgroup);
  * step: from the step's first start to the next step's first start.

With --exchange-probe it measures the exchange's floor instead: the tracing
build's probe kernel runs rounds of the one-row exchange with no other work
on one workgroup per CU (two levels through the reducers and the partials'
copies, as the chain kernel does, or all-to-all) and this tool prints, over
the rounds, the spread of the publications and when each workgroup knows
the maximum after the last publication (median and slowest workgroup).

It is a measuring tool: nothing of the chain's arithmetic is here.
"""

from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TRACE_WGS, TRACE_STEPS, TRACE_PHASES = 1024, 32, 12
TICK_US = 0.01  # 100 MHz


def load_trace_library():
    from markov_bias_chain_amd import binding, build

    if not os.path.exists(build.TRACE_LIB):
        raise RuntimeError(f"{build.TRACE_LIB} is missing: run `python -m markov_bias_chain_amd.build --trace`")
    binding.LIB_PATH = build.TRACE_LIB
    lib = binding.load()
    lib.markov_trace_read.restype = ctypes.c_int
    lib.markov_trace_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.markov_trace_exchange_probe.restype = ctypes.c_int
    lib.markov_trace_exchange_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return binding, lib


def summarize_probe(st: np.ndarray, skip: int = 10) -> dict:
    """Exchange probe stamps [rounds, G, 2] (publication, maximum known;
    ticks): medians over rounds (after the first `skip`) of the publication
    spread, the median and the slowest workgroup's time from the last
    publication to knowing the maximum, and the round period (us)."""
    st = st.astype(np.int64)[skip:]
    pub, known = st[:, :, 0], st[:, :, 1]
    last_pub = pub.max(axis=1)
    after = (known - last_pub[:, None]) * TICK_US
    med = statistics.median
    return {
        "rounds": st.shape[0],
        "spread": med(((pub.max(axis=1) - pub.min(axis=1)) * TICK_US).tolist()),
        "known_med": med(np.median(after, axis=1).tolist()),
        "known_last": med(after.max(axis=1).tolist()),
        "period": med((np.diff(pub.min(axis=1)) * TICK_US).tolist()),
    }


def exchange_probe(lib, G: int, rounds: int) -> str:
    out = [f"## Exchange floor probe: {G} workgroups of 512 threads, {rounds} rounds, medians over "
           f"rounds {10}..{rounds - 1} (us)\n",
           "| exchange | publication spread | maximum known after the last publication: median WG "
           "| slowest WG | round period |",
           "|---|---|---|---|---|"]
    for two_level, name in ((1, "two levels (reducers, 16 copies of the partials)"), (0, "all-to-all")):
        st = np.zeros((rounds, G, 2), dtype=np.uint64)
        rc = lib.markov_trace_exchange_probe(G, rounds, two_level, st.ctypes.data)
        if rc != 0:
            raise RuntimeError("markov_trace_exchange_probe failed")
        if not np.all(st[:, :, 1] > 0):
            raise RuntimeError("exchange probe: a wait gave up")
        r = summarize_probe(st)
        out.append(f"| {name} | {r['spread']:.2f} | {r['known_med']:.2f} | {r['known_last']:.2f} | "
                   f"{r['period']:.2f} |")
    return "\n".join(out)


def read(lib, G: int, N: int) -> np.ndarray:
    """Stamps [G, N, phases] in microseconds (int64 ticks converted)."""
    buf = np.zeros((TRACE_WGS, TRACE_STEPS, TRACE_PHASES), dtype=np.uint64)
    rc = lib.markov_trace_read(buf.ctypes.data, buf.nbytes)
    if rc != 0:
        raise RuntimeError("markov_trace_read failed")
    return buf[:G, :N].astype(np.int64)


def summarize(stamps: list, G: int, N: int, mode: int) -> dict:
    """Medians over calls of the per-step quantities (microseconds)."""
    rows = {k: [[] for _ in range(N)] for k in ("local", "pub", "win_med", "win_max", "step", "spread")}
    kern = {"prologue_med": [], "prologue_max": [], "entry_spread": [], "total": []}
    for t in stamps:
        t0 = t[:, 0, 6].min()
        kern["entry_spread"].append((t[:, 0, 6].max() - t0) * TICK_US)
        kern["prologue_med"].append(np.median(t[:, 0, 7] - t[:, 0, 6]) * TICK_US)
        kern["prologue_max"].append((t[:, 0, 7].max() - t0) * TICK_US)
        kern["total"].append((t[:, N - 1, 5].max() - t0) * TICK_US)
        for i in range(N):
            start = t[:, i, 0].min()
            rows["spread"][i].append((t[:, i, 0].max() - start) * TICK_US)
            rows["local"][i].append(np.median(t[:, i, 1] - t[:, i, 0]) * TICK_US)
            pub_phase = 2 if mode == 0 else 1
            last_pub = t[:, i, pub_phase].max()
            rows["pub"][i].append((last_pub - start) * TICK_US)
            # (at mode 0's last step with at most 8 rows only workgroup 0
            # waits for the winners: the workgroups that stamped)
            win = t[:, i, 4]
            win = win[win > 0] if np.any(win > 0) else win
            rows["win_med"][i].append(np.median(win - last_pub) * TICK_US)
            rows["win_max"][i].append((win.max() - last_pub) * TICK_US)
            nxt = t[:, i + 1, 0].min() if i + 1 < N else t[:, i, 5].max()
            rows["step"][i].append((nxt - start) * TICK_US)
    med = statistics.median
    return {"steps": {k: [med(v[i]) for i in range(N)] for k, v in rows.items()},
            "kernel": {k: med(v) for k, v in kern.items()}}


def summarize_invcdf(stamps: list, N: int) -> dict:
    """Inverse CDF: per step, medians over calls of when (after the last
    workgroup's partials, i.e. its end of local work) the leaders have seen
    every partial (last leader), chosen their chunks (last leader), scanned
    them and published the tokens (last leader), every workgroup knows every
    token (median / last), and the next step starts."""
    keys = ("seen", "dec", "own", "tok_med", "tok_max", "next")
    rows = {k: [[] for _ in range(N)] for k in keys}

    def last(a):
        a = a[a > 0]
        return a.max() if a.size else np.nan

    for t in stamps:
        for i in range(N):
            p1 = t[:, i, 1].max()
            us = lambda x: (x - p1) * TICK_US
            rows["seen"][i].append(us(last(t[:, i, 10])))
            rows["dec"][i].append(us(last(t[:, i, 11])))
            rows["own"][i].append(us(last(t[:, i, 9])))
            rows["tok_med"][i].append(us(np.median(t[:, i, 4])))
            rows["tok_max"][i].append(us(t[:, i, 4].max()))
            nxt = t[:, i + 1, 0].min() if i + 1 < N else t[:, i, 5].max()
            rows["next"][i].append(us(nxt))
    med = statistics.median
    return {k: [med(v[i]) for i in range(N)] for k, v in rows.items()}


def summarize_step_kernels(stamps: list, G: int, N: int) -> dict:
    """Step-kernel path (one launch per position): per launch, medians over
    calls of the entry spread, the first row block's inputs ready (median
    workgroup, from its entry), all blocks done (median and last workgroup,
    from the first entry), the last workgroup's picks (after the last
    workgroup's blocks), and the gap to the next launch's first entry."""
    keys = ("spread", "first_block", "blocks_med", "blocks_max", "pick", "gap", "launch")
    rows = {k: [[] for _ in range(N)] for k in keys}
    for t in stamps:
        for i in range(N):
            e = t[:, i, 0]
            start = e.min()
            rows["spread"][i].append((e.max() - start) * TICK_US)
            rows["first_block"][i].append(np.median(t[:, i, 1] - e) * TICK_US)
            rows["blocks_med"][i].append((np.median(t[:, i, 2]) - start) * TICK_US)
            rows["blocks_max"][i].append((t[:, i, 2].max() - start) * TICK_US)
            end = t[:, i, 3].max()  # only the last workgroup stamps phase 3
            rows["pick"][i].append((end - t[:, i, 2].max()) * TICK_US)
            rows["launch"][i].append((end - start) * TICK_US)
            if i + 1 < N:
                rows["gap"][i].append((t[:, i + 1, 0].min() - end) * TICK_US)
            else:
                rows["gap"][i].append(0.0)
    med = statistics.median
    return {k: [med(v[i]) for i in range(N)] for k, v in rows.items()}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="dsv41_single_row")
    ap.add_argument("--noise", choices=("inline", "side"), default="inline")
    ap.add_argument("--calls", type=int, default=20)
    ap.add_argument("--cold", action="store_true", help="read 1 GiB before each call (evicts L2s and MALL)")
    ap.add_argument("--batch-path", choices=("auto", "persistent", "step", "persistent-step"), default="auto")
    ap.add_argument("--dump", help="also save the raw stamps [calls, workgroups, steps, phases] (ticks) to this .npy")
    ap.add_argument("--exchange-probe", action="store_true", help="measure the exchange's floor (see above)")
    ap.add_argument("--grid", type=int, default=253, help="exchange probe: workgroups")
    ap.add_argument("--rounds", type=int, default=200, help="exchange probe: rounds")
    args = ap.parse_args()

    import torch

    binding, lib = load_trace_library()
    if args.exchange_probe:
        torch.zeros(1, device="cuda:0")  # the device, initialised
        print(exchange_probe(lib, args.grid, args.rounds))
        return 0
    from markov_bias_chain_amd import synth
    from markov_bias_chain_amd.device import DeviceChain

    dev = torch.device("cuda:0")
    binding.markov_set_batch_path({"auto": 0, "persistent": 1, "step": 2, "persistent-step": 3}[args.batch_path])
    w = synth.workload(args.workload)
    inline = args.noise == "inline" and w.mode == 0
    d = DeviceChain(w, device=dev, noise_inline=inline)
    step_path = args.batch_path in ("step", "persistent-step") or (args.batch_path == "auto" and w.rows > 64)
    G = binding.markov_grid(w.rows, w.N, w.V, w.r, w.mode)
    if step_path:  # one workgroup per chunk
        G = -(-w.V // (8 * (16384 // w.r)))
    if w.mode == 0 and not inline:
        d.noise()
    for _ in range(5):
        d.chain()
    binding.markov_status(d.workspace)
    read(lib, G, w.N)
    scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev) if args.cold else None
    sink = torch.empty((), dtype=torch.float32, device=dev)
    stamps = []
    for _ in range(args.calls):
        if scratch is not None:
            torch.sum(scratch, dim=0, out=sink)
        d.chain()
        binding.markov_status(d.workspace)
        stamps.append(read(lib, G, w.N))
    if args.dump:
        np.save(args.dump, np.stack(stamps))
    if step_path:
        st = summarize_step_kernels(stamps, G, w.N)
        kind = "inverse CDF, step and pick kernels" if w.mode == 1 else "noise in memory"
        print(f"## Step kernels: {w.name}, {kind}, {'cold' if args.cold else 'warm'} calls, "
              f"{G} workgroups per launch, medians over {args.calls} calls (us)\n")
        print("| step | entry spread | first block ready (median WG) | blocks done (median / last WG) "
              "| last WG's picks | launch (first entry to picks done) | gap to next launch |")
        print("|---|---|---|---|---|---|---|")
        for i in range(w.N):
            print(f"| {i} | {st['spread'][i]:.2f} | {st['first_block'][i]:.2f} | {st['blocks_med'][i]:.2f} / "
                  f"{st['blocks_max'][i]:.2f} | {st['pick'][i]:.2f} | {st['launch'][i]:.2f} | {st['gap'][i]:.2f} |")
        return 0
    s = summarize(stamps, G, w.N, w.mode)
    k = s["kernel"]
    noise = "no noise (inverse CDF)" if w.mode == 1 else f"{'inline' if inline else args.noise} noise"
    print(f"## Per-step breakdown: {w.name}, {noise}, "
          f"{'cold' if args.cold else 'warm'} calls, grid {G}, medians over {args.calls} calls (us)\n")
    print(f"kernel: entry spread {k['entry_spread']:.2f}, prologue done (median workgroup) "
          f"{k['prologue_med']:.2f}, (last) {k['prologue_max']:.2f}, first entry to last step end "
          f"{k['total']:.2f}\n")
    print("| step | start spread | local work (wave 0) | last key out | winner known (median / slowest WG) | step |")
    print("|---|---|---|---|---|---|")
    st = s["steps"]
    for i in range(w.N):
        print(f"| {i} | {st['spread'][i]:.2f} | {st['local'][i]:.2f} | {st['pub'][i]:.2f} | "
              f"{st['win_med'][i]:.2f} / {st['win_max'][i]:.2f} | {st['step'][i]:.2f} |")
    if w.mode == 1:
        c = summarize_invcdf(stamps, w.N)
        print("\nInverse CDF, after the last workgroup's partials (us): leaders have seen every partial, "
              "chunks chosen, the leaders' scans done and tokens out, tokens known (median / last "
              "workgroup), next step's first start\n")
        print("| step | partials seen | chunks chosen | tokens out | tokens known | next step |")
        print("|---|---|---|---|---|---|")
        for i in range(w.N):
            print(f"| {i} | {c['seen'][i]:.2f} | {c['dec'][i]:.2f} | {c['own'][i]:.2f} | "
                  f"{c['tok_med'][i]:.2f} / {c['tok_max'][i]:.2f} | {c['next'][i]:.2f} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
