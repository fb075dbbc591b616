"""Benchmark of the Markov draft-sampling chain on one MI355X.

A step is one pass of the whole hot path over one batch: for up to 8 rows
(the default, --noise auto) one launch of the persistent chain kernel that
draws its Gumbel noise itself (MARKOV_NOISE_INLINE: the idle waves of each
workgroup draw the next step's noise while the exchange is in flight); for
larger batches, or with --noise side, the noise fill kernel on a side stream
(forked after the current stream's work and joined before the chain) and the
chain reading it.  The default workload is
the DeepSeek-V4.1-sized single request row: V=129280, r=256 (a 66 MB bf16
head), rows=1, N=8 draft positions, T=0.7, synthetic inputs.

Prints ONE JSON line.  `value` is draft tokens/s over the timed steps, run
back to back with inputs resident in HBM: a step with inline noise is one
kernel launch, issued eagerly; a step with side-stream noise (fork, noise,
join, chain) is replayed as one HIP graph (the pages capture the sampler in
graphs; this keeps the fork/join launch gaps out).  Both ways of issuing are
reported (`eager_ms_per_step`, `graph_ms_per_step`).
`roofline` is for the chain kernel:
algorithmic bytes per launch (head once, base logits, noise read unless it
is drawn inline, cache writes, embedding rows, tokens) over its average
launch duration, measured with HIP
events on the stream it runs on around `steps` back-to-back chain launches.
Cold calls (a 1 GiB read between calls evicts the L2s and the 256 MB MALL
with clean lines, outside the timed interval) are reported too.
`cpu_baseline` times the CPU oracle on the same workload on this host.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "markov_bias_chain_amd", "csrc", "markov.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "chain_kernel_dsv41_single_row_pmc.md")


def kernel_source_digest() -> str:
    """sha256 prefix of the kernel source with comments and blank lines
    removed, so that a comment edit does not invalidate counter readings."""
    import hashlib
    import re

    text = open(KERNEL_SRC).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def profile_fields(noise: str):
    """The committed rocprofv3 counter summary's fields, if it was taken on
    the current kernel code with the same noise placement (else None)."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and " " not in line.split(": ")[0])
    if fields.get("kernel_code_sha256_prefix", "").strip() != kernel_source_digest():
        return None
    if fields.get("noise", "side").strip() != noise:
        return None
    return fields


def measured_traffic(noise: str):
    """HBM-side bytes per chain launch (FETCH_SIZE + WRITE_SIZE, calibrated)."""
    f = profile_fields(noise)
    return int(f["traffic_bytes_per_launch"]) if f else None


def head_residency(w, inline: bool, noise: str):
    """How much of the head traffic the resident head saves: without it every
    one of the N steps reads the head; with it the head comes from beyond the
    L2s (FETCH_SIZE, less the other algorithmic reads) about once per call."""
    f = profile_fields(noise)
    if not f or "fetch_bytes_per_launch" not in f:
        return None
    ab = algorithmic_bytes(w, inline)
    other = ab["reads"] - ab["head"] + w.real_rows * 8  # base, noise read, embedding rows, anchors
    head_fetched = int(f["fetch_bytes_per_launch"]) - other
    return {"head_bytes": ab["head"], "steps": w.N, "head_bytes_fetched_per_call": head_fetched,
            "head_reads_per_call": head_fetched / ab["head"],
            "on_chip_fraction": 1.0 - head_fetched / (w.N * ab["head"])}


def algorithmic_bytes(w, inline: bool) -> dict:
    """The algorithmic bytes of one chain call, per unit as the scope table
    counts them: the head once, base logits, noise (fp32, mode 0: counted
    whether the kernel reads it or draws it inline), cache writes and the
    embedding rows, for the real (non-padding) rows; `reads` are the bytes a
    call actually reads (no noise when it is drawn inline), for comparing
    with the measured fetch traffic."""
    real = w.real_rows
    head = w.V * w.r * 2
    base = real * w.N * w.V * 2
    noise = real * w.N * w.V * 4 if w.mode == 0 else 0
    cache = real * w.N * w.V * 2
    embed = real * w.N * w.r * 2
    noise_read = 0 if inline else noise
    return dict(head=head, base=base, noise=noise, cache=cache, embed=embed,
                total=head + base + noise + cache + embed,
                reads=head + base + noise_read + embed)


def launch_kind(w, inline: bool, batch_path: str):
    """(dominant kernel, description) of the launches a call makes, by the
    library's documented dispatch: beyond 64 rows (or when the path knob
    asks) step kernels, in mode 0 the persistent step kernel when its grid of
    one workgroup per chunk fits on the CUs at once, else one launch per
    position (mode 1: with a pick kernel); otherwise persistent chain
    launches of at most 64 rows."""
    import torch

    drawing = " drawing its noise inline" if inline else ""
    step = batch_path in ("step", "persistent-step") or (batch_path == "auto" and w.rows > 64)
    if not step:
        n = -(-w.rows // 64)
        return "chain_kernel", f"chain kernel{drawing} ({n} launch{'es' if n > 1 else ''})"
    chunks = -(-w.V // (8 * (16384 // w.r)))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if w.mode == 0 and batch_path != "step" and chunks <= cus:
        return "step_kernel", f"persistent step kernel{drawing} (one launch)"
    if w.mode == 1:
        return "step_kernel", f"step kernel + pick kernel per position ({2 * w.N} launches)"
    return "step_kernel", f"step kernel{drawing} per position ({w.N} launches)"


def cpu_baseline(w, budget_s: float) -> dict:
    """The oracle as it stands (single-threaded C), timed on whole calls of
    the same workload, with its own noise, for about budget_s seconds."""
    import numpy as np

    import oracle

    g = oracle.noise_fill(w.seeds, w.N, w.V) if w.mode == 0 else None
    calls = 0
    t0 = time.perf_counter()
    while True:
        tok, _ = oracle.chain(w.base, w.head, w.embed, w.prev, w.temperature, w.seeds, gumbel=g,
                              state_idx=w.state_idx, mult=w.mult, cap=w.cap, mode=w.mode)
        if calls == 0:
            cpu_baseline.tokens = tok
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    tokens = calls * w.real_rows * w.N
    del np
    return {"value": tokens / el, "unit": "draft tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{calls} full calls of the {w.name} workload (oracle noise included, "
                      f"{el:.1f} s, single thread on {os.cpu_count()} online cores)"}


def cpu_mt_baseline(w, budget_s: float, ref_tokens=None) -> dict:
    """The same chain on every host core, for a fairer CPU throughput figure
    than the single-threaded oracle: the bias as an fp32 BLAS matrix-vector
    product (torch CPU, all cores), the epilogue and the draw in fp32 torch
    ops, and the noise (the SplitMix64 hash in numpy uint64 arithmetic, each
    log in fp64 rounded once to fp32) over vocabulary slices on a thread
    pool.  Mode 0 only.  Not the oracle and not a product path: a measured
    baseline; `matches_oracle` says whether its tokens equal the oracle's on
    the first call."""
    import concurrent.futures

    import numpy as np
    import torch

    # every core this process may run on, at most 16 (one GPU's share of a host)
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    torch.set_num_threads(cores)
    M64 = np.uint64(0xFFFFFFFFFFFFFFFF)
    G64, C1, C2 = np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBF58476D1CE4E5B9), np.uint64(0x94D049BB133111EB)

    def sm(x):
        z = x + G64
        z = (z ^ (z >> np.uint64(30))) * C1
        z = (z ^ (z >> np.uint64(27))) * C2
        return z ^ (z >> np.uint64(31))

    def sm_int(x):
        return int(sm(np.array([x & int(M64)], dtype=np.uint64))[0])

    ids = np.arange(w.V, dtype=np.uint64)
    slices = np.array_split(np.arange(w.V), cores)
    pool = concurrent.futures.ThreadPoolExecutor(cores)

    def noise(seed, row, step):
        h = sm_int(sm_int(sm_int(seed) ^ row) ^ step)
        out = np.empty(w.V, dtype=np.float32)

        def part(sl):
            u = ((2 * (sm(np.uint64(h) ^ ids[sl]) >> np.uint64(41)) + 1).astype(np.float32)
                 * np.float32(2.0**-24))
            inner = np.log(u.astype(np.float64)).astype(np.float32)
            out[sl] = -np.log((-inner).astype(np.float64)).astype(np.float32)

        list(pool.map(part, slices))
        return torch.from_numpy(out)

    with torch.inference_mode():
        head = torch.from_numpy(w.head[:w.V].view(np.int16)).view(torch.bfloat16).float()
        embed = torch.from_numpy(w.embed.view(np.int16)).view(torch.bfloat16).float()
        base = torch.from_numpy(np.ascontiguousarray(w.base).view(np.int16)).view(torch.bfloat16)
        sidx = np.arange(w.rows) if w.state_idx is None else w.state_idx
        mult = torch.tensor(w.mult, dtype=torch.float32)
        inv_cap = torch.tensor(1.0, dtype=torch.float32) / torch.tensor(w.cap, dtype=torch.float32) if w.cap > 0 else None

        def call():
            tokens = np.full((w.rows, w.N), -1, dtype=np.int64)
            for b in range(w.rows):
                if sidx[b] < 0:
                    continue
                p, T = int(w.prev[b]), float(w.temperature[b])
                for i in range(w.N):
                    bias = (head @ embed[p]).to(torch.bfloat16).float()
                    x = (base[b, i].float() + bias) * mult
                    if inv_cap is not None:
                        x = torch.tanh(x * inv_cap) * w.cap
                    c = x.to(torch.bfloat16).float()
                    s = c / torch.tensor(T, dtype=torch.float32) + noise(int(w.seeds[b]), b, i) if T > 0 else c
                    p = int(torch.argmax(s))
                    tokens[b, i] = p
            return tokens

        first = call()
        calls = 1
        t0 = time.perf_counter()
        while True:
            call()
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    pool.shutdown()
    tokens = (calls - 1) * w.real_rows * w.N
    return {"value": tokens / el, "unit": "draft tokens/s", "cores": cores, "kind": "cpu_mt",
            "matches_oracle": None if ref_tokens is None else bool(np.array_equal(first, ref_tokens)),
            "sample": f"{calls - 1} full calls of the {w.name} workload (its own noise, {el:.1f} s, "
                      f"{cores} threads: torch CPU matrix-vector bias and epilogue, numpy noise hash)"}


def draft_step_figures(w, hidden: int, dev, reps: int = 50) -> dict:
    """The pages' deployment shape around the chain, as context: a stand-in
    draft LM head (base logits = hidden states @ W with random bf16 weights
    [hidden, V]) runs on the current stream while the noise runs on a side
    stream, then the chain; eager and captured as one HIP graph.  Also the
    same with the noise drawn inside the chain (LM head, then the chain).
    The LM head is not part of the hot path and not part of `value`."""
    import torch

    from markov_bias_chain_amd import binding
    from markov_bias_chain_amd.device import DeviceChain

    d = DeviceChain(w, device=dev)
    di = DeviceChain(w, device=dev, noise_inline=True)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0x4D41524B)
    weight = torch.empty(hidden, w.V, dtype=torch.bfloat16, device=dev)
    for k in range(0, hidden, 512):  # fp32 draws in slices, cast to bf16
        weight[k:k + 512] = (torch.randn(min(512, hidden - k), w.V, device=dev, generator=gen) * 0.02)
    hs = torch.randn(w.rows * w.N, hidden, device=dev, generator=gen).to(torch.bfloat16)
    base2d = d.base.view(w.rows * w.N, w.V)

    def lm_head():
        torch.matmul(hs, weight, out=base2d)

    def step():
        cur = torch.cuda.current_stream(dev)
        if w.mode == 0:
            d.side.wait_stream(cur)
            d.noise(stream=d.side)
        lm_head()
        if w.mode == 0:
            cur.wait_stream(d.side)
        d.chain(stream=cur)

    def timed(fn):
        for _ in range(5):
            fn()
        torch.cuda.synchronize(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        b.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    lm_us = timed(lm_head)
    chain_us = timed(lambda: d.chain())
    noise_us = timed(lambda: d.noise()) if w.mode == 0 else 0.0
    eager_us = timed(step)
    binding.markov_status(d.workspace)
    step()
    torch.cuda.synchronize(dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    # one replay against an eager step on the same inputs
    g.replay()
    binding.markov_status(d.workspace)
    t_g, c_g = d.results()
    step()
    binding.markov_status(d.workspace)
    t_e, c_e = d.results()
    same = bool((t_g == t_e).all() and (c_g == c_e).all())
    graph_us = timed(g.replay)
    binding.markov_status(d.workspace)
    del g
    # inline noise: the LM head writes the inline chain's base logits
    base2d_i = di.base.view(w.rows * w.N, w.V)

    def step_inline():
        torch.matmul(hs, weight, out=base2d_i)
        di.chain()

    chain_inline_us = timed(lambda: di.chain())
    inline_eager_us = timed(step_inline)
    step_inline()
    torch.cuda.synchronize(dev)
    gi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gi):
        step_inline()
    inline_graph_us = timed(gi.replay)
    binding.markov_status(di.workspace)
    del gi, d, di, weight, hs
    torch.cuda.empty_cache()
    return {"lm_head_stand_in": f"[{w.rows * w.N}, {hidden}] @ [{hidden}, {w.V}] bf16 (torch.matmul)",
            "lm_head_us": lm_us, "noise_us": noise_us, "chain_us": chain_us,
            "eager_step_us": eager_us, "graph_step_us": graph_us,
            "noise_hidden_us": lm_us + noise_us + chain_us - eager_us,
            "graph_replay_matches_eager": same,
            "inline_noise": {"chain_us": chain_inline_us, "eager_step_us": inline_eager_us,
                             "graph_step_us": inline_graph_us}}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv41_single_row")
    ap.add_argument("--noise", choices=("auto", "inline", "side"), default="auto",
                    help="mode 0: noise drawn inside the chain kernel, or by the noise fill "
                         "kernel on a side stream; auto: inline up to 8 rows (the chain's idle "
                         "waves draw it), side stream beyond")
    ap.add_argument("--batch-path", choices=("auto", "persistent", "step", "persistent-step"), default="auto",
                    help="mode 1, and mode 0 with the noise in memory: persistent chain launches of "
                         "at most 64 rows; step kernels per position over all rows (mode 1: with a "
                         "pick kernel); or (mode 0) one persistent step kernel for all positions; "
                         "auto: beyond 64 rows the persistent step kernel when its grid fits on "
                         "the CUs at once (mode 0), else the step kernels")
    ap.add_argument("--cold", type=int, default=50, help="cold calls timed after the main loop")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the 8-row and draft-step figures")
    ap.add_argument("--lm-hidden", type=int, default=7168,
                    help="hidden size of the stand-in draft LM head of the draft-step figures (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device-to-device copy (a known-size kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the chain runs on one GPU; --gpus {args.gpus} is not supported "
              "(it is not sharded across GPUs)", file=sys.stderr)
        return 2

    import torch

    from markov_bias_chain_amd import binding, synth
    from markov_bias_chain_amd.device import DeviceChain

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    binding.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def measure(w, steps, warmup, cold_calls, inline):
        d = DeviceChain(w, device=dev, noise_inline=inline)
        side = w.mode == 0 and not inline
        stream = torch.cuda.current_stream(dev)
        for _ in range(warmup):
            d.step()
        torch.cuda.synchronize()
        binding.markov_status(d.workspace)
        # the steps issued eagerly, back to back
        t0 = time.perf_counter()
        for _ in range(steps):
            d.step()
        torch.cuda.synchronize()
        eager_wall = time.perf_counter() - t0
        binding.markov_status(d.workspace)
        # the steps as replays of one graph (noise fork/join + chain)
        graph = d.capture_step()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_wall = time.perf_counter() - t0
        binding.markov_status(d.workspace)
        del graph
        # the steps again, each chain bracketed by events
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        torch.cuda.synchronize()
        for k in range(steps):
            if side:
                d.side.wait_stream(stream)
                d.noise(stream=d.side)
                stream.wait_stream(d.side)
            ev[k][0].record(stream)
            d.chain(stream=stream)
            ev[k][1].record(stream)
        torch.cuda.synchronize()
        binding.markov_status(d.workspace)
        chain_ms = [a.elapsed_time(b) for a, b in ev]
        # the chain alone, back to back: the average launch duration
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            d.chain(stream=stream)
        b.record(stream)
        b.synchronize()
        b2b_ms = a.elapsed_time(b) / steps
        binding.markov_status(d.workspace)
        # cold calls: evict the L2s and the MALL by reading 1 GiB before each call
        scratch = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        cold_ms = []
        for k in range(cold_calls):
            if side:
                d.noise(stream=stream)
            torch.sum(scratch, dim=0, out=sink)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            d.chain(stream=stream)
            b.record(stream)
            b.synchronize()
            cold_ms.append(a.elapsed_time(b))
        binding.markov_status(d.workspace)
        del scratch, d
        torch.cuda.empty_cache()
        # the step as it is run: one eager launch, or one graph replay when
        # the noise is forked onto a side stream
        step_wall = graph_wall if side else eager_wall
        return dict(step_wall=step_wall, eager_wall=eager_wall, graph_wall=graph_wall,
                    chain_ms=chain_ms, cold_ms=cold_ms, b2b_ms=b2b_ms,
                    issue="graph replay" if side else "eager launch")

    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    binding.markov_set_batch_path({"auto": 0, "persistent": 1, "step": 2, "persistent-step": 3}[args.batch_path])
    w = synth.workload(args.workload)
    noise = args.noise if args.noise != "auto" else ("inline" if w.real_rows <= 8 else "side")
    inline = noise == "inline" and w.mode == 0
    m = measure(w, args.steps, args.warmup, args.cold, inline)
    chain_ms, cold_ms, b2b_ms = m["chain_ms"], m["cold_ms"], m["b2b_ms"]
    tok_per_step = w.real_rows * w.N
    ms_per_step = m["step_wall"] * 1e3 / args.steps
    ab = algorithmic_bytes(w, inline)
    chain_us = b2b_ms * 1e3
    chain_us_med = statistics.median(chain_ms) * 1e3
    cold_us_med = statistics.median(cold_ms) * 1e3 if cold_ms else None
    achieved = ab["total"] / (chain_us * 1e-6) / 1e9
    kernel, chain_desc = launch_kind(w, inline, args.batch_path)
    result = {
        "metric": "µs/call & draft tokens/s, V=129280 r=256 N=8 rows=1/8; head GB/s vs HBM peak",
        "value": tok_per_step / (ms_per_step * 1e-3),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "eager_ms_per_step": m["eager_wall"] * 1e3 / args.steps,
        "graph_ms_per_step": m["graph_wall"] * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "V": w.V, "r": w.r, "rows": w.rows, "N": w.N,
                   "mode": "gumbel" if w.mode == 0 else "invcdf",
                   "grid": binding.markov_grid(w.rows, w.N, w.V, w.r, w.mode),
                   "noise": "inline" if inline else ("side stream" if w.mode == 0 else "none"),
                   "batch_path": args.batch_path,
                   "step": ("noise fill on a side stream + " if (w.mode == 0 and not inline) else "")
                           + chain_desc + ", " + m["issue"]},
        "chain_us_per_call": {"back_to_back_mean": chain_us,
                              "warm_event_mean": statistics.mean(chain_ms) * 1e3,
                              "warm_median": chain_us_med,
                              "warm_p10": sorted(chain_ms)[len(chain_ms) // 10] * 1e3,
                              "warm_p90": sorted(chain_ms)[len(chain_ms) * 9 // 10] * 1e3,
                              "cold_median": cold_us_med},
        "head_GBps": {"warm": ab["head"] / (chain_us_med * 1e-6) / 1e9,
                      "cold": ab["head"] / (cold_us_med * 1e-6) / 1e9 if cold_us_med else None},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(noise) if args.workload == "dsv41_single_row" else None,
                     "kernel": kernel, "bytes_per_launch": ab["total"]},
    }
    if args.workload == "dsv41_single_row":
        result["head_residency"] = head_residency(w, inline, noise)
    if cold_us_med:
        ach_c = ab["total"] / (cold_us_med * 1e-6) / 1e9
        result["roofline_cold"] = {"achieved": ach_c, "frac": ach_c / HBM_PEAK_GBPS}
    if not args.no_extra and args.workload == "dsv41_single_row":
        # the other noise placement of the same workload (one step, graph replay)
        other = not inline
        mo = measure(w, 100, 10, 0, other)
        result["other_noise_placement"] = {
            "noise": "inline" if other else "side stream", "issue": mo["issue"],
            "ms_per_step": mo["step_wall"] * 1e3 / 100,
            "draft_tokens_per_s": tok_per_step * 100 / mo["step_wall"],
            "chain_us_back_to_back": mo["b2b_ms"] * 1e3}
        w8 = synth.workload("dsv41_eight_rows")
        m8 = measure(w8, 50, 10, 20, inline)
        c8, k8 = m8["chain_ms"], m8["cold_ms"]
        us8 = statistics.median(c8) * 1e3
        result["rows8"] = {"workload": w8.name, "chain_us_warm_median": us8,
                           "chain_us_cold_median": statistics.median(k8) * 1e3,
                           "draft_tokens_per_s": w8.real_rows * w8.N / (us8 * 1e-6),
                           "step_tokens_per_s": w8.real_rows * w8.N * 50 / m8["step_wall"],
                           "head_GBps_warm": algorithmic_bytes(w8, inline)["head"] / (us8 * 1e-6) / 1e9}
    if not args.no_extra and args.lm_hidden > 0:
        result["draft_step"] = draft_step_figures(w, args.lm_hidden, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        if w.mode == 0:
            result["cpu_mt"] = cpu_mt_baseline(w, min(8.0, args.cpu_seconds), getattr(cpu_baseline, "tokens", None))
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
