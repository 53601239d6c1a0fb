"""Benchmark of the MoE speculative verify step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: one full verify pass at concurrency 32 -- 32 sequences x 4
positions (1 committed + K=3 drafts) = 128 tokens through 12 MoE layers
(hidden 1280, 64 routed + 2 shared SwiGLU experts with intermediate 896, top-6),
the 1280 x 129,280 LM-head argmax and greedy acceptance.  Weights and inputs
are seeded synthetic data (N(0, 0.02) bf16 weights, N(0, 1) hidden states),
resident in HBM before the timed region.  Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

ZIPF_BIAS = os.path.join(ROOT, "tests", "golden", "zipf_bias_prefill.json")
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E, GB/s
P_KEEP = 0.576                # per-position draft keep probability (the pages' acceptance rate)
Q_KEEP = 0.749                # the keep probability whose mean commits per pass, 1 + q + q^2 + q^3,
                              # equal the pages' tau of 2.73
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, TFLOP/s


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="step128",
                    choices=["step128", "batch1", "layer128", "prefill", "decode32", "spec128", "attn128", "step128attn",
                             "pages32", "copy"],
                    help="copy: a plain 1 GiB device copy, the reference for scaling the HBM traffic counters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--keep", type=float, default=None,
                    help="batch1, decode32, pages32, spec128: draft keep probability (default 0.576)")
    ap.add_argument("--no-companions", action="store_true",
                    help="step128: skip the batch-1, prefill and decode-loop lines run after the headline")
    ap.add_argument("--cpu-layers", type=int, default=12, help="layers of the oracle sample")
    ap.add_argument("--cpu-vocab", type=int, default=129280, help="LM-head rows of the oracle sample")
    ap.add_argument("--cpu-reps", type=int, default=3, help="repetitions of the oracle sample")
    ap.add_argument("--cpu-steps", type=int, default=4,
                    help="decode32: full-batch passes the oracle runs for the extrapolated loop figure")
    ap.add_argument("--cpu-tokens", type=int, default=512, help="tokens of the oracle sample (at most T)")
    ap.add_argument("--drafts", type=int, default=None, help="drafts K per sequence (positions = K + 1)")
    ap.add_argument("--no-graph", action="store_true", help="batch1: time eager launches only")
    ap.add_argument("--target", type=int, default=1085, help="decode32, pages32: committed tokens per sequence")
    ap.add_argument("--prompt", type=int, default=1156, help="pages32: prompt tokens per page")
    ap.add_argument("--seqs", type=int, default=32, help="spec128: sequences per step")
    ap.add_argument("--context", default=None,
                    help="attn128: committed lengths to time (comma list, first = reported value; default "
                         "2241,1156,8192,32768); step128attn: the committed length (default 1700)")
    return ap.parse_args()


def expert_bytes(sh) -> int:
    return 3 * sh.H * sh.I * 2


def ffn_roofline(st, h_in, sh, steps: int) -> dict:
    """The routed gate/up kernel of a verify pass over h_in: algorithmic
    bytes from the pass's own routing (gate and up rows of every touched
    expert and the shared ones, the normed tokens in; the SwiGLU rows it
    writes are an intermediate and not counted) over its mean launch
    duration, HIP events on its stream."""
    import numpy as np
    import torch
    T = h_in.shape[0]
    rec = []
    st.forward(h_in, rec)
    touched = [int(np.unique(r["ids"].cpu().numpy()).size) for r in rec]
    gu_b = float(np.mean([(t + sh.S) * 2 * sh.I * sh.H * 2 + T * sh.H * 2 for t in touched]))
    st.ffn_events = ev = []
    for _ in range(steps):
        st.forward(h_in)
    torch.cuda.synchronize()
    st.ffn_events = None
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    gbs = gu_b / (us * 1e-6) / 1e9
    return {"kernel": "moe_expert_gate_up_routed (skinny_kernel<true, true>)", "bound": "hbm", "achieved": gbs,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
            "traffic_source": f"counters recorded for the {sh.B} x {sh.P}-token verify pass (step128 workload)",
            "us_per_launch": us, "algorithmic_bytes_per_launch": gu_b, "tokens_per_pass": T}


# HBM traffic of the gate/up kernel per launch, from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by the same counters on a plain copy of known size;
# valid only while the kernel's sources are the ones that were measured
TRAFFIC = {
    "step128": (os.path.join(ROOT, "profiles", "expert_gate_up_step128_traffic.txt"),
                ["moe_decoder_step_amd/csrc/swiglu.hip", "moe_decoder_step_amd/csrc/common.hpp"]),
    "batch1": (os.path.join(ROOT, "profiles", "expert_gate_up_batch1_traffic.txt"),
               ["moe_decoder_step_amd/csrc/swiglu.hip", "moe_decoder_step_amd/csrc/common.hpp"]),
    "prefill": (os.path.join(ROOT, "profiles", "gemm_gate_up_prefill_traffic.txt"),
                ["moe_decoder_step_amd/csrc/gemm.hip", "moe_decoder_step_amd/csrc/common.hpp"]),
}


def kernel_source_hash(workload: str = "step128") -> str:
    import hashlib
    d = hashlib.sha256()
    for f in TRAFFIC[workload][1]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            d.update(fh.read())
    return d.hexdigest()[:16]


def measured_traffic(workload: str = "step128"):
    """(fetch + write bytes per launch, note) or (None, reason)."""
    if workload not in TRAFFIC:
        return None, "no counter run recorded for this workload"
    path = TRAFFIC[workload][0]
    if not os.path.exists(path):
        return None, "no counter run recorded"
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_hash(workload):
        return None, "kernel changed since the counters were taken"
    return (float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]),
            os.path.relpath(path, ROOT))


def copy_calibration(args) -> int:
    """A plain device copy of 1 GiB: the known-size reference for the counters."""
    import torch
    n = 1 << 29                      # bf16 elements = 1 GiB
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(args.warmup):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    print(json.dumps({"workload": "copy", "bytes_read": 2 * n, "bytes_written": 2 * n, "ms": ms,
                      "GBs": 4 * n / (ms * 1e-3) / 1e9}), flush=True)
    return 0


def main() -> int:
    args = parse()
    global P_KEEP
    if args.keep is not None:
        if not 0.0 <= args.keep <= 1.0:
            print("--keep is a probability", file=sys.stderr)
            return 2
        P_KEEP = args.keep
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(the step is sharded by design only; see the sharding notes).", file=sys.stderr)
        return 2

    if args.workload == "copy":
        return copy_calibration(args)
    if args.workload == "decode32":
        return decode_loop_bench(args)
    if args.workload == "spec128":
        return spec_step_bench(args)
    if args.workload == "attn128":
        return attention_bench(args)
    if args.workload == "pages32":
        return pipeline_bench(args)
    if args.workload == "step128attn":
        return attention_step_bench(args)

    import numpy as np
    import torch

    import moe_decoder_step_amd as m
    import synth

    m.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = synth.SHAPES[args.workload]
    if args.drafts is not None:
        import dataclasses
        sh = dataclasses.replace(sh, P=args.drafts + 1)
    T = sh.T
    log(f"workload {sh.name}: T={T} L={sh.L} V={sh.V}; generating weights on {dev}")
    t0 = time.time()
    prefill = sh.name == "prefill"
    cycle = 4 if sh.name == "layer128" else 1
    if prefill:
        # the real-shape layer's weights with the Zipf(1.1) router bias
        # (calibrated by tests/golden/make_zipf_bias.py); hidden states seed 3
        with open(ZIPF_BIAS) as f:
            fx = json.load(f)
        layers = [synth.layer_weights(fx["router_weight"]["seed"], fx["router_weight"]["layer"], sh, dev)]
        layers[0]["bias"] = torch.tensor(fx["bias"], dtype=torch.float32, device=dev)
        h_in = synth.hidden(3, T, sh.H, torch.bfloat16, dev)
    else:
        # the one-layer workload cycles through 4 layers of distinct weights
        # (1.8 GB) so that the 256 MB Infinity Cache cannot serve repeated reads;
        # its figures are per layer
        layers = [synth.layer_weights(0, l, sh, dev) for l in range(sh.L * cycle)]
        h_in = synth.hidden(0, T, sh.H, torch.bfloat16, dev, name="step_hidden")
    w_lm = synth.lm_weight(0, sh, dev) if sh.V else None
    drafts = synth.uniform_ids(0, (sh.B, sh.K), sh.V or 2).to(dev)
    torch.cuda.synchronize()
    log(f"weights ready in {time.time() - t0:.1f}s")

    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=T, max_seqs=sh.B, K=sh.K)

    batch1 = sh.name == "batch1"
    if batch1:
        # drafts planted from each pass's own greedy tokens, keep probability
        # 0.576 per position (200 steps of masks; the timed steps reuse step 0's)
        keep_all, repl_all = synth.plant_schedule(0, 200, sh.B, sh.K, sh.V, P_KEEP)
        keep_d, repl_d = keep_all.to(dev), repl_all.to(dev)
        keep_s, repl_s = keep_d[0].clone(), repl_d[0].clone()

        def step():
            st.step_planted(h_in, keep_s, repl_s, drafts)
    else:
        def step():
            st.forward(h_in)
            if w_lm is not None:
                st.head(T)
                st.verify(drafts)

    # routed experts touched per layer (weights the step must read)
    rec = []
    st.forward(h_in, rec)
    touched = [int(np.unique(r["ids"].cpu().numpy()).size) for r in rec]
    load = np.bincount(rec[0]["ids"].cpu().numpy().ravel(), minlength=sh.E)
    del rec
    layer_bytes = [(t + sh.S) * expert_bytes(sh) + sh.E * sh.H * 4 + 2 * T * sh.H * 2 for t in touched]
    step_bytes = sum(layer_bytes) / cycle + (sh.V * sh.H * 2 if sh.V else 0)
    # gate/up kernel per launch: gate and up rows of every touched expert and
    # the normed tokens in (the SwiGLU activation rows it writes are an
    # intermediate, left out of the algorithmic bytes)
    n_rows = T * sh.k + sh.S * T
    gu_bytes = [(t + sh.S) * 2 * sh.I * sh.H * 2 + T * sh.H * 2 for t in touched]
    gu_flops = n_rows * 2 * (2 * sh.I) * sh.H
    layer_flops = 2 * T * sh.H * sh.E + n_rows * 6 * sh.H * sh.I      # router + experts

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done; timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps / cycle
    log(f"{ms:.3f} ms/step" + (f" (per layer, {cycle} weight sets cycled)" if cycle > 1 else ""))

    graph_info = None
    if batch1:
        # committed tokens per pass over the 200 planted steps (eager)
        commits = []
        for i in range(keep_d.shape[0]):
            keep_s.copy_(keep_d[i])
            repl_s.copy_(repl_d[i])
            step()
            commits.append(st.n_commit[:sh.B].clone())
        commit_mean = float(torch.stack(commits).float().mean())
        keep_s.copy_(keep_d[0])
        repl_s.copy_(repl_d[0])
        eager_ms = ms
        graph_ms = None
        if not args.no_graph:
            # the whole pass (65 launches) captured once and replayed
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            for _ in range(args.warmup):
                graph.replay()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(args.steps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_ms = e0.elapsed_time(e1) / args.steps
            ms = graph_ms
            log(f"graph replay: {graph_ms:.3f} ms/step (eager {eager_ms:.3f})")
        expected = sum(P_KEEP ** i for i in range(sh.K + 1))
        graph_info = {"K": sh.K, "eager_ms_per_step": eager_ms, "graph_ms_per_step": graph_ms,
                      "committed_per_step_mean": commit_mean, "committed_per_step_expected": expected,
                      "committed_tokens_per_s": commit_mean * sh.B / (ms * 1e-3),
                      "keep_probability": P_KEEP, "planted_steps": int(keep_d.shape[0])}

    # per-step distribution (a separate pass, events around every step; the
    # headline above is the bracketed mean)
    pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in pev:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per_step = np.array([a.elapsed_time(b) for a, b in pev]) / cycle
    dist = {"p10": float(np.percentile(per_step, 10)), "p50": float(np.percentile(per_step, 50)),
            "p90": float(np.percentile(per_step, 90)), "steps": int(per_step.size), "launch": "eager"}

    # dominant kernel (expert gate/up, routed + shared experts): HIP events
    # around each launch on the stream it runs on, over a second timed pass
    st.ffn_events = ev = []
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    st.ffn_events = None
    gu_ms = float(np.mean([s.elapsed_time(e) for s, e in ev]))
    gu_b = float(np.mean(gu_bytes))
    achieved = gu_b / (gu_ms * 1e-3) / 1e9
    log(f"expert gate/up: {gu_ms * 1e3:.1f} us/launch, {achieved:.0f} GB/s")
    traffic, traffic_src = measured_traffic(sh.name)
    if prefill:
        tflops = gu_flops / (gu_ms * 1e-3) / 1e12
        log(f"expert gate/up: {gu_ms * 1e3:.1f} us/launch, {tflops:.0f} TFLOP/s")
        roofline = {"kernel": "moe_expert_gate_up (gemm_kernel<true>)", "bound": "mfma", "achieved": tflops,
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
                    "traffic": traffic, "traffic_source": traffic_src,
                    "us_per_launch": gu_ms * 1e3, "algorithmic_flops_per_launch": gu_flops}
    else:
        roofline = {"kernel": "moe_expert_gate_up_routed (skinny_kernel<true, true>)" if T * sh.k <= 4096
                    else "moe_expert_gate_up (skinny_kernel<true, false>)", "bound": "hbm",
                    "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "traffic_source": traffic_src,
                    "us_per_launch": gu_ms * 1e3, "algorithmic_bytes_per_launch": gu_b}

    if sh.name == "step128":
        metric = "MoE verify-step tokens/s (32 seq x 4 tok, 12 layers)"
    elif batch1:
        metric = f"MoE verify-step tokens/s (batch 1 x {sh.P} tok, 12 layers"
        metric += ", eager)" if args.no_graph else ", graph replay)"
    elif prefill:
        metric = "MoE prefill-layer tokens/s (32 pages x 1,156 tokens, Zipf(1.1) experts)"
    elif cycle > 1:
        metric = f"MoE layer tokens/s ({sh.B} seq x {sh.P} tok, one layer, {cycle} weight sets cycled)"
    else:
        metric = f"MoE verify tokens/s ({sh.name})"
    out = {
        "metric": metric,
        "value": T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"prefill MoE layer, {sh.B} pages x {sh.P} tokens = {T} tokens, "
                                "router bias for Zipf(1.1) expert popularity") if prefill else
                   (f"verify pass, {sh.B} seq x {sh.P} positions = {T} tokens, {sh.L} MoE layers"
                    + (f" + LM head {sh.H}x{sh.V} argmax + greedy acceptance" if sh.V else "")
                    + (f" (per layer over {cycle} layers of distinct weights, {cycle} x 455 MB)" if cycle > 1
                       else "")),
                   "hidden": sh.H, "experts": f"{sh.E} routed + {sh.S} shared, top-{sh.k}",
                   "expert_intermediate": sh.I, "global_batch": T},
        "step_hbm": {"algorithmic_bytes": step_bytes, "achieved_GBs": step_bytes / (ms * 1e-3) / 1e9,
                     "frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "touched_experts_per_layer": touched},
        "roofline": roofline,
    }
    if graph_info is not None:
        out["batch1"] = graph_info
    out["ms_per_step_distribution"] = dist
    if prefill:
        out["layer_mfma"] = {"algorithmic_flops": layer_flops,
                             "achieved_TFLOPs": layer_flops / (ms * 1e-3) / 1e12,
                             "frac": layer_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                             "expert_rows_desc": np.sort(load)[::-1].tolist()}

    if sh.name == "step128" and not args.no_companions:
        out["companions"] = companions(args)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, sh, layers, w_lm, h_in, T)
        one = cpu_baseline_1core(args, sh, layers, w_lm, h_in, T)
        if one is not None:
            out["cpu_baseline_1core"] = one
    print(json.dumps(out), flush=True)
    return 0


COMPANION_KEYS = {
    "layer128": ("step_hbm", "roofline", "cpu_baseline", "cpu_baseline_1core"),
    "batch1": ("step_hbm", "batch1", "roofline", "cpu_baseline", "cpu_baseline_1core"),
    "prefill": ("layer_mfma", "roofline", "step_hbm", "cpu_baseline", "cpu_baseline_1core"),
    "decode32": ("loop", "roofline", "cpu_baseline"),
    "decode32_tau": ("loop",),
}


def companions(args) -> dict:
    """The other configurations, measured in the same run: one real-shape
    layer at 128 tokens, batch-1 verify (graph replay, K = 3), the
    36,992-token prefill layer and the concurrency-32 decode loop (drafts
    kept with the pages' acceptance rate 0.576, and again with q = 0.749,
    whose mean commits per pass equal the pages' tau of 2.73), each by this
    script in a child process of its own (--workload W; the oracle baselines
    on one repetition of their samples unless --no-cpu-baseline); their
    lines, trimmed, under their names.  The headline's timed region is over
    before the first child starts."""
    import subprocess
    out = {}
    for w in COMPANION_KEYS:
        cmd = [sys.executable, "-u", os.path.abspath(__file__), "--steps", str(args.steps), "--warmup", str(args.warmup)]
        if w == "decode32_tau":   # the same loop with drafts kept at q: the pages' tau = 2.73 per pass
            cmd += ["--workload", "decode32", "--keep", str(Q_KEEP), "--no-cpu-baseline"]
        else:
            cmd += ["--workload", w] + (["--no-cpu-baseline"] if args.no_cpu_baseline else ["--cpu-reps", "1"])
        log(f"companion line: {' '.join(cmd[2:])}")
        try:
            r = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=600)
        except subprocess.TimeoutExpired:
            out[w] = {"error": "timed out"}
            continue
        lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
        if r.returncode != 0 or not lines:
            out[w] = {"error": f"exit status {r.returncode}"}
            continue
        d = json.loads(lines[-1])
        keep = {k: d[k] for k in ("metric", "value", "unit", "ms_per_step", "config") if k in d}
        keep.update({k: d[k] for k in COMPANION_KEYS[w] if k in d})
        keep["command"] = "python bench.py " + " ".join(cmd[3:])
        out[w] = keep
    return out


def decode_loop_bench(args) -> int:
    """Concurrency-32 decode loop: 32 sequences of `target` committed tokens,
    K = 3 drafts planted with keep probability 0.576, the 12-layer stack and
    LM head; finished sequences leave the batch.  Timed: whole loops, wall
    clock, including the per-pass copy of the active count to the host."""
    import numpy as np
    import torch

    import moe_decoder_step_amd as m
    import synth

    m.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = synth.SHAPES["step128"]
    S, K, P, target = sh.B, sh.K, sh.P, args.target
    log(f"decode loop: {S} sequences x {target} tokens, K={K}; generating weights and input pools")
    layers = [synth.layer_weights(0, l, sh, dev) for l in range(sh.L)]
    w_lm = synth.lm_weight(0, sh, dev)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=S * P, max_seqs=S, K=K)
    h_pool = synth.normal(synth.subseed(4, "decode_hidden"), (S, target, P, sh.H), 1.0, torch.bfloat16, dev)
    keep, repl = synth.plant_schedule(4, target, S, K, sh.V, P_KEEP)
    loop = m.DecodeLoop(st, h_pool, keep.permute(1, 0, 2).contiguous().to(dev),
                        repl.permute(1, 0, 2).contiguous().to(dev), target)
    torch.cuda.synchronize()
    for _ in range(max(args.warmup, 0) and 1):
        loop.run()
    n_loops = max(1, min(args.steps, 3))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_loops):
        res = loop.run()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / n_loops
    committed = S * target
    sizes = res["batch_sizes"]
    log(f"{res['passes']} passes, {wall * 1e3:.1f} ms per loop, {committed / wall:.0f} committed tokens/s")
    out = {
        "metric": f"MoE decode-loop committed tokens/s ({S} seq x {target} tok, K={K}, 12 layers)",
        "value": committed / wall, "unit": "tokens/s", "n_gpus": 1, "steps": n_loops, "warmup": 1,
        "ms_per_step": wall * 1e3 / res["passes"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"decode loop, {S} sequences to {target} committed tokens, {P} positions per pass, "
                               f"drafts planted with keep probability {P_KEEP}, finished sequences compacted out",
                   "hidden": sh.H, "experts": f"{sh.E} routed + {sh.S} shared, top-{sh.k}",
                   "expert_intermediate": sh.I, "vocab": sh.V, "layers": sh.L},
        "roofline": ffn_roofline(st, h_pool[:, 0].reshape(S * P, sh.H), sh, 5),
        "loop": {"passes": res["passes"], "wall_ms": wall * 1e3, "mean_batch": float(np.mean(sizes)),
                 "full_batch_passes": int(sum(1 for b in sizes if b == S)),
                 "committed_per_pass_per_seq": committed / float(np.sum(sizes)),
                 "expected_committed_per_pass": sum(P_KEEP ** i for i in range(K + 1))},
    }
    if not args.no_cpu_baseline:
        # the oracle over the loop's first full-batch passes (12 layers + LM
        # head + acceptance on 32 x 4 positions each), extrapolated per verify
        # position to every pass the GPU loop ran
        import copy
        a = copy.copy(args)
        a.cpu_layers, a.cpu_tokens, a.cpu_vocab, a.cpu_reps = sh.L, S * P, sh.V, max(1, args.cpu_steps)
        first = h_pool[:, 0].reshape(S * P, sh.H)
        cb = cpu_baseline(a, sh, layers, w_lm, first, S * P)
        positions = float(np.sum(sizes)) * P
        t_loop = positions / cb["value"]
        cb.update({"value": committed / t_loop, "unit": "tokens/s", "extrapolated": True,
                   "sample": f"{a.cpu_reps} full-batch passes of the oracle ({S} x {P} positions, {sh.L} layers + "
                             f"LM head {sh.V} rows), {cb['value']:.1f} verify positions/s, extrapolated to the "
                             f"loop's {res['passes']} passes ({positions:.0f} positions): {t_loop:.0f} s per loop"})
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)
    return 0


def pipeline_bench(args) -> int:
    """Prefill -> decode for 32 pages as one timed pipeline: the 12-layer
    stack over 32 x 1,156 prompt tokens (36,992 tokens, tiled-GEMM experts),
    the first output token of each page from its last prompt row, then the
    decode loop to 1,085 tokens per page (K = 3 planted drafts, finished pages
    compacted out).  Wall clock over whole pipelines; the prefill's gate/up
    GEMM launches are also timed with HIP events for the MFMA roofline."""
    import numpy as np
    import torch

    import moe_decoder_step_amd as m
    import synth

    m.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = synth.SHAPES["step128"]
    S, K, P, target, Lp = sh.B, sh.K, sh.P, args.target, args.prompt
    T = S * Lp
    log(f"pipeline: {S} pages x {Lp} prompt tokens, then {target} tokens per page; generating weights")
    layers = [synth.layer_weights(0, l, sh, dev) for l in range(sh.L)]
    w_lm = synth.lm_weight(0, sh, dev)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=S * P, max_seqs=S, K=K)
    del layers, w_lm
    h_pool = synth.normal(synth.subseed(4, "decode_hidden"), (S, target, P, sh.H), 1.0, torch.bfloat16, dev)
    keep, repl = synth.plant_schedule(4, target, S, K, sh.V, P_KEEP)
    loop = m.DecodeLoop(st, h_pool, keep.permute(1, 0, 2).contiguous().to(dev),
                        repl.permute(1, 0, 2).contiguous().to(dev), target)
    pipe = m.PagePipeline(st, Lp, loop)
    h_prompt = synth.hidden(5, T, sh.H, torch.bfloat16, dev, name="prompt_hidden")
    torch.cuda.synchronize()
    pipe.run(h_prompt)                      # warmup
    torch.cuda.synchronize()
    n_runs = max(1, min(args.steps, 3))
    t_pre, t_all = [], []
    for _ in range(n_runs):
        t0 = time.perf_counter()
        pipe.prefill(h_prompt)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        res = loop.run(first=pipe.first)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        t_pre.append(t1 - t0)
        t_all.append(t2 - t0)
    wall = float(np.mean(t_all))
    pre = float(np.mean(t_pre))
    # the prefill's gate/up GEMM launches, HIP events on their stream
    pipe.pre.ffn_events = ev = []
    pipe.prefill(h_prompt)
    torch.cuda.synchronize()
    pipe.pre.ffn_events = None
    gu_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gu_flops = T * (sh.k + sh.S) * 2 * (2 * sh.I) * sh.H
    tflops = gu_flops / (gu_ms * 1e-3) / 1e12
    out_tokens = S * target
    log(f"prefill {pre * 1e3:.1f} ms, decode {(wall - pre) * 1e3:.1f} ms ({res['passes']} passes), "
        f"{S / wall:.2f} pages/s, {out_tokens / wall:.0f} output tokens/s; prefill gate/up {gu_ms * 1e3:.0f} us, "
        f"{tflops:.0f} TFLOP/s")
    out = {
        "metric": f"page-batch output tokens/s ({S} pages x {Lp} prompt tokens prefill + {target} decoded tokens "
                  f"per page, 12 layers)",
        "value": out_tokens / wall, "unit": "tokens/s", "n_gpus": 1, "steps": n_runs, "warmup": 1,
        "ms_per_step": wall * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"prefill of {S} x {Lp} = {T} prompt tokens through the 12-layer stack, first "
                               f"token per page from its last prompt row, then the decode loop to {target} tokens "
                               f"per page ({P} positions per pass, drafts planted with keep probability {P_KEEP}); "
                               f"attention omitted",
                   "hidden": sh.H, "experts": f"{sh.E} routed + {sh.S} shared, top-{sh.k}", "vocab": sh.V,
                   "layers": sh.L},
        "pipeline": {"wall_ms": wall * 1e3, "prefill_ms": pre * 1e3, "decode_ms": (wall - pre) * 1e3,
                     "passes": res["passes"], "pages_per_s": S / wall,
                     "pages_context": "the pages: 2.57 pages/s, 2,792 output tokens/s on one A100 SXM4 40GB at "
                                      "concurrency 32, end to end with vision, attention and serving (context, not "
                                      "a target)"},
        "roofline": {"kernel": "moe_expert_gate_up in the prefill (gemm_kernel<true>)", "bound": "mfma",
                     "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS, "traffic": None,
                     "traffic_source": "no counter run recorded for this kernel",
                     "us_per_launch": gu_ms * 1e3, "algorithmic_flops_per_launch": gu_flops},
    }
    print(json.dumps(out), flush=True)
    return 0


def spec_step_bench(args) -> int:
    """One speculative step at concurrency 32: the dense draft block proposes
    K = 3 tokens per sequence (3 recursive steps, each through the 129,280-row
    LM head), then the verify pass checks them (32 x 4 tokens, 12 layers, LM
    head, acceptance).  Also times a plain greedy pass (32 x 1 tokens) to give
    the step cost c in greedy passes, and the speedup tau / c at the planted
    acceptance and at the pages' tau."""
    import torch

    import moe_decoder_step_amd as m
    import synth

    m.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    import dataclasses
    sh = dataclasses.replace(synth.SHAPES["step128"], B=args.seqs)
    B, K, P = sh.B, sh.K, sh.P
    log(f"spec step: {B} sequences, K={K}; generating weights")
    layers = [synth.layer_weights(0, l, sh, dev) for l in range(sh.L)]
    w_lm = synth.lm_weight(0, sh, dev)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=B * P, max_seqs=B, K=K)
    head = m.DraftHead(synth.draft_weights(0, sh, dev), st.w_lm, max_seqs=B, K=K)
    del layers, w_lm
    h_in = synth.hidden(0, B * P, sh.H, torch.bfloat16, dev, name="step_hidden")
    h_last = synth.hidden(1, B, sh.H, torch.bfloat16, dev, name="draft_hidden")
    tok = synth.uniform_ids(0, (B,), sh.V, name="last_tokens").to(dev)
    drafts = torch.empty((B, K), dtype=torch.int32, device=dev)
    no_drafts = torch.empty((B, 0), dtype=torch.int32, device=dev)

    def draft():
        drafts.copy_(head.propose(h_last, tok))

    def verify():
        st.forward(h_in)
        st.head(B * P)
        st.verify(drafts)

    def greedy():
        st.forward(h_in[:B])
        st.head(B)
        st.verify(no_drafts)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    roofline = ffn_roofline(st, h_in, sh, args.steps)
    t_draft = timed(draft)
    t_verify = timed(verify)
    t_spec = timed(lambda: (draft(), verify()))
    t_ar = timed(greedy)
    c = t_spec / t_ar
    tau_planted = sum(P_KEEP ** i for i in range(K + 1))
    log(f"draft {t_draft:.3f} ms, verify {t_verify:.3f} ms, step {t_spec:.3f} ms, greedy pass {t_ar:.3f} ms, "
        f"c = {c:.2f}")
    out = {
        "metric": f"MoE speculative-step tokens/s ({B} seq, K={K} drafts + verify, 12 layers, planted tau)",
        "value": tau_planted * B / (t_spec * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t_spec, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"dense draft block x {K} recursive steps (each through the {sh.V}-row LM head) "
                               f"+ verify pass of {B} x {P} tokens; value uses tau = {tau_planted:.3f} committed "
                               f"tokens per pass (keep probability {P_KEEP}): random draft weights cannot "
                               f"predict the verifier",
                   "hidden": sh.H, "draft_intermediate": synth.DRAFT_INTERMEDIATE, "vocab": sh.V, "layers": sh.L},
        "roofline": roofline,
        "spec": {"draft_ms": t_draft, "verify_ms": t_verify, "step_ms": t_spec, "greedy_pass_ms": t_ar,
                 "step_cost_in_greedy_passes": c, "speedup_at_planted_tau": tau_planted / c,
                 "speedup_at_pages_tau_2.73": 2.73 / c, "planted_tau": tau_planted},
    }
    print(json.dumps(out), flush=True)
    return 0


def _event_timer(steps, warmup, fn):
    """Average ms of fn over `steps` calls after `warmup`, HIP events on the
    current stream (the stream the library's kernels are launched on)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def attention_bench(args) -> int:
    """Causal attention of one layer's verify pass over its KV cache (32 seq x
    4 positions x 10 heads of 128), at several committed lengths: the rope +
    cache write and the split attention + merge (one moe_attention call), with
    the algorithmic bytes of the call (every visible key and value row once,
    the queries in, the output out)."""
    import torch

    import moe_decoder_step_amd as m
    import synth

    m.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = synth.SHAPES["step128"]
    B, P, nh, D = sh.B, sh.P, sh.H // synth.ATTN_HEAD_DIM, synth.ATTN_HEAD_DIM
    T, H = B * P, sh.H
    ctx = [int(c) for c in (args.context or "2241,1156,8192,32768").split(",")]
    qkv = synth.normal(1, (T, 3 * H), 1.0, torch.bfloat16, dev)
    q = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    rows = []
    for L in ctx:
        max_len = L + P
        kv = synth.kv_prefix(2, 0, (B, nh, max_len, 2, D), torch.bfloat16, dev, "kv")
        lengths = torch.full((B,), L, dtype=torch.int32, device=dev)
        ws = torch.empty(m.attention_workspace_bytes(B, P, nh, max_len), dtype=torch.uint8, device=dev)
        t_rope = _event_timer(args.steps, args.warmup, lambda: m.moe_attn_rope_cache(qkv, lengths, P, q, kv))
        t_att = _event_timer(args.steps, args.warmup, lambda: m.moe_attention(q, kv, lengths, P, o, ws))
        kv_bytes = B * nh * (L + P) * D * 2 * 2
        nbytes = kv_bytes + 2 * T * H * 2
        gbs = nbytes / (t_att * 1e-3) / 1e9
        log(f"context {L}: rope+cache {t_rope * 1e3:.1f} us, attention {t_att * 1e3:.1f} us, {gbs:.0f} GB/s")
        rows.append({"context": L, "rope_cache_us": t_rope * 1e3, "attention_us": t_att * 1e3,
                     "algorithmic_bytes": nbytes, "GBs": gbs, "frac": gbs / HBM_PEAK_GBS})
        del kv, ws
        torch.cuda.empty_cache()
    r0 = rows[0]
    ms = (r0["rope_cache_us"] + r0["attention_us"]) * 1e-3
    out = {
        "metric": f"verify-pass attention tokens/s (32 seq x 4 tok, one layer, context {r0['context']})",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"causal attention of {B} seq x {P} positions over a {nh}-head KV cache "
                               f"(head 128) of {r0['context']} committed positions, one layer",
                   "hidden": H, "heads": nh, "contexts": ctx},
        "roofline": {"kernel": "moe_attention (attn_split_kernel + attn_merge_kernel)", "bound": "hbm",
                     "achieved": r0["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": r0["frac"],
                     "traffic": None, "traffic_source": "no counter run recorded for this kernel",
                     "us_per_launch": r0["attention_us"], "algorithmic_bytes_per_launch": r0["algorithmic_bytes"]},
        "contexts": rows,
    }
    print(json.dumps(out), flush=True)
    return 0


def attention_step_bench(args) -> int:
    """The verify step with attention: 12 layers of (attention over a KV
    cache of `context` committed positions + MoE block), LM head, acceptance,
    32 seq x 4 tokens.  Lengths are not advanced between timed passes (each
    pass re-verifies at the same positions), so every pass costs the same."""
    import numpy as np
    import torch

    import moe_decoder_step_amd as m
    import synth

    m.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = synth.SHAPES["step128"]
    L = int(args.context or 1700)
    T, nh = sh.T, sh.H // synth.ATTN_HEAD_DIM
    log(f"verify step with attention at context {L}: generating weights")
    layers = [synth.layer_weights(0, l, sh, dev) for l in range(sh.L)]
    attn = [synth.attn_weights(0, l, sh, dev) for l in range(sh.L)]
    w_lm = synth.lm_weight(0, sh, dev)
    st = m.VerifyStack(layers, w_lm, sh.E, sh.k, sh.S, max_tokens=T, max_seqs=sh.B, K=sh.K, attn=attn,
                       n_heads=nh, max_len=L + sh.P)
    for li, blk in enumerate(st.attn):
        blk.cache_k.copy_(synth.kv_prefix(3, li, blk.cache_k.shape, torch.bfloat16, dev, "k"))
        blk.cache_v.copy_(synth.kv_prefix(3, li, blk.cache_v.shape, torch.bfloat16, dev, "v"))
    st.lengths.fill_(L)
    del layers, attn, w_lm
    h_in = synth.hidden(0, T, sh.H, torch.bfloat16, dev, name="step_hidden")
    drafts = synth.uniform_ids(0, (sh.B, sh.K), sh.V).to(dev)

    def step():
        st.forward(h_in)
        st.head(T)
        st.verify(drafts)

    ms = _event_timer(args.steps, args.warmup, step)
    # attention share: one layer's moe_attention call timed alone
    blk = st.attn[0]
    lengths = st.lengths[:sh.B]
    t_att = _event_timer(args.steps, args.warmup, lambda: m.moe_attention(
        blk.q[:T], blk.kv, lengths, sh.P, blk.o[:T], blk.ws))
    kv_bytes = sh.B * nh * (L + sh.P) * synth.ATTN_HEAD_DIM * 2 * 2
    nbytes = kv_bytes + 2 * T * sh.H * 2
    gbs = nbytes / (t_att * 1e-3) / 1e9
    log(f"{ms:.3f} ms/step; attention {t_att * 1e3:.1f} us/layer, {gbs:.0f} GB/s")
    out = {
        "metric": f"verify-step tokens/s with attention (32 seq x 4 tok, 12 layers, context {L})",
        "value": T / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"verify pass, {sh.B} seq x {sh.P} positions, {sh.L} layers of causal attention "
                               f"({nh} heads of 128, KV cache of {L} committed positions) + MoE block, LM head "
                               f"{sh.H}x{sh.V} argmax + greedy acceptance",
                   "hidden": sh.H, "context": L, "global_batch": T},
        "roofline": {"kernel": "moe_attention (attn_split_kernel + attn_merge_kernel)", "bound": "hbm",
                     "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                     "traffic": None, "traffic_source": "no counter run recorded for this kernel",
                     "us_per_launch": t_att * 1e3, "algorithmic_bytes_per_launch": nbytes},
        "attention_share": {"attention_us_per_layer": t_att * 1e3,
                            "fraction_of_step": sh.L * t_att / ms},
    }
    print(json.dumps(out), flush=True)
    return 0


def host_cpu() -> dict:
    """The host's CPU model (lscpu) and the cores this process may use."""
    model = None
    try:
        import subprocess
        r = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10)
        for line in r.stdout.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except Exception:
        nproc = os.cpu_count()
    return {"cpu_model": model, "nproc": nproc}


def cpu_baseline(args, sh, layers, w_lm, h_in, T) -> dict:
    """The fp64 oracle on the host cores over a bounded sample of the same
    step: `cpu_layers` MoE layers on `cpu_tokens` tokens plus the LM head over
    `cpu_vocab` vocabulary rows (by default the whole 128-token step), timed
    `cpu_reps` times and scaled to the full step when the sample is smaller."""
    import numpy as np
    import torch

    import oracle as O

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
    nl = min(args.cpu_layers, sh.L)
    nt = min(args.cpu_tokens, T)
    log(f"cpu baseline: oracle on {nl} layer(s) x {nt} tokens + {args.cpu_vocab} LM rows")
    hw = [{k: host(v) for k, v in layers[l].items()} for l in range(nl)]
    x = host(h_in[:nt])
    vs = min(args.cpu_vocab, sh.V) if w_lm is not None else 0
    wl = host(w_lm[:vs]) if vs else None
    reps = max(1, args.cpu_reps)
    t_layers = t_lm = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        cur = x
        for l in range(nl):
            cur = O.moe_layer(cur, hw[l], sh.k, sh.eps, "bf16")["h_out"]
        t1 = time.perf_counter()
        if vs:
            O.lm_argmax(cur, wl)
        t_layers += t1 - t0
        t_lm += time.perf_counter() - t1
    t_layers /= reps
    t_lm /= reps
    t_step = (t_layers * sh.L / nl + (t_lm * sh.V / vs if vs else 0.0)) * T / nt
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": T / t_step, "unit": "tokens/s", "cores": cores, "kind": "oracle", **host_cpu(),
            "sample": f"{nl} of {sh.L} MoE layers on {nt} of {T} tokens ({t_layers:.1f}s) + LM head over "
                      f"{vs} of {sh.V} vocabulary rows ({t_lm:.1f}s), mean of {reps} runs, scaled to the full "
                      f"step ({t_step:.1f}s per step)"}


def cpu_baseline_1core(args, sh, layers, w_lm, h_in, T):
    """The same oracle with its BLAS pools held to one thread, on a smaller
    sample (one MoE layer and an eighth of the LM head), scaled to the full
    step; None when the thread pools cannot be limited."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return None
    import copy
    a = copy.copy(args)
    a.cpu_layers, a.cpu_reps = 1, 1
    a.cpu_vocab = max(1, min(args.cpu_vocab, sh.V) // 8)
    with threadpool_limits(limits=1):
        r = cpu_baseline(a, sh, layers, w_lm, h_in, T)
    r["cores"] = 1
    return r


if __name__ == "__main__":
    sys.exit(main())
