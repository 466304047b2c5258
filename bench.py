"""Benchmark of the routed-MoE layer (NVFP4 experts) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_8192]
                [--configs decode_1,decode_64,verify_256]

A step is one moe_layer call (router, top-k, permutation, grouped gate/up +
SiLU*mul, grouped down, combine) on one batch of T synthetic tokens, with all
896 experts' NVFP4 weights (22.2 GB) resident in HBM.  Every step uses fresh
tokens (the generator's next T tokens), so each step routes to different
experts and reads their weights cold, as a decode step of a real model does.

The headline (`value`) is the prefill chunk, T = 8192: the largest workload,
bound by the matrix cores; its roofline is the grouped gate/up GEMM's MFMA
rate against the dense fp16 peak (and, as `frac_fp8`, against the dense FP8
peak, and, as `frac_of_sustained`, against what the library's calibration
kernel measures the fp16 matrix cores to sustain on this GPU under its power
limit, on operands with the GEMMs' value patterns).  In the same process and on the same resident store, `configs` times
the decode-sized workloads (single-user decode, 64-session decode,
speculative verify), which are bound by HBM, each over at least 50 ms of
back-to-back steps (`timed_steps`): layer tokens/s, the gate/up
kernel's achieved bandwidth and the layer's algorithmic bytes per second,
against 8 TB/s and against the streaming-read rate the library's calibration
kernel measures on this GPU.  `parity` checks sampled tokens of the timed
batches against the CPU oracle, and `cpu_baseline` times the oracle on those
tokens.  Prints one JSON line.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM TB/s (decode) / MFMA TFLOPS (prefill), 1 GPU"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
CONFIG_MIN_MS = 50.0            # shortest timed loop of a config (more steps for short ones)
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix, published
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix, published
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_REPS = 10                # launches per kernel in the per-kernel timing loops
MAX_ABS, REL_L2 = 2e-2, 5e-3    # output tolerance against the oracle
DEFAULT_CONFIGS = "decode_1,decode_64,verify_256"
CPU_THREADS_MAX = 16            # the host's CPU share of one GPU


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prefill_8192", help="the headline workload")
    ap.add_argument("--configs", default=None,
                    help="comma-separated workloads timed beside the headline, or 'none' (default: "
                         f"{DEFAULT_CONFIGS} for the plain NVFP4 layer, none otherwise)")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing and the parity checks")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--format", choices=("nvfp4", "mxfp4"), default="nvfp4", help="expert weight format")
    ap.add_argument("--shared", type=int, default=0,
                    help="add this many bf16 shared experts (width I) that every token uses")
    ap.add_argument("--ep", type=int, default=1,
                    help="time one device's share of an expert-parallel split into this many equal shares "
                         "(the first E/ep experts; routing still over all E)")
    return ap.parse_args(argv)


def extra_configs(args):
    """Workloads timed beside the headline."""
    plain = args.format == "nvfp4" and not args.shared and args.ep == 1
    spec = args.configs if args.configs is not None else (DEFAULT_CONFIGS if plain else "none")
    if spec.strip().lower() in ("", "none"):
        return []
    return [c.strip() for c in spec.split(",") if c.strip() and c.strip() != args.workload]


def nvfp4_bytes(N, K):
    return N * (K // 2) + N * (K // 16) + 4


def mxfp4_bytes(N, K):
    return N * (K // 2) + N * (K // 32) + 4


def code_text(src):
    """Source text without comments and whitespace: what the compiler sees
    of it (string literals in these files hold no comment markers)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return "".join(src.split())


def kernel_source_sha(sources=None):
    """Identifies the GEMM kernels' code (comments and layout excluded), so
    that counter records taken on it are used only while it is unchanged."""
    h = hashlib.sha256()
    for f in ("kernels_ffn.hip", "common.h"):
        text = sources[f] if sources else open(os.path.join(ROOT, "routed_expert_ffn_amd", "csrc", f)).read()
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def stream_read_GBps(moe, torch, region_bytes=256 << 20, regions=16):
    """What a plain streaming read reaches on this GPU: the library's
    calibration kernel reads each of `regions` regions of `region_bytes`
    once, in turn (the 4 GiB cycle exceeds every cache, so every read comes
    from HBM); median over the regions."""
    buf = torch.empty(region_bytes * regions, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(moe.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    moe.moe_stream_read(buf[-region_bytes:], sink)  # first launch, not timed
    rates = []
    for r in range(regions):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        moe.moe_stream_read(buf[r * region_bytes:(r + 1) * region_bytes], sink)
        b.record()
        b.synchronize()
        rates.append(region_bytes / (a.elapsed_time(b) * 1e-3) / 1e9)
    del buf
    return float(sorted(rates)[len(rates) // 2])


def mfma_sustained_TFLOPs(moe, torch, iters=16000, runs=5):
    """What the fp16 matrix cores sustain on this GPU under its power limit,
    on operands with the expert GEMMs' value patterns: the library's
    calibration kernel (iters * MFMA_RATE_FLOPS_PER_ITER flops a call, about
    12 ms), median over the runs after one untimed call."""
    sink = torch.zeros(moe.MFMA_RATE_BLOCKS, dtype=torch.float32, device="cuda")
    moe.moe_mfma_rate(iters // 8, sink)
    rates = []
    for _ in range(runs):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        moe.moe_mfma_rate(iters, sink)
        b.record()
        b.synchronize()
        rates.append(iters * moe.MFMA_RATE_FLOPS_PER_ITER / (a.elapsed_time(b) * 1e-3) / 1e12)
    return float(sorted(rates)[len(rates) // 2])


def load_traffic(workload, sha):
    """HBM traffic of the gate/up kernel per launch, from the committed
    rocprofv3 counter summary, if it was taken on this kernel source."""
    path = os.path.join(PROFILES, f"gateup_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_info():
    """CPU model and the CPUs this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "usable_cpus": usable}


def median(v):
    v = sorted(v)
    n = len(v)
    return v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])


class Bench:
    """The resident expert store and router weights, shared by every
    workload of the run (all workloads use the same seed and shapes)."""

    def __init__(self, args, wl):
        import torch

        import routed_expert_ffn_amd as moe
        import synth

        self.args, self.torch, self.moe, self.synth = args, torch, moe, synth
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.H, self.I, self.E, self.k = wl.H, wl.I, wl.E, wl.k
        self.Hm = wl.H_model or wl.H
        t0 = time.perf_counter()
        self.share = wl.E // args.ep  # experts held here: 0 .. share-1
        store = moe.ExpertStore(self.share, wl.H, wl.I, device=self.dev, fmt=args.format)
        buf = {m: torch.empty(store.shape(m), dtype=torch.float32, device=self.dev) for m in store.MATS}
        for e in range(self.share):
            for mi, m in enumerate(store.MATS):
                synth.gpu_expert_f32(wl.seed, e, mi, buf[m])
                store.quantize_into(e, m, buf[m])
        del buf
        self.store = store
        # the latent block's tokens, router and output have the hidden width
        self.wr = torch.empty((self.Hm, wl.E), dtype=torch.bfloat16, device=self.dev)
        synth.gpu_router_bf16(wl.seed, self.wr)
        if wl.H_model:
            self.p_down = torch.empty((self.Hm, wl.H), dtype=torch.bfloat16, device=self.dev)
            self.p_up = torch.empty((wl.H, self.Hm), dtype=torch.bfloat16, device=self.dev)
            synth.gpu_proj_bf16(wl.seed, 0, self.p_down)
            synth.gpu_proj_bf16(wl.seed, 1, self.p_up)
        if args.shared:
            self.sh_gu = torch.empty((wl.H, args.shared * 2 * wl.I), dtype=torch.bfloat16, device=self.dev)
            self.sh_dn = torch.empty((args.shared * wl.I, wl.H), dtype=torch.bfloat16, device=self.dev)
            synth.gpu_proj_bf16(wl.seed, 2, self.sh_gu)
            synth.gpu_proj_bf16(wl.seed, 3, self.sh_dn)
        torch.cuda.synchronize()
        self.setup_s = time.perf_counter() - t0
        self.stream_peak = stream_read_GBps(moe, torch)
        self.mfma_sustained = mfma_sustained_TFLOPs(moe, torch)
        self.sha = kernel_source_sha()

    def run(self, wl, steps, warmup, headline):
        """Times one workload: warmup, then exactly `steps` steps between two
        events on the launch stream.  For the headline the gate/up launches of
        the timed steps are also timed with events on that stream (each
        record costs the stream a few microseconds, under 0.1% of a prefill
        step); for the other workloads the timed steps carry no events and
        the kernels are timed in a separate loop afterwards."""
        torch, moe, synth, args = self.torch, self.moe, self.synth, self.args
        from synth.workloads import bias_for

        T, H, I, E, k, Hm = wl.T, wl.H, wl.I, wl.E, wl.k, self.Hm
        assert (H, I, E, k) == (self.H, self.I, self.E, self.k) and (wl.H_model or H) == Hm
        dev = self.dev
        n_kern = 0 if args.no_breakdown and headline else KERNEL_REPS
        b = bias_for(wl)
        bias = None if b is None else torch.tensor(b, device=dev)

        def batches(n_steps):
            # fresh token batches for warmup, the timed steps, the graph replay
            # and the kernel loop (the generator is deterministic: the first
            # batches are the same whatever the count)
            nb = n_steps + warmup
            n_gr = 0 if args.no_graph else n_steps
            tot = nb + n_gr + n_kern
            x_all = torch.empty((tot * T, Hm), dtype=torch.bfloat16, device=dev)
            synth.gpu_x_bf16(wl.seed, x_all)
            return nb, n_gr, tot, x_all, torch.empty((tot, T, k), dtype=torch.int32, device=dev), \
                torch.empty((tot, T, k), dtype=torch.float32, device=dev)

        n_batches, n_graph, total, xs, ids, wts = batches(steps)
        d = moe.dims(T, H, I, E, k)
        if wl.H_model:
            ws = torch.empty(moe.moe_latent_workspace_bytes(d, Hm), dtype=torch.uint8, device=dev)
        elif args.shared:
            ws = torch.empty(moe.moe_layer_shared_workspace_bytes(d, args.shared, I), dtype=torch.uint8, device=dev)
        else:
            ws = torch.empty(moe.moe_workspace_bytes(d), dtype=torch.uint8, device=dev)
        y = torch.empty((T, Hm), dtype=torch.float32 if args.ep > 1 else torch.bfloat16, device=dev)
        share = self.share

        def step(i):
            x = xs[i * T:(i + 1) * T]
            if args.ep > 1:
                moe.moe_layer_share(d, 0, share, x, self.wr, bias, self.store, y, None, ids[i], wts[i], ws)
            elif args.shared:
                moe.moe_layer_shared(d, args.shared, I, self.sh_gu, self.sh_dn, x, self.wr, bias, self.store, y,
                                     ids[i], wts[i], ws)
            elif wl.H_model:
                moe.moe_latent_layer(d, Hm, self.p_down, self.p_up, x, self.wr, bias, self.store, y, None, ids[i],
                                     wts[i], ws)
            else:
                moe.moe_layer(d, x, self.wr, bias, self.store, y, ids[i], wts[i], ws)

        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0.record()
        for i in range(warmup):
            step(i)
        w1.record()
        torch.cuda.synchronize()
        if not headline and warmup > 0:
            # a config's timed loop spans at least CONFIG_MIN_MS of back-to-back
            # steps, so that the launch ramp after the synchronisation before
            # it (about 0.1 ms) is not charged to a handful of 0.1 ms steps
            need = int(np.ceil(CONFIG_MIN_MS / max(w0.elapsed_time(w1) / warmup, 1e-3)))
            if need > steps:
                steps = need
                del xs, ids, wts
                n_batches, n_graph, total, xs, ids, wts = batches(steps)

        # ---- timed region ----------------------------------------------------
        if headline:
            moe.moe_profile_arm("gateup", steps)
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(warmup, n_batches):
            step(i)
        end.record()
        torch.cuda.synchronize()
        elapsed_ms = start.elapsed_time(end)
        gateup_ms = moe.moe_profile_read(steps) if headline else None
        y_last = y.float().cpu()  # output of the last timed step (for the parity check)
        i_last = n_batches - 1

        # ---- gate/up timed in a loop of its own on further fresh batches ------
        base = n_batches + n_graph
        if not headline:
            moe.moe_profile_arm("gateup", n_kern)
            for i in range(base, base + n_kern):
                step(i)
            torch.cuda.synchronize()
            gateup_ms = moe.moe_profile_read(n_kern)
        assert gateup_ms and len(gateup_ms) == (steps if headline else n_kern)
        gu_steps = list(range(warmup, n_batches)) if headline else list(range(base, base + n_kern))

        ids_np = ids.cpu().numpy()
        # distinct active experts per step (of this device's share)
        distinct_of = {i: len(np.unique(ids_np[i][ids_np[i] < share])) for i in range(total)}
        pairs_of = {i: int(np.count_nonzero(ids_np[i] < share)) for i in range(total)}
        timed = range(warmup, n_batches)
        distinct = np.array([distinct_of[i] for i in timed], dtype=np.float64)
        local_pairs = float(np.mean([pairs_of[i] for i in timed]))

        # ---- algorithmic work -------------------------------------------------
        ms_per_step = elapsed_ms / steps
        mat_bytes = mxfp4_bytes if args.format == "mxfp4" else nvfp4_bytes
        expert_bytes = 2 * mat_bytes(I, H) + mat_bytes(H, I)
        # latent block: plus the two projection weights; router and x, y at the hidden width
        proj_bytes = 2 * Hm * H * 2 if wl.H_model else 0
        proj_bytes += args.shared * 3 * H * I * 2  # bf16 shared experts
        y_bytes = T * Hm * (4 if args.ep > 1 else 2)
        layer_bytes = distinct.mean() * expert_bytes + Hm * E * 2 + T * Hm * 2 + y_bytes + proj_bytes
        layer_flops = (2 * T * Hm * E + 6 * local_pairs * H * I + (4 * T * Hm * H if wl.H_model else 0)
                       + 6 * T * args.shared * H * I)
        gateup_unit = 2 * mat_bytes(I, H)  # one active expert's gate+up weights
        gu_bytes = float(np.mean([distinct_of[i] * gateup_unit + T * H * 2 + pairs_of[i] * I * 2 for i in gu_steps]))
        gu_flops = float(np.mean([4 * pairs_of[i] * H * I for i in gu_steps]))
        gu_ms = float(np.mean(gateup_ms))
        gu_GBps = gu_bytes / (gu_ms * 1e-3) / 1e9
        gu_TF = gu_flops / (gu_ms * 1e-3) / 1e12
        layer_GBps = layer_bytes / (ms_per_step * 1e-3) / 1e9
        res = {
            "T": T, "ms_per_step": round(ms_per_step, 5), "timed_steps": steps,
            "tokens_per_s": round(T * steps / (elapsed_ms * 1e-3), 2),
            "distinct_experts_mean": float(distinct.mean()),
            "layer": {"algorithmic_bytes": int(layer_bytes), "hbm_GBps": round(layer_GBps, 1),
                      "hbm_frac": round(layer_GBps / HBM_PEAK_GBS, 4),
                      "frac_of_stream_read": round(layer_GBps / self.stream_peak, 4),
                      "algorithmic_flops": int(layer_flops),
                      "TFLOPs": round(layer_flops / (ms_per_step * 1e-3) / 1e12, 3)},
            "gateup": {"avg_launch_ms": round(gu_ms, 5), "timed_launches": len(gateup_ms),
                       "timed_in": "the timed steps" if headline else f"{n_kern} further steps after the timed region",
                       "algorithmic_bytes_per_launch": int(gu_bytes), "GBps": round(gu_GBps, 1),
                       "hbm_frac": round(gu_GBps / HBM_PEAK_GBS, 4),
                       "frac_of_stream_read": round(gu_GBps / self.stream_peak, 4),
                       "algorithmic_flops_per_launch": int(gu_flops), "TFLOPs": round(gu_TF, 1),
                       "traffic": load_traffic(wl.name, self.sha)},
        }

        # ---- per-kernel breakdown (after the timed region; not part of the value) ----
        if not args.no_breakdown:
            br = {}
            for name in moe.KERNELS:
                moe.moe_profile_arm(name, n_kern)
                for i in range(base, base + n_kern):
                    step(i)
                torch.cuda.synchronize()
                ms = moe.moe_profile_read(n_kern)
                br[name] = round(float(np.mean(ms)), 5) if ms else None
            res["kernel_ms"] = br

        # ---- HIP-graph replay (after the timed region; not part of the value) ----
        # the same step captured once per batch into one graph, on batches no
        # earlier step used (so the weights are read cold again), replayed once
        if n_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(n_batches, n_batches + n_graph):
                    step(i)
            torch.cuda.synchronize()
            a, b2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            graph.replay()
            b2.record()
            torch.cuda.synchronize()
            res["graph_ms_per_step"] = round(a.elapsed_time(b2) / n_graph, 5)
            del graph
        res["_last"] = {"y": y_last.numpy(), "ids": ids_np[i_last], "first_token": i_last * T}
        del xs, ws
        torch.cuda.empty_cache()
        return res


def workload_text(wl, fmt):
    return ((f"{wl.name}: latent MoE block, hidden {wl.H_model} -> routed latent {wl.H} (bf16 projections), "
             if wl.H_model else f"{wl.name}: MoE layer ")
            + f"T={wl.T} H={wl.H} I={wl.I} E={wl.E} top-{wl.k}, {fmt.upper()} experts, bf16 activations, "
              f"fresh tokens every step")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    from synth.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    extras = [WORKLOADS[c] for c in extra_configs(args)]
    if args.ep < 1 or wl.E % args.ep or (args.ep > 1 and wl.H_model) or (args.shared and (wl.H_model or args.ep > 1)):
        print(json.dumps({"error": "--ep must divide E; --ep and --shared go with the plain layer only, not together"}))
        sys.exit(2)
    for c in extras:
        if (c.H, c.I, c.E, c.k, c.H_model, c.seed) != (wl.H, wl.I, wl.E, wl.k, wl.H_model, wl.seed):
            print(json.dumps({"error": f"--configs: {c.name} does not share the headline's store"}))
            sys.exit(2)
    B = Bench(args, wl)
    steps, warmup = args.steps, args.warmup
    head = B.run(wl, steps, warmup, headline=True)
    prefill = wl.T >= 4096
    gu = head["gateup"]
    if prefill:
        tf = gu["TFLOPs"]
        roofline = {"bound": "mfma", "achieved": tf, "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": gu["traffic"],
                    "peak_fp8": FP8_MFMA_PEAK_TFLOPS, "frac_fp8": round(tf / FP8_MFMA_PEAK_TFLOPS, 4),
                    "sustained_TFLOPs": round(B.mfma_sustained, 1),
                    "frac_of_sustained": round(tf / B.mfma_sustained, 4),
                    "kernel": "gateup_kernel (grouped gate/up + SiLU*mul, fp16 MFMA on exactly dequantised NVFP4)",
                    "algorithmic_flops_per_launch": gu["algorithmic_flops_per_launch"],
                    "avg_launch_ms": gu["avg_launch_ms"], "timed_launches": gu["timed_launches"],
                    "achieved_GBps": gu["GBps"]}
    else:
        roofline = {"bound": "hbm", "achieved": gu["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": gu["hbm_frac"], "traffic": gu["traffic"],
                    "kernel": "gateup_kernel (grouped gate/up + SiLU*mul)",
                    "algorithmic_bytes_per_launch": gu["algorithmic_bytes_per_launch"],
                    "avg_launch_ms": gu["avg_launch_ms"], "timed_launches": gu["timed_launches"],
                    "stream_read_GBps": round(B.stream_peak, 1),
        "mfma_sustained_TFLOPs": round(B.mfma_sustained, 1), "frac_of_stream_read": gu["frac_of_stream_read"]}
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": workload_text(wl, args.format),
                   "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E, "k": wl.k, "H_model": wl.H_model,
                   "zipf_beta": wl.beta, "seed": wl.seed,
                   "expert_share": f"experts 0..{B.share - 1} of {wl.E}" if args.ep > 1 else None,
                   "shared_experts": args.shared, "weight_format": args.format},
        "roofline": roofline,
        "layer": head["layer"],
        "stream_read_GBps": round(B.stream_peak, 1),
        "mfma_sustained_TFLOPs": round(B.mfma_sustained, 1),
        "setup_s": round(B.setup_s, 2),
        "kernel_source_sha": B.sha,
    }
    for key in ("kernel_ms", "graph_ms_per_step"):
        if key in head:
            out[key] = head[key]
    cases = {}
    for c in extras:
        r = B.run(c, steps, warmup, headline=False)
        cases[c.name] = r
        out.setdefault("configs", {})[c.name] = {kk: v for kk, v in r.items() if kk != "_last"}
        out["configs"][c.name]["workload"] = workload_text(c, args.format)

    if not args.no_cpu_baseline and args.ep == 1 and not args.shared and args.format == "nvfp4":
        n_tok = args.cpu_tokens or 4
        cb, par = cpu_baseline(wl, n_tok, head["_last"])
        out["cpu_baseline"] = cb
        out["parity"] = par
        for c in extras:  # two tokens of each other workload's last timed batch
            _, p2 = cpu_baseline(c, 2, cases[c.name]["_last"], repeats=1)
            out["configs"][c.name]["parity"] = p2
    print(json.dumps(out))


def cpu_baseline(wl, n_tokens, last, repeats=3):
    """The CPU oracle, as it stands, on a bounded sample of the same
    workload: the first n_tokens tokens of the last timed batch, one
    single-token layer call each, the sample timed `repeats` times (the
    median is reported).  The experts those tokens select (found with the
    oracle's own router, untimed) are generated and quantised beforehand;
    the timed call routes, dequantises and runs its 16 experts and combines.
    The oracle's outputs are then compared with the GPU's outputs of the same
    tokens in that batch."""
    import concurrent.futures

    import oracle
    import synth
    from synth.workloads import bias_for

    n_tokens = max(1, min(n_tokens, wl.T))  # tokens of one batch
    info = cpu_info()
    threads = max(1, min(CPU_THREADS_MAX, info["usable_cpus"]))
    Hm = wl.H_model or wl.H
    wr = synth.router_bf16(wl.seed, Hm, wl.E)
    bias = bias_for(wl)
    first = last["first_token"]
    xs = [synth.x_bf16(wl.seed, 1, Hm, t0=first + t) for t in range(n_tokens)]
    if wl.H_model:
        p_down = synth.proj_bf16(wl.seed, 0, Hm, wl.H)
        p_up = synth.proj_bf16(wl.seed, 1, wl.H, Hm)
    need = set()
    for x in xs:
        ids, _ = oracle.topk_softmax(oracle.router_logits(x, wr, bias), wl.k)
        need |= set(int(e) for e in ids[0])

    def make(e):
        return tuple(oracle.nvfp4_quantize(synth.expert_f32(wl.seed, e, m, *synth.expert_shape(m, wl.H, wl.I),
                                                            nthreads=1)) for m in range(3))

    cache = {}
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        for e, v in zip(sorted(need), ex.map(make, sorted(need))):
            cache[e] = v
    times, outs = [], []
    for rep in range(repeats):
        total = 0.0
        for x in xs:
            t0 = time.perf_counter()
            if wl.H_model:
                o = oracle.latent_layer(x, cache, wl.E, wl.k, p_down, p_up, wr_bf16=wr, bias=bias, nthreads=threads)
            else:
                o = oracle.moe_layer(x, cache, wl.E, wl.k, wr_bf16=wr, bias=bias, nthreads=threads)
            total += time.perf_counter() - t0
            if rep == 0:
                outs.append(o)
        times.append(total)
    med = median(times)
    cb = {"value": round(n_tokens / med, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
          "sample": f"{n_tokens} tokens of the {wl.name} workload's last timed batch, one single-token oracle layer "
                    f"call each (router, top-k, permutation, 16 experts dequantised and run in fp64, combine"
                    f"{', and the two latent projections' if wl.H_model else ''}), "
                    f"{threads} threads over the token's experts; expert weights pre-quantised, untimed; "
                    f"median of {repeats} timings of the sample",
          "seconds": round(med, 2), "repeats": repeats, "seconds_each": [round(t, 2) for t in times],
          "cpu_model": info["cpu_model"], "host_cpus": info["host_cpus"], "usable_cpus": info["usable_cpus"]}
    # parity: the oracle (its own router) against the GPU's outputs of these tokens
    ref_ids = np.concatenate([o["ids"] for o in outs])
    ref_y = np.concatenate([o["y"] for o in outs])
    got_ids = last["ids"][:n_tokens]
    got_y = last["y"][:n_tokens].astype(np.float64)
    same = np.all(ref_ids == got_ids, axis=1)
    par = {"tokens": n_tokens, "ids_equal": bool(same.all()), "tokens_with_other_ids": int((~same).sum())}
    if same.any():
        diff = got_y[same] - ref_y[same]
        max_abs = float(np.abs(diff).max())
        rel = float(np.linalg.norm(diff) / max(np.linalg.norm(ref_y[same]), 1e-300))
        par.update({"max_abs": max_abs, "rel_l2": rel, "tolerance": {"max_abs": MAX_ABS, "rel_l2": REL_L2}})
        par["ok"] = bool(same.all() and max_abs <= MAX_ABS and rel <= REL_L2)
    else:
        par["ok"] = False
    return cb, par


if __name__ == "__main__":
    main()
