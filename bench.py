"""Benchmark of the routed-MoE layer (NVFP4 experts) on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode_1]

A step is one moe_layer call (router, top-k, permutation, grouped gate/up +
SiLU*mul, grouped down, combine) on one batch of T synthetic tokens, with all
896 experts' NVFP4 weights (22.2 GB) resident in HBM.  Every step uses fresh
tokens (the generator's next T tokens), so each step routes to different
experts and reads their weights cold, as a decode step of a real model does.
Prints one JSON line: whole-layer tokens/s, the dominant kernel's achieved
bandwidth against the HBM roofline (timed with HIP events on the launch
stream inside the timed region) and against the streaming-read rate the
library's calibration kernel measures on the same GPU, and the CPU oracle
timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM TB/s (decode) / MFMA TFLOPS (prefill), 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 matrix, published
PROFILES = os.path.join(ROOT, "profiles")
PROFILED_LAUNCHES = 10  # launches of the dominant kernel timed with events per run


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_1")
    ap.add_argument("--cpu-tokens", type=int, default=None, help="tokens in the oracle's timed sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--format", choices=("nvfp4", "mxfp4"), default="nvfp4", help="expert weight format")
    ap.add_argument("--shared", type=int, default=0,
                    help="add this many bf16 shared experts (width I) that every token uses")
    ap.add_argument("--ep", type=int, default=1,
                    help="time one device's share of an expert-parallel split into this many equal shares "
                         "(the first E/ep experts; routing still over all E)")
    return ap.parse_args()


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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np
    import torch

    import routed_expert_ffn_amd as moe
    import synth
    from synth.workloads import WORKLOADS, bias_for

    wl = WORKLOADS[args.workload]
    T, H, I, E, k = wl.T, wl.H, wl.I, wl.E, wl.k
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    steps, warmup = args.steps, args.warmup
    n_batches = steps + warmup
    n_graph = 0 if args.no_graph else steps  # fresh batches for the graph replay

    # ---- resident inputs -------------------------------------------------------
    t_setup = time.perf_counter()
    if args.ep < 1 or E % args.ep or (args.ep > 1 and wl.H_model) or (args.shared and (wl.H_model or args.ep > 1)):
        print(json.dumps({"error": "--ep must divide E; --ep and --shared go with the plain layer only, not together"}))
        sys.exit(2)
    share = E // args.ep  # experts held here: 0 .. share-1
    store = moe.ExpertStore(share, H, I, device=dev, fmt=args.format)
    buf = {m: torch.empty(store.shape(m), dtype=torch.float32, device=dev) for m in store.MATS}
    for e in range(share):
        for mi, m in enumerate(store.MATS):
            synth.gpu_expert_f32(wl.seed, e, mi, buf[m])
            store.quantize_into(e, m, buf[m])
    del buf
    # the latent block's tokens, router and output have the hidden width
    Hm = wl.H_model or H
    wr = torch.empty((Hm, E), dtype=torch.bfloat16, device=dev)
    synth.gpu_router_bf16(wl.seed, wr)
    b = bias_for(wl)
    bias = None if b is None else torch.tensor(b, device=dev)
    # one batch of T fresh tokens per step
    xs = torch.empty(((n_batches + n_graph) * T, Hm), dtype=torch.bfloat16, device=dev)
    synth.gpu_x_bf16(wl.seed, xs)
    d = moe.dims(T, H, I, E, k)
    if wl.H_model:
        p_down = torch.empty((Hm, H), dtype=torch.bfloat16, device=dev)
        p_up = torch.empty((H, Hm), dtype=torch.bfloat16, device=dev)
        synth.gpu_proj_bf16(wl.seed, 0, p_down)
        synth.gpu_proj_bf16(wl.seed, 1, p_up)
        ws = torch.empty(moe.moe_latent_workspace_bytes(d, Hm), dtype=torch.uint8, device=dev)
    elif args.shared:
        sh_gu = torch.empty((H, args.shared * 2 * I), dtype=torch.bfloat16, device=dev)
        sh_dn = torch.empty((args.shared * I, H), dtype=torch.bfloat16, device=dev)
        synth.gpu_proj_bf16(wl.seed, 2, sh_gu)
        synth.gpu_proj_bf16(wl.seed, 3, sh_dn)
        ws = torch.empty(moe.moe_layer_shared_workspace_bytes(d, args.shared, I), dtype=torch.uint8, device=dev)
    else:
        ws = torch.empty(moe.moe_workspace_bytes(d), dtype=torch.uint8, device=dev)
    y = torch.empty((T, Hm), dtype=torch.float32 if args.ep > 1 else torch.bfloat16, device=dev)
    ids = torch.empty((n_batches + n_graph, T, k), dtype=torch.int32, device=dev)
    wts = torch.empty((n_batches + n_graph, T, k), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    stream_peak = stream_read_GBps(moe, torch)

    def step(i):
        if args.ep > 1:
            moe.moe_layer_share(d, 0, share, xs[i * T:(i + 1) * T], wr, bias, store, y, None, ids[i], wts[i], ws)
        elif args.shared:
            moe.moe_layer_shared(d, args.shared, I, sh_gu, sh_dn, xs[i * T:(i + 1) * T], wr, bias, store, y, ids[i],
                                 wts[i], ws)
        elif wl.H_model:
            moe.moe_latent_layer(d, Hm, p_down, p_up, xs[i * T:(i + 1) * T], wr, bias, store, y, None, ids[i], wts[i],
                                 ws)
        else:
            moe.moe_layer(d, xs[i * T:(i + 1) * T], wr, bias, store, y, ids[i], wts[i], ws)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region ------------------------------------------------------------
    # the dominant kernel is timed on a sample of the timed steps (the first
    # n_prof): each event record stalls the stream's dispatch for a few
    # microseconds, which would otherwise weigh on every step
    n_prof = min(steps, PROFILED_LAUNCHES)
    moe.moe_profile_arm("gateup", n_prof)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(warmup, n_batches):
        step(i)
    end.record()
    torch.cuda.synchronize()
    gateup_ms = moe.moe_profile_read(n_prof)
    elapsed_ms = start.elapsed_time(end)
    assert len(gateup_ms) == n_prof

    ids_np = ids.cpu().numpy()
    # distinct active experts per step (of this device's share)
    distinct = np.array([len(np.unique(ids_np[i][ids_np[i] < share])) for i in range(warmup, n_batches)])

    # ---- algorithmic work ------------------------------------------------------------
    ms_per_step = elapsed_ms / steps
    mat_bytes = mxfp4_bytes if args.format == "mxfp4" else nvfp4_bytes
    expert_bytes = 2 * mat_bytes(I, H) + mat_bytes(H, I)
    # latent block: plus the two projection weights; router and x, y at the hidden width
    proj_bytes = 2 * Hm * H * 2 if wl.H_model else 0
    proj_bytes += args.shared * 3 * H * I * 2  # bf16 shared experts
    y_bytes = T * Hm * (4 if args.ep > 1 else 2)
    layer_bytes = distinct.mean() * expert_bytes + Hm * E * 2 + T * Hm * 2 + y_bytes + proj_bytes
    local_pairs = np.mean([np.count_nonzero(ids_np[i] < share) for i in range(warmup, n_batches)])
    layer_flops = (2 * T * Hm * E + 6 * local_pairs * H * I + (4 * T * Hm * H if wl.H_model else 0)
                   + 6 * T * args.shared * H * I)
    gateup_unit = 2 * mat_bytes(I, H)                # one active expert's gate+up weights
    gateup_bytes = distinct * gateup_unit + T * H * 2 + local_pairs * I * 2
    gateup_avg_ms = float(np.mean(gateup_ms))
    prof_bytes = float(np.mean(gateup_bytes[:n_prof]))  # the steps whose launches were timed
    achieved = prof_bytes / (gateup_avg_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    prefill = T >= 4096
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(wl.name, sha),
                "kernel": "gateup_kernel (grouped gate/up + SiLU*mul)",
                "algorithmic_bytes_per_launch": int(prof_bytes), "avg_launch_ms": round(gateup_avg_ms, 5),
                "timed_launches": n_prof, "stream_read_GBps": round(stream_peak, 1),
                "frac_of_stream_read": round(achieved / stream_peak, 4)}
    if prefill:
        gu_flops = 4 * local_pairs * H * I
        tf = gu_flops / (gateup_avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tf, 1), "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / FP16_MFMA_PEAK_TFLOPS, 4), "traffic": load_traffic(wl.name, sha),
                    "kernel": "gateup_kernel (grouped gate/up + SiLU*mul)",
                    "algorithmic_flops_per_launch": gu_flops, "avg_launch_ms": round(gateup_avg_ms, 5),
                    "timed_launches": n_prof}

    out = {
        "metric": METRIC,
        "value": round(T * steps / (elapsed_ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": (f"{wl.name}: latent MoE block, hidden {Hm} -> routed latent {H} (bf16 projections), "
                                if wl.H_model else f"{wl.name}: MoE layer ")
                               + f"T={T} H={H} I={I} E={E} top-{k}, {args.format.upper()} experts, bf16 activations, fresh tokens "
                               f"every step",
                   "T": T, "H": H, "I": I, "E": E, "k": k, "H_model": wl.H_model, "zipf_beta": wl.beta,
                   "seed": wl.seed, "expert_share": f"experts 0..{share - 1} of {E}" if args.ep > 1 else None,
                   "shared_experts": args.shared, "weight_format": args.format},
        "roofline": roofline,
        "layer": {"algorithmic_bytes": int(layer_bytes), "hbm_GBps": round(layer_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "frac_of_stream_read": round(layer_bytes / (ms_per_step * 1e-3) / 1e9 / stream_peak, 4),
                  "TFLOPs": round(layer_flops / (ms_per_step * 1e-3) / 1e12, 3),
                  "distinct_experts_mean": float(distinct.mean())},
        "setup_s": round(setup_s, 2),
        "kernel_source_sha": sha,
    }

    # ---- per-kernel breakdown (after the timed region; not part of the value) ----
    if not args.no_breakdown:
        reps = min(steps, 20)
        br = {}
        for name in moe.KERNELS:
            moe.moe_profile_arm(name, reps)
            for i in range(reps):
                step(warmup + i)
            torch.cuda.synchronize()
            ms = moe.moe_profile_read(reps)
            br[name] = round(float(np.mean(ms)), 5) if ms else None
        out["kernel_ms"] = br

    # ---- HIP-graph replay (after the timed region; not part of the value) ------
    # the same step captured once per batch into one graph, on batches no
    # earlier step used (so the weights are read cold again), replayed once
    if n_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n_batches, n_batches + n_graph):
                step(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        out["graph_ms_per_step"] = round(a.elapsed_time(b) / n_graph, 5)
        del graph

    if not args.no_cpu_baseline and args.ep == 1 and not args.shared and args.format == "nvfp4":
        n_tok = args.cpu_tokens or (8 if T <= 16 else 4)
        out["cpu_baseline"] = cpu_baseline(wl, n_tok, first_token=warmup * T)
    print(json.dumps(out))


def cpu_baseline(wl, n_tokens, first_token):
    """The CPU oracle, as it stands, on a bounded sample of the same
    workload: n_tokens tokens of the timed batches (generator tokens
    first_token..), one single-token layer call each.  The experts those
    tokens select (found with the oracle's own router, untimed) are
    generated and quantised beforehand; the timed call routes, dequantises
    and runs its 16 experts and combines."""
    import concurrent.futures

    import oracle
    import synth
    from synth.workloads import bias_for

    threads = min(16, os.cpu_count() or 1)
    Hm = wl.H_model or wl.H
    wr = synth.router_bf16(wl.seed, Hm, wl.E)
    bias = bias_for(wl)
    xs = [synth.x_bf16(wl.seed, 1, Hm, t0=first_token + t) for t in range(n_tokens)]
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
    total = 0.0
    for x in xs:
        t0 = time.perf_counter()
        if wl.H_model:
            oracle.latent_layer(x, cache, wl.E, wl.k, p_down, p_up, wr_bf16=wr, bias=bias, nthreads=threads)
        else:
            oracle.moe_layer(x, cache, wl.E, wl.k, wr_bf16=wr, bias=bias, nthreads=threads)
        total += time.perf_counter() - t0
    return {"value": round(n_tokens / total, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_tokens} tokens of the {wl.name} workload's timed batches, one single-token oracle layer "
                      f"call each (router, top-k, permutation, 16 experts dequantised and run in fp64, combine"
                      f"{', and the two latent projections' if wl.H_model else ''}), "
                      f"{threads} threads over the token's experts; expert weights pre-quantised, untimed",
            "seconds": round(total, 2)}


if __name__ == "__main__":
    main()
