"""Shared helpers of the GPU parity tests: device inputs built by the seeded
GPU generator and the library's own quantiser, the library called through
its C ABI, and the oracle fed the same seeded inputs generated on the CPU."""
import concurrent.futures
import os

import numpy as np
import torch

import oracle
import routed_expert_ffn_amd as moe
import synth
from synth.workloads import bias_for

DEV = torch.device("cuda:0")
MAX_ABS = 2e-2      # output tolerance: max-abs error
REL_L2 = 5e-3       # output tolerance: relative L2 error
LOGIT_ABS = 1e-4    # router logits: fp32 sums in a different order
WEIGHT_ABS = 2e-6   # softmax weights: fp32 on the GPU vs fp64


def say(msg):
    print(msg, flush=True)


def to_np(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max()), float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, what, max_abs=MAX_ABS, rel=REL_L2):
    a, r = errors(got, ref)
    say(f"  {what}: max_abs={a:.3e} rel_l2={r:.3e}")
    assert a <= max_abs and r <= rel, f"{what}: max_abs={a:.3e} rel_l2={r:.3e}"


def assert_close_bf16_out(got, ref, what, extra=None):
    """A bf16 output against the oracle's fp64 value: relative L2 within
    REL_L2, and each element within MAX_ABS or, where that is larger, half a
    bf16 unit of its magnitude (the output's own rounding) plus 4e-3 (the
    computation's error).  Half a unit exceeds MAX_ABS only from |y| = 8
    (0.031 there), which the shared experts and the latent block reach.
    extra (per element, optional) widens the allowance by a stated bound on
    an error source upstream of this output."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    unit = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
    allow = np.maximum(MAX_ABS, 0.5 * unit + 4e-3) + (0.0 if extra is None else extra)
    worst = float(np.max(np.abs(got - ref) / allow))
    a, r = errors(got, ref)
    say(f"  {what}: max_abs={a:.3e} (worst {worst:.2f} of its allowance, |y| up to {np.abs(ref).max():.2f}) "
        f"rel_l2={r:.3e}")
    assert worst <= 1.0 and r <= REL_L2, f"{what}: worst {worst:.2f}, rel_l2={r:.3e}"


def build_store(E, H, I, seed, experts=None, fmt="nvfp4"):
    """NVFP4 (or MXFP4) store on the GPU: fp32 weights from the GPU
    generator, quantised by the library (experts outside `experts` are left
    zero)."""
    store = moe.ExpertStore(E, H, I, device=DEV, fmt=fmt)
    for m in store.MATS:
        for t in store.t[m]:
            t.zero_()
    buf = {m: torch.empty(store.shape(m), dtype=torch.float32, device=DEV) for m in store.MATS}
    for e in (range(E) if experts is None else experts):
        for mi, m in enumerate(store.MATS):
            synth.gpu_expert_f32(seed, e, mi, buf[m])
            store.quantize_into(e, m, buf[m])
    torch.cuda.synchronize()
    return store


_ORACLE_EXPERTS = {}  # (seed, H, I, fmt) -> {expert: quantised triple}, shared by the test modules


class OracleExperts:
    """Experts generated and quantised on the CPU by the oracle, on demand,
    kept for the rest of the test session (the same experts serve several
    full-size tests)."""

    def __init__(self, seed, H, I, fmt="nvfp4"):
        self.seed, self.H, self.I = seed, H, I
        self.quant = oracle.mxfp4_quantize if fmt == "mxfp4" else oracle.nvfp4_quantize
        self.cache = _ORACLE_EXPERTS.setdefault((seed, H, I, fmt), {})

    def _make(self, e):
        return tuple(self.quant(synth.expert_f32(self.seed, e, m, *synth.expert_shape(m, self.H, self.I), nthreads=1))
                     for m in range(3))

    def get(self, ids):
        need = sorted(set(int(e) for e in np.ravel(ids)) - set(self.cache))
        if need:
            with concurrent.futures.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
                for e, v in zip(need, ex.map(self._make, need)):
                    self.cache[e] = v
        return {int(e): self.cache[int(e)] for e in set(np.ravel(ids))}


class Inputs:
    """Device inputs of one workload-shaped case."""

    def __init__(self, T, H, I, E, k, seed=0, t0=0, bias=None, store=None, router_std=synth.WEIGHT_STD):
        self.T, self.H, self.I, self.E, self.k, self.seed, self.t0 = T, H, I, E, k, seed, t0
        self.d = moe.dims(T, H, I, E, k)
        self.x = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        if T:
            synth.gpu_x_bf16(seed, self.x, t0=t0)
        self.wr = torch.empty((H, E), dtype=torch.bfloat16, device=DEV)
        synth.gpu_router_bf16(seed, self.wr, std=router_std)
        self.router_std = router_std
        self.bias_np = None if bias is None else np.asarray(bias, np.float32)
        self.bias = None if bias is None else torch.tensor(self.bias_np, device=DEV)
        self.store = store if store is not None else build_store(E, H, I, seed)
        self.ws = torch.empty(max(1, moe.moe_workspace_bytes(self.d)), dtype=torch.uint8, device=DEV)

    @classmethod
    def for_workload(cls, wl, t0=0, store=None):
        return cls(wl.T, wl.H, wl.I, wl.E, wl.k, seed=wl.seed, t0=t0, bias=bias_for(wl), store=store)

    def host_x(self, rows=None):
        x = synth.x_bf16(self.seed, self.T, self.H, t0=self.t0)
        return x if rows is None else x[rows]

    def host_wr(self):
        return synth.router_bf16(self.seed, self.H, self.E, std=self.router_std)

    def route(self, logits_in=None):
        T, E, k = self.T, self.E, self.k
        P = T * k
        out = dict(
            logits=torch.empty((T, E), dtype=torch.float32, device=DEV),
            ids=torch.empty((T, k), dtype=torch.int32, device=DEV),
            w=torch.empty((T, k), dtype=torch.float32, device=DEV),
            offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
            sorted_pairs=torch.empty(max(P, 1), dtype=torch.int32, device=DEV),
            pair_pos=torch.empty(max(P, 1), dtype=torch.int32, device=DEV))
        x = self.x
        if logits_in is not None:
            out["logits"].copy_(torch.as_tensor(logits_in))
            x = None
        moe.moe_route(self.d, x, self.wr, self.bias, out["logits"], out["ids"], out["w"], out["offsets"],
                      out["sorted_pairs"], out["pair_pos"], self.ws)
        torch.cuda.synchronize()
        return {n: to_np(t) for n, t in out.items()}

    def ffn(self, offsets, sorted_pairs):
        rows = torch.empty((self.T * self.k, self.H), dtype=torch.float32, device=DEV)
        moe.moe_expert_ffn(self.d, self.x, torch.as_tensor(offsets, device=DEV),
                           torch.as_tensor(sorted_pairs, device=DEV), self.store, rows, self.ws)
        torch.cuda.synchronize()
        return to_np(rows)

    def layer(self):
        y = torch.empty((self.T, self.H), dtype=torch.bfloat16, device=DEV)
        ids = torch.empty((self.T, self.k), dtype=torch.int32, device=DEV)
        w = torch.empty((self.T, self.k), dtype=torch.float32, device=DEV)
        moe.moe_layer(self.d, self.x, self.wr, self.bias, self.store, y, ids, w, self.ws)
        torch.cuda.synchronize()
        return to_np(y), to_np(ids), to_np(w)
