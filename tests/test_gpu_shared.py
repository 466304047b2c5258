"""GPU parity of the layer with shared experts (moe_layer_shared) against the
oracle's layer_with_shared: two bf16 shared experts summed with the routed
experts, at small shapes through every routing and GEMM path, and at the
full shape (H = 7168, two shared experts of I = 2048) for single-user decode
and, on sampled tokens, the prefill chunk.
Routing is the plain layer's (ids bit-exact); y within the layer's
tolerances of the oracle's fp64 sum, an element of |y| >= 8 also within half
a bf16 unit of its magnitude plus 4e-3 (the output's own rounding to bf16
alone reaches half a unit, more than 2e-2 there)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    import routed_expert_ffn_amd as moe
    import synth
    from synth.workloads import WORKLOADS
    from tests.gpu_helpers import DEV, Inputs, OracleExperts, assert_close_bf16_out, build_store, say, to_np

COUNT = 2  # shared experts


def shared_weights(seed, H, I):
    gu = torch.empty((H, COUNT * 2 * I), dtype=torch.bfloat16, device=DEV)
    dn = torch.empty((COUNT * I, H), dtype=torch.bfloat16, device=DEV)
    synth.gpu_proj_bf16(seed, 2, gu)
    synth.gpu_proj_bf16(seed, 3, dn)
    return gu, dn, synth.proj_bf16(seed, 2, H, COUNT * 2 * I), synth.proj_bf16(seed, 3, COUNT * I, H)


def run_shared(inp, I_s, gu, dn):
    ws = torch.empty(moe.moe_layer_shared_workspace_bytes(inp.d, COUNT, I_s), dtype=torch.uint8, device=DEV)
    y = torch.empty((inp.T, inp.H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((inp.T, inp.k), dtype=torch.int32, device=DEV)
    w = torch.empty((inp.T, inp.k), dtype=torch.float32, device=DEV)
    moe.moe_layer_shared(inp.d, COUNT, I_s, gu, dn, inp.x, inp.wr, inp.bias, inp.store, y, ids, w, ws)
    torch.cuda.synchronize()
    return to_np(y), to_np(ids), to_np(w)


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (70, 48, 4), (1100, 32, 8)])
def test_layer_with_shared_small(T, E, k):
    say(f"shared T={T} E={E} k={k}")
    inp = Inputs(T, 512, 256, E, k, seed=41, router_std=0.1)
    gu, dn, gu_h, dn_h = shared_weights(41, 512, 256)
    y, ids, w = run_shared(inp, 256, gu, dn)
    r = inp.route()
    np.testing.assert_array_equal(ids, r["ids"])
    ref = oracle.layer_with_shared(inp.host_x(), OracleExperts(41, 512, 256).get(r["ids"]), E, k, gu_h, dn_h, COUNT,
                                   256, logits_in=r["logits"], nthreads=16)
    say(f"  shared part rms {np.sqrt(np.mean(ref['y_shared'] ** 2)):.3e}, routed {np.sqrt(np.mean(ref['y_routed'] ** 2)):.3e}")
    assert_close_bf16_out(y, ref["y"], "y")


@pytest.fixture(scope="module")
def full_store():
    wl = WORKLOADS["decode_1"]
    say("building the full NVFP4 store on the GPU (896 experts)")
    return build_store(wl.E, wl.H, wl.I, wl.seed)


@pytest.mark.parametrize("name", ["decode_1", "prefill_8192"])
def test_layer_with_shared_full_size(name, full_store):
    """The full shape with two shared experts of I = 2048: every token at
    single-user decode; at the prefill chunk the routing of every token and
    the output of at least 32 sampled tokens (tile edges of the most loaded
    expert)."""
    from tests.test_gpu_full import sample_tokens

    wl = WORKLOADS[name]
    say(f"shared experts, full-size {name}: T={wl.T}")
    inp = Inputs.for_workload(wl, store=full_store)
    gu, dn, gu_h, dn_h = shared_weights(wl.seed, wl.H, wl.I)
    y, ids, w = run_shared(inp, wl.I, gu, dn)
    r = inp.route()
    np.testing.assert_array_equal(ids, r["ids"])
    assert np.all(np.isfinite(y))
    sample = sample_tokens(wl.T, r, wl.k)
    ref = oracle.layer_with_shared(inp.host_x(sample), OracleExperts(wl.seed, wl.H, wl.I).get(r["ids"][sample]),
                                   wl.E, wl.k, gu_h, dn_h, COUNT, wl.I, logits_in=r["logits"][sample], nthreads=16)
    assert_close_bf16_out(y[sample], ref["y"], f"{name} y of {len(sample)} tokens with shared experts")
