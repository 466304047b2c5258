"""GPU parity of the MXFP4 weight format: the library's quantiser against
the oracle's bit for bit (codes and e8m0 scales; gs the stated power of
two), and the layer on an MXFP4 store against the oracle's layer on the
oracle's MXFP4 experts, through moe_expert_ffn (rows) and moe_layer (y), at
small shapes (small-batch GEMMs below 1024 tokens, the large-tile GEMMs from
there) and at every full-size workload (single-user and 64-session decode,
speculative verify, the 8192-token prefill chunk), on sampled tokens that the
oracle computes."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    import routed_expert_ffn_amd as moe
    import synth
    from synth.workloads import WORKLOADS
    from tests.gpu_helpers import DEV, WEIGHT_ABS, Inputs, OracleExperts, assert_close, build_store, say, to_np
    from tests.test_gpu_full import check_sampled, sample_tokens


def mx_cases():
    rng = np.random.default_rng(5)
    yield "normal", synth.expert_f32(0, 3, 1, 64, 512)
    w = synth.expert_f32(0, 4, 2, 32, 256)
    w[3] = 0.0  # zero rows give zero blocks
    w[5, :32] = 0.0
    yield "zeros", w
    yield "wide-range", (rng.standard_normal((16, 256)) * np.exp(rng.uniform(-30, 30, (16, 1)))).astype(np.float32)
    t = np.zeros((4, 64), np.float32)  # ties between e2m1 points after scaling
    t[:, 0] = 4.0
    t[:, 1:9] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -1.25]
    yield "ties", t


@pytest.mark.parametrize("case", list(range(4)))
def test_mxfp4_quantize_bit_exact(case):
    name, w = list(mx_cases())[case]
    say(f"mxfp4 quantise: {name} {w.shape}")
    N, K = w.shape
    wd = torch.tensor(w, device=DEV)
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=DEV)
    sf = torch.empty((N, K // 32), dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    ws = torch.empty(256, dtype=torch.uint8, device=DEV)
    moe.moe_quantize_mxfp4(wd, q, sf, gs, ws)
    torch.cuda.synchronize()
    ref = oracle.mxfp4_quantize(w)
    np.testing.assert_array_equal(sf.cpu().numpy(), ref.sf)
    np.testing.assert_array_equal(q.cpu().numpy(), ref.q)
    amax = float(np.abs(w).max())
    smax = min(max(int(np.floor(np.log2(amax))) - 2 + 127, 0), 254) if amax > 0 else 0
    assert float(gs.item()) == 2.0 ** (smax - 135)


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (70, 48, 4), (1100, 32, 8), (2600, 16, 6)])
def test_mxfp4_layer(T, E, k):
    say(f"mxfp4 layer T={T} E={E} k={k}")
    store = build_store(E, 512, 256, 51, fmt="mxfp4")
    inp = Inputs(T, 512, 256, E, k, seed=51, store=store, router_std=0.1)
    r = inp.route()
    ox = OracleExperts(51, 512, 256, fmt="mxfp4")
    ref = oracle.moe_layer(inp.host_x(), ox.get(r["ids"]), E, k, logits_in=r["logits"], want_rows=True, nthreads=16)
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    assert_close(rows, ref["rows"], "rows")
    y, ids, _ = inp.layer()
    np.testing.assert_array_equal(ids, ref["ids"])
    assert_close(y, ref["y"], "y")


@pytest.fixture(scope="module")
def full_store():
    wl = WORKLOADS["decode_1"]
    say("building the full MXFP4 store on the GPU (896 experts)")
    return build_store(wl.E, wl.H, wl.I, wl.seed, fmt="mxfp4")


@pytest.mark.parametrize("name", ["decode_1", "decode_64", "verify_256", "prefill_8192"])
def test_mxfp4_layer_full_size(name, full_store):
    """Every full-size workload on the MXFP4 store: routing bit-exact (the
    plain layer's), rows and y of at least 32 sampled tokens (tile and pass
    edges of the most loaded expert) against the oracle's MXFP4 layer."""
    wl = WORKLOADS[name]
    say(f"mxfp4 full-size {name}: T={wl.T}")
    inp = Inputs.for_workload(wl, store=full_store)
    r = inp.route()
    sample = sample_tokens(wl.T, r, wl.k)
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    y, ids, w = inp.layer()
    np.testing.assert_array_equal(ids, r["ids"])
    assert np.all(np.isfinite(y))
    check_sampled(name, wl, inp, r, rows, y, sample, OracleExperts(wl.seed, wl.H, wl.I, fmt="mxfp4"), " mxfp4")
