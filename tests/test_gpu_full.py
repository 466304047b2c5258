"""GPU parity at the full layer size (H=7168, I=2048, E=896, k=16, all 896
NVFP4 experts resident, 22.2 GB), in the launch configuration the benchmark
times: single-user decode (T=1), 64-session decode (T=64), speculative
verify (T=256) and a prefill chunk (T=8192).  Routing and the permutation
are checked for every token; outputs on sampled tokens the oracle computes
one by one (it regenerates and quantises those tokens' experts on the
CPU); properties that hold at any size are checked everywhere."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    from synth.workloads import WORKLOADS
    from tests.gpu_helpers import (WEIGHT_ABS, Inputs, OracleExperts, assert_close, build_store, say)
    from tests.test_gpu_parity import check_route

FULL = ["decode_1", "decode_64", "verify_256", "prefill_8192"]


@pytest.fixture(scope="module")
def store():
    wl = WORKLOADS["decode_1"]
    say("building the full NVFP4 store on the GPU (896 experts)")
    return build_store(wl.E, wl.H, wl.I, wl.seed)


@pytest.fixture(scope="module")
def oracle_experts():
    wl = WORKLOADS["decode_1"]
    return OracleExperts(wl.seed, wl.H, wl.I)


def _sample_tokens(T, r, k):
    counts = np.diff(r["offsets"])
    hot = int(np.argmax(counts))
    last_of_hot = int(r["sorted_pairs"][r["offsets"][hot + 1] - 1]) // k
    return sorted(set([0, T // 2, T - 1, last_of_hot]))


@pytest.mark.parametrize("name", FULL)
def test_full_size(name, store, oracle_experts):
    wl = WORKLOADS[name]
    say(f"full-size {name}: T={wl.T}")
    inp = Inputs.for_workload(wl, store=store)
    r = inp.route()
    sample = _sample_tokens(wl.T, r, wl.k)
    check_route(inp, r, rows=np.array(sample))
    counts = np.diff(r["offsets"])
    say(f"  distinct experts {np.count_nonzero(counts)}, max count {counts.max()}, "
        f"max/mean {counts.max() / counts.mean():.2f}")
    assert counts.sum() == wl.P

    # rows of the sampled tokens from moe_expert_ffn, and y from moe_layer
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    y, ids, w = inp.layer()
    np.testing.assert_array_equal(ids, r["ids"])
    np.testing.assert_array_equal(w, r["w"])
    assert np.all(np.isfinite(y))
    ex = oracle_experts.get(r["ids"][sample])
    ref = oracle.moe_layer(inp.host_x(sample), ex, wl.E, wl.k, logits_in=r["logits"][sample], nthreads=16,
                           want_rows=True)
    np.testing.assert_array_equal(ref["ids"], r["ids"][sample])
    assert np.abs(ref["w"] - r["w"][sample]).max() <= WEIGHT_ABS
    got_rows = np.stack([rows[r["pair_pos"][t * wl.k + j]] for t in sample for j in range(wl.k)])
    ref_rows = np.stack([ref["rows"][ref["pair_pos"][s * wl.k + j]] for s in range(len(sample)) for j in range(wl.k)])
    assert_close(got_rows, ref_rows, f"{name} rows of tokens {sample}")
    assert_close(y[sample], ref["y"], f"{name} y of tokens {sample}")
