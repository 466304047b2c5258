"""GPU parity at the full layer size (H=7168, I=2048, E=896, k=16, all 896
NVFP4 experts resident, 22.2 GB), in the launch configuration the benchmark
times: single-user decode (T=1), 64-session decode (T=64), speculative
verify (T=256) and a prefill chunk (T=8192).  Routing and the permutation
are checked for every token.  Rows and outputs are checked on at least 32
sampled tokens per workload, chosen so that every token tile (prefill) or
16-token pass (decode sizes) of the most loaded expert has its first and
last record sampled, plus the first, middle and last token and seeded random
ones; the oracle computes them (it regenerates and quantises those tokens'
experts on the CPU).  At the prefill size every token's output is also
checked against the same tokens run in chunks of 512, which take the
small-batch kernels.  How many tokens would select a different top-16 set
under the oracle's own logits is reported, not asserted (a last-bit logit
difference can flip a near tie)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    import routed_expert_ffn_amd as moe
    from synth.workloads import WORKLOADS
    from tests.gpu_helpers import (DEV, WEIGHT_ABS, Inputs, OracleExperts, assert_close, build_store, say, to_np)
    from tests.test_gpu_parity import check_route

FULL = ["decode_1", "decode_64", "verify_256", "prefill_8192"]
BIG_TILE = 224     # token tile of the large-batch GEMMs
SMALL_PASS = 16    # token pass of the small-batch GEMMs
BIG_MIN_T = 1024   # batches from this size take the large-batch GEMMs
N_SAMPLE = 32


@pytest.fixture(scope="module")
def store():
    wl = WORKLOADS["decode_1"]
    say("building the full NVFP4 store on the GPU (896 experts)")
    return build_store(wl.E, wl.H, wl.I, wl.seed)


@pytest.fixture(scope="module")
def oracle_experts():
    wl = WORKLOADS["decode_1"]
    return OracleExperts(wl.seed, wl.H, wl.I)


def sample_tokens(T, r, k, n=N_SAMPLE, seed=0):
    """Tokens whose records sit at the edges of the most loaded expert's
    token tiles (an expert's n records are split evenly over ceil(n / 224)
    tiles) or 16-token passes, the first, middle and last token, then seeded
    random tokens up to n (all tokens when T <= n)."""
    if T <= n:
        return list(range(T))
    counts = np.diff(r["offsets"])
    hot = int(np.argmax(counts))
    c, base = int(counts[hot]), int(r["offsets"][hot])
    picks = {0, T // 2, T - 1}
    if T >= BIG_MIN_T:
        tiles = -(-c // BIG_TILE)
        ts = -(-c // tiles)
        edges = [(m * ts, min((m + 1) * ts, c) - 1) for m in range(tiles)]
        # and the last 32-token fragment of each tile
        edges += [(min(lo + 32 * ((hi - lo) // 32), hi), hi) for lo, hi in edges]
    else:
        edges = [(p, min(p + SMALL_PASS, c) - 1) for p in range(0, c, SMALL_PASS)]
    for lo, hi in edges:
        for q in (lo, hi):
            picks.add(int(r["sorted_pairs"][base + q]) // k)
    rng = np.random.default_rng(seed)
    while len(picks) < n:
        picks.add(int(rng.integers(0, T)))
    return sorted(picks)


def check_sampled(name, wl, inp, r, rows, y, sample, ox, fmt_note=""):
    ex = ox.get(r["ids"][sample])
    ref = oracle.moe_layer(inp.host_x(sample), ex, wl.E, wl.k, logits_in=r["logits"][sample], nthreads=16,
                           want_rows=True)
    np.testing.assert_array_equal(ref["ids"], r["ids"][sample])
    assert np.abs(ref["w"] - r["w"][sample]).max() <= WEIGHT_ABS
    got_rows = np.stack([rows[r["pair_pos"][t * wl.k + j]] for t in sample for j in range(wl.k)])
    ref_rows = np.stack([ref["rows"][ref["pair_pos"][s * wl.k + j]] for s in range(len(sample)) for j in range(wl.k)])
    assert_close(got_rows, ref_rows, f"{name}{fmt_note} rows of {len(sample)} tokens")
    assert_close(y[sample], ref["y"], f"{name}{fmt_note} y of {len(sample)} tokens")


def report_flips(name, inp, r, rows):
    """Tokens whose selected set differs between the GPU's logits and the
    oracle's own (its fp64 sums rounded to fp32), with the smallest gap
    between the 16th and 17th oracle logit among the sampled tokens."""
    ref_logits = oracle.router_logits(inp.host_x(rows), inp.host_wr(), inp.bias_np)
    ids_own, _ = oracle.topk_softmax(ref_logits, inp.k)
    differ = sum(set(a) != set(b) for a, b in zip(ids_own, r["ids"][rows]))
    top = -np.sort(-ref_logits, axis=1)
    gap = float((top[:, inp.k - 1] - top[:, inp.k]).min())
    dl = float(np.abs(ref_logits - r["logits"][rows]).max())
    say(f"  {name}: {differ} of {len(rows)} tokens select a different set under the oracle's own logits "
        f"(max logit difference {dl:.2e}, smallest 16th-17th gap {gap:.2e})")
    return differ


@pytest.mark.parametrize("name", FULL)
def test_full_size(name, store, oracle_experts):
    wl = WORKLOADS[name]
    say(f"full-size {name}: T={wl.T}")
    inp = Inputs.for_workload(wl, store=store)
    r = inp.route()
    sample = sample_tokens(wl.T, r, wl.k)
    check_route(inp, r, rows=np.array(sample))
    counts = np.diff(r["offsets"])
    say(f"  distinct experts {np.count_nonzero(counts)}, max count {counts.max()}, "
        f"max/mean {counts.max() / counts.mean():.2f}; {len(sample)} sampled tokens")
    assert counts.sum() == wl.P
    flip_rows = np.arange(min(wl.T, 512))
    report_flips(name, inp, r, flip_rows)

    # rows of the sampled tokens from moe_expert_ffn, and y from moe_layer
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    y, ids, w = inp.layer()
    np.testing.assert_array_equal(ids, r["ids"])
    np.testing.assert_array_equal(w, r["w"])
    assert np.all(np.isfinite(y))
    check_sampled(name, wl, inp, r, rows, y, sample, oracle_experts)

    if wl.T >= BIG_MIN_T:
        # every token's output against the same tokens in chunks of 512
        # (small-batch kernels), where both routings agree
        chunk = 512
        dch = moe.dims(chunk, wl.H, wl.I, wl.E, wl.k)
        ws = torch.empty(moe.moe_workspace_bytes(dch), dtype=torch.uint8, device=DEV)
        yc = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=DEV)
        idc = torch.empty((wl.T, wl.k), dtype=torch.int32, device=DEV)
        for c0 in range(0, wl.T, chunk):
            moe.moe_layer(dch, inp.x[c0:c0 + chunk], inp.wr, inp.bias, inp.store, yc[c0:c0 + chunk],
                          idc[c0:c0 + chunk], None, ws)
        torch.cuda.synchronize()
        yc, idc = to_np(yc), to_np(idc)
        same = np.all(idc == ids, axis=1)
        say(f"  chunked routing: {int((~same).sum())} of {wl.T} tokens select other experts")
        assert (~same).sum() <= wl.T // 1000
        assert_close(y[same], yc[same], f"{name} y of {int(same.sum())} tokens vs chunks of {chunk}")
