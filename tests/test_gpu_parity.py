"""GPU parity at sizes the oracle finishes in seconds: every stage of the HIP
path, called through the C ABI, against the CPU oracle on the same seeded
inputs.  Integer results (codes, ids, offsets, permutation) must match bit
for bit; floating point within the stated tolerances.  Routing is evaluated
by the oracle on the GPU's fp32 logits, so a last-bit difference in a logit
cannot flip a selection; the logits themselves are compared separately."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    import routed_expert_ffn_amd as moe
    import synth
    from synth.workloads import WORKLOADS
    from tests.gpu_helpers import (DEV, LOGIT_ABS, WEIGHT_ABS, Inputs, OracleExperts, assert_close, build_store,
                                   say)


def check_route(inp, r, rows=None):
    """GPU routing vs the oracle on the GPU's logits (bit-exact ids and
    permutation); GPU logits vs the oracle's own logits (tolerance)."""
    ids, w = oracle.topk_softmax(r["logits"], inp.k)
    np.testing.assert_array_equal(r["ids"], ids)
    assert np.abs(r["w"] - w).max() <= WEIGHT_ABS
    # each fp32 weight carries a rounding of about 2^-24 of itself and the
    # shared denominator one per doubling of k: 1e-6 up to k = 16, growing
    # in proportion beyond
    assert np.abs(r["w"].astype(np.float64).sum(axis=1) - 1).max() <= 1e-6 * max(1.0, inp.k / 16)
    offsets, sp, pp = oracle.permute(r["ids"], inp.E)
    np.testing.assert_array_equal(r["offsets"], offsets)
    np.testing.assert_array_equal(r["sorted_pairs"][:inp.T * inp.k], sp)
    np.testing.assert_array_equal(r["pair_pos"][:inp.T * inp.k], pp)
    if rows is not None:
        ref = oracle.router_logits(inp.host_x(rows), inp.host_wr(), inp.bias_np)
        assert np.abs(r["logits"][rows] - ref).max() <= LOGIT_ABS
    return ids, w


# ---- seeded generator and quantiser ---------------------------------------------

def test_gpu_generator_matches_cpu():
    say("generator: GPU vs CPU bits")
    x = torch.empty((37, 512), dtype=torch.bfloat16, device=DEV)
    synth.gpu_x_bf16(3, x, t0=5)
    np.testing.assert_array_equal(x.view(torch.int16).cpu().numpy().view(np.uint16), synth.x_bf16(3, 37, 512, t0=5))
    wr = torch.empty((512, 896), dtype=torch.bfloat16, device=DEV)
    synth.gpu_router_bf16(3, wr)
    np.testing.assert_array_equal(wr.view(torch.int16).cpu().numpy().view(np.uint16), synth.router_bf16(3, 512, 896))
    w = torch.empty((256, 512), dtype=torch.float32, device=DEV)
    synth.gpu_expert_f32(3, 11, 2, w)
    np.testing.assert_array_equal(w.cpu().numpy(), synth.expert_f32(3, 11, 2, 256, 512))


def _quantize_gpu(w):
    N, K = w.shape
    wt = torch.as_tensor(w, device=DEV)
    q = torch.empty((N, K // 2), dtype=torch.uint8, device=DEV)
    sf = torch.empty((N, K // 16), dtype=torch.uint8, device=DEV)
    gs = torch.empty(4, dtype=torch.float32, device=DEV)
    ws = torch.empty(moe.moe_quantize_workspace_bytes(), dtype=torch.uint8, device=DEV)
    moe.moe_quantize_nvfp4(wt, q, sf, gs, ws)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy(), gs.cpu().numpy()[0]


def _quant_cases():
    rng = np.random.default_rng(11)
    yield "normal", synth.expert_f32(0, 1, 0, 64, 512)
    yield "normal-down", synth.expert_f32(0, 2, 2, 512, 256)
    w = synth.expert_f32(0, 3, 1, 48, 256)
    w[5, 16:32] = 0.0                               # an all-zero block
    w[7, :] *= 1e-4                                 # rows whose scales are e4m3 subnormals
    w[9, 3] = 0.9                                   # one large outlier sets gs
    yield "edges", w
    yield "zeros", np.zeros((4, 64), np.float32)
    yield "tiny-values", (rng.normal(size=(8, 64)) * 1e-30).astype(np.float32)
    g = rng.integers(0, 8, size=(16, 64)).astype(np.float64)
    g = np.choose(g.astype(int), [0, .5, 1, 1.5, 2, 3, 4, 6]) * np.where(rng.random((16, 64)) < .5, -1, 1)
    g[:, ::16] = 6.0
    yield "grid", (g * 0.25).astype(np.float32)
    # values exactly at e2m1 midpoints of their block scale
    m = np.tile(np.array([6, .25, .75, 1.25, 1.75, 2.5, 3.5, 5, -.25, -.75, -1.25, -1.75, -2.5, -3.5, -5, 0.]), (4, 2))
    yield "midpoints", m.astype(np.float32)


def test_quantize_bit_exact():
    for name, w in _quant_cases():
        say(f"quantize {name} {w.shape}")
        q, sf, gs = _quantize_gpu(w)
        ref = oracle.nvfp4_quantize(w)
        assert gs == ref.gs, name
        np.testing.assert_array_equal(sf, ref.sf, err_msg=name)
        np.testing.assert_array_equal(q, ref.q, err_msg=name)


def test_quantize_full_size_matrix_bit_exact():
    say("quantize one 2048 x 7168 gate matrix")
    w = synth.expert_f32(0, 123, 0, 2048, 7168)
    q, sf, gs = _quantize_gpu(w)
    ref = oracle.nvfp4_quantize(w)
    assert gs == ref.gs
    np.testing.assert_array_equal(sf, ref.sf)
    np.testing.assert_array_equal(q, ref.q)


# ---- the tiny workload (T=8, H=512, I=256, E=896, k=16) -------------------------

@pytest.fixture(scope="module")
def tiny():
    wl = WORKLOADS["tiny"]
    say(f"tiny workload {wl}")
    inp = Inputs.for_workload(wl)
    return wl, inp, OracleExperts(wl.seed, wl.H, wl.I)


def test_tiny_route(tiny):
    wl, inp, _ = tiny
    r = inp.route()
    check_route(inp, r, rows=np.arange(wl.T))


def test_tiny_expert_ffn_and_layer(tiny):
    wl, inp, ox = tiny
    r = inp.route()
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    ref = oracle.moe_layer(inp.host_x(), ox.get(r["ids"]), wl.E, wl.k, logits_in=r["logits"], want_rows=True)
    assert_close(rows, ref["rows"], "rows")
    y, ids, w = inp.layer()
    np.testing.assert_array_equal(ids, ref["ids"])
    assert np.abs(w - ref["w"]).max() <= WEIGHT_ABS
    assert_close(y, ref["y"], "y")
    # the oracle's own routing (its fp64 logits) picks the same experts here
    own = oracle.moe_layer(inp.host_x(), ox.get(r["ids"]), wl.E, wl.k, wr_bf16=inp.host_wr())
    np.testing.assert_array_equal(own["ids"], ids)


def test_determinism(tiny):
    _, inp, _ = tiny
    y1, i1, w1 = inp.layer()
    y2, i2, w2 = inp.layer()
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(i1, i2)
    np.testing.assert_array_equal(w1, w2)


# ---- ragged and skewed shapes, edge cases ------------------------------------------

SMALL = dict(H=512, I=256)


@pytest.mark.parametrize("T,E,k,beta", [(1, 64, 8, None), (1, 40, 6, 0.5), (1, 8, 8, None), (1, 896, 1, None),
                                        (3, 32, 16, None), (2, 8, 8, None), (8, 8, 8, 1.0),
                                        (17, 64, 8, 0.5), (65, 32, 16, 0.8),
                                        (130, 16, 16, None), (200, 40, 4, 1.0), (33, 8, 8, None), (70, 48, 1, 0.3),
                                        (1100, 32, 8, 0.5), (2048, 16, 4, None), (1500, 64, 16, 1.0),
                                        (1024, 200, 2, 1.2)])
def test_ragged_layer(T, E, k, beta):
    """Token counts that are not multiples of 16 or 64, experts with more
    than 64 tokens (several passes), every expert selected (k = E), k = 1,
    single tokens (whose permutation ranks the selected ids directly) with E
    not a multiple of 64, k = E and k = 1,
    up to 8 tokens with every token on every expert,
    and batches of 1024+ tokens (the 224-token tile kernels) with experts
    holding several ragged 224-token tiles, or only a handful of tokens
    (tiles with a single 32-token fragment)."""
    say(f"ragged T={T} E={E} k={k} beta={beta}")
    bias = None if beta is None else synth.zipf_bias(9, E, beta)
    inp = Inputs(T, SMALL["H"], SMALL["I"], E, k, seed=9, bias=bias, router_std=0.1)
    r = inp.route()
    check_route(inp, r, rows=np.arange(min(T, 8)))
    counts = np.diff(r["offsets"])
    say(f"  counts: max={counts.max()} active={np.count_nonzero(counts)}")
    ox = OracleExperts(9, SMALL["H"], SMALL["I"])
    ref = oracle.moe_layer(inp.host_x(), ox.get(r["ids"]), E, k, logits_in=r["logits"], want_rows=True, nthreads=16)
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    assert_close(rows, ref["rows"], "rows")
    y, ids, _ = inp.layer()
    assert_close(y, ref["y"], "y")


@pytest.mark.parametrize("T,H,E", [(1100, 512, 200), (2300, 1024, 456), (1030, 7168, 896), (1024, 256, 8),
                                   (1279, 8448, 1024), (4096, 512, 224)])
def test_tiled_router_every_token(T, H, E):
    """From 1024 tokens the router is the LDS-tiled GEMM (256-token x
    224-column tiles over K slabs): every token's logits against the
    oracle's, with a ragged last token tile (1100 = 4 x 256 + 76; 1279),
    column tiles that are ragged or nearly empty (200 < 224; 456 = 2 x 224 +
    8; 8 experts; 1024 = 4 x 224 + 128), exactly one column tile (224), K3's
    width with K slabs of unequal length (1030 tokens: twelve slabs of nine
    64-k chunks and one of four), the smallest K of four chunks (256) and
    the largest hidden width the boundary tests (8448)."""
    say(f"tiled router T={T} H={H} E={E}")
    inp = Inputs(T, H, 256, E, 8, seed=21, store="unused")
    r = inp.route()
    ref = oracle.router_logits(inp.host_x(), inp.host_wr(), None)
    err = np.abs(r["logits"] - ref)
    say(f"  max |logit - oracle| = {err.max():.3e}")
    assert err.max() <= LOGIT_ABS
    check_route(inp, r)


@pytest.mark.parametrize("T", [1, 3, 70, 1030])
def test_largest_expert_count_and_k(T):
    """The largest shapes the routing takes: E = 1024 experts and k = 64
    (16 keys per lane in the top-k; a token's 64 records; more than 64
    top-k candidates send some tokens through the fallback selection), in
    the single-launch routing (T = 1, whose permutation ranks the selected
    ids directly, and T = 3), the single-block permutation
    (T = 70) and the multi-block permutation with the large-tile GEMMs
    (T = 1030); outputs checked on sampled tokens."""
    E, k, H, I = 1024, 64, 512, 256
    say(f"largest E={E} k={k} T={T}")
    inp = Inputs(T, H, I, E, k, seed=14, store=build_store(E, H, I, 14), router_std=0.1)
    r = inp.route()
    sample = np.unique(np.array([0, T // 2, T - 1]))
    check_route(inp, r, rows=sample)
    assert np.diff(r["offsets"]).sum() == T * k
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    y, ids, _ = inp.layer()
    np.testing.assert_array_equal(ids, r["ids"])
    ox = OracleExperts(14, H, I)
    ref = oracle.moe_layer(inp.host_x(sample), ox.get(r["ids"][sample]), E, k, logits_in=r["logits"][sample],
                           want_rows=True, nthreads=16)
    got_rows = np.stack([rows[r["pair_pos"][t * k + j]] for t in sample for j in range(k)])
    ref_rows = np.stack([ref["rows"][ref["pair_pos"][i * k + j]] for i in range(len(sample)) for j in range(k)])
    assert_close(got_rows, ref_rows, "rows")
    assert_close(y[sample], ref["y"], "y")


@pytest.mark.parametrize("I,T", [(768, 1), (1280, 16), (2048, 7)])
def test_small_batch_chunk_counts(I, T):
    """Small batches (whole-line code loads, staged scales) over odd and even
    numbers of 256-k chunks: K = I = 768, 1280 and 2048 are 3, 5 and 8
    chunks for the down GEMM, split two ways for gate/up at H = 512."""
    say(f"chunk counts I={I} T={T}")
    H, E, k = 512, 16, 4
    store = build_store(E, H, I, 13)
    inp = Inputs(T, H, I, E, k, seed=13, store=store, router_std=0.1)
    r = inp.route()
    ox = OracleExperts(13, H, I)
    ref = oracle.moe_layer(inp.host_x(), ox.get(r["ids"]), E, k, logits_in=r["logits"], want_rows=True, nthreads=16)
    assert_close(inp.ffn(r["offsets"], r["sorted_pairs"]), ref["rows"], "rows")
    y, ids, _ = inp.layer()
    np.testing.assert_array_equal(ids, ref["ids"])
    assert_close(y, ref["y"], "y")


@pytest.mark.parametrize("H,I,fmt,T", [(8448, 256, "nvfp4", 8), (512, 4352, "nvfp4", 300), (512, 4352, "nvfp4", 12),
                                       (512, 8448, "mxfp4", 40), (512, 8448, "mxfp4", 6)])
def test_wide_k_scales_from_memory(H, I, fmt, T):
    """K beyond what a block can stage of its block scales in LDS (gate/up K
    over 8192, down K over 4096 for NVFP4, twice that for MXFP4): those GEMMs
    read the scales from memory in groups of four chunks, the others stage
    them; experts with one and with several 16-token passes."""
    say(f"wide K H={H} I={I} {fmt} T={T}")
    E, k = 8, 4
    store = build_store(E, H, I, 12, fmt=fmt)
    inp = Inputs(T, H, I, E, k, seed=12, store=store, router_std=0.1)
    r = inp.route()
    ox = OracleExperts(12, H, I, fmt=fmt)
    ref = oracle.moe_layer(inp.host_x(), ox.get(r["ids"]), E, k, logits_in=r["logits"], want_rows=True, nthreads=16)
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    assert_close(rows, ref["rows"], "rows")
    y, ids, _ = inp.layer()
    np.testing.assert_array_equal(ids, ref["ids"])
    assert_close(y, ref["y"], "y")


@pytest.mark.parametrize("T,H,I,E,k", [(1100, 2048, 2048, 16, 2), (1030, 3072, 1280, 8, 2)])
def test_large_tiles_many_spans(T, H, I, E, k):
    """The large-tile GEMMs at a K of many four-chunk spans (2048: eight
    spans for gate/up and for down; 3072 and 1280: twelve and five), so the
    steady-state loop of the LDS DMA pipeline runs many times in both GEMMs:
    every token's rows and output against the oracle."""
    say(f"many spans T={T} H={H} I={I} E={E} k={k}")
    store = build_store(E, H, I, 15)
    inp = Inputs(T, H, I, E, k, seed=15, store=store, router_std=0.1, bias=synth.zipf_bias(15, E, 0.6))
    r = inp.route()
    check_route(inp, r, rows=np.arange(8))
    counts = np.diff(r["offsets"])
    say(f"  counts: max={counts.max()} min={counts.min()}")
    ox = OracleExperts(15, H, I)
    ref = oracle.moe_layer(inp.host_x(), ox.get(r["ids"]), E, k, logits_in=r["logits"], want_rows=True, nthreads=16)
    assert_close(inp.ffn(r["offsets"], r["sorted_pairs"]), ref["rows"], "rows")
    y, ids, _ = inp.layer()
    np.testing.assert_array_equal(ids, ref["ids"])
    assert_close(y, ref["y"], "y")


def test_maximum_token_count():
    """The largest batch the boundary accepts, T = 65535 (the combines launch
    one row of blocks per token), at a small H and I with Zipf-skewed routing
    (the hottest expert takes several hundred 224-token tiles' worth of
    records): routing and the permutation checked for every token, the rows
    and y of sampled tokens against the oracle, among them the first and
    last records of the hottest expert."""
    from tests.test_gpu_full import sample_tokens
    T, H, I, E, k = 65535, 512, 256, 896, 16
    say(f"maximum T={T} H={H} I={I} E={E} k={k}")
    inp = Inputs(T, H, I, E, k, seed=23, bias=synth.zipf_bias(23, E, 1.0), router_std=0.1)
    r = inp.route()
    sample = sample_tokens(T, r, k, n=24, seed=23)
    check_route(inp, r, rows=np.array(sample))
    counts = np.diff(r["offsets"])
    say(f"  max count {counts.max()}, active {np.count_nonzero(counts)}; {len(sample)} sampled tokens")
    assert counts.sum() == T * k
    rows = inp.ffn(r["offsets"], r["sorted_pairs"])
    y, ids, _ = inp.layer()
    np.testing.assert_array_equal(ids, r["ids"])
    assert np.all(np.isfinite(y))
    ref = oracle.moe_layer(inp.host_x(sample), OracleExperts(23, H, I).get(r["ids"][sample]), E, k,
                           logits_in=r["logits"][sample], want_rows=True, nthreads=16)
    got_rows = np.stack([rows[r["pair_pos"][t * k + j]] for t in sample for j in range(k)])
    ref_rows = np.stack([ref["rows"][ref["pair_pos"][i * k + j]] for i in range(len(sample)) for j in range(k)])
    assert_close(got_rows, ref_rows, f"rows of {len(sample)} tokens")
    assert_close(y[sample], ref["y"], f"y of {len(sample)} tokens")


@pytest.mark.parametrize("T", [1, 6, 40, 100])
def test_route_ties_logits_in(T):
    """Constructed fp32 logits with exact ties (all equal, +-0, duplicated
    values, more tied maxima than a wavefront has lanes): the selection must
    follow (logit desc, index asc) bit-exactly.  T = 1 and 6 run the
    single-launch routing (T = 1: all 896 logits equal, the fallback
    selection and the single-token permutation), T = 40 and 100 the
    one-block-per-token and the four-tokens-per-block top-k kernels."""
    E, k = 896, 16
    say(f"ties T={T}")
    rng = np.random.default_rng(2)
    L = rng.normal(0, 1.7, size=(T, E)).astype(np.float32)
    L[0] = 0.0
    if T > 1:
        L[1, ::2] = -0.0
        L[1, 1::2] = 0.0
        L[2] = np.round(L[2])
        L[3, 500:530] = 7.0
        L[4] = -3.0
        L[4, 895] = -2.0
        L[5, 100:170] = 9.0
    inp = Inputs(T, 256, 256, E, k, seed=1, store=build_store(E, 256, 256, 1, experts=[]))
    r = inp.route(logits_in=L)
    np.testing.assert_array_equal(r["logits"], L)
    check_route(inp, r)
    np.testing.assert_array_equal(r["ids"][0], np.arange(16))
    if T > 1:
        np.testing.assert_array_equal(r["ids"][1], np.arange(16))
        np.testing.assert_array_equal(r["ids"][3], np.arange(500, 516))
        assert r["ids"][4][0] == 895 and list(r["ids"][4][1:]) == list(range(15))
        np.testing.assert_array_equal(r["ids"][5], np.arange(100, 116))


def test_all_tokens_to_the_same_experts():
    """Every token routed to the same 16 experts (each expert gets all T
    tokens), forced through logits-in mode; then the FFN and combine."""
    T, E, k = 150, 64, 16
    L = np.zeros((T, E), np.float32)
    hot = np.arange(3, 3 + 4 * k, 4)
    L[:, hot] = 10.0 + np.arange(k, dtype=np.float32) * 0.01
    inp = Inputs(T, 512, 256, E, k, seed=4, store=build_store(E, 512, 256, 4, experts=list(hot)))
    r = inp.route(logits_in=L)
    check_route(inp, r)
    assert np.all(np.diff(r["offsets"])[hot] == T)
    ox = OracleExperts(4, 512, 256)
    ref = oracle.moe_layer(inp.host_x(), ox.get(hot), E, k, logits_in=L, want_rows=True)
    assert_close(inp.ffn(r["offsets"], r["sorted_pairs"]), ref["rows"], "rows")


def test_t_zero_is_a_no_op():
    inp = Inputs(0, 256, 256, 16, 4, seed=1, store=build_store(16, 256, 256, 1, experts=[]))
    y = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    moe.moe_layer(inp.d, inp.x, inp.wr, None, inp.store, y, None, None, inp.ws)
    torch.cuda.synchronize()


def test_kernel_profile_hook(tiny):
    """moe_profile_arm / moe_profile_read time the armed kernel's launches:
    one duration per launch up to the armed count, then disarmed."""
    _, inp, _ = tiny
    moe.moe_profile_arm("gateup", 2)
    for _ in range(3):
        inp.layer()
    ms = moe.moe_profile_read(8)
    assert len(ms) == 2 and all(0 < t < 1000 for t in ms)
    inp.layer()
    assert moe.moe_profile_read(8) == []
    moe.moe_profile_arm("combine", 4)
    inp.layer()
    assert len(moe.moe_profile_read(1)) == 1
