"""Pins of the CPU oracle to facts outside itself: the pages' byte census,
format definitions checked against torch's fp8 type and the OCP table,
constructed round trips, brute force and library routines (numpy lexsort,
argsort, matmul, scipy softmax), and exact invariants."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import softmax

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1_TABLE = {}
for line in open(os.path.join(GOLDEN, "ocp_e2m1.txt")):
    if line.strip() and not line.startswith("#"):
        c, v = line.split()
        E2M1_TABLE[int(c)] = float(v)


def e4m3_torch(codes):
    return torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


# ---- formats ------------------------------------------------------------------

def test_e2m1_values_match_ocp_table():
    for c in range(16):
        v = oracle.e2m1_value(c)
        assert v == E2M1_TABLE[c] and np.signbit(v) == np.signbit(E2M1_TABLE[c]), c


def test_e4m3_decode_matches_torch_float8():
    ref = e4m3_torch(np.arange(256))
    for c in range(256):
        v = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert np.isnan(v), c
        else:
            assert v == ref[c], c
    assert oracle.e4m3_value(0x7E) == 448.0


def test_e4m3_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    finite = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = (finite[1:] + finite[:-1]) / 2  # exact midpoints, representable in fp32
    t = np.concatenate([finite, mids, rng.uniform(0, 448, 4000), rng.uniform(0, 2 ** -6, 1000),
                        np.exp(rng.uniform(np.log(2 ** -10), np.log(448), 4000))]).astype(np.float32)
    ref = torch.tensor(t).to(torch.float8_e4m3fn).float().numpy()
    got = np.array([oracle.e4m3_value(oracle.e4m3_round(float(v))) for v in t])
    np.testing.assert_array_equal(got, ref)
    # Above the largest finite value the oracle saturates (its stated reading).
    assert oracle.e4m3_value(oracle.e4m3_round(460.0)) == 448.0
    assert oracle.e4m3_value(oracle.e4m3_round(1e9)) == 448.0


def test_e2m1_round_golden_ties():
    for line in open(os.path.join(GOLDEN, "e2m1_rounding.txt")):
        if line.strip() and not line.startswith("#"):
            r, c = line.split()
            assert oracle.e2m1_round(float(np.float32(r))) == int(c), r


def test_nvfp4_products_exact_in_fp16_not_in_e4m3():
    """Every e2m1 magnitude times every finite e4m3 scale is exactly an fp16
    (and a bf16) value, but not always an e4m3 value: the GPU dequantises to
    fp16 with no rounding, and a fused fp8 operand would not be exact."""
    mags = [Fraction(E2M1_TABLE[c]) for c in range(8)]
    scales = [Fraction(oracle.e4m3_value(c)) for c in range(127)]
    e4m3_set = set(scales)
    not_e4m3 = 0
    for a in mags:
        for s in scales:
            p = a * s
            assert Fraction(float(np.float16(float(p)))) == p
            assert Fraction(float(torch.tensor(float(p)).to(torch.bfloat16).float())) == p
            not_e4m3 += p not in e4m3_set
    assert not_e4m3 > 0
    assert max(mags) * max(scales) == 2688


# ---- byte census from the pages -------------------------------------------------

def test_k3_expert_byte_census():
    g = json.load(open(os.path.join(GOLDEN, "k3_nvfp4_census.json")))
    H, I = g["hidden_latent"], g["intermediate"]
    ours = oracle.nvfp4_matrix_bytes(I, H) * 2 + oracle.nvfp4_matrix_bytes(H, I)
    # The checkpoint's 12 tensors are 4 per matrix: codes, block scales, the
    # global scale, and a second fp32 scalar (the activation scale, unused
    # with bf16 activations) -> 3 x 4 bytes more than the layout stores.
    assert ours + 3 * 4 == g["bytes_per_expert"]
    assert g["experts_per_layer"] * g["moe_layers"] == g["experts_total"]
    assert (ours + 12) * g["experts_total"] == g["routed_bytes_total"]


# ---- quantiser ----------------------------------------------------------------

def _grid_matrix(rng, N, K, gs_exp=-12):
    """W = sign * e2m1 * sigma_b * gs with a +-6 in every block and a block
    scale of 448 somewhere, so the quantiser must return the same bytes."""
    nb = K // 16
    gs = np.float32(2.0 ** gs_exp)
    sc = rng.integers(1, 127, size=(N, nb)).astype(np.uint8)
    sc[rng.integers(N), rng.integers(nb)] = 0x7E  # 448
    zero_blocks = rng.random((N, nb)) < 0.05
    sc[zero_blocks] = 0
    sc[0, 0] = 0x7E
    mag = rng.integers(0, 8, size=(N, K)).astype(np.uint8)
    for n in range(N):
        for b in range(nb):
            mag[n, 16 * b + rng.integers(16)] = 7  # the block's 6
    sign = (rng.random((N, K)) < 0.5) & (mag != 0)
    mag[np.repeat(zero_blocks, 16, axis=1)] = 0
    sign &= mag != 0
    codes = mag | (sign.astype(np.uint8) << 3)
    sigma = e4m3_torch(sc)
    w = np.array([[E2M1_TABLE[c] for c in row] for row in codes]) * np.repeat(sigma, 16, axis=1) * float(gs)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return w.astype(np.float32), q, sc, gs


def test_quantize_grid_round_trip_is_bit_exact():
    rng = np.random.default_rng(7)
    for N, K in [(4, 32), (33, 160), (64, 512)]:
        w, q, sc, gs = _grid_matrix(rng, N, K)
        m = oracle.nvfp4_quantize(w)
        assert m.gs == gs
        np.testing.assert_array_equal(m.sf, sc)
        np.testing.assert_array_equal(m.q, q)
        np.testing.assert_array_equal(oracle.nvfp4_dequantize(m), w.astype(np.float64))


def _dequant_independent(m):
    N, K = m.shape
    codes = np.empty((N, K), np.uint8)
    codes[:, 0::2] = m.q & 15
    codes[:, 1::2] = m.q >> 4
    vals = np.vectorize(E2M1_TABLE.get)(codes)
    return vals * np.repeat(e4m3_torch(m.sf), 16, axis=1) * float(m.gs), codes


def test_quantize_random_is_nearest_on_grid():
    """For random normal weights, every code is the nearest e2m1 point to
    |w| / d_b (d_b the block's decoded scale), and each block scale is the
    e4m3 rounding (torch cast) of (blockmax/6)/gs."""
    w = synth.expert_f32(0, 5, 0, 48, 256)
    m = oracle.nvfp4_quantize(w)
    assert m.gs == np.float32(np.abs(w).max()) / np.float32(2688.0)
    deq, codes = _dequant_independent(m)
    np.testing.assert_array_equal(oracle.nvfp4_dequantize(m), deq)
    bmax = np.abs(w).reshape(48, 16, 16).max(axis=2)
    t = (bmax / np.float32(6.0)).astype(np.float32) / m.gs
    np.testing.assert_array_equal(e4m3_torch(m.sf), torch.tensor(t).to(torch.float8_e4m3fn).float().numpy())
    d = (e4m3_torch(m.sf).astype(np.float32) * m.gs).astype(np.float32)
    r = np.abs(w) / np.repeat(d, 16, axis=1)
    grid = np.array([E2M1_TABLE[c] for c in range(8)])
    dist = np.abs(r[..., None] - grid)
    best = dist.min(axis=-1)
    chosen = dist[np.arange(48)[:, None], np.arange(256)[None, :], codes & 7]
    np.testing.assert_allclose(chosen, best, rtol=0, atol=1e-6)
    assert np.all(np.sign(w[(codes & 7) != 0]) == np.where(codes[(codes & 7) != 0] & 8, -1, 1))
    assert np.all(codes[(codes & 7) == 0] == 0)  # zero is always the +0 code
    assert np.any((w < 0) & ((codes & 7) == 0))  # ... also for small negative weights


def test_quantize_all_zero_matrix():
    m = oracle.nvfp4_quantize(np.zeros((3, 32), np.float32))
    assert m.gs == 1.0 and not m.q.any() and not m.sf.any()


# ---- router, top-k, permutation -------------------------------------------------

def test_router_logits_match_numpy_matmul():
    x = synth.x_bf16(0, 5, 512)
    wr = synth.router_bf16(0, 512, 96)
    bias = synth.zipf_bias(0, 96, 0.3)
    got = oracle.router_logits(x, wr, bias)
    ref = synth.bf16_to_f32(x).astype(np.float64) @ synth.bf16_to_f32(wr).astype(np.float64) + bias
    np.testing.assert_allclose(got, ref, rtol=2 ** -23, atol=1e-7)


def _lexsort_topk(logits, k):
    E = logits.shape[1]
    return np.stack([np.lexsort((np.arange(E), -row))[:k] for row in logits]).astype(np.int32)


def test_topk_matches_lexsort_with_ties():
    rng = np.random.default_rng(3)
    E, k = 896, 16
    L = rng.normal(0, 1.7, size=(40, E)).astype(np.float32)
    L[1] = 0.0                                   # all tied -> ids 0..15
    L[2, ::2] = -0.0                             # +-0 mixed, everything else 0
    L[2, 1::2] = 0.0
    L[3] = np.round(L[3] * 2) / 2                # many duplicated values
    L[4, 100:120] = 9.0                          # a tied block at the top
    L[5] = np.float32(1.0) + np.float32(2 ** -23) * rng.integers(0, 3, E)  # ulp-level ties
    ids, w = oracle.topk_softmax(L, k)
    np.testing.assert_array_equal(ids, _lexsort_topk(L, k))
    np.testing.assert_array_equal(ids[1], np.arange(16))
    np.testing.assert_array_equal(ids[2], np.arange(16))
    np.testing.assert_array_equal(ids[4], np.arange(100, 116))


def test_topk_weights():
    rng = np.random.default_rng(4)
    L = rng.normal(0, 1.7, size=(30, 896)).astype(np.float32)
    ids, w = oracle.topk_softmax(L, 16)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) < 1e-12)
    ref = np.stack([softmax(L[t, ids[t]].astype(np.float64)) for t in range(30)])
    np.testing.assert_allclose(w, ref, rtol=1e-13)
    assert np.all(np.diff(w, axis=1) <= 0)
    ids1, w1 = oracle.topk_softmax(L, 1)
    assert np.all(w1 == 1.0)
    np.testing.assert_array_equal(ids1[:, 0], np.argmax(L, axis=1))


def test_permutation_matches_stable_argsort():
    rng = np.random.default_rng(5)
    E, k = 896, 16
    L = rng.normal(0, 1.7, size=(300, E)).astype(np.float32)
    L += synth.zipf_bias(0, E, 0.5)
    ids, _ = oracle.topk_softmax(L, k)
    offsets, sp, pp = oracle.permute(ids, E)
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(ids.ravel(), minlength=E))]))
    np.testing.assert_array_equal(sp, np.argsort(ids.ravel(), kind="stable"))
    np.testing.assert_array_equal(pp[sp], np.arange(ids.size))
    assert offsets[-1] == ids.size


def test_permutation_page_example():
    """128 tokens choosing 8 experts each in a pool of 256 gives 1,024
    assignments; after the sort expert e000's records come first, then e001
    ... ("Computation and Data Movement for Inference", section 15)."""
    rng = np.random.default_rng(6)
    L = rng.normal(size=(128, 256)).astype(np.float32)
    ids, _ = oracle.topk_softmax(L, 8)
    offsets, sp, _ = oracle.permute(ids, 256)
    assert offsets[-1] == 1024
    experts_in_order = ids.ravel()[sp]
    assert np.all(np.diff(experts_in_order) >= 0)
    tokens = sp // 8
    for e in range(256):
        seg = tokens[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


# ---- expert FFN and the whole layer ---------------------------------------------

def _tiny_experts(seed, E, H, I, identical=False):
    ex = {}
    for e in range(E):
        src = 0 if identical else e
        ex[e] = tuple(oracle.nvfp4_quantize(synth.expert_f32(seed, src, m, *synth.expert_shape(m, H, I)))
                      for m in range(3))
    return ex


def _numpy_layer(x_bf16, wr_bf16, bias, experts, k):
    """The layer written with numpy primitives and an independent dequant."""
    x = synth.bf16_to_f32(x_bf16).astype(np.float64)
    logits = (x @ synth.bf16_to_f32(wr_bf16).astype(np.float64) + (0 if bias is None else bias)).astype(np.float32)
    ids = _lexsort_topk(logits, k)
    y = np.zeros_like(x)
    deq = {e: [_dequant_independent(m)[0] for m in mats] for e, mats in experts.items()}
    for t in range(x.shape[0]):
        w = softmax(logits[t, ids[t]].astype(np.float64))
        for j, e in enumerate(ids[t]):
            g, u, d = deq[e]
            a = x[t] @ g.T
            b = x[t] @ u.T
            h = torch.nn.functional.silu(torch.from_numpy(a)).numpy() * b  # SiLU from torch, in fp64
            y[t] += w[j] * (h @ d.T)
    return logits, ids, y


@pytest.mark.parametrize("T,H,I,E,k", [(5, 64, 32, 32, 4), (3, 128, 48, 24, 6), (1, 32, 16, 8, 8)])
def test_layer_matches_numpy_brute_force(T, H, I, E, k):
    x = synth.x_bf16(1, T, H)
    wr = synth.router_bf16(1, H, E, std=0.2)
    bias = synth.zipf_bias(1, E, 0.4)
    ex = _tiny_experts(1, E, H, I)
    out = oracle.moe_layer(x, ex, E, k, wr_bf16=wr, bias=bias, want_rows=True)
    logits, ids, y = _numpy_layer(x, wr, bias, ex, k)
    np.testing.assert_array_equal(out["ids"], ids)
    np.testing.assert_allclose(out["logits"], logits, rtol=2 ** -22)
    np.testing.assert_allclose(out["y"], y, rtol=1e-11, atol=1e-13)
    # rows are unweighted per record in sorted order
    recon = np.zeros_like(y)
    for t in range(T):
        for j in range(k):
            recon[t] += out["w"][t, j] * out["rows"][out["pair_pos"][t * k + j]]
    np.testing.assert_array_equal(recon, out["y"])


def test_identical_experts_equal_dense_ffn():
    """With every expert the same matrices, routing cannot matter: y is the
    dense SwiGLU of that expert, since the weights sum to one."""
    T, H, I, E, k = 4, 64, 32, 16, 5
    x = synth.x_bf16(2, T, H)
    wr = synth.router_bf16(2, H, E, std=0.3)
    ex = _tiny_experts(2, E, H, I, identical=True)
    out = oracle.moe_layer(x, ex, E, k, wr_bf16=wr)
    g, u, d = [_dequant_independent(m)[0] for m in ex[0]]
    xf = synth.bf16_to_f32(x).astype(np.float64)
    a, b = xf @ g.T, xf @ u.T
    dense = (a / (1 + np.exp(-a)) * b) @ d.T
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-14)


def test_single_expert_routing_equals_its_ffn():
    """k = 1 with a bias that makes expert 3 win for every token: y is
    expert 3's dense FFN exactly (weight 1)."""
    T, H, I, E = 6, 64, 32, 16
    x = synth.x_bf16(3, T, H)
    wr = synth.router_bf16(3, H, E)
    bias = np.zeros(E, np.float32)
    bias[3] = 100.0
    ex = _tiny_experts(3, E, H, I)
    out = oracle.moe_layer(x, ex, E, 1, wr_bf16=wr, bias=bias)
    assert np.all(out["ids"] == 3) and np.all(out["w"] == 1.0)
    g, u, d = [_dequant_independent(m)[0] for m in ex[3]]
    xf = synth.bf16_to_f32(x).astype(np.float64)
    a, b = xf @ g.T, xf @ u.T
    np.testing.assert_allclose(out["y"], (a / (1 + np.exp(-a)) * b) @ d.T, rtol=1e-12, atol=1e-14)
    assert list(out["offsets"][3:5]) == [0, T]


def test_token_permutation_and_scale_invariances():
    T, H, I, E, k = 7, 64, 32, 32, 4
    x = synth.x_bf16(4, T, H)
    wr = synth.router_bf16(4, H, E, std=0.2)
    ex = _tiny_experts(4, E, H, I)
    base = oracle.moe_layer(x, ex, E, k, wr_bf16=wr)
    perm = np.random.default_rng(0).permutation(T)
    moved = oracle.moe_layer(x[perm], ex, E, k, wr_bf16=wr)
    np.testing.assert_array_equal(moved["y"], base["y"][perm])
    np.testing.assert_array_equal(moved["ids"], base["ids"][perm])
    doubled = {e: (g, u, oracle.NVFP4(d.q, d.sf, d.gs * 2)) for e, (g, u, d) in ex.items()}
    out2 = oracle.moe_layer(x, doubled, E, k, wr_bf16=wr)
    np.testing.assert_array_equal(out2["y"], 2 * base["y"])


def test_thread_count_invariance_and_logits_in():
    T, H, I, E, k = 9, 64, 32, 32, 6
    x = synth.x_bf16(5, T, H)
    wr = synth.router_bf16(5, H, E, std=0.2)
    ex = _tiny_experts(5, E, H, I)
    ref = oracle.moe_layer(x, ex, E, k, wr_bf16=wr, nthreads=1, want_rows=True)
    for n in (2, 3, 8):
        o = oracle.moe_layer(x, ex, E, k, wr_bf16=wr, nthreads=n, want_rows=True)
        np.testing.assert_array_equal(o["y"], ref["y"])
        np.testing.assert_array_equal(o["rows"], ref["rows"])
    li = oracle.moe_layer(x, ex, E, k, logits_in=ref["logits"])
    np.testing.assert_array_equal(li["y"], ref["y"])


def test_missing_selected_expert_is_an_error():
    T, H, I, E, k = 2, 32, 16, 8, 2
    x = synth.x_bf16(6, T, H)
    wr = synth.router_bf16(6, H, E)
    ex = _tiny_experts(6, E, H, I)
    out = oracle.moe_layer(x, ex, E, k, wr_bf16=wr)
    used = set(out["ids"].ravel())
    del ex[min(used)]
    with pytest.raises(RuntimeError):
        oracle.moe_layer(x, ex, E, k, wr_bf16=wr)


# ---- latent routed-expert block ----------------------------------------------------

def test_round_bf16_golden_and_direct_from_fp64():
    """Hand-derived bf16 patterns: ties go to the even pattern, just above a
    tie rounds up (which a detour through fp32 would lose), overflow at half
    an ulp above the largest finite value, subnormals, signed zeros."""
    cases = [(1.0 + 2 ** -8, 0x3F80), (1.0 + 3 * 2 ** -8, 0x3F82), (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),
             (-(1.0 + 2 ** -8), 0xBF80), (0.0, 0x0000), (-0.0, 0x8000), ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),
             ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80), ((2 - 2 ** -8 - 2 ** -20) * 2.0 ** 127, 0x7F7F),
             (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000), (3 * 2.0 ** -135, 0x0001), (float("inf"), 0x7F80)]
    got = oracle.round_bf16(np.array([v for v, _ in cases]))
    assert [int(g) for g in got] == [want for _, want in cases]


def test_round_bf16_matches_torch_and_generator_on_fp32_values():
    rng = np.random.default_rng(11)
    f = (rng.standard_normal(100000) * np.exp(rng.uniform(-60, 60, 100000))).astype(np.float32)
    ours = oracle.round_bf16(f.astype(np.float64))
    np.testing.assert_array_equal(ours, torch.tensor(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(ours, synth.round_bf16(f))


def test_bf16_matmul_exact_on_small_integers():
    """Integer-valued bf16 operands keep every product and partial sum exact,
    so the fp64 result must equal the integer matrix product."""
    rng = np.random.default_rng(12)
    xi = rng.integers(-8, 9, (5, 96))
    wi = rng.integers(-8, 9, (96, 40))
    x = synth.round_bf16(xi.astype(np.float32))
    w = synth.round_bf16(wi.astype(np.float32))
    np.testing.assert_array_equal(oracle.bf16_matmul(x, w), (xi @ wi).astype(np.float64))


def test_latent_layer_with_embedding_projections_is_the_plain_layer():
    """P_down = [I; 0] (Hm = 2H) takes the first H features as the latent
    and P_up = [I 0] writes the latent back into them: the block's output is
    the plain layer's output on those features, rounded to bf16, and zeros."""
    T, H, I, E, k = 5, 64, 32, 16, 4
    Hm = 2 * H
    x = synth.x_bf16(13, T, Hm)
    wr = synth.router_bf16(13, Hm, E, std=0.2)
    one = synth.round_bf16(np.ones(1, np.float32))[0]
    pd = np.zeros((Hm, H), np.uint16)
    pd[np.arange(H), np.arange(H)] = one
    pu = np.zeros((H, Hm), np.uint16)
    pu[np.arange(H), np.arange(H)] = one
    ex = _tiny_experts(13, E, H, I)
    lat = oracle.latent_layer(x, ex, E, k, pd, pu, wr_bf16=wr)
    np.testing.assert_array_equal(lat["z"], x[:, :H])
    plain = oracle.moe_layer(np.ascontiguousarray(x[:, :H]), ex, E, k,
                             logits_in=oracle.router_logits(x, wr))
    np.testing.assert_array_equal(lat["ids"], plain["ids"])
    np.testing.assert_array_equal(lat["y"][:, :H], synth.bf16_to_f32(oracle.round_bf16(plain["y"])))
    assert not lat["y"][:, H:].any()


def test_layer_shares_partition_the_layer():
    """Shares that partition the experts: their served masks are disjoint and
    cover every record, and their partial outputs add up to the layer's
    output (to fp64 rounding; exactly where a token's experts all fall in
    one share)."""
    T, H, I, E, k = 6, 64, 32, 16, 4
    x = synth.x_bf16(14, T, H)
    wr = synth.router_bf16(14, H, E, std=0.3)
    out = oracle.moe_layer(x, _tiny_experts(14, E, H, I), E, k, wr_bf16=wr, want_rows=True)
    parts = [oracle.layer_share(out, b, c, k) for b, c in [(0, 5), (5, 1), (6, 10)]]
    np.testing.assert_array_equal(sum(p[0].astype(int) for p in parts), np.ones((T, k), int))
    total = sum(p[1] for p in parts)
    np.testing.assert_allclose(total, out["y"], rtol=1e-13, atol=1e-15)
    whole = oracle.layer_share(out, 0, E, k)
    assert whole[0].all() and np.array_equal(whole[1], out["y"])


# ---- masked ids (one device's experts, the rest served elsewhere) -------------------

def test_masked_permutation_matches_stable_argsort():
    """Records whose id is -1 (or any id outside [0, E)) are masked: they are
    not counted, take no position (pair_pos -1), and the served records keep
    the (expert, token) order among themselves."""
    rng = np.random.default_rng(21)
    T, E, k = 200, 64, 8
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    masked = rng.random((T, k)) < 0.4
    ids[masked] = -1
    ids[3, 2], ids[7, 0] = E, -9  # also outside [0, E)
    flat = ids.ravel()
    keep = (flat >= 0) & (flat < E)
    offsets, sp, pp = oracle.permute(ids, E)
    n = int(keep.sum())
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat[keep], minlength=E))]))
    served_records = np.flatnonzero(keep)
    np.testing.assert_array_equal(sp[:n], served_records[np.argsort(flat[keep], kind="stable")])
    assert np.all(sp[n:] == -1)
    assert np.all(pp[~keep] == -1)
    np.testing.assert_array_equal(pp[sp[:n]], np.arange(n))
    # nothing masked: the unmasked permutation
    full = np.where(keep, flat, 0).reshape(T, k)
    o2, s2, p2 = oracle.permute(full, E)
    np.testing.assert_array_equal(s2, np.argsort(full.ravel(), kind="stable"))
    # everything masked: no records
    o3, s3, p3 = oracle.permute(np.full((T, k), -1, np.int32), E)
    assert not o3.any() and np.all(s3 == -1) and np.all(p3 == -1)


def _random_partition(rng, E, parts):
    """A random assignment of the E experts to `parts` devices, each device's
    experts in a random slot order: one global -> local map per device."""
    owner = rng.integers(0, parts, size=E)
    maps = []
    for d in range(parts):
        mine = np.flatnonzero(owner == d)
        m = np.full(E, -1, np.int64)
        m[mine] = rng.permutation(len(mine))
        maps.append(m)
    return maps


def test_masked_expert_pass_gives_the_layer_rows():
    """A device's store holds its experts in its own slot order; the router's
    ids mapped to those slots (-1 for experts held elsewhere) run through the
    expert pass, and every served record's row equals the whole layer's row
    for that record, bit for bit."""
    T, H, I, E, k = 7, 64, 32, 24, 4
    x = synth.x_bf16(31, T, H)
    wr = synth.router_bf16(31, H, E, std=0.3)
    ex = _tiny_experts(31, E, H, I)
    out = oracle.moe_layer(x, ex, E, k, wr_bf16=wr, want_rows=True)
    for m in _random_partition(np.random.default_rng(3), E, 3):
        n_local = int((m >= 0).sum())
        local_ids, served, _ = oracle.layer_mapped(out, m)
        store = {int(m[e]): ex[e] for e in range(E) if m[e] >= 0}
        offsets, sp, pp = oracle.permute(local_ids, n_local)
        rows = oracle.expert_rows(x, store, n_local, k, offsets, sp)
        for f in range(T * k):
            if served.ravel()[f]:
                np.testing.assert_array_equal(rows[pp[f]], out["rows"][out["pair_pos"][f]])
            else:
                assert pp[f] == -1
        assert np.all(np.isnan(rows[offsets[-1]:]))


def test_mapped_partials_partition_the_layer():
    """Devices whose experts partition the E experts: served masks are
    disjoint and cover every record, and the partial outputs add up to the
    layer's output.  Each partial is also checked against a numpy brute
    force over the served records (independent dequantiser)."""
    T, H, I, E, k = 6, 64, 32, 20, 5
    x = synth.x_bf16(33, T, H)
    wr = synth.router_bf16(33, H, E, std=0.3)
    ex = _tiny_experts(33, E, H, I)
    out = oracle.moe_layer(x, ex, E, k, wr_bf16=wr, want_rows=True)
    xd = synth.bf16_to_f32(x).astype(np.float64)
    deq = {e: [_dequant_independent(mm)[0] for mm in mats] for e, mats in ex.items()}
    maps = _random_partition(np.random.default_rng(8), E, 4)
    parts = [oracle.layer_mapped(out, m) for m in maps]
    np.testing.assert_array_equal(sum(p[1].astype(int) for p in parts), np.ones((T, k), int))
    np.testing.assert_allclose(sum(p[2] for p in parts), out["y"], rtol=1e-13, atol=1e-15)
    for m, (local_ids, served, yp) in zip(maps, parts):
        np.testing.assert_array_equal(local_ids, np.where(m[out["ids"]] >= 0, m[out["ids"]], -1))
        ref = np.zeros_like(yp)
        for t in range(T):
            for j in range(k):
                e = out["ids"][t, j]
                if m[e] >= 0:
                    g, u, d = deq[e]
                    a, b = xd[t] @ g.T, xd[t] @ u.T
                    ref[t] += out["w"][t, j] * ((a / (1 + np.exp(-a)) * b) @ d.T)
        np.testing.assert_allclose(yp, ref, rtol=1e-11, atol=1e-13)


# ---- shared experts -------------------------------------------------------------------

def _shared_weights(seed, H, I, count):
    wgu = synth.round_bf16((np.random.default_rng(seed).standard_normal((H, 2 * count * I)) * 0.1).astype(np.float32))
    wd = synth.round_bf16((np.random.default_rng(seed + 1).standard_normal((count * I, H)) * 0.1).astype(np.float32))
    return wgu, wd


def test_shared_experts_match_torch_float64():
    """Against torch's float64 matmuls and SiLU (another implementation of the
    products), with the oracle's bf16 rounding of h shared by both."""
    T, H, I, count = 5, 64, 48, 2
    x = synth.x_bf16(15, T, H)
    wgu, wd = _shared_weights(15, H, I, count)
    f = lambda a: torch.tensor(synth.bf16_to_f32(a).astype(np.float64))
    gu = f(x) @ f(wgu)
    hs = []
    for s in range(count):
        g, u = gu[:, 2 * s * I:2 * s * I + I], gu[:, 2 * s * I + I:2 * s * I + 2 * I]
        hs.append(torch.nn.functional.silu(g) * u)
    h = f(oracle.round_bf16(torch.cat(hs, 1).numpy()))
    ref = (h @ f(wd)).numpy()
    np.testing.assert_allclose(oracle.shared_experts(x, wgu, wd, count, I), ref, rtol=1e-12, atol=1e-12)


def test_shared_experts_are_additive_and_vanish():
    """Two shared experts give the sum of each alone; zero input gives zero
    (SiLU(0) = 0); zero down weights leave the routed layer unchanged."""
    T, H, I = 4, 64, 32
    x = synth.x_bf16(16, T, H)
    wgu, wd = _shared_weights(16, H, I, 2)
    both = oracle.shared_experts(x, wgu, wd, 2, I)
    one = oracle.shared_experts(x, np.ascontiguousarray(wgu[:, :2 * I]), np.ascontiguousarray(wd[:I]), 1, I)
    two = oracle.shared_experts(x, np.ascontiguousarray(wgu[:, 2 * I:]), np.ascontiguousarray(wd[I:]), 1, I)
    np.testing.assert_allclose(both, one + two, rtol=1e-13, atol=1e-13)
    assert not oracle.shared_experts(np.zeros_like(x), wgu, wd, 2, I).any()
    E, k = 16, 4
    wr = synth.router_bf16(16, H, E, std=0.3)
    ex = _tiny_experts(16, E, H, I)
    plain = oracle.moe_layer(x, ex, E, k, wr_bf16=wr)
    with_zero = oracle.layer_with_shared(x, ex, E, k, wgu, np.zeros_like(wd), 2, I, wr_bf16=wr)
    np.testing.assert_array_equal(with_zero["y"], plain["y"])


# ---- MXFP4 (the OCP microscaling format) ----------------------------------------------

def e8m0_torch(codes):
    with np.errstate(invalid="ignore"):  # code 255 decodes to NaN
        return torch.tensor(np.asarray(codes, np.uint8)).view(torch.float8_e8m0fnu).float().numpy().astype(np.float64)


def _mx_dequant_independent(m):
    N, K = m.shape
    codes = np.empty((N, K), np.uint8)
    codes[:, 0::2] = m.q & 15
    codes[:, 1::2] = m.q >> 4
    return np.vectorize(E2M1_TABLE.get)(codes) * np.repeat(e8m0_torch(m.sf), 32, axis=1), codes


def test_e8m0_decode_matches_torch():
    ref = e8m0_torch(np.arange(256))
    for s in range(256):
        v = oracle.e8m0_value(s)
        assert (np.isnan(v) and np.isnan(ref[s])) or v == ref[s], s


def test_mxfp4_golden_blocks():
    """Hand-derived: a block whose largest value is 7 gets X = 2^(2-2) = 1
    (scale byte 127) and 7 clamps to 6; a block whose largest value is 0.3
    gets X = 2^(-2-2) (byte 123) and 0.3 / X = 4.8 rounds to 4; a zero
    block gets byte 0 and zero codes."""
    w = np.zeros((3, 32), np.float32)
    w[0, 5] = 7.0
    w[0, 6] = -1.25  # 1.25 is a tie between 1 and 1.5: even code 1.0
    w[1, 0] = 0.3
    w[1, 1] = 0.09375  # 1.5 * 2^-4: exactly code 1.5
    m = oracle.mxfp4_quantize(w)
    assert list(m.sf[:, 0]) == [127, 123, 0]
    deq = oracle.mxfp4_dequantize(m)
    assert deq[0, 5] == 6.0 and deq[0, 6] == -1.0
    assert deq[1, 0] == 4 * 2.0 ** -4 and deq[1, 1] == 0.09375
    assert not deq[2].any()


def test_mxfp4_grid_round_trip_is_bit_exact():
    """Blocks of e2m1 grid values times 2^s whose largest magnitude is 4 or 6
    times 2^s come back exactly, with scale byte 127 + s."""
    rng = np.random.default_rng(17)
    N, K = 8, 256
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    codes = rng.integers(0, 16, (N, K))
    vals = np.where(codes >= 8, -1, 1) * grid[codes % 8]
    s = rng.integers(-20, 20, (N, K // 32))
    for n in range(N):
        for b in range(K // 32):
            vals[n, 32 * b] = (4.0 if (n + b) % 2 else 6.0) * (1 if vals[n, 32 * b] >= 0 else -1)
    w = (vals * np.repeat(2.0 ** s, 32, axis=1)).astype(np.float32)
    m = oracle.mxfp4_quantize(w)
    np.testing.assert_array_equal(m.sf, (127 + s).astype(np.uint8))
    np.testing.assert_array_equal(oracle.mxfp4_dequantize(m), w.astype(np.float64))
    deq, _ = _mx_dequant_independent(m)
    np.testing.assert_array_equal(deq, w.astype(np.float64))


def test_mxfp4_random_is_nearest_on_grid():
    """Random weights: each scale is 2^(floor(log2 blockmax) - 2) and each
    code the nearest e2m1 point to |w| / X (clamped to 6), ties to even."""
    w = synth.expert_f32(0, 6, 0, 32, 256)
    m = oracle.mxfp4_quantize(w)
    bmax = np.abs(w).reshape(32, 8, 32).max(axis=2).astype(np.float64)
    np.testing.assert_array_equal(m.sf.astype(int), np.floor(np.log2(bmax)).astype(int) - 2 + 127)
    deq, codes = _mx_dequant_independent(m)
    np.testing.assert_array_equal(oracle.mxfp4_dequantize(m), deq)
    x = np.repeat(e8m0_torch(m.sf), 32, axis=1)
    r = np.abs(w).astype(np.float64) / x
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    dist = np.abs(r[..., None] - grid)
    best = dist.min(axis=-1)
    got = np.abs(deq) / x
    assert np.all(np.abs(r - got) <= best + 1e-15)


def test_layer_with_mxfp4_experts_matches_numpy():
    """The layer on MXFP4 experts equals the numpy layer on independently
    dequantised weights (the same checks as the NVFP4 brute force)."""
    T, H, I, E, k = 3, 64, 32, 8, 2
    x = synth.x_bf16(18, T, H)
    wr = synth.router_bf16(18, H, E, std=0.3)
    ex = {e: tuple(oracle.mxfp4_quantize(synth.expert_f32(18, e, m, *synth.expert_shape(m, H, I))) for m in range(3))
          for e in range(E)}
    out = oracle.moe_layer(x, ex, E, k, wr_bf16=wr)
    xf = synth.bf16_to_f32(x).astype(np.float64)
    y = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            g, u, d = [_mx_dequant_independent(mm)[0] for mm in ex[int(out["ids"][t, j])]]
            a, b = xf[t] @ g.T, xf[t] @ u.T
            y[t] += out["w"][t, j] * ((a / (1 + np.exp(-a)) * b) @ d.T)
    np.testing.assert_allclose(out["y"], y, rtol=1e-11, atol=1e-13)
