"""GPU parity of the latent routed-expert block (moe_latent_layer) against
the oracle's latent_layer: small shapes that take the single-launch routing,
the three-kernel permutation and the large-tile GEMMs, and K3's shape
(hidden 7168, routed latent 3584, I = 3072, all 896 experts resident) for
single-user decode and a prefill chunk on sampled tokens.

Routing is evaluated by the oracle on the GPU's fp32 router logits (taken
from moe_route on the same hidden states), so ids must match bit for bit.
The latent z is the bf16 rounding of an fp32 (GPU) or fp64 (oracle) sum, so
an element may differ by one bf16 unit in the last place where the sum sits
near a rounding boundary.  y is held to the layer's tolerances (max-abs
2e-2, relative L2 5e-3 against the oracle's fp64 value), except that an
element of |y| >= 8 may differ by half a bf16 unit of its magnitude plus
4e-3: y has the hidden width's scale, where its own rounding to bf16 alone
reaches half a unit (3.1e-2 at |y| in [8, 16)).  The block also rounds the
combined latent y_lat to bf16 before the up projection, the GPU from its fp32
sum and the oracle from its fp64 one; where the two sit on either side of a
rounding boundary they differ by one bf16 unit, which the up projection
carries into y.  Each element of y is allowed 3 times the root-sum-square of
those units weighted by its column of P_up, the spread of that carried
difference when any element of y_lat may differ."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    import routed_expert_ffn_amd as moe
    import synth
    from synth.workloads import WORKLOADS, bias_for
    from tests.gpu_helpers import DEV, OracleExperts, assert_close_bf16_out, build_store, say, to_np


class LatentCase:
    def __init__(self, T, Hm, H, I, E, k, seed=0, bias=None, store=None, router_std=0.02):
        self.T, self.Hm, self.H, self.I, self.E, self.k, self.seed = T, Hm, H, I, E, k, seed
        self.router_std = router_std
        self.d = moe.dims(T, H, I, E, k)
        self.x = torch.empty((T, Hm), dtype=torch.bfloat16, device=DEV)
        synth.gpu_x_bf16(seed, self.x)
        self.wr = torch.empty((Hm, E), dtype=torch.bfloat16, device=DEV)
        synth.gpu_router_bf16(seed, self.wr, std=router_std)
        self.pd = torch.empty((Hm, H), dtype=torch.bfloat16, device=DEV)
        self.pu = torch.empty((H, Hm), dtype=torch.bfloat16, device=DEV)
        synth.gpu_proj_bf16(seed, 0, self.pd)
        synth.gpu_proj_bf16(seed, 1, self.pu)
        self.bias_np = None if bias is None else np.asarray(bias, np.float32)
        self.bias = None if bias is None else torch.tensor(self.bias_np, device=DEV)
        self.store = store if store is not None else build_store(E, H, I, seed)
        self.ws = torch.empty(moe.moe_latent_workspace_bytes(self.d, Hm), dtype=torch.uint8, device=DEV)

    def run(self):
        T, k = self.T, self.k
        y = torch.empty((T, self.Hm), dtype=torch.bfloat16, device=DEV)
        z = torch.empty((T, self.H), dtype=torch.bfloat16, device=DEV)
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        moe.moe_latent_layer(self.d, self.Hm, self.pd, self.pu, self.x, self.wr, self.bias, self.store, y, z, ids, w,
                             self.ws)
        torch.cuda.synchronize()
        return to_np(y), z.view(torch.int16).cpu().numpy().view(np.uint16), to_np(ids), to_np(w)

    def logits(self):
        """The router's fp32 logits on the hidden states, from moe_route."""
        T, E, k = self.T, self.E, self.k
        d = moe.dims(T, self.Hm, 256, E, k)
        ws = torch.empty(moe.moe_workspace_bytes(d), dtype=torch.uint8, device=DEV)
        logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
        sp = torch.empty(T * k, dtype=torch.int32, device=DEV)
        pp = torch.empty(T * k, dtype=torch.int32, device=DEV)
        moe.moe_route(d, self.x, self.wr, self.bias, logits, ids, w, off, sp, pp, ws)
        torch.cuda.synchronize()
        return to_np(logits)

    def host(self, rows=None):
        x = synth.x_bf16(self.seed, self.T, self.Hm)
        return x if rows is None else x[rows]


def check_z(z_gpu, z_ref, x, pd):
    """bf16 latents of an fp32 (GPU) and an fp64 (oracle) sum of K products:
    apart by at most one bf16 unit plus the fp32 summation error bound
    K * 2^-24 * sum |x w| (where the sum cancels, that bound exceeds a unit of
    the small result); and equal almost everywhere."""
    a = synth.bf16_to_f32(z_gpu).astype(np.float64)
    b = synth.bf16_to_f32(z_ref).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(a), np.abs(b)))[1] - 8)
    K = x.shape[1]
    mag = np.abs(synth.bf16_to_f32(x).astype(np.float64)) @ np.abs(synth.bf16_to_f32(pd).astype(np.float64))
    bound = ulp + K * 2.0 ** -24 * mag
    worst = float(np.max(np.abs(a - b) / bound))
    frac = np.mean(a != b)
    say(f"  z: {frac:.2e} of elements differ; worst difference {worst:.2f} of its bound")
    assert worst <= 1.0
    assert frac <= 0.01


def compare(case, rows, y, z, ids, logits, ex):
    x = case.host(rows)
    pd = synth.proj_bf16(case.seed, 0, case.Hm, case.H)
    ref = oracle.latent_layer(x, ex, case.E, case.k, pd, synth.proj_bf16(case.seed, 1, case.H, case.Hm),
                              logits_in=logits[rows], nthreads=16)
    np.testing.assert_array_equal(ids[rows], ref["ids"])
    check_z(z[rows], ref["z"], x, pd)
    # the bf16 seam at y_lat: one unit per element, carried through P_up
    y_lat = synth.bf16_to_f32(ref["y_lat"]).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(y_lat))[1] - 8)
    pu = synth.bf16_to_f32(synth.proj_bf16(case.seed, 1, case.H, case.Hm)).astype(np.float64)
    seam = 3.0 * np.sqrt((ulp ** 2) @ (pu ** 2))
    assert_close_bf16_out(y[rows], ref["y"], "y", extra=seam)
    return ref


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (70, 48, 4), (1100, 32, 8)])
def test_latent_block_small(T, E, k):
    """Hidden 1024 -> latent 512, I = 256: every token checked."""
    say(f"latent T={T} E={E} k={k}")
    case = LatentCase(T, 1024, 512, 256, E, k, seed=21, router_std=0.1)
    y, z, ids, w = case.run()
    logits = case.logits()
    ox = OracleExperts(21, 512, 256)
    rows = np.arange(T)
    ref = compare(case, rows, y, z, ids, logits, ox.get(ids))
    assert np.abs(w - ref["w"]).max() <= 1e-6


def test_latent_block_one_slab_projections():
    """8192 tokens at hidden 2048 -> latent 2048: both projections fill a
    wave of 256 tiles (32 token tiles x 10 column tiles of 224), so each
    takes one K slab and the tile writes the rounded bf16 output (and the
    latent's fp16 copy for the experts) itself; every token of the first, a
    middle and the last token tile, and 64 more, checked."""
    T, Hm, H, I, E, k = 8192, 2048, 2048, 256, 32, 4
    say(f"latent one-slab projections T={T} Hm={Hm} H={H}")
    case = LatentCase(T, Hm, H, I, E, k, seed=23, router_std=0.1)
    y, z, ids, w = case.run()
    logits = case.logits()
    rng = np.random.default_rng(5)
    rows = np.array(sorted(set(range(256)) | set(range(3840, 4096)) | set(range(T - 256, T)) |
                           set(rng.choice(T, size=64, replace=False))))
    ox = OracleExperts(23, H, I)
    compare(case, rows, y, z, ids, logits, ox.get(ids[rows]))


def test_latent_block_deterministic():
    case = LatentCase(8, 1024, 512, 256, 64, 8, seed=22)
    a = case.run()
    b = case.run()
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.fixture(scope="module")
def k3_store():
    wl = WORKLOADS["latent_decode_1"]
    say("building the K3-shape NVFP4 store on the GPU (896 experts, 3584 x 3072)")
    return build_store(wl.E, wl.H, wl.I, wl.seed)


@pytest.mark.parametrize("name", ["latent_decode_1", "latent_prefill_8192"])
def test_latent_block_k3_shape(name, k3_store):
    wl = WORKLOADS[name]
    say(f"latent full-size {name}: T={wl.T}")
    case = LatentCase(wl.T, wl.H_model, wl.H, wl.I, wl.E, wl.k, seed=wl.seed, bias=bias_for(wl), store=k3_store)
    y, z, ids, w = case.run()
    assert np.all(np.isfinite(y))
    logits = case.logits()
    rng = np.random.default_rng(3)
    rows = np.array(sorted(set([0, wl.T // 2, wl.T - 1]) | set(rng.choice(wl.T, size=min(wl.T, 29), replace=False))))
    say(f"  {len(rows)} sampled tokens")
    ox = OracleExperts(wl.seed, wl.H, wl.I)
    compare(case, rows, y, z, ids, logits, ox.get(ids[rows]))
