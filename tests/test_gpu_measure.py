"""GPU checks of the measurement plumbing and of launch modes the benchmark
relies on: the HBM read calibration reads every word exactly once, and
moe_layer, moe_layer_shared (whose shared experts run on a second stream of
the library) and moe_latent_layer captured in a HIP graph give, on every
replay, exactly what the eager call gives (with other eager work between the
replays)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_amd as moe
    from tests.gpu_helpers import DEV, Inputs, say


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (64 << 20) + 48, 1 << 30])
def test_stream_read_reads_every_word_once(nbytes):
    say(f"stream read of {nbytes} bytes")
    g = torch.Generator(device=DEV)
    g.manual_seed(nbytes)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=DEV, generator=g)
    sink = torch.zeros(moe.STREAM_SINK_WORDS, dtype=torch.int32, device=DEV)
    moe.moe_stream_read(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (70, 48, 4), (1100, 32, 8)])
def test_layer_graph_replays_match_eager(T, E, k):
    """Single-launch routing (T <= 8), the three-kernel permutation (T > 64)
    and the large-tile GEMMs (T >= 1024) under capture."""
    say(f"graph T={T} E={E} k={k}")
    inp = Inputs(T, 512, 256, E, k, seed=5)
    y_ref, ids_ref, w_ref = inp.layer()
    other = Inputs(T, 512, 256, E, k, seed=6, store=inp.store)
    y = torch.empty((T, inp.H), dtype=torch.bfloat16, device=DEV)
    ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_layer(inp.d, inp.x, inp.wr, inp.bias, inp.store, y, ids, w, inp.ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_layer(inp.d, inp.x, inp.wr, inp.bias, inp.store, y, ids, w, inp.ws)
    torch.cuda.synchronize()
    for replay in range(4):
        y.zero_()
        ids.zero_()
        w.zero_()
        y_other, _, _ = other.layer()  # eager work on the same weights between replays
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.float().cpu().numpy(), y_ref, f"replay {replay}")
        np.testing.assert_array_equal(ids.cpu().numpy(), ids_ref)
        np.testing.assert_array_equal(w.cpu().numpy(), w_ref)
        assert not np.array_equal(y_other, y_ref)


def _capture(call):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (70, 48, 4), (1100, 32, 8)])
def test_shared_layer_graph_replays_match_eager(T, E, k):
    """The shared experts run on the library's second stream, forked from
    and joined to the captured stream: every replay equals the eager call,
    with eager calls that use that stream between the replays."""
    from tests.test_gpu_shared import COUNT, shared_weights
    say(f"graph shared T={T} E={E} k={k}")
    inp = Inputs(T, 512, 256, E, k, seed=43, router_std=0.1)
    other = Inputs(T, 512, 256, E, k, seed=44, store=inp.store, router_std=0.1)
    gu, dn, _, _ = shared_weights(43, 512, 256)
    nws = moe.moe_layer_shared_workspace_bytes(inp.d, COUNT, 256)

    def outs():
        return (torch.empty((T, inp.H), dtype=torch.bfloat16, device=DEV),
                torch.empty((T, k), dtype=torch.int32, device=DEV),
                torch.empty((T, k), dtype=torch.float32, device=DEV),
                torch.empty(nws, dtype=torch.uint8, device=DEV))

    y, ids, w, ws = outs()
    oy, oids, ow, ows = outs()

    def call(c=inp, o=(y, ids, w, ws)):
        moe.moe_layer_shared(c.d, COUNT, 256, gu, dn, c.x, c.wr, c.bias, c.store, o[0], o[1], o[2], o[3])

    call()
    torch.cuda.synchronize()
    ref = [t.cpu().clone() for t in (y, ids, w)]
    call(other, (oy, oids, ow, ows))
    torch.cuda.synchronize()
    ref_other = oy.cpu().clone()
    graph = _capture(call)
    for replay in range(4):
        for t in (y, ids, w, oy):
            t.zero_()
        call(other, (oy, oids, ow, ows))
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((y, ids, w), ref):
            assert torch.equal(got.cpu(), want), f"replay {replay}"
        assert torch.equal(oy.cpu(), ref_other)
        assert not torch.equal(ref_other, ref[0])


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (70, 48, 4), (1100, 32, 8)])
def test_latent_layer_graph_replays_match_eager(T, E, k):
    """The latent block (two projections around the routed experts) under
    capture: every replay equals the eager call."""
    from tests.test_gpu_latent import LatentCase
    say(f"graph latent T={T} E={E} k={k}")
    case = LatentCase(T, 1024, 512, 256, E, k, seed=23, router_std=0.1)
    other = LatentCase(T, 1024, 512, 256, E, k, seed=24, store=case.store, router_std=0.1)

    def outs(c):
        return (torch.empty((T, c.Hm), dtype=torch.bfloat16, device=DEV),
                torch.empty((T, c.H), dtype=torch.bfloat16, device=DEV),
                torch.empty((T, k), dtype=torch.int32, device=DEV),
                torch.empty((T, k), dtype=torch.float32, device=DEV))

    o = outs(case)
    oo = outs(other)

    def call(c=case, t=o):
        moe.moe_latent_layer(c.d, c.Hm, c.pd, c.pu, c.x, c.wr, c.bias, c.store, t[0], t[1], t[2], t[3], c.ws)

    call()
    torch.cuda.synchronize()
    ref = [t.cpu().clone() for t in o]
    graph = _capture(call)
    for replay in range(4):
        for t in o:
            t.zero_()
        call(other, oo)
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(o, ref):
            assert torch.equal(got.cpu(), want), f"replay {replay}"
        assert not torch.equal(oo[0].cpu(), ref[0])


def test_mfma_rate_calibration():
    """moe_mfma_rate runs its MFMA rounds and leaves finite, non-zero
    per-block checksums; its rate is plausible for the chip (between a tenth
    of the datasheet peak and the peak)."""
    sink = torch.full((moe.MFMA_RATE_BLOCKS,), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_mfma_rate(200, sink)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    moe.moe_mfma_rate(4000, sink)
    b.record()
    b.synchronize()
    tf = 4000 * moe.MFMA_RATE_FLOPS_PER_ITER / (a.elapsed_time(b) * 1e-3) / 1e12
    say(f"  sustained fp16 MFMA: {tf:.0f} TFLOP/s")
    v = sink.cpu()
    assert torch.isfinite(v).all() and (v != 0).all()
    assert 250 < tf <= 2500
    with pytest.raises(moe.MoeError):
        moe.moe_mfma_rate(0, sink)
