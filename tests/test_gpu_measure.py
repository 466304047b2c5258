"""GPU checks of the measurement plumbing and of launch modes the benchmark
relies on: the HBM read calibration reads every word exactly once, and a
moe_layer captured in a HIP graph gives, on every replay, exactly what the
eager call gives (with other eager work between the replays)."""
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
