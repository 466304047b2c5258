"""moe_layer_noalloc (the layer with the library's own scratch as its
workspace, for callers that cannot allocate) against moe_layer with a
caller workspace, through the C ABI: the same ids, weights and output bit
for bit, on two calls in a row, the second with fewer tokens, so the scratch
holds the first call's contents when the second runs."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import routed_expert_ffn_amd as moe
    import synth
    from tests.gpu_helpers import DEV, Inputs, build_store, say, to_np


def _noalloc(inp):
    y = torch.full((inp.T, inp.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    ids = torch.full((inp.T, inp.k), -5, dtype=torch.int32, device=DEV)
    w = torch.full((inp.T, inp.k), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_layer_noalloc(inp.d, inp.x, inp.wr, inp.bias, inp.store, y, ids, w)
    torch.cuda.synchronize()
    return to_np(y), to_np(ids), to_np(w)


@pytest.mark.parametrize("H,I,E,k,Ts", [(512, 256, 896, 16, (100, 3)), (7168, 2048, 64, 16, (156, 64, 1))])
def test_noalloc_matches_layer(H, I, E, k, Ts):
    store = build_store(E, H, I, 51)
    for T in Ts:
        say(f"moe_layer_noalloc T={T} H={H} I={I} E={E} k={k}")
        inp = Inputs(T, H, I, E, k, seed=51, t0=7 * T, bias=synth.zipf_bias(51, E, 0.3), store=store)
        y, ids, w = inp.layer()
        y2, ids2, w2 = _noalloc(inp)
        np.testing.assert_array_equal(ids2, ids)
        np.testing.assert_array_equal(w2, w)
        np.testing.assert_array_equal(y2, y)
        assert np.all(np.isfinite(y2))


def test_noalloc_rejects_too_many_tokens():
    d = moe.dims(157, 7168, 2048, 896, 16)
    x = torch.empty((157, 7168), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer_noalloc(d, x, x, None, moe.ExpertStore(1, 512, 256, device=DEV), x, None, None)
    assert e.value.status == 4
