"""GPU parity of one share of the experts (moe_layer_share,
moe_expert_ffn_share): experts are split into uneven contiguous shares; each
share's store holds only its experts.  Per share, the served records equal
the mask of the routing on the share (bit-exact) and the fp32 partial output
matches the oracle's partial; over the partition the served masks cover every
record once and the partials add up to the oracle's layer output.  The
share's rows from moe_expert_ffn_share equal moe_expert_ffn's bit for bit,
and rows outside the share are left untouched."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    import routed_expert_ffn_amd as moe
    import synth
    from tests.gpu_helpers import DEV, Inputs, OracleExperts, assert_close, say, to_np


def shares_of(E):
    a, b = E // 3 + 1, (2 * E) // 3 + 3
    return [(0, a), (a, b - a), (b, E - b)]


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (70, 48, 4), (1100, 32, 8)])
def test_layer_shares(T, E, k):
    say(f"shares T={T} E={E} k={k}")
    inp = Inputs(T, 512, 256, E, k, seed=31, bias=synth.zipf_bias(31, E, 0.5), router_std=0.1)
    y_full, ids_full, w_full = inp.layer()
    r = inp.route()
    ref = oracle.moe_layer(inp.host_x(), OracleExperts(31, 512, 256).get(r["ids"]), E, k, logits_in=r["logits"],
                           want_rows=True, nthreads=16)
    total = np.zeros((T, 512), np.float64)
    covered = np.zeros((T, k), np.int64)
    for base, count in shares_of(E):
        y = torch.full((T, 512), float("nan"), dtype=torch.float32, device=DEV)
        served = torch.full((T, k), 7, dtype=torch.uint8, device=DEV)
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        moe.moe_layer_share(inp.d, base, count, inp.x, inp.wr, inp.bias, inp.store.share(base, count), y, served,
                            ids, w, inp.ws)
        torch.cuda.synchronize()
        ids, w, served, y = to_np(ids), to_np(w), to_np(served), to_np(y).astype(np.float64)
        np.testing.assert_array_equal(ids, ids_full)
        np.testing.assert_array_equal(w, w_full)
        want_served, want_y = oracle.layer_share(ref, base, count, k)
        np.testing.assert_array_equal(served, want_served)
        say(f"  share [{base}, {base + count}): {int(served.sum())} of {T * k} records")
        assert np.all(np.isfinite(y))
        if served.any():
            assert_close(y, want_y, f"y_partial [{base}, {base + count})")
        else:
            assert not y.any()
        total += y
        covered += served
    np.testing.assert_array_equal(covered, np.ones((T, k), np.int64))
    assert_close(total, ref["y"], "sum of the partials")


@pytest.mark.parametrize("T,E,k", [(8, 896, 16), (1100, 32, 8)])
def test_expert_ffn_share_rows(T, E, k):
    inp = Inputs(T, 512, 256, E, k, seed=32)
    r = inp.route()
    full = inp.ffn(r["offsets"], r["sorted_pairs"])
    offsets = torch.as_tensor(r["offsets"], device=DEV)
    sorted_pairs = torch.as_tensor(r["sorted_pairs"], device=DEV)
    for base, count in shares_of(E):
        rows = torch.full((T * k, 512), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_expert_ffn_share(inp.d, base, count, inp.x, offsets, sorted_pairs, inp.store.share(base, count),
                                 rows, inp.ws)
        torch.cuda.synchronize()
        rows = to_np(rows)
        lo, hi = r["offsets"][base], r["offsets"][base + count]
        np.testing.assert_array_equal(rows[lo:hi], full[lo:hi])
        assert np.isnan(rows[:lo]).all() and np.isnan(rows[hi:]).all()
