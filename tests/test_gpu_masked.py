"""GPU parity of masked expert ids: the mask on the router's chosen ids that
splitting the experts across devices needs (al-engr.com Kimi-K3 plan, "What
has to be built - and the discovery that changed it": an id of -1 stands for
an expert another device serves).

moe_permute builds the permutation from caller ids with random subsets
masked (-1 and other ids outside [0, E)) and must equal the oracle's bit for
bit, on the single-block path (T <= 64) and the three-kernel path.
moe_expert_ffn on that permutation computes exactly the served records: their
rows equal the unmasked layer's rows for the same records, bit for bit, and
nothing else is written.  moe_layer_mapped runs one device's experts, placed
in its store by a global -> local map: its served mask and local ids are
exact, its fp32 partial matches the oracle's, and the partials of devices
whose maps partition the experts add up to the oracle's layer output."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import oracle
    import routed_expert_ffn_amd as moe
    import synth
    from tests.gpu_helpers import DEV, Inputs, OracleExperts, assert_close, say, to_np

H, I = 512, 256
SENTINEL = 0x5A5A5A5A


def _masked_ids(rng, T, E, k, frac):
    """Distinct experts per token (as a router picks them), a random fraction
    of the records masked to -1, and a few masked with other ids outside
    [0, E)."""
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[rng.random((T, k)) < frac] = -1
    odd = rng.random((T, k)) < 0.02
    ids[odd] = rng.choice(np.array([E, E + 5, -2, -(1 << 30), (1 << 30)], np.int32), size=int(odd.sum()))
    return ids


def _permute_gpu(d, ids, ws):
    T, k = ids.shape
    out = dict(offsets=torch.full((d.E + 1,), SENTINEL, dtype=torch.int32, device=DEV),
               sorted_pairs=torch.full((T * k,), SENTINEL, dtype=torch.int32, device=DEV),
               pair_pos=torch.full((T * k,), SENTINEL, dtype=torch.int32, device=DEV))
    moe.moe_permute(d, torch.as_tensor(ids, device=DEV), out["offsets"], out["sorted_pairs"], out["pair_pos"], ws)
    torch.cuda.synchronize()
    return {n: to_np(t) for n, t in out.items()}


@pytest.mark.parametrize("T,E,k,frac", [(8, 896, 16, 0.3), (64, 64, 8, 0.5), (70, 48, 4, 0.4),
                                        (1100, 32, 8, 0.6), (300, 896, 16, 1.0), (130, 40, 6, 0.0)])
def test_permute_masked_ids(T, E, k, frac):
    say(f"moe_permute T={T} E={E} k={k} masked fraction {frac}")
    rng = np.random.default_rng(T * 7 + E)
    ids = _masked_ids(rng, T, E, k, frac)
    d = moe.dims(T, H, I, E, k)
    ws = torch.empty(moe.moe_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    got = _permute_gpu(d, ids, ws)
    offsets, sp, pp = oracle.permute(ids, E)
    n = int(offsets[-1])
    say(f"  served records {n} of {T * k}")
    np.testing.assert_array_equal(got["offsets"], offsets)
    np.testing.assert_array_equal(got["sorted_pairs"][:n], sp[:n])
    assert np.all(got["sorted_pairs"][n:] == SENTINEL), "entries past the served records were written"
    np.testing.assert_array_equal(got["pair_pos"], pp)


def _local_store(store, experts_in_slot_order):
    """A device's store: the given global experts, in slot order, copied out
    of the full store."""
    idx = torch.as_tensor(np.asarray(experts_in_slot_order, np.int64), device=DEV)
    loc = moe.ExpertStore(len(experts_in_slot_order), store.H, store.I, device=DEV)
    for m in store.MATS:
        for dst, src in zip(loc.t[m], store.t[m]):
            dst.copy_(src.index_select(0, idx))
    torch.cuda.synchronize()
    return loc


def _partition(rng, E, parts):
    owner = rng.integers(0, parts, size=E)
    maps, orders = [], []
    for dv in range(parts):
        mine = rng.permutation(np.flatnonzero(owner == dv))  # slot s holds global expert mine[s]
        m = np.full(E, -1, np.int32)
        m[mine] = np.arange(len(mine), dtype=np.int32)
        maps.append(m)
        orders.append(mine)
    return maps, orders


@pytest.mark.parametrize("T,E,k", [(8, 64, 8), (70, 48, 4), (1100, 32, 8)])
def test_expert_ffn_on_masked_permutation(T, E, k):
    """Rows of the served records from a device's store equal the unmasked
    layer's rows bit for bit (every output row is its own token row times
    the same weights, in the same order); other rows are left as they were."""
    say(f"masked expert pass T={T} E={E} k={k}")
    inp = Inputs(T, H, I, E, k, seed=41, bias=synth.zipf_bias(41, E, 0.5), router_std=0.1)
    r = inp.route()
    full = inp.ffn(r["offsets"], r["sorted_pairs"])
    maps, orders = _partition(np.random.default_rng(T), E, 2)
    for m, order in zip(maps, orders):
        if len(order) == 0:
            continue
        local = np.where(m[r["ids"]] >= 0, m[r["ids"]], -1).astype(np.int32)
        d = moe.dims(T, H, I, len(order), k)
        ws = torch.empty(moe.moe_workspace_bytes(d), dtype=torch.uint8, device=DEV)
        p = _permute_gpu(d, local, ws)
        rows = torch.full((T * k, H), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_expert_ffn(d, inp.x, torch.as_tensor(p["offsets"], device=DEV),
                           torch.as_tensor(p["sorted_pairs"], device=DEV), _local_store(inp.store, order), rows, ws)
        torch.cuda.synchronize()
        rows = to_np(rows)
        n = int(p["offsets"][-1])
        served = np.flatnonzero(local.ravel() >= 0)
        say(f"  device with {len(order)} experts: {n} served records")
        assert n == len(served)
        np.testing.assert_array_equal(rows[p["pair_pos"][served]], full[r["pair_pos"][served]])
        assert np.isnan(rows[n:]).all()


@pytest.mark.parametrize("T,E,k,parts", [(8, 896, 16, 3), (70, 48, 4, 3), (1100, 32, 8, 4)])
def test_layer_mapped_partition(T, E, k, parts):
    say(f"moe_layer_mapped T={T} E={E} k={k} over {parts} devices")
    inp = Inputs(T, H, I, E, k, seed=43, bias=synth.zipf_bias(43, E, 0.5), router_std=0.1)
    y_full, ids_full, w_full = inp.layer()
    r = inp.route()
    ref = oracle.moe_layer(inp.host_x(), OracleExperts(43, H, I).get(r["ids"]), E, k, logits_in=r["logits"],
                           want_rows=True, nthreads=16)
    maps, orders = _partition(np.random.default_rng(T + 1), E, parts)
    total = np.zeros((T, H), np.float64)
    covered = np.zeros((T, k), np.int64)
    for m, order in zip(maps, orders):
        if len(order) == 0:
            continue
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
        served = torch.full((T, k), 7, dtype=torch.uint8, device=DEV)
        ids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        w = torch.empty((T, k), dtype=torch.float32, device=DEV)
        lids = torch.empty((T, k), dtype=torch.int32, device=DEV)
        moe.moe_layer_mapped(inp.d, torch.as_tensor(m, device=DEV), len(order), inp.x, inp.wr, inp.bias,
                             _local_store(inp.store, order), y, served, ids, w, lids, inp.ws)
        torch.cuda.synchronize()
        ids, w, served, lids, y = to_np(ids), to_np(w), to_np(served), to_np(lids), to_np(y).astype(np.float64)
        np.testing.assert_array_equal(ids, ids_full)
        np.testing.assert_array_equal(w, w_full)
        want_lids, want_served, want_y = oracle.layer_mapped(ref, m)
        np.testing.assert_array_equal(lids, want_lids)
        np.testing.assert_array_equal(served, want_served)
        say(f"  device with {len(order)} experts: {int(served.sum())} of {T * k} records")
        assert np.all(np.isfinite(y))
        if served.any():
            assert_close(y, want_y, f"y_partial ({len(order)} experts)")
        else:
            assert not y.any()
        total += y
        covered += served
    np.testing.assert_array_equal(covered, np.ones((T, k), np.int64))
    assert_close(total, ref["y"], "sum of the partials")
