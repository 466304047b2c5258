"""CPU oracle for the routed MoE layer with NVFP4 experts.

TEST INFRASTRUCTURE ONLY: the plain fp64 reference that the GPU library is
checked against.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this package; the GPU library never does.  The C source
(oracle.c / oracle.h) cites, per function, the passage of the pages it
follows.  This module only marshals numpy arrays to it.
"""
import ctypes
import os

import numpy as np

from .build import LIB, LIB_SAN, build, sanitize_requested

_lib = None
_c_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")  # a mutated build, for checking the pins
        if not path:
            src = os.path.join(os.path.dirname(LIB), "oracle.c")
            path = LIB_SAN if sanitize_requested() else LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(src):
                build()
        L = ctypes.CDLL(path)
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_round.restype = ctypes.c_uint8
        L.oracle_e2m1_round.argtypes = [ctypes.c_double]
        L.oracle_e4m3_round.restype = ctypes.c_uint8
        L.oracle_e4m3_round.argtypes = [ctypes.c_double]
        L.oracle_nvfp4_matrix_bytes.restype = ctypes.c_size_t
        L.oracle_nvfp4_matrix_bytes.argtypes = [_c_i64, _c_i64]
        L.oracle_nvfp4_quantize.restype = None
        L.oracle_nvfp4_quantize.argtypes = [_p, _c_i64, _c_i64, _p, _p, _p]
        L.oracle_nvfp4_dequantize.restype = None
        L.oracle_nvfp4_dequantize.argtypes = [_p, _p, ctypes.c_float, _c_i64, _c_i64, _p]
        L.oracle_router_logits.restype = None
        L.oracle_router_logits.argtypes = [_p, _c_i64, _c_i64, _p, _c_i64, _p, _p]
        L.oracle_topk_softmax.restype = None
        L.oracle_topk_softmax.argtypes = [_p, _c_i64, _c_i64, ctypes.c_int, _p, _p]
        L.oracle_permute.restype = None
        L.oracle_permute.argtypes = [_p, _c_i64, _c_i64, ctypes.c_int, _p, _p, _p]
        L.oracle_swiglu_token.restype = None
        L.oracle_swiglu_token.argtypes = [_p, _p, _p, _p, _c_i64, _c_i64, _p]
        L.oracle_moe_layer.restype = ctypes.c_int
        L.oracle_moe_layer.argtypes = [_p, _c_i64, _c_i64, _c_i64, _p, _p, _p, _c_i64, ctypes.c_int, _p,
                                       ctypes.c_int, _p, _p, _p, _p, _p, _p, _p, _p]
        L.oracle_expert_ffn.restype = ctypes.c_int
        L.oracle_expert_ffn.argtypes = [_p, _c_i64, _c_i64, _c_i64, ctypes.c_int, _p, _p, _p, ctypes.c_int, _p]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_mxfp4_quantize.restype = None
        L.oracle_mxfp4_quantize.argtypes = [_p, _c_i64, _c_i64, _p, _p]
        L.oracle_mxfp4_dequantize.restype = None
        L.oracle_mxfp4_dequantize.argtypes = [_p, _p, _c_i64, _c_i64, _p]
        L.oracle_round_bf16.restype = None
        L.oracle_round_bf16.argtypes = [_p, _c_i64, _p]
        L.oracle_bf16_matmul.restype = None
        L.oracle_bf16_matmul.argtypes = [_p, _c_i64, _c_i64, _p, _c_i64, _p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def e2m1_value(code):
    return lib().oracle_e2m1_value(code)


def e4m3_value(code):
    return lib().oracle_e4m3_value(code)


def e2m1_round(r):
    return lib().oracle_e2m1_round(float(r))


def e4m3_round(t):
    return lib().oracle_e4m3_round(float(t))


def nvfp4_matrix_bytes(N, K):
    return lib().oracle_nvfp4_matrix_bytes(N, K)


class NVFP4:
    """One quantised matrix: q [N][K/2] u8, sf [N][K/16] u8, gs fp32."""

    def __init__(self, q, sf, gs):
        self.q, self.sf, self.gs = q, sf, np.float32(gs)

    @property
    def shape(self):
        return (self.q.shape[0], self.q.shape[1] * 2)


def nvfp4_quantize(w):
    w = _c(w, np.float32)
    N, K = w.shape
    assert K % 16 == 0
    q = np.empty((N, K // 2), np.uint8)
    sf = np.empty((N, K // 16), np.uint8)
    gs = np.zeros(1, np.float32)
    lib().oracle_nvfp4_quantize(_ptr(w), N, K, _ptr(q), _ptr(sf), _ptr(gs))
    return NVFP4(q, sf, gs[0])


def nvfp4_dequantize(m):
    N, K = m.shape
    out = np.empty((N, K), np.float64)
    lib().oracle_nvfp4_dequantize(_ptr(_c(m.q, np.uint8)), _ptr(_c(m.sf, np.uint8)), float(m.gs), N, K, _ptr(out))
    return out


def router_logits(x_bf16, wr_bf16, bias=None):
    x = _c(x_bf16, np.uint16)
    wr = _c(wr_bf16, np.uint16)
    T, H = x.shape
    E = wr.shape[1]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float32)
    lib().oracle_router_logits(_ptr(x), T, H, _ptr(wr), E, _ptr(b), _ptr(out))
    return out


def topk_softmax(logits, k):
    l = _c(logits, np.float32)
    T, E = l.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().oracle_topk_softmax(_ptr(l), T, E, k, _ptr(ids), _ptr(w))
    return ids, w


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pp = np.empty(T * k, np.int32)
    lib().oracle_permute(_ptr(ids), T, E, k, _ptr(offsets), _ptr(sp), _ptr(pp))
    return offsets, sp, pp


def swiglu_token(gate, up, down, x_row_bf16):
    I, H = gate.shape
    out = np.empty(H, np.float64)
    lib().oracle_swiglu_token(_ptr(_c(gate, np.float64)), _ptr(_c(up, np.float64)), _ptr(_c(down, np.float64)),
                              _ptr(_c(x_row_bf16, np.uint16)), H, I, _ptr(out))
    return out


class _Expert(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p * 3), ("sf", ctypes.c_void_p * 3), ("gs", ctypes.c_float * 3),
                ("format", ctypes.c_int32)]


def _expert_structs(experts, E):
    """ctypes array of E expert pointers (NULL where absent) and the arrays
    it points into (kept alive by the caller)."""
    keep = []
    structs = (ctypes.POINTER(_Expert) * E)()
    for e, mats in experts.items():
        s = _Expert()
        for m in range(3):
            q = _c(mats[m].q, np.uint8)
            sf = _c(mats[m].sf, np.uint8)
            keep += [q, sf]
            s.q[m] = q.ctypes.data
            s.sf[m] = sf.ctypes.data
            s.gs[m] = float(mats[m].gs)
        s.format = getattr(mats[0], "format", 0)
        keep.append(s)
        structs[e] = ctypes.pointer(s)
    return structs, keep


def moe_layer(x_bf16, experts, E, k, wr_bf16=None, bias=None, logits_in=None, nthreads=1, want_rows=False):
    """experts: mapping expert id -> (gate, up, down) NVFP4 triples; experts
    that no token selects may be absent.  Returns a dict of numpy arrays."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    any_ex = next(iter(experts.values()))
    I = any_ex[0].shape[0]
    structs, keep = _expert_structs(experts, E)
    wr = None if wr_bf16 is None else _c(wr_bf16, np.uint16)
    b = None if bias is None else _c(bias, np.float32)
    li = None if logits_in is None else _c(logits_in, np.float32)
    if li is None and wr is None:
        raise ValueError("need router weights or logits")
    logits = np.empty((T, E), np.float32)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    offsets = np.empty(E + 1, np.int32)
    sp = np.empty(T * k, np.int32)
    pp = np.empty(T * k, np.int32)
    rows = np.empty((T * k, H), np.float64) if want_rows else None
    y = np.empty((T, H), np.float64)
    rc = lib().oracle_moe_layer(_ptr(x), T, H, I, _ptr(wr), _ptr(b), _ptr(li), E, k,
                                ctypes.cast(structs, ctypes.c_void_p), nthreads, _ptr(logits), _ptr(ids), _ptr(w),
                                _ptr(offsets), _ptr(sp), _ptr(pp), _ptr(rows), _ptr(y))
    del keep
    if rc != 0:
        raise RuntimeError("oracle_moe_layer: a selected expert was not provided")
    out = dict(logits=logits, ids=ids, w=w, offsets=offsets, sorted_pairs=sp, pair_pos=pp, y=y)
    if want_rows:
        out["rows"] = rows
    return out


def expert_rows(x_bf16, experts, E, k, offsets, sorted_pairs, nthreads=1):
    """The expert pass on a given permutation (oracle_permute's, masked
    records included): rows[p] for p < offsets[E] (fp64, unweighted, sorted
    order); later rows are NaN.  experts maps the ids 0..E-1 that have
    records to their NVFP4 / MXFP4 triples."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    offsets = _c(offsets, np.int32)
    sp = _c(sorted_pairs, np.int32)
    I = next(iter(experts.values()))[0].shape[0]
    structs, keep = _expert_structs(experts, E)
    rows = np.full((max(T * k, 1), H), np.nan, np.float64)
    rc = lib().oracle_expert_ffn(_ptr(x), H, I, E, k, ctypes.cast(structs, ctypes.c_void_p), _ptr(offsets),
                                 _ptr(sp), nthreads, _ptr(rows))
    del keep
    if rc != 0:
        raise RuntimeError("oracle_expert_ffn: an expert with records was not provided")
    return rows


# ---- latent routed-expert block (oracle.h: "latent routed-expert block") --------

def round_bf16(a):
    """Nearest bf16 bit patterns of fp64 values (ties to even)."""
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_round_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_matmul(x_bf16, w_bf16):
    """fp64 x @ W for bf16 bit patterns x [T][K] and W [K][N]."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    T, K = x.shape
    K2, N = w.shape
    assert K == K2
    out = np.empty((T, N), np.float64)
    lib().oracle_bf16_matmul(_ptr(x), T, K, _ptr(w), N, _ptr(out))
    return out


def latent_layer(x_bf16, experts, E, k, w_down_bf16, w_up_bf16, wr_bf16=None, bias=None, logits_in=None,
                 nthreads=1, want_rows=False):
    """K3's latent routed-expert block on model-width tokens x [T][Hm]:
      z     = bf16(x . P_down)                 routed latent [T][H]
      route = top-k of the router on x (the model's hidden state)
      y_lat = bf16(moe_layer(z) with that routing)   [T][H]
      y     = y_lat . P_up                     [T][Hm] fp64 (the GPU rounds it to bf16)
    P_down [Hm][H] and P_up [H][Hm] are bf16, stored input-major.  The
    roundings to bf16 are the model's activation type at the block's seams;
    where the router reads is a reading (the pages do not say): the hidden
    state, as the plain router of the non-latent layer does."""
    x = _c(x_bf16, np.uint16)
    z = round_bf16(bf16_matmul(x, w_down_bf16))
    if logits_in is None:
        logits_in = router_logits(x, wr_bf16, bias)
    out = moe_layer(z, experts, E, k, logits_in=logits_in, nthreads=nthreads, want_rows=want_rows)
    y_lat = round_bf16(out["y"])
    out["z"] = z
    out["y_lat"] = y_lat
    out["y_lat_f64"] = out["y"]
    out["y"] = bf16_matmul(y_lat, w_up_bf16)
    return out


# ---- one share of the experts (expert parallelism) ---------------------------------

def layer_partial(out, served):
    """The part of the layer that one device computes, from a
    moe_layer(..., want_rows=True) result and the mask served[t][j] of the
    records it serves: y_partial[t] = sum over the served j of
    w[t][j] * rows[pos(t, j)], fp64 over ascending j.  al-engr.com Kimi-K3
    plan, "What has to be built - and the discovery that changed it" (a mask
    on the router's chosen ids) and "Track A" (a worker returns rows plus the
    ids it served)."""
    w, rows, pos = out["w"], out["rows"], out["pair_pos"]
    T, k = w.shape
    y = np.zeros((T, rows.shape[1]), np.float64)
    for t in range(T):
        for j in range(k):
            if served[t, j]:
                y[t] += w[t, j] * rows[pos[t * k + j]]
    return y


def layer_share(out, base, count, k):
    """layer_partial for the contiguous share of experts [base, base +
    count): served[t][j] = whether record (t, j) selected one of them (a
    local expert offset of base)."""
    ids = out["ids"]
    served = (ids >= base) & (ids < base + count)
    return served.astype(np.uint8), layer_partial(out, served)


def layer_mapped(out, expert_map):
    """layer_partial for the experts a device holds, given as the map from
    global expert id to its slot in the device's store (-1: served
    elsewhere).  Returns the ids with the map applied (the router's chosen
    ids, remote ones masked to -1), served and y_partial."""
    expert_map = np.asarray(expert_map, np.int64)
    local = expert_map[out["ids"]]
    served = local >= 0
    return np.where(served, local, -1).astype(np.int32), served.astype(np.uint8), layer_partial(out, served)


# ---- shared experts (every token uses them) ------------------------------------------

def shared_experts(x_bf16, w_gate_up_bf16, w_down_bf16, count, I):
    """Dense bf16 SwiGLU experts that every token uses, summed (fp64):
    for shared expert s, g = x . Wgu[:, 2sI : 2sI+I], u = x . Wgu[:, 2sI+I :
    2sI+2I], h = bf16(SiLU(g) * u), out += h . Wd[sI : sI+I, :].  Weights are
    bf16 and stored input-major (Wgu [H][count*2I], Wd [count*I][H]); h is
    rounded to bf16, the dense module's activation type, before the down
    projection.  [p1] section 3.3: every token uses the 2 shared experts,
    whose output joins the routed experts' in the layer's sum; [p2]
    "Precision: what is stored in which format": shared experts are bf16."""
    gu = bf16_matmul(x_bf16, w_gate_up_bf16)
    T = gu.shape[0]
    h = np.empty((T, count * I), np.float64)
    for s in range(count):
        g = gu[:, 2 * s * I:2 * s * I + I]
        u = gu[:, 2 * s * I + I:2 * s * I + 2 * I]
        h[:, s * I:(s + 1) * I] = g / (1.0 + np.exp(-g)) * u
    return bf16_matmul(round_bf16(h), w_down_bf16)


def layer_with_shared(x_bf16, experts, E, k, w_gate_up_bf16, w_down_bf16, count, I_shared, wr_bf16=None, bias=None,
                      logits_in=None, nthreads=1, want_rows=False):
    """The routed layer plus its shared experts: y = routed sum + shared sum
    (fp64; the GPU rounds the total to bf16 once)."""
    out = moe_layer(x_bf16, experts, E, k, wr_bf16=wr_bf16, bias=bias, logits_in=logits_in, nthreads=nthreads,
                    want_rows=want_rows)
    out["y_routed"] = out["y"]
    out["y_shared"] = shared_experts(x_bf16, w_gate_up_bf16, w_down_bf16, count, I_shared)
    out["y"] = out["y_routed"] + out["y_shared"]
    return out


# ---- MXFP4 (oracle.h: "MXFP4 weight store") --------------------------------------

def e8m0_value(s):
    return lib().oracle_e8m0_value(int(s))


class MXFP4:
    """q [N][K/2] e2m1 codes, sf [N][K/32] e8m0 scales; no per-tensor scale."""
    format = 1
    gs = 1.0

    def __init__(self, q, sf):
        self.q, self.sf = q, sf

    @property
    def shape(self):
        return self.q.shape[0], self.q.shape[1] * 2


def mxfp4_quantize(w):
    w = _c(w, np.float32)
    N, K = w.shape
    q = np.empty((N, K // 2), np.uint8)
    sf = np.empty((N, K // 32), np.uint8)
    lib().oracle_mxfp4_quantize(_ptr(w), N, K, _ptr(q), _ptr(sf))
    return MXFP4(q, sf)


def mxfp4_dequantize(m):
    N, K = m.shape
    out = np.empty((N, K), np.float64)
    lib().oracle_mxfp4_dequantize(_ptr(_c(m.q, np.uint8)), _ptr(_c(m.sf, np.uint8)), N, K, _ptr(out))
    return out
