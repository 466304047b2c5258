"""Python binding of libmoe.so, the MI355X (gfx950) routed-MoE layer with
NVFP4 experts.

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI in include/moe.h, whose entry points this module mirrors by
name.  torch is used for device memory and streams.  If libmoe.so is not
built, loading fails loudly; there is no CPU fallback.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK = 0
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN", 4: "MOE_ERR_WORKSPACE",
                5: "MOE_ERR_HIP"}
KERNELS = {"router": 0, "topk": 1, "permute": 2, "cast": 3, "gateup": 4, "down": 5, "combine": 6, "project": 7,
           "shared": 8}
# Symbols include/moe.h declares.
EXPORTS = ("moe_workspace_bytes", "moe_quantize_workspace_bytes", "moe_quantize_nvfp4", "moe_route",
           "moe_expert_ffn", "moe_layer", "moe_status_string", "moe_last_error", "moe_profile_arm",
           "moe_profile_read", "moe_stream_read", "moe_latent_workspace_bytes", "moe_latent_layer",
           "moe_expert_ffn_share", "moe_layer_share", "moe_layer_shared_workspace_bytes", "moe_layer_shared",
           "moe_quantize_mxfp4", "moe_permute", "moe_layer_mapped",
           "moe_layer_noalloc", "moe_mfma_rate")
FORMATS = {"nvfp4": 0, "mxfp4": 1}  # moe_weight_format
# MOE_STREAM_SINK_WORDS of moe.h
STREAM_SINK_WORDS = 4096
# MOE_NOALLOC_SCRATCH_BYTES of moe.h
NOALLOC_SCRATCH_BYTES = 64 << 20
# MOE_MFMA_RATE_BLOCKS and MOE_MFMA_RATE_FLOPS_PER_ITER of moe.h
MFMA_RATE_BLOCKS = 1024
MFMA_RATE_FLOPS_PER_ITER = 1024 * 8 * 4 * 32768


class MoeError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32)]


class NVFP4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("sf", ctypes.c_void_p), ("gs", ctypes.c_void_p)]


class Experts(ctypes.Structure):
    _fields_ = [("gate", NVFP4), ("up", NVFP4), ("down", NVFP4), ("format", ctypes.c_int32)]


class Share(ctypes.Structure):
    _fields_ = [("base", ctypes.c_int32), ("count", ctypes.c_int32)]


class Shared(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("I", ctypes.c_int32), ("w_gate_up", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p)]


class Latent(ctypes.Structure):
    _fields_ = [("H_model", ctypes.c_int32), ("w_down", ctypes.c_void_p), ("w_up", ctypes.c_void_p)]


_lib = None
_p = ctypes.c_void_p


def lib():
    """Load libmoe.so (built in tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [Dims]
        L.moe_quantize_workspace_bytes.restype = ctypes.c_size_t
        L.moe_quantize_workspace_bytes.argtypes = []
        L.moe_quantize_nvfp4.restype = ctypes.c_int
        L.moe_quantize_nvfp4.argtypes = [_p, ctypes.c_int64, ctypes.c_int64, _p, _p, _p, _p, ctypes.c_size_t, _p]
        L.moe_quantize_mxfp4.restype = ctypes.c_int
        L.moe_quantize_mxfp4.argtypes = [_p, ctypes.c_int64, ctypes.c_int64, _p, _p, _p, _p, ctypes.c_size_t, _p]
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [Dims, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
        L.moe_expert_ffn.restype = ctypes.c_int
        L.moe_expert_ffn.argtypes = [Dims, _p, _p, _p, ctypes.POINTER(Experts), _p, _p, ctypes.c_size_t, _p]
        L.moe_layer.restype = ctypes.c_int
        L.moe_layer.argtypes = [Dims, _p, _p, _p, ctypes.POINTER(Experts), _p, _p, _p, _p, ctypes.c_size_t, _p]
        L.moe_expert_ffn_share.restype = ctypes.c_int
        L.moe_expert_ffn_share.argtypes = [Dims, Share, _p, _p, _p, ctypes.POINTER(Experts), _p, _p, ctypes.c_size_t,
                                           _p]
        L.moe_layer_share.restype = ctypes.c_int
        L.moe_layer_share.argtypes = [Dims, Share, _p, _p, _p, ctypes.POINTER(Experts), _p, _p, _p, _p, _p,
                                      ctypes.c_size_t, _p]
        L.moe_layer_noalloc.restype = ctypes.c_int
        L.moe_layer_noalloc.argtypes = [Dims, _p, _p, _p, ctypes.POINTER(Experts), _p, _p, _p, _p]
        L.moe_permute.restype = ctypes.c_int
        L.moe_permute.argtypes = [Dims, _p, _p, _p, _p, _p, ctypes.c_size_t, _p]
        L.moe_layer_mapped.restype = ctypes.c_int
        L.moe_layer_mapped.argtypes = [Dims, _p, ctypes.c_int32, _p, _p, _p, ctypes.POINTER(Experts), _p, _p, _p, _p,
                                       _p, _p, ctypes.c_size_t, _p]
        L.moe_layer_shared_workspace_bytes.restype = ctypes.c_size_t
        L.moe_layer_shared_workspace_bytes.argtypes = [Dims, ctypes.POINTER(Shared)]
        L.moe_layer_shared.restype = ctypes.c_int
        L.moe_layer_shared.argtypes = [Dims, ctypes.POINTER(Shared), _p, _p, _p, ctypes.POINTER(Experts), _p, _p, _p, _p,
                                       ctypes.c_size_t, _p]
        L.moe_latent_workspace_bytes.restype = ctypes.c_size_t
        L.moe_latent_workspace_bytes.argtypes = [Dims, ctypes.c_int32]
        L.moe_latent_layer.restype = ctypes.c_int
        L.moe_latent_layer.argtypes = [Dims, ctypes.POINTER(Latent), _p, _p, _p, ctypes.POINTER(Experts), _p, _p, _p,
                                       _p, _p, ctypes.c_size_t, _p]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_profile_arm.restype = ctypes.c_int
        L.moe_profile_arm.argtypes = [ctypes.c_int, ctypes.c_int]
        L.moe_profile_read.restype = ctypes.c_int
        L.moe_profile_read.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.moe_mfma_rate.restype = ctypes.c_int
        L.moe_mfma_rate.argtypes = [ctypes.c_int, _p, _p]
        L.moe_stream_read.restype = ctypes.c_int
        L.moe_stream_read.argtypes = [_p, ctypes.c_size_t, _p, _p]
        _lib = L
    return _lib


def _check(status):
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _ptr(t):
    """Device address of a torch tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def dims(T, H, I, E, k):
    return Dims(T, H, I, E, k)


# ---- the C ABI, by name ------------------------------------------------------

def moe_workspace_bytes(d):
    return lib().moe_workspace_bytes(d)


def moe_quantize_workspace_bytes():
    return lib().moe_quantize_workspace_bytes()


def moe_quantize_nvfp4(w, q, sf, gs, ws, stream=None):
    N, K = w.shape
    _check(lib().moe_quantize_nvfp4(_ptr(w), N, K, _ptr(q), _ptr(sf), _ptr(gs), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def moe_quantize_mxfp4(w, q, sf, gs, ws, stream=None):
    N, K = w.shape
    _check(lib().moe_quantize_mxfp4(_ptr(w), N, K, _ptr(q), _ptr(sf), _ptr(gs), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream)))


def moe_route(d, x, w_router, bias, logits, topk_ids, topk_w, expert_offsets, sorted_pairs, pair_pos, ws,
              stream=None):
    _check(lib().moe_route(d, _ptr(x), _ptr(w_router), _ptr(bias), _ptr(logits), _ptr(topk_ids), _ptr(topk_w),
                           _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(pair_pos), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(stream)))


def moe_expert_ffn(d, x, expert_offsets, sorted_pairs, experts, rows, ws, stream=None):
    _check(lib().moe_expert_ffn(d, _ptr(x), _ptr(expert_offsets), _ptr(sorted_pairs), ctypes.byref(experts.c()),
                                _ptr(rows), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer(d, x, w_router, bias, experts, y, topk_ids_out, topk_w_out, ws, stream=None):
    _check(lib().moe_layer(d, _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(experts.c()), _ptr(y),
                           _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws), ws.numel() * ws.element_size(),
                           _stream(stream)))


def moe_layer_noalloc(d, x, w_router, bias, experts, y, topk_ids_out, topk_w_out, stream=None):
    """moe_layer with the library's own scratch as workspace; allocates
    nothing (moe.h: moe_layer_noalloc)."""
    _check(lib().moe_layer_noalloc(d, _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(experts.c()), _ptr(y),
                                   _ptr(topk_ids_out), _ptr(topk_w_out), _stream(stream)))


def moe_expert_ffn_share(d, base, count, x, expert_offsets, sorted_pairs, experts, rows, ws, stream=None):
    """moe_expert_ffn for the share [base, base + count) of the experts;
    `experts` holds that share (e.g. ExpertStore.share(base, count))."""
    _check(lib().moe_expert_ffn_share(d, Share(int(base), int(count)), _ptr(x), _ptr(expert_offsets),
                                      _ptr(sorted_pairs), ctypes.byref(experts.c()), _ptr(rows), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_share(d, base, count, x, w_router, bias, experts, y_partial, served, topk_ids_out, topk_w_out, ws,
                    stream=None):
    """moe_layer for one share of the experts: fp32 partial output and the
    records it served (moe.h: moe_layer_share)."""
    _check(lib().moe_layer_share(d, Share(int(base), int(count)), _ptr(x), _ptr(w_router), _ptr(bias),
                                 ctypes.byref(experts.c()), _ptr(y_partial), _ptr(served), _ptr(topk_ids_out),
                                 _ptr(topk_w_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_permute(d, topk_ids, expert_offsets, sorted_pairs, pair_pos, ws, stream=None):
    """Expert-order permutation of caller ids, -1 (any id outside [0, E))
    masked (moe.h: moe_permute)."""
    _check(lib().moe_permute(d, _ptr(topk_ids), _ptr(expert_offsets), _ptr(sorted_pairs), _ptr(pair_pos), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_mapped(d, expert_map, n_local, x, w_router, bias, experts, y_partial, served, topk_ids_out, topk_w_out,
                     local_ids_out, ws, stream=None):
    """The layer's part for the experts one device holds, placed by a global
    -> local map (-1: served elsewhere) (moe.h: moe_layer_mapped)."""
    _check(lib().moe_layer_mapped(d, _ptr(expert_map), int(n_local), _ptr(x), _ptr(w_router), _ptr(bias),
                                  ctypes.byref(experts.c()), _ptr(y_partial), _ptr(served), _ptr(topk_ids_out),
                                  _ptr(topk_w_out), _ptr(local_ids_out), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def moe_layer_shared_workspace_bytes(d, count, I):
    return lib().moe_layer_shared_workspace_bytes(d, ctypes.byref(Shared(int(count), int(I), None, None)))


def moe_layer_shared(d, count, I, w_gate_up, w_down, x, w_router, bias, experts, y, topk_ids_out, topk_w_out, ws,
                     stream=None):
    """moe_layer plus `count` bf16 shared experts of width I (moe.h:
    moe_layer_shared); w_gate_up [H][count*2I], w_down [count*I][H]."""
    sh = Shared(int(count), int(I), _ptr(w_gate_up), _ptr(w_down))
    _check(lib().moe_layer_shared(d, ctypes.byref(sh), _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(experts.c()),
                                  _ptr(y), _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def moe_latent_workspace_bytes(d, H_model):
    return lib().moe_latent_workspace_bytes(d, int(H_model))


def moe_latent_layer(d, H_model, w_down, w_up, x, w_router, bias, experts, y, z_out, topk_ids_out, topk_w_out, ws,
                     stream=None):
    """The latent routed-expert block: x [T][H_model] -> y [T][H_model], with
    the experts on the routed latent of width d.H (moe.h: moe_latent_layer)."""
    lat = Latent(int(H_model), _ptr(w_down), _ptr(w_up))
    _check(lib().moe_latent_layer(d, ctypes.byref(lat), _ptr(x), _ptr(w_router), _ptr(bias), ctypes.byref(experts.c()),
                                  _ptr(y), _ptr(z_out), _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)))


def moe_profile_arm(kernel, n_pairs):
    """Arm timing of the next n_pairs launches of one kernel (name or id) on
    this thread; the library records its own events on the launch stream."""
    kid = KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    _check(lib().moe_profile_arm(kid, int(n_pairs)))


def moe_stream_read(buf, sink, stream=None):
    """Enqueue one streaming read of every byte of the device tensor buf;
    per-block XOR words go to sink (a device tensor of at least
    STREAM_SINK_WORDS 32-bit words)."""
    if sink.numel() * sink.element_size() < STREAM_SINK_WORDS * 4:
        raise ValueError("sink holds fewer than STREAM_SINK_WORDS words")
    _check(lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))


def moe_mfma_rate(iters, sink, stream=None):
    """Enqueue the matrix-core calibration kernel: iters * MFMA_RATE_FLOPS_PER_ITER
    flops; per-block checksums to sink (a device tensor of at least
    MFMA_RATE_BLOCKS fp32 values)."""
    if sink.numel() * sink.element_size() < MFMA_RATE_BLOCKS * 4:
        raise ValueError("sink holds fewer than MFMA_RATE_BLOCKS words")
    _check(lib().moe_mfma_rate(int(iters), _ptr(sink), _stream(stream)))


def moe_profile_read(max_launches):
    """Durations (ms) of the launches recorded since moe_profile_arm; disarms."""
    buf = (ctypes.c_float * max(1, int(max_launches)))()
    n = lib().moe_profile_read(buf, int(max_launches))
    if n < 0:
        _check(-n)
    return [float(buf[i]) for i in range(n)]


# ---- device memory holders (plumbing) ------------------------------------------

class ExpertStore:
    """Weights of E experts, stacked per matrix, resident in HBM: q
    [E][N][K/2] u8, sf [E][N][K/16] (NVFP4) or [E][N][K/32] (MXFP4) u8, gs [E]
    fp32 for gate/up (N = I, K = H) and down (N = H, K = I)."""

    MATS = ("gate", "up", "down")

    def __init__(self, E, H, I, device="cuda", fmt="nvfp4"):
        import torch
        self.E, self.H, self.I = E, H, I
        self.format = FORMATS[fmt]
        blk = 32 if self.format == FORMATS["mxfp4"] else 16
        self.t = {}
        for m in self.MATS:
            N, K = self.shape(m)
            self.t[m] = (torch.empty((E, N, K // 2), dtype=torch.uint8, device=device),
                         torch.empty((E, N, K // blk), dtype=torch.uint8, device=device),
                         torch.empty((E,), dtype=torch.float32, device=device))
        self._qws = torch.empty(max(256, moe_quantize_workspace_bytes()), dtype=torch.uint8, device=device)

    def shape(self, m):
        return (self.I, self.H) if m in ("gate", "up") else (self.H, self.I)

    def quantize_into(self, e, m, w_f32, stream=None):
        """Quantise fp32 w [N][K] (device) into expert e in the store's format."""
        q, sf, gs = self.t[m]
        quant = moe_quantize_mxfp4 if self.format == FORMATS["mxfp4"] else moe_quantize_nvfp4
        quant(w_f32, q[e], sf[e], gs[e:e + 1], self._qws, stream)

    def c(self):
        mats = []
        for m in self.MATS:
            q, sf, gs = self.t[m]
            mats.append(NVFP4(q.data_ptr(), sf.data_ptr(), gs.data_ptr()))
        self._c = Experts(*mats, self.format)
        return self._c

    def share(self, base, count):
        """The store of experts base .. base+count-1 alone (entry i = expert
        base + i): views into this store, as one device's share would hold."""
        return _StoreShare(self, base, count)

    def nbytes_per_expert(self):
        return sum(q[0].numel() + sf[0].numel() + 4 for q, sf, _ in self.t.values())


class _StoreShare:
    def __init__(self, store, base, count):
        if base < 0 or count < 1 or base + count > store.E:
            raise ValueError("share outside the store")
        self.store, self.base, self.count = store, base, count

    def c(self):
        mats = []
        for m in ExpertStore.MATS:
            q, sf, gs = self.store.t[m]
            mats.append(NVFP4(q[self.base].data_ptr(), sf[self.base].data_ptr(), gs[self.base:].data_ptr()))
        self._c = Experts(*mats, self.store.format)
        return self._c
