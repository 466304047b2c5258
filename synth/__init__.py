"""Seeded synthetic inputs for the MoE layer, shared by the oracle tests and
the GPU path.  Holds only input generation (no routing, quantisation or FFN
arithmetic).  The CPU functions return numpy arrays; the GPU functions fill
caller-provided torch CUDA tensors.  Both give bit-identical values."""
import ctypes
import os

import numpy as np

from .build import LIB_CPU, LIB_CPU_SAN, LIB_GPU, build_cpu, sanitize_requested

HERE = os.path.dirname(os.path.abspath(__file__))
_cpu = None
_gpu = None
_p = ctypes.c_void_p
_u64 = ctypes.c_uint64
_i64 = ctypes.c_int64
_i = ctypes.c_int
_f = ctypes.c_float

WEIGHT_STD = 0.02  # N(0, 0.02) router and expert weights (std 0.02)


def cpu():
    global _cpu
    if _cpu is None:
        src = os.path.join(HERE, "synth.c")
        hdr = os.path.join(HERE, "synth_def.h")
        path = LIB_CPU_SAN if sanitize_requested() else LIB_CPU
        if not os.path.exists(path) or os.path.getmtime(path) < max(os.path.getmtime(src), os.path.getmtime(hdr)):
            build_cpu()
        L = ctypes.CDLL(path)
        L.synth_x_bf16.argtypes = [_u64, _i64, _i, _i, _p]
        L.synth_router_bf16.argtypes = [_u64, _i, _i, _f, _p]
        L.synth_expert_f32.argtypes = [_u64, _i, _i, _i, _i, _f, _p, _i]
        L.synth_proj_bf16.argtypes = [_u64, _i, _i, _i, _f, _p]
        L.synth_zipf_bias.argtypes = [_u64, _i, ctypes.c_double, ctypes.c_double, _p]
        L.synth_popularity_perm.argtypes = [_u64, _i, _p]
        L.synth_normals_f32.argtypes = [_u64, _u64, _u64, _i64, _p]
        L.synth_round_bf16.argtypes = [_p, _i64, _p]
        for f in (L.synth_x_bf16, L.synth_router_bf16, L.synth_expert_f32, L.synth_proj_bf16, L.synth_zipf_bias,
                  L.synth_popularity_perm,
                  L.synth_normals_f32, L.synth_round_bf16):
            f.restype = None
        _cpu = L
    return _cpu


def gpu():
    global _gpu
    if _gpu is None:
        if not os.path.exists(LIB_GPU):
            raise RuntimeError(f"{LIB_GPU} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_GPU)
        L.synth_gpu_x_bf16.argtypes = [_u64, _i64, _i, _i, _p, _p]
        L.synth_gpu_router_bf16.argtypes = [_u64, _i, _i, _f, _p, _p]
        L.synth_gpu_expert_f32.argtypes = [_u64, _i, _i, _i, _i, _f, _p, _p]
        L.synth_gpu_proj_bf16.argtypes = [_u64, _i, _i, _i, _f, _p, _p]
        for f in (L.synth_gpu_x_bf16, L.synth_gpu_router_bf16, L.synth_gpu_expert_f32, L.synth_gpu_proj_bf16):
            f.restype = ctypes.c_int
        _gpu = L
    return _gpu


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---- CPU -------------------------------------------------------------------

def x_bf16(seed, T, H, t0=0):
    out = np.empty((T, H), np.uint16)
    cpu().synth_x_bf16(seed, t0, T, H, _ptr(out))
    return out


def router_bf16(seed, H, E, std=WEIGHT_STD):
    out = np.empty((H, E), np.uint16)
    cpu().synth_router_bf16(seed, H, E, std, _ptr(out))
    return out


def expert_f32(seed, e, m, N, K, std=WEIGHT_STD, nthreads=None):
    """fp32 weights of expert e, matrix m (0 gate, 1 up, 2 down), logical [N][K]."""
    out = np.empty((N, K), np.float32)
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    cpu().synth_expert_f32(seed, e, m, N, K, std, _ptr(out), nthreads)
    return out


def proj_bf16(seed, which, K, N, std=WEIGHT_STD):
    """Dense bf16 weights [K][N] (bits): which 0 = latent routed-down
    ([H_model][H]), 1 = routed-up ([H][H_model]), 2 = shared experts'
    gate/up ([H][count*2I]), 3 = their down ([count*I][H])."""
    out = np.empty((K, N), np.uint16)
    cpu().synth_proj_bf16(seed, which, K, N, std, _ptr(out))
    return out


def expert_shape(m, H, I):
    return (I, H) if m < 2 else (H, I)


def zipf_bias(seed, E, beta, s=1.1):
    out = np.empty(E, np.float32)
    cpu().synth_zipf_bias(seed, E, beta, s, _ptr(out))
    return out


def popularity_perm(seed, E):
    out = np.empty(E, np.int32)
    cpu().synth_popularity_perm(seed, E, _ptr(out))
    return out


def normals_f32(seed, stream, first, n):
    out = np.empty(n, np.float32)
    cpu().synth_normals_f32(seed, stream, first, n, _ptr(out))
    return out


def round_bf16(a):
    a = np.ascontiguousarray(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    cpu().synth_round_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_to_f32(a):
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---- GPU (torch CUDA tensors; the stream defaults to torch's current) -----

def _stream(stream):
    import torch
    return (stream or torch.cuda.current_stream()).cuda_stream


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed")


def gpu_x_bf16(seed, out, t0=0, stream=None):
    T, H = out.shape
    assert out.is_cuda and out.is_contiguous() and out.element_size() == 2
    _check(gpu().synth_gpu_x_bf16(seed, t0, T, H, out.data_ptr(), _stream(stream)), "synth_gpu_x_bf16")


def gpu_router_bf16(seed, out, std=WEIGHT_STD, stream=None):
    H, E = out.shape
    assert out.is_cuda and out.is_contiguous() and out.element_size() == 2
    _check(gpu().synth_gpu_router_bf16(seed, H, E, std, out.data_ptr(), _stream(stream)), "synth_gpu_router_bf16")


def gpu_proj_bf16(seed, which, out, std=WEIGHT_STD, stream=None):
    K, N = out.shape
    assert out.is_cuda and out.is_contiguous() and out.element_size() == 2
    _check(gpu().synth_gpu_proj_bf16(seed, which, K, N, std, out.data_ptr(), _stream(stream)), "synth_gpu_proj_bf16")


def gpu_expert_f32(seed, e, m, out, std=WEIGHT_STD, stream=None):
    N, K = out.shape
    assert out.is_cuda and out.is_contiguous() and out.element_size() == 4
    _check(gpu().synth_gpu_expert_f32(seed, e, m, N, K, std, out.data_ptr(), _stream(stream)), "synth_gpu_expert_f32")
