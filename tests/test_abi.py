"""The C ABI boundary on the host: libmoe.so loads and exports every entry
point include/moe.h declares, and argument validation rejects bad calls
before anything reaches the GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import routed_expert_ffn_amd as moe
from synth.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(moe_[a-z_0-9]+)\s*\(", text, flags=re.M))


def test_exports_match_header():
    decl = declared_functions()
    assert decl == set(moe.EXPORTS), decl ^ set(moe.EXPORTS)
    L = ctypes.CDLL(moe.LIB_PATH)
    for name in decl:
        assert hasattr(L, name), name


def test_constants_match_header():
    text = open(HEADER).read()
    enum = dict((n.lower(), int(v)) for n, v in re.findall(r"MOE_KERNEL_([A-Z]+) = (\d+)", text))
    enum.pop("count")
    assert enum == moe.KERNELS


def test_workspace_sizes():
    for wl in WORKLOADS.values():
        d = moe.dims(wl.T, wl.H, wl.I, wl.E, wl.k)
        n = moe.moe_workspace_bytes(d)
        # at least the per-pair rows, h and the fp16 copy of x
        assert n >= wl.P * wl.H * 4 + wl.P * wl.I * 2 + wl.T * wl.H * 2
        assert n % 256 == 0
    assert moe.moe_workspace_bytes(moe.dims(1, 7168, 2048, 896, 0)) == 0
    assert moe.moe_quantize_workspace_bytes() >= 4


FAKE = 1 << 20  # aligned, never dereferenced: validation fails first


def _route(d, **kw):
    a = dict(x=FAKE, wr=FAKE, bias=None, logits=FAKE, ids=FAKE, w=FAKE, off=FAKE, sp=FAKE, pp=FAKE, ws=FAKE,
             ws_bytes=moe.moe_workspace_bytes(d) if moe.moe_workspace_bytes(d) else 1 << 30)
    a.update(kw)
    return moe.lib().moe_route(d, a["x"], a["wr"], a["bias"], a["logits"], a["ids"], a["w"], a["off"], a["sp"],
                               a["pp"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("T,H,I,E,k", [(-1, 512, 256, 896, 16), (8, 500, 256, 896, 16), (8, 512, 200, 896, 16),
                                       (8, 512, 256, 896, 0), (8, 512, 256, 896, 65), (8, 512, 256, 12, 16),
                                       (8, 512, 256, 2048, 16), (8, 512, 256, 900, 16), (1 << 27, 512, 256, 896, 16)])
def test_bad_shapes_rejected(T, H, I, E, k):
    d = moe.dims(T, H, I, E, k)
    assert _route(d) == 2  # MOE_ERR_SHAPE
    assert moe.lib().moe_last_error()


def test_bad_pointers_and_workspace_rejected():
    d = moe.dims(8, 512, 256, 896, 16)
    assert _route(d, logits=None) == 1          # MOE_ERR_ARG
    assert _route(d, ids=FAKE + 4) == 3         # MOE_ERR_ALIGN
    assert _route(d, ws_bytes=1024) == 4        # MOE_ERR_WORKSPACE
    assert b"workspace" in moe.lib().moe_last_error()
    assert _route(d, ws=None) == 1
    # x == NULL is the logits-in mode, router weights may then be NULL too
    assert _route(moe.dims(8, 512, 256, 896, 16), x=None, wr=None, logits=None) == 1


def test_layer_and_ffn_validation():
    d = moe.dims(8, 512, 256, 896, 16)
    ex = moe.Experts(moe.NVFP4(FAKE, FAKE, FAKE), moe.NVFP4(FAKE, FAKE, FAKE), moe.NVFP4(FAKE, None, FAKE))
    big = moe.moe_workspace_bytes(d)
    L = moe.lib()
    assert L.moe_layer(d, FAKE, FAKE, None, ctypes.byref(ex), FAKE, None, None, FAKE, big, None) == 1
    ex.down.sf = FAKE + 8
    assert L.moe_layer(d, FAKE, FAKE, None, ctypes.byref(ex), FAKE, None, None, FAKE, big, None) == 3
    assert L.moe_layer(d, FAKE, FAKE, None, None, FAKE, None, None, FAKE, big, None) == 1
    assert L.moe_expert_ffn(d, FAKE, FAKE, FAKE, None, FAKE, FAKE, big, None) == 1
    assert L.moe_quantize_nvfp4(FAKE, 4, 24, FAKE, FAKE, FAKE, FAKE, 256, None) == 2
    assert L.moe_quantize_nvfp4(FAKE, 4, 32, FAKE, FAKE, FAKE, FAKE, 2, None) == 4


def test_t_zero_is_ok_without_touching_anything():
    d = moe.dims(0, 512, 256, 896, 16)
    assert moe.lib().moe_layer(d, None, None, None, None, None, None, None, None, 0, None) == 0
    assert _route(d, x=None, logits=None) == 0


def test_status_strings_and_errors():
    L = moe.lib()
    for s in range(6):
        assert L.moe_status_string(s)
    with pytest.raises(moe.MoeError):
        moe._check(2)


def test_profile_arguments_rejected_without_hip():
    """Out-of-range kernel ids and counts are refused before any event is
    created; reading into NULL reports -MOE_ERR_ARG."""
    L = moe.lib()
    assert L.moe_profile_arm(-1, 4) == 1
    assert L.moe_profile_arm(len(moe.KERNELS), 4) == 1
    assert L.moe_profile_arm(4, 0) == 1
    assert L.moe_profile_arm(4, 65537) == 1
    assert L.moe_profile_read(None, 4) == -1
    assert L.moe_profile_read((ctypes.c_float * 1)(), -1) == -1
    assert L.moe_profile_read((ctypes.c_float * 1)(), 1) == 0  # nothing armed: nothing recorded


def test_stream_read_arguments_rejected_without_hip():
    """The HBM read calibration refuses NULL pointers, sizes that are not
    positive multiples of 16 and misaligned pointers before any launch."""
    L = moe.lib()
    assert L.moe_stream_read(None, 4096, 4096, None) == 1
    assert L.moe_stream_read(4096, 4096, None, None) == 1
    assert L.moe_stream_read(4096, 0, 4096, None) == 1
    assert L.moe_stream_read(4096, 4100, 4096, None) == 1
    assert L.moe_stream_read(4104, 4096, 4096, None) == 3
    assert L.moe_stream_read(4096, 4096, 4098, None) == 3
    assert int(re.search(r"#define MOE_STREAM_SINK_WORDS (\d+)", open(HEADER).read()).group(1)) == moe.STREAM_SINK_WORDS


def test_latent_workspace_and_validation_without_hip():
    """The latent block's workspace covers the plain layer's, and bad widths
    or NULL projections are refused before any launch."""
    d = moe.dims(8, 3584, 3072, 896, 16)
    assert moe.moe_latent_workspace_bytes(d, 7168) > moe.moe_workspace_bytes(d)
    assert moe.moe_latent_workspace_bytes(d, 7000) == 0
    assert moe.moe_latent_workspace_bytes(d, 0) == 0
    L = moe.lib()
    ex = moe.Experts()
    lat = moe.Latent(7168, None, None)
    args = (ctypes.byref(ex), 4096, 4096, None, None, None, 4096, 1 << 40, None)
    assert L.moe_latent_layer(d, None, 4096, 4096, None, *args) == 1
    assert L.moe_latent_layer(d, ctypes.byref(lat), 4096, 4096, None, *args) == 1
    bad = moe.Latent(100, 4096, 4096)
    assert L.moe_latent_layer(d, ctypes.byref(bad), 4096, 4096, None, *args) == 2


def test_share_validation_without_hip():
    """Shares that are empty or leave [0, E) are refused before any launch."""
    L = moe.lib()
    d = moe.dims(8, 512, 256, 64, 8)
    ex = moe.Experts()
    ws_bytes = moe.moe_workspace_bytes(d)
    for base, count in [(-1, 4), (0, 0), (60, 8), (64, 1)]:
        sh = moe.Share(base, count)
        assert L.moe_layer_share(d, sh, FAKE, FAKE, None, ctypes.byref(ex), FAKE, None, None, None, FAKE, ws_bytes,
                                 None) == 2
        assert L.moe_expert_ffn_share(d, sh, FAKE, FAKE, FAKE, ctypes.byref(ex), FAKE, FAKE, ws_bytes, None) == 2


def test_shared_workspace_and_validation_without_hip():
    d = moe.dims(8, 512, 256, 64, 8)
    assert moe.moe_layer_shared_workspace_bytes(d, 2, 256) > moe.moe_workspace_bytes(d)
    assert moe.moe_layer_shared_workspace_bytes(d, 0, 256) == 0
    assert moe.moe_layer_shared_workspace_bytes(d, 2, 100) == 0
    L = moe.lib()
    ex = moe.Experts()
    args = (FAKE, FAKE, None, ctypes.byref(ex), FAKE, None, None, FAKE, 1 << 40, None)
    assert L.moe_layer_shared(d, None, *args) == 1
    assert L.moe_layer_shared(d, ctypes.byref(moe.Shared(2, 256, None, None)), *args) == 1
    assert L.moe_layer_shared(d, ctypes.byref(moe.Shared(2, 300, FAKE, FAKE)), *args) == 2


def test_mxfp4_quantize_and_format_validation_without_hip():
    L = moe.lib()
    ws = moe.moe_quantize_workspace_bytes()
    assert L.moe_quantize_mxfp4(FAKE, 4, 48, FAKE, FAKE, FAKE, FAKE, ws, None) == 2  # K % 32
    assert L.moe_quantize_mxfp4(FAKE, 0, 64, FAKE, FAKE, FAKE, FAKE, ws, None) == 2
    d = moe.dims(8, 512, 256, 64, 8)
    nv = moe.NVFP4(FAKE, FAKE, FAKE)
    ex = moe.Experts(nv, nv, nv, 5)
    rows_ws = moe.moe_workspace_bytes(d)
    assert L.moe_expert_ffn(d, FAKE, FAKE, FAKE, ctypes.byref(ex), FAKE, FAKE, rows_ws, None) == 1


def test_permute_and_mapped_validation_without_hip():
    """moe_permute and moe_layer_mapped refuse bad arguments before any
    launch; T = 0 is a no-op."""
    L = moe.lib()
    d = moe.dims(8, 512, 256, 64, 8)
    ws_bytes = moe.moe_workspace_bytes(d)
    assert L.moe_permute(d, None, FAKE, FAKE, FAKE, FAKE, ws_bytes, None) == 1
    assert L.moe_permute(d, FAKE + 4, FAKE, FAKE, FAKE, FAKE, ws_bytes, None) == 3
    assert L.moe_permute(d, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes - 256, None) == 4
    assert L.moe_permute(moe.dims(8, 512, 256, 64, 0), FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None) == 2
    assert L.moe_permute(moe.dims(0, 512, 256, 64, 8), None, None, None, None, None, 0, None) == 0
    ex = moe.Experts()
    for n_local in (0, -1, 65):
        assert L.moe_layer_mapped(d, FAKE, n_local, FAKE, FAKE, None, ctypes.byref(ex), FAKE, None, None, None, None,
                                  FAKE, ws_bytes, None) == 2
    assert L.moe_layer_mapped(d, None, 4, FAKE, FAKE, None, ctypes.byref(ex), FAKE, None, None, None, None, FAKE,
                              ws_bytes, None) == 1


def test_noalloc_limit_without_hip():
    """moe_layer_noalloc refuses, before any HIP call, a batch whose
    workspace exceeds the library's scratch (T = 157 at the full shape)."""
    L = moe.lib()
    nv = moe.NVFP4(FAKE, FAKE, FAKE)
    ex = moe.Experts(nv, nv, nv, 0)
    assert L.moe_layer_noalloc(moe.dims(157, 7168, 2048, 896, 16), FAKE, FAKE, None, ctypes.byref(ex), FAKE, None,
                               None, None) == 4
    assert L.moe_layer_noalloc(moe.dims(8, 500, 256, 896, 16), FAKE, FAKE, None, ctypes.byref(ex), FAKE, None,
                               None, None) == 2
    assert L.moe_layer_noalloc(moe.dims(8, 512, 256, 896, 16), None, FAKE, None, ctypes.byref(ex), FAKE, None,
                               None, None) == 1
    assert moe.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_token_bounds_without_hip():
    """T above 65535, or T * max(H, k*I) at 2^31 or more, is refused (the
    grids and the large-tile GEMMs' 32-bit row offsets); just below is
    accepted."""
    assert moe.moe_workspace_bytes(moe.dims(65536, 512, 256, 896, 16)) == 0
    assert moe.moe_workspace_bytes(moe.dims(65535, 512, 256, 896, 16)) > 0
    assert moe.moe_workspace_bytes(moe.dims(16384, 512, 2048, 1024, 64)) == 0  # 16384 * 131072 = 2^31
    assert moe.moe_workspace_bytes(moe.dims(16383, 512, 2048, 1024, 64)) > 0
    d = moe.dims(16384, 512, 2048, 1024, 64)
    assert _route(d, ws_bytes=1 << 40) == 2


def test_mfma_rate_validation_without_hip():
    L = moe.lib()
    assert L.moe_mfma_rate(100, None, None) == 1
    assert L.moe_mfma_rate(0, FAKE, None) == 1
    assert L.moe_mfma_rate(10 ** 7 + 1, FAKE, None) == 1
    assert L.moe_mfma_rate(100, FAKE + 2, None) == 3
