"""online_softmax_06_amd: online softmax and fused attention forward on MI355X.

A thin Python layer over ``libosm.so`` (C ABI in ``include/osm.h``).  It only
marshals arguments: every step of the computation runs in the library's HIP
kernels.  torch is used for device memory and for the current HIP stream.

Raw entry points, same names and arguments as the C ABI (device pointers as
ints; ``stream`` is a hipStream_t handle, 0 for the null stream):

    osm_softmax_rows(in_ptr, out_ptr, rows, cols, dtype, stream) -> status
    osm_attn_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, stream) -> status
    osm_status_string(status) -> str

Tensor-level helpers:

    softmax_rows(x, out=None) -> Tensor
    attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None) -> (o, lse)

If the library has not been built, every call raises ``RuntimeError``; there
is no fallback implementation.
"""

import ctypes
import math
import os

__all__ = [
    "OSM_F32", "OSM_BF16", "OSM_OK", "OSM_ERR_INVALID_ARG", "OSM_ERR_UNSUPPORTED", "OSM_ERR_HIP",
    "OsmError", "lib_path", "load_library", "osm_softmax_rows", "osm_attn_fwd",
    "osm_status_string", "osm_version", "softmax_rows", "attn_fwd",
]

OSM_F32, OSM_BF16 = 0, 1
OSM_OK, OSM_ERR_INVALID_ARG, OSM_ERR_UNSUPPORTED, OSM_ERR_HIP = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class OsmError(RuntimeError):
    """A libosm call returned a nonzero status."""

    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {osm_status_string(status)} (status {status})")


def lib_path():
    return os.path.join(_HERE, "libosm.so")


def load_library():
    """Load libosm.so once; raise RuntimeError if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m online_softmax_06_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    c_vp, c_i64, c_int, c_f = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.osm_softmax_rows.argtypes = [c_vp, c_vp, c_i64, c_i64, c_int, c_vp]
    lib.osm_softmax_rows.restype = c_int
    lib.osm_attn_fwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_f,
                                 c_int, c_vp]
    lib.osm_attn_fwd.restype = c_int
    lib.osm_status_string.argtypes = [c_int]
    lib.osm_status_string.restype = ctypes.c_char_p
    lib.osm_version.argtypes = []
    lib.osm_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


# ---------------------------------------------------------------------------
# Raw C-ABI wrappers.
# ---------------------------------------------------------------------------

def osm_softmax_rows(in_ptr, out_ptr, rows, cols, dtype, stream=0):
    return load_library().osm_softmax_rows(in_ptr, out_ptr, rows, cols, dtype, stream)


def osm_attn_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, stream=0):
    return load_library().osm_attn_fwd(q, k, v, o, lse, B, H, N, D, scale, int(causal), stream)


def osm_status_string(status):
    return load_library().osm_status_string(status).decode()


def osm_version():
    return load_library().osm_version().decode()


# ---------------------------------------------------------------------------
# Tensor-level helpers.
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(dtype):
    torch = _torch()
    if dtype == torch.float32:
        return OSM_F32
    if dtype == torch.bfloat16:
        return OSM_BF16
    raise TypeError(f"softmax_rows supports float32 and bfloat16, not {dtype}")


def softmax_rows(x, out=None):
    """Softmax over the last dimension of a contiguous CUDA tensor.

    ``x`` is viewed as [rows, cols] with cols = x.shape[-1].  ``out`` may be
    ``x`` itself (in place) or a new tensor of the same shape and dtype.
    """
    torch = _torch()
    if not x.is_cuda:
        raise ValueError("softmax_rows needs a GPU tensor")
    if not x.is_contiguous():
        raise ValueError("softmax_rows needs a contiguous tensor")
    code = _dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() \
            or out.device != x.device:
        raise ValueError("out must be a contiguous tensor of the same shape, dtype and device")
    cols = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // cols if cols else 0
    st = osm_softmax_rows(x.data_ptr(), out.data_ptr(), rows, cols, code, _stream_handle(x.device))
    if st != OSM_OK:
        raise OsmError(st, "osm_softmax_rows")
    return out


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None):
    """Fused attention forward on contiguous bfloat16 [B, H, N, D] CUDA tensors.

    Returns ``(o, lse)``: o is bfloat16 [B, H, N, D], lse float32 [B, H, N].
    ``scale`` multiplies q.k and defaults to 1/sqrt(D).
    """
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or t.dim() != 4:
            raise ValueError(f"{name} must be a contiguous bfloat16 CUDA tensor [B, H, N, D]")
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must have the same shape [B, H, N, D]")
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, H, N]")
    st = osm_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, N, D, float(scale), bool(causal), _stream_handle(q.device))
    if st != OSM_OK:
        raise OsmError(st, "osm_attn_fwd")
    return out, lse
