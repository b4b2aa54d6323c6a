"""online_softmax_06_amd: online softmax and fused attention forward on MI355X.

A thin Python layer over ``libosm.so`` (C ABI in ``include/osm.h``).  It only
marshals arguments: every step of the computation runs in the library's HIP
kernels.  torch is used for device memory and for the current HIP stream.

Raw entry points, same names and arguments as the C ABI (device pointers as
ints; ``stream`` is a hipStream_t handle, 0 for the null stream):

    osm_softmax_rows(in_ptr, out_ptr, rows, cols, dtype, stream) -> status
    osm_softmax_rows_ex(in_ptr, out_ptr, rows, cols, dtype, mask, mask_rows,
                        row_len, stream) -> status
    osm_softmax_rows_split(in_ptr, out_ptr, rows, cols, dtype, mask, mask_rows,
                           row_len, workspace, workspace_bytes, stream) -> status
    osm_softmax_rows_split_workspace(rows, cols) -> bytes
    osm_attn_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, stream) -> status
    osm_attn_fwd_ex(q, k, v, o, lse, B, H, N, D, scale, causal, kv_len, bias,
                    bias_stride_b, bias_stride_h, stream) -> status
    osm_attn_fwd_split(q, k, v, o, lse, B, H, N, D, scale, causal, kv_len, bias,
                       bias_stride_b, bias_stride_h, splits, workspace,
                       workspace_bytes, stream) -> status
    osm_attn_fwd_split_workspace(B, H, N, D, splits) -> bytes
    osm_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale, causal,
                 workspace, workspace_bytes, stream) -> status
    osm_attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale,
                    causal, kv_len, workspace, workspace_bytes, stream) -> status
    osm_attn_bwd_workspace(B, H, N, D) -> bytes
    osm_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale,
                         causal, kv_len, stream) -> status
    osm_stream_copy(src, dst, bytes, stream) -> status   (bandwidth ceiling probe)
    osm_status_string(status) -> str

Tensor-level helpers:

    softmax_rows(x, out=None, mask=None, row_len=None, split=False) -> Tensor
    attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None,
             kv_len=None, bias=None, splits=1) -> (o, lse)
    attn_bwd(q, k, v, o, lse, dout, scale=None, causal=False, kv_len=None)
             -> (dq, dk, dv)

If the library has not been built, every call raises ``RuntimeError``; there
is no fallback implementation.
"""

import ctypes
import math
import os

__all__ = [
    "OSM_F32", "OSM_BF16", "OSM_OK", "OSM_ERR_INVALID_ARG", "OSM_ERR_UNSUPPORTED", "OSM_ERR_HIP",
    "OsmError", "lib_path", "load_library", "osm_softmax_rows", "osm_softmax_rows_ex",
    "osm_softmax_rows_split", "osm_softmax_rows_split_workspace",
    "osm_attn_fwd", "osm_attn_fwd_ex", "osm_attn_fwd_split", "osm_attn_fwd_split_workspace",
    "osm_attn_bwd", "osm_attn_bwd_ex", "osm_attn_bwd_workspace", "osm_attn_bwd_noalloc",
    "OSM_ATTN_BWD_SCRATCH_BYTES", "osm_stream_copy",
    "osm_status_string", "osm_version", "softmax_rows",
    "attn_fwd", "attn_bwd", "check_tensor",
]

OSM_F32, OSM_BF16 = 0, 1
OSM_OK, OSM_ERR_INVALID_ARG, OSM_ERR_UNSUPPORTED, OSM_ERR_HIP = 0, 1, 2, 3
OSM_ATTN_BWD_SCRATCH_BYTES = 32 << 20  # include/osm.h

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
    lib.osm_softmax_rows_ex.argtypes = [c_vp, c_vp, c_i64, c_i64, c_int, c_vp, c_i64, c_vp, c_vp]
    lib.osm_softmax_rows_ex.restype = c_int
    lib.osm_softmax_rows_split.argtypes = [c_vp, c_vp, c_i64, c_i64, c_int, c_vp, c_i64, c_vp,
                                           c_vp, c_i64, c_vp]
    lib.osm_softmax_rows_split.restype = c_int
    lib.osm_softmax_rows_split_workspace.argtypes = [c_i64, c_i64]
    lib.osm_softmax_rows_split_workspace.restype = c_i64
    lib.osm_attn_fwd_ex.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                    c_f, c_int, c_vp, c_vp, c_i64, c_i64, c_vp]
    lib.osm_attn_fwd_ex.restype = c_int
    lib.osm_attn_fwd_split.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int,
                                       c_f, c_int, c_vp, c_vp, c_i64, c_i64, c_int, c_vp, c_i64,
                                       c_vp]
    lib.osm_attn_fwd_split.restype = c_int
    lib.osm_attn_fwd_split_workspace.argtypes = [c_int, c_int, c_int, c_int, c_int]
    lib.osm_attn_fwd_split_workspace.restype = c_i64
    lib.osm_attn_fwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_int, c_int, c_int, c_int, c_f,
                                 c_int, c_vp]
    lib.osm_attn_fwd.restype = c_int
    lib.osm_attn_bwd.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int,
                                 c_int, c_int, c_int, c_f, c_int, c_vp, c_i64, c_vp]
    lib.osm_attn_bwd.restype = c_int
    lib.osm_attn_bwd_ex.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_int,
                                    c_int, c_int, c_int, c_f, c_int, c_vp, c_vp, c_i64, c_vp]
    lib.osm_attn_bwd_ex.restype = c_int
    lib.osm_attn_bwd_noalloc.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                         c_int, c_int, c_int, c_int, c_f, c_int, c_vp, c_vp]
    lib.osm_attn_bwd_noalloc.restype = c_int
    lib.osm_attn_bwd_workspace.argtypes = [c_int, c_int, c_int, c_int]
    lib.osm_attn_bwd_workspace.restype = c_i64
    lib.osm_stream_copy.argtypes = [c_vp, c_vp, c_i64, c_vp]
    lib.osm_stream_copy.restype = c_int
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


def osm_softmax_rows_ex(in_ptr, out_ptr, rows, cols, dtype, mask=0, mask_rows=0, row_len=0,
                        stream=0):
    return load_library().osm_softmax_rows_ex(in_ptr, out_ptr, rows, cols, dtype, mask or None,
                                              mask_rows, row_len or None, stream)


def osm_softmax_rows_split(in_ptr, out_ptr, rows, cols, dtype, mask, mask_rows, row_len,
                           workspace, workspace_bytes, stream=0):
    return load_library().osm_softmax_rows_split(in_ptr, out_ptr, rows, cols, dtype,
                                                 mask or None, mask_rows, row_len or None,
                                                 workspace or None, workspace_bytes, stream)


def osm_softmax_rows_split_workspace(rows, cols):
    return load_library().osm_softmax_rows_split_workspace(rows, cols)


def osm_attn_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, stream=0):
    return load_library().osm_attn_fwd(q, k, v, o, lse, B, H, N, D, scale, int(causal), stream)


def osm_attn_fwd_ex(q, k, v, o, lse, B, H, N, D, scale, causal, kv_len=0, bias=0,
                    bias_stride_b=0, bias_stride_h=0, stream=0):
    return load_library().osm_attn_fwd_ex(q, k, v, o, lse, B, H, N, D, scale, int(causal),
                                          kv_len or None, bias or None, bias_stride_b,
                                          bias_stride_h, stream)


def osm_attn_fwd_split(q, k, v, o, lse, B, H, N, D, scale, causal, kv_len, bias, bias_stride_b,
                       bias_stride_h, splits, workspace, workspace_bytes, stream=0):
    return load_library().osm_attn_fwd_split(q, k, v, o, lse, B, H, N, D, scale, int(causal),
                                             kv_len or None, bias or None, bias_stride_b,
                                             bias_stride_h, splits, workspace or None,
                                             workspace_bytes, stream)


def osm_attn_fwd_split_workspace(B, H, N, D, splits):
    return load_library().osm_attn_fwd_split_workspace(B, H, N, D, splits)


def osm_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale, causal, workspace,
                 workspace_bytes, stream=0):
    return load_library().osm_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale,
                                       int(causal), workspace, workspace_bytes, stream)


def osm_attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale, causal, kv_len,
                    workspace, workspace_bytes, stream=0):
    return load_library().osm_attn_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale,
                                          int(causal), kv_len, workspace, workspace_bytes, stream)


def osm_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, scale, causal,
                         kv_len=0, stream=0):
    return load_library().osm_attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D,
                                               scale, int(causal), kv_len or None, stream)


def osm_attn_bwd_workspace(B, H, N, D):
    return load_library().osm_attn_bwd_workspace(B, H, N, D)


def osm_stream_copy(src, dst, nbytes, stream=0):
    return load_library().osm_stream_copy(src, dst, nbytes, stream)


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


def check_tensor(t, name, device, dtype, shape=None):
    """Raise ValueError unless ``t`` is a contiguous tensor of ``dtype`` on
    ``device`` (and of ``shape``, when given).

    Every tensor a helper hands to the library goes through this check before
    any launch: a kernel storing through a pointer that is not memory of the
    launching device would fault the GPU.
    """
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, not {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, not {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _gpu_device(t, name):
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a GPU tensor")
    return t.device


def softmax_rows(x, out=None, mask=None, row_len=None, split=False):
    """Softmax over the last dimension of a contiguous CUDA tensor.

    ``x`` is viewed as [rows, cols] with cols = x.shape[-1].  ``out`` may be
    ``x`` itself (in place) or a new tensor of the same shape and dtype.
    ``mask`` (same dtype, contiguous, viewed as [mask_rows, cols]; row r uses
    mask row r % mask_rows) is added to the logits; ``row_len`` (int32 CUDA
    tensor of length rows) limits each row, the rest of the row becoming 0.
    ``split=True`` uses the split-row kernels (a workspace is allocated here,
    through torch's caching allocator).
    """
    torch = _torch()
    dev = _gpu_device(x, "x")
    code = _dtype_code(x.dtype)
    check_tensor(x, "x", dev, x.dtype)
    if out is None:
        out = torch.empty_like(x)
    check_tensor(out, "out", dev, x.dtype, x.shape)
    cols = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // cols if cols else 0
    mask_ptr, mask_rows, len_ptr = 0, 0, 0
    if mask is not None:
        check_tensor(mask, "mask", dev, x.dtype)
        if mask.dim() == 0 or mask.shape[-1] != cols or mask.numel() == 0:
            raise ValueError("mask must end in the row length and hold at least one row")
        mask_ptr, mask_rows = mask.data_ptr(), mask.numel() // cols
    if row_len is not None:
        check_tensor(row_len, "row_len", dev, torch.int32)
        if row_len.numel() != rows:
            raise ValueError(f"row_len must hold one entry per row ({rows})")
        len_ptr = row_len.data_ptr()
    if split:
        need = osm_softmax_rows_split_workspace(rows, cols)
        ws = torch.empty(max(need, 8), dtype=torch.uint8, device=x.device)
        st = osm_softmax_rows_split(x.data_ptr(), out.data_ptr(), rows, cols, code, mask_ptr,
                                    mask_rows, len_ptr, ws.data_ptr(), ws.numel(),
                                    _stream_handle(x.device))
        if st != OSM_OK:
            raise OsmError(st, "osm_softmax_rows_split")
        return out
    st = osm_softmax_rows_ex(x.data_ptr(), out.data_ptr(), rows, cols, code, mask_ptr, mask_rows,
                             len_ptr, _stream_handle(x.device))
    if st != OSM_OK:
        raise OsmError(st, "osm_softmax_rows_ex")
    return out


def attn_fwd(q, k, v, scale=None, causal=False, out=None, lse=None, kv_len=None, bias=None,
             splits=1):
    """Fused attention forward on contiguous bfloat16 [B, H, N, D] CUDA tensors.

    Returns ``(o, lse)``: o is bfloat16 [B, H, N, D], lse float32 [B, H, N].
    ``scale`` multiplies q.k and defaults to 1/sqrt(D).  ``kv_len`` (int32
    CUDA tensor [B]) hides keys past each batch's length; ``bias`` (float32
    CUDA tensor broadcastable to [B, H, N, N], last two dims contiguous) is
    added to the scaled scores.  ``splits`` > 1 splits every query tile's key
    range over that many workgroups (a workspace is allocated here, through
    torch's caching allocator).
    """
    torch = _torch()
    dev = _gpu_device(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be a [B, H, N, D] tensor")
    for name, t in (("q", q), ("k", k), ("v", v)):
        check_tensor(t, name, dev, torch.bfloat16, q.shape)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    check_tensor(out, "out", dev, torch.bfloat16, q.shape)
    check_tensor(lse, "lse", dev, torch.float32, (B, H, N))
    len_ptr, bias_ptr, sb, sh = 0, 0, 0, 0
    if kv_len is not None:
        check_tensor(kv_len, "kv_len", dev, torch.int32)
        if kv_len.numel() != B:
            raise ValueError(f"kv_len must hold one entry per batch ({B})")
        len_ptr = kv_len.data_ptr()
    if bias is not None:
        if not isinstance(bias, torch.Tensor) or bias.device != dev \
                or bias.dtype != torch.float32 or bias.dim() != 4:
            raise ValueError(f"bias must be a float32 tensor [B or 1, H or 1, N, N] on {dev}")
        bb = bias.expand(B, H, N, N)
        if bb.stride(3) != 1 or bb.stride(2) != N:
            raise ValueError("bias must have contiguous [N, N] trailing dims")
        bias_ptr, sb, sh = bb.data_ptr(), bb.stride(0), bb.stride(1)
    if splits > 1:
        need = osm_attn_fwd_split_workspace(B, H, N, D, splits)
        if need < 0:
            raise OsmError(OSM_ERR_INVALID_ARG, "osm_attn_fwd_split_workspace")
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
        st = osm_attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                lse.data_ptr(), B, H, N, D, float(scale), bool(causal), len_ptr,
                                bias_ptr, sb, sh, splits, ws.data_ptr(), ws.numel(),
                                _stream_handle(q.device))
        if st != OSM_OK:
            raise OsmError(st, "osm_attn_fwd_split")
        return out, lse
    st = osm_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), B, H, N, D, float(scale), bool(causal), len_ptr,
                         bias_ptr, sb, sh, _stream_handle(q.device))
    if st != OSM_OK:
        raise OsmError(st, "osm_attn_fwd_ex")
    return out, lse


def attn_bwd(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, dk=None, dv=None,
             kv_len=None):
    """Attention backward on contiguous bfloat16 [B, H, N, D] CUDA tensors.

    ``o`` and ``lse`` are the forward's outputs for ``q, k, v`` with the same
    ``scale``, ``causal`` and ``kv_len`` (int32 CUDA tensor [B], or None);
    ``dout`` is the gradient of the loss with respect to ``o``.  Returns ``(dq, dk, dv)`` (bfloat16, shaped like q).  The
    workspace is allocated here, through torch's caching allocator.
    """
    torch = _torch()
    dev = _gpu_device(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be a [B, H, N, D] tensor")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        check_tensor(t, name, dev, torch.bfloat16, q.shape)
    B, H, N, D = q.shape
    check_tensor(lse, "lse", dev, torch.float32, (B, H, N))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        check_tensor(t, name, dev, torch.bfloat16, q.shape)
        grads.append(t)
    len_ptr = 0
    if kv_len is not None:
        check_tensor(kv_len, "kv_len", dev, torch.int32)
        if kv_len.numel() != B:
            raise ValueError(f"kv_len must hold one entry per batch ({B})")
        len_ptr = kv_len.data_ptr()
    need = osm_attn_bwd_workspace(B, H, N, D)
    if need < 0:
        raise OsmError(OSM_ERR_INVALID_ARG, "osm_attn_bwd_workspace")
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = osm_attn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         dout.data_ptr(), grads[0].data_ptr(), grads[1].data_ptr(),
                         grads[2].data_ptr(), B, H, N, D, float(scale), bool(causal), len_ptr,
                         ws.data_ptr(), ws.numel(), _stream_handle(q.device))
    if st != OSM_OK:
        raise OsmError(st, "osm_attn_bwd_ex")
    return tuple(grads)
