"""C-ABI checks that need no GPU.

The library must load, export every function include/osm.h declares, and
reject invalid arguments with a status code before making any HIP call (so the
calls below are safe on a machine without a GPU: none of them launches).
"""

import ctypes
import os
import re

import pytest

import online_softmax_06_amd as osm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "osm.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(osm_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(osm.lib_path()):
        pytest.fail("libosm.so is not built: run `python -m online_softmax_06_amd.build`")
    return osm.load_library()


def test_header_declares_the_boundary():
    assert _declared_functions() == ["osm_attn_bwd", "osm_attn_bwd_ex", "osm_attn_bwd_noalloc",
                                     "osm_attn_bwd_workspace",
                                     "osm_attn_fwd", "osm_attn_fwd_ex", "osm_attn_fwd_split",
                                     "osm_attn_fwd_split_workspace", "osm_softmax_rows",
                                     "osm_softmax_rows_ex", "osm_softmax_rows_split",
                                     "osm_softmax_rows_split_workspace", "osm_status_string",
                                     "osm_stream_copy",
                                     "osm_version"]


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(osm.lib_path())
    for name in _declared_functions():
        assert hasattr(raw, name), name


def test_python_layer_exposes_the_same_names():
    for name in _declared_functions():
        assert callable(getattr(osm, name)), name


def test_status_strings(lib):
    assert osm.osm_status_string(osm.OSM_OK) == "OSM_OK"
    for st in (osm.OSM_ERR_INVALID_ARG, osm.OSM_ERR_UNSUPPORTED, osm.OSM_ERR_HIP):
        assert osm.osm_status_string(st).startswith("OSM_ERR_")
    assert "UNKNOWN" in osm.osm_status_string(12345)
    assert re.match(r"^\d+\.\d+\.\d+$", osm.osm_version())


FAKE = 0x10000  # 64 KiB-aligned fake device address; never dereferenced


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE, -1, 10, 0), osm.OSM_ERR_INVALID_ARG),        # negative rows
    ((FAKE, FAKE, 10, -1, 0), osm.OSM_ERR_INVALID_ARG),        # negative cols
    ((FAKE, FAKE, 10, 10, 2), osm.OSM_ERR_INVALID_ARG),        # unknown dtype
    ((FAKE, FAKE, 10, 10, -1), osm.OSM_ERR_INVALID_ARG),       # unknown dtype
    ((0, FAKE, 10, 10, 0), osm.OSM_ERR_INVALID_ARG),           # null input
    ((FAKE, 0, 10, 10, 1), osm.OSM_ERR_INVALID_ARG),           # null output
    ((FAKE + 2, FAKE, 10, 10, 0), osm.OSM_ERR_INVALID_ARG),    # fp32 misaligned
    ((FAKE + 1, FAKE, 10, 10, 1), osm.OSM_ERR_INVALID_ARG),    # bf16 misaligned
    ((FAKE, FAKE, 10, 2 ** 31, 0), osm.OSM_ERR_INVALID_ARG),   # cols too large
    ((FAKE, FAKE, 2 ** 62, 2 ** 20, 0), osm.OSM_ERR_INVALID_ARG),  # size overflow
    ((0, 0, 0, 10, 0), osm.OSM_OK),                            # empty: no-op
    ((0, 0, 10, 0, 1), osm.OSM_OK),                            # empty: no-op
])
def test_softmax_argument_checks(lib, args, expect):
    assert osm.osm_softmax_rows(*args, 0) == expect


def _attn(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, D=64, scale=0.125, causal=0):
    return osm.osm_attn_fwd(q, k, v, o, lse, B, H, N, D, scale, causal, 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(D=96), osm.OSM_ERR_UNSUPPORTED),
    (dict(D=32), osm.OSM_ERR_UNSUPPORTED),
    (dict(D=256), osm.OSM_ERR_UNSUPPORTED),
    (dict(B=-1), osm.OSM_ERR_INVALID_ARG),
    (dict(N=-5), osm.OSM_ERR_INVALID_ARG),
    (dict(scale=0.0), osm.OSM_ERR_INVALID_ARG),
    (dict(scale=-0.1), osm.OSM_ERR_INVALID_ARG),
    (dict(scale=float("inf")), osm.OSM_ERR_INVALID_ARG),
    (dict(scale=float("nan")), osm.OSM_ERR_INVALID_ARG),
    (dict(q=0), osm.OSM_ERR_INVALID_ARG),
    (dict(lse=0), osm.OSM_ERR_INVALID_ARG),
    (dict(o=FAKE + 8), osm.OSM_ERR_INVALID_ARG),
    (dict(B=2 ** 30, H=2 ** 30, N=2 ** 30), osm.OSM_ERR_INVALID_ARG),
    (dict(N=0, q=0, k=0, v=0, o=0, lse=0), osm.OSM_OK),
    (dict(B=0), osm.OSM_OK),
])
def test_attention_argument_checks(lib, kw, expect):
    assert _attn(**kw) == expect


def test_tensor_helpers_reject_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        osm.softmax_rows(torch.zeros(2, 3))
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        osm.attn_fwd(x, x, x)
    with pytest.raises(ValueError):
        osm.attn_bwd(x, x, x, x, torch.zeros(1, 1, 4), x)


def test_check_tensor():
    import torch
    gpu = torch.device("cuda", 0)
    cpu = torch.device("cpu")
    t = torch.zeros(2, 3, dtype=torch.float32)
    osm.check_tensor(t, "t", cpu, torch.float32, (2, 3))
    with pytest.raises(ValueError, match="must be on cuda:0"):
        osm.check_tensor(t, "t", gpu, torch.float32)
    with pytest.raises(ValueError, match="dtype"):
        osm.check_tensor(t, "t", cpu, torch.bfloat16)
    with pytest.raises(ValueError, match="shape"):
        osm.check_tensor(t, "t", cpu, torch.float32, (3, 2))
    with pytest.raises(ValueError, match="contiguous"):
        osm.check_tensor(t.t(), "t", cpu, torch.float32)
    with pytest.raises(ValueError, match="tensor"):
        osm.check_tensor(None, "t", cpu, torch.float32)


# Every tensor a helper passes on is checked against the first input's
# device.  The helpers are run here with the inputs' device taken as given
# (CPU) and one argument elsewhere ("meta"): each call must stop with
# ValueError before the library is reached.
def _on_meta(t):
    import torch
    return torch.empty(t.shape, dtype=t.dtype, device="meta")


def test_helpers_check_every_tensor_device(monkeypatch):
    import torch
    monkeypatch.setattr(osm, "_gpu_device", lambda t, name: t.device)
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="out must be on cpu"):
        osm.softmax_rows(x, out=_on_meta(x))
    with pytest.raises(ValueError, match="mask must be on cpu"):
        osm.softmax_rows(x, mask=_on_meta(x))
    with pytest.raises(ValueError, match="row_len must be on cpu"):
        osm.softmax_rows(x, row_len=_on_meta(torch.zeros(4, dtype=torch.int32)))
    q = torch.zeros(2, 1, 4, 64, dtype=torch.bfloat16)
    lse = torch.zeros(2, 1, 4)
    kv = torch.zeros(2, dtype=torch.int32)
    for kw in (dict(k=_on_meta(q)), dict(v=_on_meta(q))):
        args = dict(q=q, k=q, v=q) | kw
        with pytest.raises(ValueError, match="must be on cpu"):
            osm.attn_fwd(args["q"], args["k"], args["v"])
    for kw, name in ((dict(out=_on_meta(q)), "out"), (dict(lse=_on_meta(lse)), "lse"),
                     (dict(kv_len=_on_meta(kv)), "kv_len"),
                     (dict(bias=torch.zeros(1, 1, 4, 4, device="meta")), "bias")):
        with pytest.raises(ValueError, match=f"{name} must"):
            osm.attn_fwd(q, q, q, **kw)
    for i, name in enumerate(("k", "v", "o", "dout")):
        args = [q, q, q, q, lse, q]
        args[[1, 2, 3, 5][i]] = _on_meta(q)
        with pytest.raises(ValueError, match=f"{name} must be on cpu"):
            osm.attn_bwd(*args)
    with pytest.raises(ValueError, match="lse must be on cpu"):
        osm.attn_bwd(q, q, q, q, _on_meta(lse), q)
    for name in ("dq", "dk", "dv"):
        with pytest.raises(ValueError, match=f"{name} must be on cpu"):
            osm.attn_bwd(q, q, q, q, lse, q, **{name: _on_meta(q)})
    with pytest.raises(ValueError, match="kv_len must be on cpu"):
        osm.attn_bwd(q, q, q, q, lse, q, kv_len=_on_meta(kv))


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE, 4, 8, 0, FAKE, 0, 0), osm.OSM_ERR_INVALID_ARG),      # mask_rows < 1
    ((FAKE, FAKE, 4, 8, 0, FAKE + 2, 1, 0), osm.OSM_ERR_INVALID_ARG),  # misaligned mask
    ((FAKE, FAKE, 4, 8, 0, 0, 0, FAKE + 2), osm.OSM_ERR_INVALID_ARG),  # misaligned lengths
    ((FAKE, FAKE, 4, 8, 5, 0, 0, 0), osm.OSM_ERR_INVALID_ARG),         # unknown dtype
    ((0, 0, 0, 8, 0, FAKE, 1, FAKE), osm.OSM_OK),                      # empty: no-op
])
def test_softmax_ex_argument_checks(lib, args, expect):
    assert osm.osm_softmax_rows_ex(*args, 0) == expect


@pytest.mark.parametrize("kw,expect", [
    (dict(kv_len=FAKE + 2), osm.OSM_ERR_INVALID_ARG),
    (dict(bias=FAKE + 2), osm.OSM_ERR_INVALID_ARG),
    (dict(bias=FAKE, bias_stride_b=-1), osm.OSM_ERR_INVALID_ARG),
    (dict(bias=FAKE, D=80), osm.OSM_ERR_UNSUPPORTED),
    (dict(N=0, kv_len=FAKE + 2), osm.OSM_OK),
])
def test_attention_ex_argument_checks(lib, kw, expect):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=16, D=64, scale=0.125,
             causal=0, kv_len=0, bias=0, bias_stride_b=0, bias_stride_h=0)
    a.update(kw)
    assert osm.osm_attn_fwd_ex(*a.values(), 0) == expect


def test_split_workspace_size(lib):
    assert osm.osm_softmax_rows_split_workspace(4, 8192) == 4 * 8
    assert osm.osm_softmax_rows_split_workspace(3, 8193) == 3 * 2 * 8
    assert osm.osm_softmax_rows_split_workspace(2, 1 << 20) == 2 * 128 * 8
    assert osm.osm_softmax_rows_split_workspace(0, 5) == 0
    assert osm.osm_softmax_rows_split_workspace(-1, 5) == -1
    assert osm.osm_softmax_rows_split_workspace(5, 2 ** 31) == -1


@pytest.mark.parametrize("ws,wsb,expect", [
    (0, 1 << 20, osm.OSM_ERR_INVALID_ARG),         # no workspace
    (FAKE, 8, osm.OSM_ERR_INVALID_ARG),            # too small (needs 2 * 4 * 8)
    (FAKE + 4, 1 << 20, osm.OSM_ERR_INVALID_ARG),  # misaligned
])
def test_split_argument_checks(lib, ws, wsb, expect):
    assert osm.osm_softmax_rows_split(FAKE, FAKE, 2, 30000, 0, 0, 0, 0, ws, wsb, 0) == expect


def test_attn_split_workspace_size(lib):
    assert osm.osm_attn_fwd_split_workspace(1, 2, 100, 64, 3) == 4 * 3 * 2 * 100 * 65
    assert osm.osm_attn_fwd_split_workspace(1, 1, 10, 96, 2) == -1
    assert osm.osm_attn_fwd_split_workspace(1, 1, 10, 64, 0) == -1
    assert osm.osm_attn_fwd_split_workspace(1, 1, 10, 64, 65) == -1


@pytest.mark.parametrize("splits,ws,wsb,expect", [
    (0, FAKE, 1 << 30, osm.OSM_ERR_INVALID_ARG),
    (65, FAKE, 1 << 30, osm.OSM_ERR_INVALID_ARG),
    (2, 0, 1 << 30, osm.OSM_ERR_INVALID_ARG),
    (2, FAKE, 16, osm.OSM_ERR_INVALID_ARG),
    (2, FAKE + 8, 1 << 30, osm.OSM_ERR_INVALID_ARG),
])
def test_attn_split_argument_checks(lib, splits, ws, wsb, expect):
    assert osm.osm_attn_fwd_split(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 2, 300, 128, 0.1, 1, 0, 0, 0, 0,
                                  splits, ws, wsb, 0) == expect


def test_attn_bwd_workspace_size(lib):
    assert osm.osm_attn_bwd_workspace(2, 3, 100, 128) == 8 * 6 * 128
    assert osm.osm_attn_bwd_workspace(1, 1, 129, 64) == 8 * 256
    assert osm.osm_attn_bwd_workspace(1, 1, 0, 64) == 0
    assert osm.osm_attn_bwd_workspace(1, 1, 10, 96) == -1
    assert osm.osm_attn_bwd_workspace(-1, 1, 10, 64) == -1


def _bwd(B=1, H=2, N=300, D=128, scale=0.1, causal=1, ptrs=None, ws=FAKE, wsb=1 << 30):
    p = [FAKE] * 9 if ptrs is None else ptrs
    return osm.osm_attn_bwd(*p, B, H, N, D, scale, causal, ws, wsb, 0)


@pytest.mark.parametrize("kw,expect", [
    (dict(D=96), osm.OSM_ERR_UNSUPPORTED),
    (dict(N=-1), osm.OSM_ERR_INVALID_ARG),
    (dict(scale=0.0), osm.OSM_ERR_INVALID_ARG),
    (dict(scale=float("nan")), osm.OSM_ERR_INVALID_ARG),
    (dict(ws=0), osm.OSM_ERR_INVALID_ARG),
    (dict(wsb=8 * 2 * 384 - 1), osm.OSM_ERR_INVALID_ARG),
    (dict(ws=FAKE + 4), osm.OSM_ERR_INVALID_ARG),
    (dict(ptrs=[FAKE] * 5 + [0] + [FAKE] * 3), osm.OSM_ERR_INVALID_ARG),   # no dout
    (dict(ptrs=[FAKE] * 6 + [FAKE + 2] + [FAKE] * 2), osm.OSM_ERR_INVALID_ARG),  # dq misaligned
    (dict(ptrs=[FAKE] * 8 + [0]), osm.OSM_ERR_INVALID_ARG),   # no dv
    (dict(N=0, ptrs=[0] * 9, ws=0, wsb=0), osm.OSM_OK),        # empty: nothing to do
])
def test_attn_bwd_argument_checks(lib, kw, expect):
    assert _bwd(**kw) == expect


def test_attn_bwd_ex_checks_kv_len_alignment(lib):
    p = [FAKE] * 9
    assert osm.osm_attn_bwd_ex(*p, 1, 2, 300, 128, 0.1, 1, FAKE + 2, FAKE, 1 << 30, 0) == \
        osm.OSM_ERR_INVALID_ARG
    assert osm.osm_attn_bwd_ex(*p, 1, 2, 300, 96, 0.1, 1, 0, FAKE, 1 << 30, 0) == \
        osm.OSM_ERR_UNSUPPORTED


def _bwd_noalloc(B=1, H=1, N=64, D=64):
    return osm.osm_attn_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    B, H, N, D, 0.125, 1, 0, 0)


def test_noalloc_backward_size_limit(lib):
    # The scratch array holds 8 bytes per padded query row: B * H * (N rounded
    # up to 128) <= 4194304.  Larger calls are refused before any HIP call.
    assert osm.OSM_ATTN_BWD_SCRATCH_BYTES == 32 << 20
    assert osm.osm_attn_bwd_workspace(1, 32768, 128, 64) == osm.OSM_ATTN_BWD_SCRATCH_BYTES
    assert _bwd_noalloc(B=1, H=32769, N=128) == osm.OSM_ERR_UNSUPPORTED
    assert _bwd_noalloc(B=8, H=40, N=16384, D=128) == osm.OSM_ERR_UNSUPPORTED
    assert _bwd_noalloc(B=2, H=16385, N=100) == osm.OSM_ERR_UNSUPPORTED  # 100 pads to 128
    assert _bwd_noalloc(D=96) == osm.OSM_ERR_UNSUPPORTED
    assert _bwd_noalloc(B=-1) == osm.OSM_ERR_INVALID_ARG
    assert osm.osm_attn_bwd_noalloc(0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    1, 1, 64, 64, 0.125, 1, 0, 0) == osm.OSM_ERR_INVALID_ARG
    assert _bwd_noalloc(N=0) == osm.OSM_OK


@pytest.mark.parametrize("args,expect", [
    ((FAKE, FAKE + (1 << 20), -1), osm.OSM_ERR_INVALID_ARG),      # negative size
    ((FAKE, FAKE + (1 << 20), (1 << 44) + 1), osm.OSM_ERR_INVALID_ARG),  # too large
    ((0, FAKE, 64), osm.OSM_ERR_INVALID_ARG),                      # null source
    ((FAKE + 8, FAKE + (1 << 20), 64), osm.OSM_ERR_INVALID_ARG),   # misaligned
    ((FAKE, FAKE + 32, 64), osm.OSM_ERR_INVALID_ARG),              # overlapping
    ((FAKE + 32, FAKE, 64), osm.OSM_ERR_INVALID_ARG),              # overlapping
    ((0, 0, 0), osm.OSM_OK),                                       # empty: no-op
])
def test_stream_copy_argument_checks(lib, args, expect):
    assert osm.osm_stream_copy(*args, 0) == expect
