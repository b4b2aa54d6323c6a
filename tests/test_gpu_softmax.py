"""GPU parity tests of osm_softmax_rows against the float64 CPU oracle.

Tolerances: float32 output, max |gpu - oracle| <= 1e-6; bfloat16 output,
|gpu - oracle| <= half a bfloat16 ulp of the oracle value plus 2^-15 relative
(round to nearest even meets it, truncation does not: tests/tolerance.py);
-inf inputs give exact zeros, and all -inf rows give all zeros.  Every call
goes through the C ABI.
"""

import numpy as np
import pytest
import torch

import online_softmax_06_amd as osm
import osm_inputs
from oracle import softmax_rows_ref
from tolerance import bf16_rne_violations

pytestmark = pytest.mark.gpu

F32_TOL = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    osm.load_library()


def _announce(*what):
    print("[case]", *what, flush=True)


def check(x_cpu, y_gpu, dtype):
    """Compare a GPU result with the oracle on the same input."""
    ref = softmax_rows_ref(x_cpu.double().numpy())
    got = y_gpu.double().cpu().numpy()
    assert not np.isnan(got).any()
    masked = np.isneginf(x_cpu.double().numpy())
    assert (got[masked] == 0.0).all(), "-inf inputs must give exact zeros"
    err = np.abs(got - ref)
    if dtype == torch.float32:
        assert err.max(initial=0.0) <= F32_TOL, f"max abs err {err.max()}"
    else:
        bad = bf16_rne_violations(got, ref)
        assert not bad.any(), f"{bad.sum()} elements beyond the nearest-even bound; max err {err.max()}"
    return err.max(initial=0.0)


def run(x_dev, out=None):
    return osm.softmax_rows(x_dev, out=out)


def test_small_config_three_calls():
    data = osm_inputs.softmax_small()
    for label, x in data["calls"]:
        _announce("softmax_small", label, tuple(x.shape))
        y = run(x.cuda())
        torch.cuda.synchronize()
        check(x, y, torch.float32)
        if label.startswith("A"):
            assert (y[60:62] == 0).all(), "all -inf rows must give zeros"
            rs = y[:60].double().sum(1).cpu()
            assert (rs - 1).abs().max() < 1e-5
        if label.startswith("C"):
            # Ch.6 §6.3.2 prints y = (0.0159, 0.8668, 0.1173).
            np.testing.assert_allclose(y.cpu().numpy()[0], [0.0159, 0.8668, 0.1173], atol=5e-5)


SHAPES = [(1, 1), (3, 3), (5, 17), (7, 100), (4, 1000), (2, 1024), (3, 2049), (3, 4097),
          (2, 8192), (2, 12289), (2, 16384), (1, 40000), (2, 65536), (1, 70001), (1, 150000),
          # Float32 rows of 4097..8192 values run two to a workgroup: odd row
          # counts leave the last workgroup's second row empty, and ragged
          # widths leave lanes without a vector.  Bfloat16 rows of that
          # length run on 512 threads: 4104 and 8184 are just past and just
          # short of the edges of that range.
          (3, 4100), (3, 5000), (5, 8188), (3, 4104), (1, 8184)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_shapes_vector_and_scalar_paths(rows, cols, dtype):
    _announce("shape", rows, cols, dtype)
    x = osm_inputs.softmax_rows(rows, cols, seed=rows * 100003 + cols, sigma=4.0, ninf_prob=0.01,
                                dtype=dtype)
    # Aligned base (vector path when cols fits the 16-byte vector).
    y = run(x.cuda())
    torch.cuda.synchronize()
    check(x, y, dtype)
    # Base shifted by one element: never 16-byte aligned, so the scalar path runs.
    buf = torch.empty(rows * cols + 1, dtype=dtype, device="cuda")
    xin = buf[1:].view(rows, cols)
    xin.copy_(x.cuda())
    obuf = torch.empty(rows * cols + 1, dtype=dtype, device="cuda")
    yout = obuf[1:].view(rows, cols)
    st = osm.osm_softmax_rows(xin.data_ptr(), yout.data_ptr(), rows, cols,
                              osm.OSM_F32 if dtype == torch.float32 else osm.OSM_BF16,
                              torch.cuda.current_stream().cuda_stream)
    assert st == osm.OSM_OK
    torch.cuda.synchronize()
    check(x, yout, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_overflow_and_masked_rows_long(dtype):
    _announce("overflow/masked long rows", dtype)
    x = osm_inputs.softmax_rows(8, 8192, seed=11, sigma=3.0, ninf_prob=0.0)
    x[0:2] += 1000.0
    x[2:4, :3000] = float("-inf")
    x[4:6] = float("-inf")
    x = x.to(dtype)
    y = run(x.cuda())
    torch.cuda.synchronize()
    check(x, y, dtype)
    assert (y[4:6] == 0).all()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_in_place(dtype):
    _announce("in place", dtype)
    x = osm_inputs.softmax_rows(64, 8192, seed=12, dtype=dtype)
    xd = x.cuda()
    run(xd, out=xd)
    torch.cuda.synchronize()
    check(x, xd, dtype)
    x2 = osm_inputs.softmax_rows(3, 70001, seed=13, dtype=dtype)  # looping kernel
    xd2 = x2.cuda()
    run(xd2, out=xd2)
    torch.cuda.synchronize()
    check(x2, xd2, dtype)


@pytest.mark.parametrize("cols", [1000, 8192, 70001])
def test_deterministic_and_guard_bands(cols):
    _announce("determinism/guard", cols)
    rows = 33
    x = osm_inputs.softmax_rows(rows, cols, seed=14).cuda()
    pad = 4096
    canary = 12345.0
    buf = torch.full((rows * cols + 2 * pad,), canary, dtype=torch.float32, device="cuda")
    out = buf[pad:pad + rows * cols].view(rows, cols)
    run(x, out=out)
    first = out.clone()
    run(x, out=out)
    torch.cuda.synchronize()
    assert torch.equal(first, out), "two runs must be bitwise identical"
    assert (buf[:pad] == canary).all() and (buf[pad + rows * cols:] == canary).all()


def test_many_rows_grid_loop():
    # More row groups than the grid cap: the kernel loops over rows.
    rows, cols = 4 * (1 << 20) + 37, 8
    _announce("grid loop", rows, cols)
    x = osm_inputs.softmax_rows(rows, cols, seed=15, device="cuda")
    y = run(x)
    torch.cuda.synchronize()
    idx = torch.tensor([0, 1, 12345, rows // 2, rows - 38, rows - 2, rows - 1])
    check(x[idx.cuda()].cpu(), y[idx.cuda()], torch.float32)
    rs = y.double().sum(1)
    live = ~torch.isneginf(x).all(1)
    assert ((rs[live] - 1).abs().max()) < 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bandwidth_config_full_size_sampled_rows(dtype):
    c = osm_inputs.SOFTMAX_LARGE
    _announce("softmax_large", c["rows"], c["cols"], dtype)
    x = osm_inputs.softmax_large(dtype=dtype, device="cuda")
    y = run(x)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert (y[torch.isneginf(x)] == 0).all()
    rs = y.double().sum(1)
    assert (rs - 1).abs().max().item() < (1e-5 if dtype == torch.float32 else 2e-2)
    g = torch.Generator().manual_seed(2024)
    rows = torch.cat([torch.tensor([0, c["rows"] - 1]),
                      torch.randint(1, c["rows"] - 1, (62,), generator=g)])
    err = check(x[rows.cuda()].cpu(), y[rows.cuda()], dtype)
    print(f"[result] softmax_large {dtype} sampled max abs err {err:.3g}", flush=True)


def test_raw_abi_small_config_vector_path():
    # osm_softmax_rows itself, raw through ctypes, on the three calls of the
    # small workload with 16-byte aligned bases: cols 1000 and 100 take the
    # float4 vector path, cols 3 the scalar path.
    data = osm_inputs.softmax_small()
    for label, x in data["calls"]:
        _announce("raw osm_softmax_rows", label, tuple(x.shape))
        xd = x.cuda()
        yd = torch.full_like(xd, float("nan"))
        assert xd.data_ptr() % 16 == 0 and yd.data_ptr() % 16 == 0
        rows, cols = x.shape
        st = osm.osm_softmax_rows(xd.data_ptr(), yd.data_ptr(), rows, cols, osm.OSM_F32,
                                  torch.cuda.current_stream().cuda_stream)
        assert st == osm.OSM_OK, osm.osm_status_string(st)
        torch.cuda.synchronize()
        err = check(x, yd, torch.float32)
        print(f"[result] raw osm_softmax_rows softmax_small {label} max abs err {err:.3g}",
              flush=True)
