"""GPU parity of the split entry points against the float64 CPU oracle.

osm_softmax_rows_split (a row shared by several workgroups, chunk states merged
with the (m, l) combine) is held to the bars of the plain row softmax: float32
1e-6 absolute, bfloat16 half a bfloat16 ulp plus 2^-15 relative
(tests/tolerance.py), hidden entries exactly 0.
osm_attn_fwd_split (split-K with the log-sum-exp merge) is held to those of the
fused attention: O 2e-2, LSE 1e-3, rows without a visible key give O = 0 and
LSE = -inf.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_06_amd as osm
import osm_inputs
from tolerance import bf16_rne_violations
from oracle import attention_ref, masked_softmax_rows_ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    osm.load_library()


def _announce(*what):
    print("[case]", *what, flush=True)


def _check_softmax(x, mask, lens, y, dtype):
    ref = masked_softmax_rows_ref(x.double().numpy(),
                                  None if mask is None else mask.double().numpy(),
                                  None if lens is None else lens.numpy())
    got = y.double().cpu().numpy()
    assert not np.isnan(got).any()
    assert (got[ref == 0] == 0).all(), "hidden entries must be exactly 0"
    err = np.abs(got - ref)
    if dtype == torch.float32:
        assert err.max(initial=0) <= 1e-6, err.max()
    else:
        assert not bf16_rne_violations(got, ref).any(), err.max()


# One chunk, a ragged second chunk, a scalar-path width, a 1M-element row.
SPLIT_SHAPES = [(3, 100), (4, 8192), (3, 8193), (2, 12289), (2, 70001), (1, 1 << 20)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", SPLIT_SHAPES)
def test_split_softmax_plain(rows, cols, dtype):
    _announce("softmax_split", rows, cols, dtype)
    x = osm_inputs.softmax_rows(rows, cols, seed=rows * 7 + cols, sigma=4.0, ninf_prob=0.01,
                                dtype=dtype)
    if rows > 1:
        x[-1] = float("-inf")   # a fully -inf row gives zeros
    y = osm.softmax_rows(x.cuda(), split=True)
    torch.cuda.synchronize()
    _check_softmax(x, None, None, y, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(5, 20000), (3, 8192 * 3 + 5)])
def test_split_softmax_mask_lengths(rows, cols, dtype):
    _announce("softmax_split masked", rows, cols, dtype)
    x = osm_inputs.softmax_rows(rows, cols, seed=cols, sigma=2.0, ninf_prob=0.0, dtype=dtype)
    g = torch.Generator().manual_seed(rows + cols)
    mask = torch.where(torch.rand(2, cols, generator=g) < 0.2, float("-inf"),
                       torch.randn(2, cols, generator=g)).to(dtype)
    lens = torch.tensor([cols, 8191, 0, 9000, cols + 9][:rows], dtype=torch.int32)
    y = osm.softmax_rows(x.cuda(), mask=mask.cuda(), row_len=lens.cuda(), split=True)
    torch.cuda.synchronize()
    _check_softmax(x, mask, lens, y, dtype)


def test_split_softmax_in_place_and_deterministic():
    rows, cols = 3, 50000
    _announce("softmax_split in place", rows, cols)
    x = osm_inputs.softmax_rows(rows, cols, seed=11, sigma=4.0, ninf_prob=0.01)
    xd = x.cuda()
    a = osm.softmax_rows(xd, split=True)
    b = osm.softmax_rows(xd, split=True)
    osm.softmax_rows(xd, out=xd, split=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, xd)
    _check_softmax(x, None, None, a, torch.float32)


def test_split_softmax_workspace_untouched_beyond_size():
    rows, cols = 2, 30000
    _announce("softmax_split workspace guard", rows, cols)
    x = osm_inputs.softmax_rows(rows, cols, seed=12).cuda()
    y = torch.empty_like(x)
    need = osm.osm_softmax_rows_split_workspace(rows, cols)
    ws = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    st = osm.osm_softmax_rows_split(x.data_ptr(), y.data_ptr(), rows, cols, osm.OSM_F32, 0, 0, 0,
                                    ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == osm.OSM_OK
    torch.cuda.synchronize()
    assert (ws[need:] == 0x5A).all()
    _check_softmax(x.cpu(), None, None, y, torch.float32)


def _compare_attn(q, k, v, scale, causal, kv_len, bias, o, lse):
    O, L = attention_ref(q.double().cpu().numpy(), k.double().cpu().numpy(),
                         v.double().cpu().numpy(), scale, causal,
                         kv_len=None if kv_len is None else kv_len.cpu().numpy(),
                         bias=None if bias is None else bias.double().cpu().numpy())
    og, lg = o.double().cpu().numpy(), lse.double().cpu().numpy()
    dead = np.isneginf(L)
    assert (np.isneginf(lg) == dead).all()
    assert (og[dead] == 0).all()
    assert np.abs(og - O).max() <= 2e-2
    assert np.abs(lg[~dead] - L[~dead]).max(initial=0) <= 1e-3


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,splits", [(1, 2), (100, 7), (301, 2), (301, 3), (1000, 4), (1000, 64)])
def test_split_attention(N, splits, causal, D):
    B, H = 1, 3
    _announce("attn_split", B, H, N, D, causal, splits)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=N + splits + D, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, k, v, scale, causal, splits=splits)
    torch.cuda.synchronize()
    _compare_attn(q, k, v, scale, causal, None, None, o, lse)


@pytest.mark.parametrize("causal", [False, True])
def test_split_attention_kv_len_and_bias(causal):
    B, H, N, D = 3, 2, 260, 128
    _announce("attn_split kv_len bias", B, H, N, D, causal)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=41, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(42)
    bias = torch.randn((1, H, N, N), generator=g, device="cuda")
    bias = torch.where(torch.rand((1, H, N, N), generator=g, device="cuda") < 0.1,
                       float("-inf"), bias)
    kv_len = torch.tensor([N, 70, 0], dtype=torch.int32, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, k, v, scale, causal, kv_len=kv_len, bias=bias, splits=3)
    torch.cuda.synchronize()
    _compare_attn(q, k, v, scale, causal, kv_len, bias, o, lse)


def test_split_attention_long_context_sampled():
    # The long-context workload's per-GPU share when its 32 heads are split
    # over 8 GPUs: 4 heads of 16384 keys, few workgroups without splits.
    cfg = osm_inputs.attention_config("attn_long", device="cuda")
    c = cfg["cfg"]
    q, k, v = (cfg[n][:, :4].contiguous() for n in ("q", "k", "v"))
    _announce("attn_split long context", tuple(q.shape), "splits 4")
    o, lse = osm.attn_fwd(q, k, v, cfg["scale"], True, splits=4)
    torch.cuda.synchronize()
    for h in (0, 3):
        sl = lambda t: t[:, h:h + 1]  # noqa: E731
        _compare_attn(sl(q), sl(k), sl(v), cfg["scale"], True, None, None, sl(o), sl(lse))
    assert c["N"] == 16384
