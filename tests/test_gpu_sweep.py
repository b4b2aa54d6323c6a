"""Seeded random sweep over option combinations, against the oracle.

Every case draws its shape and options from a fixed seed, so a failure names
a reproducible case.  The fixed-shape tests elsewhere cover each option on
its own; the sweep mixes them: odd lengths with key lengths, bias, the causal
mask and split-K in one call; the backward with key lengths at ragged sizes;
the softmax with masks, row lengths and the split-row kernels.  The
tolerances are those of the other GPU tests (the helpers are imported from
them): attention O 2e-2 and LSE 1e-3, the backward's scaled bound, float32
softmax 1e-6 and bfloat16 softmax half an ulp plus 2^-15 relative.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_06_amd as osm
import osm_inputs
from test_gpu_attn_bwd import _check_head, _oracle_fwd
from test_gpu_masked import _check_softmax, _compare_attn, _mask

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    osm.load_library()


def _announce(*what):
    print("[case]", *what, flush=True)


def _fwd_case(seed):
    r = np.random.default_rng(1000 + seed)
    B, H = int(r.integers(1, 4)), int(r.integers(1, 5))
    N = int(r.choice([int(r.integers(1, 40)), int(r.integers(40, 300)), int(r.integers(300, 700))]))
    D = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    scale = float(np.float32(r.uniform(0.05, 0.2)))
    kv_len = None
    if r.integers(0, 2):
        kv_len = [int(r.integers(0, N + 6)) for _ in range(B)]
        kv_len[0] = N
    bias = None
    if r.integers(0, 3) == 0:
        bias = ("head" if r.integers(0, 2) else "full", int(r.integers(0, 1 << 30)))
    splits = 1 if r.integers(0, 3) else int(r.integers(2, 6))
    return B, H, N, D, causal, scale, kv_len, bias, splits


@pytest.mark.parametrize("seed", range(32))
def test_forward_sweep(seed):
    B, H, N, D, causal, scale, kv_len, bias_spec, splits = _fwd_case(seed)
    _announce("fwd sweep", seed, dict(B=B, H=H, N=N, D=D, causal=causal, scale=scale,
                                      kv_len=kv_len, bias=bias_spec, splits=splits))
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=seed, device="cuda")
    kv = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    bias = None
    if bias_spec is not None:
        kind, bseed = bias_spec
        g = torch.Generator(device="cuda").manual_seed(bseed)
        shape = (1, H, N, N) if kind == "head" else (B, H, N, N)
        bias = torch.randn(shape, generator=g, device="cuda")
        bias = torch.where(torch.rand(shape, generator=g, device="cuda") < 0.1,
                           float("-inf"), bias)
    o, lse = osm.attn_fwd(q, k, v, scale, causal, kv_len=kv, bias=bias, splits=splits)
    torch.cuda.synchronize()
    _compare_attn(q, k, v, scale, causal, kv, bias, o, lse)


@pytest.mark.parametrize("seed", range(20))
def test_backward_sweep(seed):
    r = np.random.default_rng(2000 + seed)
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    N = int(r.choice([int(r.integers(1, 64)), int(r.integers(64, 400))]))
    D = int(r.choice([64, 128]))
    causal = bool(r.integers(0, 2))
    scale = float(np.float32(1 / math.sqrt(D)))
    kv_len = None
    if r.integers(0, 2):
        kv_len = [int(r.integers(0, N + 3)) for _ in range(B)]
    _announce("bwd sweep", seed, dict(B=B, H=H, N=N, D=D, causal=causal, kv_len=kv_len))
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=100 + seed)
    do = osm_inputs.attention_grad_output(B, H, N, D, seed=100 + seed)
    kv_np = None if kv_len is None else np.asarray(kv_len)
    o, lse = _oracle_fwd(q, k, v, scale, causal, kv_len=kv_np)
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    kv = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device="cuda")
    dq, dk, dv = osm.attn_bwd(*dev, scale=scale, causal=causal, kv_len=kv)
    torch.cuda.synchronize()
    got = {"dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    for b in range(B):
        for h in range(H):
            _check_head(q[b, h], k[b, h], v[b, h], do[b, h], o[b, h], scale, causal,
                        {name: t[b, h] for name, t in got.items()},
                        kv_len=None if kv_len is None else kv_len[b])


@pytest.mark.parametrize("seed", range(24))
def test_softmax_sweep(seed):
    r = np.random.default_rng(3000 + seed)
    rows = int(r.integers(1, 9))
    cols = int(r.choice([int(r.integers(1, 300)), int(r.integers(300, 9000)),
                         int(r.integers(9000, 40000))]))
    dtype = torch.float32 if r.integers(0, 2) else torch.bfloat16
    kind = ["none", "pad", "bias"][int(r.integers(0, 3))]
    mask_rows = int(r.choice([1, rows]))
    use_len = bool(r.integers(0, 2))
    split = bool(r.integers(0, 3) == 0)
    _announce("softmax sweep", seed, dict(rows=rows, cols=cols, dtype=str(dtype), kind=kind,
                                          mask_rows=mask_rows, lens=use_len, split=split))
    x = osm_inputs.softmax_rows(rows, cols, seed=seed, sigma=3.0, ninf_prob=0.02, dtype=dtype)
    mask = None if kind == "none" else _mask(mask_rows, cols, kind, seed + 7, dtype)
    lens = None
    if use_len:
        lens = torch.tensor(r.integers(-1, cols + 2, size=rows), dtype=torch.int32)
    y = osm.softmax_rows(x.cuda(), mask=None if mask is None else mask.cuda(),
                         row_len=None if lens is None else lens.cuda(), split=split)
    torch.cuda.synchronize()
    _check_softmax(x, mask, lens, y, dtype)
