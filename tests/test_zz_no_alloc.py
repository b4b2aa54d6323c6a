"""The allocation-free attention backward against the workspace one (GPU).

osm_attn_bwd_noalloc takes its per-row scratch from the library's own fixed
array instead of a caller workspace.  Called raw through the C ABI, it must
give the same gradients as osm_attn_bwd_ex on the same inputs (bitwise: the
kernels are the same), on two calls in a row, the second with a smaller
input, so that a stale scratch from the first call cannot leak into the
second.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_06_amd as osm
import osm_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    osm.load_library()


def _case(B, H, N, D, causal, seed, with_len):
    dev = "cuda"
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=seed, device=dev)
    do = osm_inputs.attention_grad_output(B, H, N, D, seed=seed, device=dev)
    scale = float(np.float32(1 / math.sqrt(D)))
    kv = None
    if with_len:
        g = torch.Generator().manual_seed(seed)
        kv = torch.randint(1, N + 1, (B,), generator=g, dtype=torch.int32).to(dev)
    o, lse = osm.attn_fwd(q, k, v, scale, causal, kv_len=kv)
    return q, k, v, o, lse, do, scale, kv


def _noalloc(q, k, v, o, lse, do, scale, causal, kv):
    B, H, N, D = q.shape
    grads = [torch.full_like(q, float("nan")) for _ in range(3)]
    st = osm.osm_attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), do.data_ptr(), grads[0].data_ptr(),
                                  grads[1].data_ptr(), grads[2].data_ptr(), B, H, N, D, scale,
                                  int(causal), 0 if kv is None else kv.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == osm.OSM_OK, osm.osm_status_string(st)
    return grads


@pytest.mark.parametrize("first,second", [
    ((2, 3, 300, 128, True, False), (1, 2, 100, 64, True, False)),
    ((2, 4, 1000, 64, False, True), (1, 3, 257, 128, False, True)),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for shape in (first, second):
        B, H, N, D, causal, with_len = shape
        print("[case] osm_attn_bwd_noalloc", shape, flush=True)
        q, k, v, o, lse, do, scale, kv = _case(B, H, N, D, causal, seed=B * 100 + N + D,
                                               with_len=with_len)
        got = _noalloc(q, k, v, o, lse, do, scale, causal, kv)
        want = osm.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=causal, kv_len=kv)
        torch.cuda.synchronize()
        for name, g, w in zip(("dq", "dk", "dv"), got, want):
            assert torch.equal(g, w), f"{name} differs from osm_attn_bwd_ex"
