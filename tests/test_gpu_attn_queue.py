"""GPU tests of the attention forward's work queue.

Launches with 128-row tiles (4 wavefronts) and more query tiles than resident
workgroups hand out their items through atomic counters in one of 64 queue
slots per GPU, each launch taking the next slot and the last workgroup of the
launch resetting it.  These tests run such launches many times in a row (every
slot used more than once), on two streams at once, with partitions of 8 and of
all heads, with a partial last group of heads and with key lengths (a batch
without keys gives items without key tiles), and check every output bitwise
against the first launch and sampled rows against the float64 oracle.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_06_amd as osm
import osm_inputs
from oracle import attention_head_ref

pytestmark = pytest.mark.gpu

O_TOL = 2e-2
LSE_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    osm.load_library()


def _announce(*what):
    print("[case]", *what, flush=True)


def _check_sampled(q, k, v, scale, causal, o, lse, seed):
    B, H, N, _ = q.shape
    rng = np.random.default_rng(seed)
    rows = sorted(set(rng.choice(N, 64, replace=False).tolist()) | {0, 127, 128, N - 1})
    for b, h in osm_inputs.sample_heads(B, H, 3, seed, must=[(0, 0), (B - 1, H - 1)]):
        qh, kh, vh = (t[b, h].cpu().double().numpy() for t in (q, k, v))
        O, L = attention_head_ref(qh, kh, vh, scale, causal, query_rows=rows)
        eo = np.abs(o[b, h].cpu().double().numpy()[rows] - O).max()
        el = np.abs(lse[b, h].cpu().double().numpy()[rows] - L).max()
        assert eo <= O_TOL and el <= LSE_TOL, ((b, h), eo, el)


# (B, H, N, D, causal): query tiles per launch against resident workgroups
# (MI355X: 512 at D = 128, 768 at D = 64).
QUEUE_GRIDS = [
    (1, 40, 2048, 128, True),   # 640 tiles, partitions of 5 heads
    (1, 37, 2048, 128, True),   # 592 tiles, B * H = 37: one partition of all heads
    (2, 48, 2048, 128, True),   # 12 heads per partition: groups of 8 and 4
    (1, 64, 2048, 64, True),    # 1024 tiles, three workgroups per CU
    (2, 48, 2048, 64, False),   # unmasked, equal items
]


@pytest.mark.parametrize("B,H,N,D,causal", QUEUE_GRIDS)
def test_queue_repeated_launches(B, H, N, D, causal):
    _announce("queue repeated", B, H, N, D, causal)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=B * 100 + H + D, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    # Outputs start as NaN: a query tile that no workgroup claimed would keep it.
    o0 = torch.full_like(q, float("nan"))
    l0 = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    osm.attn_fwd(q, k, v, scale, causal, out=o0, lse=l0)
    torch.cuda.synchronize()
    assert not torch.isnan(o0).any() and not torch.isnan(l0).any(), "unwritten rows"
    o = torch.empty_like(o0)
    lse = torch.empty_like(l0)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    # 70 launches: every one of the 64 slots is used, some twice.
    for _ in range(70):
        o.fill_(0.5)
        lse.fill_(0.5)
        osm.attn_fwd(q, k, v, scale, causal, out=o, lse=lse)
        bad += (o != o0).sum() + (lse != l0).sum()
    torch.cuda.synchronize()
    assert bad.item() == 0, f"{bad.item()} values differ from the first launch"
    _check_sampled(q, k, v, scale, causal, o0, l0, seed=N + H)


def test_queue_two_streams():
    # Launches on two streams may run at the same time; each takes its own
    # slot.  Every output must equal the one of a launch run alone.
    B, H, N, D = 1, 40, 2048, 128
    _announce("queue two streams", B, H, N, D)
    scale = float(np.float32(1 / math.sqrt(D)))
    ins = [osm_inputs.attention_inputs(B, H, N, D, seed=s, device="cuda") for s in (3, 4)]
    refs = [osm.attn_fwd(q, k, v, scale, True) for q, k, v in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty_like(refs[i][0]) for _ in range(12)] for i in range(2)]
    lses = [[torch.empty_like(refs[i][1]) for _ in range(12)] for i in range(2)]
    for r in range(12):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                q, k, v = ins[i]
                osm.attn_fwd(q, k, v, scale, True, out=outs[i][r], lse=lses[i][r])
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(12):
            assert torch.equal(outs[i][r], refs[i][0]) and torch.equal(lses[i][r], refs[i][1]), \
                (i, r)


@pytest.mark.parametrize("D", [64, 128])
def test_queue_key_lengths(D):
    # Key lengths make items of one query rank unequal, and a batch with no
    # keys gives items without any key tile: they must still claim the next
    # item (their rows get O = 0 and LSE = -inf).
    B, H, N = 4, 48, 2048
    _announce("queue key lengths", B, H, N, D)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=61 + D, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    kv_len = torch.tensor([N, 0, 1000, 33], dtype=torch.int32, device="cuda")
    o0, l0 = osm.attn_fwd(q, k, v, scale, True, kv_len=kv_len)
    for _ in range(3):
        o, lse = osm.attn_fwd(q, k, v, scale, True, kv_len=kv_len)
        assert torch.equal(o, o0) and torch.equal(lse, l0)
    torch.cuda.synchronize()
    assert (o0[1] == 0).all() and torch.isinf(l0[1]).all() and (l0[1] < 0).all()
    rng = np.random.default_rng(D)
    rows = sorted(set(rng.choice(N, 48, replace=False).tolist()) | {0, 32, 33, 999, 1000, N - 1})
    for b in range(B):
        for h in (0, H - 1):
            qh, kh, vh = (t[b, h].cpu().double().numpy() for t in (q, k, v))
            O, L = attention_head_ref(qh, kh, vh, scale, True, query_rows=rows,
                                      kv_len=int(kv_len[b]))
            og = o0[b, h].cpu().double().numpy()[rows]
            lg = l0[b, h].cpu().double().numpy()[rows]
            assert np.abs(og - O).max() <= O_TOL, (b, h)
            fin = np.isfinite(L)
            assert (np.isinf(lg) == ~fin).all(), (b, h)
            assert np.abs(lg[fin] - L[fin]).max(initial=0) <= LSE_TOL, (b, h)
