"""GPU tests of the entry points recorded into a HIP graph and replayed.

The library allocates nothing and sets no memory with the runtime, so its
launches can be captured.  The attention forward is the case to watch: eager
launches of a large enough grid claim their query tiles through one of 64
queue slots per GPU, taken in turn.  A captured launch would keep its slot for
every replay while eager launches go on cycling through all 64, so captured
launches take a fixed schedule instead.  Here a graph holding the row
softmax, the attention forward (on a queue-sized grid) and the backward is
replayed many times on one stream while eager forward launches run on
another, every slot in use along the way; every replay and every eager
launch is compared bitwise with a launch run alone, by device-side counts
taken between the replays.
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


def _announce(*what):
    print("[case]", *what, flush=True)


def test_graph_replays_beside_eager_forward_launches():
    # B1 H40 N2048 D128 causal: 640 query tiles, more than the resident
    # workgroups, so an eager launch of this shape uses a queue slot.
    B, H, N, D = 1, 40, 2048, 128
    _announce("graph replays", B, H, N, D)
    scale = float(np.float32(1 / math.sqrt(D)))
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=71, device="cuda")
    do = osm_inputs.attention_grad_output(B, H, N, D, seed=71, device="cuda")
    q2, k2, v2 = osm_inputs.attention_inputs(B, H, N, D, seed=72, device="cuda")
    x = osm_inputs.softmax_rows(512, 4096, seed=73, device="cuda")

    # Launches run alone.
    y_ref = osm.softmax_rows(x)
    o_ref, l_ref = osm.attn_fwd(q, k, v, scale, True)
    dq_ref, dk_ref, dv_ref = osm.attn_bwd(q, k, v, o_ref, l_ref, do, scale, True)
    o2_ref, l2_ref = osm.attn_fwd(q2, k2, v2, scale, True)
    torch.cuda.synchronize()

    y = torch.empty_like(x)
    o = torch.empty_like(q)
    lse = torch.empty_like(l_ref)
    grads = [torch.empty_like(q) for _ in range(3)]
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):  # one launch of each before capture
        osm.softmax_rows(x, out=y)
        osm.attn_fwd(q, k, v, scale, True, out=o, lse=lse)
        osm.attn_bwd(q, k, v, o, lse, do, scale, True, *grads)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        osm.softmax_rows(x, out=y)
        osm.attn_fwd(q, k, v, scale, True, out=o, lse=lse)
        osm.attn_bwd(q, k, v, o, lse, do, scale, True, *grads)
    torch.cuda.synchronize()

    replay_stream, eager_stream = torch.cuda.Stream(), torch.cuda.Stream()
    bad_replay = torch.zeros((), dtype=torch.int64, device="cuda")
    bad_eager = torch.zeros((), dtype=torch.int64, device="cuda")
    o2 = torch.empty_like(q2)
    l2 = torch.empty_like(l2_ref)
    replays = 24
    eager = 80  # more launches than queue slots
    for rnd in range(2):
        with torch.cuda.stream(replay_stream):
            for _ in range(replays):
                for t in (y, o, lse, *grads):
                    t.fill_(float("nan"))
                g.replay()
                bad_replay += ((y != y_ref).sum() + (o != o_ref).sum() + (lse != l_ref).sum()
                               + (grads[0] != dq_ref).sum() + (grads[1] != dk_ref).sum()
                               + (grads[2] != dv_ref).sum())
        with torch.cuda.stream(eager_stream):
            for _ in range(eager):
                o2.fill_(float("nan"))
                l2.fill_(float("nan"))
                osm.attn_fwd(q2, k2, v2, scale, True, out=o2, lse=l2)
                bad_eager += (o2 != o2_ref).sum() + (l2 != l2_ref).sum()
        torch.cuda.synchronize()
        _announce("round", rnd, "replay mismatches", bad_replay.item(),
                  "eager mismatches", bad_eager.item())
    assert bad_replay.item() == 0, f"{bad_replay.item()} values differ in graph replays"
    assert bad_eager.item() == 0, f"{bad_eager.item()} values differ in eager launches"


# Captured launches of queue-sized grids (more query tiles than resident
# workgroups: 512 at D = 128, 768 at D = 64) run the fixed pair schedules: all
# heads dealt together when B * H is not a multiple of 8, per XCD otherwise.
CAPTURE_GRIDS = [
    (1, 37, 2048, 128, True),   # B * H = 37: pairs over all heads
    (2, 48, 2048, 64, False),   # pairs per XCD, unmasked, D = 64
    (2, 40, 2048, 64, True),    # pairs per XCD, causal, D = 64
]


@pytest.mark.parametrize("B,H,N,D,causal", CAPTURE_GRIDS)
def test_captured_forward_equals_eager(B, H, N, D, causal):
    _announce("captured forward", B, H, N, D, causal)
    scale = float(np.float32(1 / math.sqrt(D)))
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=B * 10 + H + D, device="cuda")
    o_ref, l_ref = osm.attn_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    lse = torch.empty_like(l_ref)
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        osm.attn_fwd(q, k, v, scale, causal, out=o, lse=lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        osm.attn_fwd(q, k, v, scale, causal, out=o, lse=lse)
    torch.cuda.synchronize()
    for r in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), r
        # Eager work between replays.
        osm.attn_fwd(q, k, v, scale, causal)
        torch.cuda.synchronize()


def test_captured_split_and_masked_entry_points():
    # The split entry points take their workspace from the caller (here
    # torch's graph pool); masks, row lengths, key lengths and a bias are
    # plain inputs; the small-grid forward keeps its partial states in LDS.
    # Every replay must equal the eager launch bitwise.
    B, H, N, D = 2, 4, 1536, 128
    _announce("captured split/masked", B, H, N, D)
    scale = float(np.float32(1 / math.sqrt(D)))
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=81, device="cuda")
    kv = torch.tensor([N, 1000], dtype=torch.int32, device="cuda")
    g0 = torch.Generator(device="cuda").manual_seed(82)
    bias = torch.randn((1, H, N, N), generator=g0, device="cuda")
    x = osm_inputs.softmax_rows(64, 20000, seed=83, device="cuda")
    mask = torch.randn((1, 20000), generator=g0, device="cuda")
    rl = torch.randint(0, 20001, (64,), generator=g0, device="cuda", dtype=torch.int32)
    # A small grid (B1 H8 N1024 D64): 32-row workgroups that split the keys.
    qs, ks, vs = osm_inputs.attention_inputs(1, 8, 1024, 64, seed=84, device="cuda")

    def run():
        a = osm.attn_fwd(q, k, v, scale, True, kv_len=kv, splits=4)
        b = osm.attn_fwd(q, k, v, scale, False, bias=bias)
        c = osm.softmax_rows(x, mask=mask, row_len=rl, split=True)
        d = osm.attn_fwd(qs, ks, vs, 0.125, False)
        return (*a, *b, c, *d)

    refs = [t.clone() for t in run()]
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        outs = run()
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, ref) in enumerate(zip(outs, refs)):
            assert torch.equal(t, ref), (r, i)
        run()  # eager work between replays
        torch.cuda.synchronize()
