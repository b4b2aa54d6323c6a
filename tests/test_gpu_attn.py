"""GPU parity tests of osm_attn_fwd against the float64 CPU oracle.

Tolerances: bfloat16 O, max |gpu - oracle| <= 2e-2; float32 LSE,
max |gpu - oracle| <= 1e-3.  Small shapes are compared in full; the large
workloads on seeded (b, h) slices, every query row of each slice, in the same
launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_06_amd as osm
import osm_inputs
from oracle import attention_head_ref, attention_ref
from tolerance import CONSTANT_V_MIN_KEYS, O_ABS_SLACK, bf16_rne_violations

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


def compare(q, k, v, scale, causal, o, lse, heads=None):
    """Oracle on the host copies of q, k, v; returns (max O err, max LSE err)."""
    qh, kh, vh = (t.cpu().double().numpy() for t in (q, k, v))
    O, L = attention_ref(qh, kh, vh, scale, causal, heads=heads)
    og = o.cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    if heads is not None:
        og = np.stack([og[b, h] for b, h in heads])
        lg = np.stack([lg[b, h] for b, h in heads])
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    eo = np.abs(og - O).max()
    el = np.abs(lg - L).max()
    assert eo <= O_TOL, f"O max abs err {eo}"
    assert el <= LSE_TOL, f"LSE max abs err {el}"
    return eo, el


def test_small_config_full():
    cfg = osm_inputs.attention_config("attn_small")
    _announce("attn_small", cfg["cfg"])
    q, k, v = (t.cuda() for t in (cfg["q"], cfg["k"], cfg["v"]))
    o, lse = osm.attn_fwd(q, k, v, cfg["scale"], cfg["causal"])
    torch.cuda.synchronize()
    eo, el = compare(q, k, v, cfg["scale"], cfg["causal"], o, lse)
    print(f"[result] attn_small O err {eo:.3g} LSE err {el:.3g}", flush=True)


ODD = [
    (1, 1, 1, 64), (1, 2, 17, 64), (2, 1, 64, 64), (1, 3, 100, 64), (1, 1, 129, 64),
    (1, 2, 255, 64), (1, 1, 1000, 64),
    (1, 1, 1, 128), (1, 2, 17, 128), (2, 1, 64, 128), (1, 3, 100, 128), (1, 1, 129, 128),
    (1, 2, 255, 128), (1, 1, 1000, 128), (1, 1, 2049, 128),
    # A ragged tail past 4096 (at this grid size still 128-row tiles).
    (1, 2, 4100, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,D", ODD)
def test_odd_shapes_full(B, H, N, D, causal):
    _announce("odd", B, H, N, D, causal)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=B * 1000 + H * 100 + N + D,
                                          device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    compare(q, k, v, scale, causal, o, lse)


# Grids with more query tiles than resident workgroups (MI355X: 256 compute
# units; 512 slots for 128-row tiles at D = 128, 768 at D = 64, 256 for the
# 256-row tiles of 8 wavefronts) run a persistent schedule.  With 128-row
# tiles (4 wavefronts) the workgroups claim tiles from a work queue
# (tests/test_gpu_attn_queue.py repeats such launches); with 256-row tiles
# query tiles are folded in pairs (p, n - 1 - p), the middle tile alone when
# n is odd, dealt over the heads of an XCD when B * H is a multiple of 8,
# else over all heads.
PERSISTENT_GRIDS = [
    (8, 40, 1920, 128, True),   # heads per XCD, 15 tiles of 128 rows
    (4, 50, 1152, 64, True),    # heads per XCD, D = 64, 9 tiles
    (3, 67, 1152, 64, True),    # B * H = 201: all heads
    (3, 3, 7900, 128, True),    # all heads, 8 wavefronts, 31 tiles, ragged
    (3, 3, 8100, 128, False),   # all heads, 8 wavefronts, unmasked, ragged
    (2, 8, 4200, 128, False),   # heads per XCD, 8 wavefronts, 17 tiles, ragged
]


@pytest.mark.parametrize("B,H,N,D,causal", PERSISTENT_GRIDS)
def test_persistent_schedules_sampled(B, H, N, D, causal):
    _announce("persistent", B, H, N, D, causal)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=N + H, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    rows_per_tile = 256 if (D == 128 and (not causal or N >= 4096)) else 128
    n_tiles = (N + rows_per_tile - 1) // rows_per_tile
    mid = (n_tiles // 2) * rows_per_tile
    rng = np.random.default_rng(N * 7 + H)
    rows = set(rng.choice(N, 96, replace=False).tolist())
    rows |= {0, 1, mid, mid + rows_per_tile // 2, min(mid + rows_per_tile, N) - 1}
    rows |= set(range(N - 8, N))
    rows = sorted(rows)
    for b, h in osm_inputs.sample_heads(B, H, 3, N, must=[(0, 0), (B - 1, H - 1)]):
        qh, kh, vh = (t[b, h].cpu().double().numpy() for t in (q, k, v))
        O, L = attention_head_ref(qh, kh, vh, scale, causal, query_rows=rows)
        eo = np.abs(o[b, h].cpu().double().numpy()[rows] - O).max()
        el = np.abs(lse[b, h].cpu().double().numpy()[rows] - L).max()
        assert eo <= O_TOL and el <= LSE_TOL, ((b, h), eo, el)


@pytest.mark.parametrize("D", [64, 128])
def test_closed_forms(D):
    _announce("closed forms", D)
    B, H, N = 1, 2, 200
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=77, device="cuda")
    # Causal row 0 sees only key 0: O = v_0, LSE = scale * q_0 . k_0.
    o, lse = osm.attn_fwd(q, k, v, 0.1, True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    s0 = 0.1 * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert (lse[:, :, 0].double() - s0).abs().max() < 1e-4
    # Identical keys: uniform weights over the visible keys.
    kk = k[:, :, :1].expand(B, H, N, D).contiguous()
    o, lse = osm.attn_fwd(q, kk, v, 0.1, True)
    torch.cuda.synchronize()
    cnt = torch.arange(1, N + 1, device="cuda", dtype=torch.float64)
    mean = v.double().cumsum(2) / cnt[None, None, :, None]
    assert (o.double() - mean).abs().max() < O_TOL
    want = 0.1 * (q.double() * kk.double()).sum(-1) + torch.log(cnt)
    assert (lse.double() - want).abs().max() < LSE_TOL


def test_deterministic_and_no_overrun():
    _announce("determinism/guard")
    B, H, N, D = 2, 3, 300, 128
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=5, device="cuda")
    pad = 8192
    obuf = torch.full((B * H * N * D + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * N + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + B * H * N * D].view(B, H, N, D)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    osm.attn_fwd(q, k, v, 0.088, True, out=o, lse=lse)
    o1, l1 = o.clone(), lse.clone()
    osm.attn_fwd(q, k, v, 0.088, True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)
    assert (obuf[:pad] == 7).all() and (obuf[pad + o.numel():] == 7).all()
    assert (lbuf[:pad] == 7).all() and (lbuf[pad + lse.numel():] == 7).all()


@pytest.mark.parametrize("name,count,must", [
    ("attn_llama13b", 8, [(0, 0), (7, 39)]),
    ("attn_long", 4, [(0, 0), (0, 31)]),
])
def test_large_configs_sampled_heads(name, count, must):
    cfg = osm_inputs.attention_config(name, device="cuda")
    c = cfg["cfg"]
    _announce(name, c)
    o, lse = osm.attn_fwd(cfg["q"], cfg["k"], cfg["v"], cfg["scale"], cfg["causal"])
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    heads = osm_inputs.sample_heads(c["B"], c["H"], count, c["seed"], must)
    sel = lambda t: torch.stack([t[b, h] for b, h in heads])[:, None]  # noqa: E731
    qs, ks, vs = sel(cfg["q"]), sel(cfg["k"]), sel(cfg["v"])
    os_, ls = sel(o), torch.stack([lse[b, h] for b, h in heads])[:, None]
    eo, el = compare(qs, ks, vs, cfg["scale"], cfg["causal"], os_, ls)
    print(f"[result] {name} heads {heads} O err {eo:.3g} LSE err {el:.3g}", flush=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_no_reads_past_the_head(D, causal):
    # K and V are followed in their allocation by NaN: a copy that read key
    # rows past N would bring NaN into the products (0 * NaN is NaN).
    B, H, N = 1, 2, 100
    _announce("NaN past the end", B, H, N, D, causal)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=31, device="cuda")
    pad = 64 * 128
    kb = torch.full((k.numel() + pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    vb = torch.full((v.numel() + pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    kb[:k.numel()].copy_(k.flatten())
    vb[:v.numel()].copy_(v.flatten())
    kk = kb[:k.numel()].view(B, H, N, D)
    vv = vb[:v.numel()].view(B, H, N, D)
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, kk, vv, scale, causal)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    compare(q, k, v, scale, causal, o, lse)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("slope,N", [(2.0, 300), (-2.0, 300), (6.0, 160), (-6.0, 160)])
def test_reference_moves_with_the_scores(slope, N, D, causal):
    # Scores that climb (or fall) steadily along the keys, `slope` log2 units
    # per key: every 32-key sub-tile lies 64 (or 192) log2 units above the
    # previous one, so the unmasked sub-tiles keep finding partial sums past
    # 2^64 (or +inf) and must move their reference; falling scores underflow
    # instead.  Magnitudes stay small enough that float32 scores keep the
    # LSE within its tolerance.
    B, H = 1, 2
    _announce("reference moves", slope, N, D, causal)
    scale = float(np.float32(1 / math.sqrt(D)))
    c = scale * math.log2(math.e)
    g = torch.Generator().manual_seed(int(abs(slope) * 10) + N + D)
    t = slope * torch.arange(N, dtype=torch.float32) / (c * D)
    k = (t[None, None, :, None] * (1 + 0.05 * torch.randn(B, H, N, D, generator=g)))
    q = torch.ones(B, H, N, D)
    v = torch.randn(B, H, N, D, generator=g)
    q, k, v = (x.to(torch.bfloat16).cuda() for x in (q, k, v))
    o, lse = osm.attn_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    compare(q, k, v, scale, causal, o, lse)


@pytest.mark.parametrize("D,N,causal", [(64, 300, False), (64, 300, True), (128, 1000, False),
                                        (128, 1000, True), (128, 4100, True)])
def test_output_rounds_to_nearest_even(D, N, causal):
    # Q = 0: every visible key weighs exactly the same and O is the mean of
    # the visible V rows, computed almost exactly in float32.  V in [4, 8)
    # puts O where bfloat16 values are 2^-5 apart: rounding to nearest even
    # stays within half of that, truncation errs by up to a whole step (and
    # beyond the 2e-2 budget).  The 8-wavefront kernels run at D = 128 for
    # unmasked rows and for causal rows of 4096 or more.
    B, H = 1, 2
    _announce("O rounding", B, H, N, D, causal)
    q, k, v = osm_inputs.attention_rounding_inputs(B, H, N, D, seed=41, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    O, L = attention_ref(q.cpu().double().numpy(), k.cpu().double().numpy(),
                         v.cpu().double().numpy(), scale, causal)
    got = o.cpu().double().numpy()
    bad = bf16_rne_violations(got, O, abs_slack=O_ABS_SLACK)
    assert not bad.any(), f"{bad.sum()} outputs beyond the nearest-even bound"
    assert np.abs(lse.cpu().double().numpy() - L).max() <= LSE_TOL


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_probabilities_round_to_nearest_even(D, causal):
    # Every key row of V is the same vector c, so O = c whatever the weights.
    # The kernel rounds P to bfloat16 before the P V product and divides by
    # the sum of the unrounded P: with nearest-even rounding the errors of
    # P average out over the keys and O rounds back to c exactly; truncated
    # P would lose about 0.3% on every row and miss c (tests/test_tolerance.py
    # shows both on the CPU for these inputs).
    B, H, N = 1, 2, 1024
    _announce("P rounding", B, H, N, D, causal)
    q, k, v = osm_inputs.attention_constant_v_inputs(B, H, N, D, seed=43, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    o, _ = osm.attn_fwd(q, k, v, scale, causal)
    torch.cuda.synchronize()
    rows = slice(CONSTANT_V_MIN_KEYS - 1, None) if causal else slice(None)
    got = o[:, :, rows]
    want = v[:, :, :1].expand_as(got)
    assert torch.equal(got, want), f"{(got != want).sum().item()} outputs differ from c"


def test_raw_abi_attention_small_config():
    # osm_attn_fwd itself (not the _ex form the tensor helper calls), raw
    # through ctypes, on the small non-causal workload, compared in full.
    cfg = osm_inputs.attention_config("attn_small", device="cuda")
    c = cfg["cfg"]
    _announce("raw osm_attn_fwd", c)
    q, k, v = cfg["q"], cfg["k"], cfg["v"]
    o = torch.empty_like(q)
    lse = torch.empty((c["B"], c["H"], c["N"]), dtype=torch.float32, device="cuda")
    st = osm.osm_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                          lse.data_ptr(), c["B"], c["H"], c["N"], c["D"], cfg["scale"],
                          int(cfg["causal"]), torch.cuda.current_stream().cuda_stream)
    assert st == osm.OSM_OK, osm.osm_status_string(st)
    torch.cuda.synchronize()
    eo, el = compare(q, k, v, cfg["scale"], cfg["causal"], o, lse)
    print(f"[result] raw osm_attn_fwd attn_small O err {eo:.3g} LSE err {el:.3g}", flush=True)


# Small grids (128-row query tiles for at most half the compute units) run
# 32-row workgroups whose four wavefronts split the key range and merge their
# partial states: at D = 64 for every such grid, at D = 128 up to 1024 keys
# (longer D = 128 rows keep the 128-row kernel, one workgroup per tile; the
# first cases).  Cases at the limits, with wavefronts left without keys
# (N < 128) and with key lengths (a batch without keys gives rows with O = 0
# and LSE = -inf).
SMALL_GRIDS = [
    (1, 8, 2048, 128, True, None),
    (1, 2, 4100, 128, False, None),
    (2, 2, 1500, 128, True, [1500, 700]),
    (1, 1, 16384, 128, True, None),
    (1, 1, 16384, 64, True, None),
    (1, 4, 4096, 64, True, None),
    (1, 8, 1024, 128, True, None),
    (1, 8, 1024, 128, False, None),
    (2, 3, 77, 128, False, None),
    (1, 2, 33, 64, True, None),
    (2, 4, 1000, 64, True, [1000, 0]),
    (2, 4, 700, 128, False, [513, 9]),
]


@pytest.mark.parametrize("B,H,N,D,causal,kv", SMALL_GRIDS)
def test_small_grid_key_split(B, H, N, D, causal, kv):
    _announce("small grid", B, H, N, D, causal, kv)
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=N + D + H, device="cuda")
    scale = float(np.float32(1 / math.sqrt(D)))
    kv_len = None if kv is None else torch.tensor(kv, dtype=torch.int32, device="cuda")
    o, lse = osm.attn_fwd(q, k, v, scale, causal, kv_len=kv_len)
    o2, l2 = osm.attn_fwd(q, k, v, scale, causal, kv_len=kv_len)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2), "run-to-run difference"
    og, lg = o.cpu().double().numpy(), lse.cpu().double().numpy()
    rng = np.random.default_rng(N)
    rows = None if N <= 1024 else sorted(set(rng.choice(N, 256, replace=False).tolist())
                                         | {0, 31, 32, 1023, 1024, N // 2, N - 1})
    for b in range(B):
        for h in range(H):
            qh, kh, vh = (t[b, h].cpu().double().numpy() for t in (q, k, v))
            O, L = attention_head_ref(qh, kh, vh, scale, causal, query_rows=rows,
                                      kv_len=None if kv is None else kv[b])
            ob = og[b, h] if rows is None else og[b, h][rows]
            lb = lg[b, h] if rows is None else lg[b, h][rows]
            dead = np.isneginf(L)
            assert (np.isneginf(lb) == dead).all() and (ob[dead] == 0).all(), (b, h)
            assert np.abs(ob - O).max() <= O_TOL, (b, h, np.abs(ob - O).max())
            assert np.abs(lb[~dead] - L[~dead]).max(initial=0) <= LSE_TOL, (b, h)
