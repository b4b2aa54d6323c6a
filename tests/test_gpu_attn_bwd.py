"""GPU parity of osm_attn_bwd (attention backward) against the float64 oracle.

The library is fed bfloat16 Q, K, V, dO and the forward's O (bfloat16) and
LSE (float32).  Most cases take O and LSE from the oracle (rounded to those
types), so that only the backward's own arithmetic is measured; one case runs
the library's forward first, as a training step would.

Tolerance, elementwise, from the arithmetic of the kernels (u = 2^-9, the
bfloat16 unit roundoff):
  * P enters dV = P^T dO as bfloat16: |err dV| <= u (P^T |dO|), plus the final
    rounding u |dV|.
  * dS = P (dP - Delta) is rounded to bfloat16 (u |dS|), and Delta is formed
    from the bfloat16 O (|dDelta_i| <= u A_i, A_i = sum_d |dO_id O_id|), so
    |err dK| <= u scale (|dS| + P A)^T |Q| + u |dK| and
    |err dQ| <= u scale (|dS| + P A) |K| + u |dQ|.
Float32 accumulation, the hardware exp2 and the float32 LSE add terms far
below these; the test allows twice each bound (2u = 2^-8).  With the
library's own forward, O carries its own error (at most about 2u (P |V|) per
element), so A is taken with P |V| in place of |O| and the factor is 4u.
"""

import math

import numpy as np
import pytest
import torch

import online_softmax_06_amd as osm
import osm_inputs
from oracle import attention_bwd_head_ref, attention_dq_rows_ref, attention_ref

pytestmark = pytest.mark.gpu

U = 2.0 ** -9


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    osm.load_library()


def _announce(*what):
    print("[case]", *what, flush=True)


def _inputs(B, H, N, D, seed, qk_sigma=1.0):
    q, k, v = osm_inputs.attention_inputs(B, H, N, D, seed=seed, qk_sigma=qk_sigma)
    do = osm_inputs.attention_grad_output(B, H, N, D, seed=seed)
    return q, k, v, do


def _oracle_fwd(q, k, v, scale, causal, kv_len=None):
    O, L = attention_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(), scale, causal,
                         kv_len=kv_len)
    return (torch.from_numpy(O).to(torch.bfloat16), torch.from_numpy(L).to(torch.float32))


def _check_head(qh, kh, vh, doh, oh, scale, causal, got, factor=2.0, o_from_forward=False,
                kv_len=None):
    """Compare one head's (dq, dk, dv) with the oracle within the bound above."""
    q64, k64, v64, do64 = (t.double().numpy() for t in (qh, kh, vh, doh))
    dQ, dK, dV, P, dS = attention_bwd_head_ref(q64, k64, v64, do64, scale, causal,
                                               kv_len=kv_len, return_probs=True)
    c = float(np.float32(scale))
    if o_from_forward:
        A = np.sum(np.abs(do64) * (P @ np.abs(v64)), axis=1)
    else:
        A = np.sum(np.abs(do64) * np.abs(oh.double().numpy()), axis=1)
    W = np.abs(dS) + P * A[:, None]
    bounds = {
        "dq": factor * U * (c * (W @ np.abs(k64)) + np.abs(dQ)),
        "dk": factor * U * (c * (W.T @ np.abs(q64)) + np.abs(dK)),
        "dv": factor * U * (P.T @ np.abs(do64) + np.abs(dV)),
    }
    for name, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
        g = got[name].double().cpu().numpy()
        assert np.isfinite(g).all(), name
        err = np.abs(g - ref)
        bad = err > bounds[name] + 1e-30
        assert not bad.any(), (name, float(err.max()), float((err / (bounds[name] + 1e-30)).max()),
                               np.argwhere(bad)[:3].tolist())


def _run(q, k, v, o, lse, do, scale, causal):
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    dq, dk, dv = osm.attn_bwd(*dev, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return {"dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}


# Shapes: a single row, ragged tails within one tile, several key blocks and
# query tiles with ragged ends, tile-aligned sizes.
SHAPES = [(1, 1, 1), (1, 2, 17), (1, 2, 100), (1, 1, 128), (2, 2, 129), (1, 2, 300),
          (1, 1, 513), (1, 1, 640)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", SHAPES)
def test_bwd_matches_oracle(B, H, N, causal, D):
    _announce("attn_bwd", B, H, N, D, causal)
    q, k, v, do = _inputs(B, H, N, D, seed=N * 3 + D + int(causal))
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = _oracle_fwd(q, k, v, scale, causal)
    got = _run(q, k, v, o, lse, do, scale, causal)
    for b in range(B):
        for h in range(H):
            _check_head(q[b, h], k[b, h], v[b, h], do[b, h], o[b, h], scale, causal,
                        {n: t[b, h] for n, t in got.items()})


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_peaky_logits(causal):
    # Q, K ~ 1.5 N(0,1) as in the long-context workload: sharper rows.
    B, H, N, D = 1, 2, 384, 128
    _announce("attn_bwd peaky", B, H, N, D, causal)
    q, k, v, do = _inputs(B, H, N, D, seed=77, qk_sigma=1.5)
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = _oracle_fwd(q, k, v, scale, causal)
    got = _run(q, k, v, o, lse, do, scale, causal)
    for h in range(H):
        _check_head(q[0, h], k[0, h], v[0, h], do[0, h], o[0, h], scale, causal,
                    {n: t[0, h] for n, t in got.items()})


@pytest.mark.parametrize("D,causal", [(64, False), (128, True)])
def test_bwd_after_library_forward(D, causal):
    B, H, N = 2, 2, 333
    _announce("attn_bwd after forward", B, H, N, D, causal)
    q, k, v, do = (t.cuda() for t in _inputs(B, H, N, D, seed=5 + D))
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, k, v, scale, causal)
    dq, dk, dv = osm.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=causal)
    torch.cuda.synchronize()
    got = {"dq": dq.cpu(), "dk": dk.cpu(), "dv": dv.cpu()}
    for b in range(B):
        for h in range(H):
            _check_head(q[b, h].cpu(), k[b, h].cpu(), v[b, h].cpu(), do[b, h].cpu(), None, scale,
                        causal, {n: t[b, h] for n, t in got.items()}, factor=4.0,
                        o_from_forward=True)


def test_bwd_deterministic_and_workspace_reuse():
    B, H, N, D = 1, 3, 257, 128
    _announce("attn_bwd deterministic", B, H, N, D)
    q, k, v, do = (t.cuda() for t in _inputs(B, H, N, D, seed=9))
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = osm.attn_fwd(q, k, v, scale, True)
    a = osm.attn_bwd(q, k, v, o, lse, do, scale=scale, causal=True)
    # A second call into a dirty workspace and dirty outputs.
    need = osm.osm_attn_bwd_workspace(B, H, N, D)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")
    outs = [torch.full_like(q, float("nan")) for _ in range(3)]
    st = osm.osm_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                          do.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(),
                          outs[2].data_ptr(), B, H, N, D, scale, 1, ws.data_ptr(), need,
                          torch.cuda.current_stream().cuda_stream)
    assert st == osm.OSM_OK
    torch.cuda.synchronize()
    for x, y in zip(a, outs):
        assert torch.equal(x, y)


def test_bwd_full_size_llama13b_sampled():
    # The LLaMA-2-13B-shaped layer at full size (B8 H40 N2048 D128, causal);
    # three sampled heads against the oracle, every head against two
    # identities that hold at any size.
    cfg = osm_inputs.attention_config("attn_llama13b", device="cuda")
    c = cfg["cfg"]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    _announce("attn_bwd full size", B, H, N, D)
    q, k, v = cfg["q"], cfg["k"], cfg["v"]
    do = osm_inputs.attention_grad_output(B, H, N, D, seed=c["seed"], device="cuda")
    o, lse = osm.attn_fwd(q, k, v, cfg["scale"], True)
    dq, dk, dv = osm.attn_bwd(q, k, v, o, lse, do, scale=cfg["scale"], causal=True)
    torch.cuda.synchronize()
    # Sum over keys of dK is 0; sum over keys of dV is the sum over rows of dO.
    dk_sum = dk.float().sum(dim=2)
    dv_sum = dv.float().sum(dim=2)
    do_sum = do.float().sum(dim=2)
    assert dk_sum.abs().max().item() < 0.05 * dk.float().abs().sum(dim=2).max().item() + 1e-3
    assert (dv_sum - do_sum).abs().max().item() < 4 * U * do.float().abs().sum(dim=2).max().item()
    for (b, h) in osm_inputs.sample_heads(B, H, 3, seed=c["seed"], must=[(B - 1, H - 1)]):
        _announce("  head", b, h)
        _check_head(q[b, h].cpu(), k[b, h].cpu(), v[b, h].cpu(), do[b, h].cpu(), None,
                    cfg["scale"], True, {"dq": dq[b, h].cpu(), "dk": dk[b, h].cpu(),
                                         "dv": dv[b, h].cpu()},
                    factor=4.0, o_from_forward=True)


def test_bwd_small_config_full():
    # The small workload (B1 H8 N1024 D64, non-causal) at full size, every head.
    cfg = osm_inputs.attention_config("attn_small", device="cuda")
    c = cfg["cfg"]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    _announce("attn_bwd small config", B, H, N, D)
    q, k, v = cfg["q"], cfg["k"], cfg["v"]
    do = osm_inputs.attention_grad_output(B, H, N, D, seed=c["seed"], device="cuda")
    o, lse = osm.attn_fwd(q, k, v, cfg["scale"], cfg["causal"])
    dq, dk, dv = osm.attn_bwd(q, k, v, o, lse, do, scale=cfg["scale"], causal=cfg["causal"])
    torch.cuda.synchronize()
    for h in range(H):
        _check_head(q[0, h].cpu(), k[0, h].cpu(), v[0, h].cpu(), do[0, h].cpu(), None,
                    cfg["scale"], cfg["causal"], {"dq": dq[0, h].cpu(), "dk": dk[0, h].cpu(),
                                                  "dv": dv[0, h].cpu()},
                    factor=4.0, o_from_forward=True)


def test_bwd_long_context_sampled():
    # The long-context workload (B1 H32 N16384 D128, causal, Q and K ~ 1.5
    # N(0,1)) at full size: dQ of sampled rows of two heads against the
    # oracle, dK and dV of every head against the two identities.
    cfg = osm_inputs.attention_config("attn_long", device="cuda")
    c = cfg["cfg"]
    B, H, N, D = c["B"], c["H"], c["N"], c["D"]
    _announce("attn_bwd long context", B, H, N, D)
    q, k, v = cfg["q"], cfg["k"], cfg["v"]
    do = osm_inputs.attention_grad_output(B, H, N, D, seed=c["seed"], device="cuda")
    o, lse = osm.attn_fwd(q, k, v, cfg["scale"], True)
    dq, dk, dv = osm.attn_bwd(q, k, v, o, lse, do, scale=cfg["scale"], causal=True)
    torch.cuda.synchronize()
    dk_sum = dk.float().sum(dim=2)
    dv_sum = dv.float().sum(dim=2)
    do_sum = do.float().sum(dim=2)
    assert dk_sum.abs().max().item() < 0.05 * dk.float().abs().sum(dim=2).max().item() + 1e-3
    assert (dv_sum - do_sum).abs().max().item() < 4 * U * do.float().abs().sum(dim=2).max().item()
    rows = [0, 1, 63, 64, 1000, 8191, 8192, 12345, N - 2, N - 1]
    for h in (0, H - 1):
        _announce("  head", h)
        qh, kh, vh, gh, oh = (t[0, h].double().cpu().numpy() for t in (q, k, v, do, o))
        ref = attention_dq_rows_ref(qh, kh, vh, gh, cfg["scale"], True, rows)
        got = dq[0, h].double().cpu().numpy()[rows]
        # The dQ bound of the module docstring, row by row, with |O| taken as
        # P |V| (the library's forward output) and factor 4.
        c32 = float(np.float32(cfg["scale"]))
        for n, i in enumerate(rows):
            s = c32 * (kh[:i + 1] @ qh[i])
            P = np.exp(s - s.max())
            P /= P.sum()
            dP = vh[:i + 1] @ gh[i]
            dS = P * (dP - np.sum(P * dP))
            A = np.sum(np.abs(gh[i]) * (P @ np.abs(vh[:i + 1])))
            bound = 4 * U * (c32 * ((np.abs(dS) + P * A) @ np.abs(kh[:i + 1])) + np.abs(ref[n]))
            err = np.abs(got[n] - ref[n])
            assert (err <= bound + 1e-30).all(), (h, i, float(err.max()),
                                                   float((err / (bound + 1e-30)).max()))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_kv_len(D, causal):
    # Key padding: a full batch, a length inside a key block, no keys at all,
    # a short one.  Hidden keys get dk = dv = 0; rows without a visible key
    # (LSE = -inf) contribute nothing.
    B, H, N = 4, 2, 300
    lens = [300, 129, 0, 37]
    _announce("attn_bwd kv_len", B, H, N, D, causal, lens)
    q, k, v, do = _inputs(B, H, N, D, seed=31 + D + int(causal))
    scale = float(np.float32(1 / math.sqrt(D)))
    o, lse = _oracle_fwd(q, k, v, scale, causal, kv_len=np.array(lens))
    dev = [t.cuda() for t in (q, k, v, o, lse, do)]
    dq, dk, dv = osm.attn_bwd(*dev, scale=scale, causal=causal,
                              kv_len=torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for b in range(B):
        assert (dk[b, :, lens[b]:] == 0).all() and (dv[b, :, lens[b]:] == 0).all()
        for h in range(H):
            _check_head(q[b, h], k[b, h], v[b, h], do[b, h], o[b, h], scale, causal,
                        {"dq": dq[b, h].cpu(), "dk": dk[b, h].cpu(), "dv": dv[b, h].cpu()},
                        kv_len=lens[b])
