"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle runs.

This module draws random numbers and lays them out; it holds none of the
softmax or attention arithmetic.  The same tensors are fed to the HIP library
(on the device) and to the CPU oracle (copied to the host).

Workloads (sizes and value distributions of the five standard configurations):

1. ``softmax_small``: row softmax, float32, 64 rows x 1000 columns.
   Rows 0-47 are 3*N(0,1); rows 48-55 are 3*N(0,1) + 1000 (overflow rows);
   rows 56-59 have their first 300 entries set to -inf; rows 60-61 are all -inf;
   rows 62-63 use only their first 100 columns (a separate cols=100 call).
   Plus the worked-example row (1, 5, 3) as a cols=3 call.
2. ``softmax_large``: 32768 x 8192, 4*N(0,1) with each entry independently set
   to -inf with probability 0.01; one float32 run and one bfloat16 run.
3. ``attn_small``: B=1, H=8, N=1024, D=64, non-causal, Q, K, V ~ N(0,1) drawn
   in that order, rounded to bfloat16; scale = 1/8.
4. ``attn_llama13b``: B=8, H=40, N=2048, D=128, causal, Q, K, V ~ N(0,1);
   scale = float32(1/sqrt(128)).  Shaped like one LLaMA-2-13B attention layer.
5. ``attn_long``: B=1, H=32, N=16384, D=128, causal, Q, K ~ 1.5*N(0,1),
   V ~ N(0,1); scale = float32(1/sqrt(128)).

Attention backward: the same Q, K, V plus an upstream gradient dO ~ N(0,1)
in bfloat16, drawn from its own generator seeded with 1000 + the seed.

"N(mu, sigma)" is read with sigma the standard deviation.  Seeds are the
configuration number (1-5).  Random draws are float32 from a torch generator
on the requested device, in a fixed order; bfloat16 tensors are round-to-nearest
-even casts of those draws.
"""

import math

import torch

NEG_INF = float("-inf")

SOFTMAX_SMALL = dict(name="softmax_small", seed=1, rows=64, cols=1000)
SOFTMAX_LARGE = dict(name="softmax_large", seed=2, rows=32768, cols=8192)
ATTN_SMALL = dict(name="attn_small", seed=3, B=1, H=8, N=1024, D=64, causal=False,
                  qk_sigma=1.0, v_sigma=1.0)
ATTN_LLAMA13B = dict(name="attn_llama13b", seed=4, B=8, H=40, N=2048, D=128, causal=True,
                     qk_sigma=1.0, v_sigma=1.0)
ATTN_LONG = dict(name="attn_long", seed=5, B=1, H=32, N=16384, D=128, causal=True,
                 qk_sigma=1.5, v_sigma=1.0)

ATTN_CONFIGS = {c["name"]: c for c in (ATTN_SMALL, ATTN_LLAMA13B, ATTN_LONG)}


def generator(seed, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def softmax_small(device="cpu"):
    """The 64 x 1000 special-row matrix and its three calls.

    Returns a dict with ``x`` (64, 1000) float32 and ``calls``, a list of
    (label, tensor) pairs, each a contiguous row-major matrix handed to one
    softmax call: A = rows 0-61 (cols 1000), B = rows 62-63 truncated to their
    first 100 columns (cols 100), C = the row (1, 5, 3) (cols 3).
    """
    c = SOFTMAX_SMALL
    g = generator(c["seed"], device)
    x = 3.0 * torch.randn(c["rows"], c["cols"], generator=g, device=device, dtype=torch.float32)
    x[48:56] += 1000.0
    x[56:60, :300] = NEG_INF
    x[60:62, :] = NEG_INF
    calls = [
        ("A_rows0-61_cols1000", x[0:62].contiguous()),
        ("B_rows62-63_cols100", x[62:64, :100].contiguous()),
        ("C_worked_example", torch.tensor([[1.0, 5.0, 3.0]], dtype=torch.float32, device=device)),
    ]
    return {"x": x, "calls": calls}


def softmax_rows(rows, cols, seed, sigma=4.0, ninf_prob=0.01, dtype=torch.float32,
                 device="cpu"):
    """sigma*N(0,1) entries, each -inf with probability ``ninf_prob``.

    The float32 draw comes first; ``dtype`` = bfloat16 rounds it (RNE).
    """
    g = generator(seed, device)
    x = sigma * torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    if ninf_prob > 0:
        u = torch.rand(rows, cols, generator=g, device=device, dtype=torch.float32)
        x.masked_fill_(u < ninf_prob, NEG_INF)
    return x.to(dtype) if dtype != torch.float32 else x


def softmax_large(dtype=torch.float32, device="cpu", rows=None, cols=None):
    c = SOFTMAX_LARGE
    return softmax_rows(rows or c["rows"], cols or c["cols"], c["seed"], sigma=4.0,
                        ninf_prob=0.01, dtype=dtype, device=device)


def attention_inputs(B, H, N, D, seed, qk_sigma=1.0, v_sigma=1.0, device="cpu"):
    """Q, K, V of shape [B, H, N, D] in bfloat16, drawn in the order Q, K, V."""
    g = generator(seed, device)
    shape = (B, H, N, D)
    q = (qk_sigma * torch.randn(shape, generator=g, device=device)).to(torch.bfloat16)
    k = (qk_sigma * torch.randn(shape, generator=g, device=device)).to(torch.bfloat16)
    v = (v_sigma * torch.randn(shape, generator=g, device=device)).to(torch.bfloat16)
    return q, k, v


def attention_grad_output(B, H, N, D, seed, device="cpu"):
    """Upstream gradient dO of shape [B, H, N, D], N(0,1) in bfloat16, from its
    own generator (seed 1000 + seed), so Q, K, V are unchanged by drawing it."""
    g = generator(1000 + int(seed), device)
    return torch.randn((B, H, N, D), generator=g, device=device).to(torch.bfloat16)


def attention_rounding_inputs(B, H, N, D, seed, device="cpu"):
    """Inputs that expose the rounding of the attention output.

    Q = 0, so every visible key gets the same weight; K ~ N(0,1); V = 4 +
    3.9 U(0,1) rounded to bfloat16, so V and every average of its rows lie in
    [4, 8), where bfloat16 values are 2^-5 apart.  Drawn in the order K, V.
    """
    g = generator(seed, device)
    shape = (B, H, N, D)
    q = torch.zeros(shape, device=device, dtype=torch.bfloat16)
    k = torch.randn(shape, generator=g, device=device).to(torch.bfloat16)
    v = (4.0 + 3.9 * torch.rand(shape, generator=g, device=device)).to(torch.bfloat16)
    return q, k, v


#: Values of the constant V rows of ``attention_constant_v_inputs``: bfloat16
#: numbers at the bottom (1, 2, 0.5) and top (255/128, 255/64) of a binade.
CONSTANT_V_VALUES = (1.0, 255.0 / 128.0, 2.0, 255.0 / 64.0, 0.5, 255.0 / 256.0)


def attention_constant_v_inputs(B, H, N, D, seed, device="cpu"):
    """Q, K ~ N(0,1) (in that order) and V with every key row equal to one
    vector c, whose entries cycle through ``CONSTANT_V_VALUES``."""
    g = generator(seed, device)
    shape = (B, H, N, D)
    q = torch.randn(shape, generator=g, device=device).to(torch.bfloat16)
    k = torch.randn(shape, generator=g, device=device).to(torch.bfloat16)
    c = torch.tensor([CONSTANT_V_VALUES[d % len(CONSTANT_V_VALUES)] for d in range(D)],
                     dtype=torch.bfloat16, device=device)
    v = c.expand(shape).contiguous()
    return q, k, v


def attention_config(name, device="cpu", **override):
    """Inputs of one named attention workload; ``override`` changes sizes."""
    c = dict(ATTN_CONFIGS[name])
    c.update(override)
    q, k, v = attention_inputs(c["B"], c["H"], c["N"], c["D"], c["seed"], c["qk_sigma"],
                               c["v_sigma"], device=device)
    scale = float(torch.tensor(1.0 / math.sqrt(c["D"]), dtype=torch.float32))
    return dict(q=q, k=k, v=v, scale=scale, causal=c["causal"], cfg=c)


def sample_heads(B, H, count, seed, must=()):
    """A seeded choice of ``count`` distinct (b, h) slices, including ``must``."""
    g = torch.Generator().manual_seed(int(seed) + 1000)
    chosen = list(dict.fromkeys(tuple(m) for m in must))
    perm = torch.randperm(B * H, generator=g).tolist()
    for p in perm:
        if len(chosen) >= min(count, B * H):
            break
        bh = (p // H, p % H)
        if bh not in chosen:
            chosen.append(bh)
    return chosen
