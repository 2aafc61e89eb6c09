"""Seeded synthetic inputs for log-linear attention workloads.

This module only draws random numbers with the distributions of the workloads
below; it holds none of the attention arithmetic.  Both the HIP path (through
the tests and ``bench.py``) and the CPU oracle take their inputs from here.

Distributions (shared by every workload unless stated):
  q, k ~ N(0, 1) / sqrt(dk); v ~ N(0, 1);
  log a_t = -U(0.001, 0.1)   (per token and head);
  lambda_t^(l) = softplus(N(0.54, 0.5))   (per token, head and level; the 0.54
      centre is the initial bias that makes softplus start near 1 in the
      adaptive-decay page);
  Gated DeltaNet: k is L2-normalised per token, beta_t = sigmoid(N(0, 1)).
For bf16 workloads q, k, v are drawn in fp32 and rounded to bf16 (round to
nearest even); gates, lambda and beta stay fp32.

Each tensor has its own generator, seeded from the workload seed and the
tensor's index (q 0, k 1, v 2, log_gate 3, lambda 4, beta 5, one-hot level 6;
the level-weight MLP: d 7, W1 8, W2 9, bias 10; the query-contraction gate:
w 11, b 12, dense key direction 13), so any subset can be drawn alone and
yields the same values.

Level-weight MLP inputs (the adaptive-decay page's lambda producer, hidden
size 2L): d ~ N(0, 1) per token, head and level; W1 ~ N(0, 1/L);
W2 ~ N(0, 0.25/hidden); bias = 0.54 + 0.25 N(0, 1).  The page starts training
from W2 = 0 and bias 0.54 (every weight softplus(0.54), about 1); the random
W2 and bias stand in for a trained MLP, so that the weights differ per token
and level (mostly between 0.4 and 2).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

MAMBA2 = 0
GATED_DELTANET = 1


@dataclass(frozen=True)
class Workload:
    name: str
    rule: int
    B: int
    H: int
    T: int
    dk: int
    dv: int
    L: int
    C: int
    io: str  # "f32" or "bf16"
    seed: int
    steps: int = 0  # decode workloads: tokens decoded after a prefix of T tokens

    @property
    def torch_io(self) -> torch.dtype:
        return torch.float32 if self.io == "f32" else torch.bfloat16


WORKLOADS = {
    "tiny": Workload("mamba2 B1 H1 T256 d16 fp32 L9 C16", MAMBA2, 1, 1, 256, 16, 16, 9, 16, "f32", 0),
    "prefill-2k": Workload("mamba2 B4 H16 T2048 d64 bf16 L12 C64", MAMBA2, 4, 16, 2048, 64, 64, 12, 64, "bf16", 1),
    "prefill-16k": Workload("mamba2 B2 H16 T16384 d64 bf16 L15 C64", MAMBA2, 2, 16, 16384, 64, 64, 15, 64, "bf16",
                            2),
    # decode: resume from the per-level states of a 32768-token prefix, then
    # decode 512 tokens one at a time; positions up to 33279 need 17 levels.
    "decode-32k": Workload("decode B64 H16 d64 bf16 prefix 32768 +512 steps L17", MAMBA2, 64, 16, 32768, 64, 64,
                           17, 64, "bf16", 3, steps=512),
    "gdn-8k": Workload("gated-deltanet B2 H16 T8192 d128 bf16 L14 C64", GATED_DELTANET, 2, 16, 8192, 128, 128, 14,
                       64, "bf16", 4),
}


def levels_for(T: int) -> int:
    """ceil(log2 T) + 1 levels: level 0 plus one per power-of-two bucket size."""
    return max(1, math.ceil(math.log2(T))) + 1 if T > 1 else 2


def with_shape(w: Workload, **kw) -> Workload:
    """A copy of ``w`` with some fields replaced (smaller parity cases)."""
    return replace(w, **kw)


def _gen(seed: int, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 16 + index)
    return g


def _round_io(x: torch.Tensor, io: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if io == "bf16" else x


def prefill_inputs(w: Workload, device="cpu", variant: str = "default", seed: int | None = None,
                   parts=("q", "k", "v", "log_gate", "lam", "beta")) -> dict:
    """Inputs of one prefill over [B, T, H] tokens.

    variant:
      "default"   -- the distributions above;
      "nodecay"   -- log a == 0 (every level carries weight);
      "slowdecay" -- log a = -U(1e-5, 1e-4);
      "deep"      -- log a == 0 and lambda one-hot at a level drawn uniformly
                     per token and head, so that every level is read alone.
    ``parts`` selects which tensors to draw (the others are None).
    Returns q, k, v (io dtype), log_gate, lam, beta (fp32; beta None for Mamba-2).
    """
    s = w.seed if seed is None else seed
    B, T, H = w.B, w.T, w.H
    out = dict(q=None, k=None, v=None, log_gate=None, lam=None, beta=None)
    if "q" in parts:
        q = torch.randn(B, T, H, w.dk, generator=_gen(s, 0, device), device=device) / math.sqrt(w.dk)
        out["q"] = _round_io(q, w.io)
    if "k" in parts:
        k = torch.randn(B, T, H, w.dk, generator=_gen(s, 1, device), device=device)
        if w.rule == GATED_DELTANET:
            k = k / k.norm(dim=-1, keepdim=True)
        else:
            k = k / math.sqrt(w.dk)
        out["k"] = _round_io(k, w.io)
    if "v" in parts:
        out["v"] = _round_io(torch.randn(B, T, H, w.dv, generator=_gen(s, 2, device), device=device), w.io)
    if "log_gate" in parts:
        u = torch.rand(B, T, H, generator=_gen(s, 3, device), device=device)
        if variant in ("nodecay", "deep"):
            g = torch.zeros_like(u)
        elif variant == "slowdecay":
            g = -(1e-5 + 9e-5 * u)
        elif variant == "default":
            g = -(0.001 + 0.099 * u)
        else:
            raise ValueError(f"unknown variant {variant!r}")
        out["log_gate"] = g.contiguous()
    if "lam" in parts:
        if variant == "deep":
            hot = torch.randint(0, w.L, (B, T, H), generator=_gen(s, 6, device), device=device)
            lam = torch.nn.functional.one_hot(hot, w.L).to(torch.float32)
        else:
            z = torch.randn(B, T, H, w.L, generator=_gen(s, 4, device), device=device)
            lam = torch.nn.functional.softplus(0.54 + 0.5 * z)
        out["lam"] = lam.contiguous()
    if "beta" in parts and w.rule == GATED_DELTANET:
        out["beta"] = torch.sigmoid(torch.randn(B, T, H, generator=_gen(s, 5, device), device=device)).contiguous()
    return out


def decode_inputs(w: Workload, device="cpu", seed: int | None = None) -> dict:
    """Per-step inputs of ``w.steps`` decode tokens after a ``w.T``-token prefix.

    Shapes drop T and gain a leading step axis: q, k [S,B,H,dk], v [S,B,H,dv],
    log_gate/beta [S,B,H], lam [S,B,H,L].  Same distributions as a prefill.
    The generator seed is offset from the prefix's so the two never overlap.
    """
    step_w = replace(w, T=w.steps, B=w.B)
    x = prefill_inputs(step_w, device=device, seed=(w.seed if seed is None else seed) + 1000)
    # [B, S, H, ...] -> [S, B, H, ...]
    out = {}
    for name, t in x.items():
        out[name] = None if t is None else t.transpose(0, 1).contiguous()
    return out


def softplus(x: float) -> float:
    """log(1 + e^x), the activation that produces lambda."""
    return math.log1p(math.exp(x))


def lambda_mlp_inputs(lead: tuple, L: int, hidden: int | None = None, seed: int = 0, device="cpu") -> dict:
    """Inputs of the level-weight MLP: d [*lead, L] and weights W1 [L, hidden],
    W2 [hidden, L], bias [L] (fp32; hidden defaults to 2L)."""
    hidden = 2 * L if hidden is None else hidden
    d = torch.randn(*lead, L, generator=_gen(seed, 7, device), device=device)
    w1 = torch.randn(L, hidden, generator=_gen(seed, 8, device), device=device) / math.sqrt(L)
    w2 = torch.randn(hidden, L, generator=_gen(seed, 9, device), device=device) * (0.5 / math.sqrt(hidden))
    bias = 0.54 + 0.25 * torch.randn(L, generator=_gen(seed, 10, device), device=device)
    return dict(d=d.contiguous(), w1=w1.contiguous(), w2=w2.contiguous(), bias=bias.contiguous())


def ccq_inputs(H: int, dk: int, seed: int = 0, device="cpu") -> dict:
    """Gate of the curvature-conditioned query per head: w [H, dk] ~ N(0, 1/dk),
    b [H] ~ N(0, 1) (fp32)."""
    w = torch.randn(H, dk, generator=_gen(seed, 11, device), device=device) / math.sqrt(dk)
    b = torch.randn(H, generator=_gen(seed, 12, device), device=device)
    return dict(w=w.contiguous(), b=b.contiguous())


def with_dense_key_direction(k: torch.Tensor, scale: float = 3.0, seed: int = 0) -> torch.Tensor:
    """Keys with one crowded direction per head: k + scale N(0, 1) u_h, u_h a
    random unit vector of head h (zero mean, so the running covariance has an
    eigenvalue near scale^2 along u_h).  Returned in k's dtype."""
    B, T, H, dk = k.shape
    g = _gen(seed, 13, "cpu")
    u = torch.randn(H, dk, generator=g)
    u = u / u.norm(dim=-1, keepdim=True)
    a = torch.randn(B, T, H, 1, generator=g) * scale
    return (k.float().cpu() + a * u).to(k.dtype).to(k.device)
