"""Seeded synthetic inputs for the gated delta rule.

This module only draws random numbers; it contains none of the recurrence's
arithmetic, so both the GPU tests and the CPU oracle can take their inputs from
it.  Recipe (the pages give no data, only the workload structure):

* batch 1, 16 query/key heads shared 2:1 by 32 value heads, dk = dv = 128 for the
  full-size workloads (the pages' model pairs 30 recurrent layers with 10 attention
  layers; "Optimizing on-device inference for Apple Silicon", section "Qwen creates
  three distinct workload shapes");
* one generator per workload, ``torch.Generator('cpu')`` seeded, draws in the order
  q, k, v, g, beta, state, all in fp32;
* q, k ~ N(0, 1), then divided by their L2 norm per token (in fp32), then cast to
  the storage dtype -- the layer normalises queries and keys before the recurrence;
* v ~ N(0, 1); g = -softplus(N(g_mean, 1)) so a = exp(g) lies in (0, 1);
  beta = sigmoid(N(beta_mean, 1));
* an initial state, when asked for, ~ N(0, state_std^2) in fp32;
* the state and the gates stay fp32, q/k/v are stored in bf16 (section "Keep the
  recurrent state on chip": state and gate in fp32, query and key in bf16).

All tensors are returned on the CPU; callers move them where they need them.
"""
from dataclasses import dataclass
from typing import Optional

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    Hk: int
    Hv: int
    dk: int
    dv: int
    chunk: int
    seed: int
    g_mean: float = 0.0
    beta_mean: float = 0.0


# The five workloads the library is checked and measured on.
TINY = Workload("tiny_T64_H2_d32_c16", 1, 64, 2, 2, 32, 32, 16, 0)
PREFILL_4K = Workload("prefill_T4096_Hk16_Hv32_d128_c64", 1, 4096, 16, 32, 128, 128, 64, 0)
CONTINUATION_32K = Workload("continuation_T32768_Hk16_Hv32_d128_c64", 1, 32768, 16, 32, 128, 128,
                            64, 1)
LONG_128K = Workload("long_T131072_Hk16_Hv32_d128_c64_longmem", 1, 131072, 16, 32, 128, 128, 64,
                     2, g_mean=-4.0, beta_mean=2.0)
DECODE_LAYERS = 30          # independent recurrent layers one decode token passes through
DECODE_SHAPE = dict(B=1, Hk=16, Hv=32, dk=128, dv=128)
DECODE_STATE_STD = 0.1
DECODE_SEED0 = 100          # layer l uses seed 100 + l


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_inputs(B, T, Hk, Hv, dk, dv, seed, dtype=torch.bfloat16, g_mean=0.0, beta_mean=0.0,
                state_std: Optional[float] = None, unit_qk: bool = True, device="cpu"):
    """Returns dict(q, k, v, g, beta, state) of tensors on ``device`` (CPU by default; the
    values depend on the device's generator, so a draw on another device is a different draw
    of the same recipe).

    q, k [B,T,Hk,dk] and v [B,T,Hv,dv] in ``dtype``; g, beta [B,T,Hv] fp32;
    state [B,Hv,dv,dk] fp32 or None.  unit_qk=False leaves q and k unnormalised, as raw
    projections: N(0, 1) entries times a per-token length factor exp(N(0, 0.5^2)), drawn
    after everything else so the other tensors equal the unit_qk=True draw."""
    gen = torch.Generator(device).manual_seed(int(seed))
    rn = lambda *shape: torch.randn(*shape, generator=gen, device=device)  # noqa: E731
    qr = rn(B, T, Hk, dk)
    kr = rn(B, T, Hk, dk)
    v = rn(B, T, Hv, dv).to(dtype)
    g = -F.softplus(rn(B, T, Hv) + g_mean)
    beta = torch.sigmoid(rn(B, T, Hv) + beta_mean)
    state = None
    if state_std is not None:
        state = rn(B, Hv, dv, dk) * state_std
    if unit_qk:
        q, k = _unit(qr).to(dtype), _unit(kr).to(dtype)
    else:
        q = (qr * torch.exp(0.5 * rn(B, T, Hk, 1))).to(dtype)
        k = (kr * torch.exp(0.5 * rn(B, T, Hk, 1))).to(dtype)
    return dict(q=q, k=k, v=v, g=g.contiguous(), beta=beta.contiguous(), state=state)


def workload_inputs(w: Workload, dtype=torch.bfloat16, T: Optional[int] = None):
    """Inputs of a named workload (optionally only its first T tokens' worth of
    shape -- a different draw; use slicing of the full draw for prefixes)."""
    return make_inputs(w.B, w.T if T is None else T, w.Hk, w.Hv, w.dk, w.dv, w.seed, dtype,
                       w.g_mean, w.beta_mean)


def decode_inputs(layer: int, dtype=torch.bfloat16, B: int = 1):
    """One decode token for recurrent layer ``layer``: q, k [B,Hk,dk], v [B,Hv,dv],
    g, beta [B,Hv], state [B,Hv,dv,dk] ~ N(0, 0.1^2)."""
    s = DECODE_SHAPE
    d = make_inputs(B, 1, s["Hk"], s["Hv"], s["dk"], s["dv"], DECODE_SEED0 + layer, dtype,
                    state_std=DECODE_STATE_STD)
    return dict(q=d["q"][:, 0].contiguous(), k=d["k"][:, 0].contiguous(),
                v=d["v"][:, 0].contiguous(), g=d["g"][:, 0].contiguous(),
                beta=d["beta"][:, 0].contiguous(), state=d["state"])
