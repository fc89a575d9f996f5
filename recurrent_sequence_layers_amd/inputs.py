"""Seeded synthetic inputs for the Q-Delta layer (shared by tests, smoke and bench).

This module draws random numbers and shapes them into the workloads; it holds
none of the layer's arithmetic.  Both the HIP path and the CPU oracle consume
exactly the tensors returned here (the oracle takes fp64 upcasts of the very
values handed to the GPU, after any bf16 rounding).

Recipe (one torch generator per call, draws in this order):
  q, k ~ N(0, 1), each L2-normalised over the key dimension per (token, head)
  v    ~ N(0, 1)
  beta   = sigmoid(N(0, 1))
  alpha  = exp(-softplus(N(-4, 1)))          in (0, 1), typically about 0.98
  lambda = sigmoid(N(0, 1))
  S0     ~ N(0, s0_std) when requested (s0_std is a standard deviation)
then q, k, v are cast to the requested dtype (round to nearest even for bf16);
gates and states stay fp32.  These stand in for the language-model activations
the pages train on; no dataset is involved.
"""
from dataclasses import dataclass, field
from typing import Optional

import torch

# Workloads named by what they are, with their sizes.
WORKLOADS = {
    "tiny_fp32": dict(B=1, T=256, H=1, dk=64, dv=64, C=64, dtype="f32"),
    "layer_1p3b_bf16": dict(B=8, T=4096, H=16, dk=128, dv=128, C=64, dtype="bf16"),
    "gdn_bf16": dict(B=8, T=4096, H=16, dk=128, dv=128, C=64, dtype="bf16", lam="zero"),
    "deltanet_bf16": dict(B=8, T=4096, H=16, dk=128, dv=128, C=64, dtype="bf16",
                          lam="zero", alpha="one"),
    "long_64k_bf16": dict(B=1, T=65536, H=16, dk=128, dv=128, C=64, dtype="bf16", s0_std=0.02),
    "decode_256x16": dict(N=256, H=16, dk=128, dv=128, dtype="bf16", steps=1000, s0_std=0.02),
}

_DT = {"f32": torch.float32, "bf16": torch.bfloat16,
       torch.float32: torch.float32, torch.bfloat16: torch.bfloat16}


def torch_dtype(name):
    return _DT[name]


@dataclass
class ChunkInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    alpha: Optional[torch.Tensor]
    beta: torch.Tensor
    lam: Optional[torch.Tensor]
    S0: Optional[torch.Tensor]
    meta: dict = field(default_factory=dict)


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def chunk_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, lam="random", alpha="random",
                 s0_std=None, device="cpu", gates_as_none=False, key_corr=0.0,
                 alpha_logit_mean=-4.0) -> ChunkInputs:
    """Inputs for the layer forward, layout q,k [B,T,H,dk], v [B,T,H,dv],
    gates [B,T,H], S0 [B,H,dv,dk].

    lam:   "random" (sigmoid draw), "zero", "one", or a float constant.
    alpha: "random" (exp(-softplus) draw) or "one".
    gates_as_none: return None for alpha == 1 / lambda == 0 (the library's way of
    selecting the specialised instances); the tensors are still drawn so that the
    other draws do not shift.
    key_corr: weight of one shared N(0, 1) direction per (batch, head) added to every
    q and k before normalisation (drawn last, so the other draws do not shift); at 2
    the keys of a head have mean pairwise cosine about 0.8, at 3 about 0.9, a stress
    case for the triangular solve.
    alpha_logit_mean: mean of the decay logit a, alpha = exp(-softplus(a)).  The default
    -4 gives alpha about 0.98; +1 gives strong decay (median about 0.27, down to about
    0.05 at two standard deviations), so a 64-token chunk's cumulative decay reaches the
    bottom of the fp32 range."""
    dt = _DT[dtype]
    g = _generator(seed, device)
    f = dict(generator=g, device=device, dtype=torch.float32)
    q = torch.randn(B, T, H, dk, **f)
    k = torch.randn(B, T, H, dk, **f)
    v = torch.randn(B, T, H, dv, **f)
    beta_logit = torch.randn(B, T, H, **f)
    alpha_logit = torch.randn(B, T, H, **f) + float(alpha_logit_mean)
    lam_logit = torch.randn(B, T, H, **f)
    S0 = (torch.randn(B, H, dv, dk, **f) * float(s0_std)) if s0_std else None
    if key_corr:
        shared = torch.randn(B, 1, H, dk, **f) * float(key_corr)
        q = q + shared
        k = k + shared

    q = _unit(q).to(dt).contiguous()
    k = _unit(k).to(dt).contiguous()
    v = v.to(dt).contiguous()
    beta = torch.sigmoid(beta_logit).contiguous()
    if alpha == "random":
        alpha_t = torch.exp(-torch.nn.functional.softplus(alpha_logit)).contiguous()
    elif alpha == "one":
        alpha_t = None if gates_as_none else torch.ones(B, T, H, device=device)
    else:
        raise ValueError(alpha)
    if lam == "random":
        lam_t = torch.sigmoid(lam_logit).contiguous()
    elif lam == "zero":
        lam_t = None if gates_as_none else torch.zeros(B, T, H, device=device)
    elif lam == "one":
        lam_t = torch.ones(B, T, H, device=device)
    else:
        lam_t = torch.full((B, T, H), float(lam), device=device)
    return ChunkInputs(q, k, v, alpha_t, beta, lam_t, S0,
                       dict(B=B, T=T, H=H, dk=dk, dv=dv, dtype=dtype, seed=seed))


def workload_inputs(name: str, seed: int, device="cpu", gates_as_none=False) -> ChunkInputs:
    w = dict(WORKLOADS[name])
    return chunk_inputs(w["B"], w["T"], w["H"], w["dk"], w["dv"], w["dtype"], seed,
                        lam=w.get("lam", "random"), alpha=w.get("alpha", "random"),
                        s0_std=w.get("s0_std"), device=device, gates_as_none=gates_as_none)


@dataclass
class QedInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    g: torch.Tensor
    b: torch.Tensor
    w: torch.Tensor
    lam_h: torch.Tensor
    S0: Optional[torch.Tensor]


def qed_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, s0_std=None, decay_mean=-3.0, decay_std=1.5,
               lam_zero=False, device="cpu") -> QedInputs:
    """Inputs for the QED / GDN-2 layer (q, k [B,T,H,dk] unit-norm; v [B,T,H,dv]), drawn in
    this order: q, k, v ~ N(0, 1); g = -softplus(N(decay_mean, decay_std)) per key channel
    (log decay, exp(g) in (0, 1)); b = sigmoid(N(0, 1)) per key channel; w = sigmoid(N(0, 1))
    per value channel; lam_h = 0.25 sigmoid(N(-2, 1)) per head (the QED notes' strength
    parametrisation with its initial logit -2 as the mean); S0 ~ N(0, s0_std) if asked.
    lam_zero gives lam_h = 0 (GDN-2) without shifting the other draws."""
    dt = _DT[dtype]
    gen = _generator(seed, device)
    f = dict(generator=gen, device=device, dtype=torch.float32)
    q = torch.randn(B, T, H, dk, **f)
    k = torch.randn(B, T, H, dk, **f)
    v = torch.randn(B, T, H, dv, **f)
    g = -torch.nn.functional.softplus(torch.randn(B, T, H, dk, **f) * decay_std + decay_mean)
    b = torch.sigmoid(torch.randn(B, T, H, dk, **f))
    w = torch.sigmoid(torch.randn(B, T, H, dv, **f))
    lam = 0.25 * torch.sigmoid(torch.randn(H, **f) - 2.0)
    S0 = (torch.randn(B, H, dv, dk, **f) * float(s0_std)) if s0_std else None
    if lam_zero:
        lam = torch.zeros_like(lam)
    return QedInputs(_unit(q).to(dt).contiguous(), _unit(k).to(dt).contiguous(), v.to(dt).contiguous(),
                     g.contiguous(), b.contiguous(), w.contiguous(), lam.contiguous(), S0)


def eda_inputs(B, T, H, dk, dv, dtype="bf16", seed=0, s0_std=None, device="cpu"):
    """Inputs for Erase-then-Delta, drawn in this order: q, k, e ~ N(0, 1) each L2-normalised
    per (token, head); v ~ N(0, 1); S0 ~ N(0, s0_std) if asked.  Returns (q, k, v, e, S0)."""
    dt = _DT[dtype]
    gen = _generator(seed, device)
    f = dict(generator=gen, device=device, dtype=torch.float32)
    q = torch.randn(B, T, H, dk, **f)
    k = torch.randn(B, T, H, dk, **f)
    e = torch.randn(B, T, H, dk, **f)
    v = torch.randn(B, T, H, dv, **f)
    S0 = (torch.randn(B, H, dv, dk, **f) * float(s0_std)) if s0_std else None
    return (_unit(q).to(dt).contiguous(), _unit(k).to(dt).contiguous(), v.to(dt).contiguous(),
            _unit(e).to(dt).contiguous(), S0)


def upstream_grads(B, T, H, dk, dv, dtype="bf16", seed=0, dst_std=None, device="cpu"):
    """Gradients arriving from above for the layer backward: dO ~ N(0, 1) in the
    input dtype [B,T,H,dv] and, when dst_std is given, dS_T ~ N(0, dst_std) fp32
    [B,H,dv,dk].  Drawn from their own generator (seed), so the forward inputs of the
    same seed do not shift."""
    g = _generator(seed, device)
    f = dict(generator=g, device=device, dtype=torch.float32)
    dO = torch.randn(B, T, H, dv, **f).to(_DT[dtype]).contiguous()
    dST = (torch.randn(B, H, dv, dk, **f) * float(dst_std)).contiguous() if dst_std else None
    return dO, dST


def decode_state(N, H, dk, dv, s0_std=0.02, seed=0, device="cpu") -> torch.Tensor:
    """Resident fp32 decode state S ~ N(0, s0_std), layout [N,H,dv,dk]."""
    g = _generator(seed, device)
    return (torch.randn(N, H, dv, dk, generator=g, device=device) * float(s0_std)).contiguous()


def decode_tokens(steps, N, H, dk, dv, dtype="bf16", seed=0, device="cpu", alpha_logit_mean=-4.0):
    """Per-step decode inputs for `steps` consecutive tokens: q,k [steps,N,H,dk],
    v [steps,N,H,dv], alpha, beta, lam [steps,N,H].  Same distributions as
    ``chunk_inputs`` (alpha_logit_mean likewise)."""
    dt = _DT[dtype]
    g = _generator(seed, device)
    f = dict(generator=g, device=device, dtype=torch.float32)
    q = _unit(torch.randn(steps, N, H, dk, **f)).to(dt).contiguous()
    k = _unit(torch.randn(steps, N, H, dk, **f)).to(dt).contiguous()
    v = torch.randn(steps, N, H, dv, **f).to(dt).contiguous()
    beta = torch.sigmoid(torch.randn(steps, N, H, **f)).contiguous()
    alpha = torch.exp(-torch.nn.functional.softplus(torch.randn(steps, N, H, **f) + float(alpha_logit_mean))).contiguous()
    lam = torch.sigmoid(torch.randn(steps, N, H, **f)).contiguous()
    return q, k, v, alpha, beta, lam
