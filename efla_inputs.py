"""Seeded synthetic EFLA workloads.

This module holds the input recipes only: shapes, dtypes and the random
distributions of q, k, v, beta and the initial state. It contains none of the
method's arithmetic, so both the GPU path's tests and the fp64 oracle can be
fed from it.

Every draw uses a CPU ``torch.Generator`` seeded with 42 + config index (42 is
the seed the jsqmd.com article gives for the training runs, section 2.1), is
made in fp32, normalised and scaled in fp32, then cast to the config dtype.
The oracle consumes the cast tensors upcast to fp64, i.e. exactly the values
the GPU receives.

Recipes:
  * "unit direction x norm": g / ||g||_2 with g ~ N(0, I_d), times a per-token
    scalar norm.
  * "log-uniform [a, b]": exp(U(ln a, ln b)) per token.
  * beta = sigmoid(N(mu, 1)) per token.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    index: int           # seed = 42 + index
    B: int
    H: int
    T: int
    d: int
    chunk: int
    dtype: str           # "f32" or "bf16"
    q_rule: str          # "normal" | "unit"
    k_rule: str          # "normal" | "unit" | "unit_x_1p_absnormal" | "unit_x_logu"
    k_norm_lo: float = 0.0
    k_norm_hi: float = 0.0
    beta_mu: float = 0.0
    s0_std: float = 0.0  # 0 -> no initial state (NULL, zeros)
    decode_steps: int = 0

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T

    @property
    def seed(self) -> int:
        return 42 + self.index


# The five synthetic configurations (single head; two fp32 shapes; the 340M and
# 1.3B layer shapes with head_dim 128; a long stiff stream with high-energy keys).
WORKLOADS: Dict[str, Workload] = {
    "single_head_d16": Workload("single_head_d16", 0, 1, 1, 256, 16, 16, "f32",
                                "normal", "normal"),
    "fp32_d64": Workload("fp32_d64", 1, 8, 4, 2048, 64, 64, "f32",
                         "normal", "unit_x_logu", 0.1, 10.0),
    "layer340m_d128": Workload("layer340m_d128", 2, 16, 8, 2048, 128, 64, "bf16",
                               "unit", "unit_x_1p_absnormal", decode_steps=256),
    "layer1p3b_d128": Workload("layer1p3b_d128", 3, 8, 16, 4096, 128, 64, "bf16",
                               "normal", "unit", s0_std=0.1),
    "stiff_long_d128": Workload("stiff_long_d128", 4, 1, 16, 65536, 128, 64, "bf16",
                                "normal", "unit_x_logu", 1.0, 30.0, beta_mu=1.0),
}


def scaled(w: Workload, **kw) -> Workload:
    """Same recipe, different sizes (for small parity cases)."""
    return replace(w, **kw)


def _unit(g: torch.Tensor) -> torch.Tensor:
    return g / g.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _draw_qkvb(w: Workload, gen: torch.Generator, T: int):
    B, H, d = w.B, w.H, w.d
    shape = (B, H, T, d)
    q = torch.randn(shape, generator=gen, dtype=torch.float32)
    k = torch.randn(shape, generator=gen, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, dtype=torch.float32)
    if w.q_rule == "unit":
        q = _unit(q)
    if w.k_rule == "unit":
        k = _unit(k)
    elif w.k_rule == "unit_x_1p_absnormal":
        n = 1.0 + torch.randn((B, H, T, 1), generator=gen, dtype=torch.float32).abs()
        k = _unit(k) * n
    elif w.k_rule == "unit_x_logu":
        lo, hi = math.log(w.k_norm_lo), math.log(w.k_norm_hi)
        u = torch.rand((B, H, T, 1), generator=gen, dtype=torch.float32)
        k = _unit(k) * torch.exp(lo + (hi - lo) * u)
    elif w.k_rule != "normal":
        raise ValueError(w.k_rule)
    beta = torch.sigmoid(w.beta_mu + torch.randn((B, H, T), generator=gen,
                                                 dtype=torch.float32))
    dt = w.torch_dtype
    return (q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous(),
            beta.to(dt).contiguous())


def make_inputs(w: Workload) -> dict:
    """CPU tensors: q, k, v [B,H,T,d] and beta [B,H,T] in the config dtype;
    s0 [B,H,d,d] fp32 or None; and, if the config has a decode phase,
    dec_q/dec_k/dec_v [B,H,steps,d], dec_beta [B,H,steps] drawn by the same
    generator continued after the forward inputs."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    q, k, v, beta = _draw_qkvb(w, gen, w.T)
    out = {"q": q, "k": k, "v": v, "beta": beta, "s0": None}
    if w.s0_std > 0:
        out["s0"] = (w.s0_std * torch.randn((w.B, w.H, w.d, w.d), generator=gen,
                                            dtype=torch.float32)).contiguous()
    if w.decode_steps > 0:
        dq, dk, dv, db = _draw_qkvb(w, gen, w.decode_steps)
        out.update(dec_q=dq, dec_k=dk, dec_v=dv, dec_beta=db)
    return out


def random_case(seed: int, B: int, H: int, T: int, d: int, dtype: str = "f32",
                k_rule: str = "unit_x_logu", k_lo: float = 0.3, k_hi: float = 3.0,
                beta_mu: float = 0.0, s0_std: float = 0.0) -> dict:
    """A small seeded case for parity sweeps (random shapes, ragged T)."""
    w = Workload("random", seed - 42, B, H, T, d, 16, dtype, "normal", k_rule, k_lo, k_hi,
                 beta_mu, s0_std)
    return make_inputs(w)


def log_decay(seed: int, shape, mu: float = 2.0, scale: float = 1.0) -> torch.Tensor:
    """Per-token log-decays for the gated variant, fp32: log(sigmoid(x)) with
    x ~ N(mu, scale^2), so every decay g = exp(log_g) lies in (0, 1) (mu = 2
    gives g around 0.88)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    x = mu + scale * torch.randn(tuple(shape), generator=gen, dtype=torch.float32)
    return torch.nn.functional.logsigmoid(x).contiguous()
