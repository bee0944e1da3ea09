"""Seeded synthetic inputs for the six decode workloads.

Input generation only: random draws with the stated laws, the Mamba2
discretization (decay = exp(dt * A), beta = dt) that forms the step's
inputs, and the decay-rate statistic a precision map is built from.  Nothing
here performs the quantized step; both the HIP path and the oracle consume
these tensors.

Every step t of a workload draws from its own torch CPU generator seeded
with seed_base * 1_000_003 + t, so any step can be produced on its own and
the same tensors reach the GPU (copied) and the oracle.

Workloads (S[v][k] orientation; v = value / output channel, k = key):
  gla_small   GLA per-key decay, B=1 H=2 dk=dv=64 T=32; q,k ~ N(0,1)/8 fp32,
              v ~ N(0,1) fp32, a = sigmoid(N(3,1)) per (b,h,t,k); int8, SR.
  gdn         Gated DeltaNet, B=64 H=32 dk=dv=128 T=1024; q,k,v ~ N(0,1) with
              k L2-normalised in fp32, then bf16; alpha = sigmoid(N(4,1)),
              beta = sigmoid(N(0,1)) per (b,h,t); int8, SR.
  mamba2      Mamba2 scalar decay, B=256 H=32 head_dim=64 (dv) d_state=128
              (dk) T=2048; x ~ N(0,1) bf16 (v), B_t ~ N(0,1) bf16 (k),
              C_t ~ N(0,1) bf16 (q), dt = softplus(N(-2,0.5)) per (b,h,t),
              A_h = -exp(U(0,2)) per head; decay = exp(dt A_h), beta = dt;
              the 25% of heads with smallest |A_h| in bf16, others int8, SR.
  gla_int4    GLA per-key decay, B=128 H=32 dk=dv=128 T=4096; q,k,v ~ N(0,1)
              bf16, a = sigmoid(N(5,1)); int4 + low-rank bypass (rank 8,
              merge every 64 steps, 0.5 LSB) + BDR over nearest rounding.
  gdn_large   Gated DeltaNet B=1024 H=32 dk=dv=128 T=256, inputs as gdn;
              per head the 10% slowest key channels (13 of 128) in fp16,
              others int8, SR.
  gdn_int4    Gated DeltaNet B=64 H=32 dk=dv=128 T=1024, inputs as gdn;
              int4 + low-rank bypass (rank 8, merge every 64 steps, 0.5 LSB)
              + BDR over nearest rounding, as gla_int4.
  gla_int4_sr GLA per-key decay, B=128 H=32 dk=dv=128 T=256, inputs as
              gla_int4; int4 with stochastic rounding and no buffer: low
              precision for short decode horizons.
  gla_int4_bf16  gla_int4 with bf16 row scales and bf16 buffer factors (the
              layout behind the pages' "up to 5.3x" state-memory figure).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    recurrence: str          # gla | gdn | mamba2
    B: int
    H: int
    dk: int
    dv: int
    T: int
    in_dtype: str            # fp32 | bf16
    qbits: int = 8
    rounding: str = "stochastic"
    sr_bits: int = 16
    bdr: bool = False
    lrb_rank: int = 0
    lrb_period: int = 64
    lrb_theta: float = 0.5
    map_mode: str = "none"   # none | head | key
    map_frac: float = 0.0
    hp_dtype: str = "bf16"
    seed_base: int = 1000
    philox_seed: int = 0
    qk_scale: float = 1.0    # GLA: q, k ~ N(0,1) * qk_scale
    decay_mu: float = 3.0    # GLA: a = sigmoid(N(decay_mu, 1))
    aux_dtype: str = "fp32"  # row scales and low-rank buffer factors: fp32 | bf16

    @property
    def kind(self) -> str:
        return "delta" if self.recurrence == "gdn" else "additive"

    @property
    def decay_mode(self) -> str:
        return "key" if self.recurrence == "gla" else "head"

    @property
    def has_beta(self) -> bool:
        return self.recurrence != "gla"

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    # -- precision-map statistic (decay rate: smaller = slower decay) -------
    def mamba2_A(self) -> np.ndarray:
        import torch
        g = torch.Generator().manual_seed(self.seed_base * 7 + 1)
        return (-torch.exp(torch.rand(self.H, generator=g, dtype=torch.float32) * 2.0)).numpy()

    def map_stat(self):
        """(stat, groups, per_group) for the precision map, or None."""
        if self.map_mode == "none":
            return None
        if self.recurrence == "mamba2" and self.map_mode == "head":
            return np.abs(self.mamba2_A()).astype(np.float32), 1, self.H
        if self.recurrence == "gdn" and self.map_mode == "key":
            # The delta rule decays a head with one scalar alpha whose law is the
            # same for every head and channel: every key channel has the same
            # expected rate -log(sigmoid(4)), so all tie.
            rate = -math.log(1.0 / (1.0 + math.exp(-4.0)))
            return np.full(self.H * self.dk, rate, np.float32), self.H, self.dk
        raise ValueError(f"no map statistic for {self.name}")

    # -- per-step inputs ---------------------------------------------------
    def step_inputs(self, t: int, B: Optional[int] = None) -> dict:
        """Inputs of step t as torch CPU tensors: q, k, v, decay, beta (or None)."""
        import torch
        B = self.B if B is None else B
        H, dk, dv = self.H, self.dk, self.dv
        g = torch.Generator().manual_seed(self.seed_base * 1_000_003 + t)
        f32 = torch.float32
        indt = torch.bfloat16 if self.in_dtype == "bf16" else f32
        if self.recurrence == "gla":
            q = torch.randn(B, H, dk, generator=g, dtype=f32) * self.qk_scale
            k = torch.randn(B, H, dk, generator=g, dtype=f32) * self.qk_scale
            v = torch.randn(B, H, dv, generator=g, dtype=f32)
            decay = torch.sigmoid(torch.randn(B, H, dk, generator=g, dtype=f32) + self.decay_mu)
            beta = None
        elif self.recurrence == "gdn":
            q = torch.randn(B, H, dk, generator=g, dtype=f32)
            k = torch.randn(B, H, dk, generator=g, dtype=f32)
            k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)
            v = torch.randn(B, H, dv, generator=g, dtype=f32)
            decay = torch.sigmoid(torch.randn(B, H, generator=g, dtype=f32) + 4.0)
            beta = torch.sigmoid(torch.randn(B, H, generator=g, dtype=f32))
        elif self.recurrence == "mamba2":
            v = torch.randn(B, H, dv, generator=g, dtype=f32)          # x
            k = torch.randn(B, H, dk, generator=g, dtype=f32)          # B_t
            q = torch.randn(B, H, dk, generator=g, dtype=f32)          # C_t
            dt = torch.nn.functional.softplus(torch.randn(B, H, generator=g, dtype=f32) * 0.5 - 2.0)
            A = torch.from_numpy(self.mamba2_A())
            decay = torch.exp(dt * A[None, :])
            beta = dt
        else:
            raise ValueError(self.recurrence)
        return {"q": q.to(indt).contiguous(), "k": k.to(indt).contiguous(), "v": v.to(indt).contiguous(),
                "decay": decay.contiguous(), "beta": None if beta is None else beta.contiguous()}


WORKLOADS = {
    "gla_small": Workload("gla_small", "gla", B=1, H=2, dk=64, dv=64, T=32, in_dtype="fp32",
                          qk_scale=0.125, decay_mu=3.0, seed_base=1001),
    "gdn": Workload("gdn", "gdn", B=64, H=32, dk=128, dv=128, T=1024, in_dtype="bf16", seed_base=1002),
    "mamba2": Workload("mamba2", "mamba2", B=256, H=32, dk=128, dv=64, T=2048, in_dtype="bf16",
                       map_mode="head", map_frac=0.25, hp_dtype="bf16", seed_base=1003),
    "gla_int4": Workload("gla_int4", "gla", B=128, H=32, dk=128, dv=128, T=4096, in_dtype="bf16",
                         qbits=4, rounding="nearest", bdr=True, lrb_rank=8, lrb_period=64,
                         lrb_theta=0.5, decay_mu=5.0, seed_base=1004),
    "gdn_large": Workload("gdn_large", "gdn", B=1024, H=32, dk=128, dv=128, T=256, in_dtype="bf16",
                          map_mode="key", map_frac=0.10, hp_dtype="fp16", seed_base=1005),
    "gdn_int4": Workload("gdn_int4", "gdn", B=64, H=32, dk=128, dv=128, T=1024, in_dtype="bf16",
                         qbits=4, rounding="nearest", bdr=True, lrb_rank=8, lrb_period=64,
                         lrb_theta=0.5, seed_base=1006),
    "gla_int4_sr": Workload("gla_int4_sr", "gla", B=128, H=32, dk=128, dv=128, T=256, in_dtype="bf16",
                            qbits=4, rounding="stochastic", sr_bits=16, decay_mu=5.0, seed_base=1007),
    "gla_int4_bf16": Workload("gla_int4_bf16", "gla", B=128, H=32, dk=128, dv=128, T=4096, in_dtype="bf16",
                              qbits=4, rounding="nearest", bdr=True, lrb_rank=8, lrb_period=64,
                              lrb_theta=0.5, decay_mu=5.0, seed_base=1004, aux_dtype="bf16"),
}
