"""Seeded synthetic inputs for the gated delta rule.

This module only draws inputs; it holds none of the recurrence's arithmetic.
Both the GPU path (tests, bench) and the CPU oracle are fed from it.

Recipe (every draw from a torch.Generator seeded per workload):
  q, k ~ N(0,1), L2-normalised over d_k per (token, head) in fp32, then rounded
         to the storage dtype (round-to-nearest-even for bf16);
  v    ~ N(0,1) in the storage dtype;
  beta  = sigmoid(N(0,1)), fp32 [T, H];
  alpha = sigmoid(bias + N(0, std)), fp32, [T, H] (scalar gate) or [T, H, d_k]
          (per-key-channel gate); bias +5 mirrors the KDA alpha-gate bias, +4 a
          faster-forgetting scalar head;
  initial state ~ N(0, s0_std) fp32 [N, H, d_v, d_k], or None when s0_std == 0;
  varlen lengths uniform integers in [lo, hi] from numpy's PCG64 with their own
  seed, so they are identical on every device.
N(0, x) means standard deviation x.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    H: int
    dk: int
    dv: int
    seq_lens: Tuple[int, ...]          # one entry per packed sequence
    dtype: str = "bf16"                # storage dtype of q, k, v: "bf16" | "fp32"
    gate: str = "scalar"               # "scalar" | "per_key"
    alpha_bias: float = 5.0
    alpha_std: float = 1.0
    s0_std: float = 0.0                # 0 -> no initial state (zeros)
    interval: int = 0                  # snapshot interval in tokens (0 = none)
    chunk: int = 64
    seed: int = 0
    description: str = field(default="", compare=False)

    @property
    def T(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def num_seqs(self) -> int:
        return len(self.seq_lens)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> Tuple[int, ...]:
    rng = np.random.Generator(np.random.PCG64(seed))
    return tuple(int(x) for x in rng.integers(lo, hi, endpoint=True, size=n))


# The five workloads the path is measured and checked on.
TINY = Workload("tiny_recurrence_d64_T256_fp32", H=1, dk=64, dv=64, seq_lens=(256,), dtype="fp32",
                gate="scalar", alpha_bias=5.0, alpha_std=0.5, seed=1000,
                description="B=1 H=1 d=64 T=256 fp32, scalar alpha=sigmoid(5+N(0,0.5)), zero state")
KDA_LAYER = Workload("kda_layer_H14_d64_T8192", H=14, dk=64, dv=64, seq_lens=(8192,), dtype="bf16",
                     gate="per_key", alpha_bias=5.0, alpha_std=1.0, seed=1001,
                     description="Qwen2.5-0.5B-graft KDA layer shape: B=1 H=14 d=64 T=8192, per-key alpha")
DECODE = Workload("decode_B256_H16_d128", H=16, dk=128, dv=128, seq_lens=(1,) * 256, dtype="bf16",
                  gate="per_key", alpha_bias=5.0, alpha_std=1.0, s0_std=0.02, seed=1002,
                  description="batched decode: 256 sequences x one token, H=16 d=128, per-key alpha")
LONG_PREFILL = Workload("long_prefill_T262144_H16_d128", H=16, dk=128, dv=128, seq_lens=(262144,),
                        dtype="bf16", gate="scalar", alpha_bias=4.0, alpha_std=1.0, seed=1003,
                        description="B=1 H=16 d=128 T=262144, scalar alpha=sigmoid(4+N(0,1))")
VARLEN = Workload("varlen_32seq_H32_d128", H=32, dk=128, dv=128,
                  seq_lens=varlen_lengths(32, 1024, 32768, 2005), dtype="bf16", gate="per_key",
                  alpha_bias=5.0, alpha_std=1.0, s0_std=0.02, interval=4096, seed=1004,
                  description="32 packed sequences, lengths U[1024,32768], H=32 d=128, per-key alpha, "
                              "initial states N(0,0.02), snapshots every 4096 tokens")

ALL = {w.name: w for w in (TINY, KDA_LAYER, DECODE, LONG_PREFILL, VARLEN)}


def _torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[name]


def _normal(shape, gen, device, std=1.0, mean=0.0):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x


def make_prefill_inputs(wl: Workload, device="cpu", seed: Optional[int] = None) -> dict:
    """Returns q, k, v (storage dtype), alpha, beta (fp32), cu_seqlens (int64, on
    `device`), cu_seqlens_host (int64 CPU) and initial_state (fp32 or None)."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed if seed is None else seed)
    T, H, dk, dv = wl.T, wl.H, wl.dk, wl.dv
    st = _torch_dtype(wl.dtype)

    def unit_rows(shape):
        x = _normal(shape, gen, device)
        x.div_(torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30))
        return x.to(st)

    q = unit_rows((T, H, dk))
    k = unit_rows((T, H, dk))
    v = _normal((T, H, dv), gen, device).to(st)
    beta = torch.sigmoid(_normal((T, H), gen, device))
    a_shape = (T, H, dk) if wl.gate == "per_key" else (T, H)
    alpha = torch.sigmoid(_normal(a_shape, gen, device, std=wl.alpha_std, mean=wl.alpha_bias))
    init = None
    if wl.s0_std > 0:
        init = _normal((wl.num_seqs, H, dv, dk), gen, device, std=wl.s0_std)
    cu_host = torch.zeros(wl.num_seqs + 1, dtype=torch.int64)
    cu_host[1:] = torch.cumsum(torch.tensor(wl.seq_lens, dtype=torch.int64), 0)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, cu_seqlens=cu_host.to(device),
                cu_seqlens_host=cu_host, initial_state=init)


def make_decode_inputs(wl: Workload, device="cpu", seed: Optional[int] = None) -> dict:
    """One token per sequence: q, k [B,H,dk], v [B,H,dv], alpha [B,H(,dk)], beta
    [B,H], state [B,H,dv,dk] fp32 (~N(0, s0_std))."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed if seed is None else seed)
    B, H, dk, dv = wl.num_seqs, wl.H, wl.dk, wl.dv
    st = _torch_dtype(wl.dtype)

    def unit_rows(shape):
        x = _normal(shape, gen, device)
        x.div_(torch.linalg.vector_norm(x, dim=-1, keepdim=True).clamp_min(1e-30))
        return x.to(st)

    state = _normal((B, H, dv, dk), gen, device, std=wl.s0_std if wl.s0_std > 0 else 0.02)
    q = unit_rows((B, H, dk))
    k = unit_rows((B, H, dk))
    v = _normal((B, H, dv), gen, device).to(st)
    beta = torch.sigmoid(_normal((B, H), gen, device))
    a_shape = (B, H, dk) if wl.gate == "per_key" else (B, H)
    alpha = torch.sigmoid(_normal(a_shape, gen, device, std=wl.alpha_std, mean=wl.alpha_bias))
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, state=state)


def to_oracle_arrays(t: torch.Tensor) -> np.ndarray:
    """Host numpy view for the oracle: bf16 -> uint16 bit patterns, fp32 as is."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make_layer_inputs(wl: Workload, device="cpu", seed: Optional[int] = None, conv_state: bool = True) -> dict:
    """Inputs of the layer front and back end around the recurrence: conv inputs
    xq, xk, xv ~ N(0,1) [T,H,d] (storage dtype); conv taps [3,H,d,4] fp32 =
    identity tap (oldest first: 0,0,0,1) + N(0, 0.3); carried conv state
    ~ N(0,1) [N,3,3,H,d] or None; alpha logits ~ N(0,1) [T,H] or [T,H,d_k] and
    beta logits ~ N(0,1) [T,H]; for the back end o ~ N(0,1), gate logits ~ N(0,1)
    [T,H,d_v] and norm weights ~ U(0.5, 1.5) [d_v], all fp32."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed + 7 if seed is None else seed)
    T, H, d = wl.T, wl.H, wl.dk
    st = _torch_dtype(wl.dtype)
    xq, xk, xv = (_normal((T, H, d), gen, device).to(st) for _ in range(3))
    conv_w = _normal((3, H, d, 4), gen, device, std=0.3)
    conv_w[..., 3] += 1.0
    state = _normal((wl.num_seqs, 3, 3, H, d), gen, device).to(st) if conv_state else None
    a_shape = (T, H, d) if wl.gate == "per_key" else (T, H)
    alpha_logit = _normal(a_shape, gen, device)
    beta_logit = _normal((T, H), gen, device)
    o = _normal((T, H, wl.dv), gen, device)
    g_logit = _normal((T, H, wl.dv), gen, device)
    norm_w = torch.rand((wl.dv,), generator=gen, device=device, dtype=torch.float32) + 0.5
    cu_host = torch.zeros(wl.num_seqs + 1, dtype=torch.int64)
    cu_host[1:] = torch.cumsum(torch.tensor(wl.seq_lens, dtype=torch.int64), 0)
    return dict(xq=xq, xk=xk, xv=xv, conv_w=conv_w, conv_state=state, alpha_logit=alpha_logit,
                beta_logit=beta_logit, o=o, g_logit=g_logit, norm_w=norm_w, cu_seqlens=cu_host.to(device),
                cu_seqlens_host=cu_host)
