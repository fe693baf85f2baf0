"""Seeded synthetic KDA inputs shared by the tests, the smoke check and the bench.

This module holds none of the method's arithmetic: it only draws random
numbers and prepares inputs the way the workloads describe them (L2-normalised
q and k, beta = sigmoid of a normal draw, gate *logits* z). The gate itself,
g = g_min * sigmoid(exp(A_h) z), is part of the method and is applied by each
side on its own (the HIP path in its kernels, the oracle in fp64).

Workloads (all seed 0, d_k = d_v, chunk 64, g_min = -5):
  tiny      B=1,  H=2,  T=256,    d=64,  fp32, zero initial state
  single    B=1,  H=16, T=4096,   d=128, bf16, initial state 0.02*randn
  train8k   B=8,  H=32, T=8192,   d=128, bf16, zero initial state (headline)
  long256k  B=1,  H=32, T=262144, d=128, bf16, zero initial state
  varlen1m  64 sequences, lengths floor(512 * 128**u), u ~ U(0,1), summing to
            within 5% of 2**20; H=32, d=128, bf16, initial states 0.02*randn

Recipe: torch.Generator(device).manual_seed(seed); draw order (varlen lengths
first, from a CPU generator), q, k, v, beta-logits, gate-logits, h0; all fp32
randn in layout [B, T, H, D]; q and k divided by their L2 norm over D in fp32;
beta = sigmoid(logit) in fp32; q, k, v cast to bf16 (round to nearest even) for
the bf16 workloads.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

CONFIG_NAMES = ["tiny", "single", "train8k", "long256k", "varlen1m"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int            # per sequence (dense) or total tokens (varlen, B = 1)
    H: int
    Dk: int
    Dv: int
    dtype: torch.dtype
    h0_std: float     # 0.0 means no initial state (zeros)
    varlen: bool = False
    chunk: int = 64
    g_min: float = -5.0

    @property
    def dtype_name(self) -> str:
        return "bf16" if self.dtype == torch.bfloat16 else "fp32"


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 2, 64, 64, torch.float32, 0.0),
    "single": Workload("single", 1, 4096, 16, 128, 128, torch.bfloat16, 0.02),
    "train8k": Workload("train8k", 8, 8192, 32, 128, 128, torch.bfloat16, 0.0),
    "long256k": Workload("long256k", 1, 262144, 32, 128, 128, torch.bfloat16, 0.0),
    "varlen1m": Workload("varlen1m", 1, 0, 32, 128, 128, torch.bfloat16, 0.02, varlen=True),
}


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[CONFIG_NAMES[name_or_index]]
    return WORKLOADS[name_or_index]


def varlen_lengths(n_seqs: int = 64, lo: int = 512, hi: int = 65536,
                   target: int = 1 << 20, tol: float = 0.05):
    """First seed s = 0, 1, ... whose n_seqs log-uniform lengths
    floor(lo * (hi/lo)**u) sum to within `tol` of `target`. Returns (s, lengths)."""
    ratio = hi / lo
    for s in range(10000):
        gen = torch.Generator("cpu").manual_seed(s)
        u = torch.rand(n_seqs, generator=gen, dtype=torch.float64)
        lens = torch.floor(lo * ratio ** u).to(torch.int64).clamp_(lo, hi)
        if abs(int(lens.sum()) - target) <= tol * target:
            return s, [int(x) for x in lens]
    raise RuntimeError("no seed found")


def _unit_norm(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True)


def make_inputs(B: int, T: int, H: int, Dk: int, Dv: int, dtype=torch.bfloat16,
                h0_std: float = 0.0, lengths: Optional[List[int]] = None, seed: int = 0,
                device="cpu"):
    """Draw one KDA problem. With `lengths`, the sequences are packed into
    B = 1 and T = sum(lengths) with cu_seqlens. Returns a dict with q, k, v
    (dtype), beta (fp32 [B,T,H]), z (gate logits, fp32 [B,T,H,Dk]),
    h0 (fp32 [N,H,Dk,Dv] or None), cu_seqlens (int32 [N+1] or None), N."""
    device = torch.device(device)
    gen = torch.Generator(device).manual_seed(seed)
    cu = None
    N = B
    if lengths is not None:
        B, T, N = 1, int(sum(lengths)), len(lengths)
        cu = torch.zeros(N + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        cu = cu.to(device)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    q = _unit_norm(randn(B, T, H, Dk)).to(dtype)
    k = _unit_norm(randn(B, T, H, Dk)).to(dtype)
    v = randn(B, T, H, Dv).to(dtype)
    beta = torch.sigmoid(randn(B, T, H))
    z = randn(B, T, H, Dk)
    h0 = (h0_std * randn(N, H, Dk, Dv)) if h0_std > 0 else None
    return dict(q=q, k=k, v=v, beta=beta, z=z, h0=h0, cu_seqlens=cu, N=N, B=B, T=T, H=H,
                Dk=Dk, Dv=Dv)


def make_workload(name_or_index, seed: int = 0, device="cpu"):
    w = workload(name_or_index)
    lengths = None
    if w.varlen:
        _, lengths = varlen_lengths()
    d = make_inputs(w.B, w.T, w.H, w.Dk, w.Dv, w.dtype, w.h0_std, lengths, seed, device)
    d["workload"] = w
    return d
