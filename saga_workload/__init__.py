"""Seeded synthetic workloads shaped like the pages' decode benchmarks.

This module only *draws inputs*: it holds none of the attention arithmetic,
and both sides of every parity check (the HIP path and the CPU oracle) take
their inputs from it.  Shapes follow the decode-latency setup of
"More Value per Key: Asymmetric Sparse Attention for Faster LLM Decoding"
(ai.info summary, Main Findings, end-to-end speedups): Llama-3.2-1B-like
heads (h_q=32, key heads 8 -> 4, 8 value heads, d=64) and
Qwen2.5-1.5B-like heads (h_q=12, key heads 2 -> 1, 2 value heads, d=128),
context 8K..128K, N in {512, 1024, 2048}, batch 1 and 16, 32 generated
tokens.  No trained weights or datasets are used; the values are synthetic.

Recipe (per config index ``cfg`` and layer ``layer``):
  * K, V ~ N(0, 1) drawn in fp32 and rounded to bf16 (round to nearest even).
  * q_0 ~ N(0, 1)/sqrt(d) in fp32; q_t = 0.9 q_{t-1} + 0.44 e_t with
    e_t ~ N(0, 1)/sqrt(d); each q_t is rounded to bf16 on its own.
  * Heavy hitters: round(0.01 * rows) positions per (batch row, key head),
    drawn without replacement and dealt round-robin to the query heads of
    that key head's group; each such key row gets 3 * q_0/|q_0| of its query
    head added in fp32 to its bf16 values and is rounded to bf16 again, so
    those logits sit about 3 sigma high.
  * Seeds: 1000*cfg + layer for K/V/positions, that plus 500 for q.
  * The cache holds rows = L + T; decode step t attends ctx_t = L + t rows.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int           # config index used in the seeds
    batch: int
    h_q: int
    h_k: int
    h_v: int
    head_dim: int
    L: int               # prompt context
    top_n: int           # N
    refresh_n: int       # n
    steps: int           # T decode steps
    layers: int
    scale: float = 1.0   # 1/sqrt(d) is folded into q
    head_dim_v: int = 0  # value head dimension; 0: same as head_dim

    @property
    def rows(self) -> int:
        return self.L + self.steps

    def ctx(self, t: int) -> int:
        return self.L + t

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def gqa(self, h_kv: int) -> "Workload":
        """The full-attention GQA twin of this shape (h_k = h_v = h_kv)."""
        return dataclasses.replace(self, name=self.name + f"_gqa{h_kv}", h_k=h_kv, h_v=h_kv)

    def kv_bytes(self) -> int:
        dv = self.head_dim_v or self.head_dim
        return self.layers * self.batch * (self.h_k * self.head_dim + self.h_v * dv) * self.rows * 2


# The five workload families.  index is the seed base.
TINY = Workload("tiny", 0, 1, 4, 1, 2, 64, 1024, 64, 4, 8, 1)
LLAMA_8K = Workload("llama_like_8k", 1, 1, 32, 4, 8, 64, 8192, 512, 16, 32, 1)
QWEN_128K_B1 = Workload("qwen_like_128k_b1", 2, 1, 12, 1, 2, 128, 131072, 1024, 16, 32, 28)
QWEN_128K_B16 = QWEN_128K_B1.with_(name="qwen_like_128k_b16", batch=16)
LLAMA_128K_B16 = Workload("llama_like_128k_b16", 3, 16, 32, 4, 8, 64, 131072, 2048, 16, 32, 16)

GQA_HKV = {"llama": 8, "qwen": 2}

WORKLOADS: Dict[str, Workload] = {w.name: w for w in
                                  (TINY, LLAMA_8K, QWEN_128K_B1, QWEN_128K_B16, LLAMA_128K_B16)}


def sweep() -> List[Workload]:
    """Llama-like and Qwen-like shapes over L x N x B (config index 4)."""
    out = []
    for fam, base in (("llama", LLAMA_128K_B16), ("qwen", QWEN_128K_B1)):
        for L in (8192, 16384, 32768, 65536, 131072):
            for N in (512, 1024, 2048):
                for B in (1, 16):
                    out.append(base.with_(name=f"sweep_{fam}_L{L}_N{N}_B{B}", index=4,
                                          L=L, top_n=N, batch=B))
    return out


def _randn(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_layer(w: Workload, layer: int = 0, device="cpu", heavy_hitters: bool = True,
               steps: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw one layer's K/V caches and the query of every decode step.

    Returns ``K [B][h_k][rows][d]``, ``V [B][h_v][rows][d_v]`` and
    ``q [T][B][h_q][d]``, all bf16 on ``device`` (d_v = head_dim_v, or d).
    """
    device = torch.device(device)
    T = w.steps if steps is None else steps
    B, hq, hk, hv, d, rows = w.batch, w.h_q, w.h_k, w.h_v, w.head_dim, w.rows
    seed = 1000 * w.index + layer
    gq = torch.Generator(device=device)
    gq.manual_seed(seed + 500)
    inv = 1.0 / math.sqrt(d)
    q_prev = _randn((B, hq, d), gq, device) * inv
    q0 = q_prev
    qs = [q_prev.to(torch.bfloat16)]
    for _ in range(1, T):
        q_prev = 0.9 * q_prev + 0.44 * (_randn((B, hq, d), gq, device) * inv)
        qs.append(q_prev.to(torch.bfloat16))
    q = torch.stack(qs, 0).contiguous()

    gkv = torch.Generator(device=device)
    gkv.manual_seed(seed)
    # torch draws bf16 normals in fp32 and rounds them to nearest even.
    K = torch.randn((B, hk, rows, d), generator=gkv, device=device, dtype=torch.bfloat16)
    V = torch.randn((B, hv, rows, w.head_dim_v or d), generator=gkv, device=device,
                    dtype=torch.bfloat16)
    if heavy_hitters:
        count = int(round(0.01 * rows))
        Gk = hq // hk
        unit = q0 / q0.norm(dim=-1, keepdim=True)            # [B][hq][d]
        for b in range(B):
            for g in range(hk):
                pos = torch.randperm(rows, generator=gkv, device=device)[:count]
                heads = g * Gk + (torch.arange(count, device=device) % Gk)
                K[b, g, pos, :] = (K[b, g, pos, :].float() + 3.0 * unit[b, heads, :]).to(
                    torch.bfloat16)
    return {"K": K, "V": V, "q": q}


def quantize_k_e4m3(K: torch.Tensor, pow2_scales: bool = False):
    """An fp8 E4M3 (OCP) copy of a bf16 K (or V) cache ``[B][h][rows][d]``, the
    way a serving stack would store it: one fp32 scale per (batch row, head),
    scale = amax / 448 (rounded up to a power of two when ``pow2_scales``),
    codes = round-to-nearest-even(K / scale) by torch's float8_e4m3fn cast.

    Returns ``(codes uint8 [B][h][rows][d], scale float32 [B][h])`` on
    K's device.  Input preparation only: both sides of a parity check take
    these same codes and scales.
    """
    amax = K.float().abs().amax(dim=(2, 3)).clamp_min(1e-30)
    scale = amax / 448.0
    if pow2_scales:
        scale = torch.exp2(torch.ceil(torch.log2(scale)))
    x = (K.float() / scale[:, :, None, None]).clamp(-448.0, 448.0)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, scale.to(torch.float32).contiguous()


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    import numpy as np
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
