"""Seeded synthetic inputs for the RLA-2 workloads.

This module only draws random numbers and builds shapes; it holds none of the
method's arithmetic. Both the HIP path (through tests and the bench) and the
CPU oracle read the tensors it returns, so the stored tensor is the single
source of truth: bf16 inputs are the round-to-nearest-even conversion of
fp32 N(0,1) draws, and the oracle upcasts those bf16 values exactly.

Every tensor comes from its own ``torch.Generator`` seeded with
``seed * 1_000_003 + stream`` (stream numbers below), so a workload is fully
determined by its seed and shape. CPU generation is the default; the large
decode prefixes can be generated on a GPU with the same seeding rule.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

# stream numbers (fixed order)
(S_LENGTHS, S_MASK_Q, S_MASK_K, S_GAMMA_Q, S_GAMMA_K, S_Q, S_K, S_V, S_PREFIX_K, S_PREFIX_V, S_INIT_S, S_INIT_Z,
 S_DOUT) = range(13)


def _gen(seed: int, stream: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(stream))
    return g


def normal(shape, seed: int, stream: int, dtype=torch.bfloat16, device: str = "cpu") -> torch.Tensor:
    """N(0,1) drawn in fp32, then rounded (RNE) to ``dtype``."""
    x = torch.randn(*shape, generator=_gen(seed, stream, device), dtype=torch.float32, device=device)
    return x.to(dtype)


def gammas(H: int, d: int, seed: int, stream: int, kind: str) -> torch.Tensor:
    """RMSNorm weights ``[H, d]`` fp32: all ones, or U(0.5, 1.5)."""
    if kind == "ones":
        return torch.ones(H, d, dtype=torch.float32)
    if kind == "uniform":
        return 0.5 + torch.rand(H, d, generator=_gen(seed, stream), dtype=torch.float32)
    raise ValueError(kind)


def doc_lengths(total: int, lo: int, hi: int, seed: int) -> list:
    """Integers ~ U{lo..hi} drawn until they cover ``total``; the last one is
    cut so the lengths sum to exactly ``total`` (it may end up below ``lo``)."""
    g = _gen(seed, S_LENGTHS)
    out, acc = [], 0
    while acc < total:
        n = int(torch.randint(lo, hi + 1, (1,), generator=g).item())
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out


def initial_state(H: int, d: int, seed: int, scale: float = 1.0):
    """A synthetic fp32 state ``(S0 [H, d, d], z0 [H, d])``: S0 ~ scale * N(0,1) and
    z0 ~ scale * |N(0,1)| (a key-sum vector is non-negative)."""
    S0 = scale * torch.randn(H, d, d, generator=_gen(seed, S_INIT_S), dtype=torch.float32)
    z0 = scale * torch.randn(H, d, generator=_gen(seed, S_INIT_Z), dtype=torch.float32).abs()
    return S0, z0


def cotangent(shape, seed: int, device: str = "cpu") -> torch.Tensor:
    """A loss gradient dL/dout for the backward: N(0,1) bf16 of the output's shape."""
    return normal(shape, seed, S_DOUT, torch.bfloat16, device)


def cu_from_lengths(lengths) -> torch.Tensor:
    cu = [0]
    for n in lengths:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32)


def channel_mask(d: int, frac: float, seed: int, stream: int) -> torch.Tensor:
    """``round(frac * d)`` distinct channel indices, shared by all heads and tokens."""
    n = int(round(frac * d))
    return torch.randperm(d, generator=_gen(seed, stream))[:n].sort().values


@dataclasses.dataclass
class FwdInputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    gamma_q: torch.Tensor
    gamma_k: torch.Tensor
    cu_seqlens: Optional[torch.Tensor]
    eps: float = 1e-4
    rms_eps: float = 1e-6
    rope_base: float = 10000.0

    @property
    def shape(self):
        return tuple(self.q.shape)


def fwd_inputs(B: int, H: int, L: int, d: int, dtype=torch.bfloat16, seed: int = 0,
               gamma: str = "uniform", lengths=None, bias_frac: float = 0.0,
               bias: float = -1.0) -> FwdInputs:
    """q, k, v ``[B, H, L, d]`` ~ N(0,1) in ``dtype``; optional packed documents.

    ``lengths``: document lengths for packed input (B must be 1, sum == L).
    ``bias_frac``: fraction of q and k channels (one seeded set per tensor)
    shifted by ``bias`` before the rounding to ``dtype``.
    """
    q32 = normal((B, H, L, d), seed, S_Q, torch.float32)
    k32 = normal((B, H, L, d), seed, S_K, torch.float32)
    v = normal((B, H, L, d), seed, S_V, dtype)
    if bias_frac > 0:
        q32[..., channel_mask(d, bias_frac, seed, S_MASK_Q)] += bias
        k32[..., channel_mask(d, bias_frac, seed, S_MASK_K)] += bias
    cu = None
    if lengths is not None:
        if B != 1 or sum(lengths) != L:
            raise ValueError("packed input needs B == 1 and sum(lengths) == L")
        cu = cu_from_lengths(lengths)
    return FwdInputs(q=q32.to(dtype), k=k32.to(dtype), v=v,
                     gamma_q=gammas(H, d, seed, S_GAMMA_Q, gamma),
                     gamma_k=gammas(H, d, seed, S_GAMMA_K, gamma), cu_seqlens=cu)


# --- the five named workloads -------------------------------------------------

def c1_fp32_small(seed: int = 1) -> FwdInputs:
    """fp32 causal forward, B=1, H=2, L=256, d=32, one document, RMSNorm weights 1."""
    return fwd_inputs(1, 2, 256, 32, torch.float32, seed, gamma="ones")


def c2_bf16_dense(seed: int = 2) -> FwdInputs:
    """bf16 causal forward, B=4, H=8, L=2048, d=64, one document per row."""
    return fwd_inputs(4, 8, 2048, 64, torch.bfloat16, seed, gamma="uniform")


def c3_lengths(seed: int = 3, total: int = 16384) -> list:
    return doc_lengths(total, 64, 4096, seed)


def c3_packed(seed: int = 3) -> FwdInputs:
    """Packed varlen bf16 forward: 16384 tokens, H=16, d=128, lengths ~ U{64..4096}."""
    return fwd_inputs(1, 16, 16384, 128, torch.bfloat16, seed, gamma="uniform",
                      lengths=c3_lengths(seed))


def c4_long(seed: int = 4, L: int = 65536, H: int = 32) -> FwdInputs:
    """Long-context bf16 forward, B=1, H=32, L=65536, d=128; 10% of q and k
    channels shifted by -1.0 so the ReLU leaves sparse positive supports."""
    return fwd_inputs(1, H, L, 128, torch.bfloat16, seed, gamma="uniform", bias_frac=0.1)


@dataclasses.dataclass
class DecodeInputs:
    prefix_lengths: torch.Tensor     # int32 [N]
    cu_prefix: torch.Tensor          # int32 [N+1]
    prefix_k: torch.Tensor           # [1, H, T_prefix, d]
    prefix_v: torch.Tensor
    q: torch.Tensor                  # [N, H, d]
    k: torch.Tensor
    v: torch.Tensor
    gamma_q: torch.Tensor
    gamma_k: torch.Tensor
    eps: float = 1e-4
    rms_eps: float = 1e-6
    rope_base: float = 10000.0


def decode_inputs(N: int, H: int, d: int, max_prefix: int, seed: int, dtype=torch.bfloat16,
                  device: str = "cpu", min_prefix: int = 1) -> DecodeInputs:
    """Decode workload: per-sequence prefix lengths ~ U{min_prefix..max_prefix},
    packed prefixes ``[1, H, sum(len), d]`` ~ N(0,1), one new token per sequence."""
    g = _gen(seed, S_LENGTHS)
    lens = torch.randint(min_prefix, max_prefix + 1, (N,), generator=g).to(torch.int32)
    cu = cu_from_lengths(lens.tolist())
    T = int(cu[-1])
    return DecodeInputs(
        prefix_lengths=lens, cu_prefix=cu,
        prefix_k=normal((1, H, T, d), seed, S_PREFIX_K, dtype, device),
        prefix_v=normal((1, H, T, d), seed, S_PREFIX_V, dtype, device),
        q=normal((N, H, d), seed, S_Q, dtype), k=normal((N, H, d), seed, S_K, dtype),
        v=normal((N, H, d), seed, S_V, dtype),
        gamma_q=gammas(H, d, seed, S_GAMMA_Q, "uniform"),
        gamma_k=gammas(H, d, seed, S_GAMMA_K, "uniform"))


def c5_decode(seed: int = 5, device: str = "cpu", N: int = 256, H: int = 32) -> DecodeInputs:
    """Decode step: 256 sequences, H=32, d=128, prefix lengths ~ U{1..8192}."""
    return decode_inputs(N, H, 128, 8192, seed, device=device)


CONFIGS = {
    "c1": "RLA-2 causal forward fp32 [1,2,256,32], one document, RMSNorm weights 1",
    "c2": "RLA-2 causal forward bf16 [4,8,2048,64], chunk 64, one document per row",
    "c3": "packed varlen RLA-2 forward bf16, 16384 tokens, H=16, d=128, lengths U{64..4096}",
    "c4": "long-context RLA-2 causal forward bf16 [1,32,65536,128], 10% of q,k channels shifted by -1",
    "c5": "RLA-2 decode step, 256 sequences x 32 heads, d=128, fp32 state from prefixes U{1..8192}",
}
