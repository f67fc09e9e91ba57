"""Seeded synthetic inputs for the Gated DeltaNet-2 core.

This module is the only code shared by the GPU path's tests/benchmark and the CPU
oracle. It holds none of the method's arithmetic: it only draws random tensors
with the shapes and value distributions of the workloads and casts them to the
working dtype. Everything that is compared with the oracle is drawn on the host
with numpy's PCG64 in a fixed order (lengths, q, k, v, log_alpha, b, w, S0) in
fp32, then rounded to the working dtype by torch, so both sides read exactly the
same values. The *_device variants draw the same distributions on the GPU with a
seeded torch generator, for timing runs whose outputs are not compared.

Distributions (one reading per workload):
  q, k       ~ N(0,1), L2-normalised per (token, head) before the cast
  v          ~ N(0,1)
  log_alpha  = -softplus(N(0,1))  per key channel   (decay alpha in (0,1))
  b          = sigmoid(N(0,1))    per key channel, or 2*sigmoid(N(0,1)) when the
               negative-eigenvalue option of burn-gdn2 (allow_neg_eigval, "b x 2") is on
  w          = sigmoid(N(0,1))    per value channel
  S0         = 0, or N(0, 0.1^2) fp32 (0.1 read as the standard deviation)
The layouts match the C ABI: q,k [B,T,H_k,d_k]; v,w [B,T,H_v,d_v];
log_alpha,b [B,T,H_v,d_k]; S [N,H_v,d_k,d_v] fp32. Packed (varlen) batches use
B = 1 and an int32 ``cu_seqlens`` of N+1 offsets.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class ChunkWorkload:
    name: str
    dtype: torch.dtype
    batch: int            # dense batch B (1 for packed)
    seqlen: int           # dense T; ignored for packed (drawn lengths decide)
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    chunk_size: int = 64
    neg_eig: bool = False
    s0_std: Optional[float] = None      # None -> S0 = 0
    num_seqs: int = 0                    # > 0 -> packed batch with drawn lengths
    len_lo: int = 0
    len_hi: int = 0


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    dtype: torch.dtype
    num_seqs: int
    h_k: int
    h_v: int
    d_k: int
    d_v: int
    steps: int
    s0_std: float = 0.1


# The five workloads of the measurement plan, named by what they are.
CHUNK_F32_SMALL = ChunkWorkload("chunk_f32_b1_t256_h4_d64", torch.float32, 1, 256, 4, 4, 64, 64)
CHUNK_BF16_B8 = ChunkWorkload("chunk_bf16_b8_t2048_h8_d128", torch.bfloat16, 8, 2048, 8, 8,
                              128, 128)
CHUNK_BF16_T4096 = ChunkWorkload("chunk_bf16_b1_t4096_h16_d128_negeig", torch.bfloat16, 1, 4096,
                                 16, 16, 128, 128, neg_eig=True, s0_std=0.1)
DECODE_F32 = DecodeWorkload("decode_f32_n64_hv48_hk16_d128", torch.float32, 64, 16, 48, 128,
                            128, steps=256)
VARLEN_BF16 = ChunkWorkload("varlen_bf16_n16_hv32_hk16_d128", torch.bfloat16, 1, 0, 16, 32, 128,
                            128, s0_std=0.1, num_seqs=16, len_lo=512, len_hi=8192)

WORKLOADS = {w.name: w for w in (CHUNK_F32_SMALL, CHUNK_BF16_B8, CHUNK_BF16_T4096, DECODE_F32,
                                  VARLEN_BF16)}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _normal(rng, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, 1e-30)).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _cast(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def draw_gates(rng, lead, h_k, h_v, d_k, d_v, neg_eig, dtype, decay_mu=0.0):
    """q,k,v,log_alpha,b,w with leading dims ``lead`` (a tuple), in that draw order."""
    q = _unit_rows(_normal(rng, lead + (h_k, d_k)))
    k = _unit_rows(_normal(rng, lead + (h_k, d_k)))
    v = _normal(rng, lead + (h_v, d_v))
    la = -_softplus(_normal(rng, lead + (h_v, d_k)) + np.float32(decay_mu))
    b = _sigmoid(_normal(rng, lead + (h_v, d_k)))
    if neg_eig:
        b = (2.0 * b).astype(np.float32)
    w = _sigmoid(_normal(rng, lead + (h_v, d_v)))
    return {name: _cast(x, dtype) for name, x in
            (("q", q), ("k", k), ("v", v), ("log_alpha", la), ("b", b), ("w", w))}


def chunk_inputs(wl: ChunkWorkload, seed: int, decay_mu: float = 0.0) -> dict:
    """Inputs of one chunk-forward call (host tensors).

    Returns q,k,v,log_alpha,b,w [B,T,...] in ``wl.dtype``, ``S0`` fp32 [N,H_v,d_k,d_v] or
    None, ``cu_seqlens`` int32 [N+1] or None, and ``num_seqs``. ``decay_mu`` shifts the
    normal draw under the softplus (a positive value gives an extreme-decay stress input).
    """
    rng = _rng(seed)
    if wl.num_seqs > 0:
        lens = rng.integers(wl.len_lo, wl.len_hi, size=wl.num_seqs, endpoint=True)
        cu = np.zeros(wl.num_seqs + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lens)
        B, T, N = 1, int(cu[-1]), wl.num_seqs
        cu_t = torch.from_numpy(cu.astype(np.int32))
    else:
        B, T, N = wl.batch, wl.seqlen, wl.batch
        cu_t = None
    out = draw_gates(rng, (B, T), wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.neg_eig, wl.dtype, decay_mu)
    if wl.s0_std is None:
        out["S0"] = None
    else:
        out["S0"] = torch.from_numpy(
            (_normal(rng, (N, wl.h_v, wl.d_k, wl.d_v)) * np.float32(wl.s0_std)))
    out["cu_seqlens"] = cu_t
    out["num_seqs"] = N
    return out


def decode_inputs(wl: DecodeWorkload, seed: int, steps: Optional[int] = None) -> dict:
    """Inputs of ``steps`` consecutive decode steps (host tensors).

    q,k [steps,N,H_k,d_k]; v,w [steps,N,H_v,d_v]; log_alpha,b [steps,N,H_v,d_k] in
    ``wl.dtype``; S [N,H_v,d_k,d_v] fp32, the state before the first step.
    """
    rng = _rng(seed)
    st = wl.steps if steps is None else steps
    out = draw_gates(rng, (st, wl.num_seqs), wl.h_k, wl.h_v, wl.d_k, wl.d_v, False, wl.dtype)
    out["S"] = torch.from_numpy(
        _normal(rng, (wl.num_seqs, wl.h_v, wl.d_k, wl.d_v)) * np.float32(wl.s0_std))
    return out


def chunk_inputs_device(wl: ChunkWorkload, seed: int, device="cuda") -> dict:
    """Same shapes and distributions as ``chunk_inputs``, drawn directly on the GPU with a
    seeded torch generator (for timing runs of large workloads, where host generation would
    dominate). The values differ from ``chunk_inputs`` for the same seed; the packed lengths
    are drawn on the host with the same numpy recipe."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    if wl.num_seqs > 0:
        lens = _rng(seed).integers(wl.len_lo, wl.len_hi, size=wl.num_seqs, endpoint=True)
        cu = np.zeros(wl.num_seqs + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lens)
        B, T, N = 1, int(cu[-1]), wl.num_seqs
        cu_t = torch.from_numpy(cu.astype(np.int32)).to(device)
    else:
        B, T, N = wl.batch, wl.seqlen, wl.batch
        cu_t = None

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)

    out = {"q": unit(normal(B, T, wl.h_k, wl.d_k)), "k": unit(normal(B, T, wl.h_k, wl.d_k)),
           "v": normal(B, T, wl.h_v, wl.d_v),
           "log_alpha": -torch.nn.functional.softplus(normal(B, T, wl.h_v, wl.d_k)),
           "b": torch.sigmoid(normal(B, T, wl.h_v, wl.d_k)) * (2.0 if wl.neg_eig else 1.0),
           "w": torch.sigmoid(normal(B, T, wl.h_v, wl.d_v))}
    out = {n: x.to(wl.dtype).contiguous() for n, x in out.items()}
    out["S0"] = None if wl.s0_std is None else normal(N, wl.h_v, wl.d_k, wl.d_v) * wl.s0_std
    out["cu_seqlens"] = cu_t
    out["num_seqs"] = N
    return out


def decode_inputs_device(wl: DecodeWorkload, seed: int, steps: int, device="cuda") -> dict:
    """Decode inputs drawn on the GPU (same shapes and distributions as ``decode_inputs``)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)

    N = wl.num_seqs
    out = {"q": unit(normal(steps, N, wl.h_k, wl.d_k)), "k": unit(normal(steps, N, wl.h_k, wl.d_k)),
           "v": normal(steps, N, wl.h_v, wl.d_v),
           "log_alpha": -torch.nn.functional.softplus(normal(steps, N, wl.h_v, wl.d_k)),
           "b": torch.sigmoid(normal(steps, N, wl.h_v, wl.d_k)),
           "w": torch.sigmoid(normal(steps, N, wl.h_v, wl.d_v))}
    out = {n: x.to(wl.dtype).contiguous() for n, x in out.items()}
    out["S"] = normal(N, wl.h_v, wl.d_k, wl.d_v) * wl.s0_std
    return out


def small_chunk(dtype=torch.float32, batch=1, seqlen=100, h_k=2, h_v=2, d_k=64, d_v=64,
                neg_eig=False, s0_std=0.1, num_seqs=0, len_lo=0, len_hi=0,
                name="small") -> ChunkWorkload:
    """A reduced chunk workload with the same distributions (for parity at small sizes)."""
    return ChunkWorkload(name, dtype, batch, seqlen, h_k, h_v, d_k, d_v, 64, neg_eig, s0_std,
                         num_seqs, len_lo, len_hi)


def with_dtype(wl, dtype):
    return replace(wl, dtype=dtype)


def variant_inputs(mode: str, dtype, N: int, T: int, h_k: int, h_v: int, d_k: int, d_v: int,
                   seed: int, s0_std: float = 0.1) -> dict:
    """Inputs of a delta-rule variant (host tensors, leading dims [N, T]): q, k unit rows;
    v normal; log_alpha = -softplus(normal) per channel ([N,T,H_v,d_k]) or, for "gdn", per
    head ([N,T,H_v]); beta = sigmoid(normal) per head ("kda", "gdn": [N,T,H_v]) or per key
    channel ("fg2", "fg2+": [N,T,H_v,d_k]); beta_v = sigmoid(normal) [N,T,H_v,d_v] for "fg2+";
    S fp32 [N,H_v,d_k,d_v] normal * s0_std."""
    rng = _rng(seed)
    lead = (N, T)
    q = _unit_rows(_normal(rng, lead + (h_k, d_k)))
    k = _unit_rows(_normal(rng, lead + (h_k, d_k)))
    v = _normal(rng, lead + (h_v, d_v))
    la_shape = lead + ((h_v,) if mode == "gdn" else (h_v, d_k))
    la = -_softplus(_normal(rng, la_shape))
    beta = _sigmoid(_normal(rng, lead + ((h_v,) if mode in ("kda", "gdn") else (h_v, d_k))))
    out = {"q": q, "k": k, "v": v, "log_alpha": la, "beta": beta}
    if mode == "fg2+":
        out["beta_v"] = _sigmoid(_normal(rng, lead + (h_v, d_v)))
    out = {n: _cast(x, dtype) for n, x in out.items()}
    out["S"] = torch.from_numpy(_normal(rng, (N, h_v, d_k, d_v)) * np.float32(s0_std))
    return out
