"""Seeded sweeps over the parameter space of the chunked forward and its backward, each draw
checked against the oracle at the dtype's tolerance (every output, every pair).

A draw picks the dtype, the head-dim pair, the chunk size, a dense batch (1-3 sequences,
1-300 tokens, or 600-1500 tokens with one or two pairs so that the state pass is cut into
segments) or a packed one (1-4 sequences of 1-200 tokens), the number of key heads and the
value heads per key head (1-3), an initial state or none, and a negative-eigenvalue erase
gate or not. The draws are fixed by their seeds, so every run checks the same cases.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import ORACLE_THREADS, TOL, assert_chunk_parity, flat_inputs, np64, to_gpu

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (128, 128), (128, 64), (64, 128)]
GRADS = ("dq", "dk", "dv", "dw", "dlog_alpha", "db")


def draw(seed, long_ok=True):
    """One configuration of the sweep: (workload, chunk size, description)."""
    rng = np.random.default_rng(1000 + seed)
    dtype = (torch.bfloat16, torch.float32)[int(rng.integers(2))]
    dk, dv = DIMS[int(rng.integers(len(DIMS)))]
    C = (32, 64, 128)[int(rng.integers(3))]
    hk = int(rng.integers(1, 3))
    G = int(rng.integers(1, 4))
    s0 = 0.1 if rng.random() < 0.7 else None
    neg = bool(rng.random() < 0.5)
    kind = rng.random()
    if kind < 0.35:
        n = int(rng.integers(1, 5))
        wl = inputs.small_chunk(dtype=dtype, h_k=hk, h_v=hk * G, d_k=dk, d_v=dv, neg_eig=neg,
                                s0_std=s0, num_seqs=n, len_lo=1, len_hi=200)
        desc = f"packed N={n}"
    elif kind < 0.55 and long_ok:
        hk, G = 1, int(rng.integers(1, 3))
        T = int(rng.integers(600, 1501))
        wl = inputs.small_chunk(dtype=dtype, batch=1, seqlen=T, h_k=hk, h_v=hk * G, d_k=dk,
                                d_v=dv, neg_eig=neg, s0_std=s0)
        desc = f"dense B=1 T={T} (segmented)"
    else:
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 301))
        wl = inputs.small_chunk(dtype=dtype, batch=B, seqlen=T, h_k=hk, h_v=hk * G, d_k=dk,
                                d_v=dv, neg_eig=neg, s0_std=s0)
        desc = f"dense B={B} T={T}"
    name = "bf16" if dtype == torch.bfloat16 else "fp32"
    label = (f"{name} {dk}x{dv} C={C} {desc} h_k={wl.h_k} G={wl.h_v // wl.h_k} "
             f"S0={'yes' if s0 else 'no'} neg_eig={neg}")
    return wl, C, label


@pytest.mark.parametrize("seed", range(64))
def test_forward_sweep(seed):
    wl, C, label = draw(seed)
    print(f"[case] sweep forward seed={seed}: {label}", flush=True)
    x = inputs.chunk_inputs(wl, seed=2000 + seed)
    assert_chunk_parity(x, wl.dtype, label=f"sweep {seed}: {label}", worst=True, chunk_size=C)


@pytest.mark.parametrize("seed", range(32))
def test_backward_sweep(seed):
    """Every gradient of a drawn configuration against the oracle's token adjoint (dense
    draws stay at most 300 tokens long)."""
    wl, C, label = draw(100 + seed, long_ok=False)
    print(f"[case] sweep backward seed={seed}: {label}", flush=True)
    x = inputs.chunk_inputs(wl, seed=3000 + seed)
    d = to_gpu(x)
    dtype = wl.dtype
    B, T = x["q"].shape[:2]
    Hv, dv, dk = x["v"].shape[2], x["v"].shape[3], x["k"].shape[3]
    N = B if x["cu_seqlens"] is None else x["cu_seqlens"].numel() - 1
    gen = torch.Generator().manual_seed(4000 + seed)
    dO = torch.randn(B, T, Hv, dv, generator=gen).to(dtype)
    dST = torch.randn(N, Hv, dk, dv, generator=gen) if seed % 3 else None
    got = g.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO.cuda(),
                      S0=d["S0"], cu_seqlens=d["cu_seqlens"],
                      dS_T=None if dST is None else dST.cuda(), chunk_size=C)
    torch.cuda.synchronize()
    f, cu, S0 = flat_inputs(x)
    ref = oracle.recurrent_bwd(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"],
                               np64(dO).reshape(B * T, Hv, dv), S0=S0,
                               dS_T=None if dST is None else np64(dST), cu_seqlens=cu,
                               threads=ORACLE_THREADS)
    errs = {n: oracle.rel_l2(np64(got[n]).reshape(ref[n].shape), ref[n]) for n in GRADS}
    errs["dS0"] = oracle.rel_l2(np64(got["dS0"]), ref["dS0"])
    print(f"[parity] sweep backward {seed}: {label}: " +
          " ".join(f"{n}={e:.2e}" for n, e in errs.items()), flush=True)
    assert all(np.isfinite(list(errs.values())))
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("seed", range(24))
def test_recurrent_sweep(seed):
    """gdn2_recurrent_fwd on drawn configurations: dtype, stored-state dtype, head-dim pair,
    1-24 tokens per call, 1-5 sequences on a pool of up to twice as many slots (a random
    slot per sequence, sometimes a padding entry), 1-2 key heads with 1-3 value heads each,
    against the oracle's state cache; slots no sequence names must come back unchanged."""
    rng = np.random.default_rng(5000 + seed)
    dtype = (torch.bfloat16, torch.float32)[int(rng.integers(2))]
    sdt = (torch.bfloat16, torch.float32)[int(rng.integers(2))]
    dk, dv = DIMS[int(rng.integers(len(DIMS)))]
    T, N = int(rng.integers(1, 25)), int(rng.integers(1, 6))
    hk, G = int(rng.integers(1, 3)), int(rng.integers(1, 4))
    slots = N + int(rng.integers(0, N + 1))
    idx = [int(s) for s in rng.permutation(slots)[:N]]
    if N > 1 and rng.random() < 0.5:
        idx[int(rng.integers(N))] = -1                   # a padding entry
    label = (f"{'bf16' if dtype == torch.bfloat16 else 'fp32'} inputs, "
             f"{'bf16' if sdt == torch.bfloat16 else 'fp32'} state, {dk}x{dv} T={T} N={N} "
             f"slots={slots} idx={idx} h_k={hk} G={G}")
    print(f"[case] sweep recurrent seed={seed}: {label}", flush=True)
    wl = inputs.DecodeWorkload("recurrent_sweep", dtype, N, hk, hk * G, dk, dv, steps=T)
    x = inputs.decode_inputs(wl, seed=6000 + seed)
    y = {n: x[n].transpose(0, 1).contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    pool = inputs.decode_inputs(replace(wl, num_seqs=slots), seed=7000 + seed, steps=1)["S"]
    pool = pool.to(sdt)
    d = {n: t.cuda() for n, t in y.items()}
    P = pool.cuda()
    o = g.recurrent_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], P,
                        state_idx=torch.tensor(idx, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o_r, P_r = oracle.recurrent_cache(*(np64(y[n]) for n in ("q", "k", "v", "log_alpha", "b", "w")),
                                      np64(pool), idx, bf16_state=sdt == torch.bfloat16,
                                      threads=ORACLE_THREADS)
    live = [n for n in range(N) if idx[n] >= 0]
    for n in range(N):
        if idx[n] < 0:
            assert torch.all(o[n] == 0)
    for s in set(range(slots)) - {idx[n] for n in live}:
        assert torch.equal(P[s].cpu(), pool[s])
    o_g = np64(o)
    eo = oracle.rel_l2(o_g[live], o_r[live])
    es = oracle.rel_l2(np64(P)[[idx[n] for n in live]], P_r[[idx[n] for n in live]])
    bar = 1e-4 if dtype == torch.float32 and sdt == torch.float32 else 2e-2
    print(f"[parity] sweep recurrent {seed}: {label}: o={eo:.2e} S={es:.2e} tol={bar:g}", flush=True)
    assert eo <= bar and es <= bar
