"""GPU parity of the multi-token recurrent forward against a state cache (gdn2_recurrent_fwd):
T tokens per sequence, slot indirection with padding entries, fp32 and bf16 stored states.

Gate (relative L2 error per output tensor): 1e-4 when inputs and state are fp32, 2e-2 when
either is bf16, on o and on the updated slots. Slots that no sequence names must come back
bit for bit unchanged.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import np64

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "b", "w")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


def seq_major(x):
    """decode_inputs draws [steps, N, ...]; the multi-token call takes [N, T, ...]."""
    return {n: x[n].transpose(0, 1).contiguous() for n in NAMES}


def tol(dtype, state_dtype):
    return 1e-4 if dtype == torch.float32 and state_dtype == torch.float32 else 2e-2


def run_gpu(x, pool, idx=None):
    d = {n: x[n].cuda() for n in NAMES}
    S = pool.cuda()
    o = g.recurrent_fwd(*(d[n] for n in NAMES), S, state_idx=None if idx is None else
                        torch.tensor(idx, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    return np64(o), S


def run_oracle(x, pool, idx=None, bf16_state=False):
    return oracle.recurrent_cache(*(np64(x[n]) for n in NAMES), np64(pool), idx,
                                  bf16_state=bf16_state, threads=16)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 5, 8, 19])
def test_multi_token_fp32_state(dtype, dk, dv, T):
    wl = inputs.DecodeWorkload("recurrent_small", dtype, 3, 2, 6, dk, dv, steps=T)
    x = inputs.decode_inputs(wl, seed=40 + T)
    y = seq_major(x)
    o_g, S = run_gpu(y, x["S"])
    o_r, S_r = run_oracle(y, x["S"])
    eo, es = oracle.rel_l2(o_g, o_r), oracle.rel_l2(np64(S), S_r)
    print(f"[parity] recurrent_fwd {dtype} {dk}x{dv} T={T}: o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= tol(dtype, torch.float32) and es <= tol(dtype, torch.float32)


@pytest.mark.parametrize("state_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_slots_and_padding_entries(dtype, state_dtype):
    wl = inputs.DecodeWorkload("recurrent_slots", dtype, 6, 2, 4, 128, 128, steps=3)
    x = inputs.decode_inputs(wl, seed=50)
    y = seq_major(x)
    pool = inputs.decode_inputs(replace(wl, num_seqs=10), seed=51, steps=1)["S"]
    pool = pool.to(state_dtype)
    idx = [7, 2, -1, 9, 0, 12]                 # -1 and 12 (>= 10 slots) are padding entries
    o_g, S = run_gpu(y, pool, idx)
    o_r, S_r = run_oracle(y, pool, idx, bf16_state=state_dtype == torch.bfloat16)
    S_g = np64(S)
    for n in (2, 5):
        assert np.all(o_g[n] == 0.0)
    for s in (1, 3, 4, 5, 6, 8):               # slots no sequence names
        assert torch.equal(S[s].cpu(), pool[s])
    live = [7, 2, 9, 0]
    eo = oracle.rel_l2(o_g[[0, 1, 3, 4]], o_r[[0, 1, 3, 4]])
    es = oracle.rel_l2(S_g[live], S_r[live])
    print(f"[parity] slots {dtype} state {state_dtype}: o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= tol(dtype, state_dtype) and es <= tol(dtype, state_dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T", [1, 4])
def test_bf16_state_over_many_calls(dtype, T):
    """20 consecutive calls on a bf16 pool: the oracle rounds the stored state after each."""
    calls = 20
    wl = inputs.DecodeWorkload("recurrent_bf16_state", dtype, 4, 2, 6, 128, 128, steps=calls * T)
    x = inputs.decode_inputs(wl, seed=60 + T)
    y = seq_major(x)
    pool = x["S"].to(torch.bfloat16)
    P = pool.cuda()
    Pr = np64(pool)
    o_g, o_r = [], []
    for c in range(calls):
        sl = slice(c * T, (c + 1) * T)
        part = {n: y[n][:, sl].contiguous() for n in NAMES}
        d = {n: part[n].cuda() for n in NAMES}
        o_g.append(np64(g.recurrent_fwd(*(d[n] for n in NAMES), P)))
        oc, Pr = oracle.recurrent_cache(*(np64(part[n]) for n in NAMES), Pr, None,
                                        bf16_state=True, threads=16)
        o_r.append(oc)
    torch.cuda.synchronize()
    eo = oracle.rel_l2(np.concatenate(o_g, 1), np.concatenate(o_r, 1))
    es = oracle.rel_l2(np64(P), Pr)
    print(f"[parity] bf16 state {dtype} T={T} x {calls} calls: o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


def sampled_pairs(wl, seed, count=24):
    rng = np.random.default_rng(seed)
    return [(int(n), int(h)) for n, h in zip(rng.integers(0, wl.num_seqs, count),
                                             rng.integers(0, wl.h_v, count))]


def test_decode_full_size_bf16_state_256_steps():
    """64 sequences x 48 value heads over 16 key heads, d=128, bf16 stored state, 256
    single-token calls; 24 sampled states against the oracle, which rounds the stored state
    to bf16 after every call as the library does."""
    wl = inputs.DECODE_F32
    x = inputs.decode_inputs(wl, seed=3)
    y = seq_major(x)
    dev = {n: y[n].cuda() for n in NAMES}
    P = x["S"].to(torch.bfloat16).cuda()
    o_all = torch.empty(wl.num_seqs, wl.steps, wl.h_v, wl.d_v, device="cuda")
    for t in range(wl.steps):
        o_all[:, t] = g.recurrent_fwd(*(dev[n][:, t:t + 1].contiguous() for n in NAMES),
                                      P)[:, 0]
    torch.cuda.synchronize()
    o_g, S_g = np64(o_all), np64(P)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(S_g))
    G = wl.h_v // wl.h_k
    go, gs, ro, rs = [], [], [], []
    for n, h in sampled_pairs(wl, 5):
        one = {nm: np64(y[nm][n:n + 1, :, (h // G if nm in ("q", "k") else h)])[:, :, None]
               for nm in NAMES}
        S = oracle.round_to_bf16(np64(x["S"][n:n + 1, h:h + 1]))
        on = []
        for t in range(wl.steps):
            ot, S = oracle.recurrent_cache(*(one[nm][:, t:t + 1] for nm in NAMES), S, None,
                                           bf16_state=True, threads=1)
            on.append(ot[0, 0, 0])
        go.append(o_g[n, :, h].ravel()); ro.append(np.stack(on).ravel())
        gs.append(S_g[n, h].ravel()); rs.append(S[0, 0].ravel())
    eo = oracle.rel_l2(np.concatenate(go), np.concatenate(ro))
    es = oracle.rel_l2(np.concatenate(gs), np.concatenate(rs))
    print(f"[parity] decode bf16 state 256 steps, 24 sampled states: o={eo:.2e} S={es:.2e}",
          flush=True)
    assert eo <= 2e-2 and es <= 2e-2


def test_multi_token_full_size_fp32_state():
    """The decode workload in calls of 4 tokens (64 calls = 256 tokens), fp32 state: equal to
    one 256-token recurrence per state; 24 sampled states."""
    wl = inputs.DECODE_F32
    x = inputs.decode_inputs(wl, seed=4)
    y = seq_major(x)
    dev = {n: y[n].cuda() for n in NAMES}
    P = x["S"].cuda()
    o_all = torch.empty(wl.num_seqs, wl.steps, wl.h_v, wl.d_v, device="cuda")
    for c in range(wl.steps // 4):
        sl = slice(4 * c, 4 * c + 4)
        o_all[:, sl] = g.recurrent_fwd(*(dev[n][:, sl].contiguous() for n in NAMES), P)
    torch.cuda.synchronize()
    o_g, S_g = np64(o_all), np64(P)
    G = wl.h_v // wl.h_k
    go, gs, ro, rs = [], [], [], []
    for n, h in sampled_pairs(wl, 6):
        hk = h // G
        on, Sn = oracle.sequence(np64(y["q"][n, :, hk]), np64(y["k"][n, :, hk]),
                                 np64(y["v"][n, :, h]), np64(y["w"][n, :, h]),
                                 np64(y["log_alpha"][n, :, h]), np64(y["b"][n, :, h]),
                                 np64(x["S"][n, h]))
        go.append(o_g[n, :, h].ravel()); ro.append(on.ravel())
        gs.append(S_g[n, h].ravel()); rs.append(Sn.ravel())
    eo = oracle.rel_l2(np.concatenate(go), np.concatenate(ro))
    es = oracle.rel_l2(np.concatenate(gs), np.concatenate(rs))
    print(f"[parity] multi-token T=4 x 64 calls, 24 sampled states: o={eo:.2e} S={es:.2e}",
          flush=True)
    assert eo <= 1e-4 and es <= 1e-4


def test_multi_token_call_equals_single_steps_and_chunk_forward():
    """Invariants at T = 37: one call equals 37 single-token calls (bitwise for o is not
    required; both against the same tolerance), and equals the chunked forward from the
    same initial state."""
    wl = inputs.DecodeWorkload("recurrent_vs_chunk", torch.bfloat16, 2, 1, 3, 128, 128, steps=37)
    x = inputs.decode_inputs(wl, seed=70)
    y = seq_major(x)
    d = {n: y[n].cuda() for n in NAMES}
    P1 = x["S"].cuda()
    o1 = g.recurrent_fwd(*(d[n] for n in NAMES), P1)
    P2 = x["S"].cuda()
    o2 = torch.stack([g.recurrent_fwd(*(d[n][:, t:t + 1].contiguous() for n in NAMES), P2)[:, 0]
                      for t in range(wl.steps)], 1)
    oc, Sc = g.chunk_fwd(*(d[n] for n in NAMES), S0=x["S"].cuda())
    torch.cuda.synchronize()
    assert oracle.rel_l2(np64(o1), np64(o2)) <= 1e-5
    assert oracle.rel_l2(np64(P1), np64(P2)) <= 1e-5
    assert oracle.rel_l2(np64(o1), np64(oc)) <= 2e-2
    assert oracle.rel_l2(np64(P1), np64(Sc)) <= 2e-2
