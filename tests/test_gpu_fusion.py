"""GPU parity of the optional fusions around the recurrence (gdn2_fusion): the q/k L2-norm
before it and the SiLU-gated RMS norm after it (burn-gdn2 "Architecture"), in the chunked
forward and in the recurrent forward, against the fp64 oracle composed the same way:
    o_ref = gated_rms_norm(recurrence(l2_normalize(q), l2_normalize(k), ...), gate, w, eps)

q and k are drawn with row norms far from one (each row scaled by exp(N(0, 0.5))), so the
L2-norm changes the result. Gate: relative L2 error 1e-4 for fp32, 2e-2 for bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import TOL, flat_inputs, np64

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "b", "w")
L2EPS, NEPS = 1e-6, 1e-5


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


def unnormalise(x, seed):
    """Scale every q and k row by exp(N(0, 0.5)) (recast to the working dtype)."""
    rng = np.random.default_rng(seed)
    for n in ("q", "k"):
        t = x[n]
        s = np.exp(0.5 * rng.standard_normal(t.shape[:-1] + (1,))).astype(np.float32)
        x[n] = (t.float() * torch.from_numpy(s)).to(t.dtype).contiguous()
    return x


def gate_and_weight(shape, dtype, d_v, seed):
    rng = np.random.default_rng(seed)
    gate = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dtype)
    w = torch.from_numpy(rng.uniform(0.5, 1.5, d_v).astype(np.float32))
    return gate, w


def oracle_fused(o_rec, gate, w, qk_norm, with_gate):
    if not with_gate:
        return o_rec
    return oracle.gated_rms_norm(o_rec, np64(gate), np64(w), NEPS)


@pytest.mark.parametrize("qk_norm,with_gate", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("dtype,dk,dv,B,T,hk,hv", [
    (torch.bfloat16, 128, 128, 1, 1000, 1, 2),      # segmented state pass
    (torch.bfloat16, 128, 64, 2, 130, 1, 3),        # GVA, ragged tail
    (torch.bfloat16, 64, 128, 3, 65, 2, 2),
    (torch.float32, 64, 64, 2, 200, 1, 2),
])
def test_chunk_fusions(dtype, dk, dv, B, T, hk, hv, qk_norm, with_gate):
    wl = inputs.small_chunk(dtype=dtype, batch=B, seqlen=T, h_k=hk, h_v=hv, d_k=dk, d_v=dv,
                            neg_eig=True, s0_std=0.1)
    x = unnormalise(inputs.chunk_inputs(wl, seed=80 + T), seed=81)
    gate, w = gate_and_weight((B, T, hv, dv), dtype, dv, seed=82)
    d = {n: x[n].cuda() for n in NAMES}
    o, S_T = g.chunk_fwd(*(d[n] for n in NAMES), S0=x["S0"].cuda(), qk_l2norm=qk_norm,
                         l2norm_eps=L2EPS, gate=gate.cuda() if with_gate else None,
                         norm_weight=w.cuda() if with_gate else None, norm_eps=NEPS)
    torch.cuda.synchronize()
    f, cu, S0 = flat_inputs(x)
    if qk_norm:
        f["q"], f["k"] = oracle.l2_normalize(f["q"], L2EPS), oracle.l2_normalize(f["k"], L2EPS)
    o_r, S_r = oracle.recurrent(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], S0=S0,
                                cu_seqlens=cu, threads=16)
    o_r = oracle_fused(o_r, gate.reshape(B * T, hv, dv), w, qk_norm, with_gate)
    eo = oracle.rel_l2(np64(o).reshape(B * T, hv, dv), o_r)
    es = oracle.rel_l2(np64(S_T), S_r)
    print(f"[parity] chunk fusion qk={qk_norm} gate={with_gate} {dtype} {dk}x{dv} B={B} T={T}: "
          f"o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_chunk_fusions_packed_and_full_size():
    """Varlen batch with an empty sequence, then the timed workload (B=1, T=4096, 16 heads,
    d=128), both with the L2-norm and the gated norm."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, h_k=2, h_v=4, d_k=128, d_v=128, num_seqs=5,
                            len_lo=1, len_hi=300)
    cases = [unnormalise(inputs.chunk_inputs(wl, seed=90), seed=91),
             unnormalise(inputs.chunk_inputs(inputs.CHUNK_BF16_T4096, seed=1002), seed=92)]
    cu = cases[0]["cu_seqlens"].clone()
    lens = (cu[1:] - cu[:-1]).tolist()
    lens[1] = 0
    cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
    for n in NAMES:
        cases[0][n] = cases[0][n][:, :int(cu[-1])].contiguous()
    cases[0]["cu_seqlens"] = cu
    for i, x in enumerate(cases):
        B, T, hv, dv = x["v"].shape
        gate, w = gate_and_weight((B, T, hv, dv), torch.bfloat16, dv, seed=93 + i)
        d = {n: x[n].cuda() for n in NAMES}
        o, S_T = g.chunk_fwd(*(d[n] for n in NAMES), S0=x["S0"].cuda(),
                             cu_seqlens=None if x["cu_seqlens"] is None else x["cu_seqlens"].cuda(),
                             qk_l2norm=True, l2norm_eps=L2EPS, gate=gate.cuda(),
                             norm_weight=w.cuda(), norm_eps=NEPS)
        torch.cuda.synchronize()
        f, cu_np, S0 = flat_inputs(x)
        o_r, S_r = oracle.recurrent(oracle.l2_normalize(f["q"], L2EPS),
                                    oracle.l2_normalize(f["k"], L2EPS), f["v"], f["log_alpha"],
                                    f["b"], f["w"], S0=S0, cu_seqlens=cu_np, threads=16)
        o_r = oracle.gated_rms_norm(o_r, np64(gate).reshape(B * T, hv, dv), np64(w), NEPS)
        eo = oracle.rel_l2(np64(o).reshape(B * T, hv, dv), o_r)
        es = oracle.rel_l2(np64(S_T), S_r)
        print(f"[parity] chunk fusion case {i} (T={T}, {hv} heads): o={eo:.2e} S_T={es:.2e}",
              flush=True)
        assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("qk_norm,with_gate", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("dtype,state_dtype,T", [(torch.float32, torch.float32, 1),
                                                  (torch.float32, torch.float32, 5),
                                                  (torch.bfloat16, torch.bfloat16, 1),
                                                  (torch.bfloat16, torch.float32, 11)])
def test_recurrent_fusions(dtype, state_dtype, T, qk_norm, with_gate):
    wl = inputs.DecodeWorkload("recurrent_fusion", dtype, 5, 2, 6, 128, 128, steps=T)
    x = inputs.decode_inputs(wl, seed=100 + T)
    y = unnormalise({n: x[n].transpose(0, 1).contiguous() for n in NAMES}, seed=101)
    pool = torch.cat([x["S"], x["S"][:2]]).to(state_dtype)          # 7 slots
    idx = [6, 0, -1, 3, 2]                                          # one padding entry
    gate, w = gate_and_weight((5, T, 6, 128), dtype, 128, seed=102)
    P = pool.cuda()
    o = g.recurrent_fwd(*(y[n].cuda() for n in NAMES), P,
                        state_idx=torch.tensor(idx, dtype=torch.int32, device="cuda"),
                        qk_l2norm=qk_norm, l2norm_eps=L2EPS,
                        gate=gate.cuda() if with_gate else None,
                        norm_weight=w.cuda() if with_gate else None, norm_eps=NEPS)
    torch.cuda.synchronize()
    q, k = np64(y["q"]), np64(y["k"])
    if qk_norm:
        q, k = oracle.l2_normalize(q, L2EPS), oracle.l2_normalize(k, L2EPS)
    o_r, P_r = oracle.recurrent_cache(q, k, *(np64(y[n]) for n in NAMES[2:]), np64(pool), idx,
                                      bf16_state=state_dtype == torch.bfloat16, threads=16)
    o_r = oracle_fused(o_r, gate, w, qk_norm, with_gate)
    o_g = np64(o)
    assert np.all(o_g[2] == 0.0)                                    # padding entry
    tol = 1e-4 if dtype == torch.float32 and state_dtype == torch.float32 else 2e-2
    eo, es = oracle.rel_l2(o_g, o_r), oracle.rel_l2(np64(P), P_r)
    print(f"[parity] recurrent fusion qk={qk_norm} gate={with_gate} {dtype} state "
          f"{state_dtype} T={T}: o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= tol and es <= tol


def test_fusions_on_unit_rows_change_only_the_output_stage():
    """The workloads' q and k rows already have unit norm: with the L2-norm alone the
    result stays within the bf16 bar of the unfused call, and the state is unchanged by the
    gated norm (which only rescales outputs)."""
    x = inputs.chunk_inputs(inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=300,
                                               h_k=2, h_v=2, d_k=128, d_v=128), seed=110)
    d = {n: x[n].cuda() for n in NAMES}
    S0 = x["S0"].cuda()
    o0, S0_T = g.chunk_fwd(*(d[n] for n in NAMES), S0=S0)
    o1, S1_T = g.chunk_fwd(*(d[n] for n in NAMES), S0=S0, qk_l2norm=True, l2norm_eps=L2EPS)
    gate, w = gate_and_weight((1, 300, 2, 128), torch.bfloat16, 128, seed=111)
    o2, S2_T = g.chunk_fwd(*(d[n] for n in NAMES), S0=S0, gate=gate.cuda(), norm_weight=w.cuda())
    torch.cuda.synchronize()
    assert oracle.rel_l2(np64(o1), np64(o0)) <= 2e-2
    assert oracle.rel_l2(np64(S1_T), np64(S0_T)) <= 2e-2
    assert torch.equal(S2_T, S0_T)


# ---- short causal convolution of q, k, v fused into the recurrent forward ---------------

def conv_case(dtype, N, T, hk, hv, d, slots, seed):
    wl = inputs.DecodeWorkload("recurrent_conv", dtype, N, hk, hv, d, d, steps=T)
    x = inputs.decode_inputs(wl, seed=seed)
    y = {n: x[n].transpose(0, 1).contiguous() for n in NAMES}
    C = 2 * hk * d + hv * d
    rng = np.random.default_rng(seed + 1)
    cw = torch.from_numpy((0.5 * rng.standard_normal((C, 4))).astype(np.float32))
    cpool = torch.from_numpy(rng.standard_normal((slots, 3, C)).astype(np.float32))
    pool = torch.from_numpy((0.1 * rng.standard_normal((slots, hv, d, d))).astype(np.float32))
    return y, cw, cpool, pool


def oracle_conv_call(y, cw, cpool, pool, idx, silu, qk_norm, gate=None, w=None,
                     bf16_state=False):
    q, k, v, cnew = oracle.conv_qkv(np64(y["q"]), np64(y["k"]), np64(y["v"]), np64(cw),
                                    cpool, idx, silu)
    if qk_norm:
        q, k = oracle.l2_normalize(q, L2EPS), oracle.l2_normalize(k, L2EPS)
    o, pnew = oracle.recurrent_cache(q, k, v, np64(y["log_alpha"]), np64(y["b"]), np64(y["w"]),
                                     pool, idx, bf16_state=bf16_state, threads=16)
    if gate is not None:
        o = oracle.gated_rms_norm(o, np64(gate), np64(w), NEPS)
        o[[i for i, s in enumerate(idx) if not 0 <= s < pool.shape[0]]] = 0.0
    return o, pnew, cnew


@pytest.mark.parametrize("silu", [False, True])
@pytest.mark.parametrize("dtype,T,extra", [(torch.float32, 1, False), (torch.float32, 2, True),
                                           (torch.float32, 5, False), (torch.bfloat16, 1, True),
                                           (torch.bfloat16, 11, False), (torch.bfloat16, 3, True)])
def test_recurrent_short_conv(dtype, T, extra, silu):
    """GVA (3 value heads per key head), 7 slots with a padding entry; `extra` also turns on
    the L2-norm and the gated output norm."""
    y, cw, cpool, pool = conv_case(dtype, 5, T, 2, 6, 128, 7, seed=120 + T)
    idx = [6, 0, -1, 3, 2]
    gate, w = gate_and_weight((5, T, 6, 128), dtype, 128, seed=121) if extra else (None, None)
    P, CP = pool.cuda(), cpool.cuda()
    o = g.recurrent_fwd(*(y[n].cuda() for n in NAMES), P,
                        state_idx=torch.tensor(idx, dtype=torch.int32, device="cuda"),
                        qk_l2norm=extra, l2norm_eps=L2EPS,
                        gate=None if gate is None else gate.cuda(),
                        norm_weight=None if w is None else w.cuda(), norm_eps=NEPS,
                        conv_weight=cw.cuda(), conv_state=CP, conv_silu=silu)
    torch.cuda.synchronize()
    o_r, P_r, C_r = oracle_conv_call(y, cw, np64(cpool), np64(pool), idx, silu, extra, gate, w)
    assert np.array_equal(np64(CP), C_r)          # the new conv state is the raw inputs
    assert np.all(np64(o)[2] == 0.0)
    tol = TOL[dtype]
    eo, es = oracle.rel_l2(np64(o), o_r), oracle.rel_l2(np64(P), P_r)
    print(f"[parity] short conv silu={silu} {dtype} T={T} extra={extra}: o={eo:.2e} S={es:.2e}",
          flush=True)
    assert eo <= tol and es <= tol


def test_short_conv_state_carried_over_calls():
    """Eight calls of two tokens each (fewer than the conv width) on one pair of pools, with
    a bf16 recurrent state: every call against the oracle carrying both pools."""
    dtype, calls, T = torch.bfloat16, 8, 2
    y, cw, cpool, pool = conv_case(dtype, 4, calls * T, 1, 2, 64, 4, seed=130)
    P, CP = pool.to(torch.bfloat16).cuda(), cpool.cuda()
    Pr, Cr = oracle.round_to_bf16(np64(pool)), np64(cpool)
    eo_max = 0.0
    for c in range(calls):
        part = {n: y[n][:, c * T:(c + 1) * T].contiguous() for n in NAMES}
        o = g.recurrent_fwd(*(part[n].cuda() for n in NAMES), P, conv_weight=cw.cuda(),
                            conv_state=CP, conv_silu=True)
        o_r, Pr, Cr = oracle_conv_call(part, cw, Cr, Pr, None, True, False, bf16_state=True)
        torch.cuda.synchronize()
        eo_max = max(eo_max, oracle.rel_l2(np64(o), o_r))
        assert np.array_equal(np64(CP), Cr)
    es = oracle.rel_l2(np64(P), Pr)
    print(f"[parity] short conv over {calls} calls of {T} tokens: o max={eo_max:.2e} S={es:.2e}",
          flush=True)
    assert eo_max <= 2e-2 and es <= 2e-2
