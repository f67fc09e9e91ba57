"""GPU cross-path checks: the two computations of the recurrence agree with each other and
with the oracle, resuming from a state equals one long call, packing equals separate
calls, in-place continuation works, and repeated runs are bitwise identical."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import TOL, gpu_chunk, np64, oracle_chunk, to_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_steps_equal_chunk_forward(dtype):
    wl = inputs.small_chunk(dtype=dtype, batch=3, seqlen=70, h_k=2, h_v=4, d_k=64, d_v=64,
                            neg_eig=True)
    x = inputs.chunk_inputs(wl, seed=31)
    o_c, S_c = gpu_chunk(x)
    d = to_gpu(x)
    S = d["S0"].clone()
    outs = []
    for t in range(70):
        o = g.recurrent_step(*(d[n][:, t].contiguous() for n in
                               ("q", "k", "v", "log_alpha", "b", "w")), S)
        outs.append(np64(o))
    torch.cuda.synchronize()
    o_d = np.stack(outs, axis=1).reshape(3 * 70, 4, 64)
    o_r, S_r = oracle_chunk(x)
    tol = TOL[dtype]
    for name, a, b in (("decode o", o_d, o_r), ("chunk o", o_c, o_r),
                       ("decode S", np64(S), S_r), ("chunk S", S_c, S_r)):
        e = oracle.rel_l2(a, b)
        print(f"[cross] {dtype} {name} vs oracle {e:.2e}", flush=True)
        assert e <= tol
    assert oracle.rel_l2(o_d, o_c) <= 2 * tol


def test_split_resume_equals_one_call():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=300, h_k=2, h_v=2, d_k=128,
                            d_v=128, neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=32)
    o_all, S_all = gpu_chunk(x)
    t = 100                                     # not a multiple of the chunk size
    xa = dict(x)
    xb = dict(x)
    for n in ("q", "k", "v", "log_alpha", "b", "w"):
        xa[n] = x[n][:, :t].contiguous()
        xb[n] = x[n][:, t:].contiguous()
    o_a, S_a = gpu_chunk(xa)
    xb["S0"] = torch.from_numpy(S_a.astype(np.float32))
    o_b, S_b = gpu_chunk(xb)
    o_r, S_r = oracle_chunk(x)
    assert oracle.rel_l2(np.concatenate([o_a, o_b]), o_r) <= 2e-2
    assert oracle.rel_l2(S_b, S_r) <= 2e-2
    assert oracle.rel_l2(np.concatenate([o_a, o_b]), o_all) <= 2e-2
    assert oracle.rel_l2(S_b, S_all) <= 2e-2


def test_packed_equals_separate_calls():
    wl = inputs.small_chunk(dtype=torch.bfloat16, h_k=1, h_v=2, d_k=128, d_v=128, num_seqs=3,
                            len_lo=30, len_hi=200)
    x = inputs.chunk_inputs(wl, seed=33)
    o_p, S_p = gpu_chunk(x)
    cu = x["cu_seqlens"].tolist()
    for n in range(3):
        xs = {k: v for k, v in x.items()}
        for nm in ("q", "k", "v", "log_alpha", "b", "w"):
            xs[nm] = x[nm][:, cu[n]:cu[n + 1]].contiguous()
        xs["S0"] = x["S0"][n:n + 1].contiguous()
        xs["cu_seqlens"] = None
        o_s, S_s = gpu_chunk(xs)
        assert np.array_equal(o_p[cu[n]:cu[n + 1]], o_s)
        assert np.array_equal(S_p[n], S_s[0])


def test_final_state_may_alias_initial_state():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=2, seqlen=150, h_k=1, h_v=2, d_k=128,
                            d_v=64, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=34)
    o_ref, S_ref = gpu_chunk(x)
    d = to_gpu(x)
    S = d["S0"].clone()
    o, S_T = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=S,
                         final_state=S)
    torch.cuda.synchronize()
    assert S_T.data_ptr() == S.data_ptr()
    assert np.array_equal(np64(S), S_ref)
    assert np.array_equal(np64(o).reshape(o_ref.shape), o_ref)


def test_repeated_runs_are_bitwise_identical():
    x = inputs.chunk_inputs(inputs.CHUNK_BF16_T4096, seed=35)
    o1, S1 = gpu_chunk(x)
    o2, S2 = gpu_chunk(x)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    wl = inputs.DecodeWorkload("decode_det", torch.float32, 8, 4, 12, 128, 128, steps=1)
    y = inputs.decode_inputs(wl, seed=36)
    outs = []
    for _ in range(2):
        S = y["S"].cuda()
        o = g.recurrent_step(*(y[n][0].cuda() for n in ("q", "k", "v", "log_alpha", "b", "w")), S)
        outs.append((np64(o), np64(S)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
