"""gdn2_chunk_fwd_noalloc (the chunked forward on the library's static device workspace)
against gdn2_chunk_fwd (a caller workspace) and the fp64 oracle, through the C ABI.

Two calls in a row on the static array, the second smaller than the first, so that the
second runs over what the first left behind: each must give exactly the bits of the regular
call on the same inputs, and both must meet the oracle's bf16 / fp32 gates.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import TOL, np64, oracle_chunk, to_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


def run_both(x, chunk_size=64):
    d = to_gpu(x)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    o_ref, S_ref = g.chunk_fwd(*args, S0=d["S0"], cu_seqlens=d["cu_seqlens"], chunk_size=chunk_size)
    o_na, S_na = g.chunk_fwd_noalloc(*args, S0=d["S0"], cu_seqlens=d["cu_seqlens"],
                                     chunk_size=chunk_size)
    torch.cuda.synchronize()
    return np64(o_ref), np64(S_ref), np64(o_na), np64(S_na)


def check(x, dtype, label, chunk_size=64):
    o_ref, S_ref, o_na, S_na = run_both(x, chunk_size)
    assert np.array_equal(o_na, o_ref) and np.array_equal(S_na, S_ref), label
    o_r, S_r = oracle_chunk(x)
    B, T = x["q"].shape[:2]
    eo = oracle.rel_l2(o_na.reshape(B * T, *o_na.shape[2:]), o_r)
    es = oracle.rel_l2(S_na, S_r)
    print(f"[no-alloc] {label}: equal to gdn2_chunk_fwd; rel_l2 o={eo:.3e} S_T={es:.3e}",
          flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_static_workspace_two_calls_second_smaller():
    # 1: bf16, B=1, T=4096, 16 heads, d=128 (about 82 MB of workspace)
    x1 = inputs.chunk_inputs(inputs.CHUNK_BF16_T4096, seed=1002)
    check(x1, torch.bfloat16, "bf16 B=1 T=4096 H=16 d=128")
    # 2: a smaller packed fp32 batch over the same array
    wl = inputs.small_chunk(dtype=torch.float32, h_k=1, h_v=2, d_k=64, d_v=64, num_seqs=3,
                            len_lo=1, len_hi=200, s0_std=0.1)
    x2 = inputs.chunk_inputs(wl, seed=99)
    check(x2, torch.float32, "fp32 packed 3 seqs, 2 heads, d=64")


def test_static_workspace_generic_path():
    """The generic path over the static array: 128-token chunks (segmented panel passes),
    then fp32 at d = 128, each smaller than the call before it."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=2000, h_k=2, h_v=4, d_k=128,
                            d_v=128, neg_eig=True)
    check(inputs.chunk_inputs(wl, seed=1003), torch.bfloat16, "bf16 chunk 128 B=1 T=2000 H=4",
          chunk_size=128)
    wl = inputs.small_chunk(dtype=torch.float32, batch=1, seqlen=700, h_k=1, h_v=2, d_k=128,
                            d_v=128, neg_eig=True)
    check(inputs.chunk_inputs(wl, seed=1004), torch.float32, "fp32 d=128 B=1 T=700 H=2")


def test_static_workspace_refuses_oversized_calls():
    x = inputs.chunk_inputs(inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=8192,
                                               h_k=16, h_v=16, d_k=128, d_v=128), seed=3)
    d = to_gpu(x)
    with pytest.raises(g.GDN2Error) as e:
        g.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    assert e.value.status == 4
