"""GPU parity: the HIP path through the C ABI against the fp64 oracle on seeded inputs.

Gate (relative L2 error per output tensor): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs, on
o and on the final states. Every case compares every element of o and of the final states,
the full-size decode and varlen workloads included (the threaded fp64 oracle on the host's
cores); those two also report their worst single (sequence, head) pair.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import (ORACLE_THREADS, TOL, assert_chunk_parity, decode_oracle_pair,
                        flat_inputs, gpu_chunk, np64, oracle_chunk, to_gpu)

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


# ---------------------------------------------------------------- decode step -----------

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
def test_decode_small(dtype, dk, dv):
    wl = inputs.DecodeWorkload("decode_small", dtype, 3, 2, 6, dk, dv, steps=5)
    x = inputs.decode_inputs(wl, seed=11)
    S = x["S"].cuda()
    os_ = []
    for t in range(wl.steps):
        o = g.recurrent_step(x["q"][t].cuda(), x["k"][t].cuda(), x["v"][t].cuda(),
                             x["log_alpha"][t].cuda(), x["b"][t].cuda(), x["w"][t].cuda(), S)
        os_.append(np64(o))
    torch.cuda.synchronize()
    o_g = np.stack(os_)                      # [steps, N, Hv, dv]
    o_r = np.zeros_like(o_g)
    S_r = np.zeros((3, 6, dk, dv))
    for n in range(3):
        for h in range(6):
            on, Sn = decode_oracle_pair(x, n, h, wl.steps, 3)
            o_r[:, n, h] = on
            S_r[n, h] = Sn
    eo, es = oracle.rel_l2(o_g, o_r), oracle.rel_l2(np64(S), S_r)
    print(f"[parity] decode {dtype} {dk}x{dv} o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def decode_oracle_all(x, steps, h_v):
    """Every (sequence, value head) state of a decode workload over `steps` steps with the
    threaded fp64 oracle: the steps of sequence n are its tokens. Returns (o [steps, N, H_v,
    d_v], S [N, H_v, d_k, d_v])."""
    N = x["S"].shape[0]
    flat = {n: np64(x[n][:steps].transpose(0, 1)).reshape(N * steps, *x[n].shape[2:])
            for n in ("q", "k", "v", "log_alpha", "b", "w")}
    o, S = oracle.recurrent(flat["q"], flat["k"], flat["v"], flat["log_alpha"], flat["b"],
                            flat["w"], S0=np64(x["S"]), cu_seqlens=np.arange(N + 1) * steps,
                            threads=ORACLE_THREADS)
    return o.reshape(N, steps, h_v, -1).transpose(1, 0, 2, 3), S


def worst_pair(o_g, o_r, S_g, S_r):
    """Largest per-(sequence, head) relative L2 error of o (over all steps) and of S."""
    N, H = S_g.shape[:2]
    wo = max(oracle.rel_l2(o_g[:, n, h], o_r[:, n, h]) for n in range(N) for h in range(H))
    ws = max(oracle.rel_l2(S_g[n, h], S_r[n, h]) for n in range(N) for h in range(H))
    return wo, ws


def test_decode_full_size_256_steps():
    """64 sequences, 48 value heads over 16 key heads, d=128, fp32 state, 256 steps in place;
    every output of every step and every state after the last step against the oracle."""
    wl = inputs.DECODE_F32
    x = inputs.decode_inputs(wl, seed=3)
    dev = {n: x[n].cuda() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    S = x["S"].cuda()
    o_all = torch.empty(wl.steps, wl.num_seqs, wl.h_v, wl.d_v, device="cuda")
    for t in range(wl.steps):
        g.recurrent_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["log_alpha"][t],
                         dev["b"][t], dev["w"][t], S, out=o_all[t])
    torch.cuda.synchronize()
    o_g = np64(o_all)
    S_g = np64(S)
    assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(S_g))
    o_r, S_r = decode_oracle_all(x, wl.steps, wl.h_v)
    eo, es = oracle.rel_l2(o_g, o_r), oracle.rel_l2(S_g, S_r)
    wo, ws = worst_pair(o_g, o_r, S_g, S_r)
    print(f"[parity] decode full 256 steps, all {wl.num_seqs * wl.h_v} states: o={eo:.2e} "
          f"S={es:.2e}; worst state o={wo:.2e} S={ws:.2e}", flush=True)
    assert eo <= 1e-4 and es <= 1e-4


def test_decode_state_larger_than_last_level_cache():
    """128 sequences x 48 heads (403 MB of state, above 256 MiB: streamed with non-temporal
    stores), 4 steps in place, every state against the oracle."""
    wl = replace(inputs.DECODE_F32, num_seqs=128, steps=4)
    x = inputs.decode_inputs(wl, seed=13)
    dev = {n: x[n].cuda() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    S = x["S"].cuda()
    o_all = torch.empty(wl.steps, wl.num_seqs, wl.h_v, wl.d_v, device="cuda")
    for t in range(wl.steps):
        g.recurrent_step(dev["q"][t], dev["k"][t], dev["v"][t], dev["log_alpha"][t],
                         dev["b"][t], dev["w"][t], S, out=o_all[t])
    torch.cuda.synchronize()
    o_g, S_g = np64(o_all), np64(S)
    o_r, S_r = decode_oracle_all(x, wl.steps, wl.h_v)
    eo, es = oracle.rel_l2(o_g, o_r), oracle.rel_l2(S_g, S_r)
    wo, ws = worst_pair(o_g, o_r, S_g, S_r)
    print(f"[parity] decode 128 seqs (streamed state), all states: o={eo:.2e} S={es:.2e}; "
          f"worst state o={wo:.2e} S={ws:.2e}", flush=True)
    assert eo <= 1e-4 and es <= 1e-4


# ---------------------------------------------------------------- chunk forward ---------

def test_chunk_f32_b1_t256_h4_d64():
    x = inputs.chunk_inputs(inputs.CHUNK_F32_SMALL, seed=1000)
    assert_chunk_parity(x, torch.float32, label="chunk f32 B1 T256 H4 d64")


def test_chunk_bf16_b8_t2048_h8_d128():
    x = inputs.chunk_inputs(inputs.CHUNK_BF16_B8, seed=1001)
    assert_chunk_parity(x, torch.bfloat16, label="chunk bf16 B8 T2048 H8 d128")


def test_chunk_bf16_b1_t4096_h16_d128_negeig():
    x = inputs.chunk_inputs(inputs.CHUNK_BF16_T4096, seed=1002)
    assert_chunk_parity(x, torch.bfloat16, label="chunk bf16 B1 T4096 H16 d128 neg-eig S0")


def test_varlen_bf16_n16_hv32_hk16_d128():
    """16 packed sequences, 32 value heads over 16 key heads: all 512 (sequence, head) pairs
    against the oracle, with the worst pair reported."""
    x = inputs.chunk_inputs(inputs.VARLEN_BF16, seed=1004)
    print("[parity] varlen tokens:", int(x["cu_seqlens"][-1]), flush=True)
    eo, es = assert_chunk_parity(x, torch.bfloat16, label="varlen bf16 16 seqs (all 512 pairs)",
                                 worst=True)


@pytest.mark.parametrize("dtype,dk,dv", [(torch.float32, 64, 64), (torch.bfloat16, 128, 128),
                                         (torch.bfloat16, 64, 128), (torch.bfloat16, 128, 64),
                                         (torch.bfloat16, 64, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_chunk_tails_gva_and_state(dtype, dk, dv, T):
    wl = inputs.small_chunk(dtype=dtype, batch=2, seqlen=T, h_k=1, h_v=3, d_k=dk, d_v=dv,
                            neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=T)
    assert_chunk_parity(x, dtype, label=f"tail {dtype} {dk}x{dv} T={T}")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_packed_with_empty_and_short_sequences(dtype):
    wl = inputs.small_chunk(dtype=dtype, h_k=2, h_v=4, d_k=64, d_v=64, num_seqs=6, len_lo=2,
                            len_hi=150)
    x = inputs.chunk_inputs(wl, seed=21)
    cu = x["cu_seqlens"].clone()
    lens = (cu[1:] - cu[:-1]).tolist()
    lens[2] = 0                               # force an empty sequence and a 1-token one
    lens[4] = 1
    cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
    T = int(cu[-1])
    for n in ("q", "k", "v", "log_alpha", "b", "w"):
        x[n] = x[n][:, :T].contiguous()
    x["cu_seqlens"] = cu
    assert_chunk_parity(x, dtype, label=f"packed {dtype} lens={lens}")
    _, S_g = gpu_chunk(x)
    assert np.array_equal(S_g[2], np64(x["S0"][2]))      # empty sequence: S_T = S0


# Packed batches are taken longest first by the state passes (the chunk-map kernel ranks up
# to 256 sequences by chunk count; more keep their own order): 200 sequences with many equal
# chunk counts (ranked, ties by index) and 300 (not ranked), empty ones included, at every
# chunk size (64: the 64-token state pass; 32 and 128: the panel state pass).
@pytest.mark.parametrize("num_seqs", [200, 300])
@pytest.mark.parametrize("C", [32, 64, 128])
def test_packed_many_sequences_state_order(num_seqs, C):
    wl = inputs.small_chunk(dtype=torch.bfloat16, h_k=1, h_v=2, d_k=64, d_v=64,
                            num_seqs=num_seqs, len_lo=1, len_hi=200)
    x = inputs.chunk_inputs(wl, seed=30 + num_seqs)
    cu = x["cu_seqlens"].clone()
    lens = (cu[1:] - cu[:-1]).tolist()
    for n in range(0, num_seqs, 37):
        lens[n] = 0                               # empty sequences among them
    cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
    T = int(cu[-1])
    for n in ("q", "k", "v", "log_alpha", "b", "w"):
        x[n] = x[n][:, :T].contiguous()
    x["cu_seqlens"] = cu
    assert_chunk_parity(x, torch.bfloat16, label=f"packed {num_seqs} sequences C={C}",
                        worst=True, chunk_size=C)
    _, S_g = gpu_chunk(x, chunk_size=C)
    for n in range(0, num_seqs, 37):
        assert np.array_equal(S_g[n], np64(x["S0"][n]))   # empty sequence: S_T = S0


# With grouped heads the prep kernel maps blocks to records so that the G value heads of a
# key head run back to back on one XCD, when the record count is a multiple of 8 G: shapes
# chosen so that it is (G = 2, 3, 4), against the oracle on every pair.
@pytest.mark.parametrize("G,T", [(2, 256), (3, 512), (4, 128)])
def test_grouped_heads_record_mapping(G, T):
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=2, seqlen=T, h_k=2, h_v=2 * G, d_k=128,
                            d_v=128, neg_eig=True)
    assert (2 * ((T + 63) // 64) * 2 * G) % (8 * G) == 0
    x = inputs.chunk_inputs(wl, seed=40 + G)
    assert_chunk_parity(x, torch.bfloat16, label=f"grouped heads G={G} T={T}", worst=True)


def test_chunk_extreme_decay_stress():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=300, h_k=2, h_v=2, d_k=128,
                            d_v=128, neg_eig=True)
    x = inputs.chunk_inputs(wl, seed=5, decay_mu=3.0)
    assert_chunk_parity(x, torch.bfloat16, label="extreme decay (log alpha ~ -softplus(N(3,1)))")


def test_chunk_zero_initial_state_and_no_final_state():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=100, h_k=1, h_v=1, d_k=128,
                            d_v=128, s0_std=None)
    x = inputs.chunk_inputs(wl, seed=8)
    o_full, _ = gpu_chunk(x)
    o_only, S_none = gpu_chunk(x, output_final_state=False)
    assert S_none is None
    assert np.array_equal(o_full, o_only)
    o_r, _ = oracle_chunk(x)
    assert oracle.rel_l2(o_only, o_r) <= 2e-2


# Dense batches with few (sequence, head) pairs take the segmented state pass: the chunks
# of each pair are split into segments that run concurrently (segment transitions, then
# every segment from its start state, which segments after the second carry over the
# transitions before them). These shapes give 4, 2, 4 and 8 segments (the workspace size
# test on the CPU pins that plan).
SEGMENTED = [
    (torch.bfloat16, 128, 128, 1, 1000, 1, 2, 0.1),
    (torch.bfloat16, 128, 128, 2, 640, 1, 3, 0.1),
    (torch.float32, 64, 64, 1, 1024, 1, 1, 0.1),
    (torch.bfloat16, 128, 64, 1, 2000, 2, 2, None),
]


@pytest.mark.parametrize("dtype,dk,dv,B,T,hk,hv,s0", SEGMENTED)
def test_segmented_state_pass(dtype, dk, dv, B, T, hk, hv, s0):
    wl = inputs.small_chunk(dtype=dtype, batch=B, seqlen=T, h_k=hk, h_v=hv, d_k=dk, d_v=dv,
                            neg_eig=True, s0_std=s0)
    x = inputs.chunk_inputs(wl, seed=T + hv)
    assert_chunk_parity(x, dtype, label=f"segmented {dtype} {dk}x{dv} B={B} T={T} hv={hv}")


def test_segmented_final_state_may_alias_initial_state():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=1000, h_k=1, h_v=2, d_k=128,
                            d_v=128, neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=77)
    o_ref, S_ref = gpu_chunk(x)
    d = to_gpu(x)
    S = d["S0"].clone()
    o, S_T = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=S,
                         final_state=S)
    torch.cuda.synchronize()
    assert S_T.data_ptr() == S.data_ptr()
    assert np.array_equal(np64(S), S_ref)
    assert np.array_equal(np64(o).reshape(o_ref.shape), o_ref)


# Many (sequence, head) pairs: the state pass uses four-column-slice workgroups.
@pytest.mark.parametrize("dk,dv,B,T,hk,hv", [(128, 128, 4, 200, 8, 32), (128, 64, 3, 150, 16, 48)])
def test_many_pairs_wide_state_workgroups(dk, dv, B, T, hk, hv):
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=B, seqlen=T, h_k=hk, h_v=hv, d_k=dk,
                            d_v=dv, neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=B * T + hv)
    assert_chunk_parity(x, torch.bfloat16, label=f"many pairs {dk}x{dv} B={B} T={T} hv={hv}")
