"""GPU parity of the chunked forward at chunk sizes 32 and 128 and of the fp32 forward at
d = 128, through the C ABI against the fp64 oracle.

The chunk size is a parameter of the chunked WY form (burn-gdn2 docs page, "Architecture"
and its Configuration table); the result does not depend on it, so every case is checked
against the same token-by-token oracle: 1e-4 relative L2 for fp32 inputs, 2e-2 for bf16,
on o and on the final states. Tails straddle every chunk boundary and a multi-chunk ragged
length; packed batches carry an empty and a one-token sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import TOL, assert_chunk_parity, flat_inputs, gpu_chunk, np64, to_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


DIMS = [(torch.bfloat16, 128, 128), (torch.bfloat16, 64, 128), (torch.bfloat16, 128, 64),
        (torch.bfloat16, 64, 64), (torch.float32, 64, 64), (torch.float32, 128, 128),
        (torch.float32, 64, 128), (torch.float32, 128, 64)]


@pytest.mark.parametrize("C", [32, 128])
@pytest.mark.parametrize("dtype,dk,dv", DIMS)
@pytest.mark.parametrize("T", [1, 31, 32, 33, 127, 128, 129, 300])
def test_chunk_sizes_tails_gva(C, dtype, dk, dv, T):
    wl = inputs.small_chunk(dtype=dtype, batch=2, seqlen=T, h_k=1, h_v=3, d_k=dk, d_v=dv,
                            neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=T + C)
    assert_chunk_parity(x, dtype, label=f"C={C} {dtype} {dk}x{dv} T={T}", chunk_size=C)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_fp32_d128_chunk64_tails(dk, dv, T):
    wl = inputs.small_chunk(dtype=torch.float32, batch=2, seqlen=T, h_k=1, h_v=3, d_k=dk, d_v=dv,
                            neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=T + dk + dv)
    assert_chunk_parity(x, torch.float32, label=f"fp32 C=64 {dk}x{dv} T={T}")


def test_fp32_b1_t4096_h16_d128():
    """The timed bf16 workload's shape in fp32 (B=1, T=4096, 16 heads, d=128, random S0,
    negative eigenvalues): every output against the oracle at 1e-4."""
    x = inputs.chunk_inputs(inputs.with_dtype(inputs.CHUNK_BF16_T4096, torch.float32), seed=1012)
    assert_chunk_parity(x, torch.float32, label="fp32 B1 T4096 H16 d128", worst=True)


@pytest.mark.parametrize("C,dtype,dk,dv,T", [
    (32, torch.bfloat16, 128, 128, 1000),   # 32 chunks over 2 pairs -> 8 segments of 4
    (128, torch.bfloat16, 128, 64, 2000),   # 16 chunks -> 4 segments
    (64, torch.float32, 128, 128, 1500),    # 24 chunks -> 6 segments
    (32, torch.float32, 64, 64, 700),       # 22 chunks -> 5 segments, a ragged last one
])
def test_segmented_panel_pass(C, dtype, dk, dv, T):
    """Dense batches with two (sequence, head) pairs: the panel state pass is cut into many
    segments, so most segment starts are carried over several transitions (random S0,
    ragged tail)."""
    wl = inputs.small_chunk(dtype=dtype, batch=1, seqlen=T, h_k=2, h_v=2, d_k=dk, d_v=dv,
                            neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=T + C + dk)
    assert_chunk_parity(x, dtype, label=f"segmented C={C} {dtype} {dk}x{dv} T={T}", chunk_size=C)


@pytest.mark.parametrize("C", [32, 128])
def test_bf16_b1_t4096_h16_d128_chunk_sizes(C):
    """The timed workload (bf16, B=1, T=4096, 16 heads, d=128, random S0, negative
    eigenvalues) at chunk sizes 32 and 128."""
    x = inputs.chunk_inputs(inputs.CHUNK_BF16_T4096, seed=1002)
    assert_chunk_parity(x, torch.bfloat16, label=f"bf16 B1 T4096 H16 d128 C={C}", chunk_size=C,
                        worst=True)


@pytest.mark.parametrize("C", [32, 128])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_sizes_packed_with_empty_and_short(C, dtype):
    wl = inputs.small_chunk(dtype=dtype, h_k=2, h_v=4, d_k=128, d_v=64, num_seqs=6, len_lo=2,
                            len_hi=300)
    x = inputs.chunk_inputs(wl, seed=C + 5)
    cu = x["cu_seqlens"].clone()
    lens = (cu[1:] - cu[:-1]).tolist()
    lens[1] = 0
    lens[3] = 1
    cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
    T = int(cu[-1])
    for n in ("q", "k", "v", "log_alpha", "b", "w"):
        x[n] = x[n][:, :T].contiguous()
    x["cu_seqlens"] = cu
    assert_chunk_parity(x, dtype, label=f"packed C={C} {dtype} lens={lens}", chunk_size=C)
    _, S_g = gpu_chunk(x, chunk_size=C)
    assert np.array_equal(S_g[1], np64(x["S0"][1]))      # empty sequence: S_T = S0


@pytest.mark.parametrize("C", [32, 128])
def test_chunk_sizes_extreme_decay(C):
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=300, h_k=2, h_v=2, d_k=128,
                            d_v=128, neg_eig=True)
    x = inputs.chunk_inputs(wl, seed=5, decay_mu=3.0)
    assert_chunk_parity(x, torch.bfloat16, label=f"extreme decay C={C}", chunk_size=C)


def test_chunk_size_does_not_change_the_result():
    """C = 32, 64 and 128 on the same inputs agree with each other to the fp32 rounding of
    different summation orders, and S_T may alias S0 at every size."""
    wl = inputs.small_chunk(dtype=torch.float32, batch=2, seqlen=333, h_k=2, h_v=4, d_k=128,
                            d_v=128, neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=44)
    outs = {C: gpu_chunk(x, chunk_size=C) for C in (32, 64, 128)}
    for C in (32, 128):
        assert oracle.rel_l2(outs[C][0], outs[64][0]) < 2e-5
        assert oracle.rel_l2(outs[C][1], outs[64][1]) < 2e-5
    d = to_gpu(x)
    for C in (32, 128):
        S = d["S0"].clone()
        o, S_T = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=S,
                             final_state=S, chunk_size=C)
        torch.cuda.synchronize()
        assert S_T.data_ptr() == S.data_ptr()
        assert np.array_equal(np64(S), outs[C][1])


@pytest.mark.parametrize("C", [32, 128])
def test_chunk_states_at_chunk_sizes(C):
    """The state entering every chunk (rows per C-token chunk) against oracle.chunk_states."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, h_k=1, h_v=2, d_k=128, d_v=128, num_seqs=3,
                            len_lo=1, len_hi=400)
    x = inputs.chunk_inputs(wl, seed=C)
    d = to_gpu(x)
    nc = g.num_chunks(x["cu_seqlens"], 1, C)
    cks = torch.empty(nc, 2, 128, 128, dtype=torch.float32, device="cuda")
    g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                cu_seqlens=d["cu_seqlens"], chunk_size=C, chunk_states=cks)
    torch.cuda.synchronize()
    f, cu, S0 = flat_inputs(x)
    ref = oracle.chunk_states(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], S0=S0,
                              cu_seqlens=cu, chunk_size=C)
    err = max(oracle.rel_l2(np64(cks[r]), ref[r]) for r in range(nc) if np.any(ref[r]))
    print(f"[parity] chunk_states C={C}: max row rel_l2 {err:.3e} (rows {nc})", flush=True)
    assert err <= TOL[torch.bfloat16]


@pytest.mark.parametrize("C", [32, 128])
@pytest.mark.parametrize("mode", ["kda", "gdn", "fg2", "fg2+"])
def test_gate_modes_at_chunk_sizes(C, mode):
    """Native gate modes at chunk sizes 32 and 128 against the variant's own update rule."""
    x = inputs.variant_inputs(mode, torch.bfloat16, 2, 150, 1, 2, 128, 128, seed=C)
    d = {n: t.cuda() for n, t in x.items()}
    o, S_T = g.gated_chunk_fwd(mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               beta_v=d.get("beta_v"), S0=d["S"], chunk_size=C)
    torch.cuda.synchronize()
    f = {n: np64(t) for n, t in x.items()}
    o_r, S_r = oracle.variant(mode, f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], S0=f["S"],
                              beta_v=f.get("beta_v"))
    eo, es = oracle.rel_l2(np64(o), o_r), oracle.rel_l2(np64(S_T), S_r)
    print(f"[parity] gate mode {mode} C={C}: o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("C", [32, 128])
def test_fusions_at_chunk_sizes(C):
    """q/k L2-norm and the gated RMS output norm at chunk sizes 32 and 128, against the
    composed oracle stages."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=2, seqlen=200, h_k=1, h_v=2, d_k=128,
                            d_v=128, neg_eig=True, s0_std=0.1)
    x = inputs.chunk_inputs(wl, seed=C + 1)
    gen = torch.Generator().manual_seed(C)
    # un-normalised q and k: the kernels normalise them
    x["q"] = (x["q"].float() * 3.0).to(torch.bfloat16)
    x["k"] = (x["k"].float() * 0.5).to(torch.bfloat16)
    gate = torch.randn(x["v"].shape, generator=gen).to(torch.bfloat16)
    nw = torch.rand(128, generator=gen) + 0.5
    d = to_gpu(x)
    o, S_T = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                         chunk_size=C, qk_l2norm=True, l2norm_eps=1e-6, gate=gate.cuda(),
                         norm_weight=nw.cuda(), norm_eps=1e-5)
    torch.cuda.synchronize()
    f, cu, S0 = flat_inputs(x)
    qn = oracle.l2_normalize(f["q"], 1e-6)
    kn = oracle.l2_normalize(f["k"], 1e-6)
    o_r, S_r = oracle.recurrent(qn, kn, f["v"], f["log_alpha"], f["b"], f["w"], S0=S0,
                                cu_seqlens=cu)
    o_r = oracle.gated_rms_norm(o_r, np64(gate).reshape(o_r.shape), np64(nw), 1e-5)
    eo = oracle.rel_l2(np64(o).reshape(o_r.shape), o_r)
    es = oracle.rel_l2(np64(S_T), S_r)
    print(f"[parity] fusions C={C}: o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= 2e-2 and es <= 2e-2
