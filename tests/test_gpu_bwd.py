"""GPU parity of the chunked backward (gdn2_chunk_bwd) against the oracle's token-by-token
adjoint of the recurrence (oracle.recurrent_bwd), every gradient by relative L2: 1e-4 for
fp32 inputs, 2e-2 for bf16 inputs. Cases: ragged tails, grouped value heads (2 and 3 per
key head, and 4 over 32 pairs), every built head shape, packed batches with an empty
sequence, zero initial state and zero dS_T, the timed chunk shape (whose forward takes
the segmented state pass and whose reverse pass is segmented too), dense batches of few pairs
in 3 to 8 reverse segments (a ragged last segment, grouped heads); bit-equal repeated calls
when no value heads share a key head."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import ORACLE_THREADS, TOL, flat_inputs, np64, to_gpu

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dw", "dlog_alpha", "db")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


def run_case(x, label, seed, with_states=True, chunk_size=64):
    dtype = x["q"].dtype
    d = to_gpu(x)
    B, T = x["q"].shape[:2]
    Hv, dv = x["v"].shape[2], x["v"].shape[3]
    N = B if x["cu_seqlens"] is None else x["cu_seqlens"].numel() - 1
    gen = torch.Generator().manual_seed(seed)
    dO = torch.randn(B, T, Hv, dv, generator=gen).to(dtype)
    dST = torch.randn(N, Hv, x["k"].shape[3], dv, generator=gen) if with_states else None
    print(f"[case] chunk_bwd {label}", flush=True)
    got = g.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO.cuda(),
                      S0=d["S0"], cu_seqlens=d["cu_seqlens"],
                      dS_T=None if dST is None else dST.cuda(), chunk_size=chunk_size)
    torch.cuda.synchronize()
    f, cu, S0 = flat_inputs(x)
    ref = oracle.recurrent_bwd(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"],
                               np64(dO).reshape(B * T, Hv, dv), S0=S0,
                               dS_T=None if dST is None else np64(dST), cu_seqlens=cu,
                               threads=ORACLE_THREADS)
    errs = {}
    for n in GRADS:
        errs[n] = oracle.rel_l2(np64(got[n]).reshape(ref[n].shape), ref[n])
    errs["dS0"] = oracle.rel_l2(np64(got["dS0"]), ref["dS0"])
    print(f"[parity] chunk_bwd {label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()),
          flush=True)
    assert all(np.isfinite(list(errs.values())))
    assert max(errs.values()) <= TOL[dtype], errs
    return got


def test_bwd_fp32_gva_ragged():
    wl = inputs.small_chunk(dtype=torch.float32, batch=2, seqlen=150, h_k=2, h_v=4)
    run_case(inputs.chunk_inputs(wl, seed=61), "fp32 64x64 B=2 T=150 GVA", 1)


def test_bwd_bf16_128():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=200, h_k=1, h_v=2, d_k=128,
                            d_v=128, neg_eig=True)
    run_case(inputs.chunk_inputs(wl, seed=62), "bf16 128x128 B=1 T=200", 2)


def test_bwd_bf16_packed_with_empty_sequence():
    wl = inputs.small_chunk(dtype=torch.bfloat16, h_k=2, h_v=4, d_k=128, d_v=64, num_seqs=4,
                            len_lo=2, len_hi=150)
    x = inputs.chunk_inputs(wl, seed=63)
    cu = x["cu_seqlens"].clone()
    lens = (cu[1:] - cu[:-1]).tolist()
    lens[1] = 0
    cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
    T = int(cu[-1])
    for n in ("q", "k", "v", "log_alpha", "b", "w"):
        x[n] = x[n][:, :T].contiguous()
    x["cu_seqlens"] = cu
    run_case(x, f"bf16 128x64 packed lens={lens}", 3)


def test_bwd_zero_initial_state_and_no_final_gradient():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=2, seqlen=130, h_k=2, h_v=6, d_k=64,
                            d_v=128, s0_std=0.0)
    x = inputs.chunk_inputs(wl, seed=64)
    x["S0"] = None
    run_case(x, "bf16 64x128 G=3, S0 = 0, dS_T = 0", 4, with_states=False)


def test_bwd_bf16_64x64_many_chunks():
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=3, seqlen=700, h_k=2, h_v=2, d_k=64,
                            d_v=64, neg_eig=True)
    run_case(inputs.chunk_inputs(wl, seed=65), "bf16 64x64 B=3 T=700", 5)


def test_bwd_timed_chunk_shape():
    """B=1 T=4096 H=16 d=128 (64 chunks per pair; the forward that stores the chunk states
    takes the segmented state pass)."""
    run_case(inputs.chunk_inputs(inputs.CHUNK_BF16_T4096, seed=66), "bf16 B=1 T=4096 H=16", 6)


def test_bwd_grouped_heads_at_scale():
    """Four value heads per key head over 32 (sequence, value head) pairs of 16 chunks: the
    q and k gradients of each key head are summed with atomics from four records at once,
    and the forward takes the segmented state pass."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=2, seqlen=1000, h_k=4, h_v=16,
                            d_k=128, d_v=128, neg_eig=True)
    run_case(inputs.chunk_inputs(wl, seed=67), "bf16 B=2 T=1000 H_k=4 H_v=16", 7)


def test_bwd_is_deterministic_without_grouped_heads():
    """With one value head per key head no gradient is summed with atomics: two calls give
    the same bits."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=2, seqlen=300, h_k=3, h_v=3,
                            d_k=128, d_v=128, neg_eig=True)
    d = to_gpu(inputs.chunk_inputs(wl, seed=68))
    dO = torch.randn(2, 300, 3, 128, device="cuda").to(torch.bfloat16)
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO)
    first = g.chunk_bwd(*args, S0=d["S0"])
    second = g.chunk_bwd(*args, S0=d["S0"])
    torch.cuda.synchronize()
    for n in first:
        assert torch.equal(first[n], second[n]), n


def test_bwd_empty_batch_passes_the_final_gradient_through():
    """T = 0: no chunks, so dS0 = dS_T (and zero without it)."""
    q = torch.zeros(2, 0, 1, 64, device="cuda")
    v = torch.zeros(2, 0, 2, 64, device="cuda")
    la = torch.zeros(2, 0, 2, 64, device="cuda")
    dST = torch.randn(2, 2, 64, 64, device="cuda")
    got = g.chunk_bwd(q, q, v, la, la, v, v, dS_T=dST)
    none = g.chunk_bwd(q, q, v, la, la, v, v)
    torch.cuda.synchronize()
    assert torch.equal(got["dS0"], dST)
    assert torch.count_nonzero(none["dS0"]) == 0


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 128), (torch.float32, 64, 64)])
def test_bwd_extreme_decay(dtype, dk, dv):
    """log alpha = -softplus(N(3, 1)) per channel (about -3 per token, down to -8): the
    decay factors of a 64-token chunk span e^-200 and beyond, so any factor taken relative
    to a far reference would overflow; every gradient must stay finite and within the gate."""
    wl = inputs.small_chunk(dtype=dtype, batch=1, seqlen=300, h_k=2, h_v=2, d_k=dk, d_v=dv,
                            neg_eig=True, s0_std=0.1)
    run_case(inputs.chunk_inputs(wl, seed=65, decay_mu=3.0), f"extreme decay {dtype} {dk}x{dv}", 9)


@pytest.mark.parametrize("batch,seqlen,h_k,h_v,dk,dv,label", [
    (1, 1300, 1, 2, 128, 128, "5 segments of 5 chunks, the last one a single ragged chunk"),
    (2, 900, 1, 2, 64, 64, "3 segments of 5 chunks"),
    (1, 2000, 2, 4, 128, 64, "8 segments of 4 chunks, two value heads per key head"),
    (1, 1000, 1, 2, 64, 128, "4 segments of 4 chunks"),
])
def test_bwd_segmented_reverse_pass(batch, seqlen, h_k, h_v, dk, dv, label):
    """Dense batches with few (sequence, value head) pairs take the segmented reverse pass:
    the segment pass forms, per later segment, the gradient transition and the zero-start
    result, and every segment's reverse chain starts from the carried gradient."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=batch, seqlen=seqlen, h_k=h_k, h_v=h_v,
                            d_k=dk, d_v=dv, neg_eig=True)
    run_case(inputs.chunk_inputs(wl, seed=80 + seqlen % 17), f"bf16 {dk}x{dv} B={batch} "
             f"T={seqlen} H_k={h_k} H_v={h_v}: {label}", 9)


def test_bwd_segmented_without_initial_state_or_final_gradient():
    """The segmented reverse pass (4 segments) with S0 = 0 and dS_T = 0: the last segment's
    chain starts from zero in both the segment pass and the pass over every segment."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=1000, h_k=1, h_v=2, d_k=128,
                            d_v=128, neg_eig=True, s0_std=0.0)
    x = inputs.chunk_inputs(wl, seed=97)
    x["S0"] = None
    run_case(x, "bf16 128x128 T=1000, 4 reverse segments, S0 = 0, dS_T = 0", 12,
             with_states=False)


@pytest.mark.parametrize("dk,dv,h_k,h_v,seqlen", [(128, 128, 1, 2, 200), (128, 64, 1, 2, 150),
                                                  (64, 128, 2, 4, 130)])
def test_bwd_fp32_every_head_dim_pair(dk, dv, h_k, h_v, seqlen):
    """fp32 inputs at d = 128 and at the mixed head dims (fp32 products throughout), ragged
    tails and grouped value heads, at the fp32 bar."""
    wl = inputs.small_chunk(dtype=torch.float32, batch=2, seqlen=seqlen, h_k=h_k, h_v=h_v,
                            d_k=dk, d_v=dv, neg_eig=True)
    run_case(inputs.chunk_inputs(wl, seed=90 + dk // 64 + dv // 32), f"fp32 {dk}x{dv} B=2 "
             f"T={seqlen} H_k={h_k} H_v={h_v}", 10)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bwd_chunk_size_does_not_change_the_gradients(dtype):
    """chunk_size names the forward's chunking; the gradients do not depend on it. Calls at
    chunk sizes 32 and 128 match the oracle and give the bits of the chunk-64 call."""
    wl = inputs.small_chunk(dtype=dtype, batch=1, seqlen=300, h_k=2, h_v=2, d_k=128, d_v=128,
                            neg_eig=True)      # (no grouped heads: no atomics, the same bits)
    x = inputs.chunk_inputs(wl, seed=95)
    ref = run_case(x, f"{dtype} 128x128 T=300, chunk_size 64", 11)
    for cs in (32, 128):
        got = run_case(x, f"{dtype} 128x128 T=300, chunk_size {cs}", 11, chunk_size=cs)
        for n in ref:
            assert torch.equal(got[n], ref[n]), (cs, n)


@pytest.mark.parametrize("label,kw", [
    ("bf16 128x128 B=1 T=4096 H=16 (the timed shape, 4 segments)", dict(wl="t4096")),
    ("bf16 64x64 B=3 T=700", dict(dtype=torch.bfloat16, batch=3, seqlen=700, h_k=2, h_v=2, d_k=64, d_v=64)),
    ("bf16 128x64 packed with an empty sequence, G=2", dict(packed=True)),
    ("fp32 64x64 B=2 T=150 G=2 (states recomputed)", dict(dtype=torch.float32, batch=2, seqlen=150, h_k=2, h_v=4, d_k=64, d_v=64)),
])
def test_bwd_from_forward_states(label, kw):
    """gdn2_chunk_bwd_states with the chunk states a chunk-64 forward of the same inputs
    wrote: the same gradients as gdn2_chunk_bwd (the same bits without grouped heads, within
    the bars with them), and within the bars of the oracle's token adjoint."""
    kw = dict(kw)
    if kw.pop("wl", None) == "t4096":
        x = inputs.chunk_inputs(inputs.CHUNK_BF16_T4096, seed=71)
    elif kw.pop("packed", False):
        wl = inputs.small_chunk(dtype=torch.bfloat16, h_k=2, h_v=4, d_k=128, d_v=64, num_seqs=4,
                                len_lo=2, len_hi=200)
        x = inputs.chunk_inputs(wl, seed=72)
        cu = x["cu_seqlens"].clone()
        lens = (cu[1:] - cu[:-1]).tolist()
        lens[2] = 0
        cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
        T = int(cu[-1])
        for n in ("q", "k", "v", "log_alpha", "b", "w"):
            x[n] = x[n][:, :T].contiguous()
        x["cu_seqlens"] = cu
    else:
        x = inputs.chunk_inputs(inputs.small_chunk(neg_eig=True, **kw), seed=73)
    d = to_gpu(x)
    dtype = x["q"].dtype
    B, T = x["q"].shape[:2]
    Hv, dv, dk = x["v"].shape[2], x["v"].shape[3], x["k"].shape[3]
    N = B if x["cu_seqlens"] is None else x["cu_seqlens"].numel() - 1
    gen = torch.Generator().manual_seed(74)
    dO = torch.randn(B, T, Hv, dv, generator=gen).to(dtype).cuda()
    dST = torch.randn(N, Hv, dk, dv, generator=gen).cuda()
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    nc = g.num_chunks(T if d["cu_seqlens"] is None else x["cu_seqlens"], B)
    ck = torch.empty(nc, Hv, dk, dv, dtype=torch.float32, device="cuda")
    print(f"[case] chunk_bwd_states {label}", flush=True)
    g.chunk_fwd(*args, S0=d["S0"], cu_seqlens=d["cu_seqlens"], chunk_states=ck)
    ref = g.chunk_bwd(*args, dO, S0=d["S0"], cu_seqlens=d["cu_seqlens"], dS_T=dST)
    got = g.chunk_bwd(*args, dO, S0=d["S0"], cu_seqlens=d["cu_seqlens"], dS_T=dST, chunk_states=ck)
    torch.cuda.synchronize()
    grouped = x["q"].shape[2] != Hv
    for n in ref:
        if grouped:
            e = oracle.rel_l2(np64(got[n]), np64(ref[n]))
            assert e <= 1e-5, (n, e)
        else:
            assert torch.equal(got[n], ref[n]), n
    if T <= 1000:
        f, cu, S0 = flat_inputs(x)
        o_ref = oracle.recurrent_bwd(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"],
                                     np64(dO).reshape(B * T, Hv, dv), S0=S0, dS_T=np64(dST),
                                     cu_seqlens=cu, threads=ORACLE_THREADS)
        errs = {n: oracle.rel_l2(np64(got[n]).reshape(o_ref[n].shape), o_ref[n]) for n in GRADS}
        errs["dS0"] = oracle.rel_l2(np64(got["dS0"]), o_ref["dS0"])
        print(f"[parity] chunk_bwd_states {label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()),
              flush=True)
        assert max(errs.values()) <= TOL[dtype], errs
    else:
        print(f"[parity] chunk_bwd_states {label}: equal to gdn2_chunk_bwd", flush=True)
