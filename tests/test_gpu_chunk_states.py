"""GPU parity of the chunk-boundary states (gdn2_fusion.chunk_states of gdn2_chunk_fwd): the
state entering every chunk, against the oracle's recurrence stopped at every whole multiple
of the chunk size (oracle.chunk_states), on dense, packed (with empty and one-token
sequences), many-pair and segmented workloads. Writing them must leave o and S_T bit for bit
as they are without them.

Gate: relative L2 per chunk row (all heads of one chunk), 1e-4 for fp32 inputs and 2e-2 for
bf16 inputs; the first chunk of every sequence holds S0 exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import ORACLE_THREADS, TOL, flat_inputs, np64, to_gpu

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


def packed_case():
    wl = inputs.small_chunk(dtype=torch.bfloat16, h_k=2, h_v=4, d_k=128, d_v=128, num_seqs=6,
                            len_lo=2, len_hi=200, neg_eig=True)
    x = inputs.chunk_inputs(wl, seed=41)
    cu = x["cu_seqlens"].clone()
    lens = (cu[1:] - cu[:-1]).tolist()
    lens[1], lens[3] = 0, 1                   # an empty and a one-token sequence
    cu[1:] = torch.cumsum(torch.tensor(lens), 0).to(torch.int32)
    T = int(cu[-1])
    for n in ("q", "k", "v", "log_alpha", "b", "w"):
        x[n] = x[n][:, :T].contiguous()
    x["cu_seqlens"] = cu
    return x


CASES = {
    "dense fp32 64x64 ragged": lambda: inputs.chunk_inputs(
        inputs.small_chunk(dtype=torch.float32, batch=2, seqlen=150, h_k=2, h_v=4), seed=42),
    "dense bf16 128x128 GVA ragged": lambda: inputs.chunk_inputs(
        inputs.small_chunk(dtype=torch.bfloat16, batch=2, seqlen=150, h_k=2, h_v=4, d_k=128,
                           d_v=128, neg_eig=True), seed=43),
    "packed bf16 with empty and one-token sequences": packed_case,
    "many pairs bf16 128x64": lambda: inputs.chunk_inputs(
        inputs.small_chunk(dtype=torch.bfloat16, batch=3, seqlen=150, h_k=16, h_v=48, d_k=128,
                           d_v=64, neg_eig=True), seed=44),
    "segmented bf16 B=1 T=4096 H=16 d=128": lambda: inputs.chunk_inputs(
        inputs.CHUNK_BF16_T4096, seed=45),
}


@pytest.mark.parametrize("label", list(CASES))
def test_chunk_states_match_the_oracle(label):
    x = CASES[label]()
    dtype = x["q"].dtype
    d = to_gpu(x)
    B, T = x["q"].shape[:2]
    Hv, dk, dv = x["v"].shape[2], x["k"].shape[3], x["v"].shape[3]
    cu = x["cu_seqlens"]
    nc = g.num_chunks(T if cu is None else cu, B)
    print(f"[case] chunk_states {label}: {nc} chunks x {Hv} heads", flush=True)
    ck = torch.full((nc, Hv, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    kw = dict(S0=d["S0"], cu_seqlens=d["cu_seqlens"])
    o1, S1 = g.chunk_fwd(*args, chunk_states=ck, **kw)
    o2, S2 = g.chunk_fwd(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    f, cu_np, S0 = flat_inputs(x)
    ref = oracle.chunk_states(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], S0=S0,
                              cu_seqlens=cu_np, threads=ORACLE_THREADS)
    got = np64(ck)
    assert got.shape == ref.shape and np.all(np.isfinite(got))
    errs = [oracle.rel_l2(got[r], ref[r]) for r in range(nc)]
    print(f"[parity] chunk_states {label}: max row rel_l2 {max(errs):.3e} "
          f"(rows {nc}, tol {TOL[dtype]:g})", flush=True)
    assert max(errs) <= TOL[dtype]
    # the first chunk of every non-empty sequence holds S0 itself
    lens = np.diff(cu_np)
    first = np.concatenate([[0], np.cumsum((lens + 63) // 64)])[:-1]
    for n in np.nonzero(lens)[0]:
        assert np.array_equal(got[first[n]], np64(x["S0"][n]))


def test_chunk_states_resume_each_sequence():
    """Resuming the chunked forward from a stored chunk state over the rest of the sequence
    gives the same final state and outputs as the one whole call (within the bf16 gate)."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=320, h_k=2, h_v=4, d_k=128,
                            d_v=128, neg_eig=True)
    x = to_gpu(inputs.chunk_inputs(wl, seed=46))
    args = [x[n] for n in ("q", "k", "v", "log_alpha", "b", "w")]
    ck = torch.empty(5, 4, 128, 128, dtype=torch.float32, device="cuda")
    o, S_T = g.chunk_fwd(*args, S0=x["S0"], chunk_states=ck)
    j = 3                                       # resume at token 192
    tail = [t[:, 64 * j:].contiguous() for t in args]
    o2, S2 = g.chunk_fwd(*tail, S0=ck[j:j + 1].contiguous())
    torch.cuda.synchronize()
    eo = oracle.rel_l2(np64(o2), np64(o[:, 64 * j:]))
    es = oracle.rel_l2(np64(S2), np64(S_T))
    print(f"[parity] resume from chunk state {j}: o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= 1e-5 and es <= 1e-5
