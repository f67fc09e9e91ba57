"""GPU parity of the delta-rule variants (KDA, scalar-decay GDN, FG2-GDN, FG2-GDN+) against
the oracle's direct update rules of those variants (oracle.variant), run two ways: natively
(gdn2_fusion.gate_mode: the chunked and recurrent kernels read beta themselves) and mapped
(gdn2_map_gates writes GDN-2 inputs, then the plain GDN-2 call).

Gate (relative L2 per output tensor): 1e-4 for fp32 inputs, 2e-2 for bf16 inputs, on o and
on the final states. In bf16 the mapped keys and values of the FG2 modes are rounded to
bf16 once more; the error this adds is far inside the gate.
"""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs
from gpu_common import TOL, np64

pytestmark = pytest.mark.gpu

MODES = ["kda", "gdn", "fg2", "fg2+"]


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


def oracle_run(mode, x):
    f = {n: np64(t) for n, t in x.items()}
    return oracle.variant(mode, f["q"], f["k"], f["v"], f["log_alpha"], f["beta"], S0=f["S"],
                          beta_v=f.get("beta_v"))


def shapes(dtype, mode):
    if dtype == torch.float32:
        return 64, 64                     # fp32: the 64-token path of d_k = d_v = 64
    return (128, 128) if mode == "fg2" else (128, 64)


@pytest.mark.parametrize("mapped", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
def test_chunk_forward_of_variants(mode, dtype, mapped):
    dk, dv = shapes(dtype, mode)
    x = inputs.variant_inputs(mode, dtype, 2, 150, 2, 4, dk, dv, seed=80 + MODES.index(mode))
    d = {n: t.cuda() for n, t in x.items()}
    o, S_T = g.gated_chunk_fwd(mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               beta_v=d.get("beta_v"), mapped=mapped, S0=d["S"])
    torch.cuda.synchronize()
    o_r, S_r = oracle_run(mode, x)
    eo, es = oracle.rel_l2(np64(o), o_r), oracle.rel_l2(np64(S_T), S_r)
    how = "mapped" if mapped else "native"
    print(f"[parity] chunk {mode} {how} {dtype} {dk}x{dv}: o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("mapped", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
def test_recurrent_forward_of_variants(mode, dtype, mapped):
    dk, dv = (128, 128) if mode == "fg2" else (128, 64)
    x = inputs.variant_inputs(mode, dtype, 3, 5, 2, 6, dk, dv, seed=90 + MODES.index(mode))
    d = {n: t.cuda() for n, t in x.items()}
    state = d["S"].clone()
    o = g.gated_recurrent_fwd(mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], state,
                              beta_v=d.get("beta_v"), mapped=mapped)
    torch.cuda.synchronize()
    o_r, S_r = oracle_run(mode, x)
    eo, es = oracle.rel_l2(np64(o), o_r), oracle.rel_l2(np64(state), S_r)
    how = "mapped" if mapped else "native"
    print(f"[parity] recurrent {mode} {how} {dtype} {dk}x{dv}: o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_mapped_inputs_are_the_gdn2_form():
    """The mapping itself, element by element: KDA broadcasts beta into b and w; FG2+ scales
    the keys by sqrt(beta) per value head and puts sqrt(beta_v) in w (fp32: exact up to the
    rounding of the square root and one product)."""
    x = inputs.variant_inputs("fg2+", torch.float32, 2, 7, 2, 4, 64, 128, seed=7)
    d = {n: t.cuda() for n, t in x.items()}
    q2, k2, v2, la2, b, w = g.map_gates("fg2+", d["q"], d["k"], d["v"], d["log_alpha"],
                                        d["beta"], d["beta_v"])
    torch.cuda.synchronize()
    G = 2
    kq = np64(x["k"]).repeat(G, axis=2)
    assert np.allclose(np64(k2), np.sqrt(np64(x["beta"])) * kq, rtol=1e-6, atol=0)
    assert np.array_equal(np64(q2), np64(x["q"]).repeat(G, axis=2))
    assert np.all(np64(b) == 1.0)
    assert np.allclose(np64(w), np.sqrt(np64(x["beta_v"])), rtol=1e-6, atol=0)
    assert v2.data_ptr() == d["v"].data_ptr() and la2.data_ptr() == d["log_alpha"].data_ptr()
    y = inputs.variant_inputs("kda", torch.bfloat16, 1, 9, 1, 3, 128, 64, seed=8)
    e = {n: t.cuda() for n, t in y.items()}
    _, _, _, _, b, w = g.map_gates("kda", e["q"], e["k"], e["v"], e["log_alpha"], e["beta"])
    torch.cuda.synchronize()
    beta = np64(y["beta"])
    assert np.array_equal(np64(b), np.broadcast_to(beta[..., None], b.shape))
    assert np.array_equal(np64(w), np.broadcast_to(beta[..., None], w.shape))


def test_fg2_rejects_unequal_head_dims_and_fused_key_stages():
    x = inputs.variant_inputs("fg2", torch.bfloat16, 1, 4, 1, 1, 128, 64, seed=9)
    d = {n: t.cuda() for n, t in x.items()}
    with pytest.raises(g.GDN2Error):
        g.map_gates("fg2", d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    with pytest.raises(ValueError):
        g.gated_chunk_fwd("fg2", d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    with pytest.raises(ValueError):
        g.gated_chunk_fwd("fg2+", d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                          beta_v=torch.ones_like(d["v"]), qk_l2norm=True)


def test_native_kda_with_fused_norms_and_multi_token_slots():
    """KDA natively with the q/k L2-norm and the gated output norm on, through the slot
    cache (padding entry included): equals the same run on GDN-2 inputs (b = w = beta)."""
    x = inputs.variant_inputs("kda", torch.bfloat16, 3, 4, 2, 6, 128, 128, seed=10)
    d = {n: t.cuda() for n, t in x.items()}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    gate = torch.randn(3, 4, 6, 128, generator=gen, device="cuda").to(torch.bfloat16)
    nw = torch.rand(128, generator=gen, device="cuda") + 0.5
    idx = torch.tensor([2, -1, 0], dtype=torch.int32, device="cuda")
    kw = dict(state_idx=idx, qk_l2norm=True, gate=gate, norm_weight=nw)
    s1, s2 = d["S"].clone(), d["S"].clone()
    o1 = g.gated_recurrent_fwd("kda", d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], s1, **kw)
    b = d["beta"][..., None].expand(3, 4, 6, 128).contiguous()
    o2 = g.recurrent_fwd(d["q"], d["k"], d["v"], d["log_alpha"], b, b.clone(), s2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("mode", MODES)
def test_native_variants_at_the_timed_chunk_shape(mode):
    """Each variant natively at the timed chunk shape (bf16, T = 4096, 16 heads, d = 128),
    where the gate tensors are large enough that a read past them leaves their allocation.
    KDA and GDN read the same gate values natively as mapped (rel. L2 <= 1e-5); the FG2
    modes differ from the mapped run by the bf16 rounding of the mapped keys and values."""
    wl = inputs.CHUNK_BF16_T4096
    x = inputs.variant_inputs(mode, wl.dtype, 1, wl.seqlen, wl.h_k, wl.h_v, wl.d_k, wl.d_v,
                              seed=120 + MODES.index(mode))
    d = {n: t.cuda() for n, t in x.items()}
    print(f"[case] native {mode} at B=1 T={wl.seqlen} H={wl.h_v} d={wl.d_k}", flush=True)
    args = (mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    o_n, s_n = g.gated_chunk_fwd(*args, beta_v=d.get("beta_v"), S0=d["S"])
    o_m, s_m = g.gated_chunk_fwd(*args, beta_v=d.get("beta_v"), S0=d["S"], mapped=True)
    torch.cuda.synchronize()
    tol = 1e-5 if mode in ("kda", "gdn") else TOL[torch.bfloat16]
    eo, es = oracle.rel_l2(np64(o_n), np64(o_m)), oracle.rel_l2(np64(s_n), np64(s_m))
    print(f"[parity] native vs mapped {mode} full size: o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= tol and es <= tol
    assert torch.isfinite(o_n.float()).all()


@pytest.mark.parametrize("mode", MODES)
def test_native_variants_at_the_decode_shape(mode):
    """One decode step of each variant natively at the timed decode shape (64 sequences,
    16 key heads, 48 value heads, d = 128) against the mapped run (tolerances as above)."""
    dw = inputs.DECODE_F32
    x = inputs.variant_inputs(mode, dw.dtype, dw.num_seqs, 1, dw.h_k, dw.h_v, dw.d_k, dw.d_v,
                              seed=130 + MODES.index(mode))
    d = {n: t.cuda() for n, t in x.items()}
    print(f"[case] native {mode} decode N={dw.num_seqs} H_v={dw.h_v} d={dw.d_k}", flush=True)
    s_n, s_m = d["S"].clone(), d["S"].clone()
    args = (mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    o_n = g.gated_recurrent_fwd(*args, s_n, beta_v=d.get("beta_v"))
    o_m = g.gated_recurrent_fwd(*args, s_m, beta_v=d.get("beta_v"), mapped=True)
    torch.cuda.synchronize()
    tol = 1e-5 if mode in ("kda", "gdn") else TOL[torch.float32]
    eo, es = oracle.rel_l2(np64(o_n), np64(o_m)), oracle.rel_l2(np64(s_n), np64(s_m))
    print(f"[parity] native vs mapped {mode} decode: o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= tol and es <= tol


# ---- training the variants: the chain rule back through the mapping (gdn2_map_gates_bwd) ---

def _pair_args(mode, f, n, h, G):
    hk = h // G
    args = (f["q"][n, :, hk], f["k"][n, :, hk], f["v"][n, :, h], f["log_alpha"][n, :, h],
            f["beta"][n, :, h])
    return args, (f["beta_v"][n, :, h] if mode == "fg2+" else None)


def _assemble(mode, f, per_pair):
    """Per-pair gradients of the variant's inputs -> tensors in the inputs' shapes; q and k
    gradients of the value heads of a key head add up."""
    N, T, Hk, dk = f["k"].shape
    Hv = f["v"].shape[2]
    G = Hv // Hk
    out = {"dq": np.zeros(f["q"].shape), "dk": np.zeros(f["k"].shape),
           "dv": np.zeros(f["v"].shape), "dlog_alpha": np.zeros(f["log_alpha"].shape),
           "dbeta": np.zeros(f["beta"].shape)}
    if mode == "fg2+":
        out["dbeta_v"] = np.zeros(f["beta_v"].shape)
    for (n, h), r in per_pair.items():
        out["dq"][n, :, h // G] += r["dq"]
        out["dk"][n, :, h // G] += r["dk"]
        for name in ("dv", "dlog_alpha", "dbeta") + (("dbeta_v",) if mode == "fg2+" else ()):
            out[name][n, :, h] = r[name]
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
def test_map_gates_bwd_against_the_oracle_chain_rule(mode, dtype):
    """gdn2_map_gates_bwd on random gradients of the mapped inputs against
    oracle.map_gates_bwd per (sequence, value head) pair (fp32 arithmetic on both sides'
    inputs: relative L2 <= 1e-5 on every output)."""
    dk, dv = (128, 128) if mode == "fg2" else (128, 64)
    x = inputs.variant_inputs(mode, dtype, 2, 33, 2, 4, dk, dv, seed=110 + MODES.index(mode))
    d = {n: t.cuda() for n, t in x.items()}
    f = {n: np64(t) for n, t in x.items()}
    N, T, Hk = 2, 33, 2
    Hv = 4
    hq = Hv if mode in ("fg2", "fg2+") else Hk     # the mapped keys are per value head in FG2
    gen = torch.Generator().manual_seed(7)
    grads = {"dq": torch.randn(N, T, hq, dk, generator=gen), "dk": torch.randn(N, T, hq, dk, generator=gen),
             "dv": torch.randn(N, T, Hv, dv, generator=gen), "dw": torch.randn(N, T, Hv, dv, generator=gen),
             "dlog_alpha": torch.randn(N, T, Hv, dk, generator=gen),
             "db": torch.randn(N, T, Hv, dk, generator=gen)}
    print(f"[case] map_gates_bwd {mode} {dtype}", flush=True)
    got = g.map_gates_bwd(mode, d["k"], d["v"], d["beta"], {n: t.cuda() for n, t in grads.items()},
                          beta_v=d.get("beta_v"))
    torch.cuda.synchronize()
    gf = {n: t.double().numpy() for n, t in grads.items()}
    per_pair = {}
    for n in range(N):
        for h in range(Hv):
            args, bv = _pair_args(mode, f, n, h, Hv // Hk)
            hm = h if hq == Hv else h // (Hv // Hk)
            gm = {"dq": gf["dq"][n, :, hm], "dk": gf["dk"][n, :, hm], "dv": gf["dv"][n, :, h],
                  "dw": gf["dw"][n, :, h], "dlog_alpha": gf["dlog_alpha"][n, :, h],
                  "db": gf["db"][n, :, h]}
            per_pair[(n, h)] = oracle.map_gates_bwd(mode, *args, gm, bv)
    ref = _assemble(mode, f, per_pair)
    if hq == Hk:       # dq, dk pass through per key head: not summed over the value heads
        ref["dq"], ref["dk"] = gf["dq"], gf["dk"]
    errs = {n: oracle.rel_l2(np64(got[n]).reshape(ref[n].shape), ref[n]) for n in ref}
    print(f"[parity] map_gates_bwd {mode} {dtype}: " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()),
          flush=True)
    assert max(errs.values()) <= 1e-5, errs


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("mode", MODES)
def test_variant_training_gradients(mode, dtype):
    """The gradients of a variant's loss with respect to its own inputs, on the GPU:
    map_gates -> chunk_bwd -> map_gates_bwd, against the oracle's map_gates -> sequence_bwd
    -> map_gates_bwd per pair (itself pinned against finite differences of the variant's own
    rule). Relative L2 per gradient tensor at the forward's bars."""
    dk, dv = (128, 128) if mode == "fg2" else (128, 64)
    x = inputs.variant_inputs(mode, dtype, 2, 150, 2, 4, dk, dv, seed=120 + MODES.index(mode))
    d = {n: t.cuda() for n, t in x.items()}
    f = {n: np64(t) for n, t in x.items()}
    N, T, Hv = 2, 150, 4
    gen = torch.Generator().manual_seed(8)
    dO = torch.randn(N, T, Hv, dv, generator=gen).to(dtype)
    dST = torch.randn(N, Hv, dk, dv, generator=gen)
    print(f"[case] variant training gradients {mode} {dtype}", flush=True)
    m = g.map_gates(mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d.get("beta_v"))
    gm = g.chunk_bwd(*m, dO.cuda(), S0=d["S"], dS_T=dST.cuda())
    got = g.map_gates_bwd(mode, d["k"], d["v"], d["beta"], gm, beta_v=d.get("beta_v"))
    torch.cuda.synchronize()
    dO64, dST64 = np64(dO), np64(dST)
    per_pair, dS0 = {}, np.zeros((N, Hv, dk, dv))
    for n in range(N):
        for h in range(Hv):
            args, bv = _pair_args(mode, f, n, h, 2)
            mm = oracle.map_gates(mode, *args, bv)
            gp = oracle.sequence_bwd(mm[0], mm[1], mm[2], mm[5], mm[3], mm[4], f["S"][n, h],
                                     dO64[n, :, h], dST64[n, h])
            per_pair[(n, h)] = oracle.map_gates_bwd(mode, *args, gp, bv)
            dS0[n, h] = gp["dS0"]
    ref = _assemble(mode, f, per_pair)
    errs = {n: oracle.rel_l2(np64(got[n]).reshape(ref[n].shape), ref[n]) for n in ref}
    errs["dS0"] = oracle.rel_l2(np64(gm["dS0"]), dS0)
    print(f"[parity] variant grads {mode} {dtype} {dk}x{dv}: " +
          " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    assert all(np.isfinite(list(errs.values())))
    assert max(errs.values()) <= TOL[dtype], errs
