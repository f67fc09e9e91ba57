"""Helpers shared by the GPU parity tests: run the HIP path and the fp64 oracle on the same
seeded inputs and compare them by relative L2 error."""
import numpy as np
import torch

import oracle
import gated_delta_rule_gdn_amd as g

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
ORACLE_THREADS = 16          # the GPU machine's CPU share


def np64(t):
    return t.detach().to("cpu").double().numpy()


def flat_inputs(x):
    """Oracle view of chunk inputs: packed [T_total, H, d] fp64 arrays and offsets."""
    B, T = x["q"].shape[:2]
    f = {n: np64(x[n]).reshape(B * T, *x[n].shape[2:]) for n in
         ("q", "k", "v", "log_alpha", "b", "w")}
    cu = np64(x["cu_seqlens"]).astype(np.int64) if x["cu_seqlens"] is not None \
        else np.arange(B + 1, dtype=np.int64) * T
    S0 = None if x["S0"] is None else np64(x["S0"])
    return f, cu, S0


def oracle_chunk(x, pairs=None):
    f, cu, S0 = flat_inputs(x)
    return oracle.recurrent(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], S0=S0,
                            cu_seqlens=cu, pairs=pairs, threads=ORACLE_THREADS)


def to_gpu(x):
    return {n: (t.cuda() if isinstance(t, torch.Tensor) else t) for n, t in x.items()}


def gpu_chunk(x, **kw):
    d = to_gpu(x)
    o, S_T = g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                         cu_seqlens=d["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    B, T = x["q"].shape[:2]
    return np64(o).reshape(B * T, *o.shape[2:]), (None if S_T is None else np64(S_T))


def select(o, S, cu, pairs):
    """Entries of (o, S_T) that belong to the given (sequence, head) pairs, flattened."""
    parts_o, parts_s = [], []
    for n, h in pairs:
        parts_o.append(o[cu[n]:cu[n + 1], h].ravel())
        parts_s.append(S[n, h].ravel())
    return np.concatenate(parts_o), np.concatenate(parts_s)


def assert_chunk_parity(x, dtype, pairs=None, label="", worst=False, **kw):
    """Runs both paths; compares all pairs (or the given ones) within the dtype's tolerance.
    worst=True also prints the largest per-(sequence, head) error as a diagnostic. Extra
    keywords go to the GPU call (chunk_size, ...)."""
    o_g, S_g = gpu_chunk(x, **kw)
    o_r, S_r = oracle_chunk(x, pairs=pairs)
    _, cu, _ = flat_inputs(x)
    if pairs is None:
        eo, es = oracle.rel_l2(o_g, o_r), oracle.rel_l2(S_g, S_r)
    else:
        go, gs = select(o_g, S_g, cu, pairs)
        ro, rs = select(o_r, S_r, cu, pairs)
        eo, es = oracle.rel_l2(go, ro), oracle.rel_l2(gs, rs)
        assert np.all(np.isfinite(o_g)) and np.all(np.isfinite(S_g))
    tol = TOL[dtype]
    extra = ""
    if worst:
        N, H = S_g.shape[:2]
        wo = max(oracle.rel_l2(o_g[cu[n]:cu[n + 1], h], o_r[cu[n]:cu[n + 1], h])
                 for n in range(N) for h in range(H) if cu[n + 1] > cu[n])
        ws = max(oracle.rel_l2(S_g[n, h], S_r[n, h]) for n in range(N) for h in range(H))
        extra = f" worst pair o={wo:.3e} S_T={ws:.3e}"
    print(f"[parity] {label} rel_l2 o={eo:.3e} S_T={es:.3e} tol={tol:g}{extra}", flush=True)
    assert eo <= tol and es <= tol, (label, eo, es)
    return eo, es


def decode_oracle_pair(x, n, h, steps, group):
    """All steps of one (sequence, value head) state with the fp64 oracle."""
    hk = h // group
    sl = slice(0, steps)
    return oracle.sequence(np64(x["q"][sl, n, hk]), np64(x["k"][sl, n, hk]),
                           np64(x["v"][sl, n, h]), np64(x["w"][sl, n, h]),
                           np64(x["log_alpha"][sl, n, h]), np64(x["b"][sl, n, h]),
                           np64(x["S"][n, h]))
