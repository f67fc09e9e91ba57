"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle for the Gated DeltaNet-2 core.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package. The GPU library never imports, links or calls it, and it
shares no code with the GPU library: the only thing both sides consume is the
seeded input generator, which holds none of the method's arithmetic.

Two independent evaluations of the method live here:

* ``recurrent`` -- the per-token recurrence of the burn-gdn2 0.1.5 docs page
  (section "Architecture"), written out in plain C (``gdn2_oracle.c``), fp64, one
  (sequence, value head) pair at a time. ``decode_step`` is one token of it, and
  ``recurrent_cache`` runs it over a pool of stored states (the recurrent cache of the
  GDN decode verify page, LocalAI mirror, section 2), optionally stored in bfloat16
  (section 4 of the same notes), with ``round_to_bf16`` the rounding of the stored state.
* ``short_conv`` / ``conv_qkv``, ``l2_normalize`` and ``gated_rms_norm`` -- the stages
  the burn-gdn2 "Architecture" diagram draws around the recurrence (ShortConv and the
  L2-Norm of q and k before it, the Gated RMS Norm with a SiLU gate after it), in numpy
  fp64.
* ``chunk_states`` -- the state of ``recurrent`` after every whole multiple of the chunk
  size (the state entering each chunk of the chunked form), by running the same C
  recurrence span by span.
* ``recurrent_bwd`` -- the gradient of ``recurrent`` with respect to every input and the
  initial state, by the token-by-token adjoint of the recurrence (chain rule through the
  decay, erase, write and read-out steps, in reverse), fp64, in the same C file.
* ``variant_sequence`` / ``variant`` -- the update rules of the neighbouring delta-rule
  models the pages name (the scalar-gate KDA that the "Architecture" section says b and w
  replace, a scalar-decay GDN, and FG2-GDN and FG2-GDN+ of the FG2-GDN summary, section 2),
  each written from its own formula in numpy fp64. ``map_gates`` gives the GDN-2 inputs of
  each variant and ``map_gates_bwd`` the chain rule back through them.
* ``chunked_sequence_bwd`` -- the gradient taken through that chunked form, step by step
  (the backward pass chunked kernels follow), checked against ``recurrent_bwd``.
* ``chunked`` -- the chunked WY form named on the same page (the "Chunk" training
  mode) and on the FG^2-GDN summary (section 2C, DPLR structure and the WY
  representation), in numpy fp64. It exists to pin the recurrence: the two are
  different algorithms and agree only if both are right.

Conventions (taken where the pages are silent):

* packed token layout: ``q, k`` are ``[T_total, H_k, d_k]``, ``v, w`` are
  ``[T_total, H_v, d_v]``, ``log_alpha, b`` are ``[T_total, H_v, d_k]``;
  sequence ``n`` owns tokens ``cu_seqlens[n] .. cu_seqlens[n+1]-1``;
* value head ``h`` reads key head ``h // (H_v // H_k)`` (contiguous groups);
* ``log_alpha`` carries ``log(alpha) <= 0``; the output reads the state after the
  update of its own token; there is no query scale;
* ``S0 is None`` means a zero initial state.

Parity of these functions is pinned by ``tests/test_oracle_pins.py`` (closed forms,
invariants, the formulas of the other pages, brute force, chunked-vs-recurrent).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_LIB_DIR = os.path.join(_HERE, "_build")
_LIB = os.path.join(_LIB_DIR, "libgdn2_oracle.so")
_lib = None


def build() -> str:
    """Compile the C oracle with gcc (-O2, no fast-math). Returns the library path."""
    os.makedirs(_LIB_DIR, exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
           "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gdn2_oracle_sequence.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             dp, dp, dp, dp, dp, dp, dp, dp]
        lib.gdn2_oracle_sequence.restype = ctypes.c_int
        lib.gdn2_oracle_sequence_bwd.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32] + \
            [dp] * 16
        lib.gdn2_oracle_sequence_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def sequence(q, k, v, w, log_alpha, b, S0):
    """One (sequence, value head) pair: q,k,log_alpha,b [T,d_k]; v,w [T,d_v]; S0 [d_k,d_v].

    Returns (o [T,d_v], S_T [d_k,d_v]) in fp64.
    """
    lib = _load()
    q, k, v, w, la, b = (_f64(x) for x in (q, k, v, w, log_alpha, b))
    T, d_k = k.shape
    d_v = v.shape[1]
    S = _f64(S0).copy()
    o = np.zeros((T, d_v), dtype=np.float64)
    rc = lib.gdn2_oracle_sequence(T, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(w),
                                  _ptr(la), _ptr(b), _ptr(S), _ptr(o))
    if rc != 0:
        raise MemoryError("gdn2_oracle_sequence failed")
    return o, S


def recurrent(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, pairs=None, threads=None):
    """Token-by-token recurrence over packed sequences.

    q, k: [T_total, H_k, d_k]; v, w: [T_total, H_v, d_v]; log_alpha, b: [T_total, H_v, d_k];
    S0: [N, H_v, d_k, d_v] or None (zeros); cu_seqlens: [N+1] offsets, or None for one
    sequence of T_total tokens. ``pairs`` restricts the work to a list of (n, h); entries of
    other pairs are left NaN. Returns (o [T_total, H_v, d_v], S_T [N, H_v, d_k, d_v]) fp64.
    """
    q, k, v, w, la, b = (np.asarray(x) for x in (q, k, v, w, log_alpha, b))
    T_total, H_k, d_k = k.shape
    H_v, d_v = v.shape[1], v.shape[2]
    if H_v % H_k:
        raise ValueError("H_v must be a multiple of H_k")
    G = H_v // H_k
    cu = np.array([0, T_total] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    if pairs is None:
        pairs = [(n, h) for n in range(N) for h in range(H_v)]
    o = np.full((T_total, H_v, d_v), np.nan)
    S_T = np.full((N, H_v, d_k, d_v), np.nan)

    def run(pair):
        n, h = pair
        s, e = int(cu[n]), int(cu[n + 1])
        hk = h // G
        S_init = np.zeros((d_k, d_v)) if S0 is None else np.asarray(S0)[n, h]
        on, Sn = sequence(q[s:e, hk], k[s:e, hk], v[s:e, h], w[s:e, h], la[s:e, h], b[s:e, h],
                          S_init)
        o[s:e, h] = on
        S_T[n, h] = Sn

    nthr = threads or default_threads()
    if nthr <= 1 or len(pairs) <= 1:
        for p in pairs:
            run(p)
    else:
        with ThreadPoolExecutor(max_workers=nthr) as ex:
            list(ex.map(run, pairs))
    return o, S_T


def chunk_states(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, chunk_size=64,
                 threads=None):
    """The state entering every chunk: for sequence n and chunk j, the state of the
    token-by-token recurrence after the first j * chunk_size tokens of the sequence (j = 0:
    S0, or zeros). Layout as ``recurrent``; returns fp64 [num_chunks, H_v, d_k, d_v] with
    sequence n's chunks at rows sum_{m<n} ceil(len_m / chunk_size) + j."""
    q, k, v, w, la, b = (np.asarray(x) for x in (q, k, v, w, log_alpha, b))
    T_total, H_k, d_k = k.shape
    H_v, d_v = v.shape[1], v.shape[2]
    G = H_v // H_k
    cu = np.array([0, T_total] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    nch = [-(-int(cu[n + 1] - cu[n]) // chunk_size) for n in range(N)]
    first = np.concatenate([[0], np.cumsum(nch)]).astype(np.int64)
    out = np.full((int(first[-1]), H_v, d_k, d_v), np.nan)

    def run(pair):
        n, h = pair
        hk = h // G
        S = np.zeros((d_k, d_v)) if S0 is None else _f64(np.asarray(S0)[n, h])
        for j in range(nch[n]):
            out[first[n] + j, h] = S
            s = int(cu[n]) + j * chunk_size
            e = min(int(cu[n + 1]), s + chunk_size)
            _, S = sequence(q[s:e, hk], k[s:e, hk], v[s:e, h], w[s:e, h], la[s:e, h],
                            b[s:e, h], S)

    pairs = [(n, h) for n in range(N) for h in range(H_v)]
    nthr = threads or default_threads()
    if nthr <= 1 or len(pairs) <= 1:
        for pr in pairs:
            run(pr)
    else:
        with ThreadPoolExecutor(max_workers=nthr) as ex:
            list(ex.map(run, pairs))
    return out


def sequence_bwd(q, k, v, w, log_alpha, b, S0, do, dS_T=None):
    """Gradient of ``sequence`` for one (sequence, value head) pair, by the token-by-token
    adjoint of the recurrence (gdn2_oracle.c). do [T,d_v] and dS_T [d_k,d_v] (None: zero)
    are the gradients of the loss with respect to o and S_T. Returns a dict of fp64 arrays
    dq, dk, dlog_alpha, db [T,d_k]; dv, dw [T,d_v]; dS0 [d_k,d_v]."""
    lib = _load()
    q, k, v, w, la, b, dO = (_f64(x) for x in (q, k, v, w, log_alpha, b, do))
    T, d_k = k.shape
    d_v = v.shape[1]
    S0 = _f64(S0)
    dST = None if dS_T is None else _f64(dS_T)
    out = {n: np.zeros((T, d_k)) for n in ("dq", "dk", "dlog_alpha", "db")}
    out.update({n: np.zeros((T, d_v)) for n in ("dv", "dw")})
    out["dS0"] = np.zeros((d_k, d_v))
    rc = lib.gdn2_oracle_sequence_bwd(
        T, d_k, d_v, _ptr(q), _ptr(k), _ptr(v), _ptr(w), _ptr(la), _ptr(b), _ptr(S0), _ptr(dO),
        None if dST is None else _ptr(dST), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
        _ptr(out["dw"]), _ptr(out["dlog_alpha"]), _ptr(out["db"]), _ptr(out["dS0"]))
    if rc != 0:
        raise MemoryError("gdn2_oracle_sequence_bwd failed")
    return out


def recurrent_bwd(q, k, v, log_alpha, b, w, do, S0=None, dS_T=None, cu_seqlens=None,
                  threads=None):
    """Gradient of ``recurrent`` (same packed layouts; do like o, dS_T like S_T or None).
    Under grouped value heads the q and k gradients sum over the value heads that read the
    key head. Returns a dict: dq, dk [T_total,H_k,d_k]; dv, dw [T_total,H_v,d_v];
    dlog_alpha, db [T_total,H_v,d_k]; dS0 [N,H_v,d_k,d_v]."""
    q, k, v, w, la, b, dO = (np.asarray(x) for x in (q, k, v, w, log_alpha, b, do))
    T_total, H_k, d_k = k.shape
    H_v, d_v = v.shape[1], v.shape[2]
    G = H_v // H_k
    cu = np.array([0, T_total] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    res = {"dq": np.zeros((T_total, H_k, d_k)), "dk": np.zeros((T_total, H_k, d_k)),
           "dv": np.zeros((T_total, H_v, d_v)), "dw": np.zeros((T_total, H_v, d_v)),
           "dlog_alpha": np.zeros((T_total, H_v, d_k)), "db": np.zeros((T_total, H_v, d_k)),
           "dS0": np.zeros((N, H_v, d_k, d_v))}
    pairs = [(n, h) for n in range(N) for h in range(H_v)]

    def run(pair):
        n, h = pair
        s, e = int(cu[n]), int(cu[n + 1])
        hk = h // G
        S_init = np.zeros((d_k, d_v)) if S0 is None else np.asarray(S0)[n, h]
        dst = None if dS_T is None else np.asarray(dS_T)[n, h]
        return pair, sequence_bwd(q[s:e, hk], k[s:e, hk], v[s:e, h], w[s:e, h], la[s:e, h],
                                  b[s:e, h], S_init, dO[s:e, h], dst)

    nthr = threads or default_threads()
    if nthr <= 1 or len(pairs) <= 1:
        results = [run(p) for p in pairs]
    else:
        with ThreadPoolExecutor(max_workers=nthr) as ex:
            results = list(ex.map(run, pairs))
    for (n, h), gr in results:           # accumulated in a fixed order
        s, e = int(cu[n]), int(cu[n + 1])
        hk = h // G
        res["dq"][s:e, hk] += gr["dq"]
        res["dk"][s:e, hk] += gr["dk"]
        for nm in ("dv", "dw", "dlog_alpha", "db"):
            res[nm][s:e, h] = gr[nm]
        res["dS0"][n, h] = gr["dS0"]
    return res


def decode_step(q, k, v, log_alpha, b, w, S, pairs=None, threads=None):
    """One token per sequence: q,k [N,H_k,d_k]; v,w [N,H_v,d_v]; log_alpha,b [N,H_v,d_k];
    S [N,H_v,d_k,d_v]. Returns (o [N,H_v,d_v], S_new)."""
    N = np.asarray(k).shape[0]
    cu = np.arange(N + 1)
    return recurrent(q, k, v, log_alpha, b, w, S0=S, cu_seqlens=cu, pairs=pairs,
                     threads=threads)


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each element, ties to even, returned as fp64.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and fp32's exponent range:
    a finite x with 2^(e-1) <= |x| < 2^e (numpy's frexp exponent e) is rounded to a
    multiple of 2^(e-8), and below the smallest normal 2^-126 to a multiple of 2^-133
    (the subnormal spacing). np.rint rounds halves to even. Magnitudes that round past the
    largest finite value (2 - 2^-7) * 2^127 become infinities; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / ulp) * ulp
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    r = np.where(np.abs(r) > big, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def recurrent_cache(q, k, v, log_alpha, b, w, state, state_idx=None, bf16_state=False,
                    threads=None):
    """T tokens per sequence against a pool of recurrent states (the decode cache).

    q, k [N,T,H_k,d_k]; v, w [N,T,H_v,d_v]; log_alpha, b [N,T,H_v,d_k]; ``state`` the pool
    [num_slots,H_v,d_k,d_v] as stored; ``state_idx`` [N] the slot of each sequence (None:
    slot n). An entry outside [0, num_slots) marks a padding sequence: its o rows are zero
    and no slot changes. Each valid sequence runs the token-by-token recurrence over its T
    tokens from the state in its slot; the slot then holds the final state, rounded to the
    nearest bfloat16 when the pool is stored in bfloat16 (``bf16_state``).
    Returns (o [N,T,H_v,d_v], new pool), fp64.
    """
    q, k, v, w, la, b = (np.asarray(x, dtype=np.float64) for x in (q, k, v, w, log_alpha, b))
    N, T = k.shape[:2]
    pool = np.array(state, dtype=np.float64, copy=True)
    num_slots = pool.shape[0]
    idx = np.arange(N) if state_idx is None else np.asarray(state_idx, dtype=np.int64)
    o = np.zeros(v.shape)
    live = [n for n in range(N) if 0 <= idx[n] < num_slots]
    if not live:
        return o, pool
    flat = lambda x: x[live].reshape(len(live) * T, *x.shape[2:])
    cu = np.arange(len(live) + 1) * T
    o_l, S_l = recurrent(flat(q), flat(k), flat(v), flat(la), flat(b), flat(w),
                         S0=pool[idx[live]], cu_seqlens=cu, threads=threads)
    o[live] = o_l.reshape(len(live), T, *o_l.shape[1:])
    pool[idx[live]] = round_to_bf16(S_l) if bf16_state else S_l
    return o, pool


def l2_normalize(x, eps):
    """Each vector along the last axis divided by sqrt(sum of its squares + eps).

    The L2-Norm stage that the burn-gdn2 page (section "Architecture") places on q and k
    before the recurrence; the epsilon is this build's reading (the page names none).
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def gated_rms_norm(o, gate, weight, eps):
    """The Gated RMS Norm with a SiLU gate after the recurrence (burn-gdn2 "Architecture";
    norm_eps in its Configuration table), per vector along the last axis:
        o / sqrt(mean(o^2) + eps) * weight * silu(gate),   silu(g) = g / (1 + exp(-g)).
    """
    o = np.asarray(o, dtype=np.float64)
    g = np.asarray(gate, dtype=np.float64)
    rms = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / rms * np.asarray(weight, dtype=np.float64) * (g / (1.0 + np.exp(-g)))


def short_conv(x, weight, state, silu=False):
    """Causal depthwise convolution of width 4 along the token axis, one sequence.

    The ShortConv stage of the burn-gdn2 "Architecture" diagram; the GDN decode verify page
    gives its width 4 (section 1) and its state, the last three inputs of every channel
    (section 2). x [T, C] the inputs; weight [C, 4], tap 3 on the current token and tap 0
    on the input three tokens back; state [3, C] the three inputs before x, oldest first.
    With ``silu`` the output passes through y / (1 + exp(-y)) (the pages name no
    activation; it is an option). Returns (y [T, C], the new state [3, C]).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    xx = np.concatenate([np.asarray(state, dtype=np.float64), x], axis=0)
    y = np.zeros_like(x)
    for t in range(x.shape[0]):
        for j in range(4):
            y[t] += w[:, j] * xx[t + j]
    if silu:
        y = y / (1.0 + np.exp(-y))
    return y, xx[-3:].copy()


def conv_qkv(q, k, v, weight, conv_pool, state_idx=None, silu=False):
    """short_conv over the q, k and v channels of each sequence against a pool of conv
    states. q, k [N,T,H_k,d_k]; v [N,T,H_v,d_v]; channels in the order q (key heads), k
    (key heads), v (value heads), each head's values contiguous; weight [C, 4]; conv_pool
    [num_slots, 3, C]; ``state_idx`` as in ``recurrent_cache`` (padding entries leave
    their slot alone and return their inputs unchanged). Returns (q', k', v', new pool)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N, T, H_k, d_k = q.shape
    H_v, d_v = v.shape[2:]
    pool = np.array(conv_pool, dtype=np.float64, copy=True)
    idx = np.arange(N) if state_idx is None else np.asarray(state_idx, dtype=np.int64)
    qo, ko, vo = q.copy(), k.copy(), v.copy()
    for n in range(N):
        s = idx[n]
        if not 0 <= s < pool.shape[0]:
            continue
        x = np.concatenate([q[n].reshape(T, -1), k[n].reshape(T, -1), v[n].reshape(T, -1)], 1)
        y, pool[s] = short_conv(x, weight, pool[s], silu)
        a, bnd = H_k * d_k, 2 * H_k * d_k
        qo[n] = y[:, :a].reshape(T, H_k, d_k)
        ko[n] = y[:, a:bnd].reshape(T, H_k, d_k)
        vo[n] = y[:, bnd:].reshape(T, H_v, d_v)
    return qo, ko, vo, pool


def _unit_lower_inverse(L: np.ndarray) -> np.ndarray:
    """Inverse of a unit lower-triangular matrix by forward substitution on the identity."""
    n = L.shape[0]
    Tm = np.zeros_like(L)
    for r in range(n):
        row = np.zeros(n)
        row[r] = 1.0
        for i in range(r):
            row -= L[r, i] * Tm[i]
        Tm[r] = row
    return Tm


def chunked_sequence(q, k, v, w, log_alpha, b, S0, chunk_size):
    """Chunked WY form of the recurrence for one (sequence, value head) pair, fp64.

    Within a chunk of L tokens entering with state S (all vectors per token are rows):
      g_r        = sum_{i<=r} log alpha_i                    (cumulative log decay, per key channel)
      A[r,i]     = sum_c b_r[c] k_r[c] k_i[c] exp(g_r[c]-g_i[c]),  i < r   (0 elsewhere)
      T          = (I + A)^{-1}
      W~         = T (exp(g) . b . k),   U~ = T (w . v)       (the WY factors)
      U          = U~ - W~ S                                  (the per-token erase-corrected writes)
      Mqk[r,i]   = sum_c q_r[c] k_i[c] exp(g_r[c]-g_i[c]),     i <= r
      O          = (exp(g) . q) S + Mqk U
      S_next     = diag(exp(g_L)) S + (exp(g_L - g) . k)^T U
    Returns (o [T,d_v], S_T).
    """
    q, k, v, w, la, b = (_f64(x) for x in (q, k, v, w, log_alpha, b))
    T = k.shape[0]
    S = _f64(S0).copy()
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk_size):
        sl = slice(c0, min(T, c0 + chunk_size))
        qc, kc, vc, wc, lac, bc = q[sl], k[sl], v[sl], w[sl], la[sl], b[sl]
        L = kc.shape[0]
        g = np.cumsum(lac, axis=0)
        A = np.zeros((L, L))
        Mqk = np.zeros((L, L))
        for r in range(L):
            for i in range(r + 1):
                dec = np.exp(g[r] - g[i])
                Mqk[r, i] = np.sum(qc[r] * kc[i] * dec)
                if i < r:
                    A[r, i] = np.sum(bc[r] * kc[r] * kc[i] * dec)
        Tm = _unit_lower_inverse(np.eye(L) + A)
        W_t = Tm @ (np.exp(g) * bc * kc)
        U_t = Tm @ (wc * vc)
        U = U_t - W_t @ S
        o[sl] = (np.exp(g) * qc) @ S + Mqk @ U
        S = np.exp(g[-1])[:, None] * S + (np.exp(g[-1][None, :] - g) * kc).T @ U
    return o, S


def chunked(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, chunk_size=64):
    """Chunked WY form over packed sequences; same layout and result as ``recurrent``."""
    q, k, v, w, la, b = (np.asarray(x) for x in (q, k, v, w, log_alpha, b))
    T_total, H_k, d_k = k.shape
    H_v, d_v = v.shape[1], v.shape[2]
    G = H_v // H_k
    cu = np.array([0, T_total] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    o = np.zeros((T_total, H_v, d_v))
    S_T = np.zeros((N, H_v, d_k, d_v))
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(H_v):
            hk = h // G
            S_init = np.zeros((d_k, d_v)) if S0 is None else np.asarray(S0)[n, h]
            on, Sn = chunked_sequence(q[s:e, hk], k[s:e, hk], v[s:e, h], w[s:e, h],
                                      la[s:e, h], b[s:e, h], S_init, chunk_size)
            o[s:e, h] = on
            S_T[n, h] = Sn
    return o, S_T


def chunked_sequence_bwd(q, k, v, w, log_alpha, b, S0, do, dS_T, chunk_size):
    """Gradient of ``chunked_sequence`` for one pair, taken through the chunked WY form
    itself (fp64): the backward pass the chunked kernels follow, written out so that it can
    be checked against the token-by-token adjoint (``sequence_bwd``). With the forward's
    chunk quantities (g, A, T, W~, U~, U, Mqk, Qg = exp(g).q, Kg = exp(g_L - g).k, the entry
    state S) and dS' = dL/dS_next, per chunk from the last:
      dU   = Mqk^T dO + Kg dS'
      dS   = diag(exp(g_L)) dS' + Qg^T dO - W~^T dU                 (handed to the chunk before)
      dMqk = lower(dO U^T),  dQg = dO S^T,  dKg = U dS'^T,  dW~ = -dU S^T,  dU~ = dU
      dX   = T^T dU~ (X = w.v),  dY = T^T dW~ (Y = exp(g).b.k)
      dT   = dU~ X^T + dW~ Y^T,  dA = strictly-lower(-T^T dT T^T)
    then the chain rule through A, Mqk, Y, Qg, Kg and exp(g_L) to q, k, b, g, and
    dlog_alpha_i = sum_{r >= i} dg_r within the chunk. Same outputs as ``sequence_bwd``."""
    q, k, v, w, la, b, dO = (_f64(x) for x in (q, k, v, w, log_alpha, b, do))
    T, d_k = k.shape
    d_v = v.shape[1]
    S = _f64(S0).copy()
    starts = list(range(0, T, chunk_size))
    entry = []
    for c0 in starts:                      # forward: the state entering each chunk
        entry.append(S.copy())
        sl = slice(c0, min(T, c0 + chunk_size))
        _, S = chunked_sequence(q[sl], k[sl], v[sl], w[sl], la[sl], b[sl], S, chunk_size)
    out = {n: np.zeros((T, d_k)) for n in ("dq", "dk", "dlog_alpha", "db")}
    out.update({n: np.zeros((T, d_v)) for n in ("dv", "dw")})
    dS = np.zeros((d_k, d_v)) if dS_T is None else _f64(dS_T).copy()
    for c0, S in zip(reversed(starts), reversed(entry)):
        sl = slice(c0, min(T, c0 + chunk_size))
        qc, kc, vc, wc, lac, bc, dOc = q[sl], k[sl], v[sl], w[sl], la[sl], b[sl], dO[sl]
        L = kc.shape[0]
        g = np.cumsum(lac, axis=0)
        E = np.exp(g[:, None, :] - g[None, :, :])          # E[r, i] = exp(g_r - g_i)
        low = np.tril(np.ones((L, L)))
        slow = np.tril(np.ones((L, L)), -1)
        bk = bc * kc
        A = np.einsum("rc,ic,ric->ri", bk, kc, E) * slow
        Mqk = np.einsum("rc,ic,ric->ri", qc, kc, E) * low
        Tm = _unit_lower_inverse(np.eye(L) + A)
        gam = np.exp(g)
        Y, X = gam * bk, wc * vc
        W_t, U_t = Tm @ Y, Tm @ X
        U = U_t - W_t @ S
        Qg = gam * qc
        fK = np.exp(g[-1][None, :] - g)
        Kg = fK * kc
        # the chunk's own adjoints
        dU = Mqk.T @ dOc + Kg @ dS
        dS_prev = gam[-1][:, None] * dS + Qg.T @ dOc - W_t.T @ dU
        dM = (dOc @ U.T) * low
        dQg = dOc @ S.T
        dKg = U @ dS.T
        dW = -dU @ S.T
        dgam_L = np.sum(dS * S, axis=1)
        dX = Tm.T @ dU
        dY = Tm.T @ dW
        dT = dU @ X.T + dW @ Y.T
        dA = -(Tm.T @ dT @ Tm.T) * slow
        # to the token vectors and g
        dq = np.einsum("ri,ic,ric->rc", dM, kc, E) + gam * dQg
        dk = (np.einsum("ri,rc,ric->ic", dM, qc, E) + np.einsum("ri,rc,ric->ic", dA, bk, E)
              + fK * dKg)
        dbk = np.einsum("ri,ic,ric->rc", dA, kc, E) + gam * dY
        tA = np.einsum("ri,rc,ic,ric->ric", dA, bk, kc, E)
        tM = np.einsum("ri,rc,ic,ric->ric", dM, qc, kc, E)
        dg = (tA.sum(1) - tA.sum(0) + tM.sum(1) - tM.sum(0)
              + gam * bk * dY + gam * qc * dQg - fK * kc * dKg)
        dg[-1] += np.sum(fK * kc * dKg, axis=0) + gam[-1] * dgam_L
        out["dq"][sl] = dq
        out["dk"][sl] = dk + bc * dbk
        out["db"][sl] = kc * dbk
        out["dv"][sl] = wc * dX
        out["dw"][sl] = vc * dX
        out["dlog_alpha"][sl] = np.cumsum(dg[::-1], axis=0)[::-1]
        dS = dS_prev
    out["dS0"] = dS
    return out


def variant_sequence(mode, q, k, v, log_alpha, beta, S0, beta_v=None):
    """One (sequence, value head) pair of another gated delta-rule variant, fp64, token by
    token from that variant's own update rule (not through the GDN-2 form):

    * ``"kda"`` (the scalar-gate model the burn-gdn2 "Architecture" section says b and w
      replace): ``S <- (I - beta k k^T) diag(alpha) S + beta k v^T``, beta [T] scalar;
    * ``"gdn"``: the same with a scalar decay, ``log_alpha`` [T];
    * ``"fg2"`` (FG2-GDN page, section 2A): ``k~ = sqrt(beta) k``, ``v~ = sqrt(beta) v`` with
      beta [T, d_k] (d_v = d_k), ``S <- (I - k~ k~^T) diag(alpha) S + k~ v~^T``;
    * ``"fg2+"`` (section 2B): as fg2 with ``v~ = sqrt(beta_v) v``, beta_v [T, d_v].

    q, k [T, d_k]; v [T, d_v]; log_alpha [T, d_k] (or [T]); S0 [d_k, d_v]. The output reads
    the updated state, ``o_t = S_t^T q_t``. Returns (o [T, d_v], S_T) fp64.
    """
    q, k, v, la, beta = (_f64(x) for x in (q, k, v, log_alpha, beta))
    bv = None if beta_v is None else _f64(beta_v)
    S = _f64(S0).copy()
    T, d_v = v.shape
    o = np.zeros((T, d_v))
    for t in range(T):
        a = np.exp(la[t])
        Sp = (a[:, None] * S) if np.ndim(a) else a * S
        if mode in ("kda", "gdn"):
            kk, vv, bt = k[t], v[t], beta[t]
            S = Sp - bt * np.outer(kk, kk @ Sp) + bt * np.outer(kk, vv)
        elif mode in ("fg2", "fg2+"):
            kk = np.sqrt(beta[t]) * k[t]
            vv = (np.sqrt(beta[t]) if mode == "fg2" else np.sqrt(bv[t])) * v[t]
            S = Sp - np.outer(kk, kk @ Sp) + np.outer(kk, vv)
        else:
            raise ValueError(f"unknown mode {mode!r}")
        o[t] = S.T @ q[t]
    return o, S


def variant(mode, q, k, v, log_alpha, beta, S0=None, beta_v=None, pairs=None):
    """``variant_sequence`` over every (sequence, value head) pair of [N, T, ...] inputs
    (value head h reads key head h // (H_v // H_k)). q, k [N,T,H_k,d_k]; v [N,T,H_v,d_v];
    log_alpha and beta per value head as in ``variant_sequence``; S0 [N,H_v,d_k,d_v] or None.
    Returns (o [N,T,H_v,d_v], S_T [N,H_v,d_k,d_v]) fp64 (NaN outside ``pairs``)."""
    q, k, v = (np.asarray(x) for x in (q, k, v))
    N, T, H_k, d_k = k.shape
    H_v, d_v = v.shape[2], v.shape[3]
    G = H_v // H_k
    o = np.full((N, T, H_v, d_v), np.nan)
    S_T = np.full((N, H_v, d_k, d_v), np.nan)
    for n, h in (pairs or [(n, h) for n in range(N) for h in range(H_v)]):
        S_init = np.zeros((d_k, d_v)) if S0 is None else np.asarray(S0)[n, h]
        o[n, :, h], S_T[n, h] = variant_sequence(
            mode, q[n, :, h // G], k[n, :, h // G], v[n, :, h], np.asarray(log_alpha)[n, :, h],
            np.asarray(beta)[n, :, h], S_init,
            None if beta_v is None else np.asarray(beta_v)[n, :, h])
    return o, S_T


def map_gates(mode, q, k, v, log_alpha, beta, beta_v=None):
    """The GDN-2 inputs under which the GDN-2 recurrence (``sequence``) is the variant
    ``mode`` of ``variant_sequence``, for one (sequence, value head) pair. The burn-gdn2
    "Architecture" section says the channel-wise b and w replace KDA's scalar gate; the FG2
    modes fold sqrt(beta) into the keys and values (FG2-GDN summary, section 2):

    * ``"kda"``: b = beta 1 [T, d_k], w = beta 1 [T, d_v]; q, k, v, log_alpha unchanged;
    * ``"gdn"``: as kda, log_alpha [T] broadcast over d_k;
    * ``"fg2"``: k' = sqrt(beta) k, v' = sqrt(beta) v, b = w = 1;
    * ``"fg2+"``: k' = sqrt(beta) k, b = 1, w = sqrt(beta_v), v unchanged.

    Shapes as in ``variant_sequence``. Returns (q', k', v', log_alpha', b, w) fp64."""
    q, k, v, la, beta = (_f64(x) for x in (q, k, v, log_alpha, beta))
    T, d_k = k.shape
    d_v = v.shape[1]
    if mode in ("kda", "gdn"):
        b = np.repeat(beta[:, None], d_k, axis=1)
        w = np.repeat(beta[:, None], d_v, axis=1)
        la2 = np.repeat(la[:, None], d_k, axis=1) if mode == "gdn" else la
        return q, k, v, la2, b, w
    if mode == "fg2":
        return q, np.sqrt(beta) * k, np.sqrt(beta) * v, la, np.ones((T, d_k)), np.ones((T, d_v))
    if mode == "fg2+":
        return q, np.sqrt(beta) * k, v, la, np.ones((T, d_k)), np.sqrt(_f64(beta_v))
    raise ValueError(f"unknown mode {mode!r}")


def map_gates_bwd(mode, q, k, v, log_alpha, beta, grads, beta_v=None):
    """The chain rule through ``map_gates`` for one pair: ``grads`` holds the gradients of
    a loss with respect to the mapped inputs (the keys of ``sequence_bwd``: dq, dk, dv,
    dlog_alpha, db, dw); returns the gradients with respect to the variant's own inputs,
    dict dq, dk, dv, dlog_alpha, dbeta (and dbeta_v for ``"fg2+"``), fp64, in the shapes of
    ``variant_sequence``'s inputs. b and w are constants in the FG2 modes, so their gradients
    end there. The derivative of sqrt(beta) is 1 / (2 sqrt(beta)): beta must be > 0 there."""
    q, k, v, la, beta = (_f64(x) for x in (q, k, v, log_alpha, beta))
    g = {n: _f64(x) for n, x in grads.items()}
    out = {"dq": g["dq"], "dv": g["dv"], "dlog_alpha": g["dlog_alpha"]}
    if mode in ("kda", "gdn"):
        # b and w are beta in every channel: dbeta sums their gradients over the channels
        out["dk"] = g["dk"]
        out["dbeta"] = g["db"].sum(axis=1) + g["dw"].sum(axis=1)
        if mode == "gdn":
            out["dlog_alpha"] = g["dlog_alpha"].sum(axis=1)
        return out
    if mode not in ("fg2", "fg2+"):
        raise ValueError(f"unknown mode {mode!r}")
    sb = np.sqrt(beta)
    out["dk"] = sb * g["dk"]                              # k' = sqrt(beta) k
    dbeta = g["dk"] * k / (2.0 * sb)
    if mode == "fg2":
        out["dv"] = sb * g["dv"]                          # v' = sqrt(beta) v
        dbeta = dbeta + g["dv"] * v / (2.0 * sb)
    else:
        out["dbeta_v"] = g["dw"] / (2.0 * np.sqrt(_f64(beta_v)))   # w = sqrt(beta_v)
    out["dbeta"] = dbeta
    return out


def rel_l2(x, ref) -> float:
    """Relative L2 error ||x - ref|| / ||ref|| (0 when both are zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    if den == 0.0:
        return float(num)
    return float(num / den)
