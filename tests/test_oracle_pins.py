"""Pins of the fp64 CPU oracle against facts fixed by the pages and by mathematics.

No page prints a worked numeric example of the recurrence, so each pin below is a
closed form, an invariant, another page's formula for a special case, brute force on
the definition, or agreement between the two independent algorithms in ``oracle``
(token-by-token recurrence in C, chunked WY form in numpy). Every pin uses d_k != d_v
where the case allows it, so a transposed operand or a swapped axis cannot pass.

Method: burn-gdn2 0.1.5 docs page, section "Architecture":
    S_t = (I - k_t (b_t . k_t)^T) diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T,  o_t = q_t^T S_t
"""
import numpy as np
import pytest

import oracle

TOL = 1e-11


def rand_case(rng, T, Hk=1, Hv=1, dk=5, dv=3, b_scale=2.0, unit_k=True):
    q = rng.standard_normal((T, Hk, dk))
    k = rng.standard_normal((T, Hk, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, Hv, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((T, Hv, dk)))
    b = b_scale / (1.0 + np.exp(-rng.standard_normal((T, Hv, dk))))
    w = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, Hv, dv))))
    return q, k, v, la, b, w


def close(a, b, tol=TOL):
    a, b = np.asarray(a), np.asarray(b)
    scale = max(1.0, float(np.max(np.abs(b))))
    return float(np.max(np.abs(a - b))) <= tol * scale


# ---- P1: brute force on the definition (explicit d_k x d_k transition matrices) ----------

def test_explicit_matrix_definition():
    rng = np.random.default_rng(1)
    T, dk, dv = 9, 5, 3
    q, k, v, la, b, w = rand_case(rng, T, dk=dk, dv=dv)
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    S = S0[0, 0].copy()
    for t in range(T):
        kt, bt = k[t, 0], b[t, 0]
        P = np.zeros((dk, dk))
        for i in range(dk):
            for j in range(dk):
                P[i, j] = (1.0 if i == j else 0.0) - kt[i] * bt[j] * kt[j]
        D = np.diag(np.exp(la[t, 0]))
        write = np.zeros((dk, dv))
        for i in range(dk):
            for j in range(dv):
                write[i, j] = kt[i] * w[t, 0, j] * v[t, 0, j]
        S = P @ D @ S + write
        ot = np.array([sum(q[t, 0, i] * S[i, j] for i in range(dk)) for j in range(dv)])
        assert close(o[t, 0], ot)
    assert close(ST[0, 0], S)


# ---- P2: chunked WY form (independent algorithm) equals the recurrence -------------------

@pytest.mark.parametrize("C", [1, 2, 3, 8, 16, 64])
def test_chunked_equals_recurrent(C):
    rng = np.random.default_rng(100 + C)
    for T in sorted({1, C - 1 if C > 1 else 1, C, C + 1, 2 * C + 3, 3 * C + 5}):
        q, k, v, la, b, w = rand_case(rng, T, Hk=2, Hv=4, dk=6, dv=4)
        S0 = rng.standard_normal((1, 4, 6, 4))
        o_r, S_r = oracle.recurrent(q, k, v, la, b, w, S0=S0, threads=1)
        o_c, S_c = oracle.chunked(q, k, v, la, b, w, S0=S0, chunk_size=C)
        assert close(o_c, o_r, 1e-10), (C, T)
        assert close(S_c, S_r, 1e-10), (C, T)


def test_chunked_equals_recurrent_varlen_with_empty_sequence():
    rng = np.random.default_rng(7)
    cu = np.array([0, 5, 5, 21, 40])
    q, k, v, la, b, w = rand_case(rng, 40, Hk=1, Hv=2, dk=4, dv=6)
    S0 = rng.standard_normal((4, 2, 4, 6))
    o_r, S_r = oracle.recurrent(q, k, v, la, b, w, S0=S0, cu_seqlens=cu)
    o_c, S_c = oracle.chunked(q, k, v, la, b, w, S0=S0, cu_seqlens=cu, chunk_size=8)
    assert close(o_c, o_r, 1e-10) and close(S_c, S_r, 1e-10)
    assert close(S_r[1], S0[1], 0.0)          # a zero-length sequence returns its S0


# ---- P3: alpha = 1, b = 0 is causal linear attention (O(T^2) brute force) ---------------

def test_linear_attention_closed_form():
    rng = np.random.default_rng(3)
    T, dk, dv = 13, 5, 3
    q, k, v, la, b, w = rand_case(rng, T, dk=dk, dv=dv, unit_k=False)
    la[:] = 0.0
    b[:] = 0.0
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    for t in range(T):
        ref = S0[0, 0].T @ q[t, 0]
        for i in range(t + 1):
            ref = ref + np.dot(q[t, 0], k[i, 0]) * (w[i, 0] * v[i, 0])
        assert close(o[t, 0], ref)
    S_ref = S0[0, 0] + sum(np.outer(k[i, 0], w[i, 0] * v[i, 0]) for i in range(T))
    assert close(ST[0, 0], S_ref)


def test_chunk_states_are_linear_attention_prefix_sums():
    """With alpha = 1 and b = 0 the state after n tokens is S0 + sum_{i<n} k_i (w_i v_i)^T,
    so the state entering chunk j is that sum up to j * chunk_size; packed sequences
    (one of them empty) and two value heads on one key head."""
    rng = np.random.default_rng(31)
    lens, C, dk, dv = [13, 0, 7], 4, 5, 3
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, la, b, w = rand_case(rng, int(cu[-1]), Hk=1, Hv=2, dk=dk, dv=dv, unit_k=False)
    la[:] = 0.0
    b[:] = 0.0
    S0 = rng.standard_normal((3, 2, dk, dv))
    ck = oracle.chunk_states(q, k, v, la, b, w, S0=S0, cu_seqlens=cu, chunk_size=C)
    assert ck.shape == (4 + 0 + 2, 2, dk, dv)
    row = 0
    for n, L in enumerate(lens):
        for j in range(-(-L // C)):
            for h in range(2):
                ref = S0[n, h].copy()
                for i in range(cu[n], cu[n] + j * C):
                    ref += np.outer(k[i, 0], w[i, h] * v[i, h])
                assert close(ck[row, h], ref)
            row += 1
    assert row == ck.shape[0]


def test_chunk_states_resume_to_the_final_state():
    """General gates: entry 0 is S0, and the recurrence resumed from the last entry over
    the sequence's last (ragged) chunk ends at the final state of the whole sequence."""
    rng = np.random.default_rng(32)
    T, C = 11, 4
    q, k, v, la, b, w = rand_case(rng, T, Hk=1, Hv=1, dk=5, dv=3)
    S0 = rng.standard_normal((1, 1, 5, 3))
    ck = oracle.chunk_states(q, k, v, la, b, w, S0=S0, chunk_size=C)
    assert ck.shape[0] == 3 and np.array_equal(ck[0], S0[0])
    _, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    _, S_end = oracle.recurrent(q[8:], k[8:], v[8:], la[8:], b[8:], w[8:], S0=ck[2][None])
    assert close(S_end, ST)
    _, S8 = oracle.recurrent(q[:8], k[:8], v[:8], la[:8], b[:8], w[:8], S0=S0)
    assert close(ck[2][None], S8)


# ---- P4: exact delta-rule retrieval ----------------------------------------------------

def test_exact_retrieval():
    rng = np.random.default_rng(4)
    T, d = 20, 8
    q, k, v, la, b, w = rand_case(rng, T, dk=d, dv=d)
    la[:] = 0.0
    b[:] = 1.0
    w[:] = 1.0
    q = k.copy()                                     # read out along the key just written
    S0 = rng.standard_normal((1, 1, d, d))
    o, _ = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    assert np.max(np.abs(o[:, 0] - v[:, 0])) < 1e-13 * 10


# ---- P5: the scalar-gate rule of the GDN decode verify page (section 2) ----------------

def test_scalar_gate_rule_of_llama_cpp_notes():
    """Decay s *= exp(g); sk = S^T k; delta d = (v - sk) * beta; s += k d^T; o = S^T q."""
    rng = np.random.default_rng(5)
    T, dk, dv = 11, 6, 4
    q, k, v, _, _, _ = rand_case(rng, T, dk=dk, dv=dv)
    g = -np.logaddexp(0.0, rng.standard_normal(T))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = rng.standard_normal((1, 1, dk, dv))
    la = np.broadcast_to(g[:, None, None], (T, 1, dk)).copy()
    b = np.broadcast_to(beta[:, None, None], (T, 1, dk)).copy()
    w = np.broadcast_to(beta[:, None, None], (T, 1, dv)).copy()
    o, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    s = S0[0, 0].copy()
    for t in range(T):
        s = s * np.exp(g[t])
        sk = s.T @ k[t, 0]
        d = (v[t, 0] - sk) * beta[t]
        s = s + np.outer(k[t, 0], d)
        assert close(o[t, 0], s.T @ q[t, 0])
    assert close(ST[0, 0], s)


# ---- P6: FG^2-GDN symmetric vector beta (gist.science summary, section 2A) -------------

def test_fg2_gdn_mapping():
    """S = (I - k~ k~^T) Diag(alpha) S + k~ v~^T with k~ = sqrt(beta).k, v~ = sqrt(beta).v
    equals the GDN-2 rule with k := k~, b := 1, w := 1, v := v~ (d_k = d_v for this variant)."""
    rng = np.random.default_rng(6)
    T, d = 10, 5
    q, k, v, la, _, _ = rand_case(rng, T, dk=d, dv=d)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, 1, d))))
    kt, vt = np.sqrt(beta) * k, np.sqrt(beta) * v
    S0 = rng.standard_normal((1, 1, d, d))
    o, ST = oracle.recurrent(q, kt, vt, la, np.ones((T, 1, d)), np.ones((T, 1, d)), S0=S0)
    S = S0[0, 0].copy()
    for t in range(T):
        S = (np.eye(d) - np.outer(kt[t, 0], kt[t, 0])) @ np.diag(np.exp(la[t, 0])) @ S \
            + np.outer(kt[t, 0], vt[t, 0])
        assert close(o[t, 0], S.T @ q[t, 0])
    assert close(ST[0, 0], S)


# ---- P7: b = 0 is gated linear attention with channel-wise decay (closed form) ---------

def test_gated_linear_attention_closed_form():
    rng = np.random.default_rng(8)
    T, dk, dv = 12, 4, 7
    q, k, v, la, b, w = rand_case(rng, T, dk=dk, dv=dv)
    b[:] = 0.0
    alpha = np.exp(la[:, 0])                     # [T, dk]
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    for t in range(T):
        St = np.prod(alpha[: t + 1], axis=0)[:, None] * S0[0, 0]
        for i in range(t + 1):
            decay_after_i = np.prod(alpha[i + 1: t + 1], axis=0)   # alpha_{i+1} ... alpha_t
            St = St + (decay_after_i * k[i, 0])[:, None] * (w[i, 0] * v[i, 0])[None, :]
        assert close(o[t, 0], St.T @ q[t, 0])
    assert close(ST[0, 0], St)


# ---- the asymmetric rank-1 erase: k on the left, b.k on the right ----------------------

def test_erase_eigenvalue_along_k():
    """With alpha = 1 and no write, S0 = k x^T maps to (1 - sum_c b_c k_c^2) k x^T."""
    rng = np.random.default_rng(9)
    dk, dv = 6, 3
    q, k, v, la, b, w = rand_case(rng, 1, dk=dk, dv=dv)
    la[:] = 0.0
    w[:] = 0.0
    x = rng.standard_normal(dv)
    S0 = np.outer(k[0, 0], x)[None, None]
    _, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    lam = 1.0 - np.sum(b[0, 0] * k[0, 0] ** 2)
    assert close(ST[0, 0], lam * S0[0, 0])
    assert -1.0 < lam < 1.0                      # b in (0,2), |k| = 1: negative eigenvalue allowed


def test_erase_fixes_directions_orthogonal_to_gated_key():
    """E x = x when (b.k)^T x = 0, and q^T E = q^T when q^T k = 0 (E = I - k (b.k)^T)."""
    rng = np.random.default_rng(10)
    dk, dv = 6, 3
    q, k, v, la, b, w = rand_case(rng, 1, dk=dk, dv=dv)
    la[:] = 0.0
    w[:] = 0.0
    bk = b[0, 0] * k[0, 0]
    x = rng.standard_normal(dk)
    x -= bk * (x @ bk) / (bk @ bk)
    S0 = np.outer(x, rng.standard_normal(dv))[None, None]
    _, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    assert close(ST[0, 0], S0[0, 0])
    qq = rng.standard_normal(dk)
    qq -= k[0, 0] * (qq @ k[0, 0])
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, _ = oracle.recurrent(qq[None, None], k, v, la, b, w, S0=S0)
    assert close(o[0, 0], S0[0, 0].T @ qq)


# ---- P8: linearity in (w.v, S0); only the product w.v matters --------------------------

def test_linearity_and_write_gate_product():
    rng = np.random.default_rng(11)
    T, dk, dv = 15, 5, 4
    q, k, v1, la, b, w = rand_case(rng, T, dk=dk, dv=dv)
    v2 = rng.standard_normal(v1.shape)
    S1, S2 = rng.standard_normal((2, 1, 1, dk, dv))
    c = -1.7
    o1, T1 = oracle.recurrent(q, k, v1, la, b, w, S0=S1)
    o2, T2 = oracle.recurrent(q, k, v2, la, b, w, S0=S2)
    o3, T3 = oracle.recurrent(q, k, v1 + c * v2, la, b, w, S0=S1 + c * S2)
    assert close(o3, o1 + c * o2, 1e-10) and close(T3, T1 + c * T2, 1e-10)
    o4, T4 = oracle.recurrent(q, k, v1 / 3.0, la, b, w * 3.0, S0=S1)
    assert close(o4, o1, 1e-12) and close(T4, T1, 1e-12)


# ---- P9: split / resume, packing, decode steps ------------------------------------------

def test_split_resume_pack_and_decode_steps():
    rng = np.random.default_rng(12)
    T, dk, dv = 23, 4, 5
    q, k, v, la, b, w = rand_case(rng, T, Hk=1, Hv=3, dk=dk, dv=dv)
    S0 = rng.standard_normal((1, 3, dk, dv))
    o, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    t = 9
    oa, Sa = oracle.recurrent(q[:t], k[:t], v[:t], la[:t], b[:t], w[:t], S0=S0)
    ob, Sb = oracle.recurrent(q[t:], k[t:], v[t:], la[t:], b[t:], w[t:], S0=Sa)
    assert close(np.concatenate([oa, ob]), o) and close(Sb, ST)
    # decode: T single steps with the state carried
    S = S0.copy()
    for i in range(T):
        oi, S = oracle.decode_step(q[i:i + 1], k[i:i + 1], v[i:i + 1], la[i:i + 1],
                                   b[i:i + 1], w[i:i + 1], S)
        assert close(oi[0], o[i])
    assert close(S, ST)
    # packing two sequences equals two separate calls
    cu = np.array([0, t, T])
    S0p = np.concatenate([S0, rng.standard_normal((1, 3, dk, dv))])
    op, Sp = oracle.recurrent(q, k, v, la, b, w, S0=S0p, cu_seqlens=cu)
    assert close(op[:t], oa) and close(Sp[0], Sa[0])
    oc, Sc = oracle.recurrent(q[t:], k[t:], v[t:], la[t:], b[t:], w[t:], S0=S0p[1:])
    assert close(op[t:], oc) and close(Sp[1], Sc[0])


def test_gva_value_head_reads_key_head_group():
    """Value head h uses key head h // (H_v / H_k): contiguous groups."""
    rng = np.random.default_rng(13)
    T, dk, dv = 7, 4, 3
    q, k, v, la, b, w = rand_case(rng, T, Hk=2, Hv=6, dk=dk, dv=dv)
    o, ST = oracle.recurrent(q, k, v, la, b, w)
    for h in range(6):
        hk = h // 3
        oh, Sh = oracle.recurrent(q[:, hk:hk + 1], k[:, hk:hk + 1], v[:, h:h + 1],
                                  la[:, h:h + 1], b[:, h:h + 1], w[:, h:h + 1])
        assert close(o[:, h], oh[:, 0]) and close(ST[0, h], Sh[0, 0])


# ---- P10: boundedness over a long run with the negative-eigenvalue gates ----------------

def test_state_stays_bounded():
    rng = np.random.default_rng(14)
    T, d = 3000, 8
    q, k, v, la, b, w = rand_case(rng, T, dk=d, dv=d, b_scale=2.0)
    o, ST = oracle.recurrent(q, k, v, la, b, w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(ST))
    assert np.max(np.abs(ST)) < 100.0


def test_identity_token_leaves_state_unchanged():
    """k = 0, w.v = 0, log alpha = 0 is the identity step (used for padding)."""
    rng = np.random.default_rng(15)
    q, k, v, la, b, w = rand_case(rng, 1, dk=4, dv=6)
    k[:] = 0.0
    la[:] = 0.0
    w[:] = 0.0
    S0 = rng.standard_normal((1, 1, 4, 6))
    o, ST = oracle.recurrent(q, k, v, la, b, w, S0=S0)
    assert close(ST, S0, 0.0)
    assert close(o[0, 0], S0[0, 0].T @ q[0, 0])


# ---- the recurrent cache: slots, padding entries, bf16-stored states ---------------------
# (GDN decode verify page, LocalAI mirror: section 2 for the slot cache read and written back
# every step, section 4 for a bf16 state)

def test_round_to_bf16_closed_forms_and_torch_cast():
    """Round-to-nearest-even onto 8 significant bits, fp32's exponent range."""
    import torch
    r = oracle.round_to_bf16
    # spacing 2^-7 on [1, 2): a half-way point goes to the even neighbour
    assert r(1.0 + 2.0 ** -8) == 1.0
    assert r(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert r(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2.0 ** -6)
    assert r(3.0 * 2.0 ** 100) == 3.0 * 2.0 ** 100          # exactly representable
    assert r(2.0 ** -133) == 2.0 ** -133                    # smallest subnormal
    assert r(2.0 ** -135) == 0.0
    assert r(0.0) == 0.0 and np.isinf(r(3.4e38)) and np.isnan(r(np.nan))
    # an independent implementation: torch's fp32 -> bf16 cast, on fp32 inputs
    x = np.random.default_rng(16).standard_normal(20000).astype(np.float32)
    x *= np.float32(2.0) ** np.random.default_rng(17).integers(-60, 60, 20000).astype(np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(r(x.astype(np.float64)), t)


def cache_case(rng, N, T, Hk=1, Hv=2, dk=4, dv=3, slots=7):
    q, k, v, la, b, w = (x.reshape(N, T, *x.shape[1:]) for x in
                         rand_case(rng, N * T, Hk=Hk, Hv=Hv, dk=dk, dv=dv))
    pool = rng.standard_normal((slots, Hv, dk, dv))
    return q, k, v, la, b, w, pool


def test_cache_slots_follow_the_index_and_padding_is_inert():
    rng = np.random.default_rng(18)
    N, T = 5, 4
    q, k, v, la, b, w, pool = cache_case(rng, N, T)
    idx = np.array([6, 1, -1, 3, 7])          # -1 and 7 (>= 7 slots) are padding entries
    o, new = oracle.recurrent_cache(q, k, v, la, b, w, pool, idx)
    for n, s in enumerate(idx):
        if 0 <= s < 7:
            on, Sn = oracle.recurrent(q[n], k[n], v[n], la[n], b[n], w[n], S0=pool[s:s + 1])
            assert close(o[n], on) and close(new[s], Sn[0])
        else:
            assert np.all(o[n] == 0.0)
    for s in (0, 2, 4, 5):                     # slots no sequence names are unchanged
        assert np.array_equal(new[s], pool[s])
    # permuting the sequences together with their slots permutes nothing else
    perm = np.array([3, 0, 4, 2, 1])
    o2, new2 = oracle.recurrent_cache(q[perm], k[perm], v[perm], la[perm], b[perm], w[perm],
                                      pool, idx[perm])
    assert close(o2, o[perm]) and close(new2, new)


def test_cache_multi_token_equals_single_token_calls():
    """T tokens in one call equal T calls of one token with the pool carried (fp32 pool)."""
    rng = np.random.default_rng(19)
    N, T = 3, 6
    q, k, v, la, b, w, pool = cache_case(rng, N, T, Hk=1, Hv=3, dk=5, dv=4)
    idx = np.array([2, 0, 5])
    o, new = oracle.recurrent_cache(q, k, v, la, b, w, pool, idx)
    P = pool
    for t in range(T):
        sl = slice(t, t + 1)
        ot, P = oracle.recurrent_cache(q[:, sl], k[:, sl], v[:, sl], la[:, sl], b[:, sl],
                                       w[:, sl], P, idx)
        assert close(ot[:, 0], o[:, t])
    assert close(P, new)


def test_cache_bf16_pool_rounds_only_the_stored_state():
    rng = np.random.default_rng(20)
    N, T = 2, 5
    q, k, v, la, b, w, pool = cache_case(rng, N, T, dk=6, dv=4, slots=3)
    pool = oracle.round_to_bf16(pool)          # a bf16 pool holds bf16 values
    o32, new32 = oracle.recurrent_cache(q, k, v, la, b, w, pool, None)
    o16, new16 = oracle.recurrent_cache(q, k, v, la, b, w, pool, None, bf16_state=True)
    assert np.array_equal(o16, o32)            # outputs inside the call see the fp64 state
    assert np.array_equal(new16[:N], oracle.round_to_bf16(new32[:N]))
    assert np.array_equal(new16[N:], pool[N:])
    rel = np.abs(new16[:N] - new32[:N]) / np.maximum(np.abs(new32[:N]), 1e-30)
    assert np.max(rel) <= 2.0 ** -8            # half a unit in the last place of 8 bits


# ---- the stages around the recurrence (burn-gdn2 "Architecture": L2-Norm before it, Gated
# RMS Norm with a SiLU gate after it) --------------------------------------------------------

def test_l2_normalize_closed_forms():
    assert np.allclose(oracle.l2_normalize([3.0, 4.0], 0.0), [0.6, 0.8], rtol=0, atol=1e-15)
    assert np.allclose(oracle.l2_normalize([3.0, 4.0], 11.0), [0.5, 4.0 / 6.0], rtol=0,
                       atol=1e-15)                       # sqrt(25 + 11) = 6
    x = np.random.default_rng(21).standard_normal((50, 7))
    n = oracle.l2_normalize(x, 0.0)
    assert np.allclose(np.linalg.norm(n, axis=-1), 1.0, rtol=0, atol=1e-14)
    assert np.allclose(oracle.l2_normalize(5.5 * x, 0.0), n, rtol=0, atol=1e-14)
    assert np.all(oracle.l2_normalize(np.zeros(4), 1e-6) == 0.0)


def test_gated_rms_norm_closed_forms():
    ln3 = np.log(3.0)                                    # sigmoid(ln 3) = 3/4
    out = oracle.gated_rms_norm([2.0, -2.0], [0.0, ln3], [5.0, 7.0], 0.0)
    assert np.allclose(out, [0.0, -7.0 * 0.75 * ln3], rtol=0, atol=1e-14)
    # mean square 4 + eps 5 -> rms 3
    out = oracle.gated_rms_norm([2.0, 2.0, 2.0, 2.0], [ln3] * 4, [1.0, 2.0, 3.0, 4.0], 5.0)
    assert np.allclose(out, np.array([1.0, 2.0, 3.0, 4.0]) * (2.0 / 3.0) * 0.75 * ln3,
                       rtol=0, atol=1e-14)
    # with eps = 0 the output divided by weight * silu(gate) has unit root-mean-square
    rng = np.random.default_rng(22)
    o, g = rng.standard_normal((40, 9)), rng.standard_normal((40, 9))
    w = rng.uniform(0.5, 2.0, 9)
    r = oracle.gated_rms_norm(o, g, w, 0.0) / (w * g / (1.0 + np.exp(-g)))
    assert np.allclose(np.sqrt(np.mean(r * r, axis=-1)), 1.0, rtol=0, atol=1e-12)
    # and it is invariant to a positive scale of o
    assert np.allclose(oracle.gated_rms_norm(3.0 * o, g, w, 0.0),
                       oracle.gated_rms_norm(o, g, w, 0.0), rtol=0, atol=1e-13)


def test_short_conv_closed_forms_and_library_convolution():
    rng = np.random.default_rng(23)
    T, C = 9, 5
    x, st = rng.standard_normal((T, C)), rng.standard_normal((3, C))
    eye = np.zeros((C, 4))
    eye[:, 3] = 1.0                                       # tap 3: the current token
    y, ns = oracle.short_conv(x, eye, st)
    assert np.array_equal(y, x) and np.array_equal(ns, x[-3:])
    back = np.zeros((C, 4))
    back[:, 0] = 1.0                                      # tap 0: three tokens back
    y, _ = oracle.short_conv(x, back, st)
    assert np.array_equal(y[:3], st) and np.array_equal(y[3:], x[:-3])
    # against numpy's convolution (a library routine) channel by channel
    w = rng.standard_normal((C, 4))
    y, _ = oracle.short_conv(x, w, st)
    xx = np.concatenate([st, x])
    for c in range(C):
        assert np.allclose(y[:, c], np.convolve(xx[:, c], w[c, ::-1], mode="valid"),
                           rtol=0, atol=1e-13)
    # a short call keeps older state entries: T = 2 shifts the state by two
    y2, ns2 = oracle.short_conv(x[:2], w, st)
    assert np.array_equal(ns2, np.concatenate([st[2:], x[:2]]))
    # split and resume with the state carried equals one call; SiLU closed form
    ya, sa = oracle.short_conv(x[:4], w, st)
    yb, sb = oracle.short_conv(x[4:], w, sa)
    yf, sf = oracle.short_conv(x, w, st)
    assert np.allclose(np.concatenate([ya, yb]), yf, rtol=0, atol=1e-14) and np.array_equal(sb, sf)
    one = np.zeros((1, 4))
    one[0, 3] = np.log(3.0)
    ys, _ = oracle.short_conv([[1.0]], one, np.zeros((3, 1)), silu=True)
    assert abs(ys[0, 0] - 0.75 * np.log(3.0)) < 1e-15


def test_conv_qkv_channel_order_and_padding():
    rng = np.random.default_rng(24)
    N, T, Hk, Hv, dk, dv = 3, 4, 1, 2, 2, 3
    q, k = rng.standard_normal((N, T, Hk, dk)), rng.standard_normal((N, T, Hk, dk))
    v = rng.standard_normal((N, T, Hv, dv))
    C = 2 * Hk * dk + Hv * dv
    w = np.zeros((C, 4))
    w[:, 3] = np.arange(1, C + 1)                         # channel c scaled by c + 1
    pool = rng.standard_normal((4, 3, C))
    qo, ko, vo, npool = oracle.conv_qkv(q, k, v, w, pool, [2, -1, 0])
    assert np.array_equal(qo[0], q[0] * np.array([1.0, 2.0]))
    assert np.array_equal(ko[0], k[0] * np.array([3.0, 4.0]))
    assert np.array_equal(vo[0], v[0] * np.arange(5, 11).reshape(2, 3))
    assert np.array_equal(qo[1], q[1]) and np.array_equal(npool[1], pool[1])   # padding
    assert np.array_equal(npool[3], pool[3])
    x2 = np.concatenate([q[2].reshape(T, -1), k[2].reshape(T, -1), v[2].reshape(T, -1)], 1)
    assert np.array_equal(npool[0], x2[-3:])


# ---- the gradient of the recurrence (oracle.recurrent_bwd) --------------------------------

def _loss_parts(rng, T, Hv, dv, N, dk):
    return rng.standard_normal((T, Hv, dv)), rng.standard_normal((N, Hv, dk, dv))


def test_recurrent_bwd_matches_central_differences():
    """Every gradient against central differences of L = sum(o . R) + sum(S_T . R2), on two
    packed sequences with grouped value heads (2 value heads over 1 key head)."""
    rng = np.random.default_rng(30)
    T, Hk, Hv, dk, dv = 7, 1, 2, 3, 2
    q, k, v, la, b, w = rand_case(rng, T, Hk=Hk, Hv=Hv, dk=dk, dv=dv)
    cu = [0, 3, 7]
    S0 = rng.standard_normal((2, Hv, dk, dv))
    R, R2 = _loss_parts(rng, T, Hv, dv, 2, dk)
    ins = {"q": q, "k": k, "v": v, "log_alpha": la, "b": b, "w": w, "S0": S0}

    def loss(x):
        o, ST = oracle.recurrent(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"],
                                 S0=x["S0"], cu_seqlens=cu, threads=1)
        return float(np.sum(o * R) + np.sum(ST * R2))

    gr = oracle.recurrent_bwd(q, k, v, la, b, w, R, S0=S0, dS_T=R2, cu_seqlens=cu, threads=1)
    names = {"q": "dq", "k": "dk", "v": "dv", "log_alpha": "dlog_alpha", "b": "db", "w": "dw",
             "S0": "dS0"}
    eps = 1e-6
    for nm, gname in names.items():
        num = np.zeros_like(ins[nm])
        for idx in np.ndindex(ins[nm].shape):
            xp = {a: c.copy() for a, c in ins.items()}
            xm = {a: c.copy() for a, c in ins.items()}
            xp[nm][idx] += eps
            xm[nm][idx] -= eps
            num[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        assert np.allclose(gr[gname], num, rtol=1e-6, atol=1e-7), nm


@pytest.mark.parametrize("C", [1, 4, 7, 23, 64])
def test_chunked_bwd_equals_token_adjoint(C):
    """The gradient through the chunked WY form (oracle.chunked_sequence_bwd: dU, dS, dMqk,
    dT, dA and the chain rule through the decay factors) equals the token-by-token adjoint
    of the recurrence, which the finite-difference and autograd pins fix. Chunk sizes: one
    token, exact multiples, a ragged tail, one chunk, and a chunk longer than the sequence;
    erase gates up to 2 (negative eigenvalues) and d_k != d_v."""
    rng = np.random.default_rng(40 + C)
    T, dk, dv = 23, 5, 3
    q, k, v, la, b, w = (x[:, 0] for x in rand_case(rng, T, dk=dk, dv=dv))
    S0 = rng.standard_normal((dk, dv))
    do = rng.standard_normal((T, dv))
    for dST in (None, rng.standard_normal((dk, dv))):
        ref = oracle.sequence_bwd(q, k, v, w, la, b, S0, do, dST)
        got = oracle.chunked_sequence_bwd(q, k, v, w, la, b, S0, do, dST, C)
        for name in ref:
            assert close(got[name], ref[name], 1e-10), (C, name)


def test_recurrent_bwd_matches_torch_autograd_across_checkpoints():
    """An independent evaluation: torch autograd in fp64 through a plain loop of the
    recurrence, at T = 150 (the oracle recomputes states from checkpoints every 64 tokens)."""
    import torch
    rng = np.random.default_rng(31)
    T, dk, dv = 150, 5, 4
    q, k, v, la, b, w = rand_case(rng, T, dk=dk, dv=dv)
    S0 = rng.standard_normal((1, 1, dk, dv))
    R, R2 = _loss_parts(rng, T, 1, dv, 1, dk)
    gr = oracle.recurrent_bwd(q, k, v, la, b, w, R, S0=S0, dS_T=R2, threads=1)
    t = {n: torch.tensor(x[:, 0], dtype=torch.float64, requires_grad=True)
         for n, x in (("q", q), ("k", k), ("v", v), ("la", la), ("b", b), ("w", w))}
    S = torch.tensor(S0[0, 0], dtype=torch.float64, requires_grad=True)
    S_in = S
    loss = torch.zeros((), dtype=torch.float64)
    Rt, R2t = torch.tensor(R[:, 0]), torch.tensor(R2[0, 0])
    for i in range(T):
        kk, qq = t["k"][i], t["q"][i]
        P = (torch.eye(dk, dtype=torch.float64) - torch.outer(kk, t["b"][i] * kk)) @ \
            torch.diag(torch.exp(t["la"][i]))
        S = P @ S + torch.outer(kk, t["w"][i] * t["v"][i])
        loss = loss + (S.T @ qq) @ Rt[i]
    loss = loss + torch.sum(S * R2t)
    loss.backward()
    pairs = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("la", "dlog_alpha"), ("b", "db"),
             ("w", "dw"))
    for n, gname in pairs:
        assert np.allclose(gr[gname][:, 0], t[n].grad.numpy(), rtol=1e-9, atol=1e-10), n
    assert np.allclose(gr["dS0"][0, 0], S_in.grad.numpy(), rtol=1e-9, atol=1e-10)


# ---- variant rules (oracle.variant_sequence): KDA, scalar-decay GDN, FG2-GDN, FG2-GDN+ ---

def variant_case(rng, T, dk, dv, mode):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((T,) if mode == "gdn" else (T, dk)))
    sig = lambda x: 1.0 / (1.0 + np.exp(-x))  # noqa: E731
    beta = sig(rng.standard_normal((T,) if mode in ("kda", "gdn") else (T, dk)))
    beta_v = sig(rng.standard_normal((T, dv))) if mode == "fg2+" else None
    return q, k, v, la, beta, beta_v


@pytest.mark.parametrize("mode", ["kda", "gdn", "fg2", "fg2+"])
def test_variant_rules_match_explicit_matrices(mode):
    """Each variant's update as explicit d_k x d_k matrices: (I - k~ e~^T) D S + k~ u~^T with
    (KDA, GDN) e~ = beta k, k~ = k, u~ = beta v; (FG2) k~ = e~ = sqrt(beta) k, u~ = sqrt(beta) v;
    (FG2+) k~ = e~ = sqrt(beta) k, u~ = sqrt(beta_v) v."""
    rng = np.random.default_rng(31)
    T, dk = 9, 5
    dv = dk if mode == "fg2" else 3
    q, k, v, la, beta, beta_v = variant_case(rng, T, dk, dv, mode)
    S0 = rng.standard_normal((dk, dv))
    o, ST = oracle.variant_sequence(mode, q, k, v, la, beta, S0, beta_v)
    S = S0.copy()
    for t in range(T):
        D = np.diag(np.exp(la[t]) * np.ones(dk))
        if mode in ("kda", "gdn"):
            kt, et, ut = k[t], beta[t] * k[t], beta[t] * v[t]
        else:
            kt = et = np.sqrt(beta[t]) * k[t]
            ut = (np.sqrt(beta[t]) if mode == "fg2" else np.sqrt(beta_v[t])) * v[t]
        S = (np.eye(dk) - np.outer(kt, et)) @ D @ S + np.outer(kt, ut)
        assert close(o[t], S.T @ q[t])
    assert close(ST, S)


def test_variant_kda_exact_retrieval():
    """alpha = 1, beta = 1, unit keys: each token's key retrieves its value, k_t^T S_t = v_t."""
    rng = np.random.default_rng(32)
    T, dk, dv = 12, 6, 4
    q, k, v, _, _, _ = variant_case(rng, T, dk, dv, "kda")
    for t in range(1, T + 1):
        _, S = oracle.variant_sequence("kda", q[:t], k[:t], v[:t], np.zeros((t, dk)),
                                       np.ones(t), rng.standard_normal((dk, dv)))
        assert close(k[t - 1] @ S, v[t - 1])


def test_variant_gdn_beta_zero_closed_form():
    """beta = 0: nothing is erased or written, S_t = (prod_{i<=t} alpha_i) S_0."""
    rng = np.random.default_rng(33)
    T, dk, dv = 7, 5, 3
    q, k, v, la, _, _ = variant_case(rng, T, dk, dv, "gdn")
    S0 = rng.standard_normal((dk, dv))
    o, ST = oracle.variant_sequence("gdn", q, k, v, la, np.zeros(T), S0)
    for t in range(T):
        assert close(o[t], np.exp(np.sum(la[:t + 1])) * (S0.T @ q[t]))
    assert close(ST, np.exp(np.sum(la)) * S0)


@pytest.mark.parametrize("mode", ["kda", "gdn"])
def test_variant_kda_gdn_are_gdn2_with_scalar_gates(mode):
    """The burn-gdn2 page's channel-wise b and w replace KDA's scalar gate: with b = w = beta
    in every channel (and, for GDN, log alpha in every channel) the C oracle of GDN-2 gives
    the variant's outputs."""
    rng = np.random.default_rng(34)
    T, dk, dv = 10, 6, 4
    q, k, v, la, beta, _ = variant_case(rng, T, dk, dv, mode)
    S0 = rng.standard_normal((dk, dv))
    o, ST = oracle.variant_sequence(mode, q, k, v, la, beta, S0)
    la2 = np.broadcast_to(la[:, None], (T, dk)) if mode == "gdn" else la
    b = np.broadcast_to(beta[:, None], (T, dk))
    w = np.broadcast_to(beta[:, None], (T, dv))
    o2, S2 = oracle.sequence(q, k, v, w, la2, b, S0)
    assert close(o, o2) and close(ST, S2)


def test_variant_fg2_plus_with_equal_scales_is_fg2():
    rng = np.random.default_rng(35)
    T, d = 8, 5
    q, k, v, la, beta, _ = variant_case(rng, T, d, d, "fg2")
    S0 = rng.standard_normal((d, d))
    o1, S1 = oracle.variant_sequence("fg2", q, k, v, la, beta, S0)
    o2, S2 = oracle.variant_sequence("fg2+", q, k, v, la, beta, S0, beta_v=beta)
    assert close(o1, o2) and close(S1, S2)


# ---- the gate mappings onto GDN-2 inputs and their chain rule (oracle.map_gates[_bwd]) ---

@pytest.mark.parametrize("mode", ["kda", "gdn", "fg2", "fg2+"])
def test_map_gates_gives_the_variant(mode):
    """The GDN-2 recurrence on the mapped inputs is the variant's own update rule."""
    rng = np.random.default_rng(36)
    T, dk = 9, 5
    dv = dk if mode == "fg2" else 3
    q, k, v, la, beta, beta_v = variant_case(rng, T, dk, dv, mode)
    S0 = rng.standard_normal((dk, dv))
    o, ST = oracle.variant_sequence(mode, q, k, v, la, beta, S0, beta_v)
    q2, k2, v2, la2, b, w = oracle.map_gates(mode, q, k, v, la, beta, beta_v)
    o2, S2 = oracle.sequence(q2, k2, v2, w, la2, b, S0)
    assert close(o, o2) and close(ST, S2)


@pytest.mark.parametrize("mode", ["kda", "gdn", "fg2", "fg2+"])
def test_map_gates_bwd_matches_finite_differences(mode):
    """Gradients of L = <dO, o> + <dS_T, S_T> of the variant with respect to each of its own
    inputs: the composition map_gates -> sequence_bwd -> map_gates_bwd against central
    differences of variant_sequence (the variant's own rule), every element."""
    rng = np.random.default_rng(37)
    T, dk = 4, 3
    dv = dk if mode == "fg2" else 2
    q, k, v, la, beta, beta_v = variant_case(rng, T, dk, dv, mode)
    S0 = rng.standard_normal((dk, dv))
    dO = rng.standard_normal((T, dv))
    dST = rng.standard_normal((dk, dv))
    m = oracle.map_gates(mode, q, k, v, la, beta, beta_v)
    gm = oracle.sequence_bwd(m[0], m[1], m[2], m[5], m[3], m[4], S0, dO, dST)
    got = oracle.map_gates_bwd(mode, q, k, v, la, beta, gm, beta_v)
    x = {"q": q, "k": k, "v": v, "log_alpha": la, "beta": beta}
    if mode == "fg2+":
        x["beta_v"] = beta_v

    def loss(xx):
        o, ST = oracle.variant_sequence(mode, xx["q"], xx["k"], xx["v"], xx["log_alpha"],
                                        xx["beta"], S0, xx.get("beta_v"))
        return float(np.sum(dO * o) + np.sum(dST * ST))

    eps = 1e-6
    for name in x:
        fd = np.zeros_like(x[name])
        for idx in np.ndindex(x[name].shape):
            xp = {n: a.copy() for n, a in x.items()}
            xm = {n: a.copy() for n, a in x.items()}
            xp[name][idx] += eps
            xm[name][idx] -= eps
            fd[idx] = (loss(xp) - loss(xm)) / (2 * eps)
        g = got["d" + name]
        assert g.shape == fd.shape, name
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-7), (name, np.abs(g - fd).max())


# ---- the parity metric and the key-head map of the variant rules ---------------------------

def test_rel_l2_closed_forms():
    """rel_l2 is ||x - ref||_2 / ||ref||_2 over every element at once (the parity gate of the
    spec tolerance): closed forms on small vectors, and the absolute norm when the
    reference is zero."""
    assert abs(oracle.rel_l2([1.0, 0.0], [0.0, 1.0]) - np.sqrt(2.0)) < 1e-15
    assert abs(oracle.rel_l2([3.0, 4.0], [0.0, 0.0]) - 5.0) < 1e-15
    assert oracle.rel_l2([0.0, 0.0], [0.0, 0.0]) == 0.0
    rng = np.random.default_rng(41)
    x = rng.standard_normal((7, 5))
    assert abs(oracle.rel_l2(2.0 * x, x) - 1.0) < 1e-14
    assert oracle.rel_l2(x, x) == 0.0
    # one norm over all elements, not a mean or maximum of per-row errors
    ref = np.array([[1.0, 0.0], [0.0, 1.0]])
    assert abs(oracle.rel_l2([[1.0, 0.0], [0.0, 2.0]], ref) - 1.0 / np.sqrt(2.0)) < 1e-15
    assert abs(oracle.rel_l2([[1.0, 0.0], [0.0, 0.0]], ref) - 1.0 / np.sqrt(2.0)) < 1e-15
    # a perturbation of norm eps * ||ref|| reads eps, at both gates
    u = rng.standard_normal(x.shape)
    u *= np.linalg.norm(x) / np.linalg.norm(u)
    for eps in (1e-4, 2e-2):
        assert abs(oracle.rel_l2(x + eps * u, x) - eps) < 1e-12
    # scale invariance
    y = x + 1e-3 * u
    assert abs(oracle.rel_l2(1e6 * y, 1e6 * x) - oracle.rel_l2(y, x)) < 1e-12


def test_variant_value_head_reads_key_head_group():
    """variant(): value head h reads key head h // (H_v / H_k) (contiguous groups). Value heads
    0, 1 and 3 get identical value-side inputs; with 6 value heads over 2 key heads, heads 0
    and 1 must then agree exactly (both read key head 0) while head 3 must not (it reads key
    head 1). The
    multi-head call also equals the C oracle of GDN-2 (its own head map, pinned above against
    single-head calls) with KDA's b = w = beta in every channel."""
    rng = np.random.default_rng(42)
    N, T, Hk, Hv, dk, dv = 2, 9, 2, 6, 5, 3
    q = rng.standard_normal((N, T, Hk, dk))
    k = rng.standard_normal((N, T, Hk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, T, Hv, dv))
    la = -np.logaddexp(0.0, rng.standard_normal((N, T, Hv, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, T, Hv))))
    S0 = rng.standard_normal((N, Hv, dk, dv))
    for arr in (v, la, beta):
        arr[:, :, 1] = arr[:, :, 0]
        arr[:, :, 3] = arr[:, :, 0]
    S0[:, 1] = S0[:, 0]
    S0[:, 3] = S0[:, 0]
    o, ST = oracle.variant("kda", q, k, v, la, beta, S0=S0)
    assert np.array_equal(o[:, :, 1], o[:, :, 0]) and np.array_equal(ST[:, 1], ST[:, 0])
    assert np.max(np.abs(o[:, :, 3] - o[:, :, 0])) > 1e-3
    b = np.broadcast_to(beta[..., None], (N, T, Hv, dk))
    w = np.broadcast_to(beta[..., None], (N, T, Hv, dv))
    flat = lambda a: np.ascontiguousarray(a).reshape(N * T, *a.shape[2:])  # noqa: E731
    o2, S2 = oracle.recurrent(flat(q), flat(k), flat(v), flat(la), flat(b), flat(w), S0=S0,
                              cu_seqlens=np.arange(N + 1) * T)
    assert close(o.reshape(N * T, Hv, dv), o2) and close(ST, S2)
