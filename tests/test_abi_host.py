"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments before touching a device.

Every call made here fails host validation by construction (a NULL dims, a bad shape, a
too-small workspace, ...), so no kernel is ever launched and no device is needed.
"""
import ctypes
import os
import re
import subprocess

import pytest

import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import Dims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")
FAKE = ctypes.c_void_p(0x1000)       # never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(g.LIB_PATH):
        from gated_delta_rule_gdn_amd import build
        build.build()
    return g.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert {"gdn2_chunk_fwd", "gdn2_recurrent_step", "gdn2_recurrent_fwd",
            "gdn2_chunk_fwd_workspace_bytes"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", g.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdn2_\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(L, n)


def test_version_and_status_strings(L):
    assert L.gdn2_abi_version() == 9
    assert L.gdn2_status_string(0) == b"ok"
    assert b"workspace" in L.gdn2_status_string(4)
    assert L.gdn2_status_string(99) == b"unknown status"


def chunk(L, dims, chunk_size=64, ws=FAKE, ws_bytes=1 << 40, cu=None, o=FAKE, q=FAKE,
          fusion=None):
    # o defaults to the q pointer: a call that passed every other check is still rejected
    return L.gdn2_chunk_fwd(q, FAKE, FAKE, FAKE, FAKE, FAKE, None, cu, chunk_size, o, None,
                            None if dims is None else ctypes.byref(dims), ws, ws_bytes, fusion,
                            None)


def test_chunk_fwd_rejects_bad_arguments(L):
    ok = dict(batch=2, seqlen=100, num_seqs=0, h_k=2, h_v=4, d_k=128, d_v=128, dtype=1)
    assert chunk(L, None) == 1
    assert b"dims" in L.gdn2_last_error()
    assert chunk(L, Dims(**{**ok, "dtype": 7})) == 3
    assert chunk(L, Dims(**{**ok, "h_v": 5})) == 2
    assert chunk(L, Dims(**{**ok, "h_k": 0})) == 2
    assert chunk(L, Dims(**{**ok, "d_k": 96})) == 3
    assert chunk(L, Dims(**{**ok, "d_v": 0})) == 2
    assert chunk(L, Dims(**ok), chunk_size=16) == 3           # built: 32, 64 and 128
    assert chunk(L, Dims(**ok), chunk_size=96) == 3
    assert chunk(L, Dims(**ok), chunk_size=0) == 2
    assert chunk(L, Dims(**{**ok, "seqlen": -1})) == 2
    assert chunk(L, Dims(**{**ok, "batch": 0})) == 2
    for cs in (32, 64, 128):                                  # valid: stopped at o aliasing q
        assert chunk(L, Dims(**{**ok, "dtype": 0}), chunk_size=cs) == 2
        assert chunk(L, Dims(**ok), chunk_size=cs) == 2
    assert chunk(L, Dims(**ok), q=None) == 1
    assert chunk(L, Dims(**ok), ws=None) == 4
    assert chunk(L, Dims(**ok), ws_bytes=1024) == 4
    assert chunk(L, Dims(**ok), ws=ctypes.c_void_p(0x1010)) == 4   # not 256-byte aligned
    assert chunk(L, Dims(**ok), o=FAKE, q=FAKE) == 2                # o aliases q
    # packed batches need batch = 1 and num_seqs >= 1
    assert chunk(L, Dims(**{**ok, "num_seqs": 3}), cu=FAKE) == 2
    assert chunk(L, Dims(**{**ok, "batch": 1, "num_seqs": 0}), cu=FAKE) == 2
    # too many tokens
    assert chunk(L, Dims(**{**ok, "batch": 1 << 20, "seqlen": 1 << 12})) == 2


def step(L, dims, S=FAKE, o=FAKE):
    # o defaults to the q pointer, so even a call that passed every other check would be
    # rejected by the aliasing check and never launch
    return L.gdn2_recurrent_step(FAKE, ctypes.c_void_p(0x3000), FAKE, FAKE, FAKE, FAKE, S, o,
                                 None if dims is None else ctypes.byref(dims), None)


def test_recurrent_step_rejects_bad_arguments(L):
    ok = dict(batch=4, seqlen=1, num_seqs=0, h_k=2, h_v=6, d_k=128, d_v=64, dtype=0)
    assert step(L, None) == 1
    assert step(L, Dims(**{**ok, "seqlen": 2})) == 2
    assert step(L, Dims(**{**ok, "h_v": 5})) == 2
    assert step(L, Dims(**{**ok, "d_v": 32})) == 3
    assert step(L, Dims(**{**ok, "dtype": 2})) == 3
    assert step(L, Dims(**{**ok, "batch": -1})) == 2
    assert step(L, Dims(**ok), S=None) == 1
    assert step(L, Dims(**ok), o=FAKE) == 2               # o aliases q
    assert step(L, Dims(**{**ok, "batch": 0})) == 0       # empty batch: nothing to do


def fwd(L, dims, state_dtype=0, idx=None, num_slots=8, S=FAKE, o=None, fusion=None):
    # o defaults to the q pointer: a call that passed every other check is still rejected
    return L.gdn2_recurrent_fwd(FAKE, ctypes.c_void_p(0x3000), FAKE, FAKE, FAKE, FAKE, S,
                                state_dtype, idx, num_slots, FAKE if o is None else o,
                                None if dims is None else ctypes.byref(dims),
                                None if fusion is None else ctypes.byref(fusion), None)


def test_fusion_options_are_validated(L):
    from gated_delta_rule_gdn_amd import Fusion
    okc = Dims(2, 100, 0, 2, 4, 128, 128, 1)
    okr = Dims(4, 3, 0, 2, 6, 128, 64, 1)
    W = ctypes.c_void_p(0x7000)
    bad = [(Fusion(1, -1.0, None, None, 0.0), 2),            # negative L2-norm epsilon
           (Fusion(1, float("nan"), None, None, 0.0), 2),
           (Fusion(0, 0.0, ctypes.c_void_p(0x6000), None, 1e-5), 1),   # gate without weight
           (Fusion(0, 0.0, ctypes.c_void_p(0x6000), W, -1.0), 2),      # negative norm epsilon
           (Fusion(0, 0.0, ctypes.c_void_p(0x6000), W, float("inf")), 2)]
    for f, want in bad:
        assert chunk(L, okc, fusion=f) == want
        assert fwd(L, okr, fusion=f) == want
    # a gate aliasing o
    assert chunk(L, okc, o=ctypes.c_void_p(0x6000), q=ctypes.c_void_p(0x4000),
                 fusion=Fusion(0, 0.0, ctypes.c_void_p(0x6000), W, 1e-5)) == 2
    assert fwd(L, okr, o=ctypes.c_void_p(0x6000),
               fusion=Fusion(0, 0.0, ctypes.c_void_p(0x6000), W, 1e-5)) == 2
    # the short convolution: recurrent forward only, and it needs its state
    CW, CS = ctypes.c_void_p(0x8000), ctypes.c_void_p(0x9000)
    assert chunk(L, okc, fusion=Fusion(0, 0.0, None, None, 0.0, CW, CS, 1)) == 3
    assert fwd(L, okr, fusion=Fusion(0, 0.0, None, None, 0.0, CW, None, 1)) == 1
    assert fwd(L, okr, o=CS, fusion=Fusion(0, 0.0, None, None, 0.0, CW, CS, 1)) == 2
    assert fwd(L, okr, fusion=Fusion(0, 0.0, None, None, 0.0, CW, CS, 1)) == 2   # o aliases q
    # valid options pass the fusion checks and are rejected later (o aliases q)
    good = Fusion(1, 1e-6, ctypes.c_void_p(0x6000), W, 1e-5)
    assert chunk(L, okc, fusion=good) == 2
    assert fwd(L, okr, fusion=good) == 2


def test_recurrent_fwd_rejects_bad_arguments(L):
    ok = dict(batch=4, seqlen=3, num_seqs=0, h_k=2, h_v=6, d_k=128, d_v=64, dtype=1)
    assert fwd(L, None) == 1
    assert fwd(L, Dims(**{**ok, "seqlen": 0})) == 2
    assert fwd(L, Dims(**{**ok, "h_v": 5})) == 2
    assert fwd(L, Dims(**{**ok, "d_k": 96})) == 3
    assert fwd(L, Dims(**ok), state_dtype=2) == 3
    assert fwd(L, Dims(**ok), num_slots=3) == 2            # no index: one slot per sequence
    assert fwd(L, Dims(**ok), num_slots=-1, idx=FAKE) == 2
    assert fwd(L, Dims(**ok), S=None) == 1
    assert fwd(L, Dims(**ok), idx=FAKE, num_slots=2) == 2   # o aliases q
    assert fwd(L, Dims(**ok), state_dtype=1, o=FAKE) == 2
    assert fwd(L, Dims(**ok), o=ctypes.c_void_p(0x5000), S=ctypes.c_void_p(0x5000)) == 2
    assert fwd(L, Dims(**{**ok, "batch": 0})) == 0          # empty batch: nothing to do


def test_workspace_size_formula(L):
    # per (chunk, value head) record: bf16 operands 2*(3*64*dk + 64*64 + 64*dv) + 4*dk,
    # rounded up to 256 bytes; dense batches hold B*ceil(T/64) chunks.
    d = Dims(2, 100, 0, 2, 4, 128, 128, 1)
    rec = (2 * (3 * 64 * 128 + 64 * 64 + 64 * 128) + 4 * 128 + 255) // 256 * 256
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == 2 * 2 * 4 * rec
    # packed: ceil(T/64) + N chunks, plus the chunk map [N + 1] and the state pass's
    # sequence order [N] (int32 each, 256-byte aligned)
    d = Dims(1, 1000, 5, 1, 2, 64, 64, 0)
    rec = (4 * (3 * 64 * 64 + 64 * 64 + 64 * 64) + 4 * 64 + 255) // 256 * 256
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == 512 + (16 + 5) * 2 * rec
    # a dense batch with few (sequence, head) pairs: the state pass is split into segments
    # (about 256 workgroups of two 16-column slices, at least 4 chunks per segment) and the
    # workspace adds fp32 states entering segments 0 and 1 [pair][2][dk][dv], transitions
    # [pair][nseg-2] (dk x dk, 4 bytes per element) and zero-start end states
    # [pair][nseg-2][dk][dv]
    def seg_bytes(pairs, nseg, dk, dv):
        a = lambda x: (x + 255) // 256 * 256       # noqa: E731
        return (a(pairs * 2 * dk * dv * 4) + a(pairs * (nseg - 2) * dk * dk * 4) +
                a(pairs * (nseg - 2) * dk * dv * 4))
    rec = (2 * (3 * 64 * 128 + 64 * 64 + 64 * 128) + 4 * 128 + 255) // 256 * 256
    d = Dims(1, 4096, 0, 16, 16, 128, 128, 1)       # 16 pairs x 64 chunks -> 4 segments
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == \
        64 * 16 * rec + seg_bytes(16, 4, 128, 128)
    d = Dims(1, 1000, 0, 1, 2, 128, 128, 1)         # 2 pairs x 16 chunks -> 4 segments
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == \
        16 * 2 * rec + seg_bytes(2, 4, 128, 128)
    d = Dims(2, 640, 0, 1, 3, 128, 128, 1)          # 6 pairs x 10 chunks -> 2 segments
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == \
        2 * 10 * 3 * rec + seg_bytes(6, 2, 128, 128)
    rec64 = (2 * (3 * 64 * 128 + 64 * 64 + 64 * 64) + 4 * 128 + 255) // 256 * 256
    d = Dims(1, 2000, 0, 2, 2, 128, 64, 1)          # 2 pairs x 32 chunks -> 8 segments
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == \
        32 * 2 * rec64 + seg_bytes(2, 8, 128, 64)
    d = Dims(8, 2048, 0, 8, 8, 128, 128, 1)         # 64 pairs: enough work, no segments
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == 8 * 32 * 8 * rec
    # chunk sizes 32 and 128, and fp32 records at d = 128: records of
    # E*(3*C*dk + C*C + C*dv) + 4*dk bytes; dense batches with few pairs add the same
    # segment area, planned for the panel state pass (two 16-column slices per workgroup at
    # these shapes: 16 pairs x 4 workgroups -> 4 segments)
    def rec_c(C, E, dk, dv):
        return (E * (3 * C * dk + C * C + C * dv) + 4 * dk + 255) // 256 * 256
    d = Dims(1, 4096, 0, 16, 16, 128, 128, 1)
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 128) == \
        32 * 16 * rec_c(128, 2, 128, 128) + seg_bytes(16, 4, 128, 128)
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 32) == \
        128 * 16 * rec_c(32, 2, 128, 128) + seg_bytes(16, 4, 128, 128)
    d = Dims(1, 4096, 0, 16, 16, 128, 128, 0)
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64) == \
        64 * 16 * rec_c(64, 4, 128, 128) + seg_bytes(16, 4, 128, 128)
    d = Dims(8, 4096, 0, 8, 8, 128, 128, 1)         # 64 pairs at chunk 128: no segments
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 128) == 8 * 32 * 8 * rec_c(128, 2, 128, 128)
    d = Dims(1, 1000, 5, 1, 2, 128, 64, 0)          # packed, fp32, 128-token chunks
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 128) == 512 + (8 + 5) * 2 * rec_c(128, 4, 128, 64)
    assert L.gdn2_chunk_fwd_workspace_bytes(None, 64) == 0
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(Dims(1, 10, 0, 1, 1, 96, 64, 1)),
                                            64) == 0


def test_cu_seqlens_host_check(L):
    def chk(vals, n, t):
        arr = (ctypes.c_int32 * len(vals))(*vals)
        return L.gdn2_check_cu_seqlens(arr, n, t)
    assert chk([0, 5, 5, 9], 3, 9) == 0
    assert chk([1, 5, 9], 2, 9) == 2
    assert chk([0, 5, 4], 2, 4) == 2
    assert chk([0, 5, 9], 2, 10) == 2
    assert L.gdn2_check_cu_seqlens(None, 2, 9) == 1


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 4, 1, 64)
    with pytest.raises(ValueError, match="GPU"):
        g.chunk_fwd(x, x, x, x, x, x)


def gates(L, mode, dims, q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, beta_v=FAKE, q_out=None,
          k_out=None, v_out=None, la_out=None, b_out=None, w_out=None):
    return L.gdn2_map_gates(mode, None if dims is None else ctypes.byref(dims), q, k, v, la,
                            beta, beta_v, q_out, k_out, v_out, la_out, b_out, w_out, None)


def test_map_gates_validation(L):
    """Every call here stops at host validation (each lacks exactly one requirement)."""
    P = [ctypes.c_void_p(0x2000 + 0x100 * i) for i in range(6)]    # distinct output pointers
    d = Dims(2, 10, 0, 2, 4, 64, 64, 1)
    assert gates(L, 1, None) == 1                                     # NULL dims
    assert gates(L, 0, d) == 3 and gates(L, 5, d) == 3                # not a gate mode
    assert gates(L, 1, Dims(2, 10, 0, 2, 4, 96, 64, 1)) == 3          # head dim not built
    assert gates(L, 1, Dims(2, 10, 0, 3, 4, 64, 64, 1)) == 2          # h_v % h_k != 0
    assert gates(L, 1, Dims(-1, 10, 0, 2, 4, 64, 64, 1)) == 2         # negative batch
    assert gates(L, 1, d, b_out=P[0]) == 1                            # KDA: w_out missing
    assert gates(L, 1, d, beta=None, b_out=P[0], w_out=P[1]) == 1     # KDA: beta missing
    assert gates(L, 4, d, b_out=P[0], w_out=P[1]) == 1                # GDN: log_alpha_out
    assert gates(L, 2, Dims(2, 10, 0, 2, 4, 128, 64, 1)) == 2         # FG2 needs d_v = d_k
    assert gates(L, 2, d, q_out=P[0], v_out=P[2], b_out=P[3], w_out=P[4]) == 1   # k_out
    assert gates(L, 2, d, k_out=P[1], v_out=P[2], b_out=P[3], w_out=P[4]) == 1   # q_out: h_v > h_k
    assert gates(L, 3, d, beta_v=None, q_out=P[0], k_out=P[1], b_out=P[3], w_out=P[4]) == 1
    assert gates(L, 1, d, b_out=FAKE, w_out=P[1]) == 2                # b_out aliases an input
    assert gates(L, 1, d, b_out=P[0], w_out=P[0]) == 2                # two outputs alike
    assert gates(L, 1, Dims(0, 10, 0, 2, 4, 64, 64, 1)) == 0          # no tokens: nothing to do


def test_gate_mode_validation(L):
    """gdn2_fusion.gate_mode: bad modes and combinations stop at host validation; the modes
    that derive w from b accept w = NULL (the call then stops at a later check)."""
    from gated_delta_rule_gdn_amd import Fusion
    d = Dims(1, 64, 0, 1, 1, 128, 128, 1)
    def call(mode, w=FAKE, qkn=0, dims=d, o=ctypes.c_void_p(0x9000)):
        fu = Fusion(qkn, 1e-6, None, None, 1e-5, None, None, 0, mode)
        return L.gdn2_chunk_fwd(FAKE, FAKE, FAKE, FAKE, FAKE, w, None, None, 64, o, None,
                                ctypes.byref(dims), FAKE, 1 << 40, ctypes.byref(fu), None)
    assert call(5) == 3 and call(-1) == 3                       # not a gate mode
    assert call(2, qkn=1) == 3 and call(3, qkn=1) == 3          # FG2 modes with the L2-norm
    assert call(2, dims=Dims(1, 64, 0, 1, 1, 128, 64, 1)) == 2  # FG2 needs d_v = d_k
    assert call(0, w=None) == 1 and call(3, w=None) == 1        # these modes need w
    assert call(1, w=None, o=FAKE) == 2                         # KDA: no w; then o aliases q


def test_chunk_states_validation(L):
    """gdn2_fusion.chunk_states: an output of the chunked forward only, and it may not alias
    an input, an output or the workspace (each call stops before any launch)."""
    from gated_delta_rule_gdn_amd import Fusion
    d = Dims(1, 64, 0, 1, 1, 128, 128, 1)
    O, WS = ctypes.c_void_p(0x9000), ctypes.c_void_p(0xA000)

    def chunk_call(cks, q=FAKE):
        fu = Fusion(0, 0.0, None, None, 0.0, None, None, 0, 0, cks)
        return L.gdn2_chunk_fwd(q, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 64, O, None,
                                ctypes.byref(d), WS, 1 << 40, ctypes.byref(fu), None)
    assert chunk_call(O) == 2                         # aliases o
    assert chunk_call(WS) == 2                        # aliases the workspace
    assert chunk_call(FAKE, q=ctypes.c_void_p(0xB000)) == 2   # aliases k (and v, b, ...)
    fu = Fusion(0, 0.0, None, None, 0.0, None, None, 0, 0, ctypes.c_void_p(0xC000))
    assert fwd(L, Dims(4, 3, 0, 2, 6, 128, 64, 1), o=ctypes.c_void_p(0xD000), fusion=fu) == 3


def test_chunk_bwd_validation(L):
    """gdn2_chunk_bwd: bad dims, missing pointers, outputs aliasing inputs or each other and
    a short workspace stop at host validation (nothing is launched)."""
    d = Dims(2, 100, 0, 2, 4, 128, 128, 1)
    P = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(20)]
    need = L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(d), 64)
    assert need > L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), 64)
    assert L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(Dims(2, 100, 0, 2, 4, 32, 128, 1)), 64) == 0
    # every built chunk size is computed with 64-token chunks (the same workspace); others
    # are refused
    assert L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(d), 128) == need
    assert L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(d), 32) == need
    assert L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(d), 48) == 0
    # fp32 at every head-dim pair
    for dk, dv in ((64, 64), (128, 128), (128, 64), (64, 128)):
        assert L.gdn2_chunk_bwd_workspace_bytes(ctypes.byref(Dims(2, 100, 0, 2, 4, dk, dv, 0)), 64) > 0

    def call(dims=d, outs=None, ws=P[19], ws_bytes=None, dO=P[8], chunk=64):
        o = P[10:17] if outs is None else outs
        return L.gdn2_chunk_bwd(P[0], P[1], P[2], P[3], P[4], P[5], None, None, chunk, dO, None,
                                *o, ctypes.byref(dims), ws, need if ws_bytes is None else ws_bytes,
                                None)
    assert call(dims=Dims(2, 100, 0, 2, 4, 128, 128, 7)) == 3          # dtype
    assert call(chunk=48) == 3                                         # chunk size not built
    assert call(dims=Dims(2, 100, 0, 2, 5, 128, 128, 1)) == 2          # h_v not a multiple of h_k
    assert call(dO=None) == 1
    assert call(outs=[None] + P[11:17]) == 1
    assert call(outs=[P[0]] + P[11:17]) == 2                           # dq aliases q
    assert call(outs=[P[10], P[10]] + P[12:17]) == 2                   # dq and dk alias
    assert call(ws_bytes=need - 1) == 4
    assert call(ws=ctypes.c_void_p(0x10001)) == 4                      # misaligned workspace

    # the entry point that takes the forward's chunk states
    def call_states(ck=P[18], chunk=64, outs=None):
        o = P[10:17] if outs is None else outs
        return L.gdn2_chunk_bwd_states(P[0], P[1], P[2], P[3], P[4], P[5], None, None, chunk, ck,
                                       P[8], None, *o, ctypes.byref(d), P[19], need, None)
    assert call_states(ck=None) == 1                                   # chunk_states required
    assert call_states(chunk=128) == 3                                 # states of a chunk-64 forward
    assert call_states(outs=[P[18]] + P[11:17]) == 2                   # dq aliases chunk_states


def test_chunk_fwd_noalloc_rejects_without_touching_a_device(L):
    """The static-workspace call checks its sizes on the host first: a NULL dims, and dims
    whose workspace exceeds GDN2_STATIC_WORKSPACE_BYTES (128 MiB), are refused before any
    HIP call (no device is needed to see it)."""
    def call(dims, chunk_size=64):
        return L.gdn2_chunk_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                        chunk_size, FAKE, None,
                                        None if dims is None else ctypes.byref(dims), None, None)
    assert call(None) == 1
    big = Dims(1, 8192, 0, 16, 16, 128, 128, 1)            # 2x the 4,096-token batch
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(big), 64) > g.STATIC_WORKSPACE_BYTES
    assert call(big) == 4
    assert b"static" in L.gdn2_last_error()
    fits = Dims(1, 4096, 0, 16, 16, 128, 128, 1)
    assert L.gdn2_chunk_fwd_workspace_bytes(ctypes.byref(fits), 64) <= g.STATIC_WORKSPACE_BYTES
