"""The library's calls under HIP graph capture: they enqueue only kernels on the caller's
stream (no allocation, copy, fill or synchronisation), so a caller may capture them. Each
graph is replayed several times with eager work and synchronisations between the replays,
and every replay must equal the eager calls bit for bit."""
import pytest
import torch

import gated_delta_rule_gdn_amd as g
from gated_delta_rule_gdn_amd import inputs

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "log_alpha", "b", "w")


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    g.lib()


def capture(fn):
    """Runs fn once on a side stream (lazy initialisation), then captures it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def test_chunk_forward_replays_in_a_graph():
    """A segmented chunked forward (4 pairs, 32 chunks) with the chunk-state output."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=2048, h_k=2, h_v=4, d_k=128,
                            d_v=128, neg_eig=True)
    x = {n: t.cuda() if isinstance(t, torch.Tensor) else t
         for n, t in inputs.chunk_inputs(wl, seed=51).items()}
    args = [x[n] for n in NAMES]
    B, T = 1, 2048
    nbytes = g.chunk_fwd_workspace_bytes(B, T, 2, 4, 128, 128, torch.bfloat16)

    def buffers():
        return (torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
                torch.empty(B, T, 4, 128, dtype=torch.bfloat16, device="cuda"),
                torch.empty(1, 4, 128, 128, dtype=torch.float32, device="cuda"),
                torch.empty(g.num_chunks(T, B), 4, 128, 128, dtype=torch.float32, device="cuda"))

    ws_e, o_e, S_e, ck_e = buffers()
    g.chunk_fwd(*args, S0=x["S0"], workspace=ws_e, out=o_e, final_state=S_e, chunk_states=ck_e)
    ws, o, S_T, ck = buffers()
    graph = capture(lambda: g.chunk_fwd(*args, S0=x["S0"], workspace=ws, out=o, final_state=S_T,
                                        chunk_states=ck))
    for rep in range(3):
        o.zero_()
        S_T.fill_(float("nan"))
        ck.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] chunk forward replay {rep}", flush=True)
        assert torch.equal(o, o_e) and torch.equal(S_T, S_e) and torch.equal(ck, ck_e)


@pytest.mark.parametrize("dtype,chunk", [(torch.bfloat16, 128), (torch.bfloat16, 32),
                                         (torch.float32, 64)])
def test_generic_chunk_path_replays_in_a_graph(dtype, chunk):
    """The generic path (prep kernel, panel segment pass, panel state pass) at chunks of 128
    and 32 and in fp32 at d = 128, segmented (4 pairs), captured once: every replay equals
    the eager call bit for bit."""
    wl = inputs.small_chunk(dtype=dtype, batch=1, seqlen=2048, h_k=2, h_v=4, d_k=128, d_v=128,
                            neg_eig=True)
    x = {n: t.cuda() if isinstance(t, torch.Tensor) else t
         for n, t in inputs.chunk_inputs(wl, seed=52).items()}
    args = [x[n] for n in NAMES]
    B, T = 1, 2048
    nbytes = g.chunk_fwd_workspace_bytes(B, T, 2, 4, 128, 128, dtype, chunk_size=chunk)

    def buffers():
        return (torch.empty(nbytes, dtype=torch.uint8, device="cuda"),
                torch.empty(B, T, 4, 128, dtype=dtype, device="cuda"),
                torch.empty(1, 4, 128, 128, dtype=torch.float32, device="cuda"))

    ws_e, o_e, S_e = buffers()
    g.chunk_fwd(*args, S0=x["S0"], chunk_size=chunk, workspace=ws_e, out=o_e, final_state=S_e)
    ws, o, S_T = buffers()
    graph = capture(lambda: g.chunk_fwd(*args, S0=x["S0"], chunk_size=chunk, workspace=ws, out=o,
                                        final_state=S_T))
    for rep in range(3):
        o.fill_(float("nan"))
        S_T.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] generic path {dtype} chunk {chunk} replay {rep}", flush=True)
        assert torch.equal(o, o_e) and torch.equal(S_T, S_e)


@pytest.mark.parametrize("seqlen,from_states", [(700, False), (1000, False), (1000, True)])
def test_chunk_backward_replays_in_a_graph(seqlen, from_states):
    """The bf16 chunked backward (its forward re-run, the reverse pass and the gradient
    kernels), captured once: every replay equals the eager call bit for bit (one value head
    per key head, so no atomics; a ragged last chunk). At T = 1000 (16 chunks, two pairs)
    the forward re-run's state pass and the reverse pass are both segmented; from_states
    runs gdn2_chunk_bwd_states on the chunk states of an eager forward."""
    wl = inputs.small_chunk(dtype=torch.bfloat16, batch=1, seqlen=seqlen, h_k=2, h_v=2, d_k=128,
                            d_v=128, neg_eig=True, s0_std=0.1)
    x = {n: t.cuda() if isinstance(t, torch.Tensor) else t
         for n, t in inputs.chunk_inputs(wl, seed=53).items()}
    args = [x[n] for n in NAMES]
    gen = torch.Generator().manual_seed(53)
    dO = torch.randn(1, seqlen, 2, 128, generator=gen).to(torch.bfloat16).cuda()
    dST = torch.randn(1, 2, 128, 128, generator=gen).cuda()
    nbytes = g.chunk_bwd_workspace_bytes(1, seqlen, 2, 2, 128, 128, torch.bfloat16)
    ck = None
    if from_states:
        ck = torch.empty(g.num_chunks(seqlen, 1), 2, 128, 128, dtype=torch.float32, device="cuda")
        g.chunk_fwd(*args, S0=x["S0"], chunk_states=ck)
    ref = g.chunk_bwd(*args, dO, S0=x["S0"], dS_T=dST, chunk_states=ck,
                      workspace=torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    box = {}

    def call():
        box["out"] = g.chunk_bwd(*args, dO, S0=x["S0"], dS_T=dST, workspace=ws, chunk_states=ck)

    graph = capture(call)
    out = box["out"]
    for rep in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] chunk backward replay {rep}", flush=True)
        for n in ref:
            assert torch.equal(out[n], ref[n]), n


def test_decode_steps_replay_in_a_graph():
    """Four in-place decode steps on one state pool, captured once: every replay advances
    the state by the same four steps as the eager calls."""
    wl = inputs.DecodeWorkload("graph_decode", torch.float32, 8, 2, 6, 128, 128, steps=4)
    x = inputs.decode_inputs(wl, seed=52)
    d = {n: x[n].cuda() for n in NAMES}
    S_eager, S_graph = x["S"].cuda(), x["S"].cuda()
    o_eager = torch.empty(4, 8, 6, 128, device="cuda")
    o_graph = torch.empty_like(o_eager)

    def steps(S, out):
        for t in range(4):
            g.recurrent_step(*(d[n][t] for n in NAMES), S, out=out[t])

    graph = capture(lambda: steps(S_graph, o_graph))
    S_graph.copy_(x["S"].cuda())           # undo the warm-up and capture-time steps
    torch.cuda.synchronize()
    for rep in range(3):
        steps(S_eager, o_eager)
        o_graph.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        print(f"[graph] decode replay {rep}", flush=True)
        assert torch.equal(o_graph, o_eager) and torch.equal(S_graph, S_eager)
