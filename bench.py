"""Benchmark of the Gated DeltaNet-2 core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One "step" is one chunked WY forward (gdn2_chunk_fwd: cumulative decay, A, (I+A)^-1 blocks,
WY factors, inter-chunk state pass, outputs) over the bf16 workload B=1, T=4096, 16 heads,
d_k = d_v = 128, chunk 64, negative-eigenvalue erase gates and a random fp32 initial state;
`value` is its throughput in tokens/s. The decode step (gdn2_recurrent_step: 64 sequences,
48 value heads over 16 key heads, d = 128, fp32 state updated in place) is timed over 256
consecutive steps and reported in the `decode` object as state GB/s against HBM peak, with
the multi-token / bf16-state variants of gdn2_recurrent_fwd on the same shape beside it.

Inputs are seeded synthetic tensors already resident in GPU memory when a timed region
starts. Timing uses HIP events on the stream the library launches on (torch's current
stream), bracketed by device synchronisation. The fp64 CPU oracle is timed on the host
cores over a bounded sample as a reported baseline (`cpu_baseline`), and its outputs double
as a parity check of the timed run.
"""
import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_delta_rule_gdn_amd as g  # noqa: E402
from gated_delta_rule_gdn_amd import inputs  # noqa: E402

METRIC = "chunk-fwd tokens/s (T=4096,H=16,d=128) + decode state GB/s vs HBM peak"
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0    # dense
CHUNK = 64


def chunk_alg(wl, tokens, nseq, chunk=CHUNK):
    """Algorithmic bytes and flops of one chunked forward (per-tensor element counts)."""
    e = 2 if wl.dtype == torch.bfloat16 else 4
    qk = 2 * tokens * wl.h_k * wl.d_k * e
    vw = 2 * tokens * wl.h_v * wl.d_v * e
    ab = 2 * tokens * wl.h_v * wl.d_k * e
    o = tokens * wl.h_v * wl.d_v * e
    states = (2 if wl.s0_std is not None else 1) * nseq * wl.h_v * wl.d_k * wl.d_v * 4
    bytes_ = qk + vw + ab + o + states
    # triangle-aware flops per (token, value head): C(3 d_k + 2 d_v) + 6 d_k d_v
    flops = tokens * wl.h_v * (chunk * (3 * wl.d_k + 2 * wl.d_v) + 6 * wl.d_k * wl.d_v)
    return bytes_, flops


def decode_alg(wl):
    st = wl.num_seqs * wl.h_v * wl.d_k * wl.d_v * 4
    vec = 4 * (2 * wl.num_seqs * wl.h_k * wl.d_k + 2 * wl.num_seqs * wl.h_v * wl.d_v +
               2 * wl.num_seqs * wl.h_v * wl.d_k + wl.num_seqs * wl.h_v * wl.d_v)
    return 2 * st + vec, 2 * st, 7 * wl.num_seqs * wl.h_v * wl.d_k * wl.d_v


# Sources of the 64-token chunked forward and of the bf16 chunked backward (a stored counter
# reading is used only while these are unchanged)
CHUNK_SRC = ("gdn2_chunk.hip", "gdn2_prep.hip", "gdn2_chunk.h", "gdn2_mfma.h", "gdn2_common.h")
BWD_SRC = ("gdn2_bwd16.hip", "gdn2_chunk.hip", "gdn2_prep.hip", "gdn2_chunk.h", "gdn2_mfma.h",
           "gdn2_common.h")


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "gated_delta_rule_gdn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it still
    describes the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec.get("bytes_per_launch")


def time_region(fn, steps, stream):
    """Average duration of fn() over `steps` back-to-back calls, by HIP events on `stream`."""
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3 / steps


def bench_chunk(steps, warmup, seed=1002):
    wl = inputs.CHUNK_BF16_T4096
    x = inputs.chunk_inputs(wl, seed=seed)
    d = {n: x[n].cuda() for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")}
    B, T = x["q"].shape[:2]
    ws = torch.empty(g.chunk_fwd_workspace_bytes(B, T, wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.dtype),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty(B, T, wl.h_v, wl.d_v, dtype=wl.dtype, device="cuda")
    S_T = torch.empty_like(d["S0"])

    def call():
        g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                    workspace=ws, out=o, final_state=S_T)

    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream()
    t_warm = time_region(call, steps, stream)
    # cold: flush the caches (a 1 GiB write) before each timed call
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    cold = []
    for _ in range(min(steps, 20)):
        flush.fill_(1.0)
        cold.append(time_region(call, 1, stream))
    del flush
    return wl, x, (o, S_T), t_warm, float(np.median(cold))


def bench_decode(seed=3, repeats=5):
    """The decode workload's 256 consecutive steps, timed `repeats` times back to back
    (median per step), eagerly and as one captured HIP graph replayed."""
    wl = inputs.DECODE_F32
    x = inputs.decode_inputs(wl, seed=seed)
    d = {n: x[n].cuda() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    S = x["S"].cuda()
    o = torch.empty(wl.steps, wl.num_seqs, wl.h_v, wl.d_v, device="cuda")

    def run_all():
        for t in range(wl.steps):
            g.recurrent_step(d["q"][t], d["k"][t], d["v"][t], d["log_alpha"][t], d["b"][t],
                             d["w"][t], S, out=o[t])

    run_all()                                   # warm-up pass (state keeps evolving)
    stream = torch.cuda.current_stream()
    eager = [time_region(run_all, 1, stream) / wl.steps for _ in range(repeats)]
    # the same 256 launches captured once and replayed (no host launch cost per step)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run_all()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            run_all()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    graphed = [time_region(graph.replay, 1, stream) / wl.steps for _ in range(repeats)]
    assert torch.isfinite(S).all()
    del graph
    return wl, float(np.median(eager)), float(np.median(graphed)), eager, graphed


def bench_chunk_workload(wl, steps, warmup, seed, chunk=CHUNK):
    """Warm back-to-back timing of one chunk-forward workload (inputs drawn on the GPU)."""
    x = inputs.chunk_inputs_device(wl, seed)
    B, T = x["q"].shape[:2]
    N = x["num_seqs"]
    ws = torch.empty(g.chunk_fwd_workspace_bytes(B, T, wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.dtype,
                                                 num_seqs=N if x["cu_seqlens"] is not None else 0,
                                                 chunk_size=chunk),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty(B, T, wl.h_v, wl.d_v, dtype=wl.dtype, device="cuda")
    S_T = torch.empty(N, wl.h_v, wl.d_k, wl.d_v, dtype=torch.float32, device="cuda")

    def call():
        g.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S0=x["S0"],
                    cu_seqlens=x["cu_seqlens"], workspace=ws, out=o, final_state=S_T,
                    chunk_size=chunk)

    for _ in range(warmup):
        call()
    t = time_region(call, steps, torch.cuda.current_stream())
    nbytes, flops = chunk_alg(wl, B * T, N, chunk)
    res = {"workload": wl.name, "chunk_size": chunk, "tokens": B * T, "us_per_call": t * 1e6,
           "tokens_per_s": B * T / t, "alg_bytes": nbytes, "alg_flops": flops,
           "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBPS,
           "mfma_frac_bf16": flops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS}
    del x, ws, o, S_T
    torch.cuda.empty_cache()
    return res


def bench_decode_large_state(seed=4, steps=32):
    """Decode with 128 sequences (403 MB of state, more than the 256 MB MALL)."""
    wl = inputs.DecodeWorkload("decode_f32_n128_hv48_hk16_d128", torch.float32, 128, 16, 48,
                               128, 128, steps=steps)
    x = inputs.decode_inputs_device(wl, seed, steps)
    S = x["S"]
    o = torch.empty(steps, wl.num_seqs, wl.h_v, wl.d_v, device="cuda")

    def run_all():
        for t in range(steps):
            g.recurrent_step(x["q"][t], x["k"][t], x["v"][t], x["log_alpha"][t], x["b"][t],
                             x["w"][t], S, out=o[t])

    run_all()
    t_step = time_region(run_all, 1, torch.cuda.current_stream()) / steps
    nbytes, st, _ = decode_alg(wl)
    res = {"workload": wl.name, "steps": steps, "us_per_step": t_step * 1e6,
           "state_GBps": st / t_step / 1e9, "total_GBps": nbytes / t_step / 1e9,
           "hbm_frac": nbytes / t_step / 1e9 / HBM_PEAK_GBPS}
    del x, S, o
    torch.cuda.empty_cache()
    return res


def bench_recurrent(T, state_dtype, calls, seed, traffic_key=None):
    """gdn2_recurrent_fwd on the decode shape (64 sequences, 48 value heads over 16 key
    heads, d = 128, fp32 inputs): `calls` back-to-back calls of T tokens each against one
    state pool of `state_dtype`; inputs drawn on the GPU, laid out per call."""
    sname = "bf16" if state_dtype == torch.bfloat16 else "f32"
    wl = inputs.DecodeWorkload(f"recurrent_t{T}_{sname}state_n64_hv48_hk16_d128", torch.float32,
                               64, 16, 48, 128, 128, steps=T * calls)
    x = inputs.decode_inputs_device(wl, seed, T * calls)
    N = wl.num_seqs
    y = {n: x[n].reshape(calls, T, N, *x[n].shape[2:]).permute(0, 2, 1, 3, 4).contiguous()
         for n in ("q", "k", "v", "log_alpha", "b", "w")}
    del x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"]
    P = x["S"].to(state_dtype)
    o = torch.empty(calls, N, T, wl.h_v, wl.d_v, device="cuda")

    def run_all():
        for c in range(calls):
            g.recurrent_fwd(y["q"][c], y["k"][c], y["v"][c], y["log_alpha"][c], y["b"][c],
                            y["w"][c], P, out=o[c])

    run_all()
    t_call = time_region(run_all, 1, torch.cuda.current_stream()) / calls
    one = inputs.DecodeWorkload(wl.name, wl.dtype, N, wl.h_k, wl.h_v, wl.d_k, wl.d_v, steps=1)
    nbytes1, st32, _ = decode_alg(one)
    esz = 2 if state_dtype == torch.bfloat16 else 4
    state_bytes = st32 * esz // 4
    nbytes = state_bytes + T * (nbytes1 - st32)
    assert torch.isfinite(P.float()).all()
    res = {"workload": wl.name, "tokens_per_call": T, "calls": calls,
           "us_per_call": t_call * 1e6, "tokens_per_s": N * T / t_call,
           "state_GBps": state_bytes / t_call / 1e9, "total_GBps": nbytes / t_call / 1e9,
           "hbm_frac": nbytes / t_call / 1e9 / HBM_PEAK_GBPS, "alg_bytes": nbytes,
           "traffic": None if traffic_key is None else measured_traffic(
               traffic_key, source_hash("gdn2_decode.hip", "gdn2_common.h"))}
    del y, P, o
    torch.cuda.empty_cache()
    return res


def bench_gate_variants(steps, warmup, seed=9):
    """The timed chunk shape (bf16, B=1 T=4096 H=16 d=128) run as KDA and as FG2-GDN+, two
    ways: natively (gdn2_fusion.gate_mode: the prep kernel reads beta itself) and through the
    gate mappings (gdn2_map_gates, then the GDN-2 chunked forward), with the mapping pass
    timed on its own. The mapping is an elementwise HBM pass: its algorithmic bytes are the
    gate tensors it reads and the GDN-2 tensors it writes."""
    wl = inputs.CHUNK_BF16_T4096
    res = {}
    stream = torch.cuda.current_stream()
    for mode in ("kda", "fg2+"):
        x = inputs.variant_inputs(mode, wl.dtype, 1, wl.seqlen, wl.h_k, wl.h_v, wl.d_k, wl.d_v,
                                  seed)
        d = {n: t.cuda() for n, t in x.items()}
        ws = torch.empty(g.chunk_fwd_workspace_bytes(1, wl.seqlen, wl.h_k, wl.h_v, wl.d_k,
                                                     wl.d_v, wl.dtype),
                         dtype=torch.uint8, device="cuda")

        def mapping():
            return g.map_gates(mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                               d.get("beta_v"))

        def mapped():
            g.chunk_fwd(*mapping(), S0=d["S"], workspace=ws)

        def native():
            g.gated_chunk_fwd(mode, d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                              beta_v=d.get("beta_v"), S0=d["S"], workspace=ws)

        for _ in range(warmup):
            mapped()
            native()
        t_map = time_region(mapping, steps, stream)
        t_mapped = time_region(mapped, steps, stream)
        t_native = time_region(native, steps, stream)
        T, H, dk, dv, e = wl.seqlen, wl.h_v, wl.d_k, wl.d_v, 2
        if mode == "kda":
            nbytes = T * H * e + T * H * (dk + dv) * e          # beta in; b, w out
        else:                                                   # beta, beta_v, k in; k', b, w out
            nbytes = T * H * (dk + dv) * e + T * wl.h_k * dk * e + T * H * (2 * dk + dv) * e
        res[mode] = {"workload": f"{wl.name}_{mode}", "us_per_call": t_native * 1e6,
                     "tokens_per_s": T / t_native, "mapped_us_per_call": t_mapped * 1e6,
                     "map_us": t_map * 1e6, "map_alg_bytes": nbytes,
                     "map_hbm_frac": nbytes / t_map / 1e9 / HBM_PEAK_GBPS}
        del d, ws
    return res


def bench_chunk_states(steps, warmup, seed=10):
    """The timed chunk workload with the state entering every chunk written out (the
    checkpoints a training backward starts from), beside the same call without them. The
    64 MB of fp32 states are added to the algorithmic bytes."""
    wl = inputs.CHUNK_BF16_T4096
    x = inputs.chunk_inputs_device(wl, seed)
    B, T = x["q"].shape[:2]
    ws = torch.empty(g.chunk_fwd_workspace_bytes(B, T, wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.dtype),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty(B, T, wl.h_v, wl.d_v, dtype=wl.dtype, device="cuda")
    S_T = torch.empty_like(x["S0"])
    nc = g.num_chunks(T, B)
    ck = torch.empty(nc, wl.h_v, wl.d_k, wl.d_v, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(states):
        def fn():
            g.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S0=x["S0"],
                        workspace=ws, out=o, final_state=S_T,
                        chunk_states=ck if states else None)
        return fn

    for _ in range(warmup):
        call(True)()
        call(False)()
    t_on = time_region(call(True), steps, stream)
    t_off = time_region(call(False), steps, stream)
    nbytes = chunk_alg(wl, B * T, B)[0] + ck.numel() * 4
    del x, ws, o, S_T
    res = {"workload": f"{wl.name}_chunk_states", "us_per_call": t_on * 1e6,
           "us_per_call_without": t_off * 1e6, "tokens_per_s": T * B / t_on,
           "alg_bytes": nbytes, "hbm_frac": nbytes / t_on / 1e9 / HBM_PEAK_GBPS}
    del ck
    return res


def bench_chunk_bwd(steps, warmup, seed=11, wl=inputs.CHUNK_BF16_T4096, from_states=False):
    """The chunked backward (gdn2_chunk_bwd) on a chunk workload (the timed one by default):
    the forward re-run that stores the chunk states, the reverse state pass and the per-chunk
    gradients. Algorithmic bytes: the forward inputs, dO, S0 and dS_T read once, the fp32
    gradients written once. from_states: gdn2_chunk_bwd_states, given the chunk states a
    forward wrote (written once, untimed; their reading is counted)."""
    x = inputs.chunk_inputs_device(wl, seed)
    B, T = x["q"].shape[:2]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    dO = torch.randn(B, T, wl.h_v, wl.d_v, generator=gen, device="cuda").to(wl.dtype)
    dST = torch.randn_like(x["S0"])
    ws = torch.empty(g.chunk_bwd_workspace_bytes(B, T, wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.dtype),
                     dtype=torch.uint8, device="cuda")
    ck = None
    if from_states:
        ck = torch.empty(g.num_chunks(T, B), wl.h_v, wl.d_k, wl.d_v, dtype=torch.float32,
                         device="cuda")
        g.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S0=x["S0"],
                    chunk_states=ck)

    def call():
        g.chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], dO, S0=x["S0"],
                    dS_T=dST, workspace=ws, chunk_states=ck)

    for _ in range(warmup):
        call()
    t = time_region(call, steps, torch.cuda.current_stream())
    e = 2 if wl.dtype == torch.bfloat16 else 4
    tok_in = T * (2 * wl.h_k * wl.d_k + wl.h_v * (2 * wl.d_k + 3 * wl.d_v)) * e   # q k, la b, v w dO
    grads = T * (2 * wl.h_k * wl.d_k + wl.h_v * (2 * wl.d_k + 2 * wl.d_v)) * 4
    states = 3 * x["S0"].numel() * 4                                          # S0, dS_T, dS0
    nbytes = tok_in + grads + states + (ck.numel() * 4 if from_states else 0)
    del x, ws, dO, dST, ck
    bsrc = source_hash(*BWD_SRC)
    timed = wl is inputs.CHUNK_BF16_T4096
    return {"workload": f"{wl.name}_bwd" + ("_from_states" if from_states else ""),
            "us_per_call": t * 1e6, "tokens_per_s": T * B / t,
            "alg_bytes": nbytes, "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBPS,
            "traffic": measured_traffic("chunk_bwd_from_states_t4096" if from_states
                                        else "chunk_bwd_t4096", bsrc) if timed else None}


def bench_fused(steps, warmup, seed=8):
    """The timed chunk workload and the decode step with the fusions of the burn-gdn2
    "Architecture" diagram turned on (q/k L2-norm before the recurrence, SiLU-gated RMS norm
    after it), timed against the same calls without them. The gate tensor adds one read of
    an o-sized tensor to the algorithmic bytes."""
    res = {}
    wl = inputs.CHUNK_BF16_T4096
    x = inputs.chunk_inputs_device(wl, seed)
    B, T = x["q"].shape[:2]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    gate = torch.randn(B, T, wl.h_v, wl.d_v, generator=gen, device="cuda").to(wl.dtype)
    nw = torch.rand(wl.d_v, generator=gen, device="cuda") + 0.5
    ws = torch.empty(g.chunk_fwd_workspace_bytes(B, T, wl.h_k, wl.h_v, wl.d_k, wl.d_v, wl.dtype),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty(B, T, wl.h_v, wl.d_v, dtype=wl.dtype, device="cuda")
    S_T = torch.empty_like(x["S0"])

    def call(fused):
        def fn():
            g.chunk_fwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], S0=x["S0"],
                        workspace=ws, out=o, final_state=S_T, qk_l2norm=fused,
                        gate=gate if fused else None, norm_weight=nw if fused else None)
        return fn

    stream = torch.cuda.current_stream()
    for fused in (False, True):
        for _ in range(warmup):
            call(fused)()
    t_plain = time_region(call(False), steps, stream)
    t_fused = time_region(call(True), steps, stream)
    nbytes, _ = chunk_alg(wl, B * T, B)
    nbytes += gate.numel() * gate.element_size()
    res["chunk"] = {"workload": wl.name + "_qkl2norm_gatednorm", "us_per_call": t_fused * 1e6,
                    "us_per_call_unfused": t_plain * 1e6, "tokens_per_s": B * T / t_fused,
                    "alg_bytes": nbytes, "hbm_frac": nbytes / t_fused / 1e9 / HBM_PEAK_GBPS}
    del x, ws, o, S_T, gate
    dw = inputs.DECODE_F32
    steps_d = 64
    y = inputs.decode_inputs_device(dw, seed, steps_d)
    yy = {n: y[n][:, :, None].contiguous() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    dgate = torch.randn(steps_d, dw.num_seqs, 1, dw.h_v, dw.d_v, generator=gen, device="cuda")
    dnw = torch.rand(dw.d_v, generator=gen, device="cuda") + 0.5
    od = torch.empty(dw.num_seqs, 1, dw.h_v, dw.d_v, device="cuda")

    def dcall(fused):
        def fn():
            for t in range(steps_d):
                g.recurrent_fwd(yy["q"][t], yy["k"][t], yy["v"][t], yy["log_alpha"][t],
                                yy["b"][t], yy["w"][t], y["S"], out=od, qk_l2norm=fused,
                                gate=dgate[t] if fused else None,
                                norm_weight=dnw if fused else None)
        return fn

    C = 2 * dw.h_k * dw.d_k + dw.h_v * dw.d_v
    cw = torch.randn(C, 4, generator=gen, device="cuda") * 0.5
    cst = torch.randn(dw.num_seqs, 3, C, generator=gen, device="cuda")

    def ccall():
        for t in range(steps_d):
            g.recurrent_fwd(yy["q"][t], yy["k"][t], yy["v"][t], yy["log_alpha"][t], yy["b"][t],
                            yy["w"][t], y["S"], out=od, qk_l2norm=True, gate=dgate[t],
                            norm_weight=dnw, conv_weight=cw, conv_state=cst, conv_silu=True)

    for fused in (False, True):
        dcall(fused)()
    ccall()
    t_plain = time_region(dcall(False), 1, stream) / steps_d
    t_fused = time_region(dcall(True), 1, stream) / steps_d
    t_conv = time_region(ccall, 1, stream) / steps_d
    dbytes, _, _ = decode_alg(dw)
    dbytes += dw.num_seqs * dw.h_v * dw.d_v * 4
    cbytes = dbytes + 2 * dw.num_seqs * 3 * C * 4 + C * 4 * 4   # conv state in and out, taps
    res["decode"] = {"workload": dw.name + "_qkl2norm_gatednorm", "us_per_step": t_fused * 1e6,
                     "us_per_step_unfused": t_plain * 1e6, "alg_bytes": dbytes,
                     "hbm_frac": dbytes / t_fused / 1e9 / HBM_PEAK_GBPS}
    res["decode_conv"] = {"workload": dw.name + "_shortconv_qkl2norm_gatednorm",
                          "us_per_step": t_conv * 1e6, "alg_bytes": cbytes,
                          "hbm_frac": cbytes / t_conv / 1e9 / HBM_PEAK_GBPS}
    del y, yy, dgate, od, cst
    torch.cuda.empty_cache()
    return res


CPU_WORK_TARGET_S = 10.0     # CPU-seconds of oracle work per baseline sample


def host_cpu():
    """(CPU model name from /proc/cpuinfo, cores this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return model, cores


def cpu_baseline_chunk(wl, x, gpu_out):
    """fp64 oracle over the whole timed workload, repeated until the sample holds about
    CPU_WORK_TARGET_S CPU-seconds (threads x wall); the first pass also gives parity."""
    import oracle
    B, T = x["q"].shape[:2]
    f = {n: x[n].double().numpy().reshape(B * T, *x[n].shape[2:]) for n in
         ("q", "k", "v", "log_alpha", "b", "w")}
    S0 = x["S0"].double().numpy()
    threads = min(oracle.default_threads(), wl.h_v * B)
    reps, wall = 0, 0.0
    while True:
        t0 = time.perf_counter()
        o_r, S_r = oracle.recurrent(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"],
                                    S0=S0, cu_seqlens=[0, T], threads=threads)
        wall += time.perf_counter() - t0
        reps += 1
        if reps == 1:
            o_g = gpu_out[0].double().cpu().numpy().reshape(B * T, wl.h_v, wl.d_v)
            S_g = gpu_out[1].double().cpu().numpy()
            parity = {"o_rel_l2": oracle.rel_l2(o_g, o_r), "S_T_rel_l2": oracle.rel_l2(S_g, S_r),
                      "tol": 2e-2}
        if wall * threads >= CPU_WORK_TARGET_S or reps >= 20:
            break
    model, host_cores = host_cpu()
    base = {"value": reps * B * T / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "host_cores": host_cores,
            "sample": f"whole workload ({B * T} tokens x {wl.h_v} heads, fp64, "
                      f"{wl.h_v * B} (sequence, head) pairs over {threads} threads) x {reps} "
                      f"passes, {wall:.2f} s wall"}
    return base, parity


def cpu_baseline_decode(wl, pairs=1024):
    """fp64 oracle on `pairs` of the workload's states for all its steps, scaled to one step
    over every state."""
    import oracle
    x = inputs.decode_inputs(wl, seed=3)
    G = wl.h_v // wl.h_k
    rng = np.random.default_rng(0)
    sel = [(int(n), int(h)) for n, h in zip(rng.integers(0, wl.num_seqs, pairs),
                                            rng.integers(0, wl.h_v, pairs))]
    threads = min(oracle.default_threads(), pairs)
    from concurrent.futures import ThreadPoolExecutor

    def one(p):
        n, h = p
        hk = h // G
        a = lambda t, hh: t[:, n, hh].double().numpy()  # noqa: E731
        oracle.sequence(a(x["q"], hk), a(x["k"], hk), a(x["v"], h), a(x["w"], h),
                        a(x["log_alpha"], h), a(x["b"], h), x["S"][n, h].double().numpy())

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, sel))
    dt = time.perf_counter() - t0
    state_updates = pairs * wl.steps
    per_step_equiv = dt / state_updates * (wl.num_seqs * wl.h_v)   # all states, one step
    st_bytes = 2 * wl.num_seqs * wl.h_v * wl.d_k * wl.d_v * 4
    model, host_cores = host_cpu()
    return {"value": st_bytes / per_step_equiv / 1e9, "unit": "state GB/s", "cores": threads,
            "kind": "oracle", "cpu_model": model, "host_cores": host_cores,
            "sample": f"{pairs} of {wl.num_seqs * wl.h_v} states x {wl.steps} steps, fp64, "
                      f"{dt:.2f} s wall, scaled to all states"}


def profile_driver():
    """Short fixed sequence for hardware-counter runs: 5 chunk forwards (bf16, B=1 T=4096
    H=16 d=128, chunk 64), 2 at chunk 128, 2 fp32 forwards of that shape, 3 chunked
    backwards, one forward that writes the chunk states and 3 backwards from them
    (gdn2_chunk_bwd_states), 20 decode steps with an fp32 state and 20 with a bf16 state, and 3 copies of
    256 MiB (the copy calibrates the FETCH_SIZE / WRITE_SIZE counters)."""
    wl = inputs.CHUNK_BF16_T4096
    x = inputs.chunk_inputs(wl, seed=1002)
    d = {n: x[n].cuda() for n in ("q", "k", "v", "log_alpha", "b", "w", "S0")}
    for _ in range(5):
        g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"])
    for _ in range(2):
        g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                    chunk_size=128)
    torch.cuda.synchronize()
    f = {n: t.float() for n, t in d.items()}
    for _ in range(2):
        g.chunk_fwd(f["q"], f["k"], f["v"], f["log_alpha"], f["b"], f["w"], S0=f["S0"])
    del f
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    dO = torch.randn(1, wl.seqlen, wl.h_v, wl.d_v, generator=gen, device="cuda").to(wl.dtype)
    for _ in range(3):
        g.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO, S0=d["S0"],
                    dS_T=torch.ones_like(d["S0"]))
    ck = torch.empty(g.num_chunks(wl.seqlen, 1), wl.h_v, wl.d_k, wl.d_v, dtype=torch.float32,
                     device="cuda")
    g.chunk_fwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], S0=d["S0"],
                chunk_states=ck)
    for _ in range(3):
        g.chunk_bwd(d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], dO, S0=d["S0"],
                    dS_T=torch.ones_like(d["S0"]), chunk_states=ck)
    torch.cuda.synchronize()
    del dO, ck
    torch.cuda.empty_cache()
    dw = inputs.DECODE_F32
    y = inputs.decode_inputs(dw, seed=3, steps=1)
    S = y["S"].cuda()
    yy = {n: y[n][0].cuda() for n in ("q", "k", "v", "log_alpha", "b", "w")}
    for _ in range(20):
        g.recurrent_step(yy["q"], yy["k"], yy["v"], yy["log_alpha"], yy["b"], yy["w"], S)
    Sb = S.to(torch.bfloat16)
    y1 = {n: t[:, None] for n, t in yy.items()}
    for _ in range(20):
        g.recurrent_fwd(y1["q"], y1["k"], y1["v"], y1["log_alpha"], y1["b"], y1["w"], Sb)
    src = torch.empty(1 << 26, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("profile driver done")


def kernel_short(k):
    """A kernel's name without its parameter list and namespaces."""
    for pre in ("void ", "gdn2::", "(anonymous namespace)::"):
        k = k.replace(pre, "")
    return k.split("(")[0]


def pmc_table(dirs):
    """Per-kernel averages of every counter found in the counter_collection CSVs under the
    given directories (one rocprofv3 --pmc run of --profile-driver each), with the derived
    ratios: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs),
    and LDS bank-conflict cycles per LDS-active cycle."""
    import csv
    import glob
    from collections import defaultdict
    agg = defaultdict(lambda: defaultdict(list))
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if "gdn2" not in r["Kernel_Name"]:
                        continue
                    agg[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    rows = []
    for k, ctrs in sorted(agg.items()):
        avg = {c: sum(v) / len(v) for c, v in ctrs.items()}
        short = kernel_short(k)
        row = {"kernel": short, "launches": max(len(v) for v in ctrs.values()), **avg}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in avg and avg.get("GRBM_GUI_ACTIVE"):
            # GRBM_GUI_ACTIVE comes summed over the 8 XCDs: busy cycles per SIMD over the
            # kernel's active cycles on one XCD (the max-over-XCDs of the tool's MfmaUtil)
            row["gui_active_cycles_per_xcd"] = avg["GRBM_GUI_ACTIVE"] / 8
            row["mfma_busy_frac"] = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (avg["GRBM_GUI_ACTIVE"] / 8 * 1024)
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            row["lds_conflict_per_active"] = avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"]
        rows.append(row)
    for r in rows:
        print(json.dumps(r))
    return rows


def pmc_summary(fetch_dir, write_dir):
    """Writes profiles/pmc_traffic.json from two `rocprofv3 --pmc` runs of --profile-driver
    (FETCH_SIZE, then WRITE_SIZE; their counter_collection CSVs under the two directories).
    Each counter is scaled by what it reads for the 256 MiB copy of the driver. Launches of
    one kernel are kept in dispatch order, so the chunk-forward kernels of the 5 plain
    forwards (the first 5 launches) are told apart from the forward re-run inside the 3
    backwards (the next 3); the forward that writes the chunk states (launch 9) is left out,
    and the 3 backwards from those states follow it (their prep launches 10-12, their
    given-states state pass and backward kernels as their own launches). Prints the
    per-launch rows of the traffic table."""
    import csv
    import glob
    from collections import defaultdict

    def load(d, ctr):
        per = defaultdict(list)
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for r in csv.DictReader(f):
                    if r["Counter_Name"] == ctr:
                        per[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        return {k: [v for _, v in sorted(x)] for k, x in per.items()}

    F, W = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    copyk = [k for k in F if "copyBuffer" in k][0]
    copy_kib = 256 * 1024
    ff, wf = copy_kib / np.mean(F[copyk]), copy_kib / np.mean(W[copyk])
    print(f"calibration: FETCH_SIZE {np.mean(F[copyk]):,.0f} KiB per 256 MiB copy -> x{ff:.2f}; "
          f"WRITE_SIZE {np.mean(W[copyk]):,.0f} KiB -> x{wf:.2f}")
    ff, wf = round(ff, 1), round(wf, 1)

    def group(key, lo, hi):
        """(read, written) bytes per launch of launches lo..hi-1 of a kernel."""
        fv, wv = F.get(key, [])[lo:hi], W.get(key, [])[lo:hi]
        if not fv:
            return None
        return float(np.mean(fv)) * ff * 1024, float(np.mean(wv)) * wf * 1024 if wv else 0.0

    groups = {"chunk_fwd_t4096": [], "chunk_fwd_t4096_c128": [], "chunk_fwd_f32_t4096": [],
              "chunk_bwd_t4096": [], "chunk_bwd_from_states_t4096": []}
    dec = {}
    for k in F:
        if "gdn2" not in k:
            continue
        name = kernel_short(k)
        base = name.split("<")[0]
        targs = name[name.index("<") + 1:name.rindex(">")].split(", ") if "<" in name else []
        c64_bf16 = base == "prep_kernel" and targs[2] == "64" and "bf16" in targs[0]
        if base == "chunk_state_kernel" and targs[-1] == "true":      # given states
            parts = [("chunk_bwd_from_states_t4096", 0, 3)]
        elif c64_bf16:
            parts = [("chunk_fwd_t4096", 0, 5), ("chunk_bwd_t4096", 5, 8),
                     ("chunk_bwd_from_states_t4096", 9, 12)]
        elif base in ("chunk_seg_kernel", "chunk_state_kernel"):
            parts = [("chunk_fwd_t4096", 0, 5), ("chunk_bwd_t4096", 5, 8)]
        elif base in ("prep_kernel", "panel_seg_kernel", "panel_state_kernel"):
            parts = [("chunk_fwd_f32_t4096" if "float" in targs[0] else "chunk_fwd_t4096_c128", 0, 2)]
        elif base.startswith("bwd_"):
            parts = [("chunk_bwd_t4096", 0, 3), ("chunk_bwd_from_states_t4096", 3, 6)]
        elif base == "recurrent_fwd_kernel":
            key = ("decode_step_bf16state_n64_hv48" if "float, bf16_t" in name
                   else "decode_step_n64_hv48")
            rw = group(k, 0, 20)
            dec[key] = {"bytes_per_launch": int(sum(rw)), "kernel": name}
            print(f"| {name} | {key} | {rw[0] / 1e6:.1f} MB | {rw[1] / 1e6:.1f} MB | {sum(rw) / 1e6:.1f} MB |")
            continue
        else:
            continue
        for gname, lo, hi in parts:
            rw = group(k, lo, hi)
            if rw is None:
                continue
            groups[gname].append((name, rw))
            print(f"| {name} | {gname} | {rw[0] / 1e6:.1f} MB | {rw[1] / 1e6:.1f} MB | {sum(rw) / 1e6:.1f} MB |")
    out = {"_note": f"HBM bytes per launch from rocprofv3 --pmc FETCH_SIZE (x{ff}) and "
                    f"WRITE_SIZE (x{wf}); commands and calibration in hbm_traffic_counters.md"}
    csrc = source_hash(*CHUNK_SRC)
    gsrc = source_hash("gdn2_prep.hip", "gdn2_state.hip", "gdn2_chunk.h", "gdn2_mfma.h",
                       "gdn2_common.h")
    bsrc = source_hash(*BWD_SRC)
    for gname, items in groups.items():
        src = {"chunk_fwd_t4096": csrc, "chunk_bwd_t4096": bsrc,
               "chunk_bwd_from_states_t4096": bsrc}.get(gname, gsrc)
        out[gname] = {"source_hash": src, "bytes_per_launch": int(sum(sum(rw) for _, rw in items)),
                      "kernels": {n: int(sum(rw)) for n, rw in items}}
    dsrc = source_hash("gdn2_decode.hip", "gdn2_common.h")
    for key, rec in dec.items():
        out[key] = {"source_hash": dsrc, **rec}
    with open(os.path.join(ROOT, "profiles", "pmc_traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the timing of the other chunk workloads and the decode control")
    ap.add_argument("--only", choices=["chunk", "decode", "bwd", "all"], default="all",
                    help="bwd: time the chunked backward alone (its own JSON line)")
    ap.add_argument("--profile-driver", action="store_true",
                    help="short fixed sequence for hardware-counter runs (see profile_driver)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/pmc_traffic.json from the two counter runs and exit")
    ap.add_argument("--pmc-table", nargs="+", metavar="DIR",
                    help="print per-kernel averages of the counters under the given rocprofv3 "
                         "--pmc output directories (with the MFMA-busy and LDS ratios) and exit")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.pmc_table:
        pmc_table(args.pmc_table)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(pass --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    g.lib()
    torch.cuda.set_device(0)
    if args.profile_driver:
        profile_driver()
        return
    if args.only == "bwd":
        print(json.dumps(bench_chunk_bwd(max(5, args.steps // 10), 2)))
        print(json.dumps(bench_chunk_bwd(max(5, args.steps // 10), 2, from_states=True)))
        return
    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}

    if args.only in ("chunk", "all"):
        wl, x, gout, t_warm, t_cold = bench_chunk(args.steps, args.warmup)
        B, T = x["q"].shape[:2]
        nbytes, flops = chunk_alg(wl, B * T, B)
        src = source_hash(*CHUNK_SRC)
        out.update({
            "value": B * T / t_warm, "unit": "tokens/s", "ms_per_step": t_warm * 1e3,
            "config": {"workload": wl.name, "batch": B, "seq_len": T, "h_k": wl.h_k,
                       "h_v": wl.h_v, "d_k": wl.d_k, "d_v": wl.d_v, "chunk_size": CHUNK,
                       "input_dtype": "bf16", "state_dtype": "fp32"},
            "roofline": {"bound": "hbm", "achieved": nbytes / t_warm / 1e9,
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": nbytes / t_warm / 1e9 / HBM_PEAK_GBPS,
                         "traffic": measured_traffic("chunk_fwd_t4096", src),
                         "kernel": "one gdn2_chunk_fwd call: prep_kernel, chunk_seg_kernel, chunk_state_kernel",
                         "alg_bytes": nbytes, "alg_flops": flops,
                         "mfma_frac_bf16": flops / t_warm / 1e12 / BF16_MFMA_PEAK_TFLOPS},
            "cold_cache": {"us_per_call": t_cold * 1e6, "tokens_per_s": B * T / t_cold,
                           "hbm_frac": nbytes / t_cold / 1e9 / HBM_PEAK_GBPS},
        })
        if not args.no_cpu_baseline:
            base, parity = cpu_baseline_chunk(wl, x, gout)
            out["cpu_baseline"] = base
            out["parity"] = parity
    if args.only in ("decode", "all"):
        dwl, t_step, t_graph, eager, graphed = bench_decode()
        dbytes, dstate, dflops = decode_alg(dwl)
        dsrc = source_hash("gdn2_decode.hip", "gdn2_common.h")
        dec = {"workload": dwl.name, "steps": dwl.steps, "us_per_step": t_step * 1e6,
               "timing": f"median over 5 timed passes of {dwl.steps} steps each, eager "
                         "launches; graph: the same steps captured once and replayed",
               "us_per_step_passes": [round(t * 1e6, 3) for t in eager],
               "us_per_step_graph": t_graph * 1e6,
               "us_per_step_graph_passes": [round(t * 1e6, 3) for t in graphed],
               "graph_hbm_frac": dbytes / t_graph / 1e9 / HBM_PEAK_GBPS,
               "tokens_per_s": dwl.num_seqs / t_step,
               "state_GBps": dstate / t_step / 1e9, "total_GBps": dbytes / t_step / 1e9,
               "roofline": {"bound": "hbm", "achieved": dbytes / t_step / 1e9,
                            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": dbytes / t_step / 1e9 / HBM_PEAK_GBPS,
                            "traffic": measured_traffic("decode_step_n64_hv48", dsrc),
                            "kernel": "recurrent_fwd_kernel", "alg_bytes": dbytes}}
        if not args.no_cpu_baseline:
            dec["cpu_baseline"] = cpu_baseline_decode(dwl)
        if not args.no_other_workloads:
            dec["large_state_control"] = bench_decode_large_state()
            dec["recurrent_variants"] = [bench_recurrent(1, torch.bfloat16, 256, 5,
                                                         "decode_step_bf16state_n64_hv48"),
                                         bench_recurrent(4, torch.float32, 64, 6),
                                         bench_recurrent(4, torch.bfloat16, 64, 7)]
        out["decode"] = dec
        if "value" not in out:
            out.update({"value": dwl.num_seqs / t_step, "unit": "tokens/s",
                        "ms_per_step": t_step * 1e3, "dtype": "f32",
                        "config": {"workload": dwl.name}, "roofline": dec["roofline"]})
    if args.only == "all" and not args.no_other_workloads:
        out["fused_qkl2norm_gatednorm"] = bench_fused(max(10, args.steps // 2), 3)
        out["gate_variants"] = bench_gate_variants(max(10, args.steps // 4), 3)
        out["chunk_states"] = bench_chunk_states(max(10, args.steps // 4), 3)
        out["chunk_bwd"] = bench_chunk_bwd(max(5, args.steps // 10), 2)
    t4096_f32 = dataclasses.replace(inputs.CHUNK_BF16_T4096, dtype=torch.float32,
                                    name="chunk_f32_b1_t4096_h16_d128_negeig")
    if args.only == "all" and not args.no_other_workloads:
        out["chunk_bwd_f32"] = bench_chunk_bwd(5, 2, wl=t4096_f32)
        out["chunk_bwd_from_states"] = bench_chunk_bwd(max(5, args.steps // 10), 2, from_states=True)
    if args.only in ("chunk", "all") and not args.no_other_workloads:
        out["other_chunk_workloads"] = [
            bench_chunk_workload(wl, max(10, args.steps // 4), 3, seed, chunk)
            for wl, seed, chunk in ((inputs.CHUNK_F32_SMALL, 2000, 64),
                                    (inputs.CHUNK_BF16_B8, 2001, 64),
                                    (inputs.VARLEN_BF16, 2004, 64),
                                    (inputs.CHUNK_BF16_T4096, 2002, 128),
                                    (inputs.CHUNK_BF16_T4096, 2002, 32),
                                    (t4096_f32, 2012, 64))]
    print(json.dumps(out))


if __name__ == "__main__":
    main()
