"""MI355X (gfx950) Gated DeltaNet-2 core -- Python binding of libgdn2.so.

This module only marshals arguments: it checks tensor shapes, allocates outputs and the
workspace with torch, and calls the C ABI (``include/gdn2.h``) on torch's current HIP
stream. Every step of the computation runs in the library's HIP kernels; there is no
CPU or PyTorch fallback, and the calls raise if the library is not built or the tensors
are not on a GPU.

    o, S_T = chunk_fwd(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, chunk_size=64)
    o      = recurrent_step(q, k, v, log_alpha, b, w, S)      # S updated in place
    o      = recurrent_fwd(q, k, v, log_alpha, b, w, state, state_idx=None)
                                      # T tokens per sequence against a state pool (fp32/bf16)

Layouts: q, k [B,T,H_k,d_k]; v, w [B,T,H_v,d_v]; log_alpha, b [B,T,H_v,d_k];
states [N,H_v,d_k,d_v] fp32. ``log_alpha`` is log of the decay (<= 0). Decode inputs drop
the T axis: q, k [N,H_k,d_k], v, w [N,H_v,d_v], log_alpha, b [N,H_v,d_k].
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_build", "libgdn2.so")

GDN2_F32, GDN2_BF16 = 0, 1
GDN2_STATE_F32, GDN2_STATE_BF16 = 0, 1
STATUS = {0: "GDN2_OK", 1: "GDN2_ERR_NULL_ARG", 2: "GDN2_ERR_BAD_SHAPE",
          3: "GDN2_ERR_UNSUPPORTED", 4: "GDN2_ERR_WORKSPACE", 5: "GDN2_ERR_HIP"}
CHUNK_SIZE = 64
STATIC_WORKSPACE_BYTES = 128 << 20    # GDN2_STATIC_WORKSPACE_BYTES of gdn2.h


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("h_k", ctypes.c_int32),
                ("h_v", ctypes.c_int32), ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class Fusion(ctypes.Structure):
    _fields_ = [("qk_l2norm", ctypes.c_int32), ("l2norm_eps", ctypes.c_float),
                ("gate", ctypes.c_void_p), ("norm_weight", ctypes.c_void_p),
                ("norm_eps", ctypes.c_float), ("conv_weight", ctypes.c_void_p),
                ("conv_state", ctypes.c_void_p), ("conv_silu", ctypes.c_int32),
                ("gate_mode", ctypes.c_int32), ("chunk_states", ctypes.c_void_p)]


class GDN2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgdn2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m gated_delta_rule_gdn_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        dp = ctypes.POINTER(Dims)
        L.gdn2_abi_version.restype = i32
        L.gdn2_abi_version.argtypes = []
        L.gdn2_status_string.restype = ctypes.c_char_p
        L.gdn2_status_string.argtypes = [i32]
        L.gdn2_last_error.restype = ctypes.c_char_p
        L.gdn2_last_error.argtypes = []
        L.gdn2_chunk_fwd_workspace_bytes.restype = sz
        L.gdn2_chunk_fwd_workspace_bytes.argtypes = [dp, i32]
        L.gdn2_chunk_fwd.restype = i32
        fp = ctypes.POINTER(Fusion)
        L.gdn2_chunk_fwd.argtypes = [vp] * 8 + [i32, vp, vp, dp, vp, sz, fp, vp]
        L.gdn2_recurrent_step.restype = i32
        L.gdn2_recurrent_step.argtypes = [vp] * 8 + [dp, vp]
        L.gdn2_recurrent_fwd.restype = i32
        L.gdn2_recurrent_fwd.argtypes = [vp] * 7 + [i32, vp, i32, vp, dp, fp, vp]
        L.gdn2_check_cu_seqlens.restype = i32
        L.gdn2_check_cu_seqlens.argtypes = [vp, i32, i32]
        L.gdn2_map_gates.restype = i32
        L.gdn2_map_gates.argtypes = [i32, dp] + [vp] * 13
        L.gdn2_map_gates_bwd.restype = i32
        L.gdn2_map_gates_bwd.argtypes = [i32, dp] + [vp] * 17
        L.gdn2_chunk_fwd_noalloc.restype = i32
        L.gdn2_chunk_fwd_noalloc.argtypes = [vp] * 8 + [i32, vp, vp, dp, fp, vp]
        L.gdn2_chunk_bwd_workspace_bytes.restype = sz
        L.gdn2_chunk_bwd_workspace_bytes.argtypes = [dp, i32]
        L.gdn2_chunk_bwd.restype = i32
        L.gdn2_chunk_bwd.argtypes = [vp] * 8 + [i32] + [vp] * 9 + [dp, vp, sz, vp]
        L.gdn2_chunk_bwd_states.restype = i32
        L.gdn2_chunk_bwd_states.argtypes = [vp] * 8 + [i32] + [vp] * 10 + [dp, vp, sz, vp]
        _lib = L
    return _lib


def _raise_on(status: int) -> None:
    if status != 0:
        msg = lib().gdn2_last_error().decode(errors="replace")
        raise GDN2Error(status, msg)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return GDN2_F32
    if t == torch.bfloat16:
        return GDN2_BF16
    raise TypeError(f"unsupported dtype {t}; use torch.float32 or torch.bfloat16")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need_gpu(name: str, t: torch.Tensor, device) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fusion(dev, out_shape, out_dtype, qk_l2norm, l2norm_eps, gate, norm_weight, norm_eps,
            conv=None, gate_mode=0, chunk_states=None):
    """The gdn2_fusion argument (None when nothing is fused). ``conv`` is
    (conv_weight, conv_state, conv_silu, channels, num_slots) or None."""
    if not qk_l2norm and gate is None and conv is None and not gate_mode and chunk_states is None:
        return None
    cw = cs = None
    silu = 0
    if conv is not None:
        cw, cs, silu, C, slots = conv
        _need_gpu("conv_weight", cw, dev)
        _need_gpu("conv_state", cs, dev)
        if cw.dtype != torch.float32 or tuple(cw.shape) != (C, 4):
            raise ValueError(f"conv_weight must be fp32 [{C},4]")
        if cs.dtype != torch.float32 or tuple(cs.shape) != (slots, 3, C):
            raise ValueError(f"conv_state must be fp32 [{slots},3,{C}]")
    if gate is not None:
        _need_gpu("gate", gate, dev)
        if gate.dtype != out_dtype or tuple(gate.shape) != tuple(out_shape):
            raise ValueError(f"gate must be {out_dtype} {tuple(out_shape)}")
        if norm_weight is None:
            raise ValueError("a gate needs norm_weight")
        _need_gpu("norm_weight", norm_weight, dev)
        if norm_weight.dtype != torch.float32 or tuple(norm_weight.shape) != (out_shape[-1],):
            raise ValueError(f"norm_weight must be fp32 [{out_shape[-1]}]")
    return Fusion(1 if qk_l2norm else 0, l2norm_eps, _ptr(gate), _ptr(norm_weight), norm_eps,
                  _ptr(cw), _ptr(cs), 1 if silu else 0, gate_mode, _ptr(chunk_states))


def _gate_shapes(mode, lead, Hv, dk, dv, log_alpha, b, w):
    """Checks log_alpha, b and w for a gate mode (None: the GDN-2 gates). Returns the mode
    code. See gdn2_fusion.gate_mode."""
    code = 0 if mode is None else GATE_MODES.get(mode)
    if code is None:
        raise ValueError(f"gate_mode must be None or one of {sorted(GATE_MODES)}")
    la_shape = lead + ((Hv,) if mode == "gdn" else (Hv, dk))
    b_shape = lead + ((Hv,) if mode in ("kda", "gdn") else (Hv, dk))
    if tuple(log_alpha.shape) != la_shape:
        raise ValueError(f"log_alpha must be {list(la_shape)}")
    if tuple(b.shape) != b_shape:
        raise ValueError(f"b must be {list(b_shape)}" + (f" (beta of mode {mode!r})" if mode else ""))
    if mode in (None, "fg2+"):
        if w is None or tuple(w.shape) != lead + (Hv, dv):
            raise ValueError(f"w must be {list(lead + (Hv, dv))}")
    elif w is not None:
        raise ValueError(f"gate mode {mode!r} takes no w (pass None)")
    if mode == "fg2" and dv != dk:
        raise ValueError("gate mode 'fg2' needs d_v = d_k")
    return code


def chunk_fwd_workspace_bytes(batch: int, seqlen: int, h_k: int, h_v: int, d_k: int, d_v: int,
                              dtype: torch.dtype, num_seqs: int = 0,
                              chunk_size: int = CHUNK_SIZE) -> int:
    d = Dims(batch, seqlen, num_seqs, h_k, h_v, d_k, d_v, _dtype_code(dtype))
    return int(lib().gdn2_chunk_fwd_workspace_bytes(ctypes.byref(d), chunk_size))


def _chunk_call(noalloc, q, k, v, log_alpha, b, w, S0, cu_seqlens, chunk_size,
                output_final_state, workspace, out, final_state, qk_l2norm, l2norm_eps, gate,
                norm_weight, norm_eps, gate_mode, chunk_states):
    """Shape checks, output allocation and the C call of chunk_fwd / chunk_fwd_noalloc."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("b", b), ("w", w)):
        if t is None and name == "w" and gate_mode not in (None, "fg2+"):
            continue
        _need_gpu(name, t, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError("q and k must both be [B,T,H_k,d_k]")
    B, T, Hk, dk = q.shape
    if v.dim() != 4 or v.shape[:2] != (B, T):
        raise ValueError("v must be [B,T,H_v,d_v]")
    Hv, dv = v.shape[2], v.shape[3]
    gcode = _gate_shapes(gate_mode, (B, T), Hv, dk, dv, log_alpha, b, w)
    if cu_seqlens is not None:
        _need_gpu("cu_seqlens", cu_seqlens, dev)
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if S0 is not None:
        _need_gpu("S0", S0, dev)
        if S0.dtype != torch.float32 or S0.shape != (N, Hv, dk, dv):
            raise ValueError(f"S0 must be fp32 [{N},{Hv},{dk},{dv}]")
    code = _dtype_code(q.dtype)
    dims = Dims(B, T, N if cu_seqlens is not None else 0, Hk, Hv, dk, dv, code)
    if not noalloc and workspace is None:
        need = int(lib().gdn2_chunk_fwd_workspace_bytes(ctypes.byref(dims), chunk_size))
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    o = out if out is not None else torch.empty(B, T, Hv, dv, dtype=q.dtype, device=dev)
    S_T = None
    if output_final_state:
        S_T = final_state if final_state is not None else torch.empty(
            N, Hv, dk, dv, dtype=torch.float32, device=dev)
    if chunk_states is not None:
        _need_gpu("chunk_states", chunk_states, dev)
        nc = num_chunks(T if cu_seqlens is None else cu_seqlens, B, chunk_size)
        if chunk_states.dtype != torch.float32 or chunk_states.shape != (nc, Hv, dk, dv):
            raise ValueError(f"chunk_states must be fp32 [{nc},{Hv},{dk},{dv}]")
    fu = _fusion(dev, (B, T, Hv, dv), q.dtype, qk_l2norm, l2norm_eps, gate, norm_weight,
                 norm_eps, gate_mode=gcode, chunk_states=chunk_states)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w), _ptr(S0),
            _ptr(cu_seqlens), chunk_size, _ptr(o), _ptr(S_T), ctypes.byref(dims))
    fptr = None if fu is None else ctypes.byref(fu)
    if noalloc:
        st = lib().gdn2_chunk_fwd_noalloc(*args, fptr, stream)
    else:
        st = lib().gdn2_chunk_fwd(*args, _ptr(workspace), workspace.numel(), fptr, stream)
    _raise_on(st)
    return o, S_T


def chunk_fwd(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None, chunk_size: int = CHUNK_SIZE,
              output_final_state: bool = True, workspace: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
              qk_l2norm: bool = False, l2norm_eps: float = 1e-6,
              gate: Optional[torch.Tensor] = None, norm_weight: Optional[torch.Tensor] = None,
              norm_eps: float = 1e-5, gate_mode: Optional[str] = None,
              chunk_states: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked WY forward. Returns (o [B,T,H_v,d_v], S_T [N,H_v,d_k,d_v] fp32 or None).

    chunk_states: an fp32 [num_chunks(...), H_v, d_k, d_v] buffer that receives the state
    entering every chunk (see num_chunks for the row of each sequence's chunks).

    qk_l2norm: L2-normalise q and k inside the kernels. gate [B,T,H_v,d_v] with norm_weight
    fp32 [d_v]: o is returned through the gated RMS norm o/rms(o) * weight * silu(gate).
    gate_mode ("kda", "gdn", "fg2", "fg2+"): run that variant natively; b carries its beta
    and w is None (or beta_v for "fg2+"), see map_gates for the shapes.
    """
    return _chunk_call(False, q, k, v, log_alpha, b, w, S0, cu_seqlens, chunk_size,
                       output_final_state, workspace, out, final_state, qk_l2norm, l2norm_eps,
                       gate, norm_weight, norm_eps, gate_mode, chunk_states)


def chunk_fwd_noalloc(q, k, v, log_alpha, b, w, S0=None, cu_seqlens=None,
                      chunk_size: int = CHUNK_SIZE, output_final_state: bool = True,
                      out: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                      l2norm_eps: float = 1e-6, gate: Optional[torch.Tensor] = None,
                      norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-5,
                      gate_mode: Optional[str] = None,
                      chunk_states: Optional[torch.Tensor] = None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """chunk_fwd through gdn2_chunk_fwd_noalloc: the workspace is the library's static device
    array (STATIC_WORKSPACE_BYTES per GPU), so the library allocates nothing. Pass `out` (and
    `final_state`) to allocate nothing on this side either. Calls that may overlap in time
    on one GPU must be ordered (they share the array)."""
    return _chunk_call(True, q, k, v, log_alpha, b, w, S0, cu_seqlens, chunk_size,
                       output_final_state, None, out, final_state, qk_l2norm, l2norm_eps,
                       gate, norm_weight, norm_eps, gate_mode, chunk_states)


def chunk_bwd_workspace_bytes(batch: int, seqlen: int, h_k: int, h_v: int, d_k: int, d_v: int,
                              dtype: torch.dtype, num_seqs: int = 0,
                              chunk_size: int = CHUNK_SIZE) -> int:
    d = Dims(batch, seqlen, num_seqs, h_k, h_v, d_k, d_v, _dtype_code(dtype))
    return int(lib().gdn2_chunk_bwd_workspace_bytes(ctypes.byref(d), chunk_size))


def chunk_bwd(q, k, v, log_alpha, b, w, dO, S0=None, cu_seqlens=None, dS_T=None,
              chunk_size: int = CHUNK_SIZE, workspace: Optional[torch.Tensor] = None,
              chunk_states: Optional[torch.Tensor] = None) -> dict:
    """Gradients of chunk_fwd (GDN-2 gates, no fusion options) given dO = dL/do and
    dS_T = dL/dS_T (None: zero). Returns fp32 tensors: dq, dk [B,T,H_k,d_k]; dv, dw
    [B,T,H_v,d_v]; dlog_alpha, db [B,T,H_v,d_k]; dS0 [N,H_v,d_k,d_v]. chunk_states: the
    chunk_states a chunk_size-64 chunk_fwd of the same inputs wrote (gdn2_chunk_bwd_states:
    the serial pass over the chunks is not re-run)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("b", b), ("w", w),
                    ("dO", dO)):
        _need_gpu(name, t, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError("q and k must both be [B,T,H_k,d_k]")
    B, T, Hk, dk_ = q.shape
    if v.dim() != 4 or v.shape[:2] != (B, T) or w.shape != v.shape or dO.shape != v.shape:
        raise ValueError("v, w and dO must be [B,T,H_v,d_v]")
    Hv, dv_ = v.shape[2], v.shape[3]
    if log_alpha.shape != (B, T, Hv, dk_) or b.shape != (B, T, Hv, dk_):
        raise ValueError("log_alpha and b must be [B,T,H_v,d_k]")
    if cu_seqlens is not None:
        _need_gpu("cu_seqlens", cu_seqlens, dev)
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for name, t in (("S0", S0), ("dS_T", dS_T)):
        if t is not None:
            _need_gpu(name, t, dev)
            if t.dtype != torch.float32 or t.shape != (N, Hv, dk_, dv_):
                raise ValueError(f"{name} must be fp32 [{N},{Hv},{dk_},{dv_}]")
    dims = Dims(B, T, N if cu_seqlens is not None else 0, Hk, Hv, dk_, dv_, _dtype_code(q.dtype))
    need = int(lib().gdn2_chunk_bwd_workspace_bytes(ctypes.byref(dims), chunk_size))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty(B, T, Hk, dk_, **f32), "dk": torch.empty(B, T, Hk, dk_, **f32),
           "dv": torch.empty(B, T, Hv, dv_, **f32), "dw": torch.empty(B, T, Hv, dv_, **f32),
           "dlog_alpha": torch.empty(B, T, Hv, dk_, **f32), "db": torch.empty(B, T, Hv, dk_, **f32),
           "dS0": torch.empty(N, Hv, dk_, dv_, **f32)}
    stream = torch.cuda.current_stream(dev).cuda_stream
    grads = [_ptr(out[n]) for n in ("dq", "dk", "dv", "dw", "dlog_alpha", "db", "dS0")]
    if chunk_states is None:
        st = lib().gdn2_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                  _ptr(S0), _ptr(cu_seqlens), chunk_size, _ptr(dO), _ptr(dS_T),
                                  *grads, ctypes.byref(dims), _ptr(workspace), workspace.numel(),
                                  stream)
    else:
        _need_gpu("chunk_states", chunk_states, dev)
        nc = num_chunks(T if cu_seqlens is None else cu_seqlens, B, chunk_size)
        if chunk_states.dtype != torch.float32 or chunk_states.shape != (nc, Hv, dk_, dv_):
            raise ValueError(f"chunk_states must be fp32 [{nc},{Hv},{dk_},{dv_}]")
        st = lib().gdn2_chunk_bwd_states(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b),
                                         _ptr(w), _ptr(S0), _ptr(cu_seqlens), chunk_size,
                                         _ptr(chunk_states), _ptr(dO), _ptr(dS_T), *grads,
                                         ctypes.byref(dims), _ptr(workspace), workspace.numel(),
                                         stream)
    _raise_on(st)
    return out


def num_chunks(seqlen_or_cu_seqlens, batch: int = 1, chunk_size: int = CHUNK_SIZE) -> int:
    """Rows of chunk_states: batch * ceil(T / chunk_size) for a dense batch (pass T), or
    sum_n ceil(len_n / chunk_size) for a packed one (pass cu_seqlens; a device tensor is
    copied to the host, which synchronises). Sequence n's chunks start at row
    n * ceil(T / chunk_size), respectively at the sum over the sequences before it."""
    if isinstance(seqlen_or_cu_seqlens, int):
        return batch * (-(-seqlen_or_cu_seqlens // chunk_size))
    cu = torch.as_tensor(seqlen_or_cu_seqlens).cpu().to(torch.int64)
    lens = cu[1:] - cu[:-1]
    return int(((lens + chunk_size - 1) // chunk_size).sum())


def recurrent_step(q, k, v, log_alpha, b, w, S, out: Optional[torch.Tensor] = None
                   ) -> torch.Tensor:
    """One fused decode step; S [N,H_v,d_k,d_v] fp32 is updated in place. Returns o."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("b", b), ("w", w)):
        _need_gpu(name, t, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    _need_gpu("S", S, dev)
    if q.dim() != 3 or k.shape != q.shape:
        raise ValueError("q and k must both be [N,H_k,d_k]")
    N, Hk, dk = q.shape
    if v.dim() != 3 or v.shape[0] != N or w.shape != v.shape:
        raise ValueError("v and w must both be [N,H_v,d_v]")
    Hv, dv = v.shape[1], v.shape[2]
    if log_alpha.shape != (N, Hv, dk) or b.shape != (N, Hv, dk):
        raise ValueError("log_alpha and b must be [N,H_v,d_k]")
    if S.dtype != torch.float32 or S.shape != (N, Hv, dk, dv):
        raise ValueError(f"S must be fp32 [{N},{Hv},{dk},{dv}]")
    dims = Dims(N, 1, 0, Hk, Hv, dk, dv, _dtype_code(q.dtype))
    o = out if out is not None else torch.empty(N, Hv, dv, dtype=q.dtype, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib().gdn2_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                   _ptr(S), _ptr(o), ctypes.byref(dims), stream)
    _raise_on(st)
    return o


def recurrent_fwd(q, k, v, log_alpha, b, w, state, state_idx: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                  l2norm_eps: float = 1e-6, gate: Optional[torch.Tensor] = None,
                  norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-5,
                  conv_weight: Optional[torch.Tensor] = None,
                  conv_state: Optional[torch.Tensor] = None, conv_silu: bool = False,
                  gate_mode: Optional[str] = None) -> torch.Tensor:
    """T tokens per sequence against a pool of recurrent states, updated in place.

    q, k [N,T,H_k,d_k]; v, w [N,T,H_v,d_v]; log_alpha, b [N,T,H_v,d_k] (fp32 or bf16);
    state [num_slots,H_v,d_k,d_v] fp32 or bf16; state_idx int32 [N] (slot of each sequence,
    None: slot n; out-of-range entries are padding: zero o rows, no state change).
    Returns o [N,T,H_v,d_v] in the input dtype. qk_l2norm, gate, norm_weight: as in chunk_fwd.
    conv_weight fp32 [C,4] with conv_state fp32 [num_slots,3,C], C = 2 H_k d_k + H_v d_v:
    the short causal convolution of q, k, v (channel order q, k, v), its state updated in
    place; conv_silu applies SiLU after it. gate_mode: as in chunk_fwd.
    """
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("b", b), ("w", w)):
        if t is None and name == "w" and gate_mode not in (None, "fg2+"):
            continue
        _need_gpu(name, t, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    _need_gpu("state", state, dev)
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError("q and k must both be [N,T,H_k,d_k]")
    N, T, Hk, dk = q.shape
    if v.dim() != 4 or v.shape[:2] != (N, T):
        raise ValueError("v must be [N,T,H_v,d_v]")
    Hv, dv = v.shape[2], v.shape[3]
    gcode = _gate_shapes(gate_mode, (N, T), Hv, dk, dv, log_alpha, b, w)
    if state.dim() != 4 or state.shape[1:] != (Hv, dk, dv):
        raise ValueError(f"state must be [num_slots,{Hv},{dk},{dv}]")
    if state.dtype == torch.float32:
        sdt = GDN2_STATE_F32
    elif state.dtype == torch.bfloat16:
        sdt = GDN2_STATE_BF16
    else:
        raise TypeError("state must be float32 or bfloat16")
    if state_idx is not None:
        _need_gpu("state_idx", state_idx, dev)
        if state_idx.dtype != torch.int32 or state_idx.shape != (N,):
            raise ValueError(f"state_idx must be int32 [{N}]")
    dims = Dims(N, T, 0, Hk, Hv, dk, dv, _dtype_code(q.dtype))
    o = out if out is not None else torch.empty(N, T, Hv, dv, dtype=q.dtype, device=dev)
    conv = None
    if conv_weight is not None or conv_state is not None:
        if conv_weight is None or conv_state is None:
            raise ValueError("conv_weight and conv_state go together")
        conv = (conv_weight, conv_state, conv_silu, 2 * Hk * dk + Hv * dv, state.shape[0])
    fu = _fusion(dev, (N, T, Hv, dv), q.dtype, qk_l2norm, l2norm_eps, gate, norm_weight,
                 norm_eps, conv, gate_mode=gcode)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib().gdn2_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(b), _ptr(w),
                                  _ptr(state), sdt, _ptr(state_idx), state.shape[0], _ptr(o),
                                  ctypes.byref(dims), None if fu is None else ctypes.byref(fu),
                                  stream)
    _raise_on(st)
    return o


# gdn2_gate_mode: other delta-rule variants as GDN-2 inputs (include/gdn2.h)
GATE_MODES = {"kda": 1, "fg2": 2, "fg2+": 3, "gdn": 4}


def map_gates(mode: str, q, k, v, log_alpha, beta, beta_v=None):
    """Maps the inputs of a delta-rule variant onto GDN-2 inputs, on the GPU (gdn2_map_gates).

    Leading dims L are those of q ([*L, H_k, d_k]: [B,T], [1,T] packed or [N,T] recurrent).
      "kda"   beta [*L, H_v]; log_alpha [*L, H_v, d_k]:  b = w = beta
      "gdn"   beta [*L, H_v]; log_alpha [*L, H_v] (scalar decay): broadcast over d_k
      "fg2"   beta [*L, H_v, d_k], d_v = d_k: k' = sqrt(beta) k, v' = sqrt(beta) v, b = w = 1
      "fg2+"  beta [*L, H_v, d_k], beta_v [*L, H_v, d_v]: k' = sqrt(beta) k, b = 1,
              w = sqrt(beta_v)
    Returns (q', k', v', log_alpha', b, w) for chunk_fwd / recurrent_fwd. In the FG2 modes k'
    (and q', when H_v > H_k) is per value head.
    """
    if mode not in GATE_MODES:
        raise ValueError(f"mode must be one of {sorted(GATE_MODES)}")
    code = GATE_MODES[mode]
    dev = q.device
    if q.dim() < 3 or k.shape != q.shape:
        raise ValueError("q and k must both be [*L, H_k, d_k]")
    lead, Hk, dk = tuple(q.shape[:-2]), q.shape[-2], q.shape[-1]
    if v.dim() != q.dim() or tuple(v.shape[:-2]) != lead:
        raise ValueError("v must be [*L, H_v, d_v]")
    Hv, dv = v.shape[-2], v.shape[-1]
    scalar = mode in ("kda", "gdn")
    want_beta = lead + ((Hv,) if scalar else (Hv, dk))
    want_la = lead + ((Hv,) if mode == "gdn" else (Hv, dk))
    if tuple(beta.shape) != want_beta:
        raise ValueError(f"beta must be {list(want_beta)} for mode {mode!r}")
    if tuple(log_alpha.shape) != want_la:
        raise ValueError(f"log_alpha must be {list(want_la)} for mode {mode!r}")
    if mode == "fg2+":
        if beta_v is None or tuple(beta_v.shape) != lead + (Hv, dv):
            raise ValueError(f"beta_v must be {list(lead + (Hv, dv))} for mode 'fg2+'")
    elif beta_v is not None:
        raise ValueError("beta_v is for mode 'fg2+' only")
    for name, t in (("q", q), ("k", k), ("v", v), ("log_alpha", log_alpha), ("beta", beta),
                    ("beta_v", beta_v)):
        if t is None:
            continue
        _need_gpu(name, t, dev)
        if t.dtype != q.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {q.dtype}")
    rows = 1
    for x in lead:
        rows *= x
    dims = Dims(rows, 1, 0, Hk, Hv, dk, dv, _dtype_code(q.dtype))
    new = lambda *shape: torch.empty(*shape, dtype=q.dtype, device=dev)  # noqa: E731
    b, w = new(*lead, Hv, dk), new(*lead, Hv, dv)
    q2, k2, v2, la2 = q, k, v, log_alpha
    if mode == "gdn":
        la2 = new(*lead, Hv, dk)
    if mode in ("fg2", "fg2+"):
        k2 = new(*lead, Hv, dk)
        if Hv > Hk:
            q2 = new(*lead, Hv, dk)
    if mode == "fg2":
        v2 = new(*lead, Hv, dv)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib().gdn2_map_gates(code, ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v),
                              _ptr(log_alpha), _ptr(beta), _ptr(beta_v),
                              _ptr(q2) if q2 is not q else None, _ptr(k2) if k2 is not k else None,
                              _ptr(v2) if v2 is not v else None,
                              _ptr(la2) if la2 is not log_alpha else None, _ptr(b), _ptr(w),
                              stream)
    _raise_on(st)
    return q2, k2, v2, la2, b, w


def map_gates_bwd(mode: str, k, v, beta, grads: dict, beta_v=None) -> dict:
    """The chain rule back through map_gates, on the GPU (gdn2_map_gates_bwd). k, v, beta and
    beta_v are map_gates' inputs; grads holds the fp32 gradients of the mapped inputs (the
    dq, dk, dv, dlog_alpha, db, dw of chunk_bwd run on map_gates' outputs). Returns the
    gradients with respect to the variant's own inputs: dq, dk, dv, dlog_alpha, dbeta (and
    dbeta_v for "fg2+"), fp32, in the shapes of map_gates' inputs; those the mapping does not
    change are the tensors of grads themselves."""
    if mode not in GATE_MODES:
        raise ValueError(f"mode must be one of {sorted(GATE_MODES)}")
    code = GATE_MODES[mode]
    dev = k.device
    lead, Hk, dk = tuple(k.shape[:-2]), k.shape[-2], k.shape[-1]
    Hv, dv = v.shape[-2], v.shape[-1]
    fg2 = mode in ("fg2", "fg2+")
    for name, t in (("k", k), ("v", v), ("beta", beta), ("beta_v", beta_v)):
        if t is not None:
            _need_gpu(name, t, dev)
            if t.dtype != k.dtype:
                raise TypeError(f"{name} has dtype {t.dtype}, expected {k.dtype}")
    want = {"dq": lead + ((Hv,) if fg2 else (Hk,)) + (dk,), "dk": lead + ((Hv,) if fg2 else (Hk,)) + (dk,),
            "dv": lead + (Hv, dv), "dw": lead + (Hv, dv), "dlog_alpha": lead + (Hv, dk),
            "db": lead + (Hv, dk)}
    for n, shape in want.items():
        t = grads[n]
        _need_gpu(n, t, dev)
        if t.dtype != torch.float32 or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"grads[{n!r}] must be contiguous fp32 {list(shape)}")
    rows = 1
    for x in lead:
        rows *= x
    dims = Dims(rows, 1, 0, Hk, Hv, dk, dv, _dtype_code(k.dtype))
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": grads["dq"], "dk": grads["dk"], "dv": grads["dv"], "dlog_alpha": grads["dlog_alpha"]}
    dq = dk_ = dv_ = dla = dbv = None
    if fg2:
        dk_ = out["dk"] = torch.empty(*lead, Hk, dk, **f32)
        if Hv > Hk:
            dq = out["dq"] = torch.empty(*lead, Hk, dk, **f32)
        else:
            out["dq"] = grads["dq"].view(*lead, Hk, dk)
    if mode == "fg2":
        dv_ = out["dv"] = torch.empty(*lead, Hv, dv, **f32)
    if mode == "gdn":
        dla = out["dlog_alpha"] = torch.empty(*lead, Hv, **f32)
    dbeta = out["dbeta"] = torch.empty(*(lead + ((Hv,) if mode in ("kda", "gdn") else (Hv, dk))), **f32)
    if mode == "fg2+":
        dbv = out["dbeta_v"] = torch.empty(*lead, Hv, dv, **f32)
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib().gdn2_map_gates_bwd(code, ctypes.byref(dims), _ptr(k), _ptr(v), _ptr(beta),
                                  _ptr(beta_v), _ptr(grads["dq"]), _ptr(grads["dk"]),
                                  _ptr(grads["dv"]), _ptr(grads["dlog_alpha"]), _ptr(grads["db"]),
                                  _ptr(grads["dw"]), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dla),
                                  _ptr(dbeta), _ptr(dbv), stream)
    _raise_on(st)
    return out


def _fg2_fusion_check(mode, kw):
    if mode in ("fg2", "fg2+") and (kw.get("qk_l2norm") or kw.get("conv_weight") is not None):
        raise ValueError("the fused q/k L2-norm and short convolution would act on the scaled "
                         "keys of the FG2 modes; normalise or convolve q and k before mapping")


def gated_chunk_fwd(mode: str, q, k, v, log_alpha, beta, beta_v=None, mapped: bool = False,
                    **kw):
    """chunk_fwd of a delta-rule variant (shapes as in map_gates). By default the variant
    runs natively (gdn2_fusion.gate_mode: the kernels read beta); mapped=True runs
    map_gates first and then the plain GDN-2 call. Keyword arguments go to chunk_fwd."""
    _fg2_fusion_check(mode, kw)
    if mapped:
        return chunk_fwd(*map_gates(mode, q, k, v, log_alpha, beta, beta_v), **kw)
    if mode not in GATE_MODES:
        raise ValueError(f"mode must be one of {sorted(GATE_MODES)}")
    return chunk_fwd(q, k, v, log_alpha, beta, beta_v, gate_mode=mode, **kw)


def gated_recurrent_fwd(mode: str, q, k, v, log_alpha, beta, state, beta_v=None,
                        mapped: bool = False, **kw):
    """recurrent_fwd of a delta-rule variant against a state pool (native by default, as in
    gated_chunk_fwd). Keyword arguments go to recurrent_fwd."""
    _fg2_fusion_check(mode, kw)
    if mapped:
        return recurrent_fwd(*map_gates(mode, q, k, v, log_alpha, beta, beta_v), state, **kw)
    if mode not in GATE_MODES:
        raise ValueError(f"mode must be one of {sorted(GATE_MODES)}")
    return recurrent_fwd(q, k, v, log_alpha, beta, beta_v, state, gate_mode=mode, **kw)


def abi_version() -> int:
    return int(lib().gdn2_abi_version())
