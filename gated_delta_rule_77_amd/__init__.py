"""Python binding of libkda, the MI355X Kimi Delta Attention (KDA) core.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkda.so (built in-tree by `python -m gated_delta_rule_77_amd.build`).
PyTorch supplies device memory and the current stream.  There is no fallback:
if the library is not built, or a tensor is not on a GPU, the call raises.

Names follow the C ABI in include/kda.h:
    kda_chunk_fwd(q, k, v, g, beta, A, initial_state=None, cu_seqlens=None,
                  chunk_size=64, output_final_state=True, workspace=None) -> (o, hT)
    kda_recurrent_step(q, k, v, g, beta, A, state) -> o     (state updated in place)
    kda_recurrent_verify(q, k, v, g, beta, A, state) -> o    (window outputs, state read only)
    kda_recurrent_fold(k, v, g, beta, A, n_accept, state)    (state updated in place)
    kda_layer_fwd(q_in, k_in, v_in, conv_w, g, beta, A, gate, norm_w, ...) -> (y, hT, conv_state)
    kda_layer_step(q_in, k_in, v_in, conv_w, conv_state, g, beta, A, state, gate, norm_w) -> y
    kda_chunk_fwd_noalloc(q, k, v, g, beta, A, o, final_state=None, ...) -> (o, hT)
    kda_chunk_fwd_debug(...) -> (o, hT, intermediates)
    kda_chunk_fwd_mode(q, k, v, g, beta, A, mode, ...) -> (o, hT)  ("kda", "gla", "deltanet")
    kda_recurrent_step_mode(q, k, v, g, beta, A, state, mode) -> o
    kda_dplr_chunk_fwd(q, k, v, a, b, g, A, ...) -> (o, hT)      (general DPLR update)
    kda_dplr_recurrent_step(q, k, v, a, b, g, A, state) -> o
`g` are the raw per-channel gate logits and `beta` the raw write-strength
logits; both activations run inside the kernels.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "KdaError", "lib", "lib_path", "kda_chunk_fwd", "kda_recurrent_step", "kda_recurrent_fold",
    "kda_recurrent_verify", "kda_layer_fwd", "kda_layer_step", "kda_layer_fwd_workspace_bytes",
    "kda_chunk_fwd_debug", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd_supported",
    "kda_recurrent_step_supported", "kda_chunk_fwd_mode", "kda_recurrent_step_mode", "MODES",
    "kda_dplr_chunk_fwd", "kda_dplr_recurrent_step", "kda_dplr_chunk_fwd_workspace_bytes",
    "kda_chunk_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
EXPORTED_SYMBOLS = (
    "kda_status_string", "kda_chunk_fwd_supported", "kda_recurrent_step_supported",
    "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_chunk_fwd_debug_floats",
    "kda_chunk_fwd_debug", "kda_chunk_fwd_timed", "kda_recurrent_step", "kda_recurrent_fold",
    "kda_layer_fwd_workspace_bytes", "kda_layer_fwd", "kda_layer_step", "kda_chunk_fwd_mode",
    "kda_recurrent_step_mode", "kda_dplr_chunk_fwd_workspace_bytes", "kda_dplr_chunk_fwd",
    "kda_dplr_chunk_fwd_timed", "kda_dplr_recurrent_step", "kda_recurrent_verify",
    "kda_chunk_fwd_noalloc",
)
# bytes of the per-GPU scratch array behind kda_chunk_fwd_noalloc (include/kda.h)
NOALLOC_SCRATCH_BYTES = 128 << 20
# family modes of kda_chunk_fwd_mode / kda_recurrent_step_mode (kda_mode_t)
MODES = {"kda": 0, "gla": 1, "deltanet": 2}


def _mode_code(mode) -> int:
    if isinstance(mode, str):
        if mode not in MODES:
            raise ValueError(f"mode must be one of {sorted(MODES)}, got {mode!r}")
        return MODES[mode]
    return int(mode)


class KdaError(RuntimeError):
    """A libkda call returned a non-OK status."""


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise KdaError(f"{lib_path} is not built; run `python -m gated_delta_rule_77_amd.build`")
    L = ctypes.CDLL(lib_path)
    vp, f, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [i]
    L.kda_chunk_fwd_supported.restype = i
    L.kda_chunk_fwd_supported.argtypes = [i, i, i, i]
    L.kda_recurrent_step_supported.restype = i
    L.kda_recurrent_step_supported.argtypes = [i, i, i]
    L.kda_chunk_fwd_workspace_bytes.restype = sz
    L.kda_chunk_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    L.kda_chunk_fwd_debug_floats.restype = sz
    L.kda_chunk_fwd_debug_floats.argtypes = [i, i, i, i, i, i, i,
                                             ctypes.POINTER(sz), ctypes.POINTER(i)]
    chunk_args = [vp, vp, vp, f, f, f, f, vp, i, i, i, i, i, i, i, i, vp, f, vp, sz]
    L.kda_chunk_fwd.restype = i
    L.kda_chunk_fwd.argtypes = chunk_args + [vp]
    L.kda_chunk_fwd_debug.restype = i
    L.kda_chunk_fwd_debug.argtypes = chunk_args + [f, f, vp]
    L.kda_chunk_fwd_noalloc.restype = i
    L.kda_chunk_fwd_noalloc.argtypes = chunk_args[:18] + [vp]
    L.kda_chunk_fwd_timed.restype = i
    L.kda_chunk_fwd_timed.argtypes = chunk_args + [ctypes.POINTER(vp), i, vp]
    L.kda_recurrent_step.restype = i
    L.kda_recurrent_step.argtypes = [vp, vp, vp, f, f, f, f, vp, i, i, i, i, i, vp]
    L.kda_recurrent_fold.restype = i
    L.kda_recurrent_fold.argtypes = [vp, vp, f, f, f, vp, f, i, i, i, i, i, i, vp]
    fl = ctypes.c_float
    L.kda_layer_fwd_workspace_bytes.restype = sz
    L.kda_layer_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.kda_layer_fwd.restype = i
    L.kda_layer_fwd.argtypes = ([vp, vp, vp, f, vp, vp, f, f, f, f, vp, vp, f, fl, fl]
                                + [i] * 7 + [vp, f, vp, sz, vp])
    L.kda_layer_step.restype = i
    L.kda_layer_step.argtypes = [vp, vp, vp, f, vp, f, f, f, f, vp, f, fl, fl, vp, i, i, i, i, vp]
    L.kda_chunk_fwd_mode.restype = i
    L.kda_chunk_fwd_mode.argtypes = chunk_args[:16] + [i] + chunk_args[16:] + [vp]
    L.kda_recurrent_step_mode.restype = i
    L.kda_recurrent_step_mode.argtypes = [vp, vp, vp, f, f, f, f, vp, i, i, i, i, i, i, vp]
    L.kda_dplr_chunk_fwd_workspace_bytes.restype = sz
    L.kda_dplr_chunk_fwd_workspace_bytes.argtypes = [i] * 8
    L.kda_dplr_chunk_fwd.restype = i
    L.kda_dplr_chunk_fwd.argtypes = [vp, vp, vp, vp, vp, f, f, f, vp] + [i] * 8 + [vp, f, vp, sz, vp]
    L.kda_dplr_chunk_fwd_timed.restype = i
    L.kda_dplr_chunk_fwd_timed.argtypes = ([vp, vp, vp, vp, vp, f, f, f, vp] + [i] * 8
                                           + [vp, f, vp, sz, ctypes.POINTER(vp), i, vp])
    L.kda_recurrent_verify.restype = i
    L.kda_recurrent_verify.argtypes = [vp, vp, vp, f, f, f, f, vp] + [i] * 6 + [vp]
    L.kda_dplr_recurrent_step.restype = i
    L.kda_dplr_recurrent_step.argtypes = [vp, vp, vp, vp, vp, f, f, f, vp] + [i] * 5 + [vp]
    _lib = L
    return L


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise KdaError(f"{what}: {lib().kda_status_string(rc).decode()}")


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _req(t, name, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _workspace(workspace, need: int, device):
    """The caller's workspace, or a fresh one when the caller passes none.

    A caller who passes a workspace owns the call's scratch memory and gets no
    allocation: it must be a contiguous uint8 tensor on `device`, at least
    `need` bytes long and 256-byte aligned, or the call raises KdaError before
    anything is enqueued."""
    torch = _torch()
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device)
    _req(workspace, "workspace", torch.uint8, device)
    if workspace.numel() < need:
        raise KdaError(f"workspace holds {workspace.numel()} bytes; this call needs {need}")
    if workspace.data_ptr() % 256:
        raise KdaError("workspace must be 256-byte aligned")
    return workspace


def _stream(device) -> int:
    return _torch().cuda.current_stream(device).cuda_stream


def kda_chunk_fwd_supported(dk: int, dv: int, chunk: int, dtype) -> bool:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return bool(lib().kda_chunk_fwd_supported(dk, dv, chunk, code))


def kda_recurrent_step_supported(dk: int, dv: int, dtype) -> bool:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return bool(lib().kda_recurrent_step_supported(dk, dv, code))


def kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(lib().kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, chunk, code))


def _prefill_args(q, k, v, g, beta, A, initial_state, cu_seqlens, gated=True):
    torch = _torch()
    _req(q, "q")
    dev = q.device
    dt = q.dtype
    _dtype_code(q)
    _req(k, "k", dt, dev)
    _req(v, "v", dt, dev)
    if beta is not None:            # None only for the general DPLR call, which has no beta
        _req(beta, "beta", torch.float32, dev)
    if gated or g is not None:
        _req(g, "g", torch.float32, dev)
    if gated or A is not None:
        _req(A, "A", torch.float32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, T, H, dv) or (g is not None and g.shape != q.shape):
        raise ValueError("k, g must match q [B, T, H, dk] and v must be [B, T, H, dv]")
    if (beta is not None and beta.shape != (B, T, H)) or (A is not None and A.shape != (H,)):
        raise ValueError("beta must be [B, T, H] and A must be [H]")
    if cu_seqlens is not None:
        _req(cu_seqlens, "cu_seqlens", torch.int32, dev)
        if B != 1 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens needs B == 1 and a 1-D int32 tensor of N+1 offsets")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _req(initial_state, "initial_state", torch.float32, dev)
        if initial_state.shape != (N, H, dk, dv):
            raise ValueError(f"initial_state must be [{N}, {H}, {dk}, {dv}]")
    return B, T, H, dk, dv, N, dev, dt


def kda_chunk_fwd(q, k, v, g, beta, A, initial_state=None, cu_seqlens=None,
                  chunk_size: int = 64, output_final_state: bool = True, workspace=None):
    """Chunked prefill.  q, k [B, T, H, dk], v [B, T, H, dv] (bf16 or fp32);
    g [B, T, H, dk] fp32 gate logits; beta [B, T, H] fp32 logits; A [H] fp32;
    initial_state [N, H, dk, dv] fp32 or None; cu_seqlens int32 [N+1] or None.
    Returns (o [B, T, H, dv], final_state [N, H, dk, dv] fp32 or None)."""
    return _chunk(q, k, v, g, beta, A, initial_state, cu_seqlens, chunk_size,
                  output_final_state, workspace, debug=False)


def kda_chunk_fwd_noalloc(q, k, v, g, beta, A, o, final_state=None, initial_state=None,
                          cu_seqlens=None, chunk_size: int = 64):
    """kda_chunk_fwd without a workspace and without allocating: the caller
    passes the output o [B, T, H, dv] (dtype of q) and, if wanted, the final
    state [N, H, dk, dv] fp32; the library's per-GPU scratch array serves as
    the workspace (calls beyond its size raise KdaError: KDA_ERR_SCRATCH).
    Calls that overlap on one GPU race on that array.  Returns (o, final_state)."""
    torch = _torch()
    B, T, H, dk, dv, N, dev, dt = _prefill_args(q, k, v, g, beta, A, initial_state, cu_seqlens)
    _req(o, "o", dt, dev)
    if o.shape != (B, T, H, dv):
        raise ValueError(f"o must be [{B}, {T}, {H}, {dv}]")
    if final_state is not None:
        _req(final_state, "final_state", torch.float32, dev)
        if final_state.shape != (N, H, dk, dv):
            raise ValueError(f"final_state must be [{N}, {H}, {dk}, {dv}]")
    _check(lib().kda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A),
                                       _ptr(initial_state), _ptr(cu_seqlens), B, T, H, dk, dv, N,
                                       chunk_size, _dtype_code(q), _ptr(o), _ptr(final_state),
                                       _stream(dev)), "kda_chunk_fwd_noalloc")
    return o, final_state


def kda_chunk_fwd_debug(q, k, v, g, beta, A, initial_state=None, cu_seqlens=None,
                        chunk_size: int = 64, workspace=None):
    """kda_chunk_fwd plus per-chunk intermediates: returns (o, hT, dict) with
    G [Cn, H, c, dk], Akk/Aqk/T [Cn, H, c, c], S0 [Cn, H, dk, dv] (fp32) and
    the number of chunks actually used is not returned: chunks are numbered
    sequence by sequence in token order, unused slots are left untouched."""
    return _chunk(q, k, v, g, beta, A, initial_state, cu_seqlens, chunk_size,
                  True, workspace, debug=True)


def kda_chunk_fwd_mode(q, k, v, g, beta, A, mode, initial_state=None, cu_seqlens=None,
                       chunk_size: int = 64, output_final_state: bool = True, workspace=None):
    """kda_chunk_fwd in a family mode: "kda", "gla" (erase off) or "deltanet"
    (alpha = 1; g and A may be None)."""
    return _chunk(q, k, v, g, beta, A, initial_state, cu_seqlens, chunk_size,
                  output_final_state, workspace, debug=False, mode=_mode_code(mode))


def _chunk(q, k, v, g, beta, A, initial_state, cu_seqlens, chunk_size, output_final_state,
           workspace, debug, mode=None):
    torch = _torch()
    B, T, H, dk, dv, N, dev, dt = _prefill_args(q, k, v, g, beta, A, initial_state, cu_seqlens,
                                                gated=mode != MODES["deltanet"])
    code = _dtype_code(q)
    L = lib()
    need = int(L.kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, chunk_size, code))
    if need == 0:
        _check(2 if not L.kda_chunk_fwd_supported(dk, dv, chunk_size, code) else 1,
               "kda_chunk_fwd_workspace_bytes")
    workspace = _workspace(workspace, need, dev)
    o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A), _ptr(initial_state),
            _ptr(cu_seqlens), B, T, H, dk, dv, N, chunk_size, code, _ptr(o), _ptr(hT),
            _ptr(workspace), workspace.numel())
    if mode is not None:
        _check(L.kda_chunk_fwd_mode(*args[:16], mode, *args[16:], _stream(dev)),
               "kda_chunk_fwd_mode")
        return o, hT
    if not debug:
        _check(L.kda_chunk_fwd(*args, _stream(dev)), "kda_chunk_fwd")
        return o, hT
    st = ctypes.c_size_t(0)
    cap = ctypes.c_int(0)
    nf = int(L.kda_chunk_fwd_debug_floats(B, T, H, dk, dv, N, chunk_size, ctypes.byref(st),
                                          ctypes.byref(cap)))
    dbg = torch.zeros(max(nf, 1), dtype=torch.float32, device=dev)
    dst = torch.zeros(max(int(st.value), 1), dtype=torch.float32, device=dev)
    _check(L.kda_chunk_fwd_debug(*args, _ptr(dbg), _ptr(dst), _stream(dev)), "kda_chunk_fwd_debug")
    Cn, c = cap.value, chunk_size
    per = c * dk + 3 * c * c
    d = dbg[: Cn * H * per].view(Cn, H, per)
    inter = dict(
        G=d[:, :, : c * dk].reshape(Cn, H, c, dk),
        Akk=d[:, :, c * dk: c * dk + c * c].reshape(Cn, H, c, c),
        Aqk=d[:, :, c * dk + c * c: c * dk + 2 * c * c].reshape(Cn, H, c, c),
        T=d[:, :, c * dk + 2 * c * c:].reshape(Cn, H, c, c),
        S0=dst[: Cn * H * dk * dv].view(Cn, H, dk, dv),
        capacity=Cn,
    )
    return o, hT, inter


def kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(lib().kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, chunk, code))


def kda_dplr_chunk_fwd(q, k, v, a, b, g, A, initial_state=None, cu_seqlens=None,
                       chunk_size: int = 64, output_final_state: bool = True, workspace=None):
    """General DPLR prefill: S' = Diag(alpha) S, S'' = S' + a (b^T S'),
    S = S'' + k v^T, o = S^T q.  q, k, a, b [B, T, H, dk], v [B, T, H, dv]
    (bf16 or fp32), g [B, T, H, dk] fp32 gate logits, A [H] fp32; the rest as
    kda_chunk_fwd.  Returns (o, final_state or None)."""
    torch = _torch()
    B, T, H, dk, dv, N, dev, dt = _prefill_args(q, k, v, g, None, A, initial_state, cu_seqlens)
    _req(a, "a", dt, dev)
    _req(b, "b", dt, dev)
    if a.shape != q.shape or b.shape != q.shape:
        raise ValueError("a and b must match q [B, T, H, dk]")
    code = _dtype_code(q)
    L = lib()
    need = int(L.kda_dplr_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, chunk_size, code))
    if need == 0:
        _check(2 if not L.kda_chunk_fwd_supported(dk, dv, chunk_size, code) else 1,
               "kda_dplr_chunk_fwd_workspace_bytes")
    workspace = _workspace(workspace, need, dev)
    o = torch.empty((B, T, H, dv), dtype=dt, device=dev)
    hT = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev) if output_final_state else None
    _check(L.kda_dplr_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(g), _ptr(A),
                                _ptr(initial_state), _ptr(cu_seqlens), B, T, H, dk, dv, N,
                                chunk_size, code, _ptr(o), _ptr(hT), _ptr(workspace),
                                workspace.numel(), _stream(dev)), "kda_dplr_chunk_fwd")
    return o, hT


def kda_dplr_recurrent_step(q, k, v, a, b, g, A, state):
    """One general-DPLR token per sequence: q, k, a, b [N, H, dk], v [N, H, dv]
    (bf16 or fp32), g [N, H, dk] fp32, A [H] fp32, state [N, H, dk, dv] fp32
    (updated in place).  Returns o [N, H, dv]."""
    torch = _torch()
    _req(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    for t, name in ((k, "k"), (v, "v"), (a, "a"), (b, "b")):
        _req(t, name, dt, dev)
    _req(g, "g", torch.float32, dev)
    _req(A, "A", torch.float32, dev)
    _req(state, "state", torch.float32, dev)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    if any(t.shape != q.shape for t in (k, a, b, g)) or v.shape != (N, H, dv):
        raise ValueError("k, a, b, g must match q [N, H, dk] and v must be [N, H, dv]")
    if A.shape != (H,) or state.shape != (N, H, dk, dv):
        raise ValueError("A [H] and state [N, H, dk, dv] expected")
    o = torch.empty((N, H, dv), dtype=dt, device=dev)
    _check(lib().kda_dplr_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(g),
                                         _ptr(A), _ptr(state), _ptr(o), N, H, dk, dv, code,
                                         _stream(dev)), "kda_dplr_recurrent_step")
    return o


def kda_recurrent_step(q, k, v, g, beta, A, state):
    """One decode token per sequence: q, k [N, H, dk], v [N, H, dv] (bf16 or
    fp32), g [N, H, dk] fp32, beta [N, H] fp32, A [H] fp32, state
    [N, H, dk, dv] fp32 (updated in place).  Returns o [N, H, dv]."""
    return _step(q, k, v, g, beta, A, state, None)


def kda_recurrent_step_mode(q, k, v, g, beta, A, state, mode):
    """kda_recurrent_step in a family mode ("kda", "gla", "deltanet"; with
    "deltanet" g and A may be None)."""
    return _step(q, k, v, g, beta, A, state, _mode_code(mode))


def _step(q, k, v, g, beta, A, state, mode):
    torch = _torch()
    _req(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    gated = mode != MODES["deltanet"]
    _req(k, "k", dt, dev)
    _req(v, "v", dt, dev)
    if gated or g is not None:
        _req(g, "g", torch.float32, dev)
    if gated or A is not None:
        _req(A, "A", torch.float32, dev)
    _req(beta, "beta", torch.float32, dev)
    _req(state, "state", torch.float32, dev)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or (g is not None and g.shape != q.shape) or v.shape != (N, H, dv):
        raise ValueError("k, g must match q [N, H, dk] and v must be [N, H, dv]")
    if beta.shape != (N, H) or (A is not None and A.shape != (H,)) or state.shape != (N, H, dk, dv):
        raise ValueError("beta [N, H], A [H] and state [N, H, dk, dv] expected")
    o = torch.empty((N, H, dv), dtype=dt, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A), _ptr(state), _ptr(o),
            N, H, dk, dv, code)
    if mode is None:
        _check(lib().kda_recurrent_step(*args, _stream(dev)), "kda_recurrent_step")
    else:
        _check(lib().kda_recurrent_step_mode(*args, mode, _stream(dev)), "kda_recurrent_step_mode")
    return o


def kda_recurrent_verify(q, k, v, g, beta, A, state):
    """Outputs of every token of each sequence's draft window from the
    checkpoint state, which is only read: q, k [N, W, H, dk], v [N, W, H, dv]
    (bf16 or fp32), g [N, W, H, dk] fp32, beta [N, W, H] fp32, A [H] fp32,
    state [N, H, dk, dv] fp32.  Returns o [N, W, H, dv], bit-identical to W
    kda_recurrent_step calls on a copy of the state."""
    torch = _torch()
    _req(q, "q")
    dev, dt = q.device, q.dtype
    code = _dtype_code(q)
    _req(k, "k", dt, dev)
    _req(v, "v", dt, dev)
    _req(g, "g", torch.float32, dev)
    _req(beta, "beta", torch.float32, dev)
    _req(A, "A", torch.float32, dev)
    _req(state, "state", torch.float32, dev)
    if q.dim() != 4:
        raise ValueError("q must be [N, W, H, dk]")
    N, W, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or g.shape != q.shape or v.shape != (N, W, H, dv):
        raise ValueError("k, g must match q [N, W, H, dk] and v must be [N, W, H, dv]")
    if beta.shape != (N, W, H) or A.shape != (H,) or state.shape != (N, H, dk, dv):
        raise ValueError("beta [N, W, H], A [H] and state [N, H, dk, dv] expected")
    o = torch.empty((N, W, H, dv), dtype=dt, device=dev)
    _check(lib().kda_recurrent_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A),
                                      _ptr(state), _ptr(o), N, W, H, dk, dv, code, _stream(dev)),
           "kda_recurrent_verify")
    return o


def kda_recurrent_fold(k, v, g, beta, A, n_accept, state) -> None:
    """Replay the first n_accept[s] tokens of each sequence's stored window
    into its state: k [N, W, H, dk], v [N, W, H, dv] (bf16 or fp32), g
    [N, W, H, dk] fp32, beta [N, W, H] fp32, A [H] fp32, n_accept [N] int32
    (device), state [N, H, dk, dv] fp32 (updated in place).  Bit-identical to
    that many kda_recurrent_step calls."""
    torch = _torch()
    _req(k, "k")
    dev, dt = k.device, k.dtype
    code = _dtype_code(k)
    _req(v, "v", dt, dev)
    _req(g, "g", torch.float32, dev)
    _req(beta, "beta", torch.float32, dev)
    _req(A, "A", torch.float32, dev)
    _req(n_accept, "n_accept", torch.int32, dev)
    _req(state, "state", torch.float32, dev)
    if k.dim() != 4:
        raise ValueError("k must be [N, W, H, dk]")
    N, W, H, dk = k.shape
    dv = v.shape[-1]
    if g.shape != k.shape or v.shape != (N, W, H, dv) or beta.shape != (N, W, H):
        raise ValueError("g must match k [N, W, H, dk], v must be [N, W, H, dv], beta [N, W, H]")
    if A.shape != (H,) or n_accept.shape != (N,) or state.shape != (N, H, dk, dv):
        raise ValueError("A [H], n_accept [N] and state [N, H, dk, dv] expected")
    rc = lib().kda_recurrent_fold(_ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A), _ptr(n_accept),
                                  _ptr(state), N, W, H, dk, dv, code, _stream(dev))
    _check(rc, "kda_recurrent_fold")


def kda_layer_fwd_workspace_bytes(B, T, H, d, N, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(_torch().empty(0, dtype=dtype))
    return int(lib().kda_layer_fwd_workspace_bytes(B, T, H, d, N, chunk, code))


def kda_layer_fwd(q_in, k_in, v_in, conv_w, g, beta, A, gate, norm_w, initial_state=None,
                  conv_state=None, cu_seqlens=None, chunk_size: int = 64, l2_eps: float = 1e-6,
                  rms_eps: float = 1e-5, output_final_state: bool = True, workspace=None):
    """The KDA layer between its projections: q, k = L2Norm(Swish(ShortConv)),
    v = Swish(ShortConv), the chunked core, y = Sigmoid(gate) * RMSNorm(o).
    q_in, k_in, v_in, gate [B, T, H, d] (bf16 or fp32); conv_w [3, H, d, 4]
    fp32; g, beta, A, initial_state, cu_seqlens as for kda_chunk_fwd; norm_w
    [d] fp32; conv_state [N, 3, 3, H, d] (input dtype) or None.  Returns
    (y, final_state or None, final conv_state or None)."""
    torch = _torch()
    B, T, H, dk, dv, N, dev, dt = _prefill_args(q_in, k_in, v_in, g, beta, A, initial_state,
                                                cu_seqlens)
    if dk != dv:
        raise ValueError("the layer entry point needs d_k == d_v")
    d = dk
    _req(conv_w, "conv_w", torch.float32, dev)
    _req(gate, "gate", dt, dev)
    _req(norm_w, "norm_w", torch.float32, dev)
    if conv_w.shape != (3, H, d, 4) or gate.shape != q_in.shape or norm_w.shape != (d,):
        raise ValueError("conv_w [3, H, d, 4], gate [B, T, H, d] and norm_w [d] expected")
    if conv_state is not None:
        _req(conv_state, "conv_state", dt, dev)
        if conv_state.shape != (N, 3, 3, H, d):
            raise ValueError(f"conv_state must be [{N}, 3, 3, {H}, {d}]")
    code = _dtype_code(q_in)
    L = lib()
    need = int(L.kda_layer_fwd_workspace_bytes(B, T, H, d, N, chunk_size, code))
    if need == 0:
        _check(2 if not L.kda_chunk_fwd_supported(d, d, chunk_size, code) else 1,
               "kda_layer_fwd_workspace_bytes")
    workspace = _workspace(workspace, need, dev)
    y = torch.empty((B, T, H, d), dtype=dt, device=dev)
    hT = torch.empty((N, H, d, d), dtype=torch.float32, device=dev) if output_final_state else None
    csT = torch.empty((N, 3, 3, H, d), dtype=dt, device=dev) if output_final_state else None
    rc = L.kda_layer_fwd(_ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(conv_w), _ptr(conv_state),
                         _ptr(csT), _ptr(g), _ptr(beta), _ptr(A), _ptr(initial_state),
                         _ptr(cu_seqlens), _ptr(gate), _ptr(norm_w), float(l2_eps), float(rms_eps),
                         B, T, H, d, N, chunk_size, code, _ptr(y), _ptr(hT), _ptr(workspace),
                         workspace.numel(), _stream(dev))
    _check(rc, "kda_layer_fwd")
    return y, hT, csT


def kda_layer_step(q_in, k_in, v_in, conv_w, conv_state, g, beta, A, state, gate, norm_w,
                   l2_eps: float = 1e-6, rms_eps: float = 1e-5):
    """One decode token of the layer in one launch: q_in, k_in, v_in, gate
    [N, H, d]; conv_w [3, H, d, 4] fp32; conv_state [N, 3, 3, H, d] (input
    dtype, shifted in place); g [N, H, d], beta [N, H], A [H] fp32; state
    [N, H, d, d] fp32 (in place); norm_w [d] fp32.  Returns y [N, H, d]."""
    torch = _torch()
    _req(q_in, "q_in")
    dev, dt = q_in.device, q_in.dtype
    code = _dtype_code(q_in)
    for t, name in ((k_in, "k_in"), (v_in, "v_in"), (gate, "gate"), (conv_state, "conv_state")):
        _req(t, name, dt, dev)
    for t, name in ((conv_w, "conv_w"), (g, "g"), (beta, "beta"), (A, "A"), (state, "state"),
                    (norm_w, "norm_w")):
        _req(t, name, torch.float32, dev)
    if q_in.dim() != 3:
        raise ValueError("q_in must be [N, H, d]")
    N, H, d = q_in.shape
    if (k_in.shape != q_in.shape or v_in.shape != q_in.shape or gate.shape != q_in.shape
            or g.shape != q_in.shape):
        raise ValueError("k_in, v_in, gate and g must match q_in [N, H, d]")
    if (conv_w.shape != (3, H, d, 4) or conv_state.shape != (N, 3, 3, H, d) or beta.shape != (N, H)
            or A.shape != (H,) or state.shape != (N, H, d, d) or norm_w.shape != (d,)):
        raise ValueError("conv_w [3, H, d, 4], conv_state [N, 3, 3, H, d], beta [N, H], A [H], "
                         "state [N, H, d, d] and norm_w [d] expected")
    y = torch.empty((N, H, d), dtype=dt, device=dev)
    rc = lib().kda_layer_step(_ptr(q_in), _ptr(k_in), _ptr(v_in), _ptr(conv_w), _ptr(conv_state),
                              _ptr(g), _ptr(beta), _ptr(A), _ptr(state), _ptr(gate), _ptr(norm_w),
                              float(l2_eps), float(rms_eps), _ptr(y), N, H, d, code, _stream(dev))
    _check(rc, "kda_layer_step")
    return y
