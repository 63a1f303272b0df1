"""MI355X-native Gated DeltaNet token mixer (gfx950).

The compute lives in ``libgdn.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/gdn.h``).  This module only marshals torch tensors to it:
torch provides device memory and the current stream, nothing else.  If the
library is missing every entry point raises; there is no CPU fallback.

Entry points (same names as the C ABI):

* ``prefill(q, k, v, alpha, beta, initial_state=None, chunk=64)``
  -> ``(y, final_state)``: whole sequences through eqs (1)-(4) of the picx.dev
  summary of "On the Design of Qwen3.8-Next Architecture" ("Theoretical
  foundations"), chunk by chunk.
* ``decode_step(q, k, v, alpha, beta, state)`` -> ``y``; ``state`` is updated
  in place.
* ``layer_fwd(x, params, H, Dk, Dv, initial_state=None, chunk=64)``
  -> ``(out, final_state)``: the token-mixing layer ("1. GDN Hybrid Token
  Mixing", eqs (9)-(11)).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
STATUS_NAMES = {0: "GDN_OK", 1: "GDN_ERR_NULL", 2: "GDN_ERR_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
                4: "GDN_ERR_ALIGN", 5: "GDN_ERR_ALIAS", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_HIP"}
EXPORTED = ("gdn_prefill_fwd", "gdn_prefill_workspace_bytes", "gdn_prefill_bwd", "gdn_prefill_bwd_workspace_bytes",
            "gdn_decode_step", "gdn_decode_verify", "gdn_layer_fwd", "gdn_layer_workspace_bytes", "gdn_layer_decode_step",
            "gdn_layer_decode_workspace_bytes", "gdn_layer_decode_step_noalloc", "gdn_status_str",
            "gdn_last_error")


class GdnError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class gdn_layer_params(ctypes.Structure):
    _fields_ = [("W_qkv", ctypes.c_void_p), ("conv_w", ctypes.c_void_p), ("W_ab", ctypes.c_void_p),
                ("A", ctypes.c_void_p), ("b_alpha", ctypes.c_void_p), ("W_gate", ctypes.c_void_p),
                ("norm_gamma", ctypes.c_void_p), ("W_o", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m linear_attention_token_gated_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.gdn_prefill_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                  ctypes.c_int, vp, sz, vp]
    L.gdn_prefill_fwd.restype = ctypes.c_int
    L.gdn_prefill_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.c_int]
    L.gdn_prefill_workspace_bytes.restype = sz
    L.gdn_prefill_bwd.argtypes = [vp] * 14 + [i64] * 6 + [ctypes.c_int, vp, sz, vp]
    L.gdn_prefill_bwd.restype = ctypes.c_int
    L.gdn_prefill_bwd_workspace_bytes.argtypes = [i64] * 6
    L.gdn_prefill_bwd_workspace_bytes.restype = sz
    L.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_int, vp]
    L.gdn_decode_step.restype = ctypes.c_int
    L.gdn_decode_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int, vp]
    L.gdn_decode_verify.restype = ctypes.c_int
    L.gdn_layer_fwd.argtypes = [vp, ctypes.POINTER(gdn_layer_params), vp, vp, vp, i64, i64, i64, i64,
                                i64, i64, i64, i64, vp, sz, vp]
    L.gdn_layer_fwd.restype = ctypes.c_int
    L.gdn_layer_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, i64, i64]
    L.gdn_layer_workspace_bytes.restype = sz
    L.gdn_layer_decode_step.argtypes = [vp, ctypes.POINTER(gdn_layer_params), vp, vp, vp, i64, i64, i64, i64, i64,
                                        i64, vp, sz, vp]
    L.gdn_layer_decode_step.restype = ctypes.c_int
    L.gdn_layer_decode_workspace_bytes.argtypes = [i64, i64, i64, i64, i64]
    L.gdn_layer_decode_workspace_bytes.restype = sz
    L.gdn_layer_decode_step_noalloc.argtypes = [vp, ctypes.POINTER(gdn_layer_params), vp, vp, vp, i64, i64, i64,
                                                i64, i64, i64, vp]
    L.gdn_layer_decode_step_noalloc.restype = ctypes.c_int
    L.gdn_status_str.argtypes = [ctypes.c_int]
    L.gdn_status_str.restype = ctypes.c_char_p
    L.gdn_last_error.argtypes = []
    L.gdn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise GdnError(status, lib().gdn_last_error().decode())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _need(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _same(ref, items):
    """Every tensor of `items` ((tensor, name, shape) triples; None tensors
    skipped) has exactly `shape` and lives on the device of `ref`."""
    for t, name, shape in items:
        if t is None:
            continue
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _same_device(ref, t, name):
    if t is not None and t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def prefill_workspace_bytes(B, T, H, Dk, Dv, chunk=64, dtype="bf16") -> int:
    code = {"f32": 0, "bf16": 1}[dtype]
    return int(lib().gdn_prefill_workspace_bytes(B, T, H, Dk, Dv, int(chunk), code))


def prefill(q, k, v, alpha, beta, initial_state=None, chunk: int = 64, return_final_state: bool = True,
            y=None, final_state=None, workspace=None, fused: bool = False):
    """Chunked prefill.  q, k: [B,T,H,Dk]; v: [B,T,H,Dv] (float32 or bfloat16);
    alpha, beta: [B,T,H] float32; initial_state: [B,H,Dk,Dv] float32 or None.
    workspace: a device buffer of prefill_workspace_bytes(...) bytes, or None
    to allocate one for this call.  fused (bfloat16 only): pass no workspace,
    which selects the library's single-kernel form.
    Returns (y [B,T,H,Dv] float32, final_state or None)."""
    import torch
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    for t, n in ((alpha, "alpha"), (beta, "beta"), (initial_state, "initial_state")):
        _need(t, n, torch.float32)
    if y is None:
        y = torch.empty((B, T, H, Dv), dtype=torch.float32, device=q.device)
    if final_state is None and return_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _need(y, "y", torch.float32)
    _need(final_state, "final_state", torch.float32)
    _same(q, [(k, "k", (B, T, H, Dk)), (v, "v", (B, T, H, Dv)), (alpha, "alpha", (B, T, H)),
              (beta, "beta", (B, T, H)), (initial_state, "initial_state", (B, H, Dk, Dv)),
              (y, "y", (B, T, H, Dv)), (final_state, "final_state", (B, H, Dk, Dv))])
    _same_device(q, workspace, "workspace")
    if fused:
        if q.dtype != torch.bfloat16 or workspace is not None:
            raise ValueError("prefill: fused=True takes bfloat16 inputs and no workspace")
        need = 0
    else:
        need = int(lib().gdn_prefill_workspace_bytes(B, T, H, Dk, Dv, int(chunk), _dtype_code(q)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().gdn_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
                                 _ptr(y), _ptr(final_state), B, T, H, Dk, Dv, int(chunk), _dtype_code(q),
                                 _ptr(workspace), ws_bytes, _stream(q.device)))
    return y, final_state


def prefill_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk=64) -> int:
    return int(lib().gdn_prefill_bwd_workspace_bytes(B, T, H, Dk, Dv, int(chunk)))


def prefill_bwd(q, k, v, alpha, beta, dy, initial_state=None, dfinal_state=None, chunk: int = 64,
                want_dinitial_state: bool = True, out=None, workspace=None):
    """Gradients of prefill for dL/dy = dy [B,T,H,Dv] float32 and dL/dS_T =
    dfinal_state (or None).  Inputs as for prefill.  `out` may hold
    preallocated float32 tensors under the names of the result.  Returns a
    dict dq, dk [B,T,H,Dk], dv [B,T,H,Dv], dalpha, dbeta [B,T,H] and
    dinitial_state [B,H,Dk,Dv] (None unless wanted)."""
    import torch
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    for t, n in ((alpha, "alpha"), (beta, "beta"), (initial_state, "initial_state"), (dy, "dy"),
                 (dfinal_state, "dfinal_state")):
        _need(t, n, torch.float32)
    shapes = dict(dq=(B, T, H, Dk), dk=(B, T, H, Dk), dv=(B, T, H, Dv), dalpha=(B, T, H), dbeta=(B, T, H),
                  dinitial_state=(B, H, Dk, Dv))
    res = dict(out or {})
    for n, shp in shapes.items():
        if n == "dinitial_state" and not want_dinitial_state:
            res.setdefault(n, None)
            continue
        if res.get(n) is None:
            res[n] = torch.empty(shp, dtype=torch.float32, device=q.device)
        _need(res[n], n, torch.float32)
    _same(q, [(k, "k", (B, T, H, Dk)), (v, "v", (B, T, H, Dv)), (alpha, "alpha", (B, T, H)),
              (beta, "beta", (B, T, H)), (initial_state, "initial_state", (B, H, Dk, Dv)),
              (dy, "dy", (B, T, H, Dv)), (dfinal_state, "dfinal_state", (B, H, Dk, Dv))]
          + [(res[n], n, shp) for n, shp in shapes.items()])
    _same_device(q, workspace, "workspace")
    need = prefill_bwd_workspace_bytes(B, T, H, Dk, Dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().gdn_prefill_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(initial_state),
                                 _ptr(dy), _ptr(dfinal_state), _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]),
                                 _ptr(res["dalpha"]), _ptr(res["dbeta"]), _ptr(res["dinitial_state"]),
                                 B, T, H, Dk, Dv, int(chunk), _dtype_code(q), _ptr(workspace), ws_bytes,
                                 _stream(q.device)))
    return res


def decode_step(q, k, v, alpha, beta, state, y=None):
    """One token per sequence.  q, k: [N,H,Dk]; v: [N,H,Dv]; alpha, beta: [N,H];
    state: [N,H,Dk,Dv] float32, updated in place.  Returns y [N,H,Dv] float32."""
    import torch
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    for t, n in ((alpha, "alpha"), (beta, "beta"), (state, "state")):
        _need(t, n, torch.float32)
    if y is None:
        y = torch.empty((N, H, Dv), dtype=torch.float32, device=q.device)
    _need(y, "y", torch.float32)
    _same(q, [(k, "k", (N, H, Dk)), (v, "v", (N, H, Dv)), (alpha, "alpha", (N, H)), (beta, "beta", (N, H)),
              (state, "state", (N, H, Dk, Dv)), (y, "y", (N, H, Dv))])
    _check(lib().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(y),
                                 N, H, Dk, Dv, _dtype_code(q), _stream(q.device)))
    return y


def decode_verify(q, k, v, alpha, beta, state, states_out=None, y=None):
    """T tokens per sequence from stored states.  q, k: [N,T,H,Dk]; v: [N,T,H,Dv]
    (float32 or bfloat16); alpha, beta: [N,T,H] float32; state: [N,H,Dk,Dv]
    float32 (not modified).  Returns (y [N,T,H,Dv], states_out [N,T,H,Dk,Dv]),
    states_out[:, t] being the state after token t."""
    import torch
    N, T, H, Dk = q.shape
    Dv = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, q.dtype)
    for t, n in ((alpha, "alpha"), (beta, "beta"), (state, "state")):
        _need(t, n, torch.float32)
    if y is None:
        y = torch.empty((N, T, H, Dv), dtype=torch.float32, device=q.device)
    if states_out is None:
        states_out = torch.empty((N, T, H, Dk, Dv), dtype=torch.float32, device=q.device)
    _need(y, "y", torch.float32)
    _need(states_out, "states_out", torch.float32)
    _same(q, [(k, "k", (N, T, H, Dk)), (v, "v", (N, T, H, Dv)), (alpha, "alpha", (N, T, H)),
              (beta, "beta", (N, T, H)), (state, "state", (N, H, Dk, Dv)), (y, "y", (N, T, H, Dv)),
              (states_out, "states_out", (N, T, H, Dk, Dv))])
    _check(lib().gdn_decode_verify(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state),
                                   _ptr(states_out), _ptr(y), N, T, H, Dk, Dv, _dtype_code(q), _stream(q.device)))
    return y, states_out


def _layer_param_shapes(params, hidden, H, Dk, Dv, conv_k):
    nqkv = H * (2 * Dk + Dv)
    return [(params["W_qkv"], "W_qkv", (nqkv, hidden)), (params["conv_w"], "conv_w", (nqkv, conv_k)),
            (params["W_ab"], "W_ab", (2 * H, hidden)), (params["A"], "A", (H,)),
            (params["b_alpha"], "b_alpha", (H,)), (params["W_gate"], "W_gate", (H * Dv, hidden)),
            (params["norm_gamma"], "norm_gamma", (Dv,)), (params["W_o"], "W_o", (hidden, H * Dv))]


def layer_workspace_bytes(B, T, hidden, H, Dk, Dv, conv_k=4, chunk=64) -> int:
    return int(lib().gdn_layer_workspace_bytes(B, T, hidden, H, Dk, Dv, conv_k, chunk))


def layer_fwd(x, params: dict, H: int, Dk: int, Dv: int, initial_state=None, chunk: int = 64,
              return_final_state: bool = True, out=None, final_state=None, workspace=None):
    """GDN layer.  x: [B,T,hidden] bfloat16; params: W_qkv, conv_w, W_ab, W_gate,
    W_o (bfloat16), A, b_alpha, norm_gamma (float32).  Returns (out float32, S_T)."""
    import torch
    B, T, hidden = x.shape
    conv_k = params["conv_w"].shape[1]
    _need(x, "x", torch.bfloat16)
    for n in ("W_qkv", "conv_w", "W_ab", "W_gate", "W_o"):
        _need(params[n], n, torch.bfloat16)
    for n in ("A", "b_alpha", "norm_gamma"):
        _need(params[n], n, torch.float32)
    _need(initial_state, "initial_state", torch.float32)
    if out is None:
        out = torch.empty((B, T, hidden), dtype=torch.float32, device=x.device)
    if final_state is None and return_final_state:
        final_state = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32)
    _need(final_state, "final_state", torch.float32)
    _same(x, _layer_param_shapes(params, hidden, H, Dk, Dv, conv_k)
          + [(initial_state, "initial_state", (B, H, Dk, Dv)), (final_state, "final_state", (B, H, Dk, Dv)),
             (out, "out", (B, T, hidden))])
    _same_device(x, workspace, "workspace")
    need = layer_workspace_bytes(B, T, hidden, H, Dk, Dv, conv_k, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    p = gdn_layer_params(*(_ptr(params[n]) for n in ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate",
                                                      "norm_gamma", "W_o")))
    _check(lib().gdn_layer_fwd(_ptr(x), ctypes.byref(p), _ptr(initial_state), _ptr(final_state), _ptr(out),
                               B, T, hidden, H, Dk, Dv, conv_k, int(chunk), _ptr(workspace),
                               workspace.numel(), _stream(x.device)))
    return out, final_state


def layer_decode_workspace_bytes(N, hidden, H, Dk, Dv) -> int:
    return int(lib().gdn_layer_decode_workspace_bytes(N, hidden, H, Dk, Dv))


def layer_decode_step(x, params: dict, H: int, Dk: int, Dv: int, conv_state, state, out=None, workspace=None):
    """One new token of the layer for each of N sequences.  x: [N, hidden]
    bfloat16; conv_state: [N, conv_k-1, H*(2Dk+Dv)] float32 (None when
    conv_k == 1) and state: [N, H, Dk, Dv] float32, both updated in place.
    Returns out [N, hidden] float32."""
    import torch
    N, hidden = x.shape
    conv_k = params["conv_w"].shape[1]
    _need(x, "x", torch.bfloat16)
    for n in ("W_qkv", "conv_w", "W_ab", "W_gate", "W_o"):
        _need(params[n], n, torch.bfloat16)
    for n in ("A", "b_alpha", "norm_gamma"):
        _need(params[n], n, torch.float32)
    _need(conv_state, "conv_state", torch.float32)
    _need(state, "state", torch.float32)
    if out is None:
        out = torch.empty((N, hidden), dtype=torch.float32, device=x.device)
    _need(out, "out", torch.float32)
    nqkv = H * (2 * Dk + Dv)
    _same(x, _layer_param_shapes(params, hidden, H, Dk, Dv, conv_k)
          + [(conv_state, "conv_state", (N, conv_k - 1, nqkv)), (state, "state", (N, H, Dk, Dv)),
             (out, "out", (N, hidden))])
    _same_device(x, workspace, "workspace")
    need = layer_decode_workspace_bytes(N, hidden, H, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    p = gdn_layer_params(*(_ptr(params[n]) for n in ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate",
                                                      "norm_gamma", "W_o")))
    _check(lib().gdn_layer_decode_step(_ptr(x), ctypes.byref(p), _ptr(conv_state), _ptr(state), _ptr(out),
                                       N, hidden, H, Dk, Dv, conv_k, _ptr(workspace), workspace.numel(),
                                       _stream(x.device)))
    return out


def layer_decode_step_noalloc(x, params: dict, H: int, Dk: int, Dv: int, conv_state, state, out):
    """layer_decode_step on the library's own scratch memory: no workspace, and
    out must be given, so that the call allocates nothing."""
    import torch
    N, hidden = x.shape
    conv_k = params["conv_w"].shape[1]
    _need(x, "x", torch.bfloat16)
    for n in ("W_qkv", "conv_w", "W_ab", "W_gate", "W_o"):
        _need(params[n], n, torch.bfloat16)
    for n in ("A", "b_alpha", "norm_gamma"):
        _need(params[n], n, torch.float32)
    _need(conv_state, "conv_state", torch.float32)
    _need(state, "state", torch.float32)
    _need(out, "out", torch.float32)
    nqkv = H * (2 * Dk + Dv)
    _same(x, _layer_param_shapes(params, hidden, H, Dk, Dv, conv_k)
          + [(conv_state, "conv_state", (N, conv_k - 1, nqkv)), (state, "state", (N, H, Dk, Dv)),
             (out, "out", (N, hidden))])
    p = gdn_layer_params(*(_ptr(params[n]) for n in ("W_qkv", "conv_w", "W_ab", "A", "b_alpha", "W_gate",
                                                      "norm_gamma", "W_o")))
    _check(lib().gdn_layer_decode_step_noalloc(_ptr(x), ctypes.byref(p), _ptr(conv_state), _ptr(state), _ptr(out),
                                               N, hidden, H, Dk, Dv, conv_k, _stream(x.device)))
    return out
