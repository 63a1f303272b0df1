"""The C ABI library loads, exports every entry point the header declares, and
rejects invalid calls on the host with the documented status before any HIP
call (so these run without a GPU: no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import linear_attention_token_gated_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS = 0, 1, 2, 3, 4, 5, 6
A = 0x10000000          # fake, 16-byte aligned device addresses (never dereferenced)
MB = 1 << 20


@pytest.fixture(scope="module")
def L():
    return gdn.lib()


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    return sorted(set(re.findall(r"GDN_API\s+[\w\s\*]*?\b(gdn_\w+)\s*\(", src)))


def test_header_declares_the_exported_set():
    assert declared_symbols() == sorted(gdn.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for name in declared_symbols():
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {gdn.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for name in declared_symbols():
        assert name in exported
    # nothing but the C ABI is exported from our own code
    ours = {s for s in exported if s.startswith("gdn") or s.startswith("_ZN3gdn")}
    assert ours == set(declared_symbols())


def test_status_strings(L):
    for s, name in gdn.STATUS_NAMES.items():
        assert L.gdn_status_str(s).decode().startswith(name)


def prefill(L, q=A, k=A + 64 * MB, v=A + 128 * MB, al=A + 192 * MB, be=A + 200 * MB, s0=None,
            y=A + 256 * MB, sT=None, B=1, T=64, H=2, Dk=16, Dv=16, C=16, dt=0, w=None, wb=0):
    return L.gdn_prefill_fwd(q, k, v, al, be, s0, y, sT, B, T, H, Dk, Dv, C, dt, w, wb, None)


def test_prefill_validation(L):
    assert prefill(L, q=None) == NULL
    assert prefill(L, y=None) == NULL
    assert prefill(L, T=-1) == SHAPE
    assert prefill(L, B=-3) == SHAPE
    assert prefill(L, Dk=48) == UNSUP
    assert prefill(L, Dv=256) == UNSUP
    assert prefill(L, C=128) == UNSUP
    assert prefill(L, C=8) == UNSUP
    assert prefill(L, dt=7) == UNSUP
    assert prefill(L, q=A + 4) == ALIGN
    assert prefill(L, sT=A + 300 * MB + 8) == ALIGN
    assert prefill(L, y=A + 16) == ALIAS                         # y inside q
    assert prefill(L, y=A + 128 * MB) == ALIAS                   # y == v
    assert prefill(L, s0=A + 300 * MB, sT=A + 300 * MB + 256) == ALIAS   # partial overlap
    assert prefill(L, B=1 << 40, T=1 << 40) == SHAPE             # overflow
    assert "Dk=48" in L.gdn_last_error().decode() or True
    prefill(L, Dk=48)
    assert "Dk=48" in L.gdn_last_error().decode()


def test_prefill_workspace_validation(L):
    # one record per (sequence, head, chunk): optional for bf16 (none selects
    # the fused kernel), required for fp32.  Every failing case below fails on
    # the host before anything is launched.
    need16 = L.gdn_prefill_workspace_bytes(1, 64, 2, 16, 16, 16, 1)
    assert need16 == 2 * 4 * 1280          # 16-token chunks: one T' block (1024 bytes), 64 decay floats
    W = A + 400 * MB
    assert prefill(L, dt=1, w=W, wb=need16 - 1) == WS            # given but too small
    assert prefill(L, dt=1, w=W + 16, wb=need16) == ALIGN        # not 256-byte aligned
    assert prefill(L, dt=1, w=A + 256 * MB, wb=need16) == ALIAS  # workspace == y
    assert prefill(L, dt=1, w=A + 64 * MB, wb=need16) == ALIAS   # workspace == k
    need = L.gdn_prefill_workspace_bytes(1, 64, 2, 16, 16, 16, 0)
    assert prefill(L, dt=0) == WS                                # missing
    assert prefill(L, dt=0, w=W, wb=need - 1) == WS              # too small
    assert prefill(L, dt=0, w=W + 16, wb=need) == ALIGN          # not 256-byte aligned
    assert prefill(L, dt=0, w=A + 256 * MB, wb=need) == ALIAS    # workspace == y
    assert prefill(L, dt=0, w=A + 64 * MB, wb=need) == ALIAS     # workspace == k
    assert "workspace" in L.gdn_last_error().decode()


def test_prefill_f32_workspace_required(L):
    need = L.gdn_prefill_workspace_bytes(1, 64, 2, 16, 16, 16, 0)
    assert need == 4 * 2 * 4 * 832
    ws = A + 512 * MB
    assert prefill(L) == WS                             # fp32 needs the record workspace too
    assert prefill(L, w=ws, wb=need - 1) == WS          # given but too small
    assert prefill(L, w=ws + 16, wb=need) == ALIGN      # given but misaligned
    assert prefill(L, w=A + 256 * MB, wb=need) == ALIAS  # over y


def decode(L, q=A, k=A + MB, v=A + 2 * MB, al=A + 3 * MB, be=A + 4 * MB, S=A + 8 * MB, y=A + 64 * MB,
           N=4, H=2, Dk=16, Dv=16, dt=1):
    return L.gdn_decode_step(q, k, v, al, be, S, y, N, H, Dk, Dv, dt, None)


def test_decode_validation(L):
    assert decode(L, S=None) == NULL
    assert decode(L, N=-1) == SHAPE
    assert decode(L, Dk=96) == UNSUP
    assert decode(L, y=A + 2) == ALIGN
    assert decode(L, y=A + 8 * MB) == ALIAS          # y == state
    assert decode(L, S=A) == ALIAS                   # state over q


def verify(L, q=A, k=A + MB, v=A + 2 * MB, al=A + 3 * MB, be=A + 4 * MB, S=A + 8 * MB, So=A + 32 * MB,
           y=A + 64 * MB, N=4, T=3, H=2, Dk=16, Dv=16, dt=1):
    return L.gdn_decode_verify(q, k, v, al, be, S, So, y, N, T, H, Dk, Dv, dt, None)


def test_verify_validation(L):
    assert verify(L, So=None) == NULL
    assert verify(L, S=None) == NULL
    assert verify(L, T=-1) == SHAPE
    assert verify(L, Dv=48) == UNSUP
    assert verify(L, dt=5) == UNSUP
    assert verify(L, y=A + 8) == ALIGN
    assert verify(L, So=A + 8 * MB) == ALIAS         # states_out over state
    assert verify(L, y=A + 32 * MB) == ALIAS         # y over states_out
    assert verify(L, y=A + 2 * MB) == ALIAS          # y over v
    assert "gdn_decode_verify" in L.gdn_last_error().decode()


def test_layer_validation(L):
    P = gdn.gdn_layer_params(A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB, A + 6 * MB, A + 7 * MB)
    ws_need = L.gdn_layer_workspace_bytes(1, 64, 128, 2, 16, 16, 4, 16)
    assert ws_need > 0
    ws = A + 512 * MB

    def call(x=A + 64 * MB, out=A + 128 * MB, T=64, hidden=128, conv_k=4, C=16, w=ws, wb=ws_need, p=P):
        return L.gdn_layer_fwd(x, ctypes.byref(p) if p is not None else None, None, None, out, 1, T, hidden, 2,
                               16, 16, conv_k, C, w, wb, None)

    assert call(p=None) == NULL
    assert call(x=None) == NULL
    assert call(T=-2) == SHAPE
    assert call(hidden=100) == UNSUP
    assert call(conv_k=5) == UNSUP
    assert call(C=48) == UNSUP
    assert call(w=None) == WS
    assert call(wb=ws_need - 1) == WS
    assert call(w=ws + 16) == ALIGN
    assert call(out=A + 64 * MB) == ALIAS
    assert call(out=ws) == ALIAS


def test_layer_decode_validation(L):
    P = gdn.gdn_layer_params(A, A + MB, A + 2 * MB, A + 3 * MB, A + 4 * MB, A + 5 * MB, A + 6 * MB, A + 7 * MB)
    ws_need = L.gdn_layer_decode_workspace_bytes(4, 128, 2, 16, 16)
    assert ws_need > 0
    ws = A + 512 * MB

    def call(x=A + 64 * MB, cs=A + 96 * MB, S=A + 160 * MB, out=A + 128 * MB, N=4, hidden=128, conv_k=4,
             w=ws, wb=ws_need, p=P, Dk=16):
        return L.gdn_layer_decode_step(x, ctypes.byref(p) if p is not None else None, cs, S, out, N, hidden, 2,
                                       Dk, 16, conv_k, w, wb, None)

    assert call(p=None) == NULL
    assert call(x=None) == NULL
    assert call(S=None) == NULL
    assert call(cs=None) == NULL                   # history needed for conv_k > 1
    assert call(N=-1) == SHAPE
    assert call(hidden=96) == UNSUP
    assert call(conv_k=0) == UNSUP
    assert call(Dk=24) == UNSUP
    assert call(w=None) == WS
    assert call(wb=ws_need - 1) == WS
    assert call(w=ws + 16) == ALIGN
    assert call(cs=A + 96 * MB + 4) == ALIGN
    assert call(out=A + 64 * MB) == ALIAS          # out over x
    assert call(S=A + 96 * MB) == ALIAS            # state over conv_state
    assert call(cs=ws) == ALIAS                    # conv_state over workspace
    assert call(out=A + 160 * MB) == ALIAS         # out over state
    assert "gdn_layer_decode_step" in L.gdn_last_error().decode()


def test_workspace_queries(L):
    # bf16 prefill: one 11072-byte record per (sequence, head, 64-token chunk):
    # T' as 10 blocks of hi/lo fragments (10240 bytes) and 208 floats of decay
    # vectors; 3520 bytes at 32-token chunks (3 blocks, 112 floats)
    assert L.gdn_prefill_workspace_bytes(1, 32768, 32, 128, 128, 64, 1) == 32 * 512 * 11072
    assert L.gdn_prefill_workspace_bytes(2, 100, 3, 64, 32, 32, 1) == 2 * 3 * 4 * 3520
    assert L.gdn_prefill_workspace_bytes(1, 0, 32, 128, 128, 64, 1) == 0
    assert L.gdn_prefill_workspace_bytes(1, 64, 2, 48, 16, 64, 1) == 0            # rejected shape
    # fp32: records of the two-kernel path, 3*64*64 + 2*64 floats per 64-token chunk
    assert L.gdn_prefill_workspace_bytes(1, 32768, 32, 128, 128, 64, 0) == 4 * 32 * 512 * 12416
    assert L.gdn_prefill_workspace_bytes(2, 100, 3, 64, 32, 32, 0) == 4 * 2 * 3 * 4 * 3136
    assert L.gdn_prefill_workspace_bytes(1, 0, 32, 128, 128, 64, 0) == 0
    assert L.gdn_prefill_workspace_bytes(1, 64, 2, 48, 16, 64, 0) == 0            # rejected shape
    assert L.gdn_layer_workspace_bytes(1, 0, 2048, 16, 128, 128, 4, 64) == 0
    assert L.gdn_layer_workspace_bytes(1, 16384, 2048, 16, 128, 128, 4, 64) > 16384 * 2048


def prefill_bwd(L, q=A, k=A + 8 * MB, v=A + 16 * MB, al=A + 24 * MB, be=A + 25 * MB, s0=A + 26 * MB,
                dy=A + 32 * MB, dsT=A + 40 * MB, dq=A + 48 * MB, dk=A + 56 * MB, dv=A + 64 * MB,
                da=A + 72 * MB, db=A + 73 * MB, ds0=A + 74 * MB, B=1, T=64, H=2, Dk=16, Dv=16, C=16, dt=0,
                w=A + 512 * MB, wb=None):
    if wb is None:
        wb = L.gdn_prefill_bwd_workspace_bytes(B, T, H, Dk, Dv, C)
    return L.gdn_prefill_bwd(q, k, v, al, be, s0, dy, dsT, dq, dk, dv, da, db, ds0, B, T, H, Dk, Dv, C, dt,
                             w, wb, None)


def test_prefill_bwd_validation(L):
    need = L.gdn_prefill_bwd_workspace_bytes(1, 64, 2, 16, 16, 16)
    # per chunk: a record of 3*16*16+16 floats (rounded up to 64), two 16x16
    # states and three 16x16 chunk matrices
    assert need == 4 * 2 * 4 * (832 + 2 * 256 + 3 * 256)
    assert L.gdn_prefill_bwd_workspace_bytes(2, 4096, 16, 128, 128, 64) == 4 * 32 * 64 * (12416 + 2 * 16384 + 3 * 8192)
    assert L.gdn_prefill_bwd_workspace_bytes(1, 0, 2, 16, 16, 16) == 0
    assert L.gdn_prefill_bwd_workspace_bytes(1, 64, 2, 48, 16, 16) == 0
    assert prefill_bwd(L, q=None) == NULL
    assert prefill_bwd(L, dy=None) == NULL
    assert prefill_bwd(L, db=None) == NULL
    assert prefill_bwd(L, T=-1) == SHAPE
    assert prefill_bwd(L, Dk=48) == UNSUP
    assert prefill_bwd(L, C=128) == UNSUP
    assert prefill_bwd(L, dt=7) == UNSUP
    assert prefill_bwd(L, w=None) == WS
    assert prefill_bwd(L, wb=need - 1) == WS
    assert prefill_bwd(L, w=A + 512 * MB + 16) == ALIGN
    assert prefill_bwd(L, dq=A + 48 * MB + 4) == ALIGN
    assert prefill_bwd(L, dq=A) == ALIAS                   # dq over q
    assert prefill_bwd(L, dv=A + 56 * MB) == ALIAS         # dv over dk
    assert prefill_bwd(L, ds0=A + 26 * MB) == ALIAS        # dS_0 over initial_state
    assert prefill_bwd(L, w=A + 64 * MB) == ALIAS          # workspace over dv
    assert "gdn_prefill_bwd" in L.gdn_last_error().decode()
    # T == 0 needs no workspace and checks only what it writes
    assert prefill_bwd(L, T=0, w=None, wb=0, q=None, dq=None, ds0=A + 26 * MB) == ALIAS


def test_binding_rejects_mismatched_shapes():
    """The binding checks every tensor's shape and device against the sizes it
    derives from q (or x) before any C call: a mismatched tensor would
    otherwise become an out-of-bounds device access."""
    import torch
    q = torch.zeros(1, 8, 2, 16)
    ok = [(torch.zeros(1, 8, 2, 16), "k", (1, 8, 2, 16)), (None, "initial_state", (1, 2, 16, 16))]
    gdn._same(q, ok)
    with pytest.raises(ValueError, match="k has shape"):
        gdn._same(q, [(torch.zeros(1, 8, 2, 32), "k", (1, 8, 2, 16))])
    with pytest.raises(ValueError, match="alpha has shape"):
        gdn._same(q, [(torch.zeros(1, 8, 3), "alpha", (1, 8, 2))])
    params = {"W_qkv": torch.zeros(96, 64), "conv_w": torch.zeros(96, 4), "W_ab": torch.zeros(4, 64),
              "A": torch.zeros(2), "b_alpha": torch.zeros(2), "W_gate": torch.zeros(32, 64),
              "norm_gamma": torch.zeros(16), "W_o": torch.zeros(64, 32)}
    gdn._same(q, gdn._layer_param_shapes(params, 64, 2, 16, 16, 4))
    params["W_o"] = torch.zeros(32, 64)
    with pytest.raises(ValueError, match="W_o has shape"):
        gdn._same(q, gdn._layer_param_shapes(params, 64, 2, 16, 16, 4))
