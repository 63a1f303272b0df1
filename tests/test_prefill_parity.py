"""GPU parity of gdn_prefill_fwd (chunked) against the fp64 token-by-token
oracle of eqs (1)-(4), plus properties of the chunked kernel."""
import numpy as np
import pytest

from helpers import TOL_BF16, TOL_F32, dev, host, oracle_prefill, rel_err
from linear_attention_token_gated_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _gpu(inp, chunk, S0=None, **kw):
    import torch
    import linear_attention_token_gated_amd as gdn
    s0 = dev(inp["S0"]) if S0 is None else S0
    y, sT = gdn.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["alpha"]), dev(inp["beta"]), s0,
                        chunk=chunk, **kw)
    torch.cuda.synchronize()
    return y, sT


def _check(oracle, inp, chunk, tol, **kw):
    y, sT = _gpu(inp, chunk, **kw)
    y_ref, S_ref = oracle_prefill(oracle, inp)
    ey, eS = rel_err(host(y), y_ref), rel_err(host(sT), S_ref)
    print(f"  err y={ey:.3e} S={eS:.3e}", flush=True)
    assert ey <= tol and eS <= tol, (ey, eS)


def test_prefill_tiny_f32(oracle_mod):
    cfg = wl.TINY
    print(f"case: {cfg.name}", flush=True)
    _check(oracle_mod, wl.prefill_config_inputs(cfg), cfg.chunk, TOL_F32)


# the two bf16 forms: records + recurrence (a workspace), one fused kernel (none)
FORMS = [pytest.param(False, id="records"), pytest.param(True, id="fused")]


@pytest.mark.parametrize("fused", FORMS)
def test_prefill_4k_bf16(oracle_mod, fused):
    cfg = wl.PREFILL_4K
    print(f"case: {cfg.name} fused={fused}", flush=True)
    _check(oracle_mod, wl.prefill_config_inputs(cfg), cfg.chunk, TOL_BF16, fused=fused)


@pytest.mark.slow
@pytest.mark.parametrize("fused", FORMS)
def test_prefill_32k_bf16(oracle_mod, fused):
    cfg = wl.PREFILL_32K
    print(f"case: {cfg.name} fused={fused}", flush=True)
    _check(oracle_mod, wl.prefill_config_inputs(cfg), cfg.chunk, TOL_BF16, fused=fused)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "bf16-fused"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("Dk,Dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128)])
def test_prefill_shapes_chunks_ragged(oracle_mod, dtype, chunk, Dk, Dv):
    T = 3 * chunk + 5            # several chunks and a ragged tail
    print(f"case: prefill B=2 T={T} H=3 Dk={Dk} Dv={Dv} C={chunk} {dtype}", flush=True)
    inp = wl.prefill_inputs(2, T, 3, Dk, Dv, dtype=dtype[:4].rstrip("-"), s0_std=0.3, seed=Dk + 3 * Dv + chunk)
    kw = {"fused": True} if dtype == "bf16-fused" else {}
    _check(oracle_mod, inp, chunk, TOL_F32 if dtype == "f32" else TOL_BF16, **kw)


@pytest.mark.parametrize("T", [1, 2, 15, 17, 63, 64, 65])
def test_prefill_short_sequences(oracle_mod, T):
    print(f"case: prefill short T={T}", flush=True)
    inp = wl.prefill_inputs(1, T, 2, 64, 64, dtype="f32", s0_std=0.2, seed=T)
    _check(oracle_mod, inp, 64, TOL_F32)


@pytest.mark.parametrize("fused", FORMS)
def test_prefill_chunk_size_invariance(oracle_mod, fused):
    print(f"case: chunk invariance C=16/32/64 fused={fused}", flush=True)
    inp = wl.prefill_inputs(1, 200, 4, 128, 128, dtype="bf16", s0_std=0.02, seed=11)
    y_ref, S_ref = oracle_prefill(oracle_mod, inp)
    ys = []
    for C in (16, 32, 64):
        y, sT = _gpu(inp, C, fused=fused)
        assert rel_err(host(y), y_ref) <= TOL_BF16 and rel_err(host(sT), S_ref) <= TOL_BF16
        ys.append(host(y))
    assert rel_err(ys[0], ys[2]) <= TOL_BF16


@pytest.mark.parametrize("fused", FORMS)
def test_prefill_split_resume(oracle_mod, fused):
    """prefill(0:T1) -> S; prefill(T1:T, S) == prefill(0:T) (state hand-off)."""
    import torch
    import linear_attention_token_gated_amd as gdn
    print(f"case: split/resume fused={fused}", flush=True)
    inp = wl.prefill_inputs(2, 300, 2, 64, 64, dtype="bf16", s0_std=0.02, seed=12)
    y_full, S_full = _gpu(inp, 64, fused=fused)
    T1 = 131
    part = {n: (inp[n][:, :T1] if inp[n] is not None and n != "S0" and n != "dtype" else inp[n]) for n in inp}
    rest = {n: (inp[n][:, T1:] if inp[n] is not None and n != "S0" and n != "dtype" else inp[n]) for n in inp}
    y1, S1 = _gpu(part, 64, fused=fused)
    y2, S2 = _gpu(rest, 64, S0=S1, fused=fused)
    # chunk boundaries move, so rounding differs: both runs meet the oracle bound
    y_ref, S_ref = oracle_prefill(oracle_mod, inp)
    assert rel_err(host(torch.cat([y1, y2], 1)), y_ref) <= TOL_BF16
    assert rel_err(host(S2), S_ref) <= TOL_BF16
    assert rel_err(host(torch.cat([y1, y2], 1)), host(y_full)) <= TOL_BF16
    assert rel_err(host(S2), host(S_full)) <= TOL_BF16


def test_prefill_in_place_state_and_null_state(oracle_mod):
    import torch
    import linear_attention_token_gated_amd as gdn
    print("case: final_state aliasing initial_state; S0 = NULL", flush=True)
    inp = wl.prefill_inputs(1, 100, 2, 32, 32, dtype="f32", s0_std=0.3, seed=13)
    S = dev(inp["S0"])
    y, sT = gdn.prefill(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["alpha"]), dev(inp["beta"]), S,
                        chunk=32, final_state=S)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle_prefill(oracle_mod, inp)
    assert sT.data_ptr() == S.data_ptr()
    assert rel_err(host(S), S_ref) <= TOL_F32 and rel_err(host(y), y_ref) <= TOL_F32
    inp["S0"] = None
    _check(oracle_mod, inp, 32, TOL_F32)


def test_prefill_empty(oracle_mod):
    import torch
    import linear_attention_token_gated_amd as gdn
    print("case: T=0 and B=0", flush=True)
    S0 = torch.randn(2, 3, 16, 32, device="cuda")
    e = lambda *s: torch.empty(*s, device="cuda")
    y, sT = gdn.prefill(e(2, 0, 3, 16), e(2, 0, 3, 16), e(2, 0, 3, 32), e(2, 0, 3), e(2, 0, 3), S0, chunk=16)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 3, 32) and torch.equal(sT, S0)
    y, sT = gdn.prefill(e(2, 0, 3, 16), e(2, 0, 3, 16), e(2, 0, 3, 32), e(2, 0, 3), e(2, 0, 3), None, chunk=16)
    torch.cuda.synchronize()
    assert torch.count_nonzero(sT) == 0
    y, sT = gdn.prefill(e(0, 5, 3, 16), e(0, 5, 3, 16), e(0, 5, 3, 32), e(0, 5, 3), e(0, 5, 3), None, chunk=16)
    assert y.shape == (0, 5, 3, 32)


def test_prefill_identity_tokens_and_pure_decay(oracle_mod):
    """alpha = 1, beta = 0 leaves the state unchanged; beta = 0 alone is pure decay."""
    import torch
    print("case: identity tokens / pure decay", flush=True)
    inp = wl.prefill_inputs(1, 77, 2, 64, 32, dtype="f32", s0_std=0.5, seed=14)
    inp["alpha"] = np.ones_like(inp["alpha"])
    inp["beta"] = np.zeros_like(inp["beta"])
    y, sT = _gpu(inp, 64)
    assert rel_err(host(sT), wl.widen(inp["S0"])) <= 1e-6
    inp2 = wl.prefill_inputs(1, 77, 2, 64, 32, dtype="f32", s0_std=0.5, seed=15)
    inp2["beta"] = np.zeros_like(inp2["beta"])
    _check(oracle_mod, inp2, 32, TOL_F32)


@pytest.mark.parametrize("fused", FORMS)
def test_prefill_column_slices_independent(oracle_mod, fused):
    """Column separability: the first 32 value columns computed alone equal the
    same columns of the full-width run (same kernel, different slice count)."""
    print(f"case: column slices fused={fused}", flush=True)
    inp = wl.prefill_inputs(1, 150, 2, 64, 128, dtype="bf16", s0_std=0.02, seed=16)
    y, sT = _gpu(inp, 64, fused=fused)
    sub = dict(inp)
    sub["v"] = np.ascontiguousarray(inp["v"][..., :32])
    sub["S0"] = np.ascontiguousarray(inp["S0"][..., :32])
    y2, s2 = _gpu(sub, 64, fused=fused)
    np.testing.assert_array_equal(host(y2), host(y)[..., :32])
    np.testing.assert_array_equal(host(s2), host(sT)[..., :32])


@pytest.mark.parametrize("fused", FORMS)
def test_prefill_deterministic(oracle_mod, fused):
    print(f"case: determinism fused={fused}", flush=True)
    inp = wl.prefill_inputs(2, 500, 4, 128, 128, dtype="bf16", s0_std=0.02, seed=17)
    y1, s1 = _gpu(inp, 64, fused=fused)
    y2, s2 = _gpu(inp, 64, fused=fused)
    np.testing.assert_array_equal(host(y1), host(y2))
    np.testing.assert_array_equal(host(s1), host(s2))


@pytest.mark.parametrize("fused", FORMS)
def test_prefill_strong_decay_no_nan(oracle_mod, fused):
    """alpha down to 1e-3 per token (log-decay prefix far below fp32 range over a chunk)."""
    print(f"case: strong decay fused={fused}", flush=True)
    inp = wl.prefill_inputs(1, 256, 2, 128, 128, dtype="bf16", s0_std=0.02, seed=18)
    rng = np.random.default_rng(0)
    inp["alpha"] = rng.uniform(1e-3, 0.2, inp["alpha"].shape).astype(np.float32)
    _check(oracle_mod, inp, 64, TOL_BF16, fused=fused)


def test_sync_check_mode(oracle_mod, monkeypatch):
    """GDN_SYNC_CHECK=1 makes every call wait for its stream and check for
    kernel errors; results are the same bits as without it."""
    import torch
    import linear_attention_token_gated_amd as gdn
    print("case: GDN_SYNC_CHECK", flush=True)
    inp = wl.prefill_inputs(1, 130, 2, 64, 64, dtype="bf16", s0_std=0.1, seed=41)
    args = [dev(inp[n]) for n in ("q", "k", "v", "alpha", "beta")]
    monkeypatch.delenv("GDN_SYNC_CHECK", raising=False)
    y1, s1 = gdn.prefill(*args, initial_state=dev(inp["S0"]), chunk=64)
    torch.cuda.synchronize()
    monkeypatch.setenv("GDN_SYNC_CHECK", "1")
    y2, s2 = gdn.prefill(*args, initial_state=dev(inp["S0"]), chunk=64)
    assert np.array_equal(host(y1), host(y2)) and np.array_equal(host(s1), host(s2))
