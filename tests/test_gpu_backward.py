"""GPU parity of gdn_chunk_bwd (gradients of the gated delta rule) against the
float64 gradient oracle (oracle/gdn_grad_ref.py, itself pinned to finite
differences): packed sequences with ragged tails, a one-token and an empty
sequence, nonzero initial states, a final-state gradient, scale != 1, and the
L2 normalisation on and off.

Tolerance: max|gpu - ref| / RMS(ref) per gradient tensor.
- fp32 inputs (the per-token fp32 chain): 1e-4.  Each gradient is a sum of a
  few thousand fp32 products per token, so a few 1e-6 of the tensor's RMS is
  expected, and 1e-4 leaves room for the cancellation in dg.
- bf16 inputs at d = 128 (the chunked matrix-core form): 1e-3.  Its
  contractions take derived operands as bf16 hi+lo pairs (each within about
  2^-17 of the fp32 value, the lo*lo term dropped), the scheme of the forward's
  bf16 path, whose fp32 final state the suite bounds at 2e-3.  Products such as
  Tb^T dU sum terms some ten to thirty times larger than the result, so errors
  of 1e-4 to 3e-4 of the RMS are expected (measured: at most 2.3e-4, in dv).
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, dev, dev_i32, host, note, rel_max
from harness import inputs as I
from oracle import gdn_grad_ref as G

pytestmark = pytest.mark.gpu

TOL = 1e-4        # fp32 inputs
TOL_BF16 = 1e-3   # bf16 inputs, chunked matrix-core form


def _tol(lay):
    return TOL_BF16 if lay.dtype == "bf16" else TOL
SMALL = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="bf16")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_mixer_causal_amd import ops as _ops
    _ops.L.load()
    return _ops


def _run(ops, lay, d, do, dfin, scale, use_l2, want_dinit=True):
    tdt = torch.bfloat16 if lay.dtype == "bf16" else torch.float32
    q, k, v = I.split_qkv(d["x"], lay)
    T, n = q.shape[0], len(d["cu_seqlens"]) - 1
    out = dict(dq=torch.full((T, lay.h_qk, lay.d_k), float("nan"), device=DEV),
               dk=torch.full((T, lay.h_qk, lay.d_k), float("nan"), device=DEV),
               dv=torch.full((T, lay.h_v, lay.d_v), float("nan"), device=DEV),
               dg=torch.full((T, lay.h_v), float("nan"), device=DEV),
               dbeta=torch.full((T, lay.h_v), float("nan"), device=DEV))
    dinit = torch.full((n, lay.h_v, lay.d_v, lay.d_k), float("nan"), device=DEV) if want_dinit else None
    ops.gdn_chunk_bwd(dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(d["g"]), dev(d["beta"]), dev(do),
                      out["dq"], out["dk"], out["dv"], out["dg"], out["dbeta"], scale=scale, use_qk_l2norm=use_l2,
                      cu_seqlens=dev_i32(d["cu_seqlens"]), initial_state=dev(d["state"]),
                      d_final=None if dfin is None else dev(dfin), d_initial=dinit)
    torch.cuda.synchronize()
    out["d_initial"] = dinit
    return out, (q, k, v)


SMALL_F32 = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="f32")

# The reverse kernel walks 16-token blocks as two 8-token halves; a sequence's
# last block holds 1..16 tokens.  The lengths below end blocks in 1, 5, 6, 7,
# 8, 9, 13, 15 and 16 tokens, so the partial second half (9..15) is covered.
CASES = [
    ("f32_d16", I.TINY_LAYOUT, [40, 1, 16, 0, 23], 0.7, True),
    ("f32_d16_nol2", I.TINY_LAYOUT, [33, 17], 1.0, False),
    ("f32_d16_tails", I.TINY_LAYOUT, [25, 31, 1, 0, 45], 1.0, True),
    ("bf16_d128", SMALL, [150, 1, 64, 0, 70], 1.0, True),
    ("bf16_d128_tails", SMALL, [25, 31, 1, 0, 45], 1.0, True),
    ("f32_d128", SMALL_F32, [57, 1, 0, 40], 0.8, True),
]


@pytest.mark.parametrize("name,lay,lengths,scale,use_l2", CASES, ids=[c[0] for c in CASES])
def test_chunk_bwd_against_oracle(ops, name, lay, lengths, scale, use_l2):
    note(f"chunk bwd {name}: lengths {lengths} scale {scale} l2 {use_l2}")
    d = I.prefill_inputs(50, lay, lengths, state_std=0.02, g_mode="tiny" if lay.dtype == "f32" else "model")
    rng = np.random.default_rng(51)
    T, n = int(sum(lengths)), len(lengths)
    do = rng.standard_normal((T, lay.h_v, lay.d_v)).astype(np.float32)
    dfin = (0.5 * rng.standard_normal((n, lay.h_v, lay.d_v, lay.d_k))).astype(np.float32)
    out, (q, k, v) = _run(ops, lay, d, do, dfin, scale, use_l2)
    ref = G.gated_delta_rule_grads(q, k, v, d["g"], d["beta"], do, dfin, scale=scale, initial_state=d["state"],
                                   cu_seqlens=d["cu_seqlens"], use_qk_l2norm=use_l2)
    errs = {key: rel_max(host(out[key]), ref[key]) for key in ("dq", "dk", "dv", "dg", "dbeta", "d_initial")}
    note("  " + ", ".join(f"{k_} {v_:.1e}" for k_, v_ in errs.items()))
    assert all(e <= _tol(lay) for e in errs.values()), errs

    # reruns are bitwise identical; without d_final the final-state term drops out
    out2, _ = _run(ops, lay, d, do, dfin, scale, use_l2)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "d_initial"):
        assert torch.equal(out[key], out2[key]), key
    out3, _ = _run(ops, lay, d, do, None, scale, use_l2, want_dinit=False)
    ref3 = G.gated_delta_rule_grads(q, k, v, d["g"], d["beta"], do, None, scale=scale, initial_state=d["state"],
                                    cu_seqlens=d["cu_seqlens"], use_qk_l2norm=use_l2)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert rel_max(host(out3[key]), ref3[key]) <= _tol(lay), key


def test_chunk_bwd_full_size_sampled_heads(ops):
    """The model shape (one 4096-token sequence, 16 q/k and 32 v heads, bf16,
    model-like decays) through gdn_chunk_bwd on all heads; the oracle checks
    eight v-heads, the two of each of q/k heads 0, 5, 10 and 15 (so their dq,
    dk, which sum over both v-heads, are compared too)."""
    lay = I.MODEL_LAYOUT
    qk_heads = [0, 5, 10, 15]
    hs = [2 * j + i for j in qk_heads for i in (0, 1)]
    note(f"chunk bwd full size T=4096, v-heads {hs}")
    d = I.model_prefill_inputs(4096, seed=1)
    rng = np.random.default_rng(52)
    T = 4096
    do = rng.standard_normal((T, lay.h_v, lay.d_v)).astype(np.float32)
    dfin = (0.5 * rng.standard_normal((1, lay.h_v, lay.d_v, lay.d_k))).astype(np.float32)
    d["state"] = (0.02 * rng.standard_normal((1, lay.h_v, lay.d_v, lay.d_k))).astype(np.float32)
    out, (q, k, v) = _run(ops, lay, d, do, dfin, 1.0, True)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "d_initial"):
        assert torch.isfinite(out[key]).all(), key
    note("  gradient oracle (about a minute)")
    ref = G.gated_delta_rule_grads(q[:, qk_heads], k[:, qk_heads], v[:, hs], d["g"][:, hs], d["beta"][:, hs],
                                   do[:, hs], dfin[:, hs], initial_state=d["state"][:, hs],
                                   qk_of_v=[i // 2 for i in range(len(hs))])
    got = dict(dq=host(out["dq"])[:, qk_heads], dk=host(out["dk"])[:, qk_heads], dv=host(out["dv"])[:, hs],
               dg=host(out["dg"])[:, hs], dbeta=host(out["dbeta"])[:, hs], d_initial=host(out["d_initial"])[:, hs])
    errs = {key: rel_max(got[key], ref[key]) for key in got}
    note("  " + ", ".join(f"{k_} {v_:.1e}" for k_, v_ in errs.items()))
    assert all(e <= TOL_BF16 for e in errs.values()), errs


@pytest.mark.parametrize("name,lay,lengths", [("f32_tiny", I.TINY_LAYOUT, [40, 1, 2, 0, 23]),
                                              ("bf16", SMALL, [150, 1, 64, 0, 70, 2])],
                         ids=["f32_tiny", "bf16"])
def test_conv1d_bwd_against_oracle(ops, name, lay, lengths):
    """gdn_conv1d_bwd against the oracle's conv gradients: varlen with one-,
    two-token and empty sequences, a history before the call and a gradient
    on the history after it."""
    note(f"conv bwd {name}: lengths {lengths}")
    tdt = torch.bfloat16 if lay.dtype == "bf16" else torch.float32
    d = I.prefill_inputs(53, lay, lengths, tail_std=1.0)
    rng = np.random.default_rng(54)
    T, n, ch = int(sum(lengths)), len(lengths), lay.channels
    dy = rng.standard_normal((T, ch)).astype(np.float32)
    dto = rng.standard_normal((n, 3, ch)).astype(np.float32)
    dx = torch.full((T, ch), float("nan"), device=DEV)
    dw = torch.full((ch, 4), float("nan"), device=DEV)
    dti = torch.full((n, 3, ch), float("nan"), device=DEV)
    ops.gdn_conv1d_bwd(dev(d["x"], tdt), dev(d["conv_w"], tdt), dev(dy), dx, dw,
                       cu_seqlens=dev_i32(d["cu_seqlens"]), conv_state_in=dev(d["tail"], tdt),
                       d_state_out=dev(dto), d_state_in=dti)
    torch.cuda.synchronize()
    ref = G.causal_conv1d_silu_grads(d["x"], d["conv_w"], d["tail"], d["cu_seqlens"], dy, dto)
    errs = {"dx": rel_max(host(dx), ref["dx"]), "dw": rel_max(host(dw), ref["dw"]),
            "d_state_in": rel_max(host(dti), ref["d_tail"])}
    note("  " + ", ".join(f"{k_} {v_:.1e}" for k_, v_ in errs.items()))
    assert all(e <= TOL for e in errs.values()), errs
    # bitwise reruns
    dw2 = torch.empty_like(dw)
    ops.gdn_conv1d_bwd(dev(d["x"], tdt), dev(d["conv_w"], tdt), dev(dy), torch.empty_like(dx), dw2,
                       cu_seqlens=dev_i32(d["cu_seqlens"]), conv_state_in=dev(d["tail"], tdt),
                       d_state_out=dev(dto))
    torch.cuda.synchronize()
    assert torch.equal(dw, dw2)


@pytest.mark.parametrize("name,lay,T", [("f32_d16", I.TINY_LAYOUT, 37), ("bf16_d128", SMALL, 137)],
                         ids=["f32_d16", "bf16_d128"])
def test_chunk_bwd_single_sequence_without_cu(ops, name, lay, T):
    """One sequence with cu_seqlens NULL and no initial state: the same
    gradients as the packed form with cu_seqlens = [0, T]."""
    note(f"chunk bwd {name}: one sequence of {T}, no cu_seqlens")
    d = I.prefill_inputs(55, lay, [T], g_mode="tiny" if lay.dtype == "f32" else "model")
    rng = np.random.default_rng(56)
    tdt = torch.bfloat16 if lay.dtype == "bf16" else torch.float32
    do = rng.standard_normal((T, lay.h_v, lay.d_v)).astype(np.float32)
    q, k, v = I.split_qkv(d["x"], lay)
    outs = [torch.empty((T, lay.h_qk, lay.d_k), device=DEV), torch.empty((T, lay.h_qk, lay.d_k), device=DEV),
            torch.empty((T, lay.h_v, lay.d_v), device=DEV), torch.empty((T, lay.h_v), device=DEV),
            torch.empty((T, lay.h_v), device=DEV)]
    dinit = torch.empty((1, lay.h_v, lay.d_v, lay.d_k), device=DEV)
    ops.gdn_chunk_bwd(dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(d["g"]), dev(d["beta"]), dev(do), *outs,
                      d_initial=dinit)
    torch.cuda.synchronize()
    ref = G.gated_delta_rule_grads(q, k, v, d["g"], d["beta"], do)
    errs = {nm: rel_max(host(got), ref[nm]) for nm, got in zip(("dq", "dk", "dv", "dg", "dbeta"), outs)}
    errs["d_initial"] = rel_max(host(dinit), ref["d_initial"])
    note("  " + ", ".join(f"{k_} {v_:.1e}" for k_, v_ in errs.items()))
    assert all(e <= _tol(lay) for e in errs.values()), errs
