"""GPU parity of the entry points with the gate preparation fused into their
prologues (gdn_chunk_fwd_gated, gdn_recurrent_step_gated) against the float64
oracle: the oracle forms g and beta from the same raw a, b, a_log and dt_bias
(gates_from_projections) and runs the token-by-token recurrence.

Tolerances are those of the unfused entry points: max|gpu - ref| / RMS(ref)
<= 1e-5 for fp32 inputs, <= 2e-3 for bf16 inputs with the fp32 state.
"""
import math

import numpy as np
import pytest
import torch

from gpu_util import DEV, dev, dev_i32, host, note, rel_max
from harness import inputs as I
from oracle import gdn_ref as R

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-3
SMALL = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="bf16")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_mixer_causal_amd import ops as _ops
    _ops.L.load()
    return _ops


def _packed_ba(gates, tdt):
    """One [rows, 2 Hv] device tensor holding b | a, and the a and b views of it
    (row stride 2 Hv; a starts Hv elements into each row)."""
    rows, hv = gates["a"].shape
    ba = dev(np.concatenate([gates["b"], gates["a"]], axis=1), tdt)
    return ba, ba[:, hv:], ba[:, :hv]


def test_gated_chunk_f32_tiny(ops):
    """Tiny fp32 shape (T=64, 2 heads, d=16, chunk 16), fp32 raw gates with a bias."""
    note("gated chunk f32 tiny")
    d = I.tiny_inputs(0)
    lay = I.TINY_LAYOUT
    q, k, v = I.split_qkv(d["x"], lay)
    gt = I.raw_gate_inputs(40, 64, lay.h_v, a_log_range=(math.log(0.02), math.log(0.3)), bias_std=0.5)
    o = torch.full((64, lay.h_v, lay.d_v), float("nan"), device=DEV)
    fin = torch.full((1, lay.h_v, lay.d_v, lay.d_k), float("nan"), device=DEV)
    ops.gdn_chunk_fwd_gated(dev(q), dev(k), dev(v), dev(gt["a"]), dev(gt["b"]), dev(gt["a_log"]), o, chunk=16,
                            dt_bias=dev(gt["dt_bias"]), cu_seqlens=dev_i32(d["cu_seqlens"]), final_state=fin)
    torch.cuda.synchronize()
    g, beta = R.gates_from_projections(gt["a"], gt["b"], gt["a_log"], gt["dt_bias"])
    o_ref, f_ref = R.gated_delta_rule(q, k, v, g, beta)
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_F32 and ef <= TOL_F32


@pytest.mark.parametrize("lengths,bias", [([200, 1, 64, 0, 130, 65], True), ([65], False)])
def test_gated_chunk_bf16_varlen(ops, lengths, bias):
    """bf16 q/k/v and bf16 raw gates packed as one b|a tensor, varlen with a
    nonzero initial state, with and without dt_bias."""
    note(f"gated chunk bf16 varlen {lengths} bias={bias}")
    d = I.prefill_inputs(41, SMALL, lengths, state_std=0.02)
    T = sum(lengths)
    yc, _ = R.causal_conv1d_silu(d["x"], d["conv_w"], d["tail"], d["cu_seqlens"], round_to_bf16=True)
    q, k, v = (a.astype(np.float32) for a in R.split_heads(yc, 2, 128, 4, 128))
    gt = I.raw_gate_inputs(42, T, SMALL.h_v, dtype="bf16", bias_std=0.5 if bias else None)
    ba, ta, tb = _packed_ba(gt, torch.bfloat16)
    o = torch.full((T, SMALL.h_v, SMALL.d_v), float("nan"), device=DEV)
    fin = torch.full(d["state"].shape, float("nan"), device=DEV)
    ops.gdn_chunk_fwd_gated(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), ta, tb,
                            dev(gt["a_log"]), o, chunk=64, dt_bias=dev(gt["dt_bias"]) if bias else None,
                            cu_seqlens=dev_i32(d["cu_seqlens"]), initial_state=dev(d["state"]), final_state=fin)
    torch.cuda.synchronize()
    g, beta = R.gates_from_projections(gt["a"], gt["b"], gt["a_log"], gt["dt_bias"])
    o_ref, f_ref = R.gated_delta_rule(q, k, v, g, beta, initial_state=d["state"], cu_seqlens=d["cu_seqlens"])
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    if 0 in lengths:
        s = lengths.index(0)
        np.testing.assert_array_equal(host(fin)[s], d["state"][s])


@pytest.mark.parametrize("layout", [SMALL, I.TINY_LAYOUT], ids=["bf16_d128", "f32_d16"])
def test_gated_recurrent_slots(ops, layout):
    """Three decode steps through a slot map with an inactive lane, fused gated
    RMSNorm on, raw gates of the input dtype with a bias."""
    note(f"gated recurrent step {layout}")
    n_req, n_slots = 5, 8
    slots = np.array([6, 0, -1, 3, 1], np.int32)
    tdt = torch.bfloat16 if layout.dtype == "bf16" else torch.float32
    tol = TOL_BF16 if layout.dtype == "bf16" else TOL_F32
    cast = I.round_bf16 if layout.dtype == "bf16" else (lambda a: a.astype(np.float32))
    rng = np.random.default_rng(43)
    hq, hv, dk, dv = layout.h_qk, layout.h_v, layout.d_k, layout.d_v
    state = (rng.standard_normal((n_slots, hv, dv, dk)) * 0.02).astype(np.float32)
    nw = (1 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    state_dev = dev(state)
    ref_state = state.astype(np.float64)
    for step in range(3):
        q = cast(rng.standard_normal((n_req, hq, dk)).astype(np.float32))
        k = cast(rng.standard_normal((n_req, hq, dk)).astype(np.float32))
        v = cast(rng.standard_normal((n_req, hv, dv)).astype(np.float32))
        z = cast(rng.standard_normal((n_req, hv, dv)).astype(np.float32))
        gt = I.raw_gate_inputs(50 + step, n_req, hv, dtype=layout.dtype, bias_std=0.5)
        o = torch.full((n_req, hv, dv), 3.0, device=DEV)
        ops.gdn_recurrent_step_gated(dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(gt["a"], tdt), dev(gt["b"], tdt),
                                     dev(gt["a_log"]), state_dev, o, dt_bias=dev(gt["dt_bias"]),
                                     state_slots=dev_i32(slots), z=dev(z, tdt), norm_w=dev(nw))
        torch.cuda.synchronize()
        g, beta = R.gates_from_projections(gt["a"], gt["b"], gt["a_log"], gt["dt_bias"])
        go = host(o)
        for r, s in enumerate(slots):
            if s < 0:
                assert np.all(go[r] == 3.0)
                continue
            o_ref, f_ref = R.gated_delta_rule(q[r:r + 1], k[r:r + 1], v[r:r + 1], g[r:r + 1], beta[r:r + 1],
                                              initial_state=ref_state[s:s + 1])
            ref_state[s] = f_ref[0]
            e = rel_max(go[r], R.gated_rmsnorm(o_ref[0], z[r], nw, 1e-6))
            assert e <= tol, (step, r, e)
    gs = host(state_dev)
    for s in range(n_slots):
        if s in slots:
            assert rel_max(gs[s], ref_state[s]) <= tol
        else:
            np.testing.assert_array_equal(gs[s], ref_state[s])


def test_gated_chunk_full_size_all_heads(ops):
    """T=4096, 16 q/k heads, 32 v heads, d=128, chunk 64, bf16 q/k/v and bf16
    raw gates (the model workload's decay distribution), oracle on every v-head."""
    lay = I.MODEL_LAYOUT
    note("gated chunk T=4096 full model layout")
    T = 4096
    rng = np.random.default_rng(44)
    qkv = I.round_bf16(rng.standard_normal((T, lay.channels)).astype(np.float32))
    gt = I.raw_gate_inputs(45, T, lay.h_v, dtype="bf16")
    x = dev(qkv, torch.bfloat16)
    from gated_deltanet_mixer_causal_amd.ops import qkv_views
    q, k, v = qkv_views(x, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    ba, ta, tb = _packed_ba(gt, torch.bfloat16)
    o = torch.empty((T, lay.h_v, lay.d_v), device=DEV)
    fin = torch.empty((1, lay.h_v, lay.d_v, lay.d_k), device=DEV)
    ops.gdn_chunk_fwd_gated(q, k, v, ta, tb, dev(gt["a_log"]), o, chunk=64, cu_seqlens=dev_i32([0, T]),
                            final_state=fin)
    torch.cuda.synchronize()
    qh, kh, vh = I.split_qkv(qkv, lay)
    g, beta = R.gates_from_projections(gt["a"], gt["b"], gt["a_log"])
    o_ref, f_ref = R.gated_delta_rule(qh, kh, vh, g, beta)
    eo = rel_max(host(o), o_ref)
    ef = rel_max(host(fin)[0], f_ref[0])
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
