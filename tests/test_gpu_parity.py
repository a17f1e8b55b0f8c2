"""GPU parity: every entry point of the C ABI against the float64 oracle.

Inputs are the seeded synthetic arrays of harness.inputs, uploaded exactly;
the oracle runs on the same host arrays.  Tolerances: max|gpu - ref| / RMS(ref)
<= 1e-5 for fp32 inputs and <= 2e-3 for bf16 inputs with the fp32 state;
conv histories, slot bookkeeping and split/packed invariances are bit-exact.
"""
import numpy as np
import pytest
import torch

from gpu_util import (DEV, bf16_ulp_check, conv_abs_sum, conv_check_all_channels, dev, dev_i32, host,
                      note, rel_max)
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


def _tdt(layout):
    return torch.bfloat16 if layout.dtype == "bf16" else torch.float32


# ---------------------------------------------------------------------------
# conv1d
# ---------------------------------------------------------------------------

def test_conv_prefill_f32_tiny(ops):
    d = I.tiny_inputs(0)
    note("conv f32 tiny T=64 Ch=96")
    for lengths, tail_std in (([64], None), ([5, 1, 0, 2, 40, 16], 1.0)):
        dd = I.prefill_inputs(0, I.TINY_LAYOUT, lengths, tail_std=tail_std, g_mode="tiny")
        x, w, tail = dev(dd["x"]), dev(dd["conv_w"]), dev(dd["tail"])
        y = torch.full_like(x, float("nan"))
        ops.gdn_conv1d_fwd(x, w, tail, y, cu_seqlens=dev_i32(dd["cu_seqlens"]))
        ref_y, ref_tail = R.causal_conv1d_silu(dd["x"], dd["conv_w"], dd["tail"], dd["cu_seqlens"],
                                               round_to_bf16=False)
        torch.cuda.synchronize()
        assert rel_max(host(y), ref_y) <= TOL_F32
        np.testing.assert_array_equal(host(tail), ref_tail)


def test_conv_prefill_bf16_varlen(ops):
    lengths = [70, 1, 0, 2, 33, 64]
    note(f"conv bf16 varlen {lengths}")
    dd = I.prefill_inputs(11, SMALL, lengths, tail_std=1.0)
    x, w, tail = dev(dd["x"], torch.bfloat16), dev(dd["conv_w"], torch.bfloat16), dev(dd["tail"], torch.bfloat16)
    y = torch.zeros_like(x)
    ops.gdn_conv1d_fwd(x, w, tail, y, cu_seqlens=dev_i32(dd["cu_seqlens"]))
    ref_r, ref_tail = R.causal_conv1d_silu(dd["x"], dd["conv_w"], dd["tail"], dd["cu_seqlens"], round_to_bf16=True)
    ref_e, _ = R.causal_conv1d_silu(dd["x"], dd["conv_w"], dd["tail"], dd["cu_seqlens"], round_to_bf16=False)
    torch.cuda.synchronize()
    frac = bf16_ulp_check(host(y), ref_r, ref_e,
                          abs_sum=conv_abs_sum(dd["x"], dd["conv_w"], dd["tail"], dd["cu_seqlens"]))
    note(f"  one-ulp fraction {frac:.2e}")
    np.testing.assert_array_equal(host(tail), ref_tail)


def test_conv_decode_slots_and_inactive(ops):
    note("conv decode step with slots")
    rng = np.random.default_rng(5)
    ch, n_slots = 1024, 7
    slots = np.array([3, -1, 0, 5, 1, 2], np.int32)
    x = I.round_bf16(rng.standard_normal((6, ch)).astype(np.float32))
    w = I.round_bf16((rng.standard_normal((ch, 4)) * 0.5).astype(np.float32))
    tails = I.round_bf16(rng.standard_normal((n_slots, 3, ch)).astype(np.float32))
    tx, tw, tt = dev(x, torch.bfloat16), dev(w, torch.bfloat16), dev(tails, torch.bfloat16)
    y = torch.full_like(tx, 7.0)
    ops.gdn_conv1d_fwd(tx, tw, tt, y, state_slots=dev_i32(slots))
    torch.cuda.synchronize()
    gy, gt = host(y), host(tt)
    ref_tail = tails.astype(np.float64).copy()
    for r, s in enumerate(slots):
        if s < 0:
            assert np.all(gy[r] == 7.0)
            continue
        yr, tr = R.causal_conv1d_silu(x[r:r + 1], w, tails[s:s + 1], [0, 1], round_to_bf16=True)
        ye, _ = R.causal_conv1d_silu(x[r:r + 1], w, tails[s:s + 1], [0, 1], round_to_bf16=False)
        bf16_ulp_check(gy[r:r + 1], yr, ye, max_frac=0.01,
                       abs_sum=conv_abs_sum(x[r:r + 1], w, tails[s:s + 1], [0, 1]))
        ref_tail[s] = tr[0]
    np.testing.assert_array_equal(gt, ref_tail)   # includes untouched slots 4 and 6


# ---------------------------------------------------------------------------
# gated RMSNorm
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,xdt,ydt", [(128, torch.float32, torch.float32), (128, torch.float32, torch.bfloat16),
                                       (16, torch.float32, torch.float32), (128, torch.bfloat16, torch.float32)])
def test_gated_rmsnorm(ops, d, xdt, ydt):
    note(f"gated rmsnorm d={d} x={xdt} y={ydt}")
    rng = np.random.default_rng(6)
    rows = 1003
    x = I.round_bf16(rng.standard_normal((rows, d)).astype(np.float32)) if xdt == torch.bfloat16 \
        else rng.standard_normal((rows, d)).astype(np.float32)
    z = I.round_bf16(rng.standard_normal((rows, d)).astype(np.float32))
    w = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    tx, tz, tw = dev(x, xdt), dev(z, torch.bfloat16), dev(w)
    y = torch.empty((rows, d), dtype=ydt, device=DEV)
    ops.gdn_gated_rmsnorm(tx, tz, tw, y, eps=1e-6)
    ref = R.gated_rmsnorm(x, z, w, 1e-6)
    torch.cuda.synchronize()
    if ydt == torch.float32:
        assert rel_max(host(y), ref) <= TOL_F32
    else:
        bf16_ulp_check(host(y), R.bf16_nearest(ref), ref, max_frac=0.01)


# ---------------------------------------------------------------------------
# recurrent decode step
# ---------------------------------------------------------------------------

def _step_case(layout, n_req, n_slots, seed):
    rng = np.random.default_rng(seed)
    hq, hv, dk, dv = layout.h_qk, layout.h_v, layout.d_k, layout.d_v
    cast = I.round_bf16 if layout.dtype == "bf16" else (lambda a: a.astype(np.float32))
    q = cast(rng.standard_normal((n_req, hq, dk)).astype(np.float32))
    k = cast(rng.standard_normal((n_req, hq, dk)).astype(np.float32))
    v = cast(rng.standard_normal((n_req, hv, dv)).astype(np.float32))
    a = rng.uniform(0, np.log(16), hv)
    g = (-np.exp(a)[None] * np.logaddexp(0, rng.standard_normal((n_req, hv)))).astype(np.float32)
    beta = (1 / (1 + np.exp(-rng.standard_normal((n_req, hv))))).astype(np.float32)
    state = (rng.standard_normal((n_slots, hv, dv, dk)) * 0.02).astype(np.float32)
    z = cast(rng.standard_normal((n_req, hv, dv)).astype(np.float32))
    nw = (1 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    return q, k, v, g, beta, state, z, nw


@pytest.mark.parametrize("layout,fused", [(SMALL, False), (SMALL, True),
                                          (I.TINY_LAYOUT, False), (I.TINY_LAYOUT, True)])
def test_recurrent_step_slots(ops, layout, fused):
    note(f"recurrent step {layout} fused={fused}")
    n_req, n_slots = 5, 8
    slots = np.array([6, 0, -1, 3, 1], np.int32)
    tdt = _tdt(layout)
    tol = TOL_BF16 if layout.dtype == "bf16" else TOL_F32
    state_dev = None
    ref_state = None
    for step in range(3):
        q, k, v, g, beta, state, z, nw = _step_case(layout, n_req, n_slots, 100 + step)
        if state_dev is None:
            state_dev = dev(state)
            ref_state = state.astype(np.float64)
        o = torch.full((n_req, layout.h_v, layout.d_v), 3.0, dtype=torch.float32, device=DEV)
        ops.gdn_recurrent_step(dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(g), dev(beta), state_dev, o,
                               state_slots=dev_i32(slots), z=dev(z, tdt) if fused else None,
                               norm_w=dev(nw) if fused else None)
        torch.cuda.synchronize()
        go = host(o)
        for r, s in enumerate(slots):
            if s < 0:
                assert np.all(go[r] == 3.0)
                continue
            o_ref, f_ref = R.gated_delta_rule(q[r:r + 1], k[r:r + 1], v[r:r + 1], g[r:r + 1], beta[r:r + 1],
                                              initial_state=ref_state[s:s + 1])
            ref_state[s] = f_ref[0]
            expect = R.gated_rmsnorm(o_ref[0], z[r], nw, 1e-6) if fused else o_ref[0]
            e = rel_max(go[r], expect)
            assert e <= tol, (r, e)
    gs = host(state_dev)
    for s in range(n_slots):
        if s in slots:
            assert rel_max(gs[s], ref_state[s]) <= tol
        else:
            np.testing.assert_array_equal(gs[s], ref_state[s])   # untouched slots


def test_recurrent_exact_integers(ops):
    """One-hot keys and queries, small integers, a=1, beta in {0,1}: exact."""
    note("recurrent exact integers")
    rng = np.random.default_rng(7)
    n, hq, hv, d = 16, 2, 4, 128
    kidx = rng.integers(0, d, (n, hq))
    qidx = rng.integers(0, d, (n, hq))
    q = np.eye(d, dtype=np.float32)[qidx]
    k = np.eye(d, dtype=np.float32)[kidx]
    v = rng.integers(-8, 9, (n, hv, d)).astype(np.float32)
    beta = rng.integers(0, 2, (n, hv)).astype(np.float32)
    g = np.zeros((n, hv), np.float32)
    state = rng.integers(-8, 9, (n, hv, d, d)).astype(np.float32)
    sd = dev(state)
    o = torch.zeros((n, hv, d), device=DEV)
    ops.gdn_recurrent_step(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(g),
                           dev(beta), sd, o, use_qk_l2norm=False)
    o_ref = np.zeros((n, hv, d))
    f_ref = np.zeros((n, hv, d, d))
    for r in range(n):
        orr, frr = R.gated_delta_rule(q[r:r + 1], k[r:r + 1], v[r:r + 1], g[r:r + 1], beta[r:r + 1],
                                      initial_state=state[r:r + 1], use_qk_l2norm=False)
        o_ref[r], f_ref[r] = orr[0], frr[0]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(o), o_ref)
    np.testing.assert_array_equal(host(sd), f_ref)


# ---------------------------------------------------------------------------
# chunked prefill
# ---------------------------------------------------------------------------

def _chunk_run(ops, layout, q, k, v, g, beta, cu, state0, *, z=None, nw=None, o_dtype=torch.float32,
               use_l2=True, final=True):
    tdt = _tdt(layout)
    T = q.shape[0]
    o = torch.full((T, layout.h_v, layout.d_v), float("nan"), dtype=o_dtype, device=DEV)
    fin = torch.full(state0.shape, float("nan"), device=DEV) if final else None
    ops.gdn_chunk_fwd(dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(g), dev(beta), o, chunk=layout.chunk,
                      cu_seqlens=dev_i32(cu), initial_state=dev(state0), final_state=fin,
                      z=None if z is None else dev(z, tdt), norm_w=None if nw is None else dev(nw),
                      use_qk_l2norm=use_l2)
    torch.cuda.synchronize()
    return o, fin


def test_chunk_f32_tiny(ops):
    """Tiny fp32 check (T=64, 2 heads, d=16, chunk 16), recurrence on raw q, k, v."""
    note("chunk f32 tiny")
    d = I.tiny_inputs(0)
    q, k, v = I.split_qkv(d["x"], I.TINY_LAYOUT)
    o, fin = _chunk_run(ops, I.TINY_LAYOUT, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"])
    o_ref, f_ref = R.gated_delta_rule(q, k, v, d["g"], d["beta"], initial_state=d["state"])
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_F32 and ef <= TOL_F32


def test_mixer_f32_tiny_full_path(ops):
    """The tiny fp32 workload (T=64, 2 heads, d=16, chunk 16) through the whole
    mixer: conv1d + SiLU on the raw q|k|v channels, the chunked rule with L2
    norm of q and k, and the gated RMSNorm epilogue, against the oracle's
    mixer_prefill at 1e-5 end to end (fp32 conv output, no bf16 boundary)."""
    from gated_deltanet_mixer_causal_amd.ops import qkv_views
    lay = I.TINY_LAYOUT
    note("mixer f32 tiny full path")
    d = I.tiny_inputs(0)
    T = d["x"].shape[0]
    x, tail = dev(d["x"]), dev(d["tail"])
    cu = dev_i32(d["cu_seqlens"])
    y_conv = torch.full_like(x, float("nan"))
    ops.gdn_conv1d_fwd(x, dev(d["conv_w"]), tail, y_conv, cu_seqlens=cu)
    q, k, v = qkv_views(y_conv, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    o = torch.full((T, lay.h_v, lay.d_v), float("nan"), device=DEV)
    y = torch.full((T, lay.h_v, lay.d_v), float("nan"), device=DEV)
    fin = torch.full((1, lay.h_v, lay.d_v, lay.d_k), float("nan"), device=DEV)
    ops.gdn_chunk_fwd(q, k, v, dev(d["g"]), dev(d["beta"]), o, chunk=16, cu_seqlens=cu,
                      initial_state=dev(d["state"]), final_state=fin)
    ops.gdn_chunk_fwd(q, k, v, dev(d["g"]), dev(d["beta"]), y, chunk=16, cu_seqlens=cu,
                      initial_state=dev(d["state"]), z=dev(d["z"]), norm_w=dev(d["norm_w"]))
    torch.cuda.synchronize()
    ref = R.mixer_prefill(d["x"], d["conv_w"], d["tail"], d["state"], d["beta"], d["g"], d["z"], d["norm_w"],
                          d["cu_seqlens"], h_qk=lay.h_qk, h_v=lay.h_v, d_k=lay.d_k, d_v=lay.d_v,
                          bf16_boundary=False)
    errs = dict(conv=rel_max(host(y_conv), ref["y_conv"]), o=rel_max(host(o), ref["o"]),
                y=rel_max(host(y), ref["y"]), state=rel_max(host(fin)[0], ref["state"][0]))
    note("  " + " ".join(f"{k_} {v_:.1e}" for k_, v_ in errs.items()))
    assert all(e <= TOL_F32 for e in errs.values()), errs
    np.testing.assert_array_equal(host(tail), ref["tail"])


@pytest.mark.parametrize("lengths", [[200, 1, 64, 0, 130, 65], [63], [64], [65]])
def test_chunk_bf16_varlen(ops, lengths):
    note(f"chunk bf16 varlen {lengths}")
    d = I.prefill_inputs(21, SMALL, lengths, state_std=0.02)
    yc, _ = R.causal_conv1d_silu(d["x"], d["conv_w"], d["tail"], d["cu_seqlens"], round_to_bf16=True)
    q, k, v = (a.astype(np.float32) for a in R.split_heads(yc, 2, 128, 4, 128))
    o, fin = _chunk_run(ops, SMALL, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"])
    o_ref, f_ref = R.gated_delta_rule(q, k, v, d["g"], d["beta"], initial_state=d["state"],
                                      cu_seqlens=d["cu_seqlens"])
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    if 0 in lengths:
        s = lengths.index(0)
        np.testing.assert_array_equal(host(fin)[s], d["state"][s])


def test_chunk_fused_norm_and_bf16_output(ops):
    note("chunk fused gated norm")
    lengths = [150, 37]
    d = I.prefill_inputs(22, SMALL, lengths, state_std=0.02)
    yc, _ = R.causal_conv1d_silu(d["x"], d["conv_w"], d["tail"], d["cu_seqlens"], round_to_bf16=True)
    q, k, v = (a.astype(np.float32) for a in R.split_heads(yc, 2, 128, 4, 128))
    y, _ = _chunk_run(ops, SMALL, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"], z=d["z"],
                      nw=d["norm_w"])
    o_ref, _ = R.gated_delta_rule(q, k, v, d["g"], d["beta"], initial_state=d["state"], cu_seqlens=d["cu_seqlens"])
    y_ref = R.gated_rmsnorm(o_ref, d["z"], d["norm_w"], 1e-6)
    e = rel_max(host(y), y_ref)
    note(f"  y {e:.2e}")
    assert e <= TOL_BF16
    # bf16 output mode equals the rounding of the fp32 output of the same kernels
    o32, _ = _chunk_run(ops, SMALL, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"], final=False)
    o16, _ = _chunk_run(ops, SMALL, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"], final=False,
                        o_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)


def test_chunk_exact_integers(ops):
    """One-hot keys/queries, small integers, a=1, beta in {0,1}: bit-exact."""
    note("chunk exact integers")
    rng = np.random.default_rng(8)
    T, hq, hv, d = 150, 2, 4, 128
    q = np.eye(d, dtype=np.float32)[rng.integers(0, d, (T, hq))]
    k = np.eye(d, dtype=np.float32)[rng.integers(0, d, (T, hq))]
    v = rng.integers(-8, 9, (T, hv, d)).astype(np.float32)
    beta = rng.integers(0, 2, (T, hv)).astype(np.float32)
    g = np.zeros((T, hv), np.float32)
    s0 = rng.integers(-8, 9, (1, hv, d, d)).astype(np.float32)
    o, fin = _chunk_run(ops, SMALL, q, k, v, g, beta, np.array([0, T]), s0, use_l2=False)
    o_ref, f_ref = R.gated_delta_rule(q, k, v, g, beta, initial_state=s0, use_qk_l2norm=False)
    np.testing.assert_array_equal(host(o), o_ref)
    np.testing.assert_array_equal(host(fin), f_ref)


def test_chunk_split_packed_rerun_bitexact(ops):
    """Bookkeeping is bit-exact: a call split at a chunk multiple equals one
    call (the state hands over exactly and the chunk grid is unchanged);
    packed sequences equal separate calls; reruns are identical.  The split
    result is also held to the parity bound against the oracle."""
    note("chunk bit-exact bookkeeping")
    d = I.prefill_inputs(23, SMALL, [256, 77, 128], state_std=0.02)
    q, k, v = I.split_qkv(d["x"], SMALL)
    cu = d["cu_seqlens"]
    o_all, f_all = _chunk_run(ops, SMALL, q, k, v, d["g"], d["beta"], cu, d["state"])
    o_again, f_again = _chunk_run(ops, SMALL, q, k, v, d["g"], d["beta"], cu, d["state"])
    assert torch.equal(o_all, o_again) and torch.equal(f_all, f_again)
    for s in range(3):
        sl = slice(cu[s], cu[s + 1])
        o1, f1 = _chunk_run(ops, SMALL, q[sl], k[sl], v[sl], d["g"][sl], d["beta"][sl],
                            np.array([0, cu[s + 1] - cu[s]]), d["state"][s:s + 1])
        assert torch.equal(o1, o_all[cu[s]:cu[s + 1]]) and torch.equal(f1[0], f_all[s])
    # split the first sequence at 128 (a multiple of the chunk)
    oa, fa = _chunk_run(ops, SMALL, q[:128], k[:128], v[:128], d["g"][:128], d["beta"][:128],
                        np.array([0, 128]), d["state"][0:1])
    fa_h = host(fa).astype(np.float32)
    ob, fb = _chunk_run(ops, SMALL, q[128:256], k[128:256], v[128:256], d["g"][128:256], d["beta"][128:256],
                        np.array([0, 128]), fa_h)
    assert torch.equal(torch.cat([oa, ob]), o_all[:256]) and torch.equal(fb[0], f_all[0])
    o_ref, f_ref = R.gated_delta_rule(q[:256], k[:256], v[:256], d["g"][:256], d["beta"][:256],
                                      initial_state=d["state"][0:1])
    e_split = rel_max(host(torch.cat([oa, ob])), o_ref)
    e_fin = rel_max(host(fb)[0], f_ref[0])
    note(f"  split call: o {e_split:.2e} state {e_fin:.2e}")
    assert e_split <= TOL_BF16 and e_fin <= TOL_BF16


# ---------------------------------------------------------------------------
# full single-sequence prefill shape, every head
# ---------------------------------------------------------------------------

def test_mixer_prefill_full_size_all_heads(ops):
    """B=1, T=4096, 16 q/k heads, 32 v heads, d=128, chunk 64, bf16; conv ->
    chunk -> fused gated RMSNorm on the full shape; the oracle follows every
    channel of the conv and every v-head of the recurrence and the norm."""
    from gated_deltanet_mixer_causal_amd.ops import qkv_views
    lay = I.MODEL_LAYOUT
    note("mixer prefill T=4096 full model layout, all heads")
    d = I.model_prefill_inputs()
    T, ch = d["x"].shape
    x = dev(d["x"], torch.bfloat16)
    tail = dev(d["tail"], torch.bfloat16)
    y_conv = torch.empty_like(x)
    cu = dev_i32(d["cu_seqlens"])
    ops.gdn_conv1d_fwd(x, dev(d["conv_w"], torch.bfloat16), tail, y_conv, cu_seqlens=cu)
    q, k, v = qkv_views(y_conv, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    o = torch.full((T, lay.h_v, lay.d_v), float("nan"), device=DEV)
    y = torch.full((T, lay.h_v, lay.d_v), float("nan"), device=DEV)
    fin = torch.full((1, lay.h_v, lay.d_v, lay.d_k), float("nan"), device=DEV)
    g, beta = dev(d["g"]), dev(d["beta"])
    ops.gdn_chunk_fwd(q, k, v, g, beta, o, chunk=64, cu_seqlens=cu, final_state=fin)
    ops.gdn_chunk_fwd(q, k, v, g, beta, y, chunk=64, cu_seqlens=cu, z=dev(d["z"], torch.bfloat16),
                      norm_w=dev(d["norm_w"]))
    torch.cuda.synchronize()
    # (1) the conv output of every channel against the oracle's conv
    gy = host(y_conv)
    frac = conv_check_all_channels(d["x"], d["conv_w"], d["tail"], d["cu_seqlens"], gy, R)
    note(f"  conv one-ulp fraction {frac:.2e}")
    # (2) recurrence and norm of every v-head against the oracle on the same
    #     bf16 q/k/v the chunk kernels read (a one-ulp conv rounding difference
    #     moves o by more than the bound: tests/test_conv_boundary_sensitivity.py)
    qs, ks, vs = R.split_heads(gy, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    o_ref, f_ref = R.gated_delta_rule(qs, ks, vs, d["g"], d["beta"])
    y_ref = R.gated_rmsnorm(o_ref, d["z"], d["norm_w"], 1e-6)
    go, gyy, gf = host(o), host(y), host(fin)
    eo, ey, ef = rel_max(go, o_ref), rel_max(gyy, y_ref), rel_max(gf[0], f_ref[0])
    worst = max(range(lay.h_v), key=lambda h: rel_max(go[:, h], o_ref[:, h]))
    note(f"  o {eo:.2e} y {ey:.2e} state {ef:.2e} (worst o head {worst})")
    assert eo <= TOL_BF16 and ey <= TOL_BF16 and ef <= TOL_BF16
