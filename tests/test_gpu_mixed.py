"""GPU parity of the mixed prefill-plus-decode calls (gdn_conv1d_mixed,
gdn_chunk_mixed) against the float64 oracle's mixer_mixed: prompt chunks and
decode tokens packed into one call over caller-owned state pools, with a
permuted slot map, fresh sequences, inactive lanes, zero-length sequences
and padding rows past the live token count.

Every row and pool entry that the pages exclude from the update (inactive
lanes, padding, fresh slots' old contents) holds NaN: outputs must not read
them and must leave them bit-identical.  Tolerances: max|gpu - ref| / RMS(ref)
<= 2e-3 (bf16 inputs), <= 1e-5 (fp32 inputs); histories bit-exact; the mixed
call bit-equal to gdn_chunk_fwd on the compacted active sequences.
"""
import numpy as np
import pytest
import torch

from gpu_util import bf16_ulp_check, conv_abs_sum, dev, dev_i32, host, note, rel_max
from harness import inputs as I
from oracle import gdn_ref as R

pytestmark = pytest.mark.gpu

SMALL = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="bf16")

CASES = {
    # lengths (a decode token is a length-1 sequence), slots (-1 inactive or padding), fresh flags
    "bf16": dict(layout=SMALL, tol=2e-3, n_slots=12, t_pad=20,
                 lengths=[150, 1, 64, 1, 0, 37, 1, 130, 0, 0],
                 slots=[7, 2, 0, 11, 5, -1, 9, -1, -1, -1],
                 fresh=[1, 0, 0, 1, 1, 0, 0, 0, 0, 0]),
    "f32": dict(layout=I.TINY_LAYOUT, tol=1e-5, n_slots=7, t_pad=5,
                lengths=[40, 1, 16, 0, 1, 23],
                slots=[3, 0, -1, 2, 5, 1],
                fresh=[0, 1, 0, 1, 0, 0]),
}


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_mixer_causal_amd import ops as _ops
    _ops.L.load()
    return _ops


def _dead_rows(cu, slots, t_cap):
    """Token rows no active sequence owns: inactive lanes and padding."""
    dead = np.ones(t_cap, bool)
    for s in range(len(cu) - 1):
        if slots[s] >= 0:
            dead[cu[s]:cu[s + 1]] = False
    return dead


@pytest.mark.parametrize("name", list(CASES))
def test_mixed_batch(ops, name):
    c = CASES[name]
    lay, tol = c["layout"], c["tol"]
    slots, fresh = np.array(c["slots"]), np.array(c["fresh"])
    note(f"mixed batch {name}: lengths {c['lengths']} slots {c['slots']} fresh {c['fresh']}")
    d = I.mixed_batch_inputs(70, lay, c["lengths"], c["n_slots"], t_pad=c["t_pad"])
    cu, t_cap = d["cu_seqlens"], d["t_cap"]
    dead = _dead_rows(cu, slots, t_cap)
    for key in ("x", "beta", "g", "z"):
        d[key][dead] = np.nan
    for s in np.nonzero(fresh)[0]:
        d["tail_pool"][slots[s]] = np.nan    # a fresh sequence's pool row is not read
        d["state_pool"][slots[s]] = np.nan
    tdt = torch.bfloat16 if lay.dtype == "bf16" else torch.float32
    bf16 = lay.dtype == "bf16"

    tails_ref = d["tail_pool"].astype(np.float64)
    states_ref = d["state_pool"].astype(np.float64)
    ref = R.mixer_mixed(d["x"], d["conv_w"], tails_ref, states_ref, slots, fresh, d["beta"], d["g"], d["z"],
                        d["norm_w"], cu, h_qk=lay.h_qk, h_v=lay.h_v, d_k=lay.d_k, d_v=lay.d_v,
                        bf16_boundary=bf16)

    # conv over the pool of histories
    cu_d, sl_d, fr_d = dev_i32(cu), dev_i32(slots), dev_i32(fresh)
    x = dev(d["x"], tdt)
    tail = dev(d["tail_pool"], tdt)
    y_conv = torch.full((t_cap, lay.channels), float("nan"), dtype=tdt, device=x.device)
    ops.gdn_conv1d_mixed(x, dev(d["conv_w"], tdt), tail, y_conv, cu_seqlens=cu_d, state_slots=sl_d, fresh=fr_d)
    torch.cuda.synchronize()
    yc = host(y_conv)
    live = ~dead
    assert np.all(np.isnan(yc[dead])), "rows of inactive lanes or padding were written"
    th = host(tail)
    named = set(int(p) for p in slots if p >= 0)
    for p in range(c["n_slots"]):
        if p in named:
            np.testing.assert_array_equal(th[p], tails_ref[p])
        else:
            np.testing.assert_array_equal(np.isnan(th[p]), np.isnan(d["tail_pool"][p]))
            np.testing.assert_array_equal(th[p][~np.isnan(th[p])], d["tail_pool"][p][~np.isnan(th[p])])
    # conv outputs of the active sequences, each from its own starting history
    exact = np.zeros_like(yc)
    abs_sum = np.zeros_like(yc)
    for s in range(len(cu) - 1):
        if slots[s] < 0 or cu[s] == cu[s + 1]:
            continue
        a, b = cu[s], cu[s + 1]
        t0 = np.zeros((1, 3, lay.channels)) if fresh[s] else d["tail_pool"][slots[s]][None]
        exact[a:b], _ = R.causal_conv1d_silu(d["x"][a:b], d["conv_w"], t0, [0, b - a], round_to_bf16=False)
        abs_sum[a:b] = conv_abs_sum(d["x"][a:b], d["conv_w"], t0, [0, b - a])
    if bf16:
        frac = bf16_ulp_check(yc[live], ref["y_conv"][live], exact[live], abs_sum=abs_sum[live])
        note(f"  conv one-ulp fraction {frac:.2e}")
    else:
        assert rel_max(yc[live], ref["y_conv"][live]) <= tol

    # the recurrence with the fused norm reads the oracle's conv output (NaN on dead rows)
    qh, kh, vh = I.split_qkv(ref["y_conv"].astype(np.float32), lay)
    q, k, v = dev(qh, tdt), dev(kh, tdt), dev(vh, tdt)
    g, beta, z, nw = dev(d["g"]), dev(d["beta"]), dev(d["z"], tdt), dev(d["norm_w"])
    state = dev(d["state_pool"])
    o = torch.full((t_cap, lay.h_v, lay.d_v), float("nan"), device=x.device)
    ops.gdn_chunk_mixed(q, k, v, g, beta, state, o, chunk=lay.chunk, cu_seqlens=cu_d, state_slots=sl_d,
                        fresh=fr_d, z=z, norm_w=nw)
    torch.cuda.synchronize()
    # oracle recurrence and norm on exactly the values the kernels read (the
    # conv output as stored: bf16, or fp32 rounded from the float64 conv),
    # from each sequence's starting state
    y_ref = np.full_like(ref["y"], np.nan)
    st_ref = d["state_pool"].astype(np.float64)
    q64, k64, v64 = host(q), host(k), host(v)
    for s in range(len(cu) - 1):
        if slots[s] < 0:
            continue
        a, b = cu[s], cu[s + 1]
        s0 = np.zeros((1,) + st_ref.shape[1:]) if fresh[s] else st_ref[slots[s]][None]
        o_s, fin_s = R.gated_delta_rule(q64[a:b], k64[a:b], v64[a:b], d["g"][a:b], d["beta"][a:b],
                                        initial_state=s0)
        y_ref[a:b] = R.gated_rmsnorm(o_s, d["z"][a:b], d["norm_w"], 1e-6)
        st_ref[slots[s]] = fin_s[0]
    if bf16:   # the bf16 conv output is exact, so this is the mixed oracle itself
        np.testing.assert_allclose(y_ref[live], ref["y"][live], rtol=1e-12, atol=1e-12)
    oh, sh = host(o), host(state)
    assert np.all(np.isnan(oh[dead]))
    err = rel_max(oh[live], y_ref[live])
    act = sorted(named)
    err_s = rel_max(sh[act], st_ref[act])
    note(f"  y err {err:.2e}, pool state err {err_s:.2e}")
    assert err <= tol and err_s <= tol
    for p in range(c["n_slots"]):
        if p not in named:
            np.testing.assert_array_equal(sh[p], d["state_pool"][p])
    for s in range(len(cu) - 1):
        if slots[s] >= 0 and fresh[s] and cu[s] == cu[s + 1]:
            assert np.all(sh[slots[s]] == 0.0)    # fresh, zero-length: the zero state

    # bit-equal to gdn_chunk_fwd over the active sequences, compacted, from
    # their gathered starting states
    act_seq = [s for s in range(len(cu) - 1) if slots[s] >= 0]
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in act_seq])
    lens = [int(cu[s + 1] - cu[s]) for s in act_seq]
    init = np.stack([np.zeros(d["state_pool"].shape[1:], np.float32) if fresh[s] else d["state_pool"][slots[s]]
                     for s in act_seq])
    rows_d = torch.from_numpy(rows).to(x.device)
    o2 = torch.empty((len(rows), lay.h_v, lay.d_v), device=x.device)
    fin = dev(init)
    ops.gdn_chunk_fwd(q[rows_d].contiguous(), k[rows_d].contiguous(), v[rows_d].contiguous(),
                      g[rows_d].contiguous(), beta[rows_d].contiguous(), o2, chunk=lay.chunk,
                      cu_seqlens=dev_i32(I.cu_from_lengths(lens)), initial_state=fin, final_state=fin,
                      z=z[rows_d].contiguous(), norm_w=nw)
    torch.cuda.synchronize()
    assert torch.equal(o2, o[rows_d]), "mixed call differs from the compacted plain call"
    assert torch.equal(fin, state[dev_i32([slots[s] for s in act_seq]).long()])


def test_mixed_batch_all_inactive_or_empty(ops):
    """Capacity-only calls: every sequence inactive or empty (fresh ones zero
    their slots), no live token rows; nothing else is written."""
    lay = SMALL
    note("mixed batch: all inactive or empty")
    n_slots, t_cap = 6, 10
    lengths = [0, 0, 0, 0]
    slots = np.array([2, -1, 4, -1], np.int32)
    fresh = np.array([1, 0, 0, 1], np.int32)
    d = I.mixed_batch_inputs(71, lay, [1], n_slots, t_pad=t_cap - 1)   # pools and row shapes only
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32, device="cuda:0")
    x = dev(d["x"], torch.bfloat16)
    tail = dev(d["tail_pool"], torch.bfloat16)
    tail0 = tail.clone()
    y_conv = torch.full((t_cap, lay.channels), float("nan"), dtype=torch.bfloat16, device=x.device)
    ops.gdn_conv1d_mixed(x, dev(d["conv_w"], torch.bfloat16), tail, y_conv, cu_seqlens=cu, state_slots=dev_i32(slots),
                         fresh=dev_i32(fresh))
    q, k, v = ops.qkv_views(y_conv, lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
    state = dev(d["state_pool"])
    state0 = state.clone()
    o = torch.full((t_cap, lay.h_v, lay.d_v), float("nan"), device=x.device)
    ops.gdn_chunk_mixed(q, k, v, dev(d["g"]), dev(d["beta"]), state, o, chunk=lay.chunk, cu_seqlens=cu,
                        state_slots=dev_i32(slots), fresh=dev_i32(fresh), z=dev(d["z"], torch.bfloat16),
                        norm_w=dev(d["norm_w"]))
    torch.cuda.synchronize()
    assert torch.isnan(y_conv.float()).all() and torch.isnan(o).all()
    assert (state[2] == 0).all() and (tail[2] == 0).all()         # fresh, empty, active
    for p in (0, 1, 3, 5):
        assert torch.equal(state[p], state0[p]) and torch.equal(tail[p], tail0[p])
    assert torch.equal(state[4], state0[4]) and torch.equal(tail[4], tail0[4])   # empty, not fresh
