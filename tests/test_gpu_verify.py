"""GPU parity of speculative verification and state maintenance against the
float64 oracle: gdn_recurrent_verify (state checkpoint columns),
gdn_conv1d_verify (conv windows per column) and gdn_state_rows_copy
(restore / snapshot / reset as indirect row copies), and one whole round:
verify W draft tokens, accept a prefix, restore it, decode the next token.

Tolerances: max|gpu - ref| / RMS(ref) <= 1e-5 (fp32 inputs), <= 2e-3 (bf16
inputs); live states, histories, windows and copies are bit-exact.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, bf16_ulp_check, conv_abs_sum, dev, dev_i32, host, note, rel_max
from harness import inputs as I
from oracle import gdn_ref as R

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-3
SMALL = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="bf16")
N_COLS = 8


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_mixer_causal_amd import ops as _ops
    _ops.L.load()
    return _ops


def _cast(layout):
    return I.round_bf16 if layout.dtype == "bf16" else (lambda a: np.asarray(a, np.float32))


def _tdt(layout):
    return torch.bfloat16 if layout.dtype == "bf16" else torch.float32


def _tokens(rng, layout, rows):
    c = _cast(layout)
    q = c(rng.standard_normal((rows, layout.h_qk, layout.d_k)).astype(np.float32))
    k = c(rng.standard_normal((rows, layout.h_qk, layout.d_k)).astype(np.float32))
    v = c(rng.standard_normal((rows, layout.h_v, layout.d_v)).astype(np.float32))
    gt = I.raw_gate_inputs(int(rng.integers(1 << 30)), rows, layout.h_v)
    g, beta = R.gates_from_projections(gt["a"], gt["b"], gt["a_log"])
    z = c(rng.standard_normal((rows, layout.h_v, layout.d_v)).astype(np.float32))
    return q, k, v, g.astype(np.float32), beta.astype(np.float32), z


@pytest.mark.parametrize("layout,w,fused", [(SMALL, 4, False), (SMALL, 1, True), (SMALL, 8, True),
                                            (I.TINY_LAYOUT, 5, False)], ids=["bf16_w4", "bf16_w1_norm",
                                                                             "bf16_w8_norm", "f32_d16_w5"])
def test_verify_columns_and_outputs(ops, layout, w, fused):
    note(f"recurrent verify {layout.dtype} d={layout.d_k} W={w} fused={fused}")
    rng = np.random.default_rng(60 + w)
    n_req, n_slots = 5, 8
    slots = np.array([6, 0, -1, 3, 1], np.int32)
    hv, dv, dk = layout.h_v, layout.d_v, layout.d_k
    tol = TOL_BF16 if layout.dtype == "bf16" else TOL_F32
    tdt = _tdt(layout)
    q, k, v, g, beta, z = _tokens(rng, layout, n_req * w)
    nw = (1 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    state = (0.02 * rng.standard_normal((n_slots, hv, dv, dk))).astype(np.float32)
    sd = dev(state)
    ck = torch.full((n_slots, N_COLS, hv, dv, dk), 7.0, device=DEV)
    o = torch.full((n_req * w, hv, dv), 3.0, device=DEV)
    ops.gdn_recurrent_verify(dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(g), dev(beta), sd, ck, o, n_tok=w,
                             state_slots=dev_i32(slots), z=dev(z, tdt) if fused else None,
                             norm_w=dev(nw) if fused else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(sd), state)            # the live states are only read
    go, gc = host(o), host(ck)
    for r, s in enumerate(slots):
        rows = slice(r * w, (r + 1) * w)
        if s < 0:
            assert np.all(go[rows] == 3.0)
            continue
        o_ref, c_ref = R.verify_checkpoints(q[rows], k[rows], v[rows], g[rows], beta[rows], initial_state=state[s])
        if fused:
            o_ref = np.stack([R.gated_rmsnorm(o_ref[t], z[r * w + t], nw, 1e-6) for t in range(w)])
        eo, ec = rel_max(go[rows], o_ref), rel_max(gc[s, :w], c_ref)
        assert eo <= tol and ec <= tol, (r, eo, ec)
        assert np.all(gc[s, w:] == 7.0)                       # columns past the round untouched
    for s in set(range(n_slots)) - set(int(x) for x in slots if x >= 0):
        assert np.all(gc[s] == 7.0)                           # slots of no active request untouched


def test_conv_verify_windows(ops):
    note("conv verify")
    rng = np.random.default_rng(70)
    lay = SMALL
    ch, n_req, n_slots, w = lay.channels, 4, 6, 3
    slots = np.array([5, -1, 0, 2], np.int32)
    x = I.round_bf16(rng.standard_normal((n_req * w, ch)).astype(np.float32))
    cw = I.round_bf16((0.5 * rng.standard_normal((ch, 4))).astype(np.float32))
    tails = I.round_bf16(rng.standard_normal((n_slots, 3, ch)).astype(np.float32))
    td = dev(tails, torch.bfloat16)
    win = torch.full((n_slots, N_COLS, 3, ch), 5.0, dtype=torch.bfloat16, device=DEV)
    y = torch.full((n_req * w, ch), 9.0, dtype=torch.bfloat16, device=DEV)
    ops.gdn_conv1d_verify(dev(x, torch.bfloat16), dev(cw, torch.bfloat16), td, y, win, n_tok=w,
                          state_slots=dev_i32(slots))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(td), tails)            # live histories only read
    gy, gw = host(y), host(win)
    for r, s in enumerate(slots):
        rows = slice(r * w, (r + 1) * w)
        if s < 0:
            assert np.all(gy[rows] == 9.0)
            continue
        ref, _ = R.causal_conv1d_silu(x[rows], cw, tails[s:s + 1], [0, w], round_to_bf16=True)
        exact, _ = R.causal_conv1d_silu(x[rows], cw, tails[s:s + 1], [0, w], round_to_bf16=False)
        bf16_ulp_check(gy[rows], ref, exact, max_frac=0.01, abs_sum=conv_abs_sum(x[rows], cw, tails[s:s + 1], [0, w]))
        np.testing.assert_array_equal(gw[s, :w], R.conv_windows(tails[s], x[rows]))
        assert np.all(gw[s, w:] == 5.0)


def test_rows_copy_restore_snapshot_reset(ops):
    note("state rows copy")
    rng = np.random.default_rng(80)
    src = rng.standard_normal((10, 4, 32)).astype(np.float32)
    dst = rng.standard_normal((6, 4, 32)).astype(np.float32)
    ts, td = dev(src), dev(dst)
    # entries: 9 -> 2, 0 -> 5, an out-of-range source (skipped), a negative destination (skipped)
    ops.gdn_state_rows_copy(td, dev_i32([2, 5, 1, -1]), ts, dev_i32([9, 0, 10, 3]))
    torch.cuda.synchronize()
    expect = dst.copy()
    expect[2], expect[5] = src[9], src[0]
    np.testing.assert_array_equal(host(td), expect)
    # reset: zero rows 0 and 3
    ops.gdn_state_rows_copy(td, dev_i32([0, 3]))
    torch.cuda.synchronize()
    expect[0] = expect[3] = 0
    np.testing.assert_array_equal(host(td), expect)
    # snapshot inside one pool: rows 4 <- 1
    ops.gdn_state_rows_copy(td, dev_i32([4]), td, dev_i32([1]))
    torch.cuda.synchronize()
    expect[4] = expect[1]
    np.testing.assert_array_equal(host(td), expect)
    # a large row (a 2 MiB state slot) crosses many 16 KiB chunks
    big_src = rng.standard_normal((3, 32, 128, 128)).astype(np.float32)
    big_dst = np.zeros((2, 32, 128, 128), np.float32)
    tbs, tbd = dev(big_src), dev(big_dst)
    ops.gdn_state_rows_copy(tbd, dev_i32([1, 0]), tbs, dev_i32([0, 2]))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(tbd), big_src[[2, 0]])


def test_speculative_round_restore_then_decode(ops):
    """Conv + recurrence verify of W = 4 draft tokens, accept a = 2, restore
    column a - 1 of the state and of the conv windows into the live slot, and
    decode one more token through the plain decode path.  The restored slot
    equals the column bit for bit, and the next token's output and state equal
    the oracle's recurrence over the two accepted tokens and the next one (on
    the bf16 conv outputs the kernels read; the conv itself is compared with
    the oracle's conv)."""
    note("speculative round: verify 4, accept 2, restore, decode")
    lay = SMALL
    rng = np.random.default_rng(90)
    ch, hv, dv, dk = lay.channels, lay.h_v, lay.d_v, lay.d_k
    n_req, n_slots, w, acc = 2, 3, 4, 2
    slots = np.array([2, 0], np.int32)
    cw = I.round_bf16((0.5 * rng.standard_normal((ch, 4))).astype(np.float32))
    tails = I.round_bf16(rng.standard_normal((n_slots, 3, ch)).astype(np.float32))
    state = (0.02 * rng.standard_normal((n_slots, hv, dv, dk))).astype(np.float32)
    x = I.round_bf16(rng.standard_normal((n_req * w, ch)).astype(np.float32))
    x_next = I.round_bf16(rng.standard_normal((n_req, ch)).astype(np.float32))
    gt = I.raw_gate_inputs(91, n_req * w + n_req, hv)
    g_all, b_all = R.gates_from_projections(gt["a"], gt["b"], gt["a_log"])
    g_all, b_all = g_all.astype(np.float32), b_all.astype(np.float32)
    g, beta, g_next, b_next = g_all[:n_req * w], b_all[:n_req * w], g_all[n_req * w:], b_all[n_req * w:]
    from gated_deltanet_mixer_causal_amd.ops import qkv_views
    bf = torch.bfloat16
    td, sd, tw, ts = dev(tails, bf), dev(state), dev(cw, bf), dev_i32(slots)
    win = torch.zeros((n_slots, N_COLS, 3, ch), dtype=bf, device=DEV)
    ck = torch.zeros((n_slots, N_COLS, hv, dv, dk), device=DEV)
    yc = torch.empty((n_req * w, ch), dtype=bf, device=DEV)
    ops.gdn_conv1d_verify(dev(x, bf), tw, td, yc, win, n_tok=w, state_slots=ts)
    q, k, v = qkv_views(yc, lay.h_qk, lay.d_k, hv, dv)
    o_ver = torch.empty((n_req * w, hv, dv), device=DEV)
    ops.gdn_recurrent_verify(q, k, v, dev(g), dev(beta), sd, ck, o_ver, n_tok=w, state_slots=ts)
    # accept `acc` tokens of every request: restore column acc - 1 (row slot * N_COLS + acc - 1)
    rows = dev_i32(slots)
    cols = dev_i32(slots * N_COLS + (acc - 1))
    ops.gdn_state_rows_copy(sd, rows, ck.view(n_slots * N_COLS, hv, dv, dk), cols)
    ops.gdn_state_rows_copy(td, rows, win.view(n_slots * N_COLS, 3, ch), cols)
    torch.cuda.synchronize()
    gy, gck, gwin, g_sd, g_td = host(yc), host(ck), host(win), host(sd), host(td)
    for r, s in enumerate(slots):
        np.testing.assert_array_equal(g_sd[s], gck[s, acc - 1])
        np.testing.assert_array_equal(g_td[s], gwin[s, acc - 1])
        np.testing.assert_array_equal(g_td[s], R.conv_windows(tails[s], x[r * w:(r + 1) * w])[acc - 1])
    # the next token through the plain decode path
    y1 = torch.empty((n_req, ch), dtype=bf, device=DEV)
    ops.gdn_conv1d_fwd(dev(x_next, bf), tw, td, y1, state_slots=ts)
    q1, k1, v1 = qkv_views(y1, lay.h_qk, lay.d_k, hv, dv)
    o1 = torch.empty((n_req, hv, dv), device=DEV)
    ops.gdn_recurrent_step(q1, k1, v1, dev(g_next), dev(b_next), sd, o1, state_slots=ts)
    torch.cuda.synchronize()
    gy1, go1, go_ver, g_sd = host(y1), host(o1), host(o_ver), host(sd)
    for r, s in enumerate(slots):
        # conv of the next token from the restored history, against the oracle's conv
        ref, _ = R.causal_conv1d_silu(x_next[r:r + 1], cw, g_td[s:s + 1], [0, 1], round_to_bf16=True)
        exact, _ = R.causal_conv1d_silu(x_next[r:r + 1], cw, g_td[s:s + 1], [0, 1], round_to_bf16=False)
        bf16_ulp_check(gy1[r:r + 1], ref, exact, max_frac=0.02,
                       abs_sum=conv_abs_sum(x_next[r:r + 1], cw, g_td[s:s + 1], [0, 1]))
        # recurrence over the accepted tokens and the next one
        seq = np.concatenate([gy[r * w:r * w + acc], gy1[r:r + 1]])
        qs, ks, vs = R.split_heads(seq, lay.h_qk, dk, hv, dv)
        gs = np.concatenate([g[r * w:r * w + acc], g_next[r:r + 1]])
        bs = np.concatenate([beta[r * w:r * w + acc], b_next[r:r + 1]])
        o_ref, f_ref = R.gated_delta_rule(qs, ks, vs, gs, bs, initial_state=state[s:s + 1])
        e_ver = rel_max(go_ver[r * w:r * w + acc], o_ref[:acc])
        e1 = rel_max(go1[r], o_ref[acc])
        ef = rel_max(g_sd[s], f_ref[0])
        note(f"  request {r} (slot {s}): accepted outputs {e_ver:.2e}, next output {e1:.2e}, state {ef:.2e}")
        assert e_ver <= TOL_BF16 and e1 <= TOL_BF16 and ef <= TOL_BF16
