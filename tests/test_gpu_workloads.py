"""GPU parity on the full workload shapes: batched decode, varlen packed
prefill and long-context chunked prefill followed by decode.

Every GPU call runs on the whole shape (all requests, all 32 v-heads).  The
float64 oracle follows every request of the decode workload, every channel
and every v-head of the packed varlen workload, and eight v-heads of the
long-context stream (one from each range of four heads, the ranges the scan
places on one XCD each) over all of its 131,328 tokens.  Two stages are compared separately:
the conv1d + SiLU output against the oracle's conv (equal to the oracle's
bf16 rounding up to one ulp, with the fp32-sum allowance), and the gated
delta rule + gated RMSNorm against the oracle run on the same bf16 q/k/v the
GPU kernels read.  Bookkeeping (conv histories, state slots, one call against
many) is compared bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_util import (DEV, bf16_ulp_check, conv_abs_sum, conv_check_all_channels, dev, dev_i32, host,
                      note, rel_max)
from harness import inputs as I
from oracle import gdn_ref as R

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
LAY = I.MODEL_LAYOUT


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_mixer_causal_amd import ops as _ops
    _ops.L.load()
    return _ops


def bf16_out_err(got, ref):
    """Parity metric for a bf16 output: the output is the bf16 rounding of a
    value y_g with |got - y_g| <= ulp(got)/2, so max(|got - ref| - ulp(got)/2)
    / RMS(ref) bounds |y_g - ref| / RMS(ref), the fp32 result's error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    _, e = np.frexp(np.maximum(np.abs(got), 1e-30))
    half_ulp = np.ldexp(1.0, e - 9)
    excess = np.maximum(np.abs(got - ref) - half_ulp, 0.0)
    rms = float(np.sqrt(np.mean(ref * ref)))
    return float(np.max(excess)) / rms


def _conv_check(x, w, tail, cu, got):
    """GPU conv output (bf16) against the oracle conv on the same channels."""
    exact, _ = R.causal_conv1d_silu(x, w, tail, cu, round_to_bf16=False)
    return bf16_ulp_check(got, R.bf16_nearest(exact), exact, abs_sum=conv_abs_sum(x, w, tail, cu))


def _sampled_qkv(y, heads):
    qk_heads = sorted({h // LAY.group for h in heads})
    q, k, v = R.split_heads(y, len(qk_heads), LAY.d_k, len(heads), LAY.d_v)
    return q, k, v, [qk_heads.index(h // LAY.group) for h in heads]


# ---------------------------------------------------------------------------
# batched decode: 64 requests x 128 single-token steps
# ---------------------------------------------------------------------------

def test_decode_64_requests_128_steps(ops):
    """Conv step + recurrent step with the fused gated norm and bf16 output,
    64 requests whose states sit at a permutation of the 64 slots, 128 steps.
    The oracle follows every request (all heads) over all steps."""
    from gated_deltanet_mixer_causal_amd.ops import qkv_views
    n_req, n_steps = 64, 128
    note(f"decode {n_req} requests x {n_steps} steps, full model layout")
    d = I.decode_inputs(2, LAY, n_req, n_steps)
    perm = np.random.default_rng(12).permutation(n_req).astype(np.int32)
    slots = dev_i32(perm)
    tail = dev(d["tail"], torch.bfloat16)
    state = dev(d["state"])
    w, nw = dev(d["conv_w"], torch.bfloat16), dev(d["norm_w"])
    y_conv = torch.empty((n_req, LAY.channels), dtype=torch.bfloat16, device=DEV)
    q, k, v = qkv_views(y_conv, LAY.h_qk, LAY.d_k, LAY.h_v, LAY.d_v)
    y = torch.empty((n_req, LAY.h_v, LAY.d_v), dtype=torch.bfloat16, device=DEV)
    sample = list(range(n_req))
    got_conv = np.zeros((len(sample), n_steps, LAY.channels))
    got_y = np.zeros((len(sample), n_steps, LAY.h_v, LAY.d_v))
    for t in range(n_steps):
        ops.gdn_conv1d_fwd(dev(d["x"][t], torch.bfloat16), w, tail, y_conv, state_slots=slots)
        ops.gdn_recurrent_step(q, k, v, dev(d["g"][t]), dev(d["beta"][t]), state, y, state_slots=slots,
                               z=dev(d["z"][t], torch.bfloat16), norm_w=nw)
        got_conv[:, t] = host(y_conv[sample])
        got_y[:, t] = host(y[sample])
        assert torch.isfinite(y).all()
    torch.cuda.synchronize()
    g_state, g_tail = host(state), host(tail)
    # conv history of every request: its last three inputs, bit for bit
    for r in range(n_req):
        np.testing.assert_array_equal(g_tail[perm[r]], d["x"][n_steps - 3:, r])
    worst_y, worst_f = (0.0, -1), (0.0, -1)
    for i, r in enumerate(sample):
        s = perm[r]
        xs = d["x"][:, r]                                   # the request's tokens, in step order
        frac = _conv_check(xs, d["conv_w"], d["tail"][s:s + 1], [0, n_steps], got_conv[i])
        qs, ks, vs = R.split_heads(got_conv[i], LAY.h_qk, LAY.d_k, LAY.h_v, LAY.d_v)
        o_ref, f_ref = R.gated_delta_rule(qs, ks, vs, d["g"][:, r], d["beta"][:, r],
                                          initial_state=d["state"][s:s + 1])
        y_ref = R.gated_rmsnorm(o_ref, d["z"][:, r], d["norm_w"], 1e-6)
        ey = bf16_out_err(got_y[i], y_ref)
        ef = rel_max(g_state[s], f_ref[0])
        worst_y, worst_f = max(worst_y, (ey, r)), max(worst_f, (ef, r))
        assert ey <= TOL_BF16 and ef <= TOL_BF16, (r, ey, ef)
    note(f"  {len(sample)} requests: worst y {worst_y[0]:.2e} (request {worst_y[1]}), "
         f"worst state {worst_f[0]:.2e} (request {worst_f[1]})")


# ---------------------------------------------------------------------------
# varlen packed prefill: 8 sequences, 30,809 tokens
# ---------------------------------------------------------------------------

def test_varlen_8_sequences(ops):
    """8 packed sequences of log-uniform lengths with nonzero states and conv
    tails; conv, then the chunked rule with final states, then again with the
    fused gated norm and the state updated in place.  The oracle follows every
    channel of the conv and every v-head of the rule over every sequence."""
    from gated_deltanet_mixer_causal_amd.ops import qkv_views
    d = I.varlen_prefill_inputs()
    lengths, cu_h = d["lengths"], d["cu_seqlens"]
    assert lengths == [731, 1370, 14338, 5764, 757, 3101, 3754, 994]
    T = int(cu_h[-1])
    note(f"varlen prefill {lengths} (T={T}), full model layout")
    x = dev(d["x"], torch.bfloat16)
    tail = dev(d["tail"], torch.bfloat16)
    cu = dev_i32(cu_h)
    y_conv = torch.empty_like(x)
    ops.gdn_conv1d_fwd(x, dev(d["conv_w"], torch.bfloat16), tail, y_conv, cu_seqlens=cu)
    q, k, v = qkv_views(y_conv, LAY.h_qk, LAY.d_k, LAY.h_v, LAY.d_v)
    g, beta = dev(d["g"]), dev(d["beta"])
    state0 = dev(d["state"])
    fin = torch.full_like(state0, float("nan"))
    o = torch.empty((T, LAY.h_v, LAY.d_v), device=DEV)
    ops.gdn_chunk_fwd(q, k, v, g, beta, o, chunk=64, cu_seqlens=cu, initial_state=state0, final_state=fin)
    st = state0.clone()
    y = torch.empty((T, LAY.h_v, LAY.d_v), device=DEV)
    ops.gdn_chunk_fwd(q, k, v, g, beta, y, chunk=64, cu_seqlens=cu, initial_state=st, final_state=st,
                      z=dev(d["z"], torch.bfloat16), norm_w=dev(d["norm_w"]))
    torch.cuda.synchronize()
    assert torch.equal(st, fin)                              # in-place state == separate final state
    g_tail = host(tail)
    for s in range(len(lengths)):
        np.testing.assert_array_equal(g_tail[s], d["x"][cu_h[s + 1] - 3:cu_h[s + 1]])
    gy = host(y_conv)
    frac = conv_check_all_channels(d["x"], d["conv_w"], d["tail"], cu_h, gy, R)
    qs, ks, vs = R.split_heads(gy, LAY.h_qk, LAY.d_k, LAY.h_v, LAY.d_v)
    del gy
    o_ref, f_ref = R.gated_delta_rule(qs, ks, vs, d["g"], d["beta"], initial_state=d["state"], cu_seqlens=cu_h)
    y_ref = R.gated_rmsnorm(o_ref, d["z"], d["norm_w"], 1e-6)
    eo = rel_max(host(o), o_ref)
    ey = rel_max(host(y), y_ref)
    gf = host(fin)
    ef = max(rel_max(gf[s], f_ref[s]) for s in range(len(lengths)))
    note(f"  conv one-ulp {frac:.1e}  o {eo:.2e}  y {ey:.2e}  worst final state {ef:.2e}")
    assert eo <= TOL_BF16 and ey <= TOL_BF16 and ef <= TOL_BF16


# ---------------------------------------------------------------------------
# long context: 16 calls of 8192 tokens, then 256 decode steps
# ---------------------------------------------------------------------------

def test_long_context_16_calls_then_decode(ops):
    """131,072 tokens as 16 chunked-prefill calls carrying the conv history and
    the fp32 state, fused gated norm, then 256 decode steps.  The 16 calls equal
    one call over all 131,072 tokens bit for bit; eight v-heads, one from each
    range of four heads, are compared with one single-shot oracle run over all
    131,328 tokens."""
    from gated_deltanet_mixer_causal_amd.ops import qkv_views
    n_calls, call_len, n_decode = 16, 8192, 256
    T = n_calls * call_len
    note(f"long context {n_calls} x {call_len} + {n_decode} decode steps, full model layout")
    heads = [1, 6, 9, 14, 17, 22, 25, 30]
    chs = I.head_channels(LAY, heads)
    chs_dev = torch.from_numpy(chs).to(DEV)
    hsel = torch.tensor(heads, device=DEV)
    ch = LAY.channels
    x_all = torch.empty((T, ch), dtype=torch.bfloat16, device=DEV)
    z_all = torch.empty((T, LAY.h_v, LAY.d_v), dtype=torch.bfloat16, device=DEV)
    g_all = torch.empty((T, LAY.h_v), device=DEV)
    b_all = torch.empty((T, LAY.h_v), device=DEV)
    yc_calls = torch.empty((T, ch), dtype=torch.bfloat16, device=DEV)
    y_calls = torch.empty((T, LAY.h_v, LAY.d_v), device=DEV)
    tail = torch.zeros((1, 3, ch), dtype=torch.bfloat16, device=DEV)
    state = torch.zeros((1, LAY.h_v, LAY.d_v, LAY.d_k), device=DEV)
    cu_call = dev_i32([0, call_len])
    host_x, host_g, host_b, host_z = [], [], [], []
    got_conv, got_y = [], []
    w = nw = None
    conv_w = norm_w = None
    for kind, c in I.long_context_calls():
        if w is None:
            conv_w, norm_w = c["conv_w"], c["norm_w"]
            w, nw = dev(conv_w, torch.bfloat16), dev(norm_w)
        host_x.append(c["x"][:, chs])
        host_g.append(c["g"][:, heads])
        host_b.append(c["beta"][:, heads])
        host_z.append(c["z"][:, heads])
        i = c["index"]
        if kind == "prefill":
            sl = slice(i * call_len, (i + 1) * call_len)
            x_all[sl] = dev(c["x"], torch.bfloat16)
            z_all[sl] = dev(c["z"], torch.bfloat16)
            g_all[sl], b_all[sl] = dev(c["g"]), dev(c["beta"])
            ops.gdn_conv1d_fwd(x_all[sl], w, tail, yc_calls[sl], cu_seqlens=cu_call)
            q, k, v = qkv_views(yc_calls[sl], LAY.h_qk, LAY.d_k, LAY.h_v, LAY.d_v)
            ops.gdn_chunk_fwd(q, k, v, g_all[sl], b_all[sl], y_calls[sl], chunk=64, cu_seqlens=cu_call,
                              initial_state=state, final_state=state, z=z_all[sl], norm_w=nw)
            got_conv.append(host(yc_calls[sl][:, chs_dev]))
            got_y.append(host(y_calls[sl][:, hsel]))
            if i == n_calls - 1:
                state_prefill = state.clone()
                tail_prefill = tail.clone()
        else:
            if i == n_calls:
                note("  prefill calls done; decode")
            yc = torch.empty((1, ch), dtype=torch.bfloat16, device=DEV)
            ops.gdn_conv1d_fwd(dev(c["x"], torch.bfloat16), w, tail, yc)
            q, k, v = qkv_views(yc, LAY.h_qk, LAY.d_k, LAY.h_v, LAY.d_v)
            y1 = torch.empty((1, LAY.h_v, LAY.d_v), device=DEV)
            ops.gdn_recurrent_step(q, k, v, dev(c["g"]), dev(c["beta"]), state, y1,
                                   z=dev(c["z"], torch.bfloat16), norm_w=nw)
            got_conv.append(host(yc[:, chs_dev]))
            got_y.append(host(y1[:, hsel]))
    torch.cuda.synchronize()
    # one call over all 131,072 tokens reproduces the 16 calls bit for bit
    note("  single-call rerun")
    tail1 = torch.zeros_like(tail)
    yc_one = torch.empty_like(yc_calls)
    cu_one = dev_i32([0, T])
    ops.gdn_conv1d_fwd(x_all, w, tail1, yc_one, cu_seqlens=cu_one)
    assert torch.equal(yc_one, yc_calls) and torch.equal(tail1, tail_prefill)
    del yc_one
    q, k, v = qkv_views(yc_calls, LAY.h_qk, LAY.d_k, LAY.h_v, LAY.d_v)
    y_one = torch.empty_like(y_calls)
    fin_one = torch.empty_like(state)
    ops.gdn_chunk_fwd(q, k, v, g_all, b_all, y_one, chunk=64, cu_seqlens=cu_one, final_state=fin_one,
                      z=z_all, norm_w=nw)
    torch.cuda.synchronize()
    assert torch.equal(y_one, y_calls) and torch.equal(fin_one, state_prefill)
    del y_one
    # oracle: one run over the whole stream for the sampled heads
    note("  oracle, single shot over 131,328 tokens")
    xs = np.concatenate(host_x)
    gy = np.concatenate(got_conv)
    ntok = xs.shape[0]
    frac = conv_check_all_channels(xs, conv_w[chs], np.zeros((1, 3, len(chs))), [0, ntok], gy, R)
    qs, ks, vs, qk_of_v = _sampled_qkv(gy, heads)
    o_ref, f_ref = R.gated_delta_rule(qs, ks, vs, np.concatenate(host_g), np.concatenate(host_b),
                                      qk_of_v=qk_of_v)
    y_ref = R.gated_rmsnorm(o_ref, np.concatenate(host_z), norm_w, 1e-6)
    gyy = np.concatenate(got_y)
    ey_pre = rel_max(gyy[:T], y_ref[:T])
    ey_dec = rel_max(gyy[T:], y_ref[T:])
    ef = rel_max(host(state[0][hsel]), f_ref[0])
    note(f"  conv one-ulp {frac:.1e}  y prefill {ey_pre:.2e}  y decode {ey_dec:.2e}  state {ef:.2e}")
    assert ey_pre <= TOL_BF16 and ey_dec <= TOL_BF16 and ef <= TOL_BF16
