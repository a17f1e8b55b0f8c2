"""GPU parity of gdn_mixer_decode_step, the one-launch decode mixer step.

Two checks per case, over three steps on one set of pools:
* bit-exact against the two-launch form (gdn_conv1d_fwd in decode form, then
  gdn_recurrent_step on the q, k, v column blocks of its output), which the
  entry point promises: outputs, conv histories and states are compared with
  torch.equal;
* against the float64 oracle: its gated delta rule and gated RMSNorm on the
  conv outputs the kernels used, with the tolerances of the two-launch parity
  tests (max|gpu - ref| / RMS(ref) <= 2e-3 for bf16 inputs, 1e-5 for fp32
  inputs; a bf16 output is allowed its own half-ulp rounding on top), and its
  history update, bit for bit.
Slots are permuted and one lane is inactive; slots no request names stay
bit-identical.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, dev, dev_i32, host, note, rel_max
from harness import inputs as I
from oracle import gdn_ref as R
from test_gpu_workloads import bf16_out_err

pytestmark = pytest.mark.gpu

SMALL_BF16 = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="bf16")
SMALL_F32 = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="f32")
GROUP8 = I.Layout(h_qk=1, h_v=8, d_k=128, d_v=128, chunk=64, dtype="bf16")


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_mixer_causal_amd import ops as _ops
    _ops.L.load()
    return _ops


CASES = [
    ("bf16_norm", SMALL_BF16, True, torch.float32),
    ("bf16_plain", SMALL_BF16, False, torch.bfloat16),
    ("f32_norm", SMALL_F32, True, torch.float32),
    ("model_norm", I.MODEL_LAYOUT, True, torch.bfloat16),
    ("group8_plain", GROUP8, False, torch.float32),
]


@pytest.mark.parametrize("name,lay,fused_norm,odt", CASES, ids=[c[0] for c in CASES])
def test_mixer_decode_step(ops, name, lay, fused_norm, odt):
    note(f"mixer decode step {name}")
    n_req, n_slots, n_steps = 5, 8, 3
    slots = np.array([6, 0, -1, 3, 1], np.int32)
    d = I.decode_inputs(70, lay, n_req, n_steps, n_slots=n_slots)
    tdt = torch.bfloat16 if lay.dtype == "bf16" else torch.float32
    nq = lay.h_qk * lay.d_k
    ch = lay.channels
    tol = 2e-3 if lay.dtype == "bf16" else 1e-5

    # fused and two-launch pools start equal; the oracle keeps float64 copies
    tail_f, state_f = dev(d["tail"], tdt), dev(d["state"])
    tail_u, state_u = tail_f.clone(), state_f.clone()
    tail_r, state_r = d["tail"].astype(np.float64), d["state"].astype(np.float64)
    w = dev(d["conv_w"], tdt)
    nw = dev(d["norm_w"])
    sl = dev_i32(slots)
    for step in range(n_steps):
        x = dev(d["x"][step], tdt)
        g, beta = dev(d["g"][step]), dev(d["beta"][step])
        z = dev(d["z"][step], tdt) if fused_norm else None
        o_f = torch.full((n_req, lay.h_v, lay.d_v), 3.0, dtype=odt, device=DEV)
        o_u = o_f.clone()
        ops.gdn_mixer_decode_step(x, w, tail_f, g, beta, state_f, o_f, h_qk=lay.h_qk, state_slots=sl, z=z,
                                  norm_w=nw if fused_norm else None)
        y = torch.full((n_req, ch), 5.0, dtype=tdt, device=DEV)   # the inactive lane's row must stay 5
        ops.gdn_conv1d_fwd(x, w, tail_u, y, state_slots=sl)
        q = y[:, :nq].view(n_req, lay.h_qk, lay.d_k)
        k = y[:, nq:2 * nq].view(n_req, lay.h_qk, lay.d_k)
        v = y[:, 2 * nq:].view(n_req, lay.h_v, lay.d_v)
        ops.gdn_recurrent_step(q, k, v, g, beta, state_u, o_u, state_slots=sl, z=z,
                               norm_w=nw if fused_norm else None)
        torch.cuda.synchronize()
        assert torch.equal(o_f, o_u), f"step {step}: outputs differ from the two-launch form"
        assert torch.equal(tail_f, tail_u), f"step {step}: conv histories differ"
        assert torch.equal(state_f, state_u), f"step {step}: states differ"

        # the oracle's recurrence and norm on the conv outputs the kernels used
        # (those of the two-launch form, which the fused step matches bit for
        # bit above), and the oracle's history update on the raw inputs
        yh = host(y)
        got = host(o_f)
        for r, s in enumerate(slots):
            if s < 0:
                assert np.all(got[r] == 3.0)
                assert np.all(yh[r] == 5.0)
                continue
            _, nt = R.causal_conv1d_silu(d["x"][step][r:r + 1], d["conv_w"], tail_r[s:s + 1], [0, 1],
                                         round_to_bf16=False)
            tail_r[s] = nt[0]
            q_, k_, v_ = R.split_heads(yh[r:r + 1], lay.h_qk, lay.d_k, lay.h_v, lay.d_v)
            o_ref, f_ref = R.gated_delta_rule(q_, k_, v_, d["g"][step][r:r + 1], d["beta"][step][r:r + 1],
                                              initial_state=state_r[s:s + 1])
            state_r[s] = f_ref[0]
            expect = R.gated_rmsnorm(o_ref[0], d["z"][step][r], d["norm_w"], 1e-6) if fused_norm else o_ref[0]
            e = bf16_out_err(got[r], expect) if odt == torch.bfloat16 else rel_max(got[r], expect)
            assert e <= tol, (step, r, e)
    gs, gt = host(state_f), host(tail_f)
    for s in range(n_slots):
        if s in slots:
            assert rel_max(gs[s], state_r[s]) <= tol
            np.testing.assert_array_equal(gt[s], tail_r[s])
        else:
            np.testing.assert_array_equal(gs[s], d["state"][s])
            np.testing.assert_array_equal(gt[s], d["tail"][s])


def test_mixer_decode_step_identity_slots_many_requests(ops):
    """256 requests of the model shape with the identity slot map (no
    state_slots): bit-exact against the two-launch form."""
    lay = I.MODEL_LAYOUT
    n_req = 256
    note(f"mixer decode step: {n_req} requests, identity slots")
    d = I.decode_inputs(71, lay, n_req, 1)
    nq = lay.h_qk * lay.d_k
    tail_f, state_f = dev(d["tail"], torch.bfloat16), dev(d["state"])
    tail_u, state_u = tail_f.clone(), state_f.clone()
    w, nw = dev(d["conv_w"], torch.bfloat16), dev(d["norm_w"])
    x, g, beta, z = dev(d["x"][0], torch.bfloat16), dev(d["g"][0]), dev(d["beta"][0]), dev(d["z"][0], torch.bfloat16)
    o_f = torch.empty((n_req, lay.h_v, lay.d_v), dtype=torch.bfloat16, device=DEV)
    o_u = torch.empty_like(o_f)
    ops.gdn_mixer_decode_step(x, w, tail_f, g, beta, state_f, o_f, h_qk=lay.h_qk, z=z, norm_w=nw)
    y = torch.empty((n_req, lay.channels), dtype=torch.bfloat16, device=DEV)
    ops.gdn_conv1d_fwd(x, w, tail_u, y)
    ops.gdn_recurrent_step(y[:, :nq].view(n_req, lay.h_qk, lay.d_k), y[:, nq:2 * nq].view(n_req, lay.h_qk, lay.d_k),
                           y[:, 2 * nq:].view(n_req, lay.h_v, lay.d_v), g, beta, state_u, o_u, z=z, norm_w=nw)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_u)
    assert torch.equal(tail_f, tail_u)
    assert torch.equal(state_f, state_u)
