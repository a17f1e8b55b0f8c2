"""GPU edge cases of the chunk and decode entry points against the oracle:
fp32 inputs at d=128, a non-unit scale with permuted sequences, head
groupings of 1 and 4 v-heads per q/k head, an optional final state, 300
packed sequences, calls whose sequences are all empty, a poisoned workspace, and a hard reset (g = -inf)
in the decode step.
"""
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


def _tdt(layout):
    return torch.bfloat16 if layout.dtype == "bf16" else torch.float32


def _run(ops, layout, q, k, v, g, beta, cu, state0, *, scale=1.0, z=None, nw=None, ws=None,
         o_fill=float("nan")):
    tdt = _tdt(layout)
    T = q.shape[0]
    o = torch.full((T, layout.h_v, layout.d_v), o_fill, device=DEV)
    fin = torch.full(state0.shape, float("nan"), device=DEV)
    ops.gdn_chunk_fwd(dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(g), dev(beta), o, chunk=layout.chunk, scale=scale,
                      cu_seqlens=dev_i32(cu), initial_state=dev(state0), final_state=fin,
                      z=None if z is None else dev(z, tdt), norm_w=None if nw is None else dev(nw), workspace=ws)
    torch.cuda.synchronize()
    return o, fin


def test_chunk_f32_d128(ops):
    """fp32 inputs at d=128, chunk 64 (fp32 matrix cores), four sequences
    with ragged tails and nonzero states, model-like decays; the one-token
    sequence runs in the one-token kernel."""
    lay = I.Layout(h_qk=2, h_v=4, d_k=128, d_v=128, chunk=64, dtype="f32")
    note("chunk fp32 d=128")
    d = I.prefill_inputs(31, lay, [150, 7, 1, 64], state_std=0.02)
    q, k, v = I.split_qkv(d["x"], lay)
    o, fin = _run(ops, lay, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"])
    o_ref, f_ref = R.gated_delta_rule(q, k, v, d["g"], d["beta"], initial_state=d["state"],
                                      cu_seqlens=d["cu_seqlens"])
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_F32 and ef <= TOL_F32


def test_chunk_scale_and_sequence_permutation(ops):
    """scale = d^-1/2 against the oracle; permuting the packed sequences (and
    their states) permutes every output and final state bit for bit."""
    note("chunk scale and permutation")
    lengths = [90, 33, 128]
    d = I.prefill_inputs(32, SMALL, lengths, state_std=0.02)
    q, k, v = I.split_qkv(d["x"], SMALL)
    cu = d["cu_seqlens"]
    scale = 128 ** -0.5
    o, fin = _run(ops, SMALL, q, k, v, d["g"], d["beta"], cu, d["state"], scale=scale)
    o_ref, f_ref = R.gated_delta_rule(q, k, v, d["g"], d["beta"], scale=scale, initial_state=d["state"],
                                      cu_seqlens=cu)
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    perm = [2, 0, 1]
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in perm])
    cu_p = I.cu_from_lengths([lengths[s] for s in perm])
    o_p, fin_p = _run(ops, SMALL, q[rows], k[rows], v[rows], d["g"][rows], d["beta"][rows], cu_p,
                      d["state"][perm], scale=scale)
    assert torch.equal(o_p, o[torch.from_numpy(rows).to(DEV)])
    assert torch.equal(fin_p, fin[torch.tensor(perm, device=DEV)])


@pytest.mark.parametrize("h_qk,h_v", [(4, 4), (1, 4), (2, 8)])
def test_chunk_head_grouping(ops, h_qk, h_v):
    """v-heads per q/k head of 1 and 4 (the model layout has 2), with a
    scale, ragged sequences and nonzero states, against the oracle."""
    lay = I.Layout(h_qk=h_qk, h_v=h_v, d_k=128, d_v=128, chunk=64, dtype="bf16")
    note(f"chunk head grouping {h_qk} q/k heads, {h_v} v-heads")
    d = I.prefill_inputs(37, lay, [100, 64, 3], state_std=0.02)
    q, k, v = I.split_qkv(d["x"], lay)
    o, fin = _run(ops, lay, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"], scale=0.25)
    o_ref, f_ref = R.gated_delta_rule(q, k, v, d["g"], d["beta"], scale=0.25, initial_state=d["state"],
                                      cu_seqlens=d["cu_seqlens"])
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16


def test_chunk_final_state_optional(ops):
    """Three sequences, 9,000 tokens, 4 q/k and 8 v-heads: the outputs do not
    depend on whether a final state is asked for or updated in place (bit for
    bit), they match the oracle, and a NULL initial state equals zeros."""
    lay = I.Layout(h_qk=4, h_v=8, d_k=128, d_v=128, chunk=64, dtype="bf16")
    note("chunk 3 sequences, 9,000 tokens, optional final state")
    lengths = [5000, 3000, 1000]
    d = I.prefill_inputs(38, lay, lengths, state_std=0.02)
    q, k, v = I.split_qkv(d["x"], lay)
    cu = d["cu_seqlens"]
    tdt = torch.bfloat16
    T = q.shape[0]
    args = (dev(q, tdt), dev(k, tdt), dev(v, tdt), dev(d["g"]), dev(d["beta"]))
    o_split = torch.full((T, lay.h_v, lay.d_v), float("nan"), device=DEV)
    fin = torch.full(d["state"].shape, float("nan"), device=DEV)
    ops.gdn_chunk_fwd(*args, o_split, chunk=64, cu_seqlens=dev_i32(cu), initial_state=dev(d["state"]),
                      final_state=fin)
    o_one = torch.full_like(o_split, float("nan"))
    ops.gdn_chunk_fwd(*args, o_one, chunk=64, cu_seqlens=dev_i32(cu), initial_state=dev(d["state"]))
    st_inplace = dev(d["state"])
    o_inplace = torch.full_like(o_split, float("nan"))
    ops.gdn_chunk_fwd(*args, o_inplace, chunk=64, cu_seqlens=dev_i32(cu), initial_state=st_inplace,
                      final_state=st_inplace)
    torch.cuda.synchronize()
    assert torch.equal(o_split, o_one) and torch.equal(o_split, o_inplace) and torch.equal(fin, st_inplace)
    o_ref, f_ref = R.gated_delta_rule(q, k, v, d["g"], d["beta"], initial_state=d["state"], cu_seqlens=cu)
    eo, ef = rel_max(host(o_split), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    # NULL initial state
    o0 = torch.empty_like(o_split)
    f0 = torch.empty_like(fin)
    ops.gdn_chunk_fwd(*args, o0, chunk=64, cu_seqlens=dev_i32(cu), final_state=f0)
    o0_one = torch.empty_like(o_split)
    ops.gdn_chunk_fwd(*args, o0_one, chunk=64, cu_seqlens=dev_i32(cu))
    torch.cuda.synchronize()
    assert torch.equal(o0, o0_one)


def test_chunk_many_sequences(ops):
    """300 packed sequences (more than one pass of the longest-first ordering
    loop), many of equal length, some empty, lengths around chunk edges."""
    note("chunk 300 sequences")
    lay = I.Layout(h_qk=1, h_v=2, d_k=128, d_v=128, chunk=64, dtype="bf16")
    rng = np.random.default_rng(36)
    lengths = [int(v) for v in rng.choice([0, 1, 5, 63, 64, 65, 130, 200], 300)]
    lengths[17] = 700   # one long sequence in the middle of the list
    d = I.prefill_inputs(36, lay, lengths, state_std=0.02)
    q, k, v = I.split_qkv(d["x"], lay)
    o, fin = _run(ops, lay, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"])
    o_ref, f_ref = R.gated_delta_rule(q, k, v, d["g"], d["beta"], initial_state=d["state"],
                                      cu_seqlens=d["cu_seqlens"])
    eo, ef = rel_max(host(o), o_ref), rel_max(host(fin), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    empty = [i for i, n in enumerate(lengths) if n == 0]
    assert torch.equal(fin[empty], dev(d["state"][empty]))


def test_chunk_all_sequences_empty(ops):
    """t_total = 0 with three zero-length sequences: the final states equal the
    initial ones (zeros without them), bit for bit; per-token buffers are empty."""
    note("chunk all sequences empty")
    lay = SMALL
    st = dev(np.random.default_rng(33).standard_normal((3, lay.h_v, lay.d_v, lay.d_k)).astype(np.float32))
    empty = lambda h, dd: torch.empty((0, h, dd), dtype=torch.bfloat16, device=DEV)
    q, k, v = empty(lay.h_qk, lay.d_k), empty(lay.h_qk, lay.d_k), empty(lay.h_v, lay.d_v)
    g = torch.empty((0, lay.h_v), device=DEV)
    cu = dev_i32([0, 0, 0, 0])
    for init in (st, None):
        fin = torch.full(st.shape, float("nan"), device=DEV)
        o = torch.empty((0, lay.h_v, lay.d_v), device=DEV)
        ops.gdn_chunk_fwd(q, k, v, g, g, o, chunk=64, cu_seqlens=cu, initial_state=init, final_state=fin)
        torch.cuda.synchronize()
        assert torch.equal(fin, st if init is not None else torch.zeros_like(st))


def test_chunk_poisoned_workspace(ops):
    """The workspace needs no initialisation: a workspace filled with 0xFF bytes
    (NaN in every float and bf16 field) gives bit-identical results to a
    zeroed one, with and without the fused norm."""
    note("chunk poisoned workspace")
    lengths = [150, 1, 66]
    d = I.prefill_inputs(34, SMALL, lengths, state_std=0.02)
    q, k, v = I.split_qkv(d["x"], SMALL)
    T = q.shape[0]
    for fused in (False, True):
        nbytes = ops.gdn_chunk_fwd_workspace_size(SMALL.h_qk, SMALL.h_v, 128, 128, 64, len(lengths), T,
                                                  torch.bfloat16, fused)
        res = []
        for fill in (0, 255):
            ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
            res.append(_run(ops, SMALL, q, k, v, d["g"], d["beta"], d["cu_seqlens"], d["state"],
                            z=d["z"] if fused else None, nw=d["norm_w"] if fused else None, ws=ws))
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
        assert torch.isfinite(res[0][0]).all()


def test_recurrent_hard_reset(ops):
    """g = -inf (a = 0): the step forgets the state; S = beta v k^T and
    o = scale beta (k^.q^) v, against the oracle, for a mix of reset and
    ordinary lanes."""
    note("recurrent step with a hard reset")
    rng = np.random.default_rng(35)
    lay = SMALL
    n = 6
    q = I.round_bf16(rng.standard_normal((n, lay.h_qk, lay.d_k)).astype(np.float32))
    k = I.round_bf16(rng.standard_normal((n, lay.h_qk, lay.d_k)).astype(np.float32))
    v = I.round_bf16(rng.standard_normal((n, lay.h_v, lay.d_v)).astype(np.float32))
    g = (-rng.uniform(0.1, 3.0, (n, lay.h_v))).astype(np.float32)
    g[::2, 1::2] = -np.inf
    beta = (1 / (1 + np.exp(-rng.standard_normal((n, lay.h_v))))).astype(np.float32)
    state = (rng.standard_normal((n, lay.h_v, lay.d_v, lay.d_k)) * 0.02).astype(np.float32)
    sd = dev(state)
    o = torch.zeros((n, lay.h_v, lay.d_v), device=DEV)
    ops.gdn_recurrent_step(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16), dev(g),
                           dev(beta), sd, o, scale=0.5)
    torch.cuda.synchronize()
    o_ref = np.zeros((n, lay.h_v, lay.d_v))
    f_ref = np.zeros_like(state, dtype=np.float64)
    for r in range(n):
        orr, frr = R.gated_delta_rule(q[r:r + 1], k[r:r + 1], v[r:r + 1], g[r:r + 1], beta[r:r + 1], scale=0.5,
                                      initial_state=state[r:r + 1])
        o_ref[r], f_ref[r] = orr[0], frr[0]
    eo, ef = rel_max(host(o), o_ref), rel_max(host(sd), f_ref)
    note(f"  o {eo:.2e} state {ef:.2e}")
    assert eo <= TOL_BF16 and ef <= TOL_BF16
    # the reset lanes hold exactly beta v k^T in fp32 arithmetic of the kernel: no trace of the old state
    kk = k[0, 0] / np.sqrt(np.sum(k[0, 0].astype(np.float64) ** 2) + 1e-6)
    np.testing.assert_allclose(host(sd)[0, 1], beta[0, 1] * np.outer(v[0, 1], kk), rtol=0, atol=1e-6)
