"""gdn_chunk_fwd_noalloc (the entry point for callers that cannot allocate)
against gdn_chunk_fwd with a caller-owned workspace: two calls in a row, the
second on a smaller input, each bit-identical to the workspace form (the two
share their kernels); a call beyond the scratch limit is rejected and writes
nothing."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, dev, dev_i32, note
from harness import inputs as I

pytestmark = pytest.mark.gpu

LAY = I.MODEL_LAYOUT


@pytest.fixture(scope="module")
def ops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_deltanet_mixer_causal_amd import ops as _ops
    _ops.L.load()
    return _ops


def _case(seed, lengths, with_norm):
    d = I.prefill_inputs(seed, LAY, lengths, state_std=0.02)
    q, k, v = I.split_qkv(d["x"], LAY)
    T, n = int(sum(lengths)), len(lengths)
    args = dict(q=dev(q, torch.bfloat16), k=dev(k, torch.bfloat16), v=dev(v, torch.bfloat16),
                g=dev(d["g"]), beta=dev(d["beta"]), cu=dev_i32(d["cu_seqlens"]), init=dev(d["state"]),
                z=dev(d["z"], torch.bfloat16) if with_norm else None, nw=dev(d["norm_w"]) if with_norm else None)
    return args, T, n


def _both(ops, a, T, n):
    outs = []
    for noalloc in (False, True):
        o = torch.full((T, LAY.h_v, LAY.d_v), float("nan"), dtype=torch.bfloat16, device=DEV)
        fin = torch.full((n, LAY.h_v, LAY.d_v, LAY.d_k), float("nan"), device=DEV)
        kw = dict(chunk=64, cu_seqlens=a["cu"], initial_state=a["init"], final_state=fin, z=a["z"], norm_w=a["nw"])
        if noalloc:
            ops.gdn_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["g"], a["beta"], o, **kw)
        else:
            ops.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], o, **kw)
        outs.append((o, fin))
    torch.cuda.synchronize()
    return outs


def test_noalloc_matches_workspace_form_two_calls(ops):
    # first call: three packed sequences (one a single token), fused norm off
    a, T, n = _case(81, [1500, 1, 701], with_norm=False)
    note(f"noalloc call 1: T={T} n={n}")
    (o_ws, f_ws), (o_na, f_na) = _both(ops, a, T, n)
    assert torch.isfinite(o_ws.float()).all() and torch.isfinite(f_ws).all()
    assert torch.equal(o_ws, o_na) and torch.equal(f_ws, f_na)
    # second call, smaller, with the fused gated norm: the scratch keeps the
    # first call's contents, which must not matter
    a, T, n = _case(82, [150], with_norm=True)
    note(f"noalloc call 2: T={T} n={n}, fused norm")
    (o_ws, f_ws), (o_na, f_na) = _both(ops, a, T, n)
    assert torch.isfinite(o_ws.float()).all()
    assert torch.equal(o_ws, o_na) and torch.equal(f_ws, f_na)


def test_noalloc_rejects_beyond_scratch(ops):
    from gated_deltanet_mixer_causal_amd import _lib as L
    T = 65536                                      # needs more workspace than the scratch holds
    need = ops.gdn_chunk_fwd_workspace_size(LAY.h_qk, LAY.h_v, 128, 128, 64, 1, T, torch.bfloat16, False)
    assert need > L.GDN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((T, LAY.h_qk, 128), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((T, LAY.h_v, 128), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((T, LAY.h_v), device=DEV)
    o = torch.full((T, LAY.h_v, 128), 7.0, device=DEV)
    with pytest.raises(L.GdnError) as e:
        ops.gdn_chunk_fwd_noalloc(q, q, v, g, g, o, chunk=64)
    assert e.value.status == L.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
