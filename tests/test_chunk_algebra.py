"""The chunked (UT/WY) algebra the GPU kernels implement equals the
sequential oracle (invariant: chunked form == sequential recurrence)."""
import numpy as np
import pytest

from chunk_algebra import chunked_gated_delta_rule
from oracle import gdn_ref as R


def _case(rng, lengths, hqk=2, hv=4, dk=8, dv=6, strong_decay=True):
    T = int(sum(lengths))
    q = rng.standard_normal((T, hqk, dk))
    k = rng.standard_normal((T, hqk, dk))
    v = rng.standard_normal((T, hv, dv))
    if strong_decay:   # model-like: g = -exp(A) softplus(n), reaching about -50
        a = rng.uniform(0, np.log(16), hv)
        g = -np.exp(a)[None] * np.logaddexp(0, rng.standard_normal((T, hv)))
    else:
        g = -rng.uniform(0.0, 0.1, (T, hv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, hv))))
    S0 = rng.standard_normal((len(lengths), hv, dv, dk)) * 0.5
    cu = np.concatenate([[0], np.cumsum(lengths)])
    return q, k, v, g, beta, S0, cu


@pytest.mark.parametrize("chunk", [1, 4, 16, 64, 200])
@pytest.mark.parametrize("strong", [True, False])
@pytest.mark.parametrize("form", ["tx", "gr"])
def test_chunked_equals_sequential(chunk, strong, form):
    rng = np.random.default_rng(100 + chunk)
    lengths = [37, 0, 130, 1, 64]
    q, k, v, g, beta, S0, cu = _case(rng, lengths, strong_decay=strong)
    o_ref, f_ref = R.gated_delta_rule(q, k, v, g, beta, scale=0.8, initial_state=S0, cu_seqlens=cu)
    o, f = chunked_gated_delta_rule(q, k, v, g, beta, chunk=chunk, scale=0.8, initial_state=S0,
                                    cu_seqlens=cu, form=form)
    scale_o = np.sqrt(np.mean(o_ref ** 2))
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * max(1.0, scale_o)
    assert np.max(np.abs(f - f_ref)) <= 1e-12
    np.testing.assert_array_equal(f[1], S0[1])


def test_chunked_without_l2norm():
    rng = np.random.default_rng(5)
    q, k, v, g, beta, S0, cu = _case(rng, [50], strong_decay=False)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q *= 0.3
    o_ref, f_ref = R.gated_delta_rule(q, k, v, g, beta, initial_state=S0, use_qk_l2norm=False)
    o, f = chunked_gated_delta_rule(q, k, v, g, beta, chunk=16, initial_state=S0, use_qk_l2norm=False)
    assert np.max(np.abs(o - o_ref)) < 1e-12 and np.max(np.abs(f - f_ref)) < 1e-12


@pytest.mark.parametrize("form", ["tx", "gr"])
def test_split_bf16_plan_precision(form):
    """Derived operands as bf16 hi+lo pairs (raw bf16 q/k/v single) stay well
    inside the 2e-3 bound of max|err|/RMS at the model's decay statistics."""
    rng = np.random.default_rng(9)
    T, hqk, hv, d = 256, 1, 2, 128
    bf = lambda a: np.asarray(a, np.float32).astype(np.float64)
    from chunk_algebra import _bf16
    q = _bf16(np.logaddexp(0, rng.standard_normal((T, hqk, d))) * rng.standard_normal((T, hqk, d)))
    k = _bf16(np.logaddexp(0, rng.standard_normal((T, hqk, d))) * rng.standard_normal((T, hqk, d)))
    v = _bf16(rng.standard_normal((T, hv, d)))
    a = rng.uniform(0, np.log(16), hv)
    g = bf(-np.exp(a)[None] * np.logaddexp(0, rng.standard_normal((T, hv))))
    beta = bf(1 / (1 + np.exp(-rng.standard_normal((T, hv)))))
    S0 = bf(rng.standard_normal((1, hv, d, d)) * 0.02)
    o_ref, f_ref = R.gated_delta_rule(q, k, v, g, beta, initial_state=S0)
    o, f = chunked_gated_delta_rule(q, k, v, g, beta, chunk=64, initial_state=S0, plan="bf16x3", form=form)
    err_o = np.max(np.abs(o - o_ref)) / np.sqrt(np.mean(o_ref ** 2))
    err_f = np.max(np.abs(f - f_ref)) / np.sqrt(np.mean(f_ref ** 2))
    assert err_o < 5e-4 and err_f < 5e-4, (err_o, err_f)


@pytest.mark.parametrize("chunk,lengths,l2", [(1, [5], True), (4, [11, 1, 0, 9], True), (16, [40, 17], False),
                                              (64, [150, 1, 64, 70], True), (200, [37], True)])
def test_chunked_backward_equals_autograd(chunk, lengths, l2):
    """The chunk-level gradient algebra of the chunked backward kernels
    (chunk_algebra.chunked_gated_delta_rule_grads: dU, dX, the state-gradient
    recurrence, dTb, dL = -T^T dT T^T, the decay terms and the suffix sum for
    dg) against the gradient oracle's reverse-mode derivative of the
    token-by-token rule, grouped heads, an initial state and a final-state
    gradient, to 1e-11 of each tensor's largest entry."""
    from chunk_algebra import chunked_gated_delta_rule_grads
    from oracle import gdn_grad_ref as G
    rng = np.random.default_rng(7 + chunk)
    T, hqk, hv, d = sum(lengths), 2, 4, 8
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q = rng.normal(size=(T, hqk, d))
    k = rng.normal(size=(T, hqk, d))
    v = rng.normal(size=(T, hv, d))
    g = -rng.uniform(0.01, 0.6, size=(T, hv))
    beta = rng.uniform(0.05, 0.95, size=(T, hv))
    s0 = 0.3 * rng.normal(size=(len(lengths), hv, d, d))
    do = rng.normal(size=(T, hv, d))
    dfin = rng.normal(size=(len(lengths), hv, d, d))
    kw = dict(scale=0.7, initial_state=s0, cu_seqlens=cu, use_qk_l2norm=l2)
    ref = G.gated_delta_rule_grads(q, k, v, g, beta, do, dfin, **kw)
    got = chunked_gated_delta_rule_grads(q, k, v, g, beta, do, dfin, chunk=chunk, **kw)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "d_initial"):
        scale_ = max(float(np.abs(ref[key]).max()), 1e-300)
        assert float(np.abs(got[key] - ref[key]).max()) <= 1e-11 * scale_, key
