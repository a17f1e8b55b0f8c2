"""Pins of the gradient oracle (oracle/gdn_grad_ref.py) on the CPU.

Every gradient is checked against central finite differences of the forward
of oracle/gdn_ref.py (a separate implementation, NumPy rather than torch),
along random directions for every input, and against closed forms where
the rule has one (no writes: the state only decays).
"""
import numpy as np
import pytest

from oracle import gdn_grad_ref as G
from oracle import gdn_ref as R


def _case(seed, lengths, hqk=1, hv=2, d=4):
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    n = len(lengths)
    return dict(q=rng.standard_normal((T, hqk, d)), k=rng.standard_normal((T, hqk, d)),
                v=rng.standard_normal((T, hv, d)), g=-rng.uniform(0.05, 0.8, (T, hv)),
                beta=rng.uniform(0.1, 0.9, (T, hv)), s0=0.3 * rng.standard_normal((n, hv, d, d)),
                do=rng.standard_normal((T, hv, d)), dfin=rng.standard_normal((n, hv, d, d)),
                cu=np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64))


def _loss(c, kw, **over):
    a = {name: c[name] for name in ("q", "k", "v", "g", "beta", "s0")}
    a.update(over)
    o, fin = R.gated_delta_rule(a["q"], a["k"], a["v"], a["g"], a["beta"], initial_state=a["s0"],
                                cu_seqlens=c["cu"], **kw)
    return float(np.sum(o * c["do"]) + np.sum(fin * c["dfin"]))


@pytest.mark.parametrize("use_l2,scale", [(True, 1.0), (False, 0.7)])
def test_rule_grads_match_finite_differences(use_l2, scale):
    c = _case(40, [5, 1, 3])
    kw = dict(scale=scale, use_qk_l2norm=use_l2)
    gr = G.gated_delta_rule_grads(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], c["dfin"],
                                  initial_state=c["s0"], cu_seqlens=c["cu"], **kw)
    # the torch forward is the NumPy oracle's forward
    o, fin = R.gated_delta_rule(c["q"], c["k"], c["v"], c["g"], c["beta"], initial_state=c["s0"],
                                cu_seqlens=c["cu"], **kw)
    np.testing.assert_allclose(gr["o"], o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(gr["final"], fin, rtol=1e-12, atol=1e-13)
    rng = np.random.default_rng(41)
    eps = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"),
                        ("s0", "d_initial")):
        for _ in range(2):
            dirn = rng.standard_normal(c[name].shape)
            fd = (_loss(c, kw, **{name: c[name] + eps * dirn}) - _loss(c, kw, **{name: c[name] - eps * dirn})) / (2 * eps)
            an = float(np.sum(gr[gname] * dirn))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_rule_grads_without_writes_closed_form():
    # beta = 0: S_t = c_t S0 with c_t = exp(sum_{s<=t} g_s), o_t = scale c_t S0 q_t
    c = _case(42, [6], hqk=2, hv=2)
    c["beta"] = np.zeros_like(c["beta"])
    scale = 0.5
    gr = G.gated_delta_rule_grads(c["q"], c["k"], c["v"], c["g"], c["beta"], c["do"], c["dfin"],
                                  initial_state=c["s0"], cu_seqlens=c["cu"], scale=scale, use_qk_l2norm=False)
    T = c["q"].shape[0]
    cum = np.exp(np.cumsum(c["g"], axis=0))                     # [T, Hv]
    S0 = c["s0"][0]
    d_init = cum[-1][:, None, None] * c["dfin"][0]
    term = np.zeros((T, 2))                                     # scale c_t do_t^T S0 q_t per head
    for t in range(T):
        d_init += scale * cum[t][:, None, None] * c["do"][t][:, :, None] * c["q"][t][:, None, :]
        term[t] = scale * cum[t] * np.einsum("hi,hij,hj->h", c["do"][t], S0, c["q"][t])
    np.testing.assert_allclose(gr["d_initial"][0], d_init, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(gr["dv"], 0.0, atol=0)
    # dg_s = sum_{t >= s} scale c_t do_t^T S0 q_t + c_T <d_final, S0>
    fin_term = cum[-1] * np.sum(c["dfin"][0] * S0, axis=(1, 2))
    dg = np.array([term[s:].sum(axis=0) for s in range(T)]) + fin_term[None]
    np.testing.assert_allclose(gr["dg"], dg, rtol=1e-11, atol=1e-12)


def test_conv_grads_match_finite_differences():
    rng = np.random.default_rng(43)
    lengths = [4, 1, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T, ch, n = int(cu[-1]), 8, len(lengths)
    x, w, tail = rng.standard_normal((T, ch)), rng.standard_normal((ch, 4)), rng.standard_normal((n, 3, ch))
    dy, dt = rng.standard_normal((T, ch)), rng.standard_normal((n, 3, ch))
    gr = G.causal_conv1d_silu_grads(x, w, tail, cu, dy, dt)

    def loss(x_, w_, t_):
        y, to = R.causal_conv1d_silu(x_, w_, t_, cu, round_to_bf16=False)
        return float(np.sum(y * dy) + np.sum(to * dt))

    np.testing.assert_allclose(gr["y"], R.causal_conv1d_silu(x, w, tail, cu, round_to_bf16=False)[0], rtol=1e-13)
    eps = 1e-6
    for which, gname in ((0, "dx"), (1, "dw"), (2, "d_tail")):
        base = [x, w, tail]
        for _ in range(2):
            dirn = rng.standard_normal(base[which].shape)
            plus, minus = list(base), list(base)
            plus[which] = base[which] + eps * dirn
            minus[which] = base[which] - eps * dirn
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            an = float(np.sum(gr[gname] * dirn))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (gname, fd, an)
