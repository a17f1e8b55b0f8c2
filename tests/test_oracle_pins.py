"""Pins of the float64 oracle against what the mathematics fixes.

Each test checks the oracle against something other than itself: hand-derived
bit patterns, closed forms, invariants of the gated delta rule, brute force
with explicit loops, or an independent formulation of the same recurrence
(the product-of-matrices form).  A plausible mistake in the oracle (a
dropped term, a wrong sign, a transposed operand, an off-by-one tap) fails at
least one of them.
"""
import math

import numpy as np
import pytest

from oracle import gdn_ref as R


# ---------------------------------------------------------------------------
# bf16 rounding
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("x,expect", [
    (1.0, 1.0),
    (1.0 + 2.0 ** -8, 1.0),                       # exact tie, 1.0 has even mantissa
    (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),       # tie between odd 1+2^-7 and even 1+2^-6
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 1.0 + 2.0 ** -7),  # just above the tie rounds up
    (-(1.0 + 2.0 ** -8), -1.0),
    (3.14159265358979, 3.140625),                 # 0x4049
    (2.0 ** -130, 2.0 ** -130),                   # bf16 subnormal, exact
    (2.0 ** -134, 0.0),                           # half the subnormal spacing, ties to 0
    (3 * 2.0 ** -134, 2.0 ** -132),               # 1.5 spacings, ties to even (2)
    (255.5, 256.0),                               # spacing 1 in [128, 256): tie to even 256
    (254.5, 254.0),
])
def test_bf16_nearest_hand_values(x, expect):
    assert R.bf16_nearest(np.float64(x)) == expect


def test_bf16_nearest_signed_zero():
    assert np.signbit(R.bf16_nearest(np.float64(-0.0)))
    assert not np.signbit(R.bf16_nearest(np.float64(0.0)))


def test_bf16_nearest_matches_bit_rounding():
    """The oracle's frexp rounding agrees with the input module's bit-pattern
    rounding (two independent implementations of round-to-nearest-even)."""
    from harness.inputs import round_bf16
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(1000)]).astype(np.float32)
    np.testing.assert_array_equal(R.bf16_nearest(a.astype(np.float64)),
                                  round_bf16(a).astype(np.float64))


# ---------------------------------------------------------------------------
# SiLU and L2 normalisation
# ---------------------------------------------------------------------------

def test_silu_closed_forms():
    assert R.silu(0.0) == 0.0
    assert math.isclose(float(R.silu(math.log(3.0))), 0.75 * math.log(3.0), rel_tol=1e-15)
    x = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(R.silu(x) - R.silu(-x), x, atol=1e-13)


def test_l2_normalize_unit_norm():
    x = np.random.default_rng(0).standard_normal((5, 7, 16))
    n = np.linalg.norm(R.l2_normalize(x, 0.0), axis=-1)
    np.testing.assert_allclose(n, 1.0, atol=1e-15)
    # eps enters as sqrt(sum x^2 + eps)
    y = R.l2_normalize(np.array([3.0, 4.0]), 11.0)
    np.testing.assert_allclose(y, [0.5, 4.0 / 6.0], rtol=1e-15)


# ---------------------------------------------------------------------------
# Causal conv1d
# ---------------------------------------------------------------------------

def _conv_brute(x, w, tail, cu):
    """Explicit loops: pre-activation y[t, c] = sum_i w[c, i] * x(t - 3 + i),
    where positions before the sequence start read the tail (oldest first)."""
    T, Ch = x.shape
    y = np.zeros((T, Ch))
    for s in range(len(cu) - 1):
        for t in range(cu[s], cu[s + 1]):
            p = t - cu[s]
            for c in range(Ch):
                acc = 0.0
                for i in range(4):
                    j = p - 3 + i
                    val = x[cu[s] + j, c] if j >= 0 else tail[s, 3 + j, c]
                    acc += w[c, i] * val
                y[t, c] = acc / (1.0 + math.exp(-acc))
    return y


def test_conv_brute_force_varlen():
    rng = np.random.default_rng(1)
    lengths = [5, 1, 0, 2, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    Ch = 6
    x = rng.standard_normal((cu[-1], Ch))
    w = rng.standard_normal((Ch, 4)) * 0.5
    tail = rng.standard_normal((len(lengths), 3, Ch))
    y, new_tail = R.causal_conv1d_silu(x, w, tail, cu, round_to_bf16=False)
    np.testing.assert_allclose(y, _conv_brute(x, w, tail, cu), rtol=1e-14, atol=1e-14)
    # new tail = last three rows of [tail; x_s]
    for s, L in enumerate(lengths):
        padded = np.concatenate([tail[s], x[cu[s]:cu[s + 1]]])
        np.testing.assert_array_equal(new_tail[s], padded[-3:])
    # a zero-length sequence keeps its tail bit-identical
    np.testing.assert_array_equal(new_tail[2], tail[2])


def test_conv_impulse_response():
    Ch, T = 3, 9
    w = np.array([[0.5, -1.0, 2.0, 0.25], [1.0, 2.0, 3.0, 4.0], [-0.5, 0.5, -0.5, 0.5]])
    x = np.zeros((T, Ch))
    x[2] = 1.0
    y, _ = R.causal_conv1d_silu(x, w, np.zeros((1, 3, Ch)), [0, T], round_to_bf16=False)
    # pre-activation at t0 + i is w[c, 3 - i]; zero elsewhere
    pre = np.zeros((T, Ch))
    for i in range(4):
        pre[2 + i] = w[:, 3 - i]
    np.testing.assert_allclose(y, pre / (1 + np.exp(-pre)), rtol=1e-15)


def test_conv_identity_taps():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 4))
    w = np.tile([0.0, 0.0, 0.0, 1.0], (4, 1))
    y, _ = R.causal_conv1d_silu(x, w, rng.standard_normal((1, 3, 4)), [0, 7], round_to_bf16=False)
    np.testing.assert_allclose(y, x / (1 + np.exp(-x)), rtol=1e-15)


def test_conv_split_equals_single():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((11, 5))
    w = rng.standard_normal((5, 4))
    tail = rng.standard_normal((1, 3, 5))
    y_all, t_all = R.causal_conv1d_silu(x, w, tail, [0, 11], round_to_bf16=False)
    y1, t1 = R.causal_conv1d_silu(x[:2], w, tail, [0, 2], round_to_bf16=False)   # shorter than 3
    y2, t2 = R.causal_conv1d_silu(x[2:6], w, t1, [0, 4], round_to_bf16=False)
    y3, t3 = R.causal_conv1d_silu(x[6:], w, t2, [0, 5], round_to_bf16=False)
    np.testing.assert_array_equal(np.concatenate([y1, y2, y3]), y_all)
    np.testing.assert_array_equal(t3, t_all)


def test_conv_bf16_boundary_rounding():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 3))
    w = rng.standard_normal((3, 4))
    y_f, _ = R.causal_conv1d_silu(x, w, np.zeros((1, 3, 3)), [0, 6], round_to_bf16=False)
    y_b, _ = R.causal_conv1d_silu(x, w, np.zeros((1, 3, 3)), [0, 6], round_to_bf16=True)
    np.testing.assert_array_equal(y_b, R.bf16_nearest(y_f))


# ---------------------------------------------------------------------------
# Gated delta rule
# ---------------------------------------------------------------------------

def _rand_case(rng, T=12, hqk=2, hv=4, dk=5, dv=3, n=1):
    q = rng.standard_normal((T, hqk, dk))
    k = rng.standard_normal((T, hqk, dk))
    v = rng.standard_normal((T, hv, dv))
    g = -rng.uniform(0.01, 0.7, (T, hv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, hv))))
    S0 = rng.standard_normal((n, hv, dv, dk)) * 0.3
    return q, k, v, g, beta, S0


def test_invariant_a_identity_when_no_decay_no_write():
    rng = np.random.default_rng(10)
    q, k, v, g, beta, S0 = _rand_case(rng)
    o, fin = R.gated_delta_rule(q, k, v, np.zeros_like(g), np.zeros_like(beta),
                                scale=0.7, initial_state=S0)
    np.testing.assert_array_equal(fin, S0)
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    for h in range(4):
        exp = 0.7 * qn[:, h // 2, :] @ S0[0, h].T
        np.testing.assert_allclose(o[:, h], exp, rtol=1e-13, atol=1e-14)


def test_invariant_b_exact_retrieval():
    """a=1, beta=1, unit keys: after each write S_t k_t = v_t; with q = k the
    output of every token is its own value."""
    rng = np.random.default_rng(11)
    T, dk, dv = 9, 6, 4
    k = rng.standard_normal((T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 1, dv))
    S0 = rng.standard_normal((1, 1, dv, dk))
    o, fin = R.gated_delta_rule(k, k, v, np.zeros((T, 1)), np.ones((T, 1)),
                                initial_state=S0, use_qk_l2norm=False)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fin[0, 0] @ k[-1, 0], v[-1, 0], atol=1e-12)


def test_orthonormal_key_table():
    """Orthonormal keys k_1..k_n, a=1, beta=1:
    S_n = S0 (I - sum k k^T) + sum v k^T and S_n k_i = v_i for every i."""
    rng = np.random.default_rng(12)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :n].T                                   # n orthonormal rows
    v = rng.standard_normal((n, 1, dv))
    S0 = rng.standard_normal((1, 1, dv, dk))
    k = keys[:, None, :]
    _, fin = R.gated_delta_rule(k, k, v, np.zeros((n, 1)), np.ones((n, 1)),
                                initial_state=S0, use_qk_l2norm=False)
    proj = keys.T @ keys
    expect = S0[0, 0] @ (np.eye(dk) - proj) + v[:, 0, :].T @ keys
    np.testing.assert_allclose(fin[0, 0], expect, atol=1e-13)
    for i in range(n):
        np.testing.assert_allclose(fin[0, 0] @ keys[i], v[i, 0], atol=1e-13)


def test_exact_integer_column_replacement():
    """One-hot keys and queries, small integers, a=1, beta in {0,1}: a write
    with key e_j replaces column j of S by v (beta=1) or leaves it (beta=0);
    the output is column q of the updated state.  Exact in float64."""
    rng = np.random.default_rng(13)
    T, dk, dv = 20, 4, 3
    kidx = rng.integers(0, dk, T)
    qidx = rng.integers(0, dk, T)
    b = rng.integers(0, 2, T).astype(float)
    v = rng.integers(-8, 9, (T, 1, dv)).astype(float)
    S0 = rng.integers(-8, 9, (1, 1, dv, dk)).astype(float)
    k = np.eye(dk)[kidx][:, None, :]
    q = np.eye(dk)[qidx][:, None, :]
    o, fin = R.gated_delta_rule(q, k, v, np.zeros((T, 1)), b[:, None],
                                scale=1.0, initial_state=S0, use_qk_l2norm=False)
    S = S0[0, 0].copy()
    for t in range(T):
        if b[t] == 1.0:
            S[:, kidx[t]] = v[t, 0]
        np.testing.assert_array_equal(o[t, 0], S[:, qidx[t]])
    np.testing.assert_array_equal(fin[0, 0], S)


def test_pure_decay_closed_form():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, S0 = _rand_case(rng)
    o, fin = R.gated_delta_rule(q, k, v, g, np.zeros_like(beta), initial_state=S0)
    decay = np.exp(np.sum(g, axis=0))
    np.testing.assert_allclose(fin[0], decay[:, None, None] * S0[0], rtol=1e-13)
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    cum = np.exp(np.cumsum(g, axis=0))
    for h in range(4):
        exp = cum[:, h:h + 1] * (qn[:, h // 2, :] @ S0[0, h].T)
        np.testing.assert_allclose(o[:, h], exp, rtol=1e-12, atol=1e-15)


def test_reset_when_alpha_zero():
    """g = -inf (a = 0): S_t = beta_t v_t k_t^T, o_t = beta_t (k_t . q_t) v_t."""
    rng = np.random.default_rng(15)
    q, k, v, g, beta, S0 = _rand_case(rng)
    o, fin = R.gated_delta_rule(q, k, v, np.full_like(g, -np.inf), beta, initial_state=S0)
    qn = q / np.sqrt(np.sum(q * q, -1, keepdims=True) + 1e-6)
    kn = k / np.sqrt(np.sum(k * k, -1, keepdims=True) + 1e-6)
    for h in range(4):
        hq = h // 2
        dots = np.sum(kn[:, hq] * qn[:, hq], axis=-1)
        np.testing.assert_allclose(o[:, h], (beta[:, h] * dots)[:, None] * v[:, h], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(fin[0, h], beta[-1, h] * np.outer(v[-1, h], kn[-1, hq]), rtol=1e-13)


def test_lms_step_is_gradient_descent():
    """a = 1: one token is S <- S - beta * grad_S (1/2 ||S k - v||^2); the
    gradient is taken by central differences (exact for a quadratic)."""
    rng = np.random.default_rng(16)
    dk, dv = 5, 4
    S = rng.standard_normal((dv, dk))
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    beta = 0.37
    loss = lambda M: 0.5 * float(np.sum((M @ k - v) ** 2))
    grad = np.zeros_like(S)
    h = 1e-3
    for i in range(dv):
        for j in range(dk):
            E = np.zeros_like(S)
            E[i, j] = h
            grad[i, j] = (loss(S + E) - loss(S - E)) / (2 * h)
    _, fin = R.gated_delta_rule(k[None, None], k[None, None], v[None, None], np.zeros((1, 1)),
                                np.full((1, 1), beta), initial_state=S[None, None],
                                use_qk_l2norm=False)
    np.testing.assert_allclose(fin[0, 0], S - beta * grad, rtol=1e-9, atol=1e-9)


def test_superposition_linear_in_state_and_values():
    rng = np.random.default_rng(17)
    q, k, v, g, beta, S0 = _rand_case(rng)
    _, _, v2, _, _, S02 = _rand_case(rng)
    a, b = 0.8, -1.3
    o1, f1 = R.gated_delta_rule(q, k, v, g, beta, initial_state=S0)
    o2, f2 = R.gated_delta_rule(q, k, v2, g, beta, initial_state=S02)
    o3, f3 = R.gated_delta_rule(q, k, a * v + b * v2, g, beta, initial_state=a * S0 + b * S02)
    np.testing.assert_allclose(o3, a * o1 + b * o2, atol=1e-12)
    np.testing.assert_allclose(f3, a * f1 + b * f2, atol=1e-12)
    o4, f4 = R.gated_delta_rule(q, k, v, g, beta, initial_state=S0, scale=2.5)
    np.testing.assert_allclose(o4, 2.5 * o1, rtol=1e-14)
    np.testing.assert_array_equal(f4, f1)


def test_product_of_matrices_form():
    """Independent formulation: with M_t = a_t (I - beta_t k_t k_t^T),
    S_t = S0 M_1 ... M_t + sum_{u<=t} beta_u v_u k_u^T M_{u+1} ... M_t,
    built from explicit products (no recursion on S)."""
    rng = np.random.default_rng(18)
    T, dk, dv = 7, 4, 3
    q = rng.standard_normal((T, 1, dk))
    k = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = -rng.uniform(0.0, 1.0, (T, 1))
    beta = rng.uniform(0.0, 1.0, (T, 1))
    S0 = rng.standard_normal((1, 1, dv, dk))
    o, fin = R.gated_delta_rule(q, k, v, g, beta, scale=1.3, initial_state=S0)
    kn = k[:, 0] / np.sqrt(np.sum(k[:, 0] ** 2, -1, keepdims=True) + 1e-6)
    qn = q[:, 0] / np.sqrt(np.sum(q[:, 0] ** 2, -1, keepdims=True) + 1e-6)
    M = [np.exp(g[t, 0]) * (np.eye(dk) - beta[t, 0] * np.outer(kn[t], kn[t])) for t in range(T)]

    def prod(lo, hi):  # M_lo ... M_hi (inclusive), identity if empty
        P = np.eye(dk)
        for t in range(lo, hi + 1):
            P = P @ M[t]
        return P

    for t in range(T):
        St = S0[0, 0] @ prod(0, t)
        for u in range(t + 1):
            St = St + beta[u, 0] * np.outer(v[u, 0], kn[u]) @ prod(u + 1, t)
        np.testing.assert_allclose(o[t, 0], 1.3 * St @ qn[t], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fin[0, 0], St, rtol=1e-12, atol=1e-13)


def test_head_grouping_contiguous():
    """v-head h reads q/k head h // G: each v-head equals a single-head run on
    its own q/k head."""
    rng = np.random.default_rng(19)
    q, k, v, g, beta, S0 = _rand_case(rng, hqk=2, hv=4)
    o, fin = R.gated_delta_rule(q, k, v, g, beta, initial_state=S0)
    for h in range(4):
        hq = h // 2
        o1, f1 = R.gated_delta_rule(q[:, hq:hq + 1], k[:, hq:hq + 1], v[:, h:h + 1], g[:, h:h + 1],
                                    beta[:, h:h + 1], initial_state=S0[:, h:h + 1])
        np.testing.assert_array_equal(o[:, h], o1[:, 0])
        np.testing.assert_array_equal(fin[:, h], f1[:, 0])


def test_varlen_packing_equals_separate_runs():
    rng = np.random.default_rng(20)
    lengths = [3, 0, 7, 1]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    q, k, v, g, beta, _ = _rand_case(rng, T=int(cu[-1]))
    S0 = rng.standard_normal((4, 4, 3, 5))
    o, fin = R.gated_delta_rule(q, k, v, g, beta, initial_state=S0, cu_seqlens=cu)
    for s in range(4):
        sl = slice(cu[s], cu[s + 1])
        o1, f1 = R.gated_delta_rule(q[sl], k[sl], v[sl], g[sl], beta[sl], initial_state=S0[s:s + 1])
        np.testing.assert_array_equal(o[sl], o1)
        np.testing.assert_array_equal(fin[s], f1[0])
    np.testing.assert_array_equal(fin[1], S0[1])        # zero-length sequence


# ---------------------------------------------------------------------------
# Gated RMSNorm
# ---------------------------------------------------------------------------

def test_gated_rmsnorm_closed_forms():
    rng = np.random.default_rng(21)
    o = rng.standard_normal((4, 3, 8))
    w = 1 + 0.1 * rng.standard_normal(8)
    np.testing.assert_array_equal(R.gated_rmsnorm(o, np.zeros_like(o), w, 1e-6), 0.0)
    for c in (-3.0, 0.01, 2.0):
        z = rng.standard_normal(8)
        y = R.gated_rmsnorm(np.full(8, c), z, w, 1e-6)
        expect = np.sign(c) / math.sqrt(1 + 1e-6 / c ** 2) * w * (z / (1 + np.exp(-z)))
        np.testing.assert_allclose(y, expect, rtol=1e-14)
    # with unit weight and SiLU(z) == 1 impossible, check RMS of the normalised part
    big = R.gated_rmsnorm(o * 100, np.full_like(o, 40.0), np.ones(8), 1e-6)  # SiLU(40) = 40 (1 - 4e-18)
    rms = np.sqrt(np.mean((big / 40.0) ** 2, axis=-1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-9)


# ---------------------------------------------------------------------------
# Decode step vs prefill (the same definition reached by two call routes)
# ---------------------------------------------------------------------------

def test_decode_steps_equal_prefill_and_inactive_lanes():
    rng = np.random.default_rng(22)
    hqk, hv, dk, dv, T = 1, 2, 4, 4, 5
    ch = 2 * hqk * dk + hv * dv
    x = rng.standard_normal((T, ch))
    w = rng.standard_normal((ch, 4))
    tail = rng.standard_normal((1, 3, ch))
    S0 = rng.standard_normal((1, hv, dv, dk)) * 0.1
    g = -rng.uniform(0, 1, (T, hv))
    beta = rng.uniform(0, 1, (T, hv))
    z = rng.standard_normal((T, hv, dv))
    nw = 1 + 0.1 * rng.standard_normal(dv)
    kw = dict(h_qk=hqk, h_v=hv, d_k=dk, d_v=dv, bf16_boundary=False)
    ref = R.mixer_prefill(x, w, tail, S0, beta, g, z, nw, [0, T], **kw)
    # decode: slot 1 holds the request, slots 0 and 2 are bystanders
    tails = np.stack([np.full((3, ch), 7.0), tail[0], np.full((3, ch), 9.0)])
    states = np.stack([np.full((hv, dv, dk), 5.0), S0[0], np.full((hv, dv, dk), 6.0)])
    for t in range(T):
        xs = np.stack([x[t], x[t]])
        out = R.mixer_decode_step(xs, w, tails, states, np.stack([beta[t]] * 2), np.stack([g[t]] * 2),
                                  np.stack([z[t]] * 2), nw, [1, -1], **kw)
        np.testing.assert_allclose(out["o"][0], ref["o"][t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(out["y"][0], ref["y"][t], rtol=1e-12, atol=1e-14)
        assert np.all(np.isnan(out["o"][1]))
    np.testing.assert_allclose(states[1], ref["state"][0], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(tails[1], ref["tail"][0])
    assert np.all(tails[0] == 7.0) and np.all(tails[2] == 9.0)
    assert np.all(states[0] == 5.0) and np.all(states[2] == 6.0)


# ---------------------------------------------------------------------------
# Gate preparation from the raw gate projections
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("x,expect", [
    (0.0, math.log(2.0)),               # ln(1 + 1)
    (math.log(3.0), 2.0 * math.log(2.0)),   # ln(1 + 3) = ln 4
    (-math.log(3.0), math.log(4.0 / 3.0)),  # ln(1 + 1/3)
    (50.0, 50.0 + math.exp(-50.0)),      # far right: x + e^-x to first order
    (-50.0, math.exp(-50.0)),            # far left: e^x to first order
    (-800.0, 0.0),                       # e^-800 underflows to 0 without overflow on the way
    (800.0, 800.0),
])
def test_softplus_closed_forms(x, expect):
    assert R.softplus(np.float64(x)) == pytest.approx(expect, rel=1e-15, abs=1e-300)


def test_softplus_odd_part_and_slope():
    # softplus(x) - softplus(-x) = x for every x, and its slope is the sigmoid
    x = np.linspace(-30.0, 30.0, 601)
    np.testing.assert_allclose(R.softplus(x) - R.softplus(-x), x, rtol=0, atol=1e-13)
    h = 1e-5
    slope = (R.softplus(x + h) - R.softplus(x - h)) / (2 * h)
    np.testing.assert_allclose(slope, 1.0 / (1.0 + np.exp(-x)), rtol=0, atol=1e-9)


@pytest.mark.parametrize("x,expect", [
    (0.0, 0.5), (math.log(3.0), 0.75), (-math.log(3.0), 0.25), (-800.0, 0.0), (800.0, 1.0),
])
def test_sigmoid_closed_forms(x, expect):
    assert R.sigmoid(np.float64(x)) == pytest.approx(expect, rel=1e-15, abs=1e-300)


def test_sigmoid_symmetry():
    x = np.linspace(-40.0, 40.0, 801)
    np.testing.assert_allclose(R.sigmoid(x) + R.sigmoid(-x), 1.0, rtol=0, atol=1e-15)


def test_gates_closed_forms_and_head_indexing():
    # a = ln 3 gives softplus = ln 4 exactly; a_log = ln 2 doubles it; b = ln 3 gives beta = 3/4
    t, hv = 5, 3
    a = np.full((t, hv), math.log(3.0))
    b = np.full((t, hv), math.log(3.0))
    a_log = np.array([0.0, math.log(2.0), math.log(0.5)])
    g, beta = R.gates_from_projections(a, b, a_log)
    for h, mult in enumerate([1.0, 2.0, 0.5]):
        np.testing.assert_allclose(g[:, h], -mult * math.log(4.0), rtol=1e-15)
    np.testing.assert_allclose(beta, 0.75, rtol=1e-15)
    assert np.all(g < 0)


def test_gates_bias_is_a_shift_of_a():
    rng = np.random.default_rng(5)
    a = rng.standard_normal((7, 4))
    b = rng.standard_normal((7, 4))
    a_log = rng.uniform(0, math.log(16.0), 4)
    bias = rng.standard_normal(4)
    g1, b1 = R.gates_from_projections(a, b, a_log, bias)
    g2, b2 = R.gates_from_projections(a + bias[None, :], b, a_log)
    np.testing.assert_allclose(g1, g2, rtol=1e-15)
    np.testing.assert_array_equal(b1, b2)
    # beta ignores a, a_log and the bias; g ignores b
    g3, b3 = R.gates_from_projections(a, -b, a_log, bias)
    np.testing.assert_array_equal(g3, g1)
    np.testing.assert_allclose(b3, 1.0 - b1, rtol=0, atol=1e-15)


def test_gates_match_log_decay_recipe():
    # g = -exp(A) softplus(n): the decay becomes exp(g) = (1 + e^n)^(-exp(A)),
    # a product form computed here without the oracle's functions
    rng = np.random.default_rng(6)
    n = rng.standard_normal((9, 2))
    A = rng.uniform(0, math.log(16.0), 2)
    g, _ = R.gates_from_projections(n, np.zeros_like(n), A)
    np.testing.assert_allclose(np.exp(g), (1.0 + np.exp(n)) ** (-np.exp(A)[None, :]), rtol=1e-13)


# ---------------------------------------------------------------------------
# Speculative verification: checkpoint columns and conv windows
# ---------------------------------------------------------------------------

def test_verify_checkpoints_match_prefix_runs():
    # column t equals the final state of the pinned rule over tokens 0..t, and
    # the outputs equal those of one run over all W tokens
    rng = np.random.default_rng(11)
    w, hqk, hv, d = 5, 1, 2, 8
    q = rng.standard_normal((w, hqk, d))
    k = rng.standard_normal((w, hqk, d))
    v = rng.standard_normal((w, hv, d))
    g = -rng.uniform(0.05, 0.5, (w, hv))
    beta = rng.uniform(0.1, 0.9, (w, hv))
    s0 = 0.1 * rng.standard_normal((hv, d, d))
    o, cols = R.verify_checkpoints(q, k, v, g, beta, initial_state=s0)
    o_all, _ = R.gated_delta_rule(q, k, v, g, beta, initial_state=s0[None])
    np.testing.assert_allclose(o, o_all, rtol=0, atol=1e-13)
    for t in range(w):
        _, fin = R.gated_delta_rule(q[:t + 1], k[:t + 1], v[:t + 1], g[:t + 1], beta[:t + 1],
                                    initial_state=s0[None])
        np.testing.assert_allclose(cols[t], fin[0], rtol=0, atol=1e-13)


def test_verify_checkpoint_exact_write():
    # a = 1, beta = 1, unit-norm key: every column retrieves its own value, S_t k_t = v_t
    d, hv = 8, 1
    eye = np.eye(d)
    q = eye[[0, 1, 2]][:, None, :]
    k = eye[[3, 4, 3]][:, None, :]
    v = np.arange(3 * d, dtype=np.float64).reshape(3, hv, d)
    g = np.zeros((3, hv))
    beta = np.ones((3, hv))
    _, cols = R.verify_checkpoints(q, k, v, g, beta, initial_state=np.zeros((hv, d, d)), use_qk_l2norm=False)
    for t in range(3):
        np.testing.assert_allclose(cols[t][0] @ k[t, 0], v[t, 0], rtol=0, atol=1e-12)
    # the third token overwrote key 3: column 2 no longer returns token 0's value for it
    np.testing.assert_allclose(cols[2][0] @ eye[4], v[1, 0], rtol=0, atol=1e-12)


def test_conv_windows_equal_conv_tail():
    # the last window is the history the conv reports after all W tokens; every
    # window is made of raw inputs in token order
    rng = np.random.default_rng(12)
    ch, w = 16, 4
    tail = rng.standard_normal((1, 3, ch))
    x = rng.standard_normal((w, ch))
    win = R.conv_windows(tail[0], x)
    _, new_tail = R.causal_conv1d_silu(x, rng.standard_normal((ch, 4)), tail, [0, w], round_to_bf16=False)
    np.testing.assert_array_equal(win[-1], new_tail[0])
    np.testing.assert_array_equal(win[0], np.concatenate([tail[0][1:], x[:1]]))
    for t in range(1, w):
        np.testing.assert_array_equal(win[t][:2], win[t - 1][1:])
        np.testing.assert_array_equal(win[t][2], x[t])


# ---------------------------------------------------------------------------
# Mixed prefill-plus-decode batches over state pools
# ---------------------------------------------------------------------------

def _mixed_case(seed, lengths, t_pad=3):
    rng = np.random.default_rng(seed)
    hqk, hv, dk, dv = 1, 2, 4, 4
    ch = 2 * hqk * dk + hv * dv
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(cu[-1]) + t_pad
    d = dict(x=rng.standard_normal((T, ch)), w=rng.standard_normal((ch, 4)),
             g=-rng.uniform(0, 1, (T, hv)), beta=rng.uniform(0, 1, (T, hv)),
             z=rng.standard_normal((T, hv, dv)), nw=1 + 0.1 * rng.standard_normal(dv), cu=cu)
    n_slots = len(lengths) + 3
    d["tails"] = rng.standard_normal((n_slots, 3, ch))
    d["states"] = 0.1 * rng.standard_normal((n_slots, hv, dv, dk))
    d["kw"] = dict(h_qk=hqk, h_v=hv, d_k=dk, d_v=dv, bf16_boundary=False)
    return d


def _run_mixed(d, slots, fresh, tails=None, states=None):
    tails = d["tails"].copy() if tails is None else tails
    states = d["states"].copy() if states is None else states
    out = R.mixer_mixed(d["x"], d["w"], tails, states, slots, fresh, d["beta"], d["g"], d["z"], d["nw"],
                        d["cu"], **d["kw"])
    return out, tails, states


def test_mixed_identity_slots_equal_packed_prefill():
    d = _mixed_case(31, [5, 1, 7, 1], t_pad=0)
    n = len(d["cu"]) - 1
    out, tails, states = _run_mixed(d, list(range(n)), None)
    ref = R.mixer_prefill(d["x"], d["w"], d["tails"][:n], d["states"][:n], d["beta"], d["g"], d["z"], d["nw"],
                          d["cu"], **d["kw"])
    np.testing.assert_array_equal(out["y"], ref["y"])
    np.testing.assert_array_equal(states[:n], ref["state"])
    np.testing.assert_array_equal(tails[:n], ref["tail"])
    np.testing.assert_array_equal(states[n:], d["states"][n:])   # slots no sequence names


def test_mixed_decode_tokens_equal_decode_step():
    # sequences of length 1 are decode tokens: equal to the decode step on those requests
    d = _mixed_case(32, [1, 1, 1], t_pad=2)
    slots = [4, 0, 2]
    out, tails, states = _run_mixed(d, slots, None)
    tails2, states2 = d["tails"].copy(), d["states"].copy()
    ref = R.mixer_decode_step(d["x"][:3], d["w"], tails2, states2, d["beta"][:3], d["g"][:3], d["z"][:3],
                              d["nw"], slots, **d["kw"])
    np.testing.assert_allclose(out["y"][:3], ref["y"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(states, states2, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(tails, tails2)
    assert np.all(np.isnan(out["y"][3:]))                          # padding rows are not written


def test_mixed_fresh_reads_nothing_inactive_writes_nothing():
    d = _mixed_case(33, [6, 1, 4, 0], t_pad=4)
    slots = [1, 3, -1, 0]
    fresh = [1, 0, 0, 1]
    tails, states = d["tails"].copy(), d["states"].copy()
    tails[1] = np.nan
    states[1] = np.nan          # a fresh slot's old contents must not be read
    out, tails, states = _run_mixed(d, slots, fresh, tails, states)
    # sequence 0 from zero history and state
    a, b = d["cu"][0], d["cu"][1]
    ref = R.mixer_prefill(d["x"][a:b], d["w"], np.zeros((1, 3, d["x"].shape[1])),
                          np.zeros((1,) + d["states"].shape[1:]), d["beta"][a:b], d["g"][a:b], d["z"][a:b],
                          d["nw"], [0, b - a], **d["kw"])
    np.testing.assert_array_equal(out["y"][a:b], ref["y"])
    np.testing.assert_array_equal(states[1], ref["state"][0])
    np.testing.assert_array_equal(tails[1], ref["tail"][0])
    # inactive sequence 2: rows unwritten; slots 2 and 4 (named by no active sequence) untouched
    a, b = d["cu"][2], d["cu"][3]
    assert np.all(np.isnan(out["y"][a:b])) and np.all(np.isnan(out["y"][d["cu"][-1]:]))
    for p in (2, 4, 5, 6):
        np.testing.assert_array_equal(states[p], d["states"][p])
        np.testing.assert_array_equal(tails[p], d["tails"][p])
    # fresh zero-length sequence 3: its slot becomes the zero state and history
    assert np.all(states[0] == 0.0) and np.all(tails[0] == 0.0)


def test_mixed_slot_permutation_and_continuation():
    d = _mixed_case(34, [9, 1, 5], t_pad=0)
    out, tails, states = _run_mixed(d, [0, 1, 2], None)
    perm = [3, 0, 5]
    tails_p, states_p = d["tails"].copy(), d["states"].copy()
    tails_p[perm] = d["tails"][[0, 1, 2]]
    states_p[perm] = d["states"][[0, 1, 2]]
    out_p, tails_p, states_p = _run_mixed(d, perm, None, tails_p, states_p)
    np.testing.assert_array_equal(out_p["y"], out["y"])
    np.testing.assert_array_equal(states_p[perm], states[[0, 1, 2]])
    np.testing.assert_array_equal(tails_p[perm], tails[[0, 1, 2]])
    # a prompt split over two batches continues through its pool row exactly
    d1 = dict(d)
    cut = 4
    d1["cu"] = np.array([0, cut]); d1["x"] = d["x"][:cut]; d1["g"] = d["g"][:cut]
    d1["beta"] = d["beta"][:cut]; d1["z"] = d["z"][:cut]
    o1, t1, s1 = _run_mixed(d1, [0], None)
    d2 = dict(d)
    d2["cu"] = np.array([0, 9 - cut]); d2["x"] = d["x"][cut:9]; d2["g"] = d["g"][cut:9]
    d2["beta"] = d["beta"][cut:9]; d2["z"] = d["z"][cut:9]
    o2, t2, s2 = _run_mixed(d2, [0], None, t1, s1)
    np.testing.assert_array_equal(np.concatenate([o1["y"], o2["y"]]), out["y"][:9])
    np.testing.assert_array_equal(s2[0], states[0])
    np.testing.assert_array_equal(t2[0], tails[0])


# ---------------------------------------------------------------------------
# The whole mixer's channel split and head map, fixed by hand
# ---------------------------------------------------------------------------

def test_mixer_channel_split_and_head_map_by_hand():
    """mixer_prefill's split of the conv output into q | k | v blocks and its
    v-head -> q/k-head map, checked without split_heads.

    With identity conv taps (tap 3 = 1), zero history, alpha = 1, beta = 1,
    l2_eps = 0 and one-hot q and k rows, every token overwrites one column of
    each v-head's state with that head's v row, and o reads one column:
        S_h[:, ik(t, h // 2)] <- v_t,h    then    o_t,h = S_h[:, iq(t, h // 2)].
    (x / sqrt(x^2) == 1 exactly in binary floating point, so the one-hot rows
    stay one-hot through the L2 norm.)  The expected values are read from the
    conv output at channel offsets written out here: q head j component i at
    channel j*dk + i, k head j at Hqk*dk + j*dk + i, v head h component i at
    2*Hqk*dk + h*dv + i.  Swapping the q and k blocks, misplacing v, swapping
    d_k and d_v in a reshape or a different head grouping fails this test.
    """
    rng = np.random.default_rng(31)
    hqk, hv, dk, dv, T = 2, 4, 4, 3, 9
    ch = 2 * hqk * dk + hv * dv
    iq = rng.integers(0, dk, (T, hqk))
    ik = rng.integers(0, dk, (T, hqk))
    x = np.zeros((T, ch))
    for t in range(T):
        for j in range(hqk):
            x[t, j * dk + iq[t, j]] = 1.5 + j                    # q head j: one-hot
            x[t, hqk * dk + j * dk + ik[t, j]] = 2.5 + j         # k head j: one-hot
    x[:, 2 * hqk * dk:] = rng.standard_normal((T, hv * dv))     # v: dense, distinct
    w = np.tile([0.0, 0.0, 0.0, 1.0], (ch, 1))
    tail = np.zeros((1, 3, ch))
    S0 = rng.standard_normal((1, hv, dv, dk))
    g = np.zeros((T, hv))
    beta = np.ones((T, hv))
    z = rng.standard_normal((T, hv, dv))
    nw = 1 + 0.1 * rng.standard_normal(dv)
    out = R.mixer_prefill(x, w, tail, S0, beta, g, z, nw, [0, T], h_qk=hqk, h_v=hv, d_k=dk, d_v=dv,
                          bf16_boundary=False, l2_eps=0.0)
    yc = out["y_conv"]
    S = S0[0].copy()
    o_exp = np.zeros((T, hv, dv))
    for t in range(T):
        for h in range(hv):
            j = h // (hv // hqk)
            v_row = yc[t, 2 * hqk * dk + h * dv: 2 * hqk * dk + (h + 1) * dv]
            S[h][:, ik[t, j]] = v_row
            o_exp[t, h] = S[h][:, iq[t, j]]
    np.testing.assert_allclose(out["o"], o_exp, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out["state"][0], S, rtol=0, atol=1e-14)
    # the gate of the norm is read per (token, v-head) in the same order
    np.testing.assert_allclose(out["y"], R.gated_rmsnorm(o_exp, z, nw, 1e-6), rtol=1e-14, atol=1e-15)
    # and the hand-built q, k rows really are one-hot after the conv and SiLU
    assert np.count_nonzero(yc[:, :2 * hqk * dk]) == 2 * hqk * T
