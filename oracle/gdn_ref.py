"""Float64 CPU oracle for the Gated DeltaNet mixer (test infrastructure).

This is test infrastructure, not part of the library: only the test suite,
the package smoke check and the benchmark's CPU-baseline leg may import or
run it.  It shares no code with the HIP path.  It is plain, slow and
written to be checked by eye: every step is token by token, in float64,
following the definition of each operation.

What it computes (sources):
  * The mixer: a width-4 causal conv1d with SiLU, the gated delta rule and a
    gated RMSNorm, in 48 of the 64 layers of the hybrid model
    (haskell-infer-demo README, "Highlights", hybrid architecture bullet;
    "Architecture", kernels gdn_conv.cu / fla_gdn.cu / gdn_norm.cu).
  * The conv runs over the raw projected q|k|v channels with dilation 1,
    SiLU, and an explicit history of raw inputs; the history of a sequence
    is its last three inputs (Flare core-design, short-convolution paragraph
    and the prepared-interface list under it; the speculative snapshot
    paragraph, which keeps a three-token conv window per position).
  * The gated delta rule: S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T
    and o_t = S_t q_t, with a_t = exp(g_t), applied token by token with an
    fp32 recurrent state on the device (Flare core-design, Qwen defaults
    table, the row giving bf16 main KV and fp32 GDN recurrence; the GDN
    chunking paragraph on bf16 intermediates and an fp32 state).
  * A prefill call ends with the state after exactly the consumed tokens
    (Flare core-design, the paragraph on exact consumed endpoints, which are
    never rounded up to a token group).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):
  * q/k scale defaults to 1; L2 norm is x / sqrt(sum x^2 + eps) after SiLU.
  * v-head h reads q/k head h // (Hv / Hqk) (contiguous groups).
  * conv: no bias; w[c, 3] multiplies the current token, w[c, 0] the token
    three back; history is raw pre-activation input, oldest first; a
    sequence never sees its neighbours in a packed buffer.
  * gated RMSNorm per (token, v-head) over d_v: o / sqrt(mean(o^2) + eps) * w
    * SiLU(z), with a plain weight w.
  * For bf16 workloads the conv output is a bf16 tensor at the library
    boundary, so the oracle rounds SiLU(conv) to bf16 (nearest, ties to even)
    before the recurrence reads it; everything else stays float64.
  * Gate preparation from the raw gate projections (the B/A projection pair
    the pages give the GDN mixer: Flare core-design, the paragraph on fused
    projection weights): g = -exp(A_log[h]) softplus(a[t,h] + dt_bias[h])
    and beta = sigmoid(b[t,h]).  The pages print neither formula; this is the
    plainest reading that fits the log-decay g < 0 of the rule above and a
    write strength beta in (0, 1).  dt_bias is an optional per-head bias
    (absent = 0).
  * Speculative verification: a round of W draft tokens starts from the live
    state and records the state after each token in its own checkpoint column,
    and the 3-token conv history after each token (Flare core-design,
    speculative target state: eight recurrent checkpoint columns per request, a
    round writes the columns of its verification inputs, and a snapshot copies a
    column with its three-token convolution window).

  * Mixed prefill-plus-decode batches over state pools (the prepared
    interface list under the short-convolution paragraph of Flare
    core-design): the host knows capacities only; a padded sequence has
    length 0 and slot -1; a fresh sequence starts from zero history and
    state without reading its pool row.

Parity status: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (closed forms, invariants, brute force, an
independent product-of-matrices form of the recurrence, and a chunked
evaluation that must agree to 1e-12).
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Elementwise pieces
# ---------------------------------------------------------------------------

def bf16_nearest(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits (1 implicit + 7 stored).  Written with
    frexp/ldexp arithmetic rather than bit patterns: x = m * 2^e with
    0.5 <= |m| < 1, so the bf16 grid spacing near x is 2^(e-8).  Values in
    the subnormal range use the fixed spacing 2^-133.  Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)                 # below 2^-126 the spacing stops shrinking
    step = np.ldexp(1.0, e - 8)
    return np.round(x / step) * step        # np.round is round-half-to-even


def silu(x):
    """SiLU(x) = x * sigmoid(x) = x / (1 + e^-x)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def l2_normalize(x, eps: float):
    """x / sqrt(sum(x^2) + eps) over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x):
    """softplus(x) = ln(1 + e^x), written as max(x, 0) + ln(1 + e^-|x|) so that
    no exponential overflows (the two forms are equal for every real x)."""
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """sigmoid(x) = 1 / (1 + e^-x), evaluated through e^-|x| so that no
    exponential overflows."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


# ---------------------------------------------------------------------------
# Gate preparation
# ---------------------------------------------------------------------------

def gates_from_projections(a, b, a_log, dt_bias=None):
    """Log-decay g and write strength beta from the raw gate projections.

    a, b [T, Hv] are the outputs of the A and B gate projections (Flare
    core-design, fused projection weights paragraph); a_log and dt_bias are
    per-v-head parameters [Hv].  For every token t and v-head h:
        g[t, h]    = -exp(a_log[h]) * softplus(a[t, h] + dt_bias[h])
        beta[t, h] = sigmoid(b[t, h])
    dt_bias None means a zero bias.  Returns (g, beta) as float64 [T, Hv].
    """
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    a_log = np.asarray(a_log, np.float64)
    t, hv = a.shape
    g = np.empty((t, hv))
    beta = np.empty((t, hv))
    for h in range(hv):
        bias = 0.0 if dt_bias is None else float(np.asarray(dt_bias, np.float64)[h])
        g[:, h] = -math.exp(a_log[h]) * softplus(a[:, h] + bias)
        beta[:, h] = sigmoid(b[:, h])
    return g, beta


# ---------------------------------------------------------------------------
# Causal conv1d + SiLU
# ---------------------------------------------------------------------------

def causal_conv1d_silu(x, w, tail, cu_seqlens, *, round_to_bf16: bool,
                       active=None):
    """Width-4 depthwise causal conv per packed sequence, then SiLU.

    x [T, Ch], w [Ch, 4], tail [N, 3, Ch] (oldest first), cu_seqlens [N+1].
    For sequence s with tokens x_s, the padded input is [tail[s]; x_s] and
    output token t of the sequence is SiLU(sum_i w[:, i] * padded[t + i]).
    Returns (y [T, Ch] float64, new_tail [N, 3, Ch]) where new_tail[s] is the
    last three rows of the padded input.  `active` (bool [N]) marks sequences
    that run; an inactive sequence leaves its y rows as NaN (they are not
    written) and its tail unchanged.
    """
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    tail = np.asarray(tail, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    n = len(cu) - 1
    y = np.full(x.shape, np.nan)
    new_tail = tail.copy()
    for s in range(n):
        if active is not None and not active[s]:
            continue
        xs = x[cu[s]:cu[s + 1]]
        padded = np.concatenate([tail[s], xs], axis=0)      # [3 + L, Ch]
        length = xs.shape[0]
        acc = np.zeros((length, x.shape[1]))
        for i in range(4):                                   # tap i reads token t - 3 + i
            acc += w[:, i][None, :] * padded[i:i + length]
        out = silu(acc)
        if round_to_bf16:
            out = bf16_nearest(out)
        y[cu[s]:cu[s + 1]] = out
        new_tail[s] = padded[-3:]
    return y, new_tail


# ---------------------------------------------------------------------------
# Gated delta rule, token by token
# ---------------------------------------------------------------------------

def gated_delta_rule(q, k, v, g, beta, *, scale=1.0, initial_state=None,
                     cu_seqlens=None, use_qk_l2norm=True, l2_eps=1e-6,
                     qk_of_v=None):
    """Sequential gated delta rule over packed sequences.

    q, k [T, Hqk, dk]; v [T, Hv, dv]; g, beta [T, Hv]; initial_state
    [N, Hv, dv, dk] (None = zeros); cu_seqlens [N+1] (None = one sequence).
    qk_of_v [Hv] gives the q/k head each v-head reads (default h // (Hv/Hqk)).

    Per sequence and v-head, with state S (dv x dk) and each token in order:
        a = exp(g_t)
        S <- a S
        e  = v_t - S k_t            (prediction error of the decayed state)
        S <- S + beta_t e k_t^T
        o_t = scale * S q_t
    which equals S_t = a S (I - beta k k^T) + beta v k^T followed by
    o_t = scale * S_t q_t.  Returns (o [T, Hv, dv], final [N, Hv, dv, dk]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    t_total, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if qk_of_v is None:
        qk_of_v = np.arange(hv) // (hv // hqk)
    qk_of_v = np.asarray(qk_of_v, np.int64)
    cu = (np.array([0, t_total], np.int64) if cu_seqlens is None
          else np.asarray(cu_seqlens, np.int64))
    n = len(cu) - 1
    if initial_state is None:
        initial_state = np.zeros((n, hv, dv, dk))
    o = np.zeros((t_total, hv, dv))
    final = np.zeros((n, hv, dv, dk))
    for s in range(n):
        S = np.array(initial_state[s], np.float64)           # [Hv, dv, dk]
        for t in range(cu[s], cu[s + 1]):
            qt = q[t][qk_of_v]                                # [Hv, dk]
            kt = k[t][qk_of_v]
            if use_qk_l2norm:
                qt = l2_normalize(qt, l2_eps)
                kt = l2_normalize(kt, l2_eps)
            a = np.exp(g[t])                                  # [Hv]
            S = a[:, None, None] * S
            e = v[t] - np.matmul(S, kt[:, :, None])[:, :, 0]   # [Hv, dv]
            S = S + beta[t][:, None, None] * e[:, :, None] * kt[:, None, :]
            o[t] = scale * np.matmul(S, qt[:, :, None])[:, :, 0]
        final[s] = S
    return o, final


# ---------------------------------------------------------------------------
# Speculative verification: per-token state checkpoints and conv windows
# ---------------------------------------------------------------------------

def verify_checkpoints(q, k, v, g, beta, *, initial_state, scale=1.0, use_qk_l2norm=True,
                       l2_eps=1e-6, qk_of_v=None):
    """The W verification tokens of one request, one at a time from its live
    state (Flare core-design, speculative target state: one recurrent
    checkpoint column per verification input).

    q, k [W, Hqk, dk]; v [W, Hv, dv]; g, beta [W, Hv]; initial_state
    [Hv, dv, dk].  Column t is the state after tokens 0..t.  Each token is one
    call of gated_delta_rule starting from the previous column.  Returns
    (o [W, Hv, dv], columns [W, Hv, dv, dk]).
    """
    w = np.asarray(q).shape[0]
    hv, dv = np.asarray(v).shape[1], np.asarray(v).shape[2]
    dk = np.asarray(q).shape[2]
    o = np.zeros((w, hv, dv))
    cols = np.zeros((w, hv, dv, dk))
    S = np.asarray(initial_state, np.float64)[None]
    for t in range(w):
        ot, S = gated_delta_rule(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1],
                                 scale=scale, initial_state=S, use_qk_l2norm=use_qk_l2norm,
                                 l2_eps=l2_eps, qk_of_v=qk_of_v)
        o[t] = ot[0]
        cols[t] = S[0]
    return o, cols


def conv_windows(tail, x):
    """The 3-token conv history after each of the W tokens x [W, Ch] of one
    request whose history before them is tail [3, Ch] (Flare core-design,
    snapshot of the three-token GDN convolution window of a column): window t
    is rows t+1 .. t+3 of [tail; x].  Returns [W, 3, Ch]."""
    full = np.concatenate([np.asarray(tail, np.float64), np.asarray(x, np.float64)], axis=0)
    return np.stack([full[t + 1:t + 4] for t in range(np.asarray(x).shape[0])])


# ---------------------------------------------------------------------------
# Gated RMSNorm
# ---------------------------------------------------------------------------

def gated_rmsnorm(o, z, w, eps: float):
    """y = o / sqrt(mean(o^2) + eps) * w * SiLU(z) over the last axis."""
    o = np.asarray(o, np.float64)
    r = np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    return o / r * np.asarray(w, np.float64) * silu(z)


# ---------------------------------------------------------------------------
# Whole mixer: prefill and decode
# ---------------------------------------------------------------------------

def split_heads(y, h_qk, d_k, h_v, d_v):
    """[T, Ch] (channels q | k | v) -> q [T,Hqk,dk], k [T,Hqk,dk], v [T,Hv,dv]."""
    t = y.shape[0]
    nq = h_qk * d_k
    return (y[:, :nq].reshape(t, h_qk, d_k), y[:, nq:2 * nq].reshape(t, h_qk, d_k),
            y[:, 2 * nq:].reshape(t, h_v, d_v))


def mixer_prefill(x, conv_w, tail, state, beta, g, z, norm_w, cu_seqlens, *,
                  h_qk, h_v, d_k, d_v, bf16_boundary: bool, scale=1.0,
                  l2_eps=1e-6, norm_eps=1e-6, qk_of_v=None):
    """conv1d + SiLU -> split q|k|v -> gated delta rule -> gated RMSNorm.

    Returns dict(y_conv, tail, o, y, state).  `z` None skips the norm.
    """
    y_conv, new_tail = causal_conv1d_silu(x, conv_w, tail, cu_seqlens,
                                          round_to_bf16=bf16_boundary)
    q, k, v = split_heads(y_conv, h_qk, d_k, h_v, d_v)
    o, final = gated_delta_rule(q, k, v, g, beta, scale=scale, initial_state=state,
                                cu_seqlens=cu_seqlens, use_qk_l2norm=True,
                                l2_eps=l2_eps, qk_of_v=qk_of_v)
    y = None if z is None else gated_rmsnorm(o, z, norm_w, norm_eps)
    return dict(y_conv=y_conv, tail=new_tail, o=o, y=y, state=final)


def mixer_decode_step(x, conv_w, tail, state, beta, g, z, norm_w, slots, *,
                      h_qk, h_v, d_k, d_v, bf16_boundary: bool, scale=1.0,
                      l2_eps=1e-6, norm_eps=1e-6, qk_of_v=None):
    """One token for each request r, reading and updating slot slots[r].

    tail [n_slots, 3, Ch] and state [n_slots, Hv, dv, dk] are updated in
    place (float64 arrays).  A negative slot is an inactive lane: nothing is
    read or written for it and its output rows stay NaN.
    Returns dict(y_conv, o, y).
    """
    n_req = x.shape[0]
    slots = np.asarray(slots, np.int64)
    y_conv = np.full(x.shape, np.nan)
    o = np.full((n_req, h_v, d_v), np.nan)
    y = np.full((n_req, h_v, d_v), np.nan)
    for r in range(n_req):
        s = slots[r]
        if s < 0:
            continue
        yc, nt = causal_conv1d_silu(x[r:r + 1], conv_w, tail[s:s + 1], [0, 1],
                                    round_to_bf16=bf16_boundary)
        tail[s] = nt[0]
        y_conv[r] = yc[0]
        q, k, v = split_heads(yc, h_qk, d_k, h_v, d_v)
        orow, fin = gated_delta_rule(q, k, v, g[r:r + 1], beta[r:r + 1], scale=scale,
                                     initial_state=state[s:s + 1], use_qk_l2norm=True,
                                     l2_eps=l2_eps, qk_of_v=qk_of_v)
        state[s] = fin[0]
        o[r] = orow[0]
        if z is not None:
            y[r] = gated_rmsnorm(orow[0], z[r], norm_w, norm_eps)
    return dict(y_conv=y_conv, o=o, y=y)


def mixer_mixed(x, conv_w, conv_pool, state_pool, slots, fresh, beta, g, z, norm_w, cu_seqlens, *,
                h_qk, h_v, d_k, d_v, bf16_boundary: bool, scale=1.0, l2_eps=1e-6, norm_eps=1e-6,
                qk_of_v=None):
    """A mixed prefill-plus-decode batch over caller-owned state pools (Flare
    core-design: the prepared short-convolution interface with state-slot ids,
    a fresh-state flag, device-resident counts, fixed capacities and a mixed
    prefill-plus-decode mode; inactive lanes write no state; padding changes
    capacity, never logical length, and padded rows take no part in any update).

    x [T_cap, Ch] holds cu_seqlens[-1] <= T_cap live rows; the rest is padding.
    For each sequence s with slot p = slots[s] >= 0: the history and the state
    it starts from are zeros if fresh[s] else conv_pool[p] and state_pool[p];
    it runs the mixer (mixer_prefill on its own tokens); the pools' row p then
    holds its history and state after exactly its tokens.  A sequence with
    p < 0 is inactive: nothing is read or written.  conv_pool [n_slots, 3, Ch]
    and state_pool [n_slots, Hv, dv, dk] are float64 arrays updated in place;
    output rows that no active sequence writes (inactive, padding) are NaN.
    A decode token is a sequence of length 1.  Returns dict(y_conv, o, y).
    """
    cu = np.asarray(cu_seqlens, np.int64)
    t_cap, ch = np.asarray(x).shape
    y_conv = np.full((t_cap, ch), np.nan)
    o = np.full((t_cap, h_v, d_v), np.nan)
    y = np.full((t_cap, h_v, d_v), np.nan)
    for s in range(len(cu) - 1):
        p = int(slots[s])
        if p < 0:
            continue
        a, b = int(cu[s]), int(cu[s + 1])
        is_fresh = fresh is not None and bool(fresh[s])
        tail0 = np.zeros((1, 3, ch)) if is_fresh else conv_pool[p:p + 1]
        state0 = np.zeros((1, h_v, d_v, d_k)) if is_fresh else state_pool[p:p + 1]
        r = mixer_prefill(x[a:b], conv_w, tail0, state0, beta[a:b], g[a:b],
                          None if z is None else z[a:b], norm_w, [0, b - a],
                          h_qk=h_qk, h_v=h_v, d_k=d_k, d_v=d_v, bf16_boundary=bf16_boundary,
                          scale=scale, l2_eps=l2_eps, norm_eps=norm_eps, qk_of_v=qk_of_v)
        y_conv[a:b] = r["y_conv"]
        o[a:b] = r["o"]
        if z is not None:
            y[a:b] = r["y"]
        conv_pool[p] = r["tail"][0]
        state_pool[p] = r["state"][0]
    return dict(y_conv=y_conv, o=o, y=y)


def max_abs_over_rms(got, ref) -> float:
    """max |got - ref| / RMS(ref) over all elements (the parity metric)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got - ref)))
