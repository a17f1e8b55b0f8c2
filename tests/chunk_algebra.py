"""Chunked (UT/WY) form of the gated delta rule, evaluated on the CPU.

Test helper, not the oracle: it states the chunk algebra the GPU kernels
implement so that it can be checked against the sequential oracle to 1e-12,
and it emulates the rounding of candidate MFMA operand plans.

Within a chunk of C tokens entering with state S0 (dv x dk), with raw q, k
rows, rk_i = 1/sqrt(|k_i|^2 + eps) (1 without L2 norm), rq likewise,
gamma = inclusive cumsum of g over the chunk and b = exp(gamma):
    L_ij  = beta_i exp(gamma_i - gamma_j) rk_i rk_j (k_i . k_j)     j < i
    T     = (I + L)^-1                         (forward substitution)
    Tb    = T diag(beta)
    X     = V - diag(b rk) K S0^T              (error against the entering state)
    U     = Tb X                               (the per-token delta-rule writes)
    P_ij  = scale exp(gamma_i - gamma_j) rq_i rk_j (q_i . k_j)       j <= i
    O     = scale diag(b rq) Q S0^T + P U
    S_C   = b_C S0 + U^T diag(exp(gamma_C - gamma) rk) K
U solves u_i = beta_i (v_i - a_i S_{i-1} k^_i) token by token, which is the
delta rule written with the decayed entering state.

Form "gr" folds Tb into the two products that read U, so a chunk needs X only:
    R     = P Tb                                (C x C, lower triangular)
    G     = K^T diag(exp(gamma_C - gamma) rk) Tb   (dk x C)
    O     = scale diag(b rq) Q S0^T + R X
    S_C^T = b_C S0^T + G X
"""
from __future__ import annotations

import numpy as np


def _round_f32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def _bf16(x):
    x = np.asarray(x, np.float64).astype(np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32).view(np.float32).astype(np.float64)


def split_hi_lo(x):
    """fp32 value -> (hi, lo) bf16 pair with hi + lo ~ x to ~2^-17 relative."""
    x = _round_f32(x)
    hi = _bf16(x)
    lo = _bf16(x - hi)
    return hi, lo


class Plan:
    """How each contraction's operands are represented.

    exact : float64 throughout (the algebra check)
    f32   : fp32 operands and fp32 rounding of stored intermediates
    bf16x3: raw bf16 q/k/v single, derived operands as bf16 hi+lo pairs
            (hi*hi + hi*lo + lo*hi for derived x derived, hi*raw + lo*raw for
            derived x raw); fp32 stored intermediates and fp32 state
    bf16  : derived operands rounded to a single bf16
    """

    def __init__(self, name: str):
        assert name in ("exact", "f32", "bf16x3", "bf16")
        self.name = name

    def store(self, x):
        return x if self.name == "exact" else _round_f32(x)

    def mm(self, a, b, a_derived: bool, b_derived: bool, subscripts: str):
        e = lambda x, y: np.einsum(subscripts, x, y)
        if self.name in ("exact", "f32"):
            return self.store(e(a, b))
        if self.name == "bf16":
            a1 = _bf16(a) if a_derived else a
            b1 = _bf16(b) if b_derived else b
            return _round_f32(e(a1, b1))
        ah, al = split_hi_lo(a) if a_derived else (a, None)
        bh, bl = split_hi_lo(b) if b_derived else (b, None)
        r = e(ah, bh)
        if bl is not None:
            r = r + e(ah, bl)
        if al is not None:
            r = r + e(al, bh)
        return _round_f32(r)


def chunked_gated_delta_rule(q, k, v, g, beta, *, chunk, scale=1.0, initial_state=None,
                             cu_seqlens=None, use_qk_l2norm=True, l2_eps=1e-6,
                             plan: str = "exact", form: str = "tx"):
    """Same contract as the oracle's gated_delta_rule, evaluated chunk by chunk.
    Chunks restart at every sequence start; the last chunk may be partial.
    form "tx" forms U = Tb X; form "gr" uses R = P Tb and G = K^T diag(.) Tb."""
    assert form in ("tx", "gr")
    P = Plan(plan)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    t_total, hqk, dk = q.shape
    hv, dv = v.shape[1:]
    grp = hv // hqk
    cu = np.array([0, t_total]) if cu_seqlens is None else np.asarray(cu_seqlens, np.int64)
    n = len(cu) - 1
    S0 = np.zeros((n, hv, dv, dk)) if initial_state is None else np.asarray(initial_state, np.float64)
    o = np.zeros((t_total, hv, dv))
    final = np.zeros((n, hv, dv, dk))
    hq = np.arange(hv) // grp
    for s in range(n):
        S = P.store(S0[s].copy())                               # [Hv, dv, dk]
        for c0 in range(cu[s], cu[s + 1], chunk):
            c1 = min(c0 + chunk, cu[s + 1])
            C = c1 - c0
            K = k[c0:c1][:, hq].transpose(1, 0, 2)              # [Hv, C, dk] raw
            Q = q[c0:c1][:, hq].transpose(1, 0, 2)
            V = v[c0:c1].transpose(1, 0, 2)                     # [Hv, C, dv]
            bt = beta[c0:c1].T                                  # [Hv, C]
            if use_qk_l2norm:
                rk = 1.0 / np.sqrt(np.sum(K * K, -1) + l2_eps)
                rq = 1.0 / np.sqrt(np.sum(Q * Q, -1) + l2_eps)
            else:
                rk = np.ones(K.shape[:2])
                rq = np.ones(Q.shape[:2])
            gam = np.cumsum(g[c0:c1].T, axis=1)                 # [Hv, C]
            b = np.exp(gam)
            diff = gam[:, :, None] - gam[:, None, :]
            strict = np.tril(np.ones((C, C), bool), -1)
            incl = np.tril(np.ones((C, C), bool), 0)
            gam_s = np.where(strict, np.exp(np.where(strict, diff, 0.0)), 0.0)
            gam_i = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
            GK = np.einsum("hid,hjd->hij", K, K)                # raw x raw, exact products
            GQ = np.einsum("hid,hjd->hij", Q, K)
            L = P.store(bt[:, :, None] * gam_s * rk[:, :, None] * rk[:, None, :] * GK)
            T = np.zeros_like(L)
            eye = np.eye(C)
            for i in range(C):                                  # forward substitution
                T[:, i] = eye[i] - np.einsum("hj,hjc->hc", L[:, i, :i], T[:, :i])
            T = P.store(T)
            Tb = P.store(T * bt[:, None, :])
            Pm = P.store(scale * gam_i * rq[:, :, None] * rk[:, None, :] * GQ)
            KS = P.mm(K, S, False, True, "hcd,hvd->hcv")        # K S^T  [Hv, C, dv]
            QS = P.mm(Q, S, False, True, "hcd,hvd->hcv")
            X = P.store(V - (b * rk)[:, :, None] * KS)
            dec = np.exp(gam[:, -1:] - gam) * rk                # [Hv, C]
            if form == "tx":
                U = P.mm(Tb, X, True, True, "hij,hjv->hiv")
                O = scale * (b * rq)[:, :, None] * QS + P.mm(Pm, U, True, True, "hij,hjv->hiv")
                Ud = P.store(U * dec[:, :, None])
                S = P.store(b[:, -1][:, None, None] * S + P.mm(Ud, K, True, False, "hcv,hcd->hvd"))
            else:
                Rm = P.mm(Pm, Tb, True, True, "hik,hkj->hij")
                G = P.mm(K, P.store(dec[:, :, None] * Tb), False, True, "hcd,hcj->hdj")
                O = scale * (b * rq)[:, :, None] * QS + P.mm(Rm, X, True, True, "hij,hjv->hiv")
                S = P.store(b[:, -1][:, None, None] * S + P.mm(X, G, True, True, "hjv,hdj->hvd"))
            o[c0:c1] = O.transpose(1, 0, 2)
        final[s] = S
    return o, final


def chunked_gated_delta_rule_grads(q, k, v, g, beta, do, d_final=None, *, chunk, scale=1.0,
                                   initial_state=None, cu_seqlens=None, use_qk_l2norm=True,
                                   l2_eps=1e-6):
    """Gradients of L = sum(do * o) + sum(d_final * S_T), chunk by chunk, in
    float64: the algebra of the chunked backward kernels.

    A forward pass over the chunks keeps the state entering each chunk.  A
    reverse pass carries dS (the gradient of the state leaving the chunk)
    from the last chunk to the first; inside a chunk, with the forward's
    K^ = diag(rk) K, Q^ = diag(rq) Q, D_ij = exp(gamma_i - gamma_j) (j <= i),
    d = exp(gamma_C - gamma), A = K^ K^^T, T, Tb, X, U and P:
        dU  = P^T dO + diag(d) K^ dS^T
        dX  = Tb^T dU                         (= dV)
        dS0 = b_C dS + scale dO^T diag(b) Q^ - dX^T diag(b) K^
        dTb = dU X^T;  dbeta_j = sum_i dTb_ij T_ij;  dT = dTb diag(beta)
        dL  = -T^T dT T^T (strictly lower);  dbeta_i += sum_j dL_ij A_ij Ds_ij
        dP  = dO U^T (lower);  dAq = scale dP * D;  dA = diag(beta) dL * Ds
        dQ^ = scale diag(b) dO S0 + dAq K^
        dK^ = diag(d) U dS - diag(b) dX S0 + dAq^T Q^ + dA K^ + dA^T K^
        dgamma_i = rows of dP*P and dL*L (i) minus their columns (j),
                   + q^_i . (scale b_i (dO S0)_i) - b_i k^_i . (dX S0)_i
                   - d_j k^_j . (U dS)_j, and at the chunk's last token
                   + sum_j d_j k^_j . (U dS)_j + b_C <dS, S0>
        dg_t = sum_{i >= t} dgamma_i (inside the chunk)
    then dq, dk through the L2 normalisation after summing the v-heads that
    read each q/k head.  Returns the dict layout of the gradient oracle."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    do = np.asarray(do, np.float64)
    t_total, hqk, dk = q.shape
    hv, dv = v.shape[1:]
    grp = hv // hqk
    cu = np.array([0, t_total]) if cu_seqlens is None else np.asarray(cu_seqlens, np.int64)
    n = len(cu) - 1
    S0 = np.zeros((n, hv, dv, dk)) if initial_state is None else np.asarray(initial_state, np.float64)
    dF = np.zeros((n, hv, dv, dk)) if d_final is None else np.asarray(d_final, np.float64)
    hq = np.arange(hv) // grp
    dqh = np.zeros((t_total, hv, dk))    # per v-head, before the group sum
    dkh = np.zeros((t_total, hv, dk))
    out = {"dv": np.zeros((t_total, hv, dv)), "dg": np.zeros((t_total, hv)),
           "dbeta": np.zeros((t_total, hv)), "d_initial": np.zeros((n, hv, dv, dk))}
    if use_qk_l2norm:
        rq_all = 1.0 / np.sqrt(np.sum(q * q, -1) + l2_eps)          # [T, Hqk]
        rk_all = 1.0 / np.sqrt(np.sum(k * k, -1) + l2_eps)
    else:
        rq_all = np.ones(q.shape[:2])
        rk_all = np.ones(k.shape[:2])
    qn = q * rq_all[..., None]
    kn = k * rk_all[..., None]
    for s in range(n):
        bounds = [(c0, min(c0 + chunk, cu[s + 1])) for c0 in range(cu[s], cu[s + 1], chunk)]
        # forward: the state entering every chunk
        ent = []
        S = S0[s].copy()
        for c0, c1 in bounds:
            ent.append(S.copy())
            _, S = _chunk_fwd_terms(qn, kn, v, g, beta, c0, c1, hq, scale, S)
        dS = dF[s].copy()
        for (c0, c1), S in zip(reversed(bounds), reversed(ent)):
            f, _ = _chunk_fwd_terms(qn, kn, v, g, beta, c0, c1, hq, scale, S)
            Kh, Qh, b, d, bC, Ds, Dm, A, T, Tb, X, U, Pm, L = (f[x] for x in (
                "K", "Q", "b", "d", "bC", "Ds", "D", "A", "T", "Tb", "X", "U", "P", "L"))
            dO = do[c0:c1].transpose(1, 0, 2)                                  # [Hv, C, dv]
            bt = beta[c0:c1].T
            dU = np.einsum("hji,hjv->hiv", Pm, dO) + d[:, :, None] * np.einsum("hcd,hvd->hcv", Kh, dS)
            dX = np.einsum("hji,hjv->hiv", Tb, dU)
            dS_in = (bC[:, None, None] * dS + scale * np.einsum("hcv,hcd->hvd", dO * b[:, :, None], Qh)
                     - np.einsum("hcv,hcd->hvd", dX * b[:, :, None], Kh))
            dTb = np.einsum("hiv,hjv->hij", dU, X)
            db = np.einsum("hij,hij->hj", dTb, T)
            dT = dTb * bt[:, None, :]
            C = c1 - c0
            strict = np.tril(np.ones((C, C)), -1)
            incl = np.tril(np.ones((C, C)), 0)
            dL = -np.einsum("hki,hkl,hjl->hij", T, dT, T) * strict             # -T^T dT T^T, strict lower
            db = db + np.einsum("hij,hij->hi", dL, A * Ds)
            dP = np.einsum("hiv,hjv->hij", dO, U) * incl
            dAq = scale * dP * Dm
            dA = bt[:, :, None] * dL * Ds
            dOS = np.einsum("hcv,hvd->hcd", dO, S)
            dXS = np.einsum("hcv,hvd->hcd", dX, S)
            UdS = np.einsum("hcv,hvd->hcd", U, dS)
            dQh = scale * b[:, :, None] * dOS + np.einsum("hij,hjd->hid", dAq, Kh)
            dKh = (d[:, :, None] * UdS - b[:, :, None] * dXS + np.einsum("hji,hjd->hid", dAq, Qh)
                   + np.einsum("hij,hjd->hid", dA, Kh) + np.einsum("hji,hjd->hid", dA, Kh))
            M1 = dP * Pm
            M2 = dL * L
            dgam = (M1.sum(2) - M1.sum(1) + M2.sum(2) - M2.sum(1)
                    + scale * b * np.einsum("hcd,hcd->hc", Qh, dOS)
                    - b * np.einsum("hcd,hcd->hc", Kh, dXS))
            ddj = d * np.einsum("hcd,hcd->hc", Kh, UdS)
            dgam = dgam - ddj
            dgam[:, -1] += ddj.sum(1) + bC * np.einsum("hvd,hvd->h", dS, S)
            out["dg"][c0:c1] = np.cumsum(dgam[:, ::-1], axis=1)[:, ::-1].T
            out["dbeta"][c0:c1] = db.T
            out["dv"][c0:c1] = dX.transpose(1, 0, 2)
            dqh[c0:c1] = dQh.transpose(1, 0, 2)
            dkh[c0:c1] = dKh.transpose(1, 0, 2)
            dS = dS_in
        out["d_initial"][s] = dS
    # sum over the v-heads of each q/k head, then through the L2 normalisation
    dq_n = dqh.reshape(t_total, hqk, grp, dk).sum(2)
    dk_n = dkh.reshape(t_total, hqk, grp, dk).sum(2)
    if use_qk_l2norm:
        out["dq"] = rq_all[..., None] * (dq_n - qn * np.sum(qn * dq_n, -1, keepdims=True))
        out["dk"] = rk_all[..., None] * (dk_n - kn * np.sum(kn * dk_n, -1, keepdims=True))
    else:
        out["dq"], out["dk"] = dq_n, dk_n
    return out


def _chunk_fwd_terms(qn, kn, v, g, beta, c0, c1, hq, scale, S):
    """Forward terms of one chunk (all v-heads) from normalised q, k rows and
    the entering state S [Hv, dv, dk]; returns (terms, leaving state)."""
    C = c1 - c0
    Kh = kn[c0:c1][:, hq].transpose(1, 0, 2)
    Qh = qn[c0:c1][:, hq].transpose(1, 0, 2)
    V = v[c0:c1].transpose(1, 0, 2)
    bt = beta[c0:c1].T
    gam = np.cumsum(g[c0:c1].T, axis=1)
    b = np.exp(gam)
    bC = b[:, -1]
    d = np.exp(gam[:, -1:] - gam)
    diff = gam[:, :, None] - gam[:, None, :]
    strict = np.tril(np.ones((C, C), bool), -1)
    incl = np.tril(np.ones((C, C), bool), 0)
    Ds = np.where(strict, np.exp(np.where(strict, diff, 0.0)), 0.0)
    Dm = np.where(incl, np.exp(np.where(incl, diff, 0.0)), 0.0)
    A = np.einsum("hid,hjd->hij", Kh, Kh)
    L = bt[:, :, None] * A * Ds
    T = np.linalg.inv(np.eye(C)[None] + L)
    Tb = T * bt[:, None, :]
    X = V - b[:, :, None] * np.einsum("hcd,hvd->hcv", Kh, S)
    U = np.einsum("hij,hjv->hiv", Tb, X)
    Pm = scale * np.einsum("hid,hjd->hij", Qh, Kh) * Dm
    S_out = bC[:, None, None] * S + np.einsum("hcv,hc,hcd->hvd", U, d, Kh)
    return dict(K=Kh, Q=Qh, b=b, d=d, bC=bC, Ds=Ds, D=Dm, A=A, T=T, Tb=Tb, X=X, U=U, P=Pm, L=L), S_out
