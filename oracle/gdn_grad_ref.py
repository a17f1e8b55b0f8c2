"""Float64 CPU oracle for the gradients of the Gated DeltaNet mixer
(test infrastructure).

This is test infrastructure, not part of the library: only the test suite
may import or run it.  It shares no code with the HIP path.

What it computes: the gradients of a scalar loss
    L = sum(do * o) + sum(d_final * S_T)
with respect to every input of the gated delta rule (q, k, v, g, beta and
the initial state), and of
    L = sum(dy * y) + sum(d_tail_out * tail_out)
with respect to the inputs of the causal conv1d + SiLU (x, w and the
incoming history).  The forward computation is the one of oracle/gdn_ref.py
(the gated delta rule S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
o_t = scale S_t q_t with a_t = exp(g_t): haskell-infer-demo README,
"Highlights" and "Architecture"; the width-4 conv with SiLU over a 3-token
raw-input history: Flare core-design, short-convolution paragraph), written
here token by token in float64 PyTorch, and the gradients are its reverse-mode
derivatives by torch.autograd (a library routine used as one step).  The
pages print no gradient values; the CPU tests pin these functions against
central finite differences of oracle/gdn_ref.py's own forward and against
closed forms.
"""
from __future__ import annotations

import numpy as np
import torch


def _t(a):
    return torch.as_tensor(np.asarray(a, np.float64), dtype=torch.float64).clone().requires_grad_(True)


def _l2(x, eps):
    return x / torch.sqrt((x * x).sum(-1, keepdim=True) + eps)


def _rule_forward(q, k, v, g, beta, s0, cu, scale, use_l2, l2_eps, qk_of_v):
    """Token-by-token forward: o [T, Hv, dv] and the final states [N, Hv, dv, dk]."""
    outs, finals = [], []
    for s in range(len(cu) - 1):
        S = s0[s]
        for t in range(int(cu[s]), int(cu[s + 1])):
            qt, kt = q[t][qk_of_v], k[t][qk_of_v]
            if use_l2:
                qt, kt = _l2(qt, l2_eps), _l2(kt, l2_eps)
            a = torch.exp(g[t])
            S = a[:, None, None] * S
            e = v[t] - torch.matmul(S, kt[:, :, None])[:, :, 0]
            S = S + beta[t][:, None, None] * e[:, :, None] * kt[:, None, :]
            outs.append(scale * torch.matmul(S, qt[:, :, None])[:, :, 0])
        finals.append(S)
    o = torch.stack(outs) if outs else torch.zeros((0,) + tuple(v.shape[1:]), dtype=torch.float64)
    return o, torch.stack(finals)


def gated_delta_rule_grads(q, k, v, g, beta, do, d_final=None, *, scale=1.0, initial_state=None,
                           cu_seqlens=None, use_qk_l2norm=True, l2_eps=1e-6, qk_of_v=None):
    """Gradients of L = sum(do * o) + sum(d_final * S_T) for the gated delta
    rule of oracle/gdn_ref.gated_delta_rule (same arguments and layouts).

    do [T, Hv, dv]; d_final [N, Hv, dv, dk] or None (zero).  Returns a dict
    of float64 arrays: dq, dk [T, Hqk, dk] (through the L2 normalisation when
    use_qk_l2norm), dv [T, Hv, dv], dg, dbeta [T, Hv], d_initial [N, Hv, dv, dk],
    and the forward's o and final for reference.
    """
    q, k, v, g, beta = _t(q), _t(k), _t(v), _t(g), _t(beta)
    t_total, hqk, dk_ = q.shape
    hv, dv_ = v.shape[1], v.shape[2]
    cu = np.array([0, t_total]) if cu_seqlens is None else np.asarray(cu_seqlens, np.int64)
    n = len(cu) - 1
    s0 = _t(np.zeros((n, hv, dv_, dk_)) if initial_state is None else initial_state)
    qk = np.arange(hv) // (hv // hqk) if qk_of_v is None else np.asarray(qk_of_v, np.int64)
    qk = torch.as_tensor(qk)
    o, fin = _rule_forward(q, k, v, g, beta, s0, cu, float(scale), bool(use_qk_l2norm), float(l2_eps), qk)
    loss = (o * torch.as_tensor(np.asarray(do, np.float64))).sum()
    if d_final is not None:
        loss = loss + (fin * torch.as_tensor(np.asarray(d_final, np.float64))).sum()
    grads = torch.autograd.grad(loss, [q, k, v, g, beta, s0], allow_unused=True)
    names = ["dq", "dk", "dv", "dg", "dbeta", "d_initial"]
    shapes = [q.shape, k.shape, v.shape, g.shape, beta.shape, s0.shape]
    out = {nm: (np.zeros(tuple(sh)) if gr is None else gr.detach().numpy()) for nm, gr, sh in zip(names, grads, shapes)}
    out["o"] = o.detach().numpy()
    out["final"] = fin.detach().numpy()
    return out


def causal_conv1d_silu_grads(x, w, tail, cu_seqlens, dy, d_tail_out=None):
    """Gradients of L = sum(dy * y) + sum(d_tail_out * tail_out) for
    oracle/gdn_ref.causal_conv1d_silu without the output rounding (same
    layouts: x [T, Ch], w [Ch, 4], tail [N, 3, Ch], oldest first).  Returns
    float64 dx [T, Ch], dw [Ch, 4], d_tail [N, 3, Ch] (the gradient of the
    incoming history) and the forward's y and tail_out."""
    x, w, tail = _t(x), _t(w), _t(tail)
    cu = np.asarray(cu_seqlens, np.int64)
    ys, tails_out = [], []
    for s in range(len(cu) - 1):
        xs = x[int(cu[s]):int(cu[s + 1])]
        padded = torch.cat([tail[s], xs], dim=0)
        length = xs.shape[0]
        acc = torch.zeros((length, x.shape[1]), dtype=torch.float64)
        for i in range(4):                                   # tap i reads token t - 3 + i
            acc = acc + w[:, i][None, :] * padded[i:i + length]
        ys.append(acc / (1.0 + torch.exp(-acc)))
        tails_out.append(padded[-3:])
    y = torch.cat(ys, dim=0)
    tail_out = torch.stack(tails_out)
    loss = (y * torch.as_tensor(np.asarray(dy, np.float64))).sum()
    if d_tail_out is not None:
        loss = loss + (tail_out * torch.as_tensor(np.asarray(d_tail_out, np.float64))).sum()
    gx, gw, gt = torch.autograd.grad(loss, [x, w, tail], allow_unused=True)
    z = lambda gr, ref: np.zeros(tuple(ref.shape)) if gr is None else gr.detach().numpy()
    return dict(dx=z(gx, x), dw=z(gw, w), d_tail=z(gt, tail), y=y.detach().numpy(),
                tail_out=tail_out.detach().numpy())
