"""Seeded synthetic inputs for the Gated DeltaNet mixer.

This module is the only code shared by the float64 oracle and the GPU path.
It draws random numbers and arranges them into arrays; it holds none of the
mixer's arithmetic (no convolution, normalisation, decay or recurrence).

Every floating-point array is returned as float32.  For bf16 workloads the
values are rounded to the nearest bf16 (ties to even) before they are
returned, so the same array is exact both as a bf16 device tensor and as the
oracle's float64 input.

Shapes follow the mixer's layout:
  x        [T, Ch]           conv input, channels ordered q | k | v
  conv_w   [Ch, 4]           depthwise conv taps, tap 3 multiplies the current token
  tail     [N, 3, Ch]        conv history, oldest token first
  state    [N, Hv, dv, dk]   recurrent state S (S k = v orientation)
  beta, g  [T, Hv]           write strength and log-decay per token and v-head
  z        [T, Hv, dv]       gate of the gated RMSNorm
  norm_w   [dv]              RMSNorm weight
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Layout:
    h_qk: int
    h_v: int
    d_k: int
    d_v: int
    chunk: int
    dtype: str  # "bf16" or "f32"

    @property
    def channels(self) -> int:
        return 2 * self.h_qk * self.d_k + self.h_v * self.d_v

    @property
    def group(self) -> int:
        return self.h_v // self.h_qk


# Hybrid-model mixer shape: 16 q/k heads shared by 32 v heads, head dim 128.
MODEL_LAYOUT = Layout(h_qk=16, h_v=32, d_k=128, d_v=128, chunk=64, dtype="bf16")
# Tiny fp32 check shape.
TINY_LAYOUT = Layout(h_qk=2, h_v=2, d_k=16, d_v=16, chunk=16, dtype="f32")

L2_EPS = 1e-6
NORM_EPS = 1e-6


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 value (ties to even), returned as float32.

    Pure bit manipulation on the IEEE encoding; inputs are finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    r = ((u + bias) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of bf16-representable float32 values (for device upload)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def _normal(rng, shape, std=1.0) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float64) * std).astype(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _beta(rng, shape) -> np.ndarray:
    return _sigmoid(rng.standard_normal(shape)).astype(np.float32)


def _model_g(rng, a_head: np.ndarray, shape) -> np.ndarray:
    """g = -exp(A) * softplus(n), n ~ N(0,1) per (token, head), A fixed per head."""
    n = rng.standard_normal(shape)
    return (-np.exp(a_head)[None, :] * _softplus(n)).astype(np.float32)


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


def c3_lengths(seed: int = 3, n: int = 8) -> list[int]:
    """Sequence lengths log-uniform in [512, 32768]."""
    rng = np.random.default_rng(seed)
    lo, hi = math.log(512), math.log(32768)
    return [int(v) for v in np.floor(np.exp(rng.uniform(lo, hi, n)))]


def prefill_inputs(seed: int, layout: Layout, lengths, *, state_std: float | None = None,
                   tail_std: float | None = None, g_mode: str = "model",
                   rng: np.random.Generator | None = None) -> dict:
    """Packed prefill inputs for the conv -> gated delta rule -> gated RMSNorm path.

    Draw order: x, conv w, tails, states, beta noise, A, softplus noise, z, norm w.
    g_mode "model": g = -exp(A) softplus(N(0,1)), A ~ U(0, ln 16) per v-head.
    g_mode "tiny":  g ~ -U(0.01, 0.5).
    state_std / tail_std None means zero initial state / zero conv tail.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = [int(v) for v in lengths]
    n, t = len(lengths), int(sum(lengths))
    ch, hv, dv, dk = layout.channels, layout.h_v, layout.d_v, layout.d_k
    dt = layout.dtype
    x = _cast(_normal(rng, (t, ch)), dt)
    conv_w = _cast(_normal(rng, (ch, 4), 0.5), dt)
    tail = (_cast(_normal(rng, (n, 3, ch), tail_std), dt) if tail_std is not None
            else np.zeros((n, 3, ch), np.float32))
    state = (_normal(rng, (n, hv, dv, dk), state_std) if state_std is not None
             else np.zeros((n, hv, dv, dk), np.float32))
    beta = _beta(rng, (t, hv))
    if g_mode == "model":
        a_head = rng.uniform(0.0, math.log(16.0), hv)
        g = _model_g(rng, a_head, (t, hv))
    elif g_mode == "tiny":
        g = (-rng.uniform(0.01, 0.5, (t, hv))).astype(np.float32)
    else:
        raise ValueError(g_mode)
    z = _cast(_normal(rng, (t, hv, dv)), dt)
    norm_w = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    return dict(layout=layout, x=x, conv_w=conv_w, tail=tail, state=state, beta=beta,
                g=g, z=z, norm_w=norm_w, cu_seqlens=cu_from_lengths(lengths),
                lengths=lengths, scale=1.0, l2_eps=L2_EPS, norm_eps=NORM_EPS)


def mixed_batch_inputs(seed: int, layout: Layout, lengths, n_slots: int, *, t_pad: int = 0) -> dict:
    """A serving batch packed for the mixed prefill-plus-decode calls: prompt
    chunks and decode tokens (length-1 sequences) with per-token data drawn as
    prefill_inputs draws it, t_pad padding rows after the live ones, and state
    pools of n_slots rows: histories N(0,1), states N(0, 0.02^2).

    Draw order: the prefill_inputs draws for the live tokens (zero states),
    then the history pool, then the state pool.  Padding rows of x, beta, g
    and z are zeros here; tests poison them.
    """
    rng = np.random.default_rng(seed)
    d = prefill_inputs(seed, layout, lengths, rng=rng)
    ch, hv, dv, dk = layout.channels, layout.h_v, layout.d_v, layout.d_k
    d["tail_pool"] = _cast(_normal(rng, (n_slots, 3, ch)), layout.dtype)
    d["state_pool"] = _normal(rng, (n_slots, hv, dv, dk), 0.02)
    if t_pad:
        for key in ("x", "beta", "g", "z"):
            a = d[key]
            d[key] = np.concatenate([a, np.zeros((t_pad,) + a.shape[1:], a.dtype)])
    d["t_cap"] = int(sum(lengths)) + t_pad
    return d


def raw_gate_inputs(seed: int, t: int, h_v: int, *, dtype: str = "f32",
                    a_log_range=(0.0, math.log(16.0)), bias_std: float | None = None) -> dict:
    """Raw gate projections for the fused gate preparation.

    a, b ~ N(0,1) [T, Hv] (rounded to bf16 when dtype is "bf16"); a_log ~
    U(a_log_range) per v-head; dt_bias ~ N(0, bias_std^2) per v-head, or None.
    With the default range and no bias, -exp(a_log) softplus(a) has the same
    distribution as the model workload's log-decay.  Draw order: a_log, a, b,
    dt_bias.
    """
    rng = np.random.default_rng(seed)
    a_log = rng.uniform(a_log_range[0], a_log_range[1], h_v).astype(np.float32)
    a = _cast(_normal(rng, (t, h_v)), dtype)
    b = _cast(_normal(rng, (t, h_v)), dtype)
    dt_bias = None if bias_std is None else _normal(rng, (h_v,), bias_std)
    return dict(a=a, b=b, a_log=a_log, dt_bias=dt_bias)


def split_qkv(x: np.ndarray, layout: Layout):
    """Views of the q | k | v channel blocks of a [T, Ch] array as per-head arrays."""
    t = x.shape[0]
    nq = layout.h_qk * layout.d_k
    q = x[:, :nq].reshape(t, layout.h_qk, layout.d_k)
    k = x[:, nq:2 * nq].reshape(t, layout.h_qk, layout.d_k)
    v = x[:, 2 * nq:].reshape(t, layout.h_v, layout.d_v)
    return q, k, v


def tiny_inputs(seed: int = 0, t: int = 64) -> dict:
    """Tiny fp32 check: B=1, T=64, 2 heads, d=16, chunk 16.

    q, k, v ~ N(0,1) are the raw channels x = [q | k | v]; the recurrence
    alone reads them directly (normalising q and k), the full path convolves
    them first.  beta = sigmoid(N(0,1)); g ~ -U(0.01, 0.5); zero state; conv
    weights N(0, 0.5^2).
    """
    d = prefill_inputs(seed, TINY_LAYOUT, [t], g_mode="tiny")
    return d


def model_prefill_inputs(t: int = 4096, seed: int = 1) -> dict:
    """Single-sequence prefill: B=1, T=4096, zero state and tail."""
    return prefill_inputs(seed, MODEL_LAYOUT, [t])


def varlen_prefill_inputs(lengths=None, seed: int = 3) -> dict:
    """Varlen packed prefill: 8 sequences, log-uniform lengths, nonzero state/tail."""
    rng = np.random.default_rng(seed)
    if lengths is None:
        lo, hi = math.log(512), math.log(32768)
        lengths = [int(v) for v in np.floor(np.exp(rng.uniform(lo, hi, 8)))]
    return prefill_inputs(seed, MODEL_LAYOUT, lengths, state_std=0.02, tail_std=1.0, rng=rng)


def decode_inputs(seed: int, layout: Layout, n_req: int, n_steps: int, *,
                  state_std: float = 0.02, tail_std: float = 1.0,
                  n_slots: int | None = None) -> dict:
    """Batched decode: n_req requests x n_steps single-token steps.

    Draw order: conv w, tails, states, A, norm w, then per step in step
    order: x, beta noise, softplus noise, z.  Tails and states are drawn for
    n_slots slots (default n_req).
    """
    rng = np.random.default_rng(seed)
    n_slots = n_req if n_slots is None else n_slots
    ch, hv, dv, dk, dt = layout.channels, layout.h_v, layout.d_v, layout.d_k, layout.dtype
    conv_w = _cast(_normal(rng, (ch, 4), 0.5), dt)
    tail = _cast(_normal(rng, (n_slots, 3, ch), tail_std), dt)
    state = _normal(rng, (n_slots, hv, dv, dk), state_std)
    a_head = rng.uniform(0.0, math.log(16.0), hv)
    norm_w = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    xs, betas, gs, zs = [], [], [], []
    for _ in range(n_steps):
        xs.append(_cast(_normal(rng, (n_req, ch)), dt))
        betas.append(_beta(rng, (n_req, hv)))
        gs.append(_model_g(rng, a_head, (n_req, hv)))
        zs.append(_cast(_normal(rng, (n_req, hv, dv)), dt))
    return dict(layout=layout, conv_w=conv_w, tail=tail, state=state, norm_w=norm_w,
                x=np.stack(xs), beta=np.stack(betas), g=np.stack(gs), z=np.stack(zs),
                scale=1.0, l2_eps=L2_EPS, norm_eps=NORM_EPS)


def long_context_calls(seed: int = 4, n_calls: int = 16, call_len: int = 8192,
                       n_decode: int = 256, layout: Layout = MODEL_LAYOUT,
                       heads: list[int] | None = None):
    """Long-context chunked prefill then decode, one sequence.

    Yields ("prefill", dict) for each of n_calls calls of call_len tokens and
    then ("decode", dict) for each of n_decode single-token steps, all drawn
    from one generator in that order, after conv w, A and norm w.  Zero
    initial state and tail.  With `heads` (v-head indices), each array keeps
    only the channels of those heads and of their q/k heads, so the whole
    stream can be held in host memory for a sampled oracle run; the draws are
    the same either way.
    """
    rng = np.random.default_rng(seed)
    ch, hv, dv, dt = layout.channels, layout.h_v, layout.d_v, layout.dtype
    conv_w = _cast(_normal(rng, (ch, 4), 0.5), dt)
    a_head = rng.uniform(0.0, math.log(16.0), hv)
    norm_w = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    sel_ch, sel_h = None, None
    if heads is not None:
        sel_h = np.asarray(heads, dtype=np.int64)
        sel_ch = head_channels(layout, heads)
        conv_w = conv_w[sel_ch]
    common = dict(layout=layout, conv_w=conv_w, norm_w=norm_w, scale=1.0,
                  l2_eps=L2_EPS, norm_eps=NORM_EPS, channels=sel_ch, heads=sel_h)
    for i in range(n_calls + n_decode):
        tlen = call_len if i < n_calls else 1
        x = _cast(_normal(rng, (tlen, ch)), dt)
        beta = _beta(rng, (tlen, hv))
        g = _model_g(rng, a_head, (tlen, hv))
        z = _cast(_normal(rng, (tlen, hv, dv)), dt)
        if heads is not None:
            x, beta, g, z = x[:, sel_ch], beta[:, sel_h], g[:, sel_h], z[:, sel_h]
        kind = "prefill" if i < n_calls else "decode"
        yield kind, dict(common, x=x, beta=beta, g=g, z=z, index=i)


def head_channels(layout: Layout, heads) -> np.ndarray:
    """Conv channel indices feeding the given v-heads (their q, k and v channels),
    ordered q | k | v with the q/k heads of the selection deduplicated in order."""
    g = layout.group
    qk_heads = sorted({int(h) // g for h in heads})
    nq = layout.h_qk * layout.d_k
    q = [hq * layout.d_k + j for hq in qk_heads for j in range(layout.d_k)]
    k = [nq + hq * layout.d_k + j for hq in qk_heads for j in range(layout.d_k)]
    v = [2 * nq + int(h) * layout.d_v + j for h in heads for j in range(layout.d_v)]
    return np.asarray(q + k + v, dtype=np.int64)
