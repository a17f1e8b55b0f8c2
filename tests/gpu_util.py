"""Helpers for the GPU tests: device upload and the parity metric."""
import math
import sys

import numpy as np
import torch

DEV = "cuda:0"


def dev(a, dtype=torch.float32):
    """Host float array (exactly representable in dtype) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype).to(DEV)


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_max(got, ref):
    """max |got - ref| / RMS(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = math.sqrt(float(np.mean(ref * ref)))
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    return err / rms if rms > 0 else err


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def conv_abs_sum(x, w, tail, cu):
    """sum_i |w[c, i] * padded[t + i, c]| per output element: the scale of the
    fp32 rounding error of the 4-tap sum (its condition)."""
    x = np.abs(np.asarray(x, np.float64))
    w = np.abs(np.asarray(w, np.float64))
    tail = np.abs(np.asarray(tail, np.float64))
    out = np.zeros_like(x)
    for s in range(len(cu) - 1):
        xs = x[cu[s]:cu[s + 1]]
        p = np.concatenate([tail[s], xs])
        for i in range(4):
            out[cu[s]:cu[s + 1]] += w[:, i][None] * p[i:i + xs.shape[0]]
    return out


def bf16_ulp_check(got, ref_rounded, ref_exact, max_frac=1e-3, abs_sum=None):
    """bf16 outputs: every element equals the oracle's bf16 rounding or an
    adjacent bf16 value (the rounding decision taken on an fp32 sum instead of
    a float64 one), and such disagreements are rare.  With `abs_sum` (the
    condition of the fp32 sum, see conv_abs_sum) the allowance adds the fp32
    accumulation error bound 8 * 2^-24 * abs_sum * max|SiLU'| for outputs
    that come from cancelling sums."""
    got = np.asarray(got, np.float64)
    ref_rounded = np.asarray(ref_rounded, np.float64)
    diff = np.abs(got - ref_rounded)
    mant, expo = np.frexp(np.maximum(np.abs(ref_exact), 1e-30))
    ulp = np.ldexp(1.0, expo - 8)
    allow = ulp * 1.0000001
    if abs_sum is not None:
        allow = allow + 8 * 2.0 ** -24 * 1.1 * np.asarray(abs_sum, np.float64)
    assert np.all(diff <= allow), f"max diff/allowance {np.max(diff / allow):.3f}"
    frac = float(np.mean(diff > 0))
    assert frac <= max_frac, f"one-ulp disagreements {frac:.2e}"
    return frac


def conv_check_all_channels(x, w, tail, cu, got, oracle, block=1024, max_frac=1e-3):
    """bf16 conv output `got` [T, Ch] against the oracle's conv on every
    channel, in blocks of channels so the float64 temporaries stay bounded.
    Returns the fraction of one-ulp disagreements over all elements."""
    x = np.asarray(x)
    ch = x.shape[1]
    n_diff = 0
    for c0 in range(0, ch, block):
        sl = slice(c0, min(ch, c0 + block))
        exact, _ = oracle.causal_conv1d_silu(x[:, sl], w[sl], tail[:, :, sl], cu, round_to_bf16=False)
        frac = bf16_ulp_check(got[:, sl], oracle.bf16_nearest(exact), exact, max_frac=max_frac,
                              abs_sum=conv_abs_sum(x[:, sl], w[sl], tail[:, :, sl], cu))
        n_diff += frac * exact.size
    return n_diff / x.size
