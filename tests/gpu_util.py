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


def bf16_ulp_check(got, ref_rounded, ref_exact, max_frac=1e-3):
    """bf16 outputs: every element equals the oracle's bf16 rounding or an
    adjacent bf16 value (the rounding decision taken on fp32 vs float64 sums),
    and such one-ulp disagreements are rare."""
    got = np.asarray(got, np.float64)
    ref_rounded = np.asarray(ref_rounded, np.float64)
    diff = np.abs(got - ref_rounded)
    mant, expo = np.frexp(np.maximum(np.abs(ref_exact), 1e-30))
    ulp = np.ldexp(1.0, expo - 8)
    assert np.all(diff <= ulp * 1.0000001), f"max diff/ulp {np.max(diff / ulp):.3f}"
    frac = float(np.mean(diff > 0))
    assert frac <= max_frac, f"one-ulp disagreements {frac:.2e}"
    return frac
