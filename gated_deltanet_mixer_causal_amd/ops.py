"""Torch-facing binding of the GDN mixer C ABI (argument marshalling only).

Each function has the name of the C entry point it calls and passes the
tensors' device pointers, sizes and the current HIP stream straight through;
every step of the mixer runs in libgdn.so's kernels.  Tensors must live on
the GPU; outputs are written in place into the tensors passed in.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L

_DT = {torch.bfloat16: L.GDN_BF16, torch.float32: L.GDN_F32}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32") from None


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _rows_view(t: torch.Tensor, name: str) -> int:
    """Token stride of a [T, H, d] view whose last two dims are dense."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name} must be a [T, H, d] view with dense heads (got strides {t.stride()})")
    return t.stride(0)


def gdn_conv1d_fwd(x, w, conv_state, y, *, cu_seqlens=None, state_slots=None, n_seq=None, stream=None):
    """Width-4 causal conv1d + SiLU.  x, y [T, Ch]; w [Ch, 4]; conv_state [slots, 3, Ch].
    With cu_seqlens None every row of x is its own sequence (decode)."""
    t_total, ch = x.shape
    if n_seq is None:
        n_seq = (cu_seqlens.numel() - 1) if cu_seqlens is not None else t_total
    st = L.load().gdn_conv1d_fwd(_ptr(x), _dt(x), _ptr(w), ch, _ptr(cu_seqlens), n_seq, t_total,
                                 _ptr(conv_state), conv_state.shape[0], _ptr(state_slots), _ptr(y),
                                 _stream(stream))
    L.check("gdn_conv1d_fwd", st)
    return y


def gdn_chunk_fwd_workspace_size(h_qk, h_v, d_k, d_v, chunk, n_seq, t_total, dtype, with_norm) -> int:
    out = ctypes.c_size_t(0)
    st = L.load().gdn_chunk_fwd_workspace_size(h_qk, h_v, d_k, d_v, chunk, n_seq, t_total,
                                               _DT[dtype], int(bool(with_norm)), ctypes.byref(out))
    L.check("gdn_chunk_fwd_workspace_size", st)
    return out.value


def gdn_chunk_fwd(q, k, v, g, beta, o, *, chunk, scale=1.0, use_qk_l2norm=True, l2_eps=1e-6,
                  cu_seqlens=None, initial_state=None, final_state=None, z=None, norm_w=None,
                  norm_eps=1e-6, workspace=None, stream=None):
    """Chunked gated delta rule.  q, k [T, Hqk, dk]; v [T, Hv, dv] (token-strided views
    allowed); g, beta [T, Hv] fp32; o [T, Hv, dv]; states [N, Hv, dv, dk] fp32."""
    t_total, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n_seq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 1
    if workspace is None:
        nbytes = gdn_chunk_fwd_workspace_size(h_qk, h_v, d_k, d_v, chunk, n_seq, t_total, q.dtype, z is not None)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.load().gdn_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(g), _ptr(beta), float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, chunk, _ptr(cu_seqlens), n_seq, t_total,
        _ptr(initial_state), _ptr(final_state), _ptr(o), _dt(o),
        _ptr(z), _ptr(norm_w), float(norm_eps), _ptr(workspace), workspace.numel(), _stream(stream))
    L.check("gdn_chunk_fwd", st)
    return o


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, o, *, chunk, scale=1.0, use_qk_l2norm=True, l2_eps=1e-6,
                          cu_seqlens=None, initial_state=None, final_state=None, z=None, norm_w=None,
                          norm_eps=1e-6, stream=None):
    """gdn_chunk_fwd with the library's own device scratch instead of a workspace
    (for callers that cannot allocate); calls on one device must not overlap."""
    t_total, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n_seq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 1
    st = L.load().gdn_chunk_fwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(g), _ptr(beta), float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, chunk, _ptr(cu_seqlens), n_seq, t_total,
        _ptr(initial_state), _ptr(final_state), _ptr(o), _dt(o),
        _ptr(z), _ptr(norm_w), float(norm_eps), _stream(stream))
    L.check("gdn_chunk_fwd_noalloc", st)
    return o


def gdn_recurrent_step(q, k, v, g, beta, state, o, *, scale=1.0, use_qk_l2norm=True, l2_eps=1e-6,
                       state_slots=None, z=None, norm_w=None, norm_eps=1e-6, stream=None):
    """One decode token per request.  q, k [N, Hqk, dk]; v [N, Hv, dv]; g, beta [N, Hv];
    state [slots, Hv, dv, dk] fp32 updated in place; o [N, Hv, dv]."""
    n_req, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    st = L.load().gdn_recurrent_step(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(g), _ptr(beta), float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, n_req, _ptr(state), state.shape[0], _ptr(state_slots), _ptr(o), _dt(o),
        _ptr(z), _ptr(norm_w), float(norm_eps), _stream(stream))
    L.check("gdn_recurrent_step", st)
    return o


def _gate_rows(a: torch.Tensor, b: torch.Tensor) -> int:
    """Common row stride of the [rows, Hv] gate projection views a and b."""
    if a.dim() != 2 or b.dim() != 2 or a.shape != b.shape:
        raise ValueError(f"a and b must be [rows, Hv] views of one shape (got {tuple(a.shape)}, {tuple(b.shape)})")
    if a.stride(1) != 1 or b.stride(1) != 1 or a.stride(0) != b.stride(0) or a.dtype != b.dtype:
        raise ValueError("a and b need unit head stride, one row stride and one dtype")
    return a.stride(0)


def gdn_chunk_fwd_gated(q, k, v, a, b, a_log, o, *, chunk, dt_bias=None, scale=1.0, use_qk_l2norm=True,
                        l2_eps=1e-6, cu_seqlens=None, initial_state=None, final_state=None, z=None,
                        norm_w=None, norm_eps=1e-6, workspace=None, stream=None):
    """gdn_chunk_fwd with the gates formed in the kernel from the raw gate projections:
    g = -exp(a_log) * softplus(a + dt_bias), beta = sigmoid(b).  a, b [T, Hv] (bf16 or
    fp32, one row stride); a_log, dt_bias [Hv] fp32 (dt_bias None = 0)."""
    t_total, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n_seq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 1
    if workspace is None:
        nbytes = gdn_chunk_fwd_workspace_size(h_qk, h_v, d_k, d_v, chunk, n_seq, t_total, q.dtype, z is not None)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.load().gdn_chunk_fwd_gated(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(a), _ptr(b), _gate_rows(a, b), _dt(a), _ptr(a_log), _ptr(dt_bias),
        float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, chunk, _ptr(cu_seqlens), n_seq, t_total,
        _ptr(initial_state), _ptr(final_state), _ptr(o), _dt(o),
        _ptr(z), _ptr(norm_w), float(norm_eps), _ptr(workspace), workspace.numel(), _stream(stream))
    L.check("gdn_chunk_fwd_gated", st)
    return o


def gdn_recurrent_step_gated(q, k, v, a, b, a_log, state, o, *, dt_bias=None, scale=1.0, use_qk_l2norm=True,
                             l2_eps=1e-6, state_slots=None, z=None, norm_w=None, norm_eps=1e-6, stream=None):
    """gdn_recurrent_step with the gates formed in the kernel from a, b [N, Hv] and
    a_log, dt_bias [Hv] (as gdn_chunk_fwd_gated)."""
    n_req, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    st = L.load().gdn_recurrent_step_gated(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(a), _ptr(b), _gate_rows(a, b), _dt(a), _ptr(a_log), _ptr(dt_bias),
        float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, n_req, _ptr(state), state.shape[0], _ptr(state_slots), _ptr(o), _dt(o),
        _ptr(z), _ptr(norm_w), float(norm_eps), _stream(stream))
    L.check("gdn_recurrent_step_gated", st)
    return o


def gdn_recurrent_verify(q, k, v, g, beta, state, checkpoints, o, *, n_tok, scale=1.0, use_qk_l2norm=True,
                         l2_eps=1e-6, state_slots=None, z=None, norm_w=None, norm_eps=1e-6, stream=None):
    """Speculative verification of n_tok tokens per request.  q, k [N*W, Hqk, dk]; v [N*W, Hv, dv];
    g, beta [N*W, Hv] (request r: rows r*W .. r*W+W-1); state [slots, Hv, dv, dk] fp32 (read
    only); checkpoints [slots, cols, Hv, dv, dk] fp32 (column t = state after token t); o [N*W, Hv, dv]."""
    rows, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    if rows % n_tok:
        raise ValueError(f"{rows} token rows are not a multiple of n_tok={n_tok}")
    st = L.load().gdn_recurrent_verify(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(g), _ptr(beta), float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, rows // n_tok, n_tok, _ptr(state), state.shape[0], _ptr(state_slots),
        _ptr(checkpoints), checkpoints.shape[1], _ptr(o), _dt(o), _ptr(z), _ptr(norm_w), float(norm_eps),
        _stream(stream))
    L.check("gdn_recurrent_verify", st)
    return o


def gdn_conv1d_verify(x, w, conv_state, y, windows, *, n_tok, state_slots=None, stream=None):
    """Conv + SiLU of n_tok tokens per request from the live histories conv_state [slots, 3, Ch]
    (read only); windows [slots, cols, 3, Ch] receives the history after each token."""
    rows, ch = x.shape
    if rows % n_tok:
        raise ValueError(f"{rows} token rows are not a multiple of n_tok={n_tok}")
    st = L.load().gdn_conv1d_verify(_ptr(x), _dt(x), _ptr(w), ch, rows // n_tok, n_tok, _ptr(conv_state),
                                    conv_state.shape[0], _ptr(state_slots), _ptr(y), _ptr(windows),
                                    windows.shape[1], _stream(stream))
    L.check("gdn_conv1d_verify", st)
    return y


def gdn_state_rows_copy(dst, dst_rows, src=None, src_rows=None, *, stream=None):
    """dst[dst_rows[e]] = src[src_rows[e]] (or zeros when src is None) over rows of the leading
    dimension; dst and src rows must have the same size in bytes."""
    row_bytes = dst[0].numel() * dst.element_size()
    if src is not None and src[0].numel() * src.element_size() != row_bytes:
        raise ValueError("dst and src rows differ in size")
    st = L.load().gdn_state_rows_copy(_ptr(dst), dst.shape[0], _ptr(dst_rows), _ptr(src),
                                      0 if src is None else src.shape[0], _ptr(src_rows), row_bytes,
                                      dst_rows.numel(), _stream(stream))
    L.check("gdn_state_rows_copy", st)
    return dst


def gdn_conv1d_mixed(x, w, conv_state, y, *, cu_seqlens, state_slots, fresh=None, stream=None):
    """Mixed prefill + decode conv1d + SiLU.  x, y [T_cap, Ch]; cu_seqlens [N_cap + 1]
    (cu[N_cap] <= T_cap live rows); state_slots, fresh [N_cap] int32; conv_state
    [slots, 3, Ch] updated in place at each active slot."""
    t_cap, ch = x.shape
    n_seq = cu_seqlens.numel() - 1
    st = L.load().gdn_conv1d_mixed(_ptr(x), _dt(x), _ptr(w), ch, _ptr(cu_seqlens), n_seq, t_cap,
                                   _ptr(conv_state), conv_state.shape[0], _ptr(state_slots), _ptr(fresh),
                                   _ptr(y), _stream(stream))
    L.check("gdn_conv1d_mixed", st)
    return y


def gdn_chunk_mixed(q, k, v, g, beta, state, o, *, chunk, cu_seqlens, state_slots, fresh=None, scale=1.0,
                    use_qk_l2norm=True, l2_eps=1e-6, z=None, norm_w=None, norm_eps=1e-6, workspace=None,
                    stream=None):
    """Mixed prefill + decode gated delta rule over a state pool.  q, k [T_cap, Hqk, dk];
    v [T_cap, Hv, dv]; g, beta [T_cap, Hv]; state [slots, Hv, dv, dk] fp32 updated in
    place at each active slot; o [T_cap, Hv, dv] (rows of inactive sequences and
    padding rows untouched)."""
    t_cap, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n_seq = cu_seqlens.numel() - 1
    if workspace is None:
        nbytes = gdn_chunk_fwd_workspace_size(h_qk, h_v, d_k, d_v, chunk, n_seq, t_cap, q.dtype, z is not None)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.load().gdn_chunk_mixed(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(g), _ptr(beta), float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, chunk, _ptr(cu_seqlens), n_seq, t_cap,
        _ptr(state), state.shape[0], _ptr(state_slots), _ptr(fresh), _ptr(o), _dt(o),
        _ptr(z), _ptr(norm_w), float(norm_eps), _ptr(workspace), workspace.numel(), _stream(stream))
    L.check("gdn_chunk_mixed", st)
    return o


def gdn_chunk_bwd_workspace_size(h_qk, h_v, d_k, d_v, n_seq, t_total) -> int:
    out = ctypes.c_size_t(0)
    st = L.load().gdn_chunk_bwd_workspace_size(h_qk, h_v, d_k, d_v, n_seq, t_total, ctypes.byref(out))
    L.check("gdn_chunk_bwd_workspace_size", st)
    return out.value


def gdn_chunk_bwd(q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta, *, scale=1.0, use_qk_l2norm=True, l2_eps=1e-6,
                  cu_seqlens=None, initial_state=None, d_final=None, d_initial=None, workspace=None, stream=None):
    """Gradients of sum(d_o * o) + sum(d_final * S_T) for the chunked gated delta rule.
    q, k [T, Hqk, dk]; v [T, Hv, dv]; g, beta [T, Hv] fp32; d_o [T, Hv, dv] fp32; outputs
    dq, dk [T, Hqk, dk], dv [T, Hv, dv], dg, dbeta [T, Hv], d_initial [N, Hv, dv, dk], fp32."""
    t_total, h_qk, d_k = q.shape
    h_v, d_v = v.shape[1], v.shape[2]
    n_seq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 1
    if workspace is None:
        nbytes = gdn_chunk_bwd_workspace_size(h_qk, h_v, d_k, d_v, n_seq, t_total)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    st = L.load().gdn_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _rows_view(q, "q"), _rows_view(k, "k"), _rows_view(v, "v"), _dt(q),
        _ptr(g), _ptr(beta), float(scale), int(bool(use_qk_l2norm)), float(l2_eps),
        h_qk, h_v, d_k, d_v, _ptr(cu_seqlens), n_seq, t_total, _ptr(initial_state), _ptr(d_o), _ptr(d_final),
        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(d_initial), _ptr(workspace), workspace.numel(),
        _stream(stream))
    L.check("gdn_chunk_bwd", st)
    return dq, dk, dv, dg, dbeta


def gdn_conv1d_bwd(x, w, dy, dx, dw, *, cu_seqlens=None, conv_state_in=None, d_state_out=None, d_state_in=None,
                   workspace=None, stream=None):
    """Gradients of the width-4 conv + SiLU.  x [T, Ch] (bf16/fp32); w [Ch, 4]; dy, dx [T, Ch] fp32;
    dw [Ch, 4] fp32; histories [N, 3, Ch] (conv_state_in of x's dtype, the gradients fp32)."""
    t_total, ch = x.shape
    n_seq = cu_seqlens.numel() - 1 if cu_seqlens is not None else 1
    if workspace is None:
        out = ctypes.c_size_t(0)
        L.check("gdn_conv1d_bwd_workspace_size",
                L.load().gdn_conv1d_bwd_workspace_size(ch, n_seq, t_total, ctypes.byref(out)))
        workspace = torch.empty(max(out.value, 1), dtype=torch.uint8, device=x.device)
    st = L.load().gdn_conv1d_bwd(_ptr(x), _dt(x), _ptr(w), ch, _ptr(cu_seqlens), n_seq, t_total, _ptr(conv_state_in),
                                 _ptr(dy), _ptr(d_state_out), _ptr(dx), _ptr(dw), _ptr(d_state_in), _ptr(workspace),
                                 workspace.numel(), _stream(stream))
    L.check("gdn_conv1d_bwd", st)
    return dx, dw


def gdn_mixer_decode_step(x, conv_w, conv_state, g, beta, state, o, *, h_qk, scale=1.0, use_qk_l2norm=True,
                          l2_eps=1e-6, state_slots=None, z=None, norm_w=None, norm_eps=1e-6, stream=None):
    """Conv step + recurrent step (+ gated RMSNorm with z) of one decode token per request
    in one launch.  x [N, 2 Hqk dk + Hv dv] raw q|k|v; conv_w [Ch, 4]; conv_state
    [slots, 3, Ch]; state [slots, Hv, dv, dk] fp32; o [N, Hv, dv]."""
    n_req = x.shape[0]
    h_v, d_v, d_k = state.shape[1], state.shape[2], state.shape[3]
    st = L.load().gdn_mixer_decode_step(
        _ptr(x), _dt(x), _ptr(conv_w), _ptr(conv_state), _ptr(g), _ptr(beta), float(scale),
        int(bool(use_qk_l2norm)), float(l2_eps), h_qk, h_v, d_k, d_v, n_req, _ptr(state), state.shape[0],
        _ptr(state_slots), _ptr(o), _dt(o), _ptr(z), _ptr(norm_w), float(norm_eps), _stream(stream))
    L.check("gdn_mixer_decode_step", st)
    return o


def gdn_gated_rmsnorm(x, z, w, y, *, eps=1e-6, stream=None):
    """y = x / sqrt(mean(x^2) + eps) * w * SiLU(z) over the last dim (16 or 128)."""
    d = x.shape[-1]
    rows = x.numel() // d
    st = L.load().gdn_gated_rmsnorm(_ptr(x), _dt(x), _ptr(z), _dt(z), _ptr(w), float(eps), rows, d,
                                    _ptr(y), _dt(y), _stream(stream))
    L.check("gdn_gated_rmsnorm", st)
    return y


def qkv_views(y_conv: torch.Tensor, h_qk: int, d_k: int, h_v: int, d_v: int):
    """q, k, v views of a conv output [T, Ch] (channels q | k | v), no copies."""
    t = y_conv.shape[0]
    nq = h_qk * d_k
    ch = y_conv.shape[1]
    q = y_conv.as_strided((t, h_qk, d_k), (ch, d_k, 1), y_conv.storage_offset())
    k = y_conv.as_strided((t, h_qk, d_k), (ch, d_k, 1), y_conv.storage_offset() + nq)
    v = y_conv.as_strided((t, h_v, d_v), (ch, d_v, 1), y_conv.storage_offset() + 2 * nq)
    return q, k, v
