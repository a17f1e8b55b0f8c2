"""Host-side checks of the C ABI: the library loads, exports every function
include/gdn.h declares, and rejects invalid calls before launching anything.

No call here reaches a kernel: every one is rejected by host validation
(device pointers are fake integers that are never dereferenced) or is a
documented no-op, so this runs without a GPU.
"""
import ctypes
import os
import re

import pytest

from gated_deltanet_mixer_causal_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def lib():
    return L.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_\w+)\s*\(", text)))


def test_header_functions_exported(lib):
    names = _declared()
    assert set(names) == set(L.PROTOTYPES), names
    for n in names:
        assert hasattr(lib, n)


def test_status_strings(lib):
    for s in range(8):
        assert lib.gdn_status_string(s).decode().startswith(L.STATUS_NAMES[s])
    assert b"unknown" in lib.gdn_status_string(99)
    assert lib.gdn_last_hip_error() == 0
    assert b"gfx950" in lib.gdn_version()


A = 0x10000000  # fake, 16-byte aligned device addresses spaced far apart


def _addr(i):
    return A * (i + 1)


def conv(lib, **kw):
    a = dict(x=_addr(0), dt=L.GDN_BF16, w=_addr(1), ch=1024, cu=_addr(2), n=2, t=10, st=_addr(3), ns=2,
             sl=None, y=_addr(4))
    a.update(kw)
    return lib.gdn_conv1d_fwd(a["x"], a["dt"], a["w"], a["ch"], a["cu"], a["n"], a["t"], a["st"], a["ns"],
                              a["sl"], a["y"], None)


def test_conv_validation(lib):
    assert conv(lib, n=0) == L.GDN_OK                       # no-op
    assert conv(lib, n=-1) == L.GDN_ERR_INVALID
    assert conv(lib, ch=12) == L.GDN_ERR_INVALID             # not a multiple of 8
    assert conv(lib, dt=5) == L.GDN_ERR_UNSUPPORTED
    assert conv(lib, w=None) == L.GDN_ERR_NULL
    assert conv(lib, st=None) == L.GDN_ERR_NULL
    assert conv(lib, cu=None, t=3, n=2) == L.GDN_ERR_INVALID  # decode needs t_total == n_seq
    assert conv(lib, ns=1) == L.GDN_ERR_INVALID              # identity slots need n_slots >= n_seq
    assert conv(lib, x=_addr(0) + 4) == L.GDN_ERR_ALIGN
    assert conv(lib, y=_addr(0) + 16) == L.GDN_ERR_ALIAS     # y overlaps x
    assert conv(lib, st=_addr(4) + 32) == L.GDN_ERR_ALIAS    # state overlaps y


def chunk(lib, **kw):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), qs=0, ks=0, vs=0, dt=L.GDN_BF16, g=_addr(3), b=_addr(4),
             hq=2, hv=4, dk=128, dv=128, c=64, cu=_addr(5), n=1, t=100, init=None, fin=_addr(6), o=_addr(7),
             odt=L.GDN_F32, z=None, nw=None, ws=_addr(8), wsb=1 << 26)
    a.update(kw)
    return lib.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["dt"], a["g"], a["b"], 1.0, 1,
                             1e-6, a["hq"], a["hv"], a["dk"], a["dv"], a["c"], a["cu"], a["n"], a["t"], a["init"],
                             a["fin"], a["o"], a["odt"], a["z"], a["nw"], 1e-6, a["ws"], a["wsb"], None)


def test_chunk_validation(lib):
    assert chunk(lib, n=0) == L.GDN_OK
    assert chunk(lib, t=-1) == L.GDN_ERR_INVALID
    assert chunk(lib, q=None) == L.GDN_ERR_NULL
    assert chunk(lib, o=None) == L.GDN_ERR_NULL
    assert chunk(lib, ws=None) == L.GDN_ERR_WORKSPACE
    assert chunk(lib, wsb=1024) == L.GDN_ERR_WORKSPACE
    assert chunk(lib, hv=3) == L.GDN_ERR_INVALID             # h_v % h_qk
    assert chunk(lib, dk=64, dv=64) == L.GDN_ERR_UNSUPPORTED
    assert chunk(lib, c=32) == L.GDN_ERR_UNSUPPORTED
    assert chunk(lib, dk=16, dv=16, c=16) == L.GDN_ERR_UNSUPPORTED   # bf16 needs the 128/64 shape
    assert chunk(lib, odt=9) == L.GDN_ERR_UNSUPPORTED
    assert chunk(lib, qs=100) == L.GDN_ERR_INVALID           # stride below a row
    assert chunk(lib, qs=260) == L.GDN_ERR_ALIGN             # stride not a multiple of 8
    assert chunk(lib, vs=(1 << 24) + 8) == L.GDN_ERR_INVALID  # stride above 2^24 elements
    assert chunk(lib, g=_addr(3) + 8) == L.GDN_ERR_ALIGN
    assert chunk(lib, z=_addr(9)) == L.GDN_ERR_NULL          # z without norm weight
    assert chunk(lib, cu=None, n=2) == L.GDN_ERR_NULL        # NULL cu_seqlens only for one sequence
    assert chunk(lib, o=_addr(0) + 4096) == L.GDN_ERR_ALIAS  # o overlaps q
    assert chunk(lib, fin=_addr(8) + 256) == L.GDN_ERR_ALIAS  # final state inside the workspace
    assert chunk(lib, init=_addr(6) + 64) == L.GDN_ERR_ALIAS  # partial overlap of the states


def conv_mixed(lib, **kw):
    a = dict(x=_addr(0), dt=L.GDN_BF16, w=_addr(1), ch=1024, cu=_addr(2), n=2, t=10, st=_addr(3), ns=4,
             sl=_addr(5), fr=_addr(6), y=_addr(4))
    a.update(kw)
    return lib.gdn_conv1d_mixed(a["x"], a["dt"], a["w"], a["ch"], a["cu"], a["n"], a["t"], a["st"], a["ns"],
                                a["sl"], a["fr"], a["y"], None)


def test_conv_mixed_validation(lib):
    assert conv_mixed(lib, n=0) == L.GDN_OK
    assert conv_mixed(lib, ns=-1) == L.GDN_ERR_INVALID
    assert conv_mixed(lib, cu=None) == L.GDN_ERR_NULL        # the mixed form always takes cu_seqlens
    assert conv_mixed(lib, sl=None) == L.GDN_ERR_NULL        # ... and an explicit slot map
    assert conv_mixed(lib, fr=_addr(6) + 4) == L.GDN_ERR_ALIGN
    assert conv_mixed(lib, y=_addr(5)) == L.GDN_ERR_ALIAS    # y over the slot map
    assert conv_mixed(lib, st=_addr(6) - 16) == L.GDN_ERR_ALIAS   # history pool over the fresh flags


def chunk_mixed(lib, **kw):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), qs=0, ks=0, vs=0, dt=L.GDN_BF16, g=_addr(3), b=_addr(4),
             hq=2, hv=4, dk=128, dv=128, c=64, cu=_addr(5), n=3, t=100, st=_addr(6), ns=8, sl=_addr(9),
             fr=_addr(10), o=_addr(7), odt=L.GDN_F32, z=None, nw=None, ws=_addr(8), wsb=1 << 26)
    a.update(kw)
    return lib.gdn_chunk_mixed(a["q"], a["k"], a["v"], a["qs"], a["ks"], a["vs"], a["dt"], a["g"], a["b"], 1.0,
                               1, 1e-6, a["hq"], a["hv"], a["dk"], a["dv"], a["c"], a["cu"], a["n"], a["t"],
                               a["st"], a["ns"], a["sl"], a["fr"], a["o"], a["odt"], a["z"], a["nw"], 1e-6, a["ws"],
                               a["wsb"], None)


def test_chunk_mixed_validation(lib):
    assert chunk_mixed(lib, n=0) == L.GDN_OK
    assert chunk_mixed(lib, ns=-2) == L.GDN_ERR_INVALID
    assert chunk_mixed(lib, cu=None) == L.GDN_ERR_NULL
    assert chunk_mixed(lib, sl=None) == L.GDN_ERR_NULL
    assert chunk_mixed(lib, st=None) == L.GDN_ERR_NULL
    assert chunk_mixed(lib, wsb=1024) == L.GDN_ERR_WORKSPACE
    assert chunk_mixed(lib, sl=_addr(9) + 8) == L.GDN_ERR_ALIGN
    assert chunk_mixed(lib, o=_addr(9)) == L.GDN_ERR_ALIAS   # o over the slot map
    # the pool spans n_slots rows of 4 x 128 x 128 fp32 (2 MiB): one ending inside the fresh flags
    pool = 8 * 4 * 128 * 128 * 4
    assert chunk_mixed(lib, st=_addr(10) - pool + 16) == L.GDN_ERR_ALIAS


def chunk_bwd(lib, **kw):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dt=L.GDN_BF16, g=_addr(3), b=_addr(4), hq=2, hv=4, d=128,
             cu=_addr(5), n=2, t=100, init=None, do=_addr(6), dfin=None, dq=_addr(7), dk=_addr(8), dv=_addr(9),
             dg=_addr(10), db=_addr(11), dinit=None, ws=_addr(12), wsb=1 << 30)
    a.update(kw)
    return lib.gdn_chunk_bwd(a["q"], a["k"], a["v"], 0, 0, 0, a["dt"], a["g"], a["b"], 1.0, 1, 1e-6, a["hq"], a["hv"],
                             a["d"], a["d"], a["cu"], a["n"], a["t"], a["init"], a["do"], a["dfin"], a["dq"], a["dk"],
                             a["dv"], a["dg"], a["db"], a["dinit"], a["ws"], a["wsb"], None)


def test_chunk_bwd_validation(lib):
    assert chunk_bwd(lib, n=0) == L.GDN_OK
    assert chunk_bwd(lib, t=-1) == L.GDN_ERR_INVALID
    assert chunk_bwd(lib, g=None) == L.GDN_ERR_NULL
    assert chunk_bwd(lib, do=None) == L.GDN_ERR_NULL
    assert chunk_bwd(lib, dg=None) == L.GDN_ERR_NULL
    assert chunk_bwd(lib, cu=None) == L.GDN_ERR_NULL            # several sequences need cu_seqlens
    assert chunk_bwd(lib, d=16) == L.GDN_ERR_UNSUPPORTED        # bf16 needs d = 128
    assert chunk_bwd(lib, d=64, dt=L.GDN_F32) == L.GDN_ERR_UNSUPPORTED
    assert chunk_bwd(lib, ws=None) == L.GDN_ERR_WORKSPACE
    assert chunk_bwd(lib, wsb=4096) == L.GDN_ERR_WORKSPACE
    assert chunk_bwd(lib, dq=_addr(7) + 4) == L.GDN_ERR_ALIGN
    assert chunk_bwd(lib, dq=_addr(0)) == L.GDN_ERR_ALIAS       # dq over q
    assert chunk_bwd(lib, dk=_addr(7) + 1024) == L.GDN_ERR_ALIAS   # dk over dq
    out = ctypes.c_size_t(0)
    assert lib.gdn_chunk_bwd_workspace_size(16, 32, 128, 128, 1, 4096, ctypes.byref(out)) == 0
    slots = 4096 // 16 + 1
    expect = slots * 32 * 128 * 128 * 4 + 2 * 4096 * 32 * 8 * 128 * 4 + 2 * 4096 * 32 * 8 * 4
    assert out.value == expect


def test_conv1d_bwd_validation(lib):
    def call(**kw):
        a = dict(x=_addr(0), dt=L.GDN_BF16, w=_addr(1), ch=1024, cu=_addr(2), n=2, t=10, h=None, dy=_addr(3),
                 dho=None, dx=_addr(4), dw=_addr(5), dhi=None, ws=_addr(6), wsb=1 << 24)
        a.update(kw)
        return lib.gdn_conv1d_bwd(a["x"], a["dt"], a["w"], a["ch"], a["cu"], a["n"], a["t"], a["h"], a["dy"],
                                  a["dho"], a["dx"], a["dw"], a["dhi"], a["ws"], a["wsb"], None)
    assert call(n=0) == L.GDN_OK
    assert call(ch=12) == L.GDN_ERR_INVALID
    assert call(dw=None) == L.GDN_ERR_NULL
    assert call(dy=None) == L.GDN_ERR_NULL
    assert call(ws=None) == L.GDN_ERR_WORKSPACE
    assert call(wsb=16) == L.GDN_ERR_WORKSPACE
    assert call(dx=_addr(3)) == L.GDN_ERR_ALIAS                 # dx over dy
    out = ctypes.c_size_t(0)
    assert lib.gdn_conv1d_bwd_workspace_size(8192, 1, 4096, ctypes.byref(out)) == 0
    assert out.value == (4096 // 32 + 1) * 8192 * 4 * 4   # one dw partial per 32-token strip


def test_chunk_workspace_size(lib):
    out = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(16, 32, 128, 128, 64, 1, 4096, L.GDN_BF16, 0, ctypes.byref(out)) == 0
    slots = 4096 // 64 + 1
    # per q/k head: K and Q fragments (bf16); per v-head: Tb and P as bf16 hi+lo,
    # fp32 scalars (the bf16 scan builds K^T from K in LDS)
    expect = (slots * 16 * 2 * 64 * 128 * 2 + 2 * slots * 32 * 2 * 64 * 64 * 2 + slots * 32 * 4 * 64 * 4)
    assert out.value == expect
    assert lib.gdn_chunk_fwd_workspace_size(16, 32, 128, 128, 64, 1, 4096, L.GDN_BF16, 1, ctypes.byref(out)) == 0
    assert out.value == expect + 4096 * 32 * 128 * 4
    # several sequences: one slot more per sequence, and the longest-first order (int32 each)
    assert lib.gdn_chunk_fwd_workspace_size(16, 32, 128, 128, 64, 8, 4096, L.GDN_BF16, 0, ctypes.byref(out)) == 0
    slots = 4096 // 64 + 8
    expect = (slots * 16 * 2 * 64 * 128 * 2 + 2 * slots * 32 * 2 * 64 * 64 * 2 + slots * 32 * 4 * 64 * 4 + 256)
    assert out.value == expect
    assert lib.gdn_chunk_fwd_workspace_size(16, 32, 128, 128, 64, 1, 4096, L.GDN_BF16, 0, None) == L.GDN_ERR_NULL
    assert lib.gdn_chunk_fwd_workspace_size(16, 32, 64, 64, 64, 1, 4096, L.GDN_BF16, 0,
                                            ctypes.byref(out)) == L.GDN_ERR_UNSUPPORTED


def step(lib, **kw):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dt=L.GDN_BF16, g=_addr(3), b=_addr(4), hq=2, hv=4, d=128,
             n=3, st=_addr(5), ns=3, sl=None, o=_addr(6), odt=L.GDN_F32, z=None, nw=None)
    a.update(kw)
    return lib.gdn_recurrent_step(a["q"], a["k"], a["v"], 0, 0, 0, a["dt"], a["g"], a["b"], 1.0, 1, 1e-6,
                                  a["hq"], a["hv"], a["d"], a["d"], a["n"], a["st"], a["ns"], a["sl"], a["o"],
                                  a["odt"], a["z"], a["nw"], 1e-6, None)


def test_recurrent_validation(lib):
    assert step(lib, n=0) == L.GDN_OK
    assert step(lib, n=-2) == L.GDN_ERR_INVALID
    assert step(lib, st=None) == L.GDN_ERR_NULL
    assert step(lib, d=64) == L.GDN_ERR_UNSUPPORTED
    assert step(lib, ns=2) == L.GDN_ERR_INVALID
    assert step(lib, o=_addr(5) + 1024) == L.GDN_ERR_ALIAS    # o inside the state
    assert step(lib, st=_addr(4) + 16) == L.GDN_ERR_ALIAS     # state overlaps beta
    assert step(lib, o=_addr(6) + 8) == L.GDN_ERR_ALIGN


def norm(lib, **kw):
    a = dict(x=_addr(0), xdt=L.GDN_F32, z=_addr(1), zdt=L.GDN_BF16, w=_addr(2), rows=10, d=128, y=_addr(3),
             ydt=L.GDN_F32)
    a.update(kw)
    return lib.gdn_gated_rmsnorm(a["x"], a["xdt"], a["z"], a["zdt"], a["w"], 1e-6, a["rows"], a["d"], a["y"],
                                 a["ydt"], None)


def test_norm_validation(lib):
    assert norm(lib, rows=0) == L.GDN_OK
    assert norm(lib, rows=-1) == L.GDN_ERR_INVALID
    assert norm(lib, d=64) == L.GDN_ERR_UNSUPPORTED
    assert norm(lib, z=None) == L.GDN_ERR_NULL
    assert norm(lib, y=_addr(0) + 16) == L.GDN_ERR_ALIAS      # partial overlap with x
    assert norm(lib, y=_addr(1)) == L.GDN_ERR_ALIAS           # y over z
    assert norm(lib, w=_addr(2) + 4) == L.GDN_ERR_ALIGN


def chunk_gated(lib, **kw):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dt=L.GDN_BF16, ga=_addr(3), gb=_addr(4), abs=0,
             abdt=L.GDN_BF16, alog=_addr(10), bias=None, hq=2, hv=4, c=64, cu=_addr(5), n=1, t=100,
             fin=_addr(6), o=_addr(7), ws=_addr(8), wsb=1 << 26)
    a.update(kw)
    return lib.gdn_chunk_fwd_gated(a["q"], a["k"], a["v"], 0, 0, 0, a["dt"], a["ga"], a["gb"], a["abs"], a["abdt"],
                                   a["alog"], a["bias"], 1.0, 1, 1e-6, a["hq"], a["hv"], 128, 128, a["c"], a["cu"],
                                   a["n"], a["t"], None, a["fin"], a["o"], L.GDN_F32, None, None, 1e-6, a["ws"],
                                   a["wsb"], None)


def test_chunk_gated_validation(lib):
    assert chunk_gated(lib, n=0) == L.GDN_OK
    assert chunk_gated(lib, ga=None) == L.GDN_ERR_NULL           # a missing
    assert chunk_gated(lib, gb=None) == L.GDN_ERR_NULL           # b missing
    assert chunk_gated(lib, alog=None) == L.GDN_ERR_NULL         # a_log is always required
    assert chunk_gated(lib, abdt=7) == L.GDN_ERR_UNSUPPORTED
    assert chunk_gated(lib, abs=3) == L.GDN_ERR_INVALID          # row stride below h_v
    assert chunk_gated(lib, ga=_addr(3) + 1) == L.GDN_ERR_ALIGN  # bf16 needs 2-byte alignment
    assert chunk_gated(lib, abdt=L.GDN_F32, gb=_addr(4) + 2) == L.GDN_ERR_ALIGN
    assert chunk_gated(lib, alog=_addr(10) + 2) == L.GDN_ERR_ALIGN
    assert chunk_gated(lib, bias=_addr(11) + 1) == L.GDN_ERR_ALIGN
    assert chunk_gated(lib, o=_addr(3) + 64) == L.GDN_ERR_ALIAS  # o overlaps a
    assert chunk_gated(lib, ws=_addr(10) - 64) == L.GDN_ERR_ALIAS   # workspace covers a_log
    assert chunk_gated(lib, fin=_addr(11), bias=_addr(11) + 16) == L.GDN_ERR_ALIAS  # state over dt_bias
    # a packed [t, 2 h_v] b|a tensor: a starts h_v bf16 elements (8 bytes) into the row
    assert chunk_gated(lib, ga=_addr(3) + 8, gb=_addr(3), abs=8, o=None) == L.GDN_ERR_NULL   # gets past gate checks


def step_gated(lib, **kw):
    a = dict(ga=_addr(3), gb=_addr(4), abs=0, abdt=L.GDN_F32, alog=_addr(10), bias=None, n=3, st=_addr(5),
             o=_addr(6))
    a.update(kw)
    return lib.gdn_recurrent_step_gated(_addr(0), _addr(1), _addr(2), 0, 0, 0, L.GDN_BF16, a["ga"], a["gb"], a["abs"],
                                        a["abdt"], a["alog"], a["bias"], 1.0, 1, 1e-6, 2, 4, 128, 128, a["n"],
                                        a["st"], 3, None, a["o"], L.GDN_F32, None, None, 1e-6, None)


def test_recurrent_gated_validation(lib):
    assert step_gated(lib, n=0) == L.GDN_OK
    assert step_gated(lib, ga=None) == L.GDN_ERR_NULL
    assert step_gated(lib, alog=None) == L.GDN_ERR_NULL
    assert step_gated(lib, abs=2) == L.GDN_ERR_INVALID
    assert step_gated(lib, gb=_addr(4) + 2) == L.GDN_ERR_ALIGN
    assert step_gated(lib, st=_addr(3) + 16) == L.GDN_ERR_ALIAS   # state overlaps a
    assert step_gated(lib, o=_addr(10) - 16) == L.GDN_ERR_ALIAS   # o overlaps a_log


def verify(lib, **kw):
    a = dict(g=_addr(3), n=3, w=4, st=_addr(5), ns=3, sl=None, ck=_addr(9), nc=8, o=_addr(6), z=None, nw=None)
    a.update(kw)
    return lib.gdn_recurrent_verify(_addr(0), _addr(1), _addr(2), 0, 0, 0, L.GDN_BF16, a["g"], _addr(4), 1.0, 1,
                                    1e-6, 2, 4, 128, 128, a["n"], a["w"], a["st"], a["ns"], a["sl"], a["ck"], a["nc"],
                                    a["o"], L.GDN_F32, a["z"], a["nw"], 1e-6, None)


def test_verify_validation(lib):
    assert verify(lib, n=0) == L.GDN_OK
    assert verify(lib, w=0) == L.GDN_ERR_INVALID              # no tokens
    assert verify(lib, w=9) == L.GDN_ERR_INVALID              # more tokens than checkpoint columns
    assert verify(lib, ck=None) == L.GDN_ERR_NULL
    assert verify(lib, g=None) == L.GDN_ERR_NULL
    assert verify(lib, ns=2) == L.GDN_ERR_INVALID             # identity slots need n_slots >= n_req
    assert verify(lib, ck=_addr(9) + 8) == L.GDN_ERR_ALIGN
    assert verify(lib, ck=_addr(5) + 1024) == L.GDN_ERR_ALIAS  # checkpoints inside the live states
    assert verify(lib, o=_addr(9) + 4096) == L.GDN_ERR_ALIAS   # outputs inside the checkpoints


def conv_verify(lib, **kw):
    a = dict(n=2, w=3, st=_addr(3), ns=2, y=_addr(4), win=_addr(5), nc=8)
    a.update(kw)
    return lib.gdn_conv1d_verify(_addr(0), L.GDN_BF16, _addr(1), 1024, a["n"], a["w"], a["st"], a["ns"], None,
                                 a["y"], a["win"], a["nc"], None)


def test_conv_verify_validation(lib):
    assert conv_verify(lib, n=0) == L.GDN_OK
    assert conv_verify(lib, w=0) == L.GDN_ERR_INVALID
    assert conv_verify(lib, w=9) == L.GDN_ERR_INVALID
    assert conv_verify(lib, win=None) == L.GDN_ERR_NULL
    assert conv_verify(lib, ns=1) == L.GDN_ERR_INVALID
    assert conv_verify(lib, win=_addr(3) + 64) == L.GDN_ERR_ALIAS   # windows over the live histories
    assert conv_verify(lib, y=_addr(5) + 16) == L.GDN_ERR_ALIAS     # outputs inside the windows


def rows_copy(lib, **kw):
    a = dict(dst=_addr(0), nd=4, dr=_addr(1), src=_addr(2), ns=8, sr=_addr(3), rb=1 << 20, n=2)
    a.update(kw)
    return lib.gdn_state_rows_copy(a["dst"], a["nd"], a["dr"], a["src"], a["ns"], a["sr"], a["rb"], a["n"], None)


def test_rows_copy_validation(lib):
    assert rows_copy(lib, n=0) == L.GDN_OK
    assert rows_copy(lib, n=-1) == L.GDN_ERR_INVALID
    assert rows_copy(lib, rb=0) == L.GDN_ERR_INVALID
    assert rows_copy(lib, rb=1000) == L.GDN_ERR_ALIGN            # rows of a whole number of 16-byte units
    assert rows_copy(lib, dr=None) == L.GDN_ERR_NULL
    assert rows_copy(lib, sr=None) == L.GDN_ERR_NULL             # a source needs its rows
    assert rows_copy(lib, dst=_addr(0) + 8) == L.GDN_ERR_ALIGN
    assert rows_copy(lib, dr=_addr(0) + 4096) == L.GDN_ERR_ALIAS  # index array inside the destination
    assert rows_copy(lib, src=_addr(0) + (1 << 20)) == L.GDN_ERR_ALIAS   # partial overlap of two pools


def mixer_step(lib, **kw):
    a = dict(x=_addr(0), dt=L.GDN_BF16, w=_addr(1), cs=_addr(2), g=_addr(3), b=_addr(4), hq=2, hv=4, d=128, n=4,
             st=_addr(5), ns=4, sl=None, o=_addr(6), odt=L.GDN_F32, z=None, nw=None)
    a.update(kw)
    return lib.gdn_mixer_decode_step(a["x"], a["dt"], a["w"], a["cs"], a["g"], a["b"], 1.0, 1, 1e-6, a["hq"],
                                     a["hv"], a["d"], a["d"], a["n"], a["st"], a["ns"], a["sl"], a["o"], a["odt"],
                                     a["z"], a["nw"], 1e-6, None)


def test_mixer_decode_validation(lib):
    assert mixer_step(lib, n=0) == L.GDN_OK
    assert mixer_step(lib, n=-1) == L.GDN_ERR_INVALID
    assert mixer_step(lib, hv=5) == L.GDN_ERR_INVALID           # h_v not a multiple of h_qk
    assert mixer_step(lib, d=16) == L.GDN_ERR_UNSUPPORTED       # the fused form is for 128-wide heads
    assert mixer_step(lib, hq=1, hv=16) == L.GDN_ERR_UNSUPPORTED  # group above 8
    assert mixer_step(lib, ns=2) == L.GDN_ERR_INVALID           # identity slots need n_slots >= n_req
    assert mixer_step(lib, cs=None) == L.GDN_ERR_NULL
    assert mixer_step(lib, z=_addr(7)) == L.GDN_ERR_NULL        # z without norm_w
    assert mixer_step(lib, sl=_addr(8) + 2) == L.GDN_ERR_ALIGN
    assert mixer_step(lib, o=_addr(5) + 4096) == L.GDN_ERR_ALIAS   # o inside the state
    assert mixer_step(lib, cs=_addr(0) + 256) == L.GDN_ERR_ALIAS   # history pool over x
    assert mixer_step(lib, st=_addr(2) + 64) == L.GDN_ERR_ALIAS    # state over the history pool
