"""The C ABI on the host: the library loads, exports every declared entry point,
and rejects bad arguments before enqueueing anything (no GPU needed: every
call below fails validation, so no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hga.h")

hga = pytest.importorskip("sparse_long_context_hga_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hga.LIB_PATH):
        pytest.fail("libhga.so not built (run __graft_entry__.build())")
    return hga.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hga_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert set(names) == {"hga_build_summaries", "hga_forward", "hga_forward_causal", "hga_stage_history",
                          "hga_stage_history_min",
                          "hga_route", "hga_route_causal", "hga_attend_fwd",
                          "hga_attend_bwd_workspace_size", "hga_attend_bwd", "hga_attend_bwd_timed",
                          "hga_decode_step", "hga_decode_route", "hga_decode_attend", "hga_decode_workspace_size",
                          "hga_decode_step_noalloc",
                          "hga_status_string"}
    for n in names:
        assert hasattr(L, n), n
        assert n in hga._lib.SIGNATURES


def test_status_strings(L):
    for code in range(-7, 1):
        assert hga.hga_status_string(code) not in ("", "unknown status")
    assert hga.hga_status_string(-99) == "unknown status"


def _shape(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, top_chunks=16, top_groups=64,
                dtype="bf16")
    base.update(kw)
    return hga.make_shape(**base)


A = ctypes.c_void_p(0x10000)   # fake, aligned, never dereferenced (every call fails validation)
M = ctypes.c_void_p(0x10008)   # fake, misaligned


def _route(L, s, t_cap=16384, t_hist=14336, seg=2048, q=A, cidx=A, gidx=A):
    return L.hga_route(ctypes.byref(s) if s is not None else None, q, A, A, t_cap, t_hist, seg, cidx, gidx,
                       None, None, None)


def test_route_validation(L):
    assert _route(L, None) == -1
    assert _route(L, _shape(), q=None) == -1
    assert _route(L, _shape(), cidx=None) == -1
    assert _route(L, _shape(n_q_heads=24)) == -3            # G = 3
    assert _route(L, _shape(n_q_heads=30)) == -2            # not a multiple
    assert _route(L, _shape(head_dim=96)) == -3
    assert _route(L, _shape(top_chunks=65, top_groups=64)) == -3
    assert _route(L, _shape(top_groups=129)) == -2          # > 8 * top_chunks
    assert _route(L, _shape(top_chunks=-1)) == -2
    assert _route(L, _shape(), t_hist=100) == -2
    assert _route(L, _shape(), seg=0) == -2
    assert _route(L, _shape(), t_hist=16384) == -4          # beyond t_cap
    assert _route(L, _shape(), t_cap=1 << 20, t_hist=(1 << 19), seg=2048) == -3   # > max chunks
    assert _route(L, _shape(), q=M) == -5
    s = _shape()
    s.chunk = 32
    assert _route(L, s) == -3
    s = _shape()
    s.dtype = 7
    assert _route(L, s) == -3
    s = _shape()
    s.softmax_scale = float("nan")
    assert _route(L, s) == -2


def test_route_causal_validation(L):
    s = _shape()
    f = L.hga_route_causal

    def call(q_prev=A, t_hist=14336, q=A, shape=s):
        return f(ctypes.byref(shape), q, q_prev, A, A, 16384, t_hist, 2048, A, A, None, None, None)
    assert call(q_prev=None) == -1                    # history present: the previous block is needed
    assert call(q_prev=M) == -5
    assert call(q=None) == -1
    assert call(t_hist=100) == -2
    assert call(shape=_shape(n_q_heads=24)) == -3
    assert f(None, A, A, A, A, 16384, 0, 2048, A, A, None, None, None) == -1


def test_forward_validation(L):
    """hga_forward and hga_forward_causal (the causal one also needs q_prev over history)."""
    s = _shape()

    def fwd(q=A, k=A, cs=A, t_cap=16384, t_hist=14336, seg=2048, cidx=A, gidx=A, o=A, shape=s):
        return L.hga_forward(ctypes.byref(shape) if shape is not None else None, q, k, A, cs, A, t_cap, t_hist,
                             seg, cidx, gidx, o, A, None, None)

    def fwdc(q_prev=A, q=A, k=A, t_hist=14336, seg=2048, gidx=A, shape=s):
        return L.hga_forward_causal(ctypes.byref(shape), q, q_prev, k, A, A, A, 16384, t_hist, seg, A, gidx, A, A,
                                    None, None)
    for f in (fwd, fwdc):
        assert f(q=None) == -1
        assert f(k=None) == -1
        assert f(gidx=None) == -1
        assert f(q=M) == -5
        assert f(k=M) == -5
        assert f(t_hist=100) == -2
        assert f(seg=0) == -2
        assert f(shape=_shape(n_q_heads=24)) == -3
        assert f(shape=_shape(top_groups=129)) == -2
    assert fwd(shape=None) == -1
    assert fwd(cs=None) == -1
    assert fwd(cidx=None) == -1
    assert fwd(o=None) == -1
    assert fwd(t_hist=16384) == -4
    assert fwd(t_cap=1 << 20, t_hist=1 << 19) == -3        # more chunks than the router takes
    assert fwdc(q_prev=None) == -1                          # history present: the previous block is needed
    assert fwdc(q_prev=M) == -5


def test_summaries_validation(L):
    s = _shape()
    f = L.hga_build_summaries
    assert f(None, A, 16384, 0, 64, A, A, None) == -1
    assert f(ctypes.byref(s), A, 16384, 32, 64, A, A, None) == -2
    assert f(ctypes.byref(s), A, 16384, 128, 64, A, A, None) == -2
    assert f(ctypes.byref(s), A, 16384, 0, 16448, A, A, None) == -4
    assert f(ctypes.byref(s), None, 16384, 0, 64, A, A, None) == -1
    assert f(ctypes.byref(s), M, 16384, 0, 64, A, A, None) == -5
    assert f(ctypes.byref(s), None, 16384, 64, 64, None, None, None) == 0   # empty range: no-op


def test_attend_validation(L):
    s = _shape()
    fw = L.hga_attend_fwd
    assert fw(ctypes.byref(s), A, A, A, 16384, 14336, 2048, None, A, A, None) == -1   # group_idx needed
    assert fw(ctypes.byref(s), A, A, A, 16384, 14336, 4096, A, A, A, None) == -4
    assert fw(ctypes.byref(s), A, A, M, 16384, 14336, 2048, A, A, A, None) == -5
    need = hga.hga_attend_bwd_workspace_size(s, 14336, 2048)
    assert need >= 32 * 2048 * 4 and need % 256 == 0
    bw = L.hga_attend_bwd
    args = [A, A, A, A, A, A, 16384, 14336, 2048, A, A, A, A]
    assert bw(ctypes.byref(s), *args, A, need - 1, None) == -6
    assert bw(ctypes.byref(s), *args, None, need, None) == -6
    assert bw(ctypes.byref(s), *args[:-1], None, A, need, None) == -1
    args_m = list(args)
    args_m[5] = M
    assert bw(ctypes.byref(s), *args_m, A, need, None) == -5
    big = hga.hga_attend_bwd_workspace_size(s, 0, 64 * 1025)
    assert bw(ctypes.byref(s), A, A, A, A, A, A, 1 << 17, 0, 64 * 1025, A, A, A, A, A, big, None) == -3
    assert hga.hga_attend_bwd_workspace_size(_shape(head_dim=80), 0, 64) == 0
    tw = L.hga_attend_bwd_timed
    assert tw(ctypes.byref(s), *args, A, need, None, None) == -1                # events required
    ev = (ctypes.c_void_p * 8)()
    assert tw(ctypes.byref(s), *args, A, need - 1, ev, None) == -6


def test_decode_validation(L):
    s = _shape(batch=8)
    need = hga.hga_decode_workspace_size(s, 32768)
    assert need >= 8 * 8 * 512 * 4 and need % 256 == 0
    assert hga.hga_decode_workspace_size(_shape(head_dim=80), 32768) == 0
    assert hga.hga_decode_workspace_size(s, 100) == 0
    r = L.hga_decode_route

    def route(shape=s, t_cap=32768, q=A, pos=A, cidx=A, ws=A, nbytes=need):
        return r(ctypes.byref(shape) if shape is not None else None, q, A, A, t_cap, pos, cidx, A, None, None,
                 ws, nbytes, None)
    assert route(shape=None) == -1
    assert route(pos=None) == -1
    assert route(cidx=None) == -1
    assert route(q=M) == -5
    assert route(ws=None) == -6
    assert route(nbytes=need - 1) == -6
    assert route(ws=M) == -5
    assert route(t_cap=100) == -2
    assert route(t_cap=64 * 8193, nbytes=1 << 40) == -3
    assert route(shape=_shape(n_q_heads=24)) == -3
    at = L.hga_decode_attend

    def attend(gsum=None, csum=None, k=A, lse=A, gidx=A, nbytes=need):
        return at(ctypes.byref(s), A, k, A, 32768, A, gidx, A, lse, gsum, csum, A, nbytes, None)
    assert attend(k=None) == -1
    assert attend(lse=None) == -1
    assert attend(gidx=None) == -1
    assert attend(gsum=A) == -1                       # summaries: both or neither
    assert attend(gsum=A, csum=M) == -5
    assert attend(nbytes=0) == -6
    st = L.hga_decode_step

    def step(csum=A, o=A, cidx=None, gidx=A, t_cap=32768, nbytes=need):
        return st(ctypes.byref(s), A, A, A, csum, A, t_cap, A, cidx, gidx, o, A, A, nbytes, None)
    assert step(csum=None) == -1
    assert step(o=None) == -1
    assert step(gidx=None) == -1
    assert step(cidx=M) == -5
    assert step(nbytes=need - 1) == -6
    assert step(t_cap=64 * 8193, nbytes=1 << 40) == -3


def test_decode_noalloc_validation(L):
    """The entry point that allocates nothing rejects, before touching the device,
    calls that need more than its static scratch holds."""
    s = _shape(batch=8)
    assert L.hga_decode_step_noalloc(None, A, A, A, A, A, 8192, A, A, A, A, A, None) == -1
    assert L.hga_decode_step_noalloc(ctypes.byref(s), None, A, A, A, A, 8192, A, A, A, A, A, None) == -1
    assert L.hga_decode_step_noalloc(ctypes.byref(s), M, A, A, A, A, 8192, A, A, A, A, A, None) == -5
    big = _shape(batch=4096)                       # 32,768 (sequence, KV head) units: too many counters
    assert L.hga_decode_step_noalloc(ctypes.byref(big), A, A, A, A, A, 8192, A, A, A, A, A, None) == -6
    wide = _shape(batch=64, top_chunks=64, top_groups=512)   # candidates over 512K tokens: too large
    assert L.hga_decode_step_noalloc(ctypes.byref(wide), A, A, A, A, A, 1 << 19, A, A, A, A, A, None) == -6
