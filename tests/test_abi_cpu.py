"""The C ABI without a GPU: the library loads, exports every symbol that
include/bsg.h declares, computes layout offsets by the documented formula,
and rejects invalid arguments before any HIP call.

Every call below either is a pure host function or fails validation: no
call here enqueues GPU work.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_gemv_packed_amd as bsg
import oracle
from bit_gemv_packed_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsg.h")

OK, ENULL, ESHAPE, EDTYPE, EALIGN, EUNSUP, EWS, EHIP = 0, -1, -2, -3, -4, -5, -6, -7

# Fake device addresses: only ever passed to calls that fail validation.  As
# a second guard, the tests that pass them are skipped where a GPU is
# visible, so a validation slip can never launch a kernel on them.
A16 = 0x100000
A16b = 0x200000
A16c = 0x300000
A16d = 0x400000


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


fake_ptrs = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers are only passed where no GPU is visible")


def _declared():
    txt = open(HEADER).read()
    return re.findall(r"^BSG_API\s+[\w\s\*]+?\b(\w+)\s*\(", txt, flags=re.M)


def test_header_declares_the_calls_the_pages_name():
    names = set(_declared())
    for n in ("bsq_pack", "bs_gemv", "binlr_apply", "salient_int8_apply"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(bsg.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert bsg.lib().bsg_abi_version() == 1
    for s in (OK, ENULL, ESHAPE, EDTYPE, EALIGN, EUNSUP, EWS, EHIP):
        assert len(bsg.status_string(s)) >= 2
    assert bsg.status_string(12345) == "unknown status"


@pytest.mark.parametrize("K,M,N", [(1, 64, 128), (2, 70, 160), (3, 130, 32), (1, 1, 96), (2, 200, 544), (4, 257, 4096)])
def test_layout_formula_matches_oracle(K, M, N):
    assert bsg.layout_words(K, M, N) == oracle.layout_words(K, M, N)
    rng = np.random.default_rng(K * M + N)
    nd = N // 32
    for _ in range(300):
        k, m, w = int(rng.integers(K)), int(rng.integers(M)), int(rng.integers(nd))
        assert bsg.layout_word_offset(K, M, N, k, m, w) == oracle.layout_offset(K, M, N, k, m, w)
    assert bsg.layout_word_offset(K, M, N, K, 0, 0) == -1
    assert bsg.layout_word_offset(K, M, N, 0, M, 0) == -1
    assert bsg.layout_word_offset(K, M, N, 0, 0, nd) == -1
    assert bsg.layout_words(K, M, 33) == 0


def test_workspace_sizes():
    assert bsg.binlr_workspace_bytes(512, 5120, 5120, 1) >= 512 * 4
    assert bsg.binlr_workspace_bytes(512, 5120, 5120, 16) >= 512 * 16 * 4
    assert bsg.binlr_workspace_bytes(500, 5120, 5120, 1) == 0
    assert bsg.lib().bsq_pack_workspace_bytes(100, 64) >= 100 * 64 * 8


def _gemv(bits=A16, K=2, M=128, N=256, alpha=A16b, cs=None, x=A16c, dt=2, B=1, y=A16d, acc=0):
    return bsg.lib().bs_gemv(bits, K, M, N, alpha, cs, x, dt, B, y, acc, None)


@fake_ptrs
def test_bs_gemv_validation():
    assert _gemv(dt=7) == EDTYPE
    assert _gemv(N=33) == ESHAPE
    assert _gemv(N=0) == ESHAPE
    assert _gemv(K=0) == ESHAPE
    assert _gemv(K=9) == ESHAPE
    assert _gemv(B=0) == ESHAPE
    assert _gemv(B=65) == ESHAPE
    assert _gemv(M=-1) == ESHAPE
    assert _gemv(M=0) == OK                      # empty output: a no-op
    assert _gemv(bits=None) == ENULL
    assert _gemv(alpha=None) == ENULL
    assert _gemv(x=None) == ENULL
    assert _gemv(y=None) == ENULL
    assert _gemv(bits=A16 + 4) == EALIGN
    assert _gemv(alpha=A16b + 2) == EALIGN
    assert _gemv(x=A16c + 1, dt=2) == EALIGN
    assert _gemv(cs=A16 + 1) == EALIGN
    assert _gemv(y=A16d + 2) == EALIGN


def _multi(projs, K=2, N=256, x=A16c, dt=2, B=1, acc=0, P=None):
    arr = (bsg.BsgProj * max(1, len(projs)))(*[bsg.BsgProj(*p) for p in projs])
    return bsg.lib().bs_gemv_multi(ctypes.cast(arr, ctypes.c_void_p), len(projs) if P is None else P, K, N, x, dt, B,
                                   acc, None)


@fake_ptrs
def test_bs_gemv_multi_validation():
    q = (A16, A16b, None, A16d, 128)
    assert _multi([q], dt=7) == EDTYPE
    assert bsg.lib().bs_gemv_multi(None, 1, 2, 256, A16c, 2, 1, 0, None) == ENULL
    assert _multi([q], P=0) == ESHAPE
    assert _multi([q] * 9) == ESHAPE                # at most 8 projections
    assert _multi([q], K=0) == ESHAPE
    assert _multi([q], K=9) == ESHAPE
    assert _multi([q], N=33) == ESHAPE
    assert _multi([q], B=0) == ESHAPE
    assert _multi([q], B=65) == ESHAPE
    assert _multi([q, (A16, A16b, None, A16d, -1)]) == ESHAPE
    assert _multi([q, (A16, A16b, A16c, A16d, 64)]) == ESHAPE   # column scales for some projections only
    assert _multi([q], x=None) == ENULL
    assert _multi([q], x=A16c + 1) == EALIGN
    assert _multi([q, (None, A16b, None, A16d, 64)]) == ENULL
    assert _multi([q, (A16, None, None, A16d, 64)]) == ENULL
    assert _multi([q, (A16, A16b, None, None, 64)]) == ENULL
    assert _multi([q, (A16 + 4, A16b, None, A16d, 64)]) == EALIGN
    assert _multi([q, (A16, A16b + 2, None, A16d, 64)]) == EALIGN
    assert _multi([q, (A16, A16b, None, A16d + 2, 64)]) == EALIGN
    assert _multi([(A16, A16b, A16c, A16d, 64), (A16, A16b, A16c + 1, A16d, 64)]) == EALIGN
    assert _multi([(None, None, None, None, 0)]) == OK   # empty outputs: a no-op


def _fit(W=A16, M=64, N=64, r=8, rounds=5, v0=A16b, U=A16c, V=A16d, a16=A16, ws=A16b, nb=None):
    if nb is None:
        nb = bsg.lib().binlr_fit_workspace_bytes(M, N, r) if r > 0 and N % 32 == 0 and M > 0 else 0
    return bsg.lib().binlr_fit(W, M, N, r, rounds, v0, U, V, a16, None, None, None, None, ws, nb, None)


def test_binlr_fit_workspace_bytes():
    nb = bsg.lib().binlr_fit_workspace_bytes(5120, 5120, 512)
    assert nb >= 8 * 5120 * 5120                 # the fp64 residual
    assert nb < 8 * 5120 * 5120 + (64 << 20)
    assert bsg.lib().binlr_fit_workspace_bytes(64, 33, 8) == 0
    assert bsg.lib().binlr_fit_workspace_bytes(64, 64, 0) == 0
    assert bsg.lib().binlr_fit_workspace_bytes(64, 64, 2049) == 0


@fake_ptrs
def test_binlr_fit_validation():
    assert _fit(M=0) == ESHAPE
    assert _fit(N=33) == ESHAPE
    assert _fit(r=0) == ESHAPE
    assert _fit(r=2049) == ESHAPE
    assert _fit(rounds=0) == ESHAPE
    assert _fit(rounds=65) == ESHAPE
    assert _fit(W=None) == ENULL
    assert _fit(v0=None) == ENULL
    assert _fit(U=None) == ENULL
    assert _fit(V=None) == ENULL
    assert _fit(a16=None) == ENULL
    assert _fit(W=A16 + 2) == EALIGN
    assert _fit(U=A16c + 4) == EALIGN
    assert _fit(ws=A16b + 16) == EALIGN
    assert _fit(ws=None) == EWS
    assert _fit(nb=100) == EWS


def _gg(bits=A16, K=2, M=128, N=256, g=128, alpha=A16b, cs=None, x=A16c, dt=2, B=1, y=A16d, acc=0):
    return bsg.lib().bs_gemv_grouped(bits, K, M, N, g, alpha, cs, x, dt, B, y, acc, None)


@fake_ptrs
def test_grouped_validation():
    assert _gg(dt=7) == EDTYPE
    assert _gg(g=96) == ESHAPE          # not a power of two
    assert _gg(g=32) == ESHAPE          # below 64
    assert _gg(N=192, g=128) == ESHAPE  # does not divide N
    assert _gg(K=5) == ESHAPE
    assert _gg(K=0) == ESHAPE
    assert _gg(B=65) == ESHAPE
    assert _gg(M=0) == OK
    assert _gg(bits=None) == ENULL
    assert _gg(alpha=None) == ENULL
    assert _gg(alpha=A16b + 1) == EALIGN   # fp16 scales
    assert _gg(bits=A16 + 4) == EALIGN
    assert bsg.lib().bsq_pack_grouped_workspace_bytes(64, 256, 128) >= 64 * 256 * 8
    assert bsg.lib().bsq_pack_grouped_workspace_bytes(64, 256, 96) == 0
    nb = bsg.lib().bsq_pack_grouped_workspace_bytes(64, 256, 128)
    pg = bsg.lib().bsq_pack_grouped
    assert pg(A16, 64, 256, 2, 100, 0, A16b, A16c, None, A16d, nb, None) == ESHAPE
    assert pg(A16, 64, 256, 2, 128, 1, A16b, A16c, None, A16d, nb, None) == ENULL   # colscale requested
    assert pg(A16, 64, 256, 2, 128, 0, A16b, A16c, None, A16d, nb - 1, None) == EWS
    assert pg(A16, 64, 256, 2, 128, 4, A16b, A16c, None, A16d, nb, None) == ESHAPE  # unknown flag


def _gh(s=16, sbits=A16, idx=A16b, salpha=A16c, scs=None, cs=None, K=2, M=128, N=256, g=128, dt=2, B=1):
    return bsg.lib().bs_gemv_hybrid(A16, K, M, N, g, A16b, cs, sbits, s, idx, salpha, scs, A16c, dt, B, A16d, 0,
                                    None)


@fake_ptrs
def test_hybrid_validation():
    assert _gh(s=12) == ESHAPE
    assert _gh(s=4) == ESHAPE
    assert _gh(s=64) == ESHAPE
    assert _gh(K=5) == ESHAPE
    assert _gh(cs=A16d) == ESHAPE              # column scales on one branch only
    assert _gh(scs=A16d) == ESHAPE
    assert _gh(sbits=None) == ENULL
    assert _gh(idx=None) == ENULL
    assert _gh(salpha=None) == ENULL
    assert _gh(s=0, sbits=None, idx=None, salpha=None, M=0) == OK   # no salient branch: nothing needed
    assert _gh(idx=A16b + 4) == EALIGN         # 16-byte index loads
    assert _gh(salpha=A16c + 4) == EALIGN      # 8-byte scale loads
    assert _gh(M=0) == OK
    wb = bsg.lib().bsq_pack_hybrid_workspace_bytes
    assert wb(64, 256, 128, 16) >= 64 * 256 * 8 + 64 * 32 * 8
    assert wb(64, 256, 128, 12) == 0
    assert wb(64, 256, 128, 0) == bsg.lib().bsq_pack_grouped_workspace_bytes(64, 256, 128)
    nb = wb(64, 256, 128, 8)
    ph = bsg.lib().bsq_pack_hybrid
    assert ph(A16, 64, 256, 2, 128, 8, None, 0, A16b, A16c, None, A16d, A16c, None, A16d, nb, None) == ENULL
    assert ph(A16, 64, 256, 2, 128, 8, A16b, 0, A16b, A16c, None, None, A16c, None, A16d, nb, None) == ENULL
    assert ph(A16, 64, 256, 2, 128, 8, A16b, 1, A16b, A16c, A16d, A16d, A16c, None, A16d, nb, None) == ENULL
    assert ph(A16, 64, 256, 2, 128, 8, A16b, 0, A16b, A16c, None, A16d, A16c, None, A16d, nb - 1, None) == EWS
    assert ph(A16, 64, 256, 2, 128, 24, A16b, 0, A16b, A16c, None, A16d, A16c, None, A16d, nb, None) == ESHAPE


@fake_ptrs
def test_bs_gemv_i8_validation():
    L = bsg.lib()
    f = lambda **kw: L.bs_gemv_i8(kw.get("bits", A16), kw.get("K", 2), kw.get("M", 128), kw.get("N", 256),
                                  kw.get("alpha", A16b), kw.get("xq", A16c), kw.get("sx", A16d), kw.get("B", 1),
                                  kw.get("acc", A16), kw.get("y", None), 0, None)
    assert f(N=48) == ESHAPE
    assert f(N=(1 << 24) + 32) == ESHAPE
    assert f(acc=None, y=None) == ENULL
    assert f(xq=None) == ENULL
    assert f(y=A16d, sx=None) == ENULL
    assert f(M=0, ns=0) == OK


@fake_ptrs
def test_binlr_and_salient_validation():
    L = bsg.lib()
    assert L.binlr_apply(A16, A16b, A16c, 500, 64, 64, A16d, 2, 1, A16, None, 0, None) == ESHAPE
    assert L.binlr_apply(A16, A16b, A16c, 32, 64, 64, A16d, 2, 1, A16, None, 0, None) == EWS
    assert L.binlr_apply(A16, A16b, A16c, 32, 64, 64, A16d, 2, 1, A16, 0x500000, 64, None) == EWS
    assert L.binlr_apply(None, A16b, A16c, 32, 64, 64, A16d, 2, 1, A16, None, 0, None) == ENULL
    assert L.binlr_apply(A16, A16b, A16c, 32, 64, 64, A16d, 9, 1, A16, None, 0, None) == EDTYPE
    assert L.salient_int8_apply(A16, 3, A16b, A16c, 64, 64, A16d, 2, 1, None, None) == ENULL
    assert L.salient_int8_apply(A16, -1, A16b, A16c, 64, 64, A16d, 2, 1, A16, None) == ESHAPE
    assert L.salient_int8_apply(A16, 0, A16b, A16c, 64, 64, A16d, 2, 1, A16, None) == OK
    assert L.salient_int8_apply(A16 + 2, 3, A16b, A16c, 64, 64, A16d, 2, 1, A16, None) == EALIGN


@fake_ptrs
def test_bsg_linear_validation():
    L = bsg.lib()

    def f(**kw):
        d = dict(bits=A16, K=2, M=128, N=256, alpha=A16b, cs=None, U=A16c, V=A16d, ar=A16, r=32, rows=A16b,
                 ns=3, q=A16c, s=A16d, x=A16, dt=2, B=1, y=A16b, acc=0, ws=None, wsn=0)
        d.update(kw)
        return L.bsg_linear(d["bits"], d["K"], d["M"], d["N"], d["alpha"], d["cs"], d["U"], d["V"], d["ar"], d["r"],
                            d["rows"], d["ns"], d["q"], d["s"], d["x"], d["dt"], d["B"], d["y"], d["acc"], d["ws"],
                            d["wsn"], None)
    assert f(dt=9) == EDTYPE
    assert f(N=48) == ESHAPE
    assert f(r=40) == ESHAPE
    assert f(r=-32) == ESHAPE
    assert f(ns=-1) == ESHAPE
    assert f(ns=129) == ESHAPE                   # more protected rows than rows
    assert f(K=9) == ESHAPE
    assert f(M=0, ns=0) == OK
    assert f(U=None) == ENULL                    # r > 0 needs U, V and alpha_r
    assert f(ar=None) == ENULL
    assert f(q=None) == ENULL                    # ns > 0 needs rows, q and s
    assert f(alpha=None) == ENULL
    assert f(q=A16c + 8) == EALIGN               # q rows are read 16 bytes at a time
    assert f(rows=A16b + 2) == EALIGN
    assert f(U=A16c + 4) == EALIGN
    assert f(ws=None) == EWS                     # r > 0 needs the z workspace
    assert f(ws=0x500000, wsn=64) == EWS
    assert L.bsg_linear_workspace_bytes(32, 1) >= 32 * 4
    assert L.bsg_linear_workspace_bytes(0, 1) == 0
    assert L.bsg_linear_workspace_bytes(40, 1) == 0


@fake_ptrs
def test_pack_validation():
    L = bsg.lib()
    assert L.bsq_pack(A16, 64, 64, 0, 0, A16b, A16c, None, A16d, 1 << 20, None) == ESHAPE
    assert L.bsq_pack(A16, 64, 48, 1, 0, A16b, A16c, None, A16d, 1 << 20, None) == ESHAPE
    assert L.bsq_pack(A16, 64, 64, 1, 4, A16b, A16c, None, A16d, 1 << 20, None) == ESHAPE
    assert L.bsq_pack(A16, 64, 64, 1, 1, A16b, A16c, None, A16d, 1 << 20, None) == ENULL
    assert L.bsq_pack(A16, 64, 64, 1, 0, A16b + 4, A16c, None, A16d, 1 << 20, None) == EALIGN
    assert L.bsq_pack(A16, 64, 64, 1, 0, A16b, A16c, None, A16d, 100, None) == EWS
    assert L.bsq_salient(A16, 64, 64, A16b, 65, A16c, A16d, A16, A16b, 1, A16c, 1 << 20, None) == ESHAPE
    assert L.bsq_quantize_i8(A16, 5, 64, 1, A16b, A16c, None) == EDTYPE
    assert L.bsg_logical_to_layout(A16, 1, 64, 40, A16b, None) == ESHAPE


@fake_ptrs
def test_grouped_multi_validation():
    import ctypes
    P = bsg.BsgProj * 3
    good = lambda: P(bsg.BsgProj(A16, A16b, None, A16d, 64), bsg.BsgProj(A16, A16b, None, A16d, 32),
                     bsg.BsgProj(A16, A16b, None, A16d, 0))
    gm = bsg.lib().bs_gemv_grouped_multi
    arr = good()
    ptr = ctypes.cast(arr, ctypes.c_void_p)
    assert gm(ptr, 0, 2, 256, 128, A16c, 2, 1, 0, None) == ESHAPE
    assert gm(ptr, 9, 2, 256, 128, A16c, 2, 1, 0, None) == ESHAPE
    assert gm(ptr, 3, 5, 256, 128, A16c, 2, 1, 0, None) == ESHAPE      # K > 4
    assert gm(ptr, 3, 2, 256, 96, A16c, 2, 1, 0, None) == ESHAPE       # bad group
    assert gm(ptr, 3, 2, 256, 128, A16c, 7, 1, 0, None) == EDTYPE
    assert gm(None, 3, 2, 256, 128, A16c, 2, 1, 0, None) == ENULL
    assert gm(ptr, 3, 2, 256, 128, None, 2, 1, 0, None) == ENULL
    arr[1].colscale = A16d
    assert gm(ptr, 3, 2, 256, 128, A16c, 2, 1, 0, None) == ESHAPE      # column scales on one projection only
    arr = good()
    arr[0].alpha = A16b + 1
    assert gm(ctypes.cast(arr, ctypes.c_void_p), 3, 2, 256, 128, A16c, 2, 1, 0, None) == EALIGN
    arr = good()
    arr[1].bits = None
    assert gm(ctypes.cast(arr, ctypes.c_void_p), 3, 2, 256, 128, A16c, 2, 1, 0, None) == ENULL
    zero = P(bsg.BsgProj(A16, A16b, None, A16d, 0), bsg.BsgProj(A16, A16b, None, A16d, 0),
             bsg.BsgProj(None, None, None, None, 0))
    assert gm(ctypes.cast(zero, ctypes.c_void_p), 3, 2, 256, 128, A16c, 2, 1, 0, None) == OK
