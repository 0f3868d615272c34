"""CPU oracle for the binary sign-GEMV path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``bit_gemv_packed_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one bit at a
time, ascending index order); this module only marshals numpy arrays into it
and adds the parity tolerance.  Each C function names the page passage it
follows.  Functions whose results have no value printed on the pages are
marked "parity unpinned" in the design doc and below:

* the least-squares column scale of the packer (``pack``, ``pack_grouped`` and
  ``pack_hybrid`` with ``with_colscale=True``), pinned only to its closed-form
  optimality,
* the protected-row selection rule (``salient_select``),
* the salient-column refinement of ``pack_hybrid`` as a refit of the residual
  (a reading: the pages' equations for it are lost), pinned to its special
  case with every column salient and to its effect on the error.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        sig = {
            "or_f16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
            "or_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
            "or_f16_array_to_f64": (None, [_P, _SZ, _P]),
            "or_f32_array_to_f16": (None, [_P, _SZ, _P]),
            "or_sign_gemv": (None, [_P, _I, _I, _I, _P, _P, _P, _I, _P]),
            "or_binlr": (None, [_P, _P, _P, _I, _I, _I, _P, _I, _P]),
            "or_salient": (None, [_P, _I, _P, _P, _I, _I, _P, _I, _P]),
            "or_sign_gemv_i8": (None, [_P, _I, _I, _I, _P, _I, _P]),
            "or_quantize_i8": (None, [_P, _I, _I, _P, _P]),
            "or_pack": (_I, [_P, _I, _I, _I, _I, _P, _P, _P]),
            "or_pack_signs": (None, [_P, _I, _I, _P]),
            "or_absmean": (None, [_P, _I, _I, _P]),
            "or_salient_select": (_I, [_P, _I, _I, _P, _I, _P, _P, _P, _P, _I]),
            "or_layout_plane_words": (_SZ, [_I, _I]),
            "or_layout_offset": (_SZ, [_I, _I, _I, _I, _I, _I]),
            "or_logical_to_layout": (None, [_P, _I, _I, _I, _P]),
            "or_layout_to_logical": (None, [_P, _I, _I, _I, _P]),
            "or_binlr_fit": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
            "or_pack_grouped": (_I, [_P, _I, _I, _I, _I, _I, _P, _P, _P]),
            "or_sign_gemv_grouped": (None, [_P, _I, _I, _I, _I, _P, _P, _P, _I, _P]),
            "or_pack_hybrid": (_I, [_P, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P]),
            "or_sign_gemv_hybrid": (None, [_P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _I, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def words(N: int) -> int:
    """Sign words per row: ceil(N / 32)."""
    return (N + 31) // 32


# ---------------------------------------------------------------- conversions
def f16_to_f64(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().or_f16_array_to_f64(_ptr(h), h.size, _ptr(out))
    return out


def f32_to_f16(f) -> np.ndarray:
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().or_f32_array_to_f16(_ptr(f), f.size, _ptr(out))
    return out


# ---------------------------------------------------------------- the product
def sign_gemv(bits, K, M, N, alpha, x, colscale_f16=None) -> np.ndarray:
    """y_bin [M][B] in float64.  bits: logical uint32 [K][M][ceil(N/32)];
    alpha: fp32 [K][M]; colscale_f16: uint16 [K][N] or None; x: [N][B] (or [N]).
    """
    x = np.asarray(x, np.float64)
    if x.ndim == 1:
        x = x[:, None]
    B = x.shape[1]
    bits = _c(bits, np.uint32).reshape(-1)
    assert bits.size == K * M * words(N)
    a = _c(np.asarray(alpha, np.float32).astype(np.float64), np.float64).reshape(-1)
    c = None if colscale_f16 is None else f16_to_f64(colscale_f16).reshape(-1)
    x = _c(x, np.float64)
    y = np.empty((M, B), np.float64)
    lib().or_sign_gemv(_ptr(bits), K, M, N, _ptr(a), _ptr(c), _ptr(x), B, _ptr(y))
    return y


def binlr(ubits, vbits, alpha_r_f16, r, M, N, x) -> np.ndarray:
    """y_lr [M][B] in float64.  ubits: logical [M][ceil(r/32)];
    vbits: logical [r][ceil(N/32)]; alpha_r_f16: uint16 [r]."""
    x = np.asarray(x, np.float64)
    if x.ndim == 1:
        x = x[:, None]
    B = x.shape[1]
    u = _c(ubits, np.uint32).reshape(-1)
    v = _c(vbits, np.uint32).reshape(-1)
    assert u.size == M * words(r) and v.size == r * words(N)
    ar = f16_to_f64(alpha_r_f16).reshape(-1)
    y = np.empty((M, B), np.float64)
    lib().or_binlr(_ptr(u), _ptr(v), _ptr(ar), r, M, N, _ptr(_c(x, np.float64)), B, _ptr(y))
    return y


def salient(rows, q, s_f16, M, N, x) -> np.ndarray:
    """y_sal [M][B] in float64 (zero except the protected rows)."""
    x = np.asarray(x, np.float64)
    if x.ndim == 1:
        x = x[:, None]
    B = x.shape[1]
    rows = _c(rows, np.int32).reshape(-1)
    ns = rows.size
    q = _c(q, np.int8).reshape(-1)
    assert q.size == ns * N
    s = f16_to_f64(s_f16).reshape(-1)
    y = np.empty((M, B), np.float64)
    lib().or_salient(_ptr(rows), ns, _ptr(q), _ptr(s), M, N, _ptr(_c(x, np.float64)), B, _ptr(y))
    return y


def sign_gemv_i8(bits, K, M, N, xq) -> np.ndarray:
    """Exact integer sign product, int64 [K][M][B]."""
    xq = np.asarray(xq, np.int8)
    if xq.ndim == 1:
        xq = xq[:, None]
    B = xq.shape[1]
    bits = _c(bits, np.uint32).reshape(-1)
    acc = np.empty((K, M, B), np.int64)
    lib().or_sign_gemv_i8(_ptr(bits), K, M, N, _ptr(_c(xq, np.int8)), B, _ptr(acc))
    return acc


def quantize_i8(x):
    """(xq int8 [N][B], sx fp32 [B]) from fp32 values x [N][B]."""
    x = np.asarray(x, np.float32)
    if x.ndim == 1:
        x = x[:, None]
    N, B = x.shape
    xq = np.empty((N, B), np.int8)
    sx = np.empty((B,), np.float32)
    lib().or_quantize_i8(_ptr(_c(x, np.float32)), N, B, _ptr(xq), _ptr(sx))
    return xq, sx


# ---------------------------------------------------------------- packing
def pack(W, K: int, with_colscale: bool = False):
    """Greedy residual bases.  Returns (bits logical uint32 [K][M][ceil(N/32)],
    alpha fp32 [K][M], colscale fp16 bits uint16 [K][N] or None)."""
    W = _c(W, np.float32)
    M, N = W.shape
    bits = np.zeros((K, M, words(N)), np.uint32)
    alpha = np.zeros((K, M), np.float32)
    cs = np.zeros((K, N), np.uint16) if with_colscale else None
    rc = lib().or_pack(_ptr(W), M, N, K, 1 if with_colscale else 0, _ptr(bits), _ptr(alpha),
                       _ptr(cs) if cs is not None else None)
    if rc != 0:
        raise ValueError("oracle pack failed (%d)" % rc)
    return bits, alpha, cs


def pack_signs(S) -> np.ndarray:
    """Logical sign bits of a real matrix (bit = [S >= 0])."""
    S = _c(S, np.float32)
    M, N = S.shape
    bits = np.zeros((M, words(N)), np.uint32)
    lib().or_pack_signs(_ptr(S), M, N, _ptr(bits))
    return bits


def absmean(X) -> np.ndarray:
    """xbar[n] = fp32(mean_s |X[s][n]|) for calibration vectors X [S][N] (fp32 values)."""
    X = _c(X, np.float32)
    S, N = X.shape
    out = np.empty((N,), np.float32)
    lib().or_absmean(_ptr(X), S, N, _ptr(out))
    return out


def salient_select(W, xbar, ns: int, alpha=None):
    """(rows int32 [ns], q int8 [ns][N], s fp16 bits [ns], alpha with kept rows
    zeroed).  Parity unpinned: the selection rule has no page values."""
    W = _c(W, np.float32)
    M, N = W.shape
    rows = np.zeros((ns,), np.int32)
    q = np.zeros((ns, N), np.int8)
    s = np.zeros((ns,), np.uint16)
    if alpha is None:
        a = np.zeros((0, M), np.float32)
    else:
        a = np.array(alpha, np.float32, copy=True)
    K = a.shape[0]
    rc = lib().or_salient_select(_ptr(W), M, N, _ptr(_c(xbar, np.float32)), ns, _ptr(rows), _ptr(q),
                                 _ptr(s), _ptr(a) if K else None, K)
    if rc != 0:
        raise ValueError("oracle salient_select failed (%d)" % rc)
    return rows, q, s, a


# ---------------------------------------------------------------- layout
def pack_grouped(W, K: int, g: int, with_colscale: bool = False):
    """Greedy residual bases with one fp16 row scale per group of g columns (FluxBin Sec. 3.1,
    App. C.2); see or_pack_grouped.  Returns (bits [K][M][ceil(N/32)], alpha fp16 bits [K][M][N/g],
    colscale fp16 bits [K][N] or None)."""
    W = _c(np.asarray(W, np.float32), np.float32)
    M, N = W.shape
    bits = np.zeros((K, M, words(N)), np.uint32)
    alpha = np.zeros((K, M, N // g), np.uint16)
    cs = np.zeros((K, N), np.uint16) if with_colscale else None
    rc = lib().or_pack_grouped(_ptr(W), M, N, K, g, 1 if with_colscale else 0, _ptr(bits), _ptr(alpha), _ptr(cs))
    if rc != 0:
        raise ValueError("pack_grouped failed (%d)" % rc)
    return bits, alpha, cs


def sign_gemv_grouped(bits, K, M, N, g, alpha, x, colscale_f16=None) -> np.ndarray:
    """y [M][B] in float64 for group-wise row scales alpha fp16 bits [K][M][N/g]."""
    x = np.asarray(x, np.float64)
    if x.ndim == 1:
        x = x[:, None]
    B = x.shape[1]
    bits = _c(bits, np.uint32).reshape(-1)
    a = _c(np.asarray(alpha, np.uint16), np.uint16).reshape(-1)
    assert a.size == K * M * (N // g)
    cs = None if colscale_f16 is None else _c(np.asarray(colscale_f16, np.uint16), np.uint16).reshape(-1)
    xc = _c(x, np.float64)
    y = np.zeros((M, B), np.float64)
    lib().or_sign_gemv_grouped(_ptr(bits), K, M, N, g, _ptr(a), _ptr(cs), _ptr(xc), B, _ptr(y))
    return y


def pack_hybrid(W, K: int, g: int, s: int, idx, with_colscale: bool = False):
    """Global grouped bases plus salient-column refinement through a dense physical matrix (FluxBin
    Sec. 3.1 hybrid bases, Sec. 3.2 VCM); see or_pack_hybrid.  idx: int32 [s * N/g] column indices.
    Returns (bits, alpha, colscale, sbits [K][M][ceil(S/32)], salpha fp16 bits [K][M][N/g],
    scolscale fp16 bits [K][S] or None)."""
    W = _c(np.asarray(W, np.float32), np.float32)
    M, N = W.shape
    G = N // g
    S = s * G
    idx = _c(np.asarray(idx, np.int32), np.int32)
    assert idx.size == S
    bits = np.zeros((K, M, words(N)), np.uint32)
    alpha = np.zeros((K, M, G), np.uint16)
    cs = np.zeros((K, N), np.uint16) if with_colscale else None
    sbits = np.zeros((K, M, words(S)), np.uint32)
    salpha = np.zeros((K, M, G), np.uint16)
    scs = np.zeros((K, S), np.uint16) if with_colscale else None
    rc = lib().or_pack_hybrid(_ptr(W), M, N, K, g, s, _ptr(idx), 1 if with_colscale else 0, _ptr(bits),
                              _ptr(alpha), _ptr(cs), _ptr(sbits), _ptr(salpha), _ptr(scs))
    if rc != 0:
        raise ValueError("pack_hybrid failed (%d)" % rc)
    return bits, alpha, cs, sbits, salpha, scs


def sign_gemv_hybrid(bits, K, M, N, g, alpha, colscale_f16, sbits, s, idx, salpha, scolscale_f16, x) -> np.ndarray:
    """y [M][B] in float64: the grouped product plus the salient branch on x[idx]; see or_sign_gemv_hybrid."""
    x = np.asarray(x, np.float64)
    if x.ndim == 1:
        x = x[:, None]
    B = x.shape[1]
    G = N // g
    S = s * G
    u16 = lambda a: None if a is None else _c(np.asarray(a, np.uint16), np.uint16).reshape(-1)
    bits = _c(bits, np.uint32).reshape(-1)
    sbits = _c(sbits, np.uint32).reshape(-1)
    idx = _c(np.asarray(idx, np.int32), np.int32).reshape(-1)
    assert idx.size == S and sbits.size == K * M * words(S)
    a, cs, sa, scs = u16(alpha), u16(colscale_f16), u16(salpha), u16(scolscale_f16)
    assert a.size == K * M * G and sa.size == K * M * G
    xc = _c(x, np.float64)
    y = np.zeros((M, B), np.float64)
    lib().or_sign_gemv_hybrid(_ptr(bits), K, M, N, g, _ptr(a), _ptr(cs), _ptr(sbits), s, _ptr(idx), _ptr(sa),
                              _ptr(scs), _ptr(xc), B, _ptr(y))
    return y


def average_bits(K: int, M: int, N: int, g: int, s: int = 0, colscale: bool = True, scale_bits: int = 16) -> float:
    """Effective average bit-width of the stored format (FluxBin App. C.2 storage analysis: every
    scale and index stored in 16 bits): bits of the K global bases, their group row scales and
    column scales, and for s > 0 the K salient bases over S = s N/g columns, their group row scales,
    column scales and the S column indices, over the M N weights."""
    G = N // g
    S = s * G
    total = K * M * N + K * M * G * scale_bits + (K * N * scale_bits if colscale else 0)
    if s:
        total += K * M * S + K * M * G * scale_bits + (K * S * scale_bits if colscale else 0) + S * 16
    return total / (M * N)


def binlr_fit(W, r: int, vinit, rounds: int = 5):
    """Offline binary low-rank fit (BiLoCo "Finding the sign vectors", "Joint
    refit"); see or_binlr_fit.  W: fp32 [M][N] (any N > 0); vinit: logical
    sign words [r][ceil(N/32)] of the start vectors.  Returns (ubits [M][ceil(r/32)], vbits
    [r][N/32], alpha_greedy [r], alpha [r] refitted, (sse_greedy, sse_refit),
    solved)."""
    W = _c(np.asarray(W, np.float32), np.float32)
    M, N = W.shape
    rd, nd = (r + 31) // 32, (N + 31) // 32
    vinit = _c(np.asarray(vinit, np.uint32).reshape(r, nd), np.uint32)
    ub = np.zeros((M, rd), np.uint32)
    vb = np.zeros((r, nd), np.uint32)
    ag = np.zeros(r, np.float64)
    al = np.zeros(r, np.float64)
    sse = np.zeros(2, np.float64)
    rc = lib().or_binlr_fit(_ptr(W), M, N, r, rounds, _ptr(vinit), _ptr(ub), _ptr(vb), _ptr(ag), _ptr(al),
                            _ptr(sse))
    if rc < 0:
        raise ValueError("binlr_fit: bad sizes")
    return ub, vb, ag, al, (float(sse[0]), float(sse[1])), bool(rc)


def layout_words(K, M, N) -> int:
    return K * int(lib().or_layout_plane_words(M, N))


def layout_offset(K, M, N, k, m, w) -> int:
    return int(lib().or_layout_offset(K, M, N, k, m, w))


def to_layout(logical, K, M, N) -> np.ndarray:
    logical = _c(logical, np.uint32).reshape(-1)
    phys = np.zeros((layout_words(K, M, N),), np.uint32)
    lib().or_logical_to_layout(_ptr(logical), K, M, N, _ptr(phys))
    return phys


def from_layout(phys, K, M, N) -> np.ndarray:
    phys = _c(phys, np.uint32).reshape(-1)
    logical = np.zeros((K, M, words(N)), np.uint32)
    lib().or_layout_to_logical(_ptr(phys), K, M, N, _ptr(logical))
    return logical


# ---------------------------------------------------------------- tolerance
def tolerance(x, alpha=None, colscale_f16=None, alpha_r_f16=None, rows=None, q=None, s_f16=None,
              M=None, rel=2e-3) -> np.ndarray:
    """Per-(m, b) bound on |y - y_ref|:
    rel * ( sum_k |alpha_k[m]| * sum_n |c_k[n] x[n,b]|
          + sum_j |alpha_r[j]| * sum_n |x[n,b]|
          + [m = rows[i]] |s_i| * sum_n |q[i,n] x[n,b]| ).
    With no colscale, no low-rank term and no protected rows this is the
    stated per-row bound rel * (sum_k |alpha_k|) * ||x||_1."""
    x = np.asarray(x, np.float64)
    if x.ndim == 1:
        x = x[:, None]
    N, B = x.shape
    ax = np.abs(x)
    if M is None:
        M = np.asarray(alpha).shape[1]
    t = np.zeros((M, B), np.float64)
    if alpha is not None:
        a = np.abs(np.asarray(alpha, np.float64))            # [K][M]
        if colscale_f16 is None:
            t += a.sum(0)[:, None] * ax.sum(0)[None, :]
        else:
            c = np.abs(f16_to_f64(colscale_f16))              # [K][N]
            t += np.einsum("km,kb->mb", a, c @ ax)
    if alpha_r_f16 is not None:
        ar = np.abs(f16_to_f64(alpha_r_f16)).sum()
        t += ar * ax.sum(0)[None, :]
    if rows is not None and len(rows):
        s = np.abs(f16_to_f64(s_f16))
        contrib = (np.abs(np.asarray(q, np.float64)) @ ax) * s[:, None]   # [ns][B]
        np.add.at(t, np.asarray(rows, np.int64), contrib)
    return rel * t
