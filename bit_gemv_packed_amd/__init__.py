"""bit_gemv_packed_amd -- binary sign-GEMV for AMD Instinct MI355X (gfx950).

A thin ctypes binding over libbsg.so (the C ABI in include/bsg.h).  Every
function marshals torch tensors into device pointers and the current HIP
stream and calls the entry point of the same name; all arithmetic runs in
the library's HIP kernels.  There is no CPU fallback: if libbsg.so is
missing, or a tensor is not on the GPU, the call raises.

The page passages each operation follows are cited in include/bsg.h.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsg.so")

BSG_F32, BSG_F16, BSG_BF16 = 0, 1, 2
BSG_PACK_COLSCALE = 1
BSG_ERR_HIP = -7

_STATUS_NAMES = {0: "BSG_OK", -1: "BSG_ERR_NULL", -2: "BSG_ERR_SHAPE", -3: "BSG_ERR_DTYPE",
                 -4: "BSG_ERR_ALIGN", -5: "BSG_ERR_UNSUPPORTED", -6: "BSG_ERR_WORKSPACE", -7: "BSG_ERR_HIP"}


class BsgError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__("%s failed: %s (%d: %s)" % (fn, _STATUS_NAMES.get(status, "?"), status, message))
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "bsg_abi_version": (ctypes.c_int32, []),
    "bsg_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "bsg_last_hip_error": (ctypes.c_int32, []),
    "bsg_last_hip_error_string": (ctypes.c_char_p, []),
    "bsg_layout_words": (_SZ, [_I, _I, _I]),
    "bsg_layout_word_offset": (ctypes.c_int64, [_I, _I, _I, _I, _I, _I]),
    "bsg_binlr_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "bsq_pack_workspace_bytes": (_SZ, [_I, _I]),
    "bsq_salient_workspace_bytes": (_SZ, [_I, _I]),
    "bsq_pack": (ctypes.c_int32, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "bsq_pack_signs": (ctypes.c_int32, [_P, _I, _I, _P, _P]),
    "bsq_absmean": (ctypes.c_int32, [_P, _I, _I, _P, _P]),
    "bsq_salient": (ctypes.c_int32, [_P, _I, _I, _P, _I, _P, _P, _P, _P, _I, _P, _SZ, _P]),
    "bsq_quantize_i8": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P, _P]),
    "bsg_logical_to_layout": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P]),
    "bsg_layout_to_logical": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P]),
    "bs_gemv": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P]),
    "bs_gemv_i8": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P, _P, _I, _P, _P, _I, _P]),
    "bs_gemv_multi": (ctypes.c_int32, [_P, _I, _I, _I, _P, _I, _I, _I, _P]),
    "bsq_pack_grouped_workspace_bytes": (_SZ, [_I, _I, _I]),
    "bsq_pack_grouped": (ctypes.c_int32, [_P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "bs_gemv_grouped": (ctypes.c_int32, [_P, _I, _I, _I, _I, _P, _P, _P, _I, _I, _P, _I, _P]),
    "bsq_pack_hybrid_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "bsq_pack_hybrid": (ctypes.c_int32, [_P, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "bs_gemv_grouped_multi": (ctypes.c_int32, [_P, _I, _I, _I, _I, _P, _I, _I, _I, _P]),
    "bs_gemv_hybrid": (ctypes.c_int32, [_P, _I, _I, _I, _I, _P, _P, _P, _I, _P, _P, _P, _P, _I, _I, _P, _I, _P]),
    "binlr_fit_workspace_bytes": (_SZ, [_I, _I, _I]),
    "binlr_fit": (ctypes.c_int32, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "binlr_apply": (ctypes.c_int32, [_P, _P, _P, _I, _I, _I, _P, _I, _I, _P, _P, _SZ, _P]),
    "salient_int8_apply": (ctypes.c_int32, [_P, _I, _P, _P, _I, _I, _P, _I, _I, _P, _P]),
    "bsg_linear_workspace_bytes": (_SZ, [_I, _I]),
    "bsg_linear": (ctypes.c_int32, [_P, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P, _I, _I, _P, _I,
                                    _P, _SZ, _P]),
}


def lib():
    """Load libbsg.so (built in-tree by bit_gemv_packed_amd.build).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libbsg.so is not built (%s); run bit_gemv_packed_amd.build.build() "
                              "or __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().bsg_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        msg = status_string(status)
        if status == BSG_ERR_HIP:
            msg += "; HIP error %d: %s" % (lib().bsg_last_hip_error(), lib().bsg_last_hip_error_string().decode())
        raise BsgError(fn, status, msg)


# ------------------------------------------------------------------ helpers
def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU (device %s given)" % t.device)
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(device=None) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return BSG_F32
    if t.dtype == torch.float16:
        return BSG_F16
    if t.dtype == torch.bfloat16:
        return BSG_BF16
    raise TypeError("unsupported activation dtype %s" % t.dtype)


def _xshape(x, N: int) -> int:
    if x.dim() == 1:
        if x.shape[0] != N:
            raise ValueError("x must have N=%d elements" % N)
        return 1
    if x.dim() != 2 or x.shape[0] != N:
        raise ValueError("x must be [N][B] with N=%d" % N)
    return x.shape[1]


def new_workspace(nbytes: int, device) -> Optional["object"]:
    """A device workspace of at least nbytes, 16-byte aligned (None when nbytes == 0)."""
    if nbytes == 0:
        return None
    torch = _torch()
    return torch.empty((nbytes + 15) // 16 * 16, dtype=torch.uint8, device=device)


class Workspace:
    """Per-device cache of one workspace, grown on demand.  Calls through the
    binding are stream-ordered on the current stream, so they may share it."""

    def __init__(self):
        self._bufs = {}

    def get(self, nbytes: int, device):
        if nbytes == 0:
            return None
        key = str(device)
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = new_workspace(max(nbytes, 1 << 20), device)
            self._bufs[key] = buf
        return buf


_WS = Workspace()


def _ws_args(ws):
    if ws is None:
        return None, 0
    return ws.data_ptr(), ws.numel() * ws.element_size()


# ------------------------------------------------------------------ sizes
def layout_words(K: int, M: int, N: int) -> int:
    return int(lib().bsg_layout_words(K, M, N))


def layout_word_offset(K: int, M: int, N: int, k: int, m: int, w: int) -> int:
    return int(lib().bsg_layout_word_offset(K, M, N, k, m, w))


def binlr_workspace_bytes(r: int, M: int, N: int, B: int) -> int:
    return int(lib().bsg_binlr_workspace_bytes(r, M, N, B))


# ------------------------------------------------------------------ packing
def bsq_pack(W, K: int, colscale: bool = False, workspace=None):
    """Greedy residual binary bases of W (fp32 [M][N] on the GPU).
    Returns (bits int32 [layout words], alpha fp32 [K][M], colscale fp16-bits int16 [K][N] or None)."""
    torch = _torch()
    M, N = W.shape
    dev = W.device
    bits = torch.empty(layout_words(K, M, N), dtype=torch.int32, device=dev)
    alpha = torch.empty((K, M), dtype=torch.float32, device=dev)
    cs = torch.empty((K, N), dtype=torch.int16, device=dev) if colscale else None
    nb = int(lib().bsq_pack_workspace_bytes(M, N))
    ws = workspace if workspace is not None else torch.empty(nb, dtype=torch.uint8, device=dev)
    _check("bsq_pack", lib().bsq_pack(_ptr(W), M, N, K, BSG_PACK_COLSCALE if colscale else 0, _ptr(bits),
                                      _ptr(alpha), _ptr(cs), ws.data_ptr(), ws.numel(), _stream(dev)))
    return bits, alpha, cs


def salient_cols(N: int, g: int, s: int) -> int:
    """Physical salient columns S = s * N / g of the hybrid format."""
    return s * (N // g) if s else 0


def salient_scale_shape(K: int, M: int, N: int, g: int, s: int):
    """Shape of the word-grouped salient row scales: [K][ceil(S/32)][M][32/s]."""
    return (K, (salient_cols(N, g, s) + 31) // 32, M, 32 // s)


def bsq_pack_hybrid(W, K: int, g: int, s: int = 0, idx=None, colscale: bool = False, workspace=None):
    """Grouped bases (fp16 row scales per group of g, group-major [K][N/g][M]) plus, for s > 0, K
    salient-column bases over the S = s N/g columns idx (int32 device tensor).  Returns (bits, alpha,
    colscale or None, sbits or None, salpha or None, scolscale or None); fp16 values as int16."""
    torch = _torch()
    M, N = W.shape
    dev = W.device
    G = max(1, N // g)
    S = salient_cols(N, g, s)
    bits = torch.empty(layout_words(K, M, N), dtype=torch.int32, device=dev)
    alpha = torch.empty((K, G, M), dtype=torch.int16, device=dev)
    cs = torch.empty((K, N), dtype=torch.int16, device=dev) if colscale else None
    sbits = salpha = scs = None
    if s:
        sp = (S + 31) // 32 * 32
        sbits = torch.empty(layout_words(K, M, sp), dtype=torch.int32, device=dev)
        salpha = torch.empty(salient_scale_shape(K, M, N, g, s), dtype=torch.int16, device=dev)
        scs = torch.empty((K, S), dtype=torch.int16, device=dev) if colscale else None
    nb = int(lib().bsq_pack_hybrid_workspace_bytes(M, N, g, s))
    ws = workspace if workspace is not None else torch.empty(max(1, nb), dtype=torch.uint8, device=dev)
    _check("bsq_pack_hybrid", lib().bsq_pack_hybrid(
        _ptr(W), M, N, K, g, s, _ptr(idx), BSG_PACK_COLSCALE if colscale else 0, _ptr(bits), _ptr(alpha), _ptr(cs),
        _ptr(sbits), _ptr(salpha), _ptr(scs), ws.data_ptr(), ws.numel(), _stream(dev)))
    return bits, alpha, cs, sbits, salpha, scs


def bsq_pack_grouped(W, K: int, g: int, colscale: bool = False, workspace=None):
    """bsq_pack with one fp16 row scale per group of g columns.  Returns (bits, alpha fp16 bits int16
    [K][N/g][M] (group-major), colscale fp16 bits int16 [K][N] or None)."""
    return bsq_pack_hybrid(W, K, g, 0, None, colscale, workspace)[:3]


def bs_gemv_hybrid(bits, K: int, M: int, N: int, g: int, alpha, x, colscale=None, sbits=None, s: int = 0,
                   idx=None, salpha=None, scolscale=None, y=None, accumulate: bool = False):
    """y (fp32 [M][B]) = or += the grouped product plus, for s > 0, the salient-column bases read
    through idx (one launch per batch column)."""
    torch = _torch()
    B = _xshape(x, N)
    dev = x.device
    if y is None:
        y = torch.empty((M, B), dtype=torch.float32, device=dev)
    _check("bs_gemv_hybrid", lib().bs_gemv_hybrid(
        _ptr(bits), K, M, N, g, _ptr(alpha), _ptr(colscale), _ptr(sbits), s, _ptr(idx), _ptr(salpha),
        _ptr(scolscale), _ptr(x), _dtype_code(x), B, _ptr(y), 1 if accumulate else 0, _stream(dev)))
    return y


def bs_gemv_grouped(bits, K: int, M: int, N: int, g: int, alpha, x, colscale=None, y=None, accumulate: bool = False):
    """y (fp32 [M][B]) = or += the product with group-wise fp16 row scales alpha [K][N/g][M]
    (group-major, as bsq_pack_grouped writes them)."""
    torch = _torch()
    B = _xshape(x, N)
    dev = x.device
    if y is None:
        y = torch.empty((M, B), dtype=torch.float32, device=dev)
    _check("bs_gemv_grouped", lib().bs_gemv_grouped(_ptr(bits), K, M, N, g, _ptr(alpha), _ptr(colscale), _ptr(x),
                                                    _dtype_code(x), B, _ptr(y), 1 if accumulate else 0, _stream(dev)))
    return y


def bsq_pack_signs(S):
    """Device sign layout (K = 1) of a real matrix S (fp32 [M][N] on the GPU): bit = [S >= 0]."""
    torch = _torch()
    M, N = S.shape
    bits = torch.empty(layout_words(1, M, N), dtype=torch.int32, device=S.device)
    _check("bsq_pack_signs", lib().bsq_pack_signs(_ptr(S), M, N, _ptr(bits), _stream(S.device)))
    return bits


def bsq_absmean(X):
    torch = _torch()
    S, N = X.shape
    xbar = torch.empty(N, dtype=torch.float32, device=X.device)
    _check("bsq_absmean", lib().bsq_absmean(_ptr(X), S, N, _ptr(xbar), _stream(X.device)))
    return xbar


def bsq_salient(W, xbar, ns: int, alpha=None):
    """Protected int8 rows.  Returns (rows int32 [ns], q int8 [ns][N], s fp16-bits int16 [ns]);
    alpha (fp32 [K][M]) is updated in place (kept rows zeroed)."""
    torch = _torch()
    M, N = W.shape
    dev = W.device
    rows = torch.empty(max(ns, 1), dtype=torch.int32, device=dev)[:ns]
    q = torch.empty((max(ns, 1), N), dtype=torch.int8, device=dev)[:ns]
    s = torch.empty(max(ns, 1), dtype=torch.int16, device=dev)[:ns]
    K = 0 if alpha is None else alpha.shape[0]
    nb = int(lib().bsq_salient_workspace_bytes(M, N))
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    _check("bsq_salient", lib().bsq_salient(_ptr(W), M, N, _ptr(xbar), ns, rows.data_ptr(), q.data_ptr(),
                                            s.data_ptr(), _ptr(alpha), K, ws.data_ptr(), nb, _stream(dev)))
    return rows, q, s


def bsq_quantize_i8(x):
    torch = _torch()
    N = x.shape[0]
    B = _xshape(x, N)
    xq = torch.empty((N, B), dtype=torch.int8, device=x.device)
    sx = torch.empty(B, dtype=torch.float32, device=x.device)
    _check("bsq_quantize_i8", lib().bsq_quantize_i8(_ptr(x), _dtype_code(x), N, B, _ptr(xq), _ptr(sx),
                                                    _stream(x.device)))
    return xq, sx


def bsg_logical_to_layout(logical, K: int, M: int, N: int):
    torch = _torch()
    bits = torch.zeros(layout_words(K, M, N), dtype=torch.int32, device=logical.device)
    _check("bsg_logical_to_layout", lib().bsg_logical_to_layout(_ptr(logical), K, M, N, _ptr(bits),
                                                                _stream(logical.device)))
    return bits


def bsg_layout_to_logical(bits, K: int, M: int, N: int):
    torch = _torch()
    logical = torch.empty((K, M, N // 32), dtype=torch.int32, device=bits.device)
    _check("bsg_layout_to_logical", lib().bsg_layout_to_logical(_ptr(bits), K, M, N, _ptr(logical),
                                                                _stream(bits.device)))
    return logical


# ------------------------------------------------------------------ hot path
def bs_gemv(bits, K: int, M: int, N: int, alpha, x, colscale=None, y=None, accumulate: bool = False):
    """y (fp32 [M][B]) = or += sum_k alpha_k (.) (B_k (c_k (.) x)).  x: [N] or [N][B]."""
    torch = _torch()
    B = _xshape(x, N)
    dev = x.device
    if y is None:
        y = torch.empty((M, B), dtype=torch.float32, device=dev)
    _check("bs_gemv", lib().bs_gemv(_ptr(bits), K, M, N, _ptr(alpha), _ptr(colscale), _ptr(x), _dtype_code(x), B,
                                    _ptr(y), 1 if accumulate else 0, _stream(dev)))
    return y


class BsgProj(ctypes.Structure):
    """Mirror of bsg_proj and bsg_proj_grouped (include/bsg.h): the same field layout."""
    _fields_ = [("bits", ctypes.c_void_p), ("alpha", ctypes.c_void_p), ("colscale", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("M", ctypes.c_int)]


def bs_gemv_multi(projs, K: int, N: int, x, accumulate: bool = False):
    """Several bs_gemv products sharing x in one launch.  projs: list of (bits, M, alpha, colscale or None,
    y or None); returns the list of y (fp32 [M][B])."""
    torch = _torch()
    B = _xshape(x, N)
    dev = x.device
    arr = (BsgProj * max(1, len(projs)))()
    ys = []
    for i, (bits, M, alpha, cs, y) in enumerate(projs):
        if y is None:
            y = torch.empty((M, B), dtype=torch.float32, device=dev)
        ys.append(y)
        arr[i] = BsgProj(_ptr(bits), _ptr(alpha), _ptr(cs), _ptr(y), M)
    _check("bs_gemv_multi", lib().bs_gemv_multi(ctypes.cast(arr, ctypes.c_void_p), len(projs), K, N, _ptr(x),
                                                _dtype_code(x), B, 1 if accumulate else 0, _stream(dev)))
    return ys


def bs_gemv_grouped_multi(projs, K: int, N: int, g: int, x, accumulate: bool = False):
    """Several bs_gemv_grouped products sharing x, in one launch at B = 1.  projs: list of (bits, M,
    alpha fp16 [K][N/g][M], colscale or None, y or None); returns the list of y (fp32 [M][B])."""
    torch = _torch()
    B = _xshape(x, N)
    dev = x.device
    arr = (BsgProj * max(1, len(projs)))()
    ys = []
    for i, (bits, M, alpha, cs, y) in enumerate(projs):
        if y is None:
            y = torch.empty((M, B), dtype=torch.float32, device=dev)
        ys.append(y)
        arr[i] = BsgProj(_ptr(bits), _ptr(alpha), _ptr(cs), _ptr(y), M)
    _check("bs_gemv_grouped_multi", lib().bs_gemv_grouped_multi(ctypes.cast(arr, ctypes.c_void_p), len(projs), K, N,
                                                                g, _ptr(x), _dtype_code(x), B,
                                                                1 if accumulate else 0, _stream(dev)))
    return ys


def binlr_fit(W, r: int, v_init, rounds: int = 5, workspace=None):
    """Offline binary low-rank fit of W (fp32 [M][N] on the GPU).  v_init: int32/uint32 device tensor of the
    start vectors' logical sign words [r][N/32].  Returns (U_bits, V_bits, alpha_r_f16, rp, alpha, alpha_greedy,
    (sse_greedy, sse_refit), solved): device-layout signs and fp16 coefficients for rp = r rounded up to 32
    components (binlr_apply's inputs), and host numpy fp64 coefficients."""
    import numpy as np
    torch = _torch()
    M, N = W.shape
    dev = W.device
    rp = (r + 31) // 32 * 32
    U = torch.zeros(layout_words(1, M, rp), dtype=torch.int32, device=dev)
    V = torch.zeros(layout_words(1, rp, N), dtype=torch.int32, device=dev)
    a16 = torch.zeros(rp, dtype=torch.int16, device=dev)
    al = np.zeros(r, np.float64)
    ag = np.zeros(r, np.float64)
    sse = np.zeros(2, np.float64)
    solved = ctypes.c_int(0)
    nb = int(lib().binlr_fit_workspace_bytes(M, N, r))
    ws = workspace if workspace is not None else new_workspace(nb + 256, dev)
    wp = ws.data_ptr()
    wp_al = (wp + 255) // 256 * 256
    wn = ws.numel() * ws.element_size() - (wp_al - wp)
    _check("binlr_fit", lib().binlr_fit(_ptr(W), M, N, r, rounds, _ptr(v_init), _ptr(U), _ptr(V), _ptr(a16),
                                        al.ctypes.data_as(ctypes.c_void_p), ag.ctypes.data_as(ctypes.c_void_p),
                                        sse.ctypes.data_as(ctypes.c_void_p), ctypes.addressof(solved), wp_al, wn,
                                        _stream(dev)))
    return U, V, a16, rp, al, ag, (float(sse[0]), float(sse[1])), bool(solved.value)


def bs_gemv_i8(bits, K: int, M: int, N: int, alpha, xq, sx, want_acc: bool = True, want_y: bool = True,
               y=None, accumulate: bool = False) -> Tuple[Optional[object], Optional[object]]:
    """Exact int8-activation product.  Returns (acc int32 [K][M][B] or None, y fp32 [M][B] or None)."""
    torch = _torch()
    B = _xshape(xq, N)
    dev = xq.device
    acc = torch.empty((K, M, B), dtype=torch.int32, device=dev) if want_acc else None
    if want_y and y is None:
        y = torch.empty((M, B), dtype=torch.float32, device=dev)
    if not want_y:
        y = None
    _check("bs_gemv_i8", lib().bs_gemv_i8(_ptr(bits), K, M, N, _ptr(alpha), _ptr(xq), _ptr(sx), B, _ptr(acc),
                                          _ptr(y), 1 if accumulate else 0, _stream(dev)))
    return acc, y


def binlr_apply(U_bits, V_bits, alpha_r, r: int, M: int, N: int, x, y, workspace=None):
    """y += sum_j su(:, j) * alpha_r[j] * (sv(j, :) . x)  (binary low-rank correction)."""
    B = _xshape(x, N)
    dev = x.device
    nb = binlr_workspace_bytes(r, M, N, B)
    ws = workspace if workspace is not None else _WS.get(nb, dev)
    wp, wn = _ws_args(ws)
    _check("binlr_apply", lib().binlr_apply(_ptr(U_bits), _ptr(V_bits), _ptr(alpha_r), r, M, N, _ptr(x),
                                            _dtype_code(x), B, _ptr(y), wp, wn, _stream(dev)))
    return y


def bsg_linear(bits, K: int, M: int, N: int, alpha, x, colscale=None, lowrank=None, salient=None, y=None,
               accumulate: bool = False, workspace=None):
    """The whole layer in one pass over x: y (=/+=) bs_gemv term + binary low-rank correction + protected
    int8 rows.  lowrank = (U_bits, V_bits, alpha_r, r) or None; salient = (rows, q, s) or None (rows
    ascending)."""
    torch = _torch()
    B = _xshape(x, N)
    dev = x.device
    if y is None:
        y = torch.empty((M, B), dtype=torch.float32, device=dev)
    U, V, ar, r = lowrank if lowrank is not None else (None, None, None, 0)
    rows, q, sv = salient if salient is not None else (None, None, None)
    ns = rows.numel() if rows is not None else 0
    if ns == 0:
        rows = q = sv = None
    nb = int(lib().bsg_linear_workspace_bytes(r, B))
    ws = workspace if workspace is not None else (_WS.get(nb, dev) if nb else None)
    wp, wn = _ws_args(ws)
    _check("bsg_linear", lib().bsg_linear(_ptr(bits), K, M, N, _ptr(alpha), _ptr(colscale), _ptr(U), _ptr(V),
                                          _ptr(ar), r, _ptr(rows), ns, _ptr(q), _ptr(sv), _ptr(x), _dtype_code(x),
                                          B, _ptr(y), 1 if accumulate else 0, wp, wn, _stream(dev)))
    return y


def salient_int8_apply(rows, q, s, M: int, N: int, x, y):
    """y[rows[i]] += s_i * (q[i] . x)  (protected int8 rows)."""
    B = _xshape(x, N)
    ns = rows.numel()
    if ns == 0:
        return y
    _check("salient_int8_apply", lib().salient_int8_apply(_ptr(rows), ns, _ptr(q), _ptr(s), M, N, _ptr(x),
                                                          _dtype_code(x), B, _ptr(y), _stream(x.device)))
    return y
