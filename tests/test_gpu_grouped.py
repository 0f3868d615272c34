"""GPU parity of group-wise row scales (one scale per row, basis and group of
g consecutive columns) against the CPU oracle: the grouped packer bit for bit
(sign words, fp32 group scales, fp16 column scales) and the grouped product
within the per-output bound

    2e-3 * sum_k sum_n |alpha_k[m][n / g]| * |c_k[n]| * |x[n, b]|

(the fp16 column scales c_k are 1 when absent).  The library keeps the
scales group-major, [K][N/g][M]; the oracle row-major, [K][M][N/g].

Cases cover group widths 64 (which forces more lanes per row than the
ungrouped plan), 128 and 256; one to four bases; ragged M; bf16, fp16 and
fp32 activations; several batch columns; a partial last chunk of sign
words; accumulation into y; and the 4096 x 4096 shape.
"""
import numpy as np
import pytest

import oracle
from bit_gemv_packed_amd import synth
from gpu_util import DEV, check_close, f16_dev, say, to_dev, u16, u32, x_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import bit_gemv_packed_amd as bsg  # noqa: E402


def _gm(alpha):
    """Oracle scales [K][M][N/g] -> the library's group-major [K][N/g][M]."""
    return np.ascontiguousarray(np.asarray(alpha).transpose(0, 2, 1))


def _tol(alpha, cs, x, g, rel=2e-3):
    K, M, G = alpha.shape
    ax = np.abs(np.asarray(x, np.float64))
    if ax.ndim == 1:
        ax = ax[:, None]
    c = np.ones((K, G * g)) if cs is None else np.abs(cs.view(np.float16).astype(np.float64))
    # per group: sum over its columns of |c_k[n]| |x[n, b]|
    cx = (c[:, :, None] * ax[None]).reshape(K, G, g, -1).sum(2)           # [K][G][B]
    return rel * np.einsum("kmg,kgb->mb", np.abs(alpha.astype(np.float64)), cx)


PACK_CASES = [
    # M, N, K, g, colscale
    (256, 256, 1, 64, False),
    (130, 512, 2, 128, True),
    (70, 1024, 3, 256, True),
    (300, 384, 4, 128, False),
    (1, 128, 2, 64, True),
    (4096, 4096, 2, 128, True),
]


@pytest.mark.parametrize("case", PACK_CASES, ids=lambda c: "M%d_N%d_K%d_g%d_cs%d" % c)
def test_pack_grouped_bit_exact(case):
    M, N, K, g, cs = case
    say("bsq_pack_grouped", case)
    W = synth.weights(M + N + g, K, M, N)
    bits, alpha, csd = bsg.bsq_pack_grouped(to_dev(W), K, g, colscale=cs)
    torch.cuda.synchronize()
    rb, ra, rc = oracle.pack_grouped(W, K, g, cs)
    np.testing.assert_array_equal(u32(bsg.bsg_layout_to_logical(bits, K, M, N)).reshape(K, M, -1), rb)
    np.testing.assert_array_equal(alpha.cpu().numpy().view(np.uint32), _gm(ra).view(np.uint32))
    if cs:
        np.testing.assert_array_equal(u16(csd), rc)


def _inputs(M, N, K, g, B, cs, dt, seed):
    L = synth.random_bits(seed, K, M, N)
    r = np.random.default_rng([515, seed])
    alpha = np.abs(r.normal(0.016, 0.004, size=(K, M, N // g))).astype(np.float32)
    csb = r.uniform(0.5, 1.5, size=(K, N)).astype(np.float16).view(np.uint16) if cs else None
    x = synth.random_x(seed, N, B, dt)
    return L, alpha, csb, x


GEMV_CASES = [
    # M, N, K, g, B, colscale, dtype
    (256, 512, 1, 64, 1, False, "bf16"),
    (130, 1024, 2, 128, 1, True, "bf16"),
    (200, 2048, 2, 64, 1, True, "f16"),
    (64, 768, 3, 256, 1, False, "f32"),
    (300, 1024, 3, 128, 1, True, "bf16"),
    (96, 512, 4, 64, 1, True, "bf16"),
    (1000, 4096, 4, 128, 1, False, "f16"),
    (130, 1024, 2, 128, 3, True, "bf16"),
    (70, 512, 4, 256, 5, False, "f32"),
    (4096, 4096, 2, 128, 1, True, "bf16"),
    # a partial last chunk of sign words (N / 32 not a multiple of 8)
    (150, 1088, 2, 64, 1, True, "bf16"),
    (70, 576, 3, 64, 2, True, "f16"),
    (33, 1344, 1, 64, 1, False, "f32"),
]


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "M%d_N%d_K%d_g%d_B%d_cs%d_%s" % c)
def test_gemv_grouped_matches_oracle(case):
    M, N, K, g, B, cs, dt = case
    say("bs_gemv_grouped", case)
    L, alpha, csb, x = _inputs(M, N, K, g, B, cs, dt, M * 3 + N + K + g + B)
    bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
    y = bsg.bs_gemv_grouped(bits, K, M, N, g, to_dev(_gm(alpha)), x_dev(x, dt),
                            colscale=f16_dev(csb) if cs else None)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv_grouped(L, K, M, N, g, alpha, x, csb)
    check_close(y.cpu().numpy(), ref, _tol(alpha, csb, x, g) + 1e-9, "grouped %s" % (case,))


def test_gemv_grouped_accumulates():
    M, N, K, g, B = 130, 1024, 2, 128, 2
    say("bs_gemv_grouped accumulate", M, N, K, g, B)
    L, alpha, csb, x = _inputs(M, N, K, g, B, True, "bf16", 31)
    bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
    y0 = np.random.default_rng(5).standard_normal((M, B)).astype(np.float32)
    y = to_dev(y0)
    bsg.bs_gemv_grouped(bits, K, M, N, g, to_dev(_gm(alpha)), x_dev(x, "bf16"), colscale=f16_dev(csb),
                        y=y, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv_grouped(L, K, M, N, g, alpha, x, csb) + y0
    check_close(y.cpu().numpy(), ref, _tol(alpha, csb, x, g) + 1e-6, "grouped accumulate")


def test_gemv_grouped_with_one_group_equals_ungrouped():
    """g = N: one scale per row and basis, so the grouped product is the
    ungrouped one on the same inputs (both sides checked against the oracle's
    ungrouped product)."""
    M, N, K = 200, 512, 2
    say("bs_gemv_grouped g=N", M, N, K)
    L, alpha, csb, x = _inputs(M, N, K, N, 1, True, "bf16", 77)
    bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
    a2 = alpha.reshape(K, M)
    yg = bsg.bs_gemv_grouped(bits, K, M, N, N, to_dev(_gm(alpha)), x_dev(x, "bf16"), colscale=f16_dev(csb))
    y1 = bsg.bs_gemv(bits, K, M, N, to_dev(a2), x_dev(x, "bf16"), colscale=f16_dev(csb))
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, a2, x, csb)
    tol = oracle.tolerance(x, alpha=a2, colscale_f16=csb) + 1e-9
    check_close(yg.cpu().numpy(), ref, tol, "grouped g=N")
    check_close(y1.cpu().numpy(), ref, tol, "ungrouped")


def test_pack_then_gemv_grouped_end_to_end():
    M, N, K, g = 300, 1024, 2, 128
    say("bsq_pack_grouped -> bs_gemv_grouped", M, N, K, g)
    W = synth.weights(11, K, M, N)
    bits, alpha, csd = bsg.bsq_pack_grouped(to_dev(W), K, g, colscale=True)
    x = synth.random_x(12, N, 1, "bf16")
    y = bsg.bs_gemv_grouped(bits, K, M, N, g, alpha, x_dev(x, "bf16"), colscale=csd)
    torch.cuda.synchronize()
    rb, ra, rc = oracle.pack_grouped(W, K, g, True)
    ref = oracle.sign_gemv_grouped(rb, K, M, N, g, ra, x, rc)
    check_close(y.cpu().numpy(), ref, _tol(ra, rc, x, g) + 1e-9, "pack -> gemv grouped")
