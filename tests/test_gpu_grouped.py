"""GPU parity of group-wise row scales and of the salient-column (VCM)
branch against the CPU oracle.

Group-wise row scales: one fp16 scale per row, basis and group of g
consecutive columns.  The grouped packer matches bit for bit (sign words,
fp16 group scales, fp16 column scales); the grouped product stays within
the per-output bound

    2e-3 * sum_k sum_n |alpha_k[m][n / g]| * |c_k[n]| * |x[n, b]|

(the fp16 column scales c_k are 1 when absent).  The salient branch adds K
bases over the S = s N/g gathered columns idx; its packer output matches bit
for bit and its product adds the same bound over the gathered columns.  The
library keeps the global scales group-major, [K][N/g][M], and the salient
scales word-grouped, [K][ceil(S/32)][M][32/s]; the oracle keeps both
row-major, [K][M][N/g].

Cases cover group widths 64 (which forces more lanes per row than the
ungrouped plan), 128 and 256; s = 8, 16 and 32 salient columns per group,
with S a multiple of 32 or not; one to four bases; ragged M; bf16, fp16 and
fp32 activations; several batch columns; a partial last chunk of sign
words; accumulation into y; an index outside the matrix; and the
4096 x 4096 shape.
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


def _wg(salpha, s):
    """Oracle salient scales [K][M][G] -> the library's word-grouped [K][ceil(S/32)][M][32/s]."""
    K, M, G = salpha.shape
    gpw = 32 // s
    out = np.zeros((K, (G * s + 31) // 32, M, gpw), np.uint16)
    for j in range(G):
        out[:, j // gpw, :, j % gpw] = salpha[:, :, j]
    return out


def _bound(alpha16, cs16, xg, g, rel=2e-3):
    """rel * sum_k sum_j |a_k[m][j]| sum_{n in j} |c_k[n] x[n, b]| for scales [K][M][G], columns xg [n][B]."""
    K, M, G = alpha16.shape
    a = np.abs(oracle.f16_to_f64(alpha16))
    ax = np.abs(np.asarray(xg, np.float64))
    if ax.ndim == 1:
        ax = ax[:, None]
    c = np.ones((K, G * g)) if cs16 is None else np.abs(oracle.f16_to_f64(cs16))
    cx = (c[:, :, None] * ax[None]).reshape(K, G, g, -1).sum(2)           # [K][G][B]
    return rel * np.einsum("kmg,kgb->mb", a, cx)


def _tol(alpha, cs, x, g):
    return _bound(alpha, cs, x, g)


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
    np.testing.assert_array_equal(u16(alpha), _gm(ra))
    if cs:
        np.testing.assert_array_equal(u16(csd), rc)


def _inputs(M, N, K, g, B, cs, dt, seed):
    L = synth.random_bits(seed, K, M, N)
    r = np.random.default_rng([515, seed])
    alpha = np.abs(r.normal(0.016, 0.004, size=(K, M, N // g))).astype(np.float16).view(np.uint16)
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
    # more workgroups than compute units: two workgroups per unit
    (11008, 4096, 2, 128, 1, True, "f16"),
    (6144, 2048, 3, 128, 1, True, "bf16"),
]


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "M%d_N%d_K%d_g%d_B%d_cs%d_%s" % c)
def test_gemv_grouped_matches_oracle(case):
    M, N, K, g, B, cs, dt = case
    say("bs_gemv_grouped", case)
    L, alpha, csb, x = _inputs(M, N, K, g, B, cs, dt, M * 3 + N + K + g + B)
    bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
    y = bsg.bs_gemv_grouped(bits, K, M, N, g, f16_dev(_gm(alpha)), x_dev(x, dt),
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
    bsg.bs_gemv_grouped(bits, K, M, N, g, f16_dev(_gm(alpha)), x_dev(x, "bf16"), colscale=f16_dev(csb),
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
    a2 = oracle.f16_to_f64(alpha.reshape(K, M)).astype(np.float32)
    yg = bsg.bs_gemv_grouped(bits, K, M, N, N, f16_dev(_gm(alpha)), x_dev(x, "bf16"), colscale=f16_dev(csb))
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


# ------------------------------------------------------------------ salient columns (VCM)
def _group_idx(seed, N, g, s):
    """s distinct ascending columns of every group of g (seeded)."""
    r = np.random.default_rng([616, seed])
    return np.concatenate([np.sort(r.choice(g, s, replace=False)) + j * g for j in range(N // g)]).astype(np.int32)


def _logical_sbits(sbits, K, M, S):
    sp = (S + 31) // 32 * 32
    return u32(bsg.bsg_layout_to_logical(sbits, K, M, sp)).reshape(K, M, -1)


HYBRID_PACK_CASES = [
    # M, N, K, g, s, colscale
    (256, 512, 2, 128, 16, True),
    (130, 1024, 1, 64, 8, False),
    (70, 1088, 2, 64, 8, True),      # S = 136: a partial last salient word
    (300, 768, 3, 256, 32, True),
    (1, 256, 2, 128, 8, False),
    (4096, 4096, 2, 128, 16, True),
]


@pytest.mark.parametrize("case", HYBRID_PACK_CASES, ids=lambda c: "M%d_N%d_K%d_g%d_s%d_cs%d" % c)
def test_pack_hybrid_bit_exact(case):
    M, N, K, g, s, cs = case
    say("bsq_pack_hybrid", case)
    W = synth.weights(M + N + g + s, K, M, N)
    idx = _group_idx(M + s, N, g, s)
    S = s * (N // g)
    bits, alpha, csd, sbits, salpha, scs = bsg.bsq_pack_hybrid(to_dev(W), K, g, s, to_dev(idx), colscale=cs)
    torch.cuda.synchronize()
    rb, ra, rc, rsb, rsa, rsc = oracle.pack_hybrid(W, K, g, s, idx, cs)
    np.testing.assert_array_equal(u32(bsg.bsg_layout_to_logical(bits, K, M, N)).reshape(K, M, -1), rb)
    np.testing.assert_array_equal(u16(alpha), _gm(ra))
    np.testing.assert_array_equal(_logical_sbits(sbits, K, M, S), rsb)
    np.testing.assert_array_equal(u16(salpha), _wg(rsa, s))
    if cs:
        np.testing.assert_array_equal(u16(csd), rc)
        np.testing.assert_array_equal(u16(scs), rsc)


def _hybrid_inputs(M, N, K, g, s, B, cs, dt, seed):
    L, alpha, csb, x = _inputs(M, N, K, g, B, cs, dt, seed)
    S = s * (N // g)
    r = np.random.default_rng([717, seed])
    SL = synth.random_bits(seed + 1, K, M, S)
    salpha = np.abs(r.normal(0.01, 0.003, size=(K, M, N // g))).astype(np.float16).view(np.uint16)
    scs = r.uniform(0.5, 1.5, size=(K, S)).astype(np.float16).view(np.uint16) if cs else None
    idx = _group_idx(seed, N, g, s)
    return L, alpha, csb, SL, salpha, scs, idx, x


def _hybrid_run(M, N, K, g, s, cs, dt, L, alpha, csb, SL, salpha, scs, idx, x, y=None, accumulate=False):
    S = s * (N // g)
    sp = (S + 31) // 32 * 32
    bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
    sl = np.zeros((K, M, sp // 32), np.uint32)
    sl[:, :, :SL.shape[2]] = SL
    sbits = bsg.bsg_logical_to_layout(to_dev(sl.view(np.int32)), K, M, sp)
    return bsg.bs_gemv_hybrid(bits, K, M, N, g, f16_dev(_gm(alpha)), x_dev(x, dt),
                              colscale=f16_dev(csb) if cs else None, sbits=sbits, s=s, idx=to_dev(idx),
                              salpha=f16_dev(_wg(salpha, s)), scolscale=f16_dev(scs) if cs else None,
                              y=y, accumulate=accumulate)


def _hybrid_tol(alpha, csb, salpha, scs, idx, x, g, s):
    xa = np.asarray(x, np.float64)
    if xa.ndim == 1:
        xa = xa[:, None]
    return _bound(alpha, csb, xa, g) + _bound(salpha, scs, xa[idx], s)


HYBRID_CASES = [
    # M, N, K, g, s, B, colscale, dtype
    (256, 512, 2, 128, 16, 1, True, "bf16"),
    (130, 1024, 1, 64, 8, 1, False, "bf16"),
    (200, 1088, 2, 64, 8, 1, True, "f16"),       # S = 136
    (64, 768, 3, 256, 32, 1, False, "f32"),
    (300, 1024, 3, 128, 8, 1, True, "bf16"),
    (96, 512, 4, 64, 16, 1, True, "bf16"),
    (1000, 4096, 4, 128, 8, 1, False, "f16"),
    (130, 1024, 2, 128, 16, 3, True, "bf16"),
    (70, 576, 3, 64, 8, 2, True, "f16"),         # S = 72
    (4096, 4096, 2, 128, 16, 1, True, "bf16"),
    (4096, 4096, 2, 128, 8, 1, True, "bf16"),
]


@pytest.mark.parametrize("case", HYBRID_CASES, ids=lambda c: "M%d_N%d_K%d_g%d_s%d_B%d_cs%d_%s" % c)
def test_gemv_hybrid_matches_oracle(case):
    M, N, K, g, s, B, cs, dt = case
    say("bs_gemv_hybrid", case)
    L, alpha, csb, SL, salpha, scs, idx, x = _hybrid_inputs(M, N, K, g, s, B, cs, dt, M + N + K + g + s + B)
    y = _hybrid_run(M, N, K, g, s, cs, dt, L, alpha, csb, SL, salpha, scs, idx, x)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv_hybrid(L, K, M, N, g, alpha, csb, SL, s, idx, salpha, scs, x)
    check_close(y.cpu().numpy(), ref, _hybrid_tol(alpha, csb, salpha, scs, idx, x, g, s) + 1e-9,
                "hybrid %s" % (case,))


def test_gemv_hybrid_accumulates():
    M, N, K, g, s, B = 130, 1024, 2, 128, 8, 2
    say("bs_gemv_hybrid accumulate", M, N, K, g, s, B)
    L, alpha, csb, SL, salpha, scs, idx, x = _hybrid_inputs(M, N, K, g, s, B, True, "bf16", 41)
    y0 = np.random.default_rng(6).standard_normal((M, B)).astype(np.float32)
    y = to_dev(y0)
    _hybrid_run(M, N, K, g, s, True, "bf16", L, alpha, csb, SL, salpha, scs, idx, x, y=y, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv_hybrid(L, K, M, N, g, alpha, csb, SL, s, idx, salpha, scs, x) + y0
    check_close(y.cpu().numpy(), ref, _hybrid_tol(alpha, csb, salpha, scs, idx, x, g, s) + 1e-6,
                "hybrid accumulate")


def test_gemv_hybrid_index_outside_the_matrix_reads_zero():
    """Salient columns whose index lies outside [0, N) contribute nothing: the
    same as a zero column scale there (the oracle takes any valid index)."""
    M, N, K, g, s = 130, 512, 2, 128, 16
    say("bs_gemv_hybrid bad index", M, N, K, g, s)
    L, alpha, csb, SL, salpha, scs, idx, x = _hybrid_inputs(M, N, K, g, s, 1, True, "bf16", 43)
    bad = [3, 17, 40]
    idx_bad = idx.copy()
    idx_bad[bad] = [N, -1, 1 << 30]
    y = _hybrid_run(M, N, K, g, s, True, "bf16", L, alpha, csb, SL, salpha, scs, idx_bad, x)
    torch.cuda.synchronize()
    scs0 = scs.copy()
    scs0[:, bad] = 0
    ref = oracle.sign_gemv_hybrid(L, K, M, N, g, alpha, csb, SL, s, idx, salpha, scs0, x)
    check_close(y.cpu().numpy(), ref, _hybrid_tol(alpha, csb, salpha, scs, idx, x, g, s) + 1e-9, "bad index")


def test_gemv_hybrid_without_salient_columns_is_the_grouped_product():
    M, N, K, g = 200, 1024, 2, 128
    say("bs_gemv_hybrid s=0", M, N, K, g)
    L, alpha, csb, x = _inputs(M, N, K, g, 1, True, "bf16", 45)
    bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
    args = (bits, K, M, N, g, f16_dev(_gm(alpha)), x_dev(x, "bf16"))
    y1 = bsg.bs_gemv_hybrid(*args, colscale=f16_dev(csb))
    y2 = bsg.bs_gemv_grouped(*args, colscale=f16_dev(csb))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_pack_then_gemv_hybrid_end_to_end():
    M, N, K, g, s = 300, 1024, 2, 128, 16
    say("bsq_pack_hybrid -> bs_gemv_hybrid", M, N, K, g, s)
    W = synth.weights(13, K, M, N)
    idx = _group_idx(13, N, g, s)
    out = bsg.bsq_pack_hybrid(to_dev(W), K, g, s, to_dev(idx), colscale=True)
    bits, alpha, csd, sbits, salpha, scs = out
    x = synth.random_x(14, N, 1, "bf16")
    y = bsg.bs_gemv_hybrid(bits, K, M, N, g, alpha, x_dev(x, "bf16"), colscale=csd, sbits=sbits, s=s,
                           idx=to_dev(idx), salpha=salpha, scolscale=scs)
    torch.cuda.synchronize()
    rb, ra, rc, rsb, rsa, rsc = oracle.pack_hybrid(W, K, g, s, idx, True)
    ref = oracle.sign_gemv_hybrid(rb, K, M, N, g, ra, rc, rsb, s, idx, rsa, rsc, x)
    check_close(y.cpu().numpy(), ref, _hybrid_tol(ra, rc, rsa, rsc, idx, x, g, s) + 1e-9, "pack -> gemv hybrid")


# ------------------------------------------------------------------ batches on the matrix cores
# B >= 4 columns of 16-bit x with g >= 128 and M % 4 == 0 (and fp16 x when
# there are column scales) run on the matrix cores; the others per column on
# the table kernel.  Both are held to the per-group bound; the matrix-core
# cases also to a ten times tighter one (exact products, fp32 sums).
GROUPED_BATCH_CASES = [
    # M, N, K, g, B, colscale, dtype, matrix cores
    (256, 512, 2, 128, 4, False, "bf16", True),
    (132, 1024, 3, 256, 8, True, "f16", True),
    (1000, 4096, 4, 128, 16, False, "bf16", True),
    (4096, 4096, 2, 128, 16, True, "f16", True),
    (300, 1024, 1, 512, 32, False, "f16", True),
    (9000, 512, 2, 128, 20, True, "f16", True),     # 32-row tiles, two batch launches
    (130, 1024, 2, 128, 16, True, "f16", False),    # M % 4 != 0
    (200, 2048, 2, 64, 8, True, "f16", False),      # g = 64
    (256, 1024, 2, 128, 8, True, "bf16", False),    # column scales with bf16 x
]


@pytest.mark.parametrize("case", GROUPED_BATCH_CASES, ids=lambda c: "M%d_N%d_K%d_g%d_B%d_cs%d_%s_mc%d" % c)
def test_gemv_grouped_batches(case):
    M, N, K, g, B, cs, dt, mc = case
    say("bs_gemv_grouped batch", case)
    L, alpha, csb, x = _inputs(M, N, K, g, B, cs, dt, M + N + K + g + B + 7)
    bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
    y = bsg.bs_gemv_grouped(bits, K, M, N, g, f16_dev(_gm(alpha)), x_dev(x, dt),
                            colscale=f16_dev(csb) if cs else None)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv_grouped(L, K, M, N, g, alpha, x, csb)
    check_close(y.cpu().numpy(), ref, _bound(alpha, csb, x, g, 2e-4 if mc else 2e-3) + 1e-9,
                "grouped batch %s" % (case,))


# B >= 4 columns of fp16 x: the main bases on the matrix cores, then the salient
# bases in a second matrix-core launch (gathered x in LDS, the group scale
# folded into the A values); bf16 x or M % 4 != 0: per column on the table
# kernel.  All within the per-group bound.
HYBRID_BATCH_CASES = [
    # M, N, K, g, s, B, colscale, dtype
    (256, 512, 2, 128, 16, 4, True, "f16"),
    (132, 1152, 2, 128, 8, 8, True, "f16"),       # S = 72: a partial tile and word
    (1000, 4096, 3, 128, 16, 16, False, "f16"),
    (4096, 4096, 2, 128, 8, 16, True, "f16"),
    (300, 1024, 4, 256, 32, 20, True, "f16"),     # two batch launches
    (9000, 512, 2, 128, 16, 16, True, "f16"),     # 32-row tiles
    (256, 512, 2, 128, 16, 4, True, "bf16"),      # table path
    (130, 1024, 2, 128, 8, 8, True, "f16"),       # M % 4 != 0: table path
]


@pytest.mark.parametrize("case", HYBRID_BATCH_CASES, ids=lambda c: "M%d_N%d_K%d_g%d_s%d_B%d_cs%d_%s" % c)
def test_gemv_hybrid_batches(case):
    M, N, K, g, s, B, cs, dt = case
    say("bs_gemv_hybrid batch", case)
    L, alpha, csb, SL, salpha, scs, idx, x = _hybrid_inputs(M, N, K, g, s, B, cs, dt, M + N + K + g + s + B + 11)
    y = _hybrid_run(M, N, K, g, s, cs, dt, L, alpha, csb, SL, salpha, scs, idx, x)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv_hybrid(L, K, M, N, g, alpha, csb, SL, s, idx, salpha, scs, x)
    check_close(y.cpu().numpy(), ref, _hybrid_tol(alpha, csb, salpha, scs, idx, x, g, s) + 1e-9,
                "hybrid batch %s" % (case,))


def test_gemv_hybrid_batch_index_outside_the_matrix_reads_zero():
    M, N, K, g, s, B = 256, 512, 2, 128, 16, 8
    say("bs_gemv_hybrid batch bad index", M, N, K, g, s, B)
    L, alpha, csb, SL, salpha, scs, idx, x = _hybrid_inputs(M, N, K, g, s, B, True, "f16", 47)
    bad = [0, 31, 63]
    idx_bad = idx.copy()
    idx_bad[bad] = [N, -7, 1 << 29]
    y = _hybrid_run(M, N, K, g, s, True, "f16", L, alpha, csb, SL, salpha, scs, idx_bad, x)
    torch.cuda.synchronize()
    scs0 = scs.copy()
    scs0[:, bad] = 0
    ref = oracle.sign_gemv_hybrid(L, K, M, N, g, alpha, csb, SL, s, idx, salpha, scs0, x)
    check_close(y.cpu().numpy(), ref, _hybrid_tol(alpha, csb, salpha, scs, idx, x, g, s) + 1e-9, "batch bad index")


# ------------------------------------------------------------------ fused projections
GROUPED_MULTI_CASES = [
    # heights, N, K, g, B, colscale, dtype
    ((256, 64, 64), 1024, 2, 128, 1, True, "f16"),            # q, k, v
    ((130, 0, 33, 200), 512, 1, 64, 1, False, "bf16"),        # ragged, an empty projection
    ((64,) * 8, 768, 3, 256, 1, True, "bf16"),                # eight projections
    ((300, 100), 1088, 4, 64, 1, True, "f32"),                # partial last chunk
    ((256, 128), 1024, 2, 128, 3, True, "bf16"),              # B > 1: a call each
    ((256, 128), 1024, 2, 128, 16, True, "f16"),              # B = 16: matrix cores each
]


@pytest.mark.parametrize("case", GROUPED_MULTI_CASES, ids=lambda c: "P%d_N%d_K%d_g%d_B%d_cs%d_%s" % ((len(c[0]),) + c[1:]))
def test_gemv_grouped_multi_matches_oracle(case):
    Ms, N, K, g, B, cs, dt = case
    say("bs_gemv_grouped_multi", case)
    x = synth.random_x(sum(Ms) + N, N, B, dt)
    projs, refs = [], []
    for i, M in enumerate(Ms):
        L, alpha, csb, _ = _inputs(max(M, 1), N, K, g, B, cs, dt, 900 + 31 * i + M)
        L, alpha = L[:, :M], alpha[:, :M]
        bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N) if M else \
            torch.zeros(16, dtype=torch.int32, device=DEV)
        projs.append((bits, M, f16_dev(_gm(alpha)) if M else torch.zeros(8, dtype=torch.int16, device=DEV),
                      f16_dev(csb) if cs else None, None))
        refs.append((L, alpha, csb))
    ys = bsg.bs_gemv_grouped_multi(projs, K, N, g, x_dev(x, dt))
    torch.cuda.synchronize()
    for (L, alpha, csb), y, M in zip(refs, ys, Ms):
        if M == 0:
            continue
        ref = oracle.sign_gemv_grouped(L, K, M, N, g, alpha, x, csb)
        check_close(y.cpu().numpy(), ref, _tol(alpha, csb, x, g) + 1e-9, "grouped multi %s M=%d" % (case[1:], M))


def test_gemv_grouped_multi_accumulates():
    Ms, N, K, g = (256, 64, 64), 1024, 2, 128
    say("bs_gemv_grouped_multi accumulate", Ms)
    x = synth.random_x(5, N, 1, "bf16")
    projs, refs = [], []
    for i, M in enumerate(Ms):
        L, alpha, csb, _ = _inputs(M, N, K, g, 1, True, "bf16", 950 + i)
        y0 = np.random.default_rng(i).standard_normal((M, 1)).astype(np.float32)
        bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)
        projs.append((bits, M, f16_dev(_gm(alpha)), f16_dev(csb), to_dev(y0)))
        refs.append((L, alpha, csb, y0))
    ys = bsg.bs_gemv_grouped_multi(projs, K, N, g, x_dev(x, "bf16"), accumulate=True)
    torch.cuda.synchronize()
    for (L, alpha, csb, y0), y, M in zip(refs, ys, Ms):
        ref = oracle.sign_gemv_grouped(L, K, M, N, g, alpha, x, csb) + y0
        check_close(y.cpu().numpy(), ref, _tol(alpha, csb, x, g) + 1e-6, "grouped multi accumulate M=%d" % M)
