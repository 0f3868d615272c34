"""GPU parity of the batched matrix-core sign product (bs_gemv with B >= 4
columns of bf16 / fp16 x and no column scales) against the CPU oracle.

The matrix-core path multiplies exact +-1 signs by exact bf16 / fp16 x and
sums in fp32, so its error is fp32 rounding of the sums alone: each output
is held to 2e-4 * sum_k |alpha_k[m]| * sum_n |x[n,b]|, ten times tighter
than the bound of the table path (steps per wavefront plus the cross-wave
sum stay below a few hundred fp32 additions at these sizes: (few hundred) *
2^-24 << 2e-4).

Cases cover one and several launch groups of bases (K up to 8), row tiles
of 16 and 32 rows (M large enough for 256 workgroups of 32 rows), ragged M
(partial row tiles, a partial 64-row block), N from one 32-column step to
many tiles per wavefront, batch widths below, at and above 16 (several
launches) and not a multiple of 8 (2-byte x loads), x at an address that is
not 16-byte aligned, and accumulation into y.
"""
import numpy as np
import pytest

import oracle
from bit_gemv_packed_amd import synth
from gpu_util import DEV, check_close, say, to_dev, x_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import bit_gemv_packed_amd as bsg  # noqa: E402

MFMA_REL = 2e-4

MFMA_CASES = [
    # K, M, N, B, x dtype
    (1, 16, 32, 4, "bf16"),
    (2, 64, 128, 8, "bf16"),
    (2, 100, 4096, 16, "bf16"),
    (3, 257, 544, 5, "f16"),
    (4, 130, 1056, 20, "bf16"),
    (5, 77, 320, 16, "f16"),
    (8, 65, 256, 8, "bf16"),
    (6, 300, 2080, 33, "bf16"),
    (2, 9000, 256, 16, "bf16"),   # 32-row tiles
    (1, 8200, 1024, 64, "f16"),   # 32-row tiles, four batch launches
    (4, 8192, 512, 8, "bf16"),    # 32-row tiles, 4 bases
    (3, 8193, 96, 6, "bf16"),     # 32-row tiles, ragged tail
    (2, 48, 14336, 4, "bf16"),    # long rows: many tiles per wavefront
    (7, 33, 32, 17, "f16"),
]


def _inputs(case):
    K, M, N, B, dt = case
    seed = 50000 + K * 7919 + M * 31 + N + B
    L = synth.random_bits(seed, K, M, N)
    alpha, _ = synth.random_scales(seed, K, M, N, False)
    x = synth.random_x(seed, N, B, dt, "normal")
    return L, alpha, x


def _layout(L, K, M, N):
    return bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N)


@pytest.mark.parametrize("case", MFMA_CASES, ids=lambda c: "K%d_M%d_N%d_B%d_%s" % c)
def test_mfma_product_matches_oracle(case):
    K, M, N, B, dt = case
    say("mfma bs_gemv", case)
    L, alpha, x = _inputs(case)
    bits = _layout(L, K, M, N)
    ad = to_dev(alpha)
    xd = x_dev(x, dt)
    y = bsg.bs_gemv(bits, K, M, N, ad, xd)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, alpha, x)
    tol = oracle.tolerance(x, alpha=alpha, rel=MFMA_REL)
    check_close(y.cpu().numpy(), ref, tol, "mfma bs_gemv %s" % (case,))
    y2 = bsg.bs_gemv(bits, K, M, N, ad, xd)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)  # fixed-order sums: the same bits on every call


@pytest.mark.parametrize("case", [(2, 130, 1056, 16, "bf16"), (5, 200, 544, 8, "f16"), (3, 8300, 256, 24, "bf16")],
                         ids=lambda c: "K%d_M%d_N%d_B%d_%s" % c)
def test_mfma_accumulate_and_unaligned_x(case):
    K, M, N, B, dt = case
    say("mfma accumulate/unaligned", case)
    L, alpha, x = _inputs(case)
    bits = _layout(L, K, M, N)
    ad = to_dev(alpha)
    # x at an address 8 bytes past a 16-byte boundary: the 2-byte load form
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    buf = torch.zeros(N * B + 4, dtype=tdt, device=DEV)
    xv = buf[4:].view(N, B)
    xv.copy_(x_dev(x, dt))
    assert xv.data_ptr() % 16 == 8
    y0 = torch.from_numpy(synth.random_x(K + M, M, B, "f32", "normal")).to(DEV)
    y = y0.clone()
    bsg.bs_gemv(bits, K, M, N, ad, xv, y=y, accumulate=True)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, alpha, x) + y0.cpu().numpy().astype(np.float64)
    tol = oracle.tolerance(x, alpha=alpha, rel=MFMA_REL) + 1e-6 * np.abs(y0.cpu().numpy())
    check_close(y.cpu().numpy(), ref, tol, "mfma accumulate %s" % (case,))
    # the aligned copy gives the same result as the unaligned one
    ya = bsg.bs_gemv(bits, K, M, N, ad, x_dev(x, dt))
    yu = bsg.bs_gemv(bits, K, M, N, ad, xv)
    torch.cuda.synchronize()
    assert torch.equal(ya, yu)


def test_mfma_agrees_with_table_path_on_integer_x():
    """Small-integer x: every partial sum is an integer below 2^24, so both
    the matrix-core path (B = 8) and the table path (the same columns one at a
    time, B = 1) are exact before the row scale, and agree to a few fp32
    roundings of the scaled sum."""
    K, M, N, B = 3, 300, 2048, 8
    say("mfma vs table, integer x", K, M, N, B)
    L = synth.random_bits(77, K, M, N)
    alpha, _ = synth.random_scales(77, K, M, N, False)
    g = np.random.default_rng([9100, 1])
    x = g.integers(-8, 9, size=(N, B)).astype(np.float32)
    bits = _layout(L, K, M, N)
    ad = to_dev(alpha)
    xd = x_dev(x, "bf16")
    y = bsg.bs_gemv(bits, K, M, N, ad, xd)
    cols = [bsg.bs_gemv(bits, K, M, N, ad, xd[:, b].contiguous()) for b in range(B)]
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, alpha, x)
    # y = sum_k alpha_k * S_k with exact integer S_k: only the three fp32
    # products and their sum round
    tol = oracle.tolerance(x, alpha=alpha, rel=1e-6)
    check_close(y.cpu().numpy(), ref, tol, "mfma integer x")
    for b in range(B):
        check_close(cols[b][:, 0].cpu().numpy(), y[:, b].cpu().numpy().astype(np.float64), tol[:, b],
                    "table vs mfma, column %d" % b)


# ------------------------------------------------------------------ column scales (fp16 x)
# The A values are the column scales' own fp16 bits with the sign flipped for
# a set weight bit, so products with fp16 x stay exact and the same 2e-4 bound
# holds (sum_n |c_k[n] x[n,b]| in place of sum_n |x[n,b]|).
CS_CASES = [
    # K, M, N, B, negative scales too
    (1, 16, 32, 4, False),
    (2, 64, 128, 8, False),
    (2, 100, 4096, 16, False),
    (3, 257, 544, 4, True),
    (4, 130, 1056, 20, False),
    (6, 300, 2080, 32, True),     # two launches of bases
    (2, 9000, 256, 16, False),    # 32-row tiles
    (8, 65, 256, 8, True),
    (2, 200, 512, 6, False),      # B % 4 != 0: the table path
]


@pytest.mark.parametrize("case", CS_CASES, ids=lambda c: "K%d_M%d_N%d_B%d_neg%d" % c)
def test_mfma_colscale_matches_oracle(case):
    K, M, N, B, neg = case
    say("mfma bs_gemv colscale", case)
    seed = 60000 + K * 7919 + M * 31 + N + B
    L = synth.random_bits(seed, K, M, N)
    alpha, cs = synth.random_scales(seed, K, M, N, True)
    if neg:
        r = np.random.default_rng([61, seed])
        cs = (cs.view(np.float16) * np.where(r.integers(0, 2, cs.shape) == 1, 1, -1).astype(np.float16)).view(np.uint16)
    x = synth.random_x(seed, N, B, "f16", "normal")
    bits = _layout(L, K, M, N)
    csd = torch.from_numpy(np.ascontiguousarray(cs).view(np.int16)).to(DEV)
    y = bsg.bs_gemv(bits, K, M, N, to_dev(alpha), x_dev(x, "f16"), colscale=csd)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, alpha, x, cs)
    rel = MFMA_REL if B % 4 == 0 else 2e-3
    tol = oracle.tolerance(x, alpha=alpha, colscale_f16=cs, rel=rel)
    check_close(y.cpu().numpy(), ref, tol + 1e-9, "mfma colscale %s" % (case,))


def test_mfma_colscale_equals_the_table_path_on_small_integers():
    """Small-integer x and power-of-two column scales: every partial sum is
    exact on both paths, so the batched product equals the per-column (table)
    products up to the final row-scale rounding."""
    K, M, N, B = 2, 200, 1024, 8
    say("mfma colscale vs table", K, M, N, B)
    L = synth.random_bits(71, K, M, N)
    alpha, _ = synth.random_scales(71, K, M, N, False)
    r = np.random.default_rng(71)
    cs = (2.0 ** r.integers(-2, 3, size=(K, N))).astype(np.float16).view(np.uint16)
    x = r.integers(-8, 9, size=(N, B)).astype(np.float32)
    bits = _layout(L, K, M, N)
    csd = torch.from_numpy(cs.view(np.int16)).to(DEV)
    ad = to_dev(alpha)
    y = bsg.bs_gemv(bits, K, M, N, ad, x_dev(x, "f16"), colscale=csd)
    cols = [bsg.bs_gemv(bits, K, M, N, ad, x_dev(np.ascontiguousarray(x[:, b]), "f16"), colscale=csd)
            for b in range(B)]
    torch.cuda.synchronize()
    yt = torch.cat(cols, dim=1).cpu().numpy()
    np.testing.assert_allclose(y.cpu().numpy(), yt, rtol=1e-6, atol=1e-6)
