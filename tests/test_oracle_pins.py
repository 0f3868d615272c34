"""Pins for the CPU oracle: it is checked against what the pages and the
mathematics fix, never against itself or the HIP path.

Each test names the fact it checks.  A plausible mistake anywhere in the
oracle (a dropped term, a wrong sign or bit order, a transposed operand, a
missing residual update) fails at least one of them.
"""
import math
import os
import re
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_gemv_packed_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = [s.strip() for s in line.split("=", 1)]
        vals[k] = [float(t) for t in v.split()]
    return vals


def _signs_to_word(signs):
    w = 0
    for i, s in enumerate(signs):
        if s > 0:
            w |= 1 << i
    return w


def _dense_signs(bits, K, M, N):
    """+-1 matrices [K][M][N] from logical words, via numpy's little-endian unpackbits."""
    b = np.asarray(bits, np.uint32).reshape(K, M, -1)
    by = b.view(np.uint8).reshape(K, M, -1)
    unpacked = np.unpackbits(by, axis=-1, bitorder="little")[..., :N]
    return unpacked.astype(np.float64) * 2.0 - 1.0


# ----------------------------------------------------------- worked examples
def test_worked_example_signed_sum():
    g = _golden("biloco_worked_example.txt")
    v, x, expect = g["v"], g["x"], g["v.x"][0]
    word = _signs_to_word(v)
    assert word == 0b0101
    y = oracle.sign_gemv(np.array([[[word]]], np.uint32), 1, 1, 4, np.ones((1, 1), np.float32),
                         np.array(x, np.float64))
    assert abs(y[0, 0] - expect) <= 1e-12
    # Same with the input dimension padded to 32: extra columns carry x = 0.
    xp = np.zeros(32)
    xp[:4] = x
    rng = np.random.default_rng(1)
    wpad = word | (int(rng.integers(0, 2**28)) << 4)
    y = oracle.sign_gemv(np.array([[[wpad]]], np.uint32), 1, 1, 32, np.ones((1, 1), np.float32), xp)
    assert abs(y[0, 0] - expect) <= 1e-12


def test_worked_example_lowrank_expansion():
    """alpha * u * (v . x): with alpha = 1 each output is +-3.4 by the sign of u."""
    g = _golden("biloco_worked_example.txt")
    v, x, expect = g["v"], g["x"], g["v.x"][0]
    M, r, N = 37, 32, 4
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2, size=M) * 2 - 1
    ubits = np.zeros((M, 1), np.uint32)
    ubits[:, 0] = (u > 0).astype(np.uint32)          # rank component 0 only
    vbits = np.zeros((r, 1), np.uint32)
    vbits[0, 0] = _signs_to_word(v)
    alpha_r = np.zeros(r, np.float16)
    alpha_r[0] = 1.0
    y = oracle.binlr(ubits, vbits, alpha_r.view(np.uint16), r, M, N, np.array(x))
    np.testing.assert_allclose(y[:, 0], u * expect, rtol=0, atol=1e-12)


# ----------------------------------------------------------- dense equality
@pytest.mark.parametrize("K,M,N,B,cs", [(1, 5, 7, 1, False), (2, 33, 64, 3, True), (3, 64, 128, 4, True),
                                        (2, 17, 100, 2, False), (1, 1, 1, 1, True)])
def test_equals_dense_dequantised_matmul(K, M, N, B, cs):
    seed = K * 1000 + M * 10 + N
    bits = synth.random_bits(seed, K, M, N)
    alpha, csb = synth.random_scales(seed, K, M, N, cs)
    x = synth.random_x(seed, N, B, "f32")
    S = _dense_signs(bits, K, M, N)
    c = np.ones((K, N)) if csb is None else csb.view(np.float16).astype(np.float64)
    What = np.einsum("km,kmn,kn->mn", alpha.astype(np.float64), S, c)
    ref = What @ x.astype(np.float64)
    y = oracle.sign_gemv(bits, K, M, N, alpha, x, csb)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_one_hot_reads_every_bit():
    K, M, N = 1, 9, 70
    bits = synth.random_bits(5, K, M, N)
    alpha, cs = synth.random_scales(5, K, M, N, True)
    S = _dense_signs(bits, K, M, N)[0]
    c = cs.view(np.float16).astype(np.float64)[0]
    for n in range(N):
        x = np.zeros(N)
        x[n] = 1.0
        y = oracle.sign_gemv(bits, K, M, N, alpha, x, cs)[:, 0]
        np.testing.assert_array_equal(y, alpha[0].astype(np.float64) * c[n] * S[:, n])


def test_popcount_closed_form():
    """x = 1, c = 1, K = 1: y_m = alpha_m * (2 * popcount(row m) - N) exactly."""
    K, M, N = 1, 50, 96
    bits = synth.random_bits(6, K, M, N)
    alpha, _ = synth.random_scales(6, K, M, N, False)
    y = oracle.sign_gemv(bits, K, M, N, alpha, np.ones(N))[:, 0]
    for m in range(M):
        pc = sum(bin(int(w)).count("1") for w in bits[0, m])
        assert y[m] == float(alpha[0, m]) * (2 * pc - N)


def test_negating_all_signs_negates_y():
    K, M, N, B = 2, 40, 77, 2
    bits = synth.random_bits(7, K, M, N)
    alpha, cs = synth.random_scales(7, K, M, N, True)
    x = synth.random_x(7, N, B, "bf16")
    y = oracle.sign_gemv(bits, K, M, N, alpha, x, cs)
    yn = oracle.sign_gemv(~bits, K, M, N, alpha, x, cs)
    np.testing.assert_array_equal(yn, -y)


def test_linearity_small_integers():
    K, M, N = 2, 20, 64
    bits = synth.random_bits(8, K, M, N)
    alpha = np.array([[0.5] * M, [0.25] * M], np.float32)
    rng = np.random.default_rng(8)
    x1 = rng.integers(-5, 6, size=N).astype(np.float64)
    x2 = rng.integers(-5, 6, size=N).astype(np.float64)
    a = 3.0
    lhs = oracle.sign_gemv(bits, K, M, N, alpha, a * x1 + x2)
    rhs = a * oracle.sign_gemv(bits, K, M, N, alpha, x1) + oracle.sign_gemv(bits, K, M, N, alpha, x2)
    np.testing.assert_array_equal(lhs, rhs)


def test_column_permutation_invariance():
    K, M, N = 1, 12, 64
    bits = synth.random_bits(9, K, M, N)
    S = _dense_signs(bits, K, M, N)[0]
    rng = np.random.default_rng(9)
    perm = rng.permutation(N)
    x = rng.integers(-9, 10, size=N).astype(np.float64)
    pbits = oracle.pack_signs(S[:, perm].astype(np.float32))[None]
    alpha = np.ones((1, M), np.float32)
    np.testing.assert_array_equal(oracle.sign_gemv(bits, K, M, N, alpha, x),
                                  oracle.sign_gemv(pbits, K, M, N, alpha, x[perm]))


def test_brute_force_all_patterns_1x8():
    rng = np.random.default_rng(10)
    x = rng.standard_normal(8)
    for p in range(256):
        signs = [1.0 if (p >> i) & 1 else -1.0 for i in range(8)]
        expect = 0.0
        for s, xv in zip(signs, x):
            expect += s * xv
        y = oracle.sign_gemv(np.array([[[p]]], np.uint32), 1, 1, 8, np.ones((1, 1), np.float32), x)
        assert abs(y[0, 0] - expect) <= 1e-15 * max(1.0, abs(expect)) * 8


# ----------------------------------------------------------- int8 mode
def test_int8_exact_identity_and_brute_force():
    K, M, N, B = 2, 30, 96, 3
    bits = synth.random_bits(11, K, M, N)
    rng = np.random.default_rng(11)
    xq = rng.integers(-127, 128, size=(N, B)).astype(np.int8)
    acc = oracle.sign_gemv_i8(bits, K, M, N, xq)
    S = _dense_signs(bits, K, M, N)
    on = (S > 0).astype(np.int64)
    ident = 2 * np.einsum("kmn,nb->kmb", on, xq.astype(np.int64)) - xq.astype(np.int64).sum(0)[None, None, :]
    np.testing.assert_array_equal(acc, ident)
    for k in range(K):
        for m in (0, M - 1):
            for b in range(B):
                s = 0
                for n in range(N):
                    s += int(S[k, m, n]) * int(xq[n, b])
                assert acc[k, m, b] == s
    assert np.abs(acc).max() < 2**31


def test_quantize_i8_rules():
    x = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -127.0, 3.49], np.float32)
    xq, sx = oracle.quantize_i8(x)
    assert sx[0] == np.float32(1.0)
    np.testing.assert_array_equal(xq[:, 0], [127, 0, 2, 2, 0, -2, -127, 3])   # ties to even
    xq, sx = oracle.quantize_i8(np.zeros(5, np.float32))
    assert sx[0] == 0 and not xq.any()
    rng = np.random.default_rng(12)
    xs = synth.random_x(12, 500, 4, "bf16", "student_t3")
    xq, sx = oracle.quantize_i8(xs)
    assert np.abs(xq.astype(int)).max() <= 127
    for b in range(4):
        col = xs[:, b]
        assert abs(int(xq[np.argmax(np.abs(col)), b])) == 127
        err = np.abs(col.astype(np.float64) - sx[b] * xq[:, b].astype(np.float64))
        assert err.max() <= 0.5 * sx[b] * (1 + 1e-6)
        assert np.all((np.sign(xq[:, b]) == np.sign(col)) | (xq[:, b] == 0))


# ----------------------------------------------------------- protected rows
def test_salient_rows_textbook():
    M, N, ns, B = 40, 64, 5, 2
    rng = np.random.default_rng(13)
    rows = np.sort(rng.choice(M, ns, replace=False)).astype(np.int32)
    q = rng.integers(-127, 128, size=(ns, N)).astype(np.int8)
    s = rng.uniform(1e-4, 1e-3, size=ns).astype(np.float16)
    x = synth.random_x(13, N, B, "bf16")
    y = oracle.salient(rows, q, s.view(np.uint16), M, N, x)
    ref = np.zeros((M, B))
    ref[rows] = s.astype(np.float64)[:, None] * (q.astype(np.float64) @ x.astype(np.float64))
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=0)


# ----------------------------------------------------------- fp16 conversion
def test_f16_decode_all_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_f16_encode_matches_ieee_rne():
    rng = np.random.default_rng(14)
    vals = [rng.standard_normal(20000).astype(np.float32) * np.float32(s) for s in (1e-8, 1e-6, 1e-4, 1, 100, 6e4)]
    grid = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    grid = grid[np.isfinite(grid)]
    g64 = np.sort(np.unique(grid.astype(np.float64)))
    mids = ((g64[1:] + g64[:-1]) / 2).astype(np.float32)      # exact ties (representable in fp32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.99, 65520, 1e-9, 2.0**-25, 2.0**-24,
                        3 * 2.0**-26, 2.0**-14, 2.0**-14 * (1 - 2.0**-12)], np.float32)
    allv = np.concatenate(vals + [grid, mids, special])
    ours = oracle.f32_to_f16(allv)
    ref = allv.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert np.isnan(oracle.f32_to_f16(np.array([np.nan], np.float32)).view(np.float16)[0])


# ----------------------------------------------------------- packing
def _residuals_from_outputs(W, bits, alpha, cs, K):
    """R_k = W - sum_{j<=k} alpha_j c_j s_j, reconstructed in float64 from the outputs."""
    M, N = W.shape
    S = _dense_signs(bits, K, M, N)
    c = np.ones((K, N)) if cs is None else cs.view(np.float16).astype(np.float64)
    Rs = [W.astype(np.float64)]
    for k in range(K):
        Rs.append(Rs[-1] - alpha[k].astype(np.float64)[:, None] * c[k][None, :] * S[k])
    return Rs, S


@pytest.mark.parametrize("K,cs", [(1, False), (2, False), (3, False), (2, True)])
def test_pack_signs_follow_residual_and_energy_drops(K, cs):
    M, N = 48, 160
    W = synth.weights(99, K, M, N)
    bits, alpha, csb = oracle.pack(W, K, cs)
    Rs, S = _residuals_from_outputs(W, bits, alpha, csb, K)
    for k in range(K):
        # B_k = sign(R_{k-1}), sign(0) = +1
        np.testing.assert_array_equal(S[k] > 0, Rs[k] >= 0)
        # alpha_k = mean |R_{k-1}| rounded to fp32
        np.testing.assert_array_equal(alpha[k], (np.abs(Rs[k]).sum(1) / N).astype(np.float32))
        e0 = (Rs[k] ** 2).sum(1)
        e1 = (Rs[k + 1] ** 2).sum(1)
        assert np.all(e1 < e0)
        if not cs:
            # ||R - alpha S||^2 = ||R||^2 - N alpha^2 at alpha = mean|R| (fp32 rounding aside)
            np.testing.assert_allclose(e1, e0 - N * alpha[k].astype(np.float64) ** 2, rtol=1e-6)


def test_pack_alpha_is_fp32_argmin_exact():
    """Moving alpha by one fp32 ulp either way never lowers the row error (exact rationals)."""
    M, N = 6, 24
    W = synth.weights(98, 0, M, N)
    bits, alpha, _ = oracle.pack(W, 1, False)
    S = _dense_signs(bits, 1, M, N)[0]
    for m in range(M):
        R = [Fraction(float(v)) for v in W[m]]
        s = [int(v) for v in S[m]]

        def sse(a):
            a = Fraction(float(a))
            return sum((r - a * si) ** 2 for r, si in zip(R, s))

        a0 = alpha[0, m]
        base = sse(a0)
        for d in (np.inf, -np.inf):
            assert sse(np.nextafter(a0, np.float32(d))) >= base


def test_pack_colscale_is_fp16_argmin_exact():
    """Parity unpinned by page values; pinned by least-squares optimality:
    each column scale is the fp16 value minimising the column error given alpha and B."""
    M, N = 10, 40
    W = synth.weights(97, 0, M, N)
    bits, alpha, cs = oracle.pack(W, 1, True)
    S = _dense_signs(bits, 1, M, N)[0]
    c16 = cs[0].view(np.float16)
    for n in range(N):
        R = [Fraction(float(W[m, n])) for m in range(M)]
        a = [Fraction(float(alpha[0, m])) for m in range(M)]

        def sse(c):
            c = Fraction(float(c))
            return sum((R[m] - a[m] * c * int(S[m, n])) ** 2 for m in range(M))

        base = sse(c16[n])
        for d in (np.inf, -np.inf):
            assert sse(np.nextafter(c16[n], np.float16(d))) >= base


def test_pack_zero_maps_to_plus_one():
    W = np.array([[0.0, -0.0, -1.0, 2.0]], np.float32)
    bits, alpha, _ = oracle.pack(W, 1, False)
    assert int(bits[0, 0, 0]) == 0b1011
    assert alpha[0, 0] == np.float32(0.75)


def test_pack_signs_helper():
    S = np.array([[1, -1, 0, -0.0, -3]], np.float32)
    assert int(oracle.pack_signs(S)[0, 0]) == 0b01101


# ----------------------------------------------------------- protected-row selection
def test_salient_select_rules():
    """Parity unpinned by page values; pinned by the selection definition:
    top-ns rows by sum_n |W| xbar, ties to the smaller row, symmetric int8."""
    M, N, ns, K = 60, 48, 7, 2
    W = synth.weights(96, 0, M, N)
    W[10] = W[3]        # a tie: rows 3 and 10 have identical scores
    W[3] *= 4
    W[10] *= 4
    xbar = np.abs(synth.random_x(96, N, 1, "f32"))[:, 0].astype(np.float32)
    alpha = np.ones((K, M), np.float32)
    rows, q, s, a = oracle.salient_select(W, xbar, ns, alpha)
    score = np.abs(W.astype(np.float64)) @ xbar.astype(np.float64)
    order = sorted(range(M), key=lambda m: (-score[m], m))
    assert list(rows) == sorted(order[:ns])
    assert 3 in rows and 10 in rows
    sd = s.view(np.float16).astype(np.float64)
    for i, m in enumerate(rows):
        mx = np.abs(W[m]).max()
        assert s[i] == np.float32(np.float64(mx) / 127).astype(np.float16).view(np.uint16)
        assert np.abs(q[i].astype(int)).max() <= 127
        err = np.abs(W[m].astype(np.float64) - sd[i] * q[i])
        clip = np.abs(W[m].astype(np.float64) / sd[i]) > 127
        assert np.all(err[~clip] <= 0.5 * sd[i] * (1 + 1e-12))
    kept = np.zeros(M, bool)
    kept[rows] = True
    assert np.all(a[:, kept] == 0) and np.all(a[:, ~kept] == 1)
    # the smaller index wins a tie at the cut
    W2 = np.zeros((4, 8), np.float32)
    W2[:] = 1.0
    rows2, _, _, _ = oracle.salient_select(W2, np.ones(8, np.float32), 2)
    assert list(rows2) == [0, 1]


def test_absmean():
    X = synth.calibration(synth.WORKLOADS[5], 0, 300, 128)
    ours = oracle.absmean(X)
    ref = np.abs(X.astype(np.float64)).mean(0).astype(np.float32)
    np.testing.assert_allclose(ours, ref, rtol=2e-7, atol=0)


# ----------------------------------------------------------- layout
@pytest.mark.parametrize("K,M,N", [(1, 64, 128), (2, 70, 160), (3, 130, 32), (1, 1, 96), (2, 200, 544)])
def test_layout_is_a_bijection_of_padded_tiles(K, M, N):
    nd = oracle.words(N)
    mp, ndp = -(-M // 64) * 64, -(-nd // 4) * 4
    total = oracle.layout_words(K, M, N)
    plane = total // K
    assert plane == mp * ndp and total == K * plane
    seen = set()
    for k in range(K):
        for m in range(M):
            for w in range(nd):
                o = oracle.layout_offset(K, M, N, k, m, w)
                assert k * plane <= o < (k + 1) * plane
                seen.add(o)
    assert len(seen) == K * M * nd
    # every tile (64 rows x 4 words) is one contiguous row-major block of 256 words
    for k in range(K):
        for rb in range(mp // 64):
            for g in range(ndp // 4):
                m0, w0 = rb * 64, g * 4
                if m0 < M and w0 < nd:
                    base = oracle.layout_offset(K, M, N, k, m0, w0)
                    assert base % 256 == 0
                    for m in range(m0, min(M, m0 + 64)):
                        for w in range(w0, min(nd, w0 + 4)):
                            assert oracle.layout_offset(K, M, N, k, m, w) == base + (m - m0) * 4 + (w - w0)
    L = synth.random_bits(K * M + N, K, M, N)
    phys = oracle.to_layout(L, K, M, N)
    assert phys.size == total
    pad = np.ones(total, bool)
    pad[sorted(seen)] = False
    assert not phys[pad].any()  # padding rows and words are zero words
    np.testing.assert_array_equal(oracle.from_layout(phys, K, M, N), L)


# ----------------------------------------------------------- storage arithmetic
def test_storage_arithmetic_5120_rank512():
    g = _golden("biloco_storage.txt")
    M, N = [int(v) for v in g["matrix"]]
    r_bin, r_bf16 = int(g["binary_rank"][0]), int(g["bf16_rank"][0])
    u = np.ones((M, r_bin), np.float32)
    v = np.ones((r_bin, N), np.float32)
    bits = oracle.pack_signs(u).nbytes * 8 + oracle.pack_signs(v).nbytes * 8
    assert bits == 2 * 5120 * 512 == 5_242_880
    assert bits == 2 * M * r_bf16 * 16                         # same storage as BF16 rank 32
    assert abs(bits / 1e6 - g["both_corrections_mbit_approx"][0]) < 0.05
    assert r_bin // r_bf16 == g["rank_ratio_same_storage"][0]
    fp4_bits = M * N * 4.5                                   # 4 bits + one FP8 scale per 16 values
    assert abs(fp4_bits / 1e6 - g["fp4_weight_mbit_approx"][0]) / g["fp4_weight_mbit_approx"][0] < 0.03
    assert round(100 * bits / fp4_bits) == g["overhead_percent_approx"][0]
    r128 = oracle.pack_signs(np.ones((M, 128), np.float32)).nbytes + oracle.pack_signs(np.ones((128, N), np.float32)).nbytes
    assert r128 == 163_840
    assert abs(r128 / 2**20 - g["rank128_sign_bits_mib_approx"][0]) < 0.005
    fp4_bytes = M * N * 4 // 8
    assert fp4_bytes / 2**20 == g["fp4_weights_mib_approx"][0]
    assert round(fp4_bytes / r128) == g["read_ratio_approx"][0]


def test_tolerance_reduces_to_row_bound():
    K, M, N = 2, 8, 64
    alpha, _ = synth.random_scales(3, K, M, N, False)
    x = synth.random_x(3, N, 1, "bf16")
    t = oracle.tolerance(x, alpha=alpha)
    ref = 2e-3 * np.abs(alpha.astype(np.float64)).sum(0) * np.abs(x).sum()
    np.testing.assert_allclose(t[:, 0], ref, rtol=1e-12)


# ----------------------------------------------------------- low-rank fit (offline)
def _signs_of_bits(words, n):
    w = np.asarray(words, np.uint32).reshape(-1)
    return np.array([1.0 if (w[i >> 5] >> (i & 31)) & 1 else -1.0 for i in range(n)])


def _fit_factors(ub, vb, M, N, r):
    U = np.stack([_signs_of_bits(ub[m], r) for m in range(M)])          # [M][r]
    V = np.stack([_signs_of_bits(vb[j], N) for j in range(r)])          # [r][N]
    return U, V


def test_lr_fit_toy_example():
    """Every value the page prints for its 3 x 2 example."""
    g = _golden("biloco_toy_fit.txt")
    W = np.array(g["W_rows"], np.float32).reshape(3, 2)
    vinit = np.array([[_signs_to_word(g["v_start"])]] * 2, np.uint32)
    ub, vb, ag, al, (sse_g, sse_r), solved = oracle.binlr_fit(W, 2, vinit)
    U, V = _fit_factors(ub, vb, 3, 2, 2)
    num, den = g["component1_alpha_num_den"]
    np.testing.assert_array_equal(U[:, 0], g["component1_u"])
    np.testing.assert_array_equal(W.astype(np.float64) @ np.array(g["v_start"]), g["component1_Rv"])
    np.testing.assert_array_equal(W.astype(np.float64).T @ U[:, 0], g["component1_RTu"])
    assert ag[0] == num / den == 2.0
    R1 = W.astype(np.float64) - ag[0] * np.outer(U[:, 0], V[0])
    np.testing.assert_array_equal(R1.ravel(), g["residual_rows"])
    np.testing.assert_array_equal(U[:, 1], g["component2_u"])
    np.testing.assert_array_equal(V[1], g["component2_v"])
    num, den = g["component2_alpha_num_den"]
    assert abs(ag[1] - num / den) < 1e-15
    assert round(ag[1], 2) == g["component2_alpha_approx"][0]
    assert abs(sse_g - 4.0 / 3.0) < 1e-12 and round(sse_g, 2) == g["greedy_sse_approx"][0]
    assert solved
    np.testing.assert_allclose(al, g["refit_alpha"], rtol=0, atol=1e-12)
    assert abs(sse_r - g["refit_sse"][0]) < 1e-20


def test_lr_fit_recovers_a_signed_rank_one_matrix():
    """W = a u v^T with sign vectors: one component recovers it exactly (up
    to flipping both signs), alpha = a, no error left."""
    rng = np.random.default_rng(11)
    M, N, a = 40, 64, 0.75
    u = np.where(rng.integers(0, 2, M) == 1, 1.0, -1.0)
    v = np.where(rng.integers(0, 2, N) == 1, 1.0, -1.0)
    W = (a * np.outer(u, v)).astype(np.float32)
    vinit = synth.random_bits(5, 1, 1, N)[0]
    ub, vb, ag, al, (sse_g, sse_r), solved = oracle.binlr_fit(W, 1, vinit)
    U, V = _fit_factors(ub, vb, M, N, 1)
    s = U[0, 0] * u[0]
    np.testing.assert_array_equal(U[:, 0], s * u)
    np.testing.assert_array_equal(V[0], s * v)
    assert abs(ag[0] - a) < 1e-12 and abs(al[0] - a) < 1e-12
    assert sse_g < 1e-20 and sse_r < 1e-20


def test_lr_fit_one_round_is_the_alternation_rule():
    """With one round: u = sign(W v_start), v = sign(W^T u), sign(0) = +1
    (a zero row of W gives a zero sum), alpha = u^T W v / (M N)."""
    rng = np.random.default_rng(12)
    M, N = 24, 40
    W = rng.standard_normal((M, N)).astype(np.float32)
    W[5] = 0.0
    vinit = synth.random_bits(6, 1, 1, N)[0]
    ub, vb, ag, al, _, _ = oracle.binlr_fit(W, 1, vinit, rounds=1)
    U, V = _fit_factors(ub, vb, M, N, 1)
    v0 = _signs_of_bits(vinit, N)
    Wd = W.astype(np.float64)
    u = np.where(Wd @ v0 >= 0, 1.0, -1.0)
    assert u[5] == 1.0
    v = np.where(Wd.T @ u >= 0, 1.0, -1.0)
    np.testing.assert_array_equal(U[:, 0], u)
    np.testing.assert_array_equal(V[0], v)
    assert abs(ag[0] - u @ Wd @ v / (M * N)) < 1e-12 * abs(ag[0])
    assert ag[0] == al[0] or abs(ag[0] - al[0]) < 1e-12 * abs(ag[0])  # one component: refit = greedy


def test_lr_fit_greedy_coefficients_are_least_squares_and_sse_falls():
    """Each greedy alpha_j minimises ||R_j - alpha u_j v_j^T|| over alpha, so
    the residual energy falls by (u^T R_j v)^2 / (M N) per component."""
    rng = np.random.default_rng(13)
    M, N, r = 30, 48, 5
    W = rng.standard_normal((M, N)).astype(np.float32)
    vinit = synth.random_bits(7, 1, r, N)[0]
    ub, vb, ag, al, (sse_g, _), _ = oracle.binlr_fit(W, r, vinit)
    U, V = _fit_factors(ub, vb, M, N, r)
    R = W.astype(np.float64)
    energy = [float((R ** 2).sum())]
    for j in range(r):
        A = np.outer(U[:, j], V[j])
        best = (A * R).sum() / (A * A).sum()            # least squares over alpha, written out
        assert abs(ag[j] - best) < 1e-12 * max(1.0, abs(best))
        R = R - ag[j] * A
        energy.append(float((R ** 2).sum()))
    assert all(energy[i + 1] <= energy[i] + 1e-9 for i in range(r))
    assert abs(sse_g - energy[-1]) < 1e-9 * energy[0]


def test_lr_fit_refit_is_the_least_squares_solution():
    """The refitted coefficients solve min ||W - sum alpha_j u_j v_j^T||_F,
    checked against a generic least-squares solve over the vectorised rank-one
    terms; the refit never does worse than the greedy coefficients."""
    rng = np.random.default_rng(14)
    M, N, r = 20, 32, 6
    W = rng.standard_normal((M, N)).astype(np.float32)
    vinit = synth.random_bits(8, 1, r, N)[0]
    ub, vb, ag, al, (sse_g, sse_r), solved = oracle.binlr_fit(W, r, vinit)
    assert solved
    U, V = _fit_factors(ub, vb, M, N, r)
    A = np.stack([np.outer(U[:, j], V[j]).ravel() for j in range(r)], 1)
    ls, res, _, _ = np.linalg.lstsq(A, W.astype(np.float64).ravel(), rcond=None)
    np.testing.assert_allclose(al, ls, rtol=1e-9, atol=1e-12)
    assert abs(sse_r - float(res[0])) < 1e-9 * float(res[0])
    assert sse_r <= sse_g + 1e-12


def test_lr_fit_singular_refit_keeps_the_greedy_coefficients():
    """A constant matrix: the first component takes all of it, the second
    sees a zero residual (sign(0) = +1 gives the same all-plus vectors), so the
    normal equations are singular and the greedy coefficients stay."""
    M, N = 8, 32
    W = np.full((M, N), 0.5, np.float32)
    vinit = np.full((2, 1), 0xFFFFFFFF, np.uint32)
    ub, vb, ag, al, (sse_g, sse_r), solved = oracle.binlr_fit(W, 2, vinit)
    assert not solved
    np.testing.assert_array_equal(ag, [0.5, 0.0])
    np.testing.assert_array_equal(al, ag)
    assert sse_g == 0.0 and sse_r == 0.0


# ----------------------------------------------------------- group-wise row scales
def test_grouped_pack_with_one_group_is_the_row_scale_pack():
    """g = N: one group per row.  The first base is or_pack's (the same signs;
    the scale is or_pack's fp32 mean rounded to fp16), and the product with
    those scales is or_sign_gemv's with the same values."""
    M, N = 12, 96
    W = synth.weights(61, 0, M, N)
    b1, a1, _ = oracle.pack(W, 1, False)
    b2, a2, _ = oracle.pack_grouped(W, 1, N, False)
    np.testing.assert_array_equal(b1, b2)
    np.testing.assert_array_equal(a2[:, :, 0], oracle.f32_to_f16(a1))
    x = synth.random_x(61, N, 2, "f32")
    a16 = oracle.f16_to_f64(a2[:, :, 0]).astype(np.float32)
    np.testing.assert_array_equal(oracle.sign_gemv(b1, 1, M, N, a16, x),
                                  oracle.sign_gemv_grouped(b2, 1, M, N, N, a2, x))


@pytest.mark.parametrize("cs", [False, True])
def test_grouped_product_equals_the_dense_dequantised_matmul(cs):
    M, N, K, g = 9, 256, 2, 64
    W = synth.weights(62, 0, M, N)
    bits, alpha, csb = oracle.pack_grouped(W, K, g, cs)
    S = _dense_signs(bits, K, M, N)
    c = oracle.f16_to_f64(csb).reshape(K, N) if cs else np.ones((K, N))
    a = np.repeat(oracle.f16_to_f64(alpha), g, axis=2)          # [K][M][N]: the scale of each entry's group
    What = (a * c[:, None, :] * S).sum(0)
    x = synth.random_x(62, N, 3, "f32").astype(np.float64)
    np.testing.assert_allclose(oracle.sign_gemv_grouped(bits, K, M, N, g, alpha, x, csb), What @ x,
                               rtol=1e-12, atol=1e-15)


def test_grouped_alpha_is_the_fp16_argmin_per_group():
    """Moving a group scale by one fp16 step either way never lowers that
    group's error (exact rationals): the stored fp16 scale is the best fp16
    value for its group."""
    M, N, g = 4, 96, 32
    W = synth.weights(63, 0, M, N)
    bits, alpha, _ = oracle.pack_grouped(W, 1, g, False)
    S = _dense_signs(bits, 1, M, N)[0]
    a16 = alpha.view(np.float16)
    for m in range(M):
        for j in range(N // g):
            R = [Fraction(float(v)) for v in W[m, j * g:(j + 1) * g]]
            sg = [int(v) for v in S[m, j * g:(j + 1) * g]]

            def sse(a):
                a = Fraction(float(a))
                return sum((r - a * si) ** 2 for r, si in zip(R, sg))

            a0 = a16[0, m, j]
            base = sse(a0)
            for d in (np.inf, -np.inf):
                assert sse(np.nextafter(a0, np.float16(d))) >= base


def test_grouped_colscale_is_the_least_squares_value_per_group():
    """c[n] = fp16(fp32(sum_m a[m][j] |R| / sum_m a[m][j]^2)) with the stored
    fp16 scales a of the group j of column n, in exact rationals (first base)."""
    M, N, g = 5, 64, 32
    W = synth.weights(64, 0, M, N)
    bits, alpha, cs = oracle.pack_grouped(W, 1, g, True)
    a = oracle.f16_to_f64(alpha)
    for n in range(N):
        j = n // g
        num = sum(Fraction(float(a[0, m, j])) * abs(Fraction(float(W[m, n]))) for m in range(M))
        den = sum(Fraction(float(a[0, m, j])) ** 2 for m in range(M))
        want = oracle.f32_to_f16(np.array([np.float32(float(num / den))], np.float32))[0]
        assert cs[0, n] == want


def test_grouped_scales_never_fit_worse_than_row_scales():
    """Same signs, scales fitted per group instead of per row: the error of
    the first base does not grow (each group scale is optimal on its group;
    fp16 storage costs far less than the grouping gains here)."""
    M, N = 16, 512
    W = synth.weights(65, 0, M, N)
    Wd = W.astype(np.float64)
    b1, a1, _ = oracle.pack(W, 1, False)
    b2, a2, _ = oracle.pack_grouped(W, 1, 128, False)
    np.testing.assert_array_equal(b1, b2)
    S = _dense_signs(b1, 1, M, N)[0]
    e_row = ((Wd - a1[0].astype(np.float64)[:, None] * S) ** 2).sum()
    e_grp = ((Wd - np.repeat(oracle.f16_to_f64(a2[0]), 128, axis=1) * S) ** 2).sum()
    assert e_grp <= e_row


# ----------------------------------------------------------- salient columns (VCM)
def _group_idx(seed, N, g, s):
    """s distinct ascending columns of every group of g (seeded)."""
    r = np.random.default_rng(seed)
    return np.concatenate([np.sort(r.choice(g, s, replace=False)) + j * g for j in range(N // g)]).astype(np.int32)


@pytest.mark.parametrize("cs", [False, True])
def test_hybrid_with_every_column_salient_continues_the_greedy_bases(cs):
    """s = g and idx = 0..N-1: the salient branch sees the global residual in
    place, so its K bases are bases K..2K-1 of the 2K-base grouped pack, bit
    for bit (signs, fp16 group scales, column scales)."""
    M, N, K, g = 10, 256, 2, 64
    W = synth.weights(66, 0, M, N)
    b, a, c, sb, sa, sc = oracle.pack_hybrid(W, K, g, g, np.arange(N, dtype=np.int32), cs)
    b2, a2, c2 = oracle.pack_grouped(W, 2 * K, g, cs)
    np.testing.assert_array_equal(b, b2[:K])
    np.testing.assert_array_equal(a, a2[:K])
    np.testing.assert_array_equal(sb, b2[K:])
    np.testing.assert_array_equal(sa, a2[K:])
    if cs:
        np.testing.assert_array_equal(c, c2[:K])
        np.testing.assert_array_equal(sc, c2[K:])


@pytest.mark.parametrize("cs", [False, True])
def test_hybrid_product_equals_the_dense_dequantised_matmul(cs):
    """The salient bases scattered back to their logical columns (VCM undone)
    and added to the global reconstruction give the dense matrix whose
    product the hybrid product is."""
    M, N, K, g, s = 7, 256, 2, 64, 8
    W = synth.weights(67, 0, M, N)
    idx = _group_idx(67, N, g, s)
    S = s * (N // g)
    b, a, c, sb, sa, sc = oracle.pack_hybrid(W, K, g, s, idx, cs)
    Sg = _dense_signs(b, K, M, N)
    cg = oracle.f16_to_f64(c) if cs else np.ones((K, N))
    What = (np.repeat(oracle.f16_to_f64(a), g, axis=2) * cg[:, None, :] * Sg).sum(0)
    Ss = _dense_signs(sb, K, M, S)
    csal = oracle.f16_to_f64(sc) if cs else np.ones((K, S))
    phys = (np.repeat(oracle.f16_to_f64(sa), s, axis=2) * csal[:, None, :] * Ss).sum(0)   # [M][S]
    for p in range(S):
        What[:, idx[p]] += phys[:, p]
    x = synth.random_x(67, N, 2, "f32").astype(np.float64)
    y = oracle.sign_gemv_hybrid(b, K, M, N, g, a, c, sb, s, idx, sa, sc, x)
    np.testing.assert_allclose(y, What @ x, rtol=1e-12, atol=1e-14)


def test_hybrid_refinement_lowers_the_error_on_the_salient_columns():
    M, N, K, g, s = 32, 512, 2, 128, 16
    W = synth.weights(68, 0, M, N)
    idx = _group_idx(68, N, g, s)
    b, a, c, sb, sa, sc = oracle.pack_hybrid(W, K, g, s, idx, True)
    eye = np.eye(N)
    Wg = oracle.sign_gemv_grouped(b, K, M, N, g, a, eye, c)
    Wh = oracle.sign_gemv_hybrid(b, K, M, N, g, a, c, sb, s, idx, sa, sc, eye)
    e_g = ((W[:, idx] - Wg[:, idx]) ** 2).sum()
    e_h = ((W[:, idx] - Wh[:, idx]) ** 2).sum()
    assert e_h < 0.5 * e_g
    rest = np.setdiff1d(np.arange(N), idx)
    np.testing.assert_array_equal(Wg[:, rest], Wh[:, rest])


def test_hybrid_rejects_an_index_outside_the_matrix():
    W = synth.weights(69, 0, 4, 128)
    idx = _group_idx(69, 128, 64, 8)
    idx[3] = 128
    with pytest.raises(ValueError):
        oracle.pack_hybrid(W, 1, 64, 8, idx)


def test_average_bits_of_the_hybrid_format():
    """FluxBin App. C.2: with K = 2 global and 2 salient bases, g = 128 and
    16-bit scales and indices, s = 8 salient columns per group settle at about
    2.63 bits per weight and s = 16 at about 2.75; without salient columns the
    two bases and their group scales take 2 + 2*16/128 = 2.25."""
    assert abs(oracle.average_bits(2, 4096, 4096, 128, 8) - 2.63) < 0.01
    assert abs(oracle.average_bits(2, 4096, 4096, 128, 16) - 2.75) < 0.015
    # the per-weight terms alone: K + 16K/g + K s/g + 16K/g
    big = 1 << 24
    assert abs(oracle.average_bits(2, big, 4096, 128, 8, colscale=False) - 2.625) < 1e-4
    assert abs(oracle.average_bits(2, big, 4096, 128, 16, colscale=False) - 2.75) < 1e-4
    assert abs(oracle.average_bits(2, big, 4096, 128, 0, colscale=False) - 2.25) < 1e-9
