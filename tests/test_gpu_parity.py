"""GPU parity: every entry point of the C ABI (through the Python binding)
against the CPU oracle on the same seeded inputs.

Integer results (sign bits, layouts, int8 codes, int32 accumulators, row
indices, fp16/fp32 scales written by the packer) must match bit for bit;
floating-point outputs must lie within the per-output bound
2e-3 * (sum_k |alpha_k| sum_n |c_k x| + sum_j |alpha_r| sum_n |x| + |s| sum_n |q x|).
Sizes span several 64x4-word tiles and ragged row blocks / word groups.
"""
import numpy as np
import pytest

import oracle
from bit_gemv_packed_amd import synth
from gpu_util import DEV, check_close, f16_dev, say, to_dev, u16, u32, x_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import bit_gemv_packed_amd as bsg  # noqa: E402


def _layout(logical, K, M, N):
    return bsg.bsg_logical_to_layout(to_dev(logical.view(np.int32)), K, M, N)


# ------------------------------------------------------------------ layout
@pytest.mark.parametrize("K,M,N", [(1, 64, 128), (2, 70, 160), (3, 130, 32), (2, 200, 544), (2, 1, 32), (1, 4097, 4096)])
def test_layout_conversion_bit_exact(K, M, N):
    say("layout", K, M, N)
    L = synth.random_bits(K + M + N, K, M, N)
    phys = _layout(L, K, M, N)
    torch.cuda.synchronize()
    ref = oracle.to_layout(L, K, M, N)
    got = u32(phys)
    np.testing.assert_array_equal(got, ref)  # padding included: zero words on both sides
    back = bsg.bsg_layout_to_logical(phys, K, M, N)
    np.testing.assert_array_equal(u32(back).reshape(K, M, N // 32), L)


# ------------------------------------------------------------------ bs_gemv
GEMV_CASES = [
    # K, M, N, B, colscale, x dtype, x distribution
    (1, 256, 256, 1, False, "f32", "normal"),
    (2, 300, 544, 1, True, "bf16", "normal"),
    (3, 70, 96, 2, False, "f16", "normal"),
    (2, 1000, 4096, 1, True, "bf16", "normal"),
    (2, 129, 1056, 3, True, "bf16", "student_t3"),
    (1, 64, 32, 1, False, "f32", "normal"),
    (1, 1, 32, 1, True, "bf16", "normal"),
    (2, 4096, 4096, 4, False, "bf16", "normal"),
    (2, 333, 2080, 16, True, "bf16", "normal"),
    (1, 50, 128, 20, False, "f32", "normal"),
    (8, 65, 256, 1, True, "f32", "normal"),
    (4, 2000, 768, 8, False, "bf16", "normal"),
    (2, 5, 14336, 1, False, "bf16", "normal"),
    (3, 300, 544, 1, True, "bf16", "normal"),
    (4, 130, 1024, 2, True, "f32", "normal"),
    (5, 77, 320, 3, False, "bf16", "normal"),
    (2, 17000, 256, 1, True, "bf16", "normal"),
    (1, 9000, 96, 2, False, "f16", "normal"),
    (3, 257, 1056, 1, False, "bf16", "normal"),
    (4, 130, 2080, 1, False, "f16", "normal"),
    (4, 200, 544, 1, False, "f32", "student_t3"),
    (3, 17000, 256, 1, False, "bf16", "normal"),
    # more workgroups than compute units with more than half the LDS each: the
    # planner halves the wavefronts so that two workgroups share a unit
    (2, 6144, 4096, 1, True, "bf16", "normal"),
    (2, 14336, 4096, 1, True, "f16", "normal"),
    (3, 5000, 4096, 1, True, "bf16", "student_t3"),
    (2, 6144, 2048, 3, True, "bf16", "normal"),      # batch tile of 4 columns
]


def _gemv_inputs(case):
    K, M, N, B, cs, dt, dist = case
    seed = K * 7919 + M * 31 + N + B
    L = synth.random_bits(seed, K, M, N)
    alpha, csb = synth.random_scales(seed, K, M, N, cs)
    x = synth.random_x(seed, N, B, dt, dist)
    return L, alpha, csb, x


@pytest.mark.parametrize("case", GEMV_CASES, ids=lambda c: "K%d_M%d_N%d_B%d_cs%d_%s_%s" % c)
def test_bs_gemv_matches_oracle(case):
    K, M, N, B, cs, dt, dist = case
    say("bs_gemv", case)
    L, alpha, csb, x = _gemv_inputs(case)
    bits = _layout(L, K, M, N)
    ad = to_dev(alpha)
    cd = f16_dev(csb) if cs else None
    xd = x_dev(x, dt)
    y = bsg.bs_gemv(bits, K, M, N, ad, xd, colscale=cd)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, alpha, x, csb)
    tol = oracle.tolerance(x, alpha=alpha, colscale_f16=csb)
    check_close(y.cpu().numpy(), ref, tol, "bs_gemv %s" % (case,))
    # a second call gives the same bits (fixed-order reduction)
    y2 = bsg.bs_gemv(bits, K, M, N, ad, xd, colscale=cd)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)


# Every kernel instance and the multi-chunk loop, by forcing the lanes per
# row (Q) and the wavefronts per workgroup (fewer wavefronts -> more chunks).
FORCED = [(q, w) for q in (1, 2, 4) for w in (1, 3, 16)]
FORCED_SHAPES = [(1, 200, 1056, 1, False, "bf16", "normal"), (2, 130, 2080, 1, True, "bf16", "normal"),
                 (4, 70, 800, 1, True, "f32", "normal"), (3, 90, 544, 2, False, "bf16", "normal"),
                 (6, 65, 256, 4, False, "f16", "normal"), (2, 64, 4096, 3, True, "bf16", "student_t3")]


@pytest.mark.parametrize("qw", FORCED, ids=lambda c: "Q%d_W%d" % c)
def test_bs_gemv_every_instance(qw, monkeypatch):
    monkeypatch.setenv("BSG_Q", str(qw[0]))
    monkeypatch.setenv("BSG_WAVES", str(qw[1]))
    for case in FORCED_SHAPES:
        K, M, N, B, cs, dt, dist = case
        say("bs_gemv forced", qw, case)
        L, alpha, csb, x = _gemv_inputs(case)
        bits = _layout(L, K, M, N)
        y = bsg.bs_gemv(bits, K, M, N, to_dev(alpha), x_dev(x, dt), colscale=f16_dev(csb) if cs else None)
        torch.cuda.synchronize()
        ref = oracle.sign_gemv(L, K, M, N, alpha, x, csb)
        check_close(y.cpu().numpy(), ref, oracle.tolerance(x, alpha=alpha, colscale_f16=csb), "forced %s %s" % (qw, case))
        # int8 mode through the same decomposition
        xq, sx = oracle.quantize_i8(x)
        acc, _ = bsg.bs_gemv_i8(bits, K, M, N, to_dev(alpha), to_dev(xq), to_dev(sx), want_y=False)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), oracle.sign_gemv_i8(L, K, M, N, xq))


def test_bs_gemv_accumulate_and_negation():
    case = (2, 700, 2048, 2, True, "bf16", "normal")
    K, M, N, B, cs, dt, _ = case
    say("bs_gemv accumulate/negation", case)
    L, alpha, csb, x = _gemv_inputs(case)
    bits = _layout(L, K, M, N)
    nbits = _layout(~L, K, M, N)
    ad, cd, xd = to_dev(alpha), f16_dev(csb), x_dev(x, dt)
    y = bsg.bs_gemv(bits, K, M, N, ad, xd, colscale=cd)
    yn = bsg.bs_gemv(nbits, K, M, N, ad, xd, colscale=cd)
    y0 = torch.randn((M, B), dtype=torch.float32, device=DEV, generator=torch.Generator(DEV).manual_seed(3))
    ya = y0.clone()
    bsg.bs_gemv(bits, K, M, N, ad, xd, colscale=cd, y=ya, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(yn, -y), "negating every sign must negate y exactly"
    ref = oracle.sign_gemv(L, K, M, N, alpha, x, csb)
    tol = oracle.tolerance(x, alpha=alpha, colscale_f16=csb) + 1e-6 * np.abs(y0.cpu().numpy())
    check_close(ya.cpu().numpy(), y0.cpu().numpy().astype(np.float64) + ref, tol, "accumulate")


def test_bs_gemv_one_hot_reads_every_column():
    K, M, N = 1, 130, 256
    say("bs_gemv one-hot", K, M, N)
    L = synth.random_bits(77, K, M, N)
    alpha = np.ones((K, M), np.float32)
    bits = _layout(L, K, M, N)
    X = np.eye(N, dtype=np.float32)[:, :64]          # 64 one-hot columns as a batch
    y = bsg.bs_gemv(bits, K, M, N, to_dev(alpha), x_dev(X, "f32"))
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, alpha, X.astype(np.float64))
    np.testing.assert_array_equal(y.cpu().numpy().astype(np.float64), ref)


# ------------------------------------------------------------------ int8 mode
I8_CASES = [(1, 256, 256, 1), (2, 300, 544, 1), (3, 70, 96, 2), (2, 4096, 4096, 1), (2, 333, 2080, 16),
            (1, 5, 14336, 3), (2, 129, 1056, 20), (2, 14336, 4096, 1), (1, 20000, 512, 1)]


@pytest.mark.parametrize("case", I8_CASES, ids=lambda c: "K%d_M%d_N%d_B%d" % c)
def test_bs_gemv_i8_exact(case):
    K, M, N, B = case
    say("bs_gemv_i8", case)
    seed = 5000 + K * 101 + M + N + B
    L = synth.random_bits(seed, K, M, N)
    alpha, _ = synth.random_scales(seed, K, M, N, False)
    x = synth.random_x(seed, N, B, "bf16", "student_t3")
    xq, sx = oracle.quantize_i8(x)
    bits = _layout(L, K, M, N)
    acc, y = bsg.bs_gemv_i8(bits, K, M, N, to_dev(alpha), to_dev(xq), to_dev(sx))
    torch.cuda.synchronize()
    ref_acc = oracle.sign_gemv_i8(L, K, M, N, xq)
    np.testing.assert_array_equal(acc.cpu().numpy().astype(np.int64), ref_acc)
    xt = xq.astype(np.float64) * sx.astype(np.float64)[None, :]
    ref = oracle.sign_gemv(L, K, M, N, alpha, xt)
    check_close(y.cpu().numpy(), ref, oracle.tolerance(xt, alpha=alpha), "bs_gemv_i8 y")


def test_quantize_i8_bit_exact():
    # one 16-bit column with N % 8 == 0 takes the vector path (registers up to
    # N = 32768, then a second read of x); the others the generic one
    for (N, B, dt, dist) in [(4096, 1, "bf16", "normal"), (5120, 16, "bf16", "student_t3"), (96, 3, "f32", "normal"),
                             (256, 2, "f16", "normal"), (8, 1, "f16", "normal"), (1024, 1, "f16", "student_t3"),
                             (40000, 1, "bf16", "normal"), (4100, 1, "bf16", "normal"), (4096, 1, "f32", "normal")]:
        say("quantize", N, B, dt, dist)
        x = synth.random_x(N + B, N, B, dt, dist)
        xq, sx = bsg.bsq_quantize_i8(x_dev(x, dt))
        torch.cuda.synchronize()
        rq, rs = oracle.quantize_i8(x)
        np.testing.assert_array_equal(xq.cpu().numpy(), rq)
        np.testing.assert_array_equal(sx.cpu().numpy().view(np.uint32), rs.view(np.uint32))


# ------------------------------------------------------------------ low rank
LR_CASES = [(32, 256, 256, 1, "f32"), (512, 5120, 5120, 1, "bf16"), (64, 100, 96, 3, "f16"),
            (512, 1000, 2048, 16, "bf16"), (32, 1, 32, 1, "f32"),
            # B >= 4 columns of 16-bit x: the matrix cores (z in bf16 halves)
            (96, 300, 544, 4, "f16"), (512, 2000, 5120, 20, "bf16"), (32, 70, 96, 6, "bf16")]


@pytest.mark.parametrize("case", LR_CASES, ids=lambda c: "r%d_M%d_N%d_B%d_%s" % c)
def test_binlr_apply_matches_oracle(case):
    r, M, N, B, dt = case
    say("binlr", case)
    g = np.random.default_rng(r + M + N + B)
    u = np.where(g.integers(0, 2, (M, r)) == 1, 1.0, -1.0).astype(np.float32)
    v = np.where(g.integers(0, 2, (r, N)) == 1, 1.0, -1.0).astype(np.float32)
    ar = np.abs(g.normal(0, 0.005, r)).astype(np.float16).view(np.uint16)
    x = synth.random_x(r + N, N, B, dt)
    Ub, Vb = bsg.bsq_pack_signs(to_dev(u)), bsg.bsq_pack_signs(to_dev(v))
    y0 = torch.zeros((M, B), dtype=torch.float32, device=DEV) + 0.5
    bsg.binlr_apply(Ub, Vb, f16_dev(ar), r, M, N, x_dev(x, dt), y0)
    torch.cuda.synchronize()
    ub, vb = oracle.pack_signs(u), oracle.pack_signs(v)
    np.testing.assert_array_equal(u32(bsg.bsg_layout_to_logical(Ub, 1, M, r)).reshape(M, -1), ub)
    np.testing.assert_array_equal(u32(bsg.bsg_layout_to_logical(Vb, 1, r, N)).reshape(r, -1), vb)
    ref = 0.5 + oracle.binlr(ub, vb, ar, r, M, N, x)
    tol = oracle.tolerance(x, alpha_r_f16=ar, M=M) + 1e-6
    check_close(y0.cpu().numpy(), ref, tol, "binlr %s" % (case,))


# ------------------------------------------------------------------ protected rows
# More than 256 protected rows, B % 8 == 0, N % 8 == 0 and 16-bit x: 16 protected rows per workgroup
# on the matrix cores (ragged row tiles, half-empty and several batch tiles, partial and single
# 128-column runs); otherwise B % 4 == 0 with 16-bit x: four rows and four batch columns per
# workgroup (ragged row groups); otherwise one row per workgroup and one load per value
SAL_CASES = [(256, 256, 3, 1, "bf16"), (13824, 5120, 138, 1, "bf16"), (100, 100, 5, 2, "bf16"),
             (5120, 13824, 51, 16, "bf16"), (64, 32, 64, 1, "bf16"), (64, 48, 3, 1, "bf16"),
             (300, 100, 7, 1, "bf16"), (5120, 13824, 51, 1, "bf16"), (13824, 5120, 138, 16, "bf16"),
             (13824, 5120, 138, 16, "f16"), (300, 200, 20, 8, "bf16"), (64, 40, 17, 24, "f16"),
             (100, 100, 5, 16, "bf16"), (200, 256, 9, 12, "f16"),
             (28672, 8192, 287, 16, "bf16"), (2000, 520, 300, 16, "f16"), (1000, 4104, 270, 32, "bf16"),
             (600, 40, 260, 8, "bf16"), (700, 100, 280, 16, "bf16"), (300, 96, 11, 3, "bf16"),
             (2000, 1000, 30, 4, "f16"), (600, 200, 270, 12, "bf16"), (300, 98, 9, 8, "bf16"),
             (500, 98, 7, 4, "bf16")]


@pytest.mark.parametrize("case", SAL_CASES, ids=lambda c: "M%d_N%d_ns%d_B%d_%s" % c)
def test_salient_apply_matches_oracle(case):
    M, N, ns, B, dt = case
    say("salient_apply", case)
    g = np.random.default_rng(M + N + ns)
    rows = np.sort(g.choice(M, ns, replace=False)).astype(np.int32)
    q = g.integers(-127, 128, (ns, N)).astype(np.int8)
    s = g.uniform(1e-4, 1e-3, ns).astype(np.float16).view(np.uint16)
    x = synth.random_x(M + N, N, B, dt, "student_t3")
    y = torch.zeros((M, B), dtype=torch.float32, device=DEV)
    bsg.salient_int8_apply(to_dev(rows), to_dev(q), f16_dev(s), M, N, x_dev(x, dt), y)
    torch.cuda.synchronize()
    ref = oracle.salient(rows, q, s, M, N, x)
    tol = oracle.tolerance(x, rows=rows, q=q, s_f16=s, M=M)
    check_close(y.cpu().numpy(), ref, tol, "salient %s" % (case,))
    # rows that are not protected stay exactly zero
    other = np.setdiff1d(np.arange(M), rows)
    assert not y.cpu().numpy()[other].any()


# ------------------------------------------------------------------ fused layer
LINEAR_CASES = [
    # K, M, N, B, colscale, x dtype, rank r, protected rows ns
    (2, 300, 544, 1, True, "bf16", 64, 5),
    (3, 5120, 5120, 1, False, "bf16", 512, 51),
    (2, 1000, 1024, 4, False, "f32", 32, 10),
    (1, 64, 32, 1, False, "f16", 32, 64),
    (2, 200, 256, 16, True, "bf16", 96, 3),
    (2, 700, 4096, 2, False, "bf16", 0, 7),
    (2, 17000, 512, 1, False, "bf16", 128, 170),
    (2, 129, 1056, 3, True, "bf16", 32, 0),
    # B >= 4 columns of 16-bit x: bases, correction and protected rows as
    # separate matrix-core launches
    (2, 1000, 2048, 16, False, "bf16", 128, 10),
    (3, 300, 544, 8, True, "f16", 64, 3),         # fp16 column scales on the matrix cores
    (5, 130, 1024, 4, False, "f16", 32, 0),       # two launches of bases
    (2, 2000, 5120, 20, False, "bf16", 512, 20),  # two batch launches
]


def _linear_inputs(case):
    K, M, N, B, cs, dt, r, ns = case
    seed = 104729 + K * 7919 + M * 31 + N + B + r + ns
    L = synth.random_bits(seed, K, M, N)
    alpha, csb = synth.random_scales(seed, K, M, N, cs)
    x = synth.random_x(seed, N, B, dt, "student_t3")
    g = np.random.default_rng(seed)
    u = np.where(g.integers(0, 2, (M, r)) == 1, 1.0, -1.0).astype(np.float32)
    v = np.where(g.integers(0, 2, (r, N)) == 1, 1.0, -1.0).astype(np.float32)
    ar = np.abs(g.normal(0, 0.005, r)).astype(np.float16).view(np.uint16)
    rows = np.sort(g.choice(M, ns, replace=False)).astype(np.int32)
    q = g.integers(-127, 128, (ns, N)).astype(np.int8)
    sv = g.uniform(1e-4, 1e-3, ns).astype(np.float16).view(np.uint16)
    alpha[:, rows] = 0.0  # protected rows replace the binary part
    return L, alpha, csb, x, u, v, ar, rows, q, sv


def _run_linear(case, y0=None):
    K, M, N, B, cs, dt, r, ns = case
    L, alpha, csb, x, u, v, ar, rows, q, sv = _linear_inputs(case)
    bits = _layout(L, K, M, N)
    lowrank = None
    if r:
        lowrank = (bsg.bsq_pack_signs(to_dev(u)), bsg.bsq_pack_signs(to_dev(v)), f16_dev(ar), r)
    salient = (to_dev(rows), to_dev(q), f16_dev(sv)) if ns else None
    y = None if y0 is None else to_dev(y0)
    y = bsg.bsg_linear(bits, K, M, N, to_dev(alpha), x_dev(x, dt), colscale=f16_dev(csb) if cs else None,
                       lowrank=lowrank, salient=salient, y=y, accumulate=y0 is not None)
    torch.cuda.synchronize()
    ref = oracle.sign_gemv(L, K, M, N, alpha, x, csb)
    if r:
        ref = ref + oracle.binlr(oracle.pack_signs(u), oracle.pack_signs(v), ar, r, M, N, x)
    if ns:
        ref = ref + oracle.salient(rows, q, sv, M, N, x)
    if y0 is not None:
        ref = ref + y0
    tol = oracle.tolerance(x, alpha=alpha, colscale_f16=csb, alpha_r_f16=ar if r else None,
                           rows=rows if ns else None, q=q if ns else None, s_f16=sv if ns else None, M=M)
    return y, ref, tol


@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "K%d_M%d_N%d_B%d_cs%d_%s_r%d_ns%d" % c)
def test_bsg_linear_matches_oracle(case):
    say("bsg_linear", case)
    y, ref, tol = _run_linear(case)
    check_close(y.cpu().numpy(), ref, tol, "bsg_linear %s" % (case,))


def test_bsg_linear_accumulates_and_reduces_to_bs_gemv():
    case = (2, 300, 544, 2, True, "bf16", 64, 5)
    say("bsg_linear accumulate", case)
    y0 = np.linspace(-1, 1, 300 * 2, dtype=np.float32).reshape(300, 2)
    y, ref, tol = _run_linear(case, y0)
    check_close(y.cpu().numpy(), ref, tol + 1e-6, "bsg_linear accumulate")
    # without a correction or protected rows it is bs_gemv, bit for bit
    K, M, N, B, cs, dt = 2, 1000, 4096, 1, True, "bf16"
    L, alpha, csb, x = _gemv_inputs((K, M, N, B, cs, dt, "normal"))
    bits = _layout(L, K, M, N)
    args = (bits, K, M, N, to_dev(alpha), x_dev(x, dt))
    y1 = bsg.bs_gemv(*args, colscale=f16_dev(csb))
    y2 = bsg.bsg_linear(*args, colscale=f16_dev(csb))
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("qw", [(1, 1), (2, 3), (4, 16), (2, 8)], ids=lambda c: "Q%d_W%d" % c)
def test_bsg_linear_every_decomposition(qw, monkeypatch):
    # few wavefronts: several low-rank chunks and protected rows per wavefront
    monkeypatch.setenv("BSG_Q", str(qw[0]))
    monkeypatch.setenv("BSG_WAVES", str(qw[1]))
    for case in [(2, 300, 544, 1, True, "bf16", 256, 40), (3, 130, 1024, 3, False, "f32", 96, 9)]:
        say("bsg_linear forced", qw, case)
        y, ref, tol = _run_linear(case)
        check_close(y.cpu().numpy(), ref, tol, "bsg_linear forced %s %s" % (qw, case))


# ------------------------------------------------------------------ packing
PACK_CASES = [(256, 256, 1, False), (320, 544, 3, False), (130, 96, 2, True), (4096, 4096, 2, True),
              (1, 32, 2, True), (70, 4096, 4, True)]


@pytest.mark.parametrize("case", PACK_CASES, ids=lambda c: "M%d_N%d_K%d_cs%d" % c)
def test_pack_bit_exact(case):
    M, N, K, cs = case
    say("bsq_pack", case)
    W = synth.weights(M + N, K, M, N)
    bits, alpha, csd = bsg.bsq_pack(to_dev(W), K, colscale=cs)
    torch.cuda.synchronize()
    rb, ra, rc = oracle.pack(W, K, cs)
    np.testing.assert_array_equal(u32(bsg.bsg_layout_to_logical(bits, K, M, N)).reshape(K, M, -1), rb)
    np.testing.assert_array_equal(alpha.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    if cs:
        np.testing.assert_array_equal(u16(csd), rc)


def test_absmean_and_salient_select_bit_exact():
    for (M, N, ns, K) in [(256, 256, 3, 1), (13824, 5120, 138, 2), (1000, 96, 10, 2), (300, 64, 0, 1)]:
        say("bsq_salient", M, N, ns, K)
        w = synth.WORKLOADS[5]
        W = synth.weights(5, 9, M, N)
        W[7] = W[3]                    # tied scores
        X = synth.calibration(w, 9, N, 128)
        alpha = np.full((K, M), 0.5, np.float32)
        xbar = bsg.bsq_absmean(to_dev(X))
        ad = to_dev(alpha)
        rows, q, s = bsg.bsq_salient(to_dev(W), xbar, ns, ad)
        torch.cuda.synchronize()
        rx = oracle.absmean(X)
        np.testing.assert_array_equal(xbar.cpu().numpy().view(np.uint32), rx.view(np.uint32))
        rr, rq, rs, ra = oracle.salient_select(W, rx, ns, alpha)
        np.testing.assert_array_equal(rows.cpu().numpy(), rr)
        np.testing.assert_array_equal(q.cpu().numpy(), rq)
        np.testing.assert_array_equal(u16(s), rs)
        np.testing.assert_array_equal(ad.cpu().numpy(), ra)
