"""GPU parity of the offline binary low-rank fit (binlr_fit) against the CPU
oracle: the sign vectors bit for bit, the greedy and refitted coefficients
and the residual energies to fp64 rounding, the fp16 coefficients to one
unit in the last place, and the padding components (u = v = +1,
coefficient 0) that round the rank up to a multiple of 32.

Cases cover ragged M (a partial sign word of u), ranks below, at and above
32, one and several alternation rounds, a signed rank-one matrix (recovered
exactly), and the fitted correction applied through binlr_apply.
"""
import numpy as np
import pytest

import oracle
from bit_gemv_packed_amd import synth
from gpu_util import DEV, check_close, f16_dev, say, to_dev, u16, u32, x_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import bit_gemv_packed_amd as bsg  # noqa: E402

FIT_CASES = [
    # M, N, r, rounds
    (64, 64, 8, 5),
    (100, 96, 40, 5),
    (33, 32, 1, 1),
    (300, 512, 32, 5),
    (1000, 256, 70, 3),
]


def _fit_both(M, N, r, rounds, W):
    vinit = synth.random_bits(M * 7 + N + r, 1, r, N)[0]
    U, V, a16, rp, al, ag, sse, solved = bsg.binlr_fit(to_dev(W), r, to_dev(vinit.view(np.int32)), rounds=rounds)
    torch.cuda.synchronize()
    ref = oracle.binlr_fit(W, r, vinit, rounds=rounds)
    return (U, V, a16, rp, al, ag, sse, solved), ref


def _check_fit(M, N, r, got, ref, W):
    U, V, a16, rp, al, ag, sse, solved = got
    ub, vb, rag, ral, rsse, rsolved = ref
    assert rp == (r + 31) // 32 * 32
    # u_j is column j of U: compare the r fitted bits, padding bits are +1
    ul = u32(bsg.bsg_layout_to_logical(U, 1, M, rp)).reshape(M, rp // 32)
    for w in range(rp // 32):
        nfit = max(0, min(32, r - 32 * w))
        mask = np.uint32((1 << nfit) - 1) if nfit < 32 else np.uint32(0xFFFFFFFF)
        ref_w = ub[:, w] if w < ub.shape[1] else np.zeros(M, np.uint32)
        np.testing.assert_array_equal(ul[:, w] & mask, ref_w & mask)
        np.testing.assert_array_equal(ul[:, w] | mask, np.full(M, 0xFFFFFFFF, np.uint32))
    vl = u32(bsg.bsg_layout_to_logical(V, 1, rp, N)).reshape(rp, N // 32)
    np.testing.assert_array_equal(vl[:r], vb)
    assert (vl[r:] == 0xFFFFFFFF).all()
    assert solved == rsolved
    np.testing.assert_allclose(ag, rag, rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(al, ral, rtol=1e-8, atol=1e-14)
    w2 = float((W.astype(np.float64) ** 2).sum())
    assert abs(sse[0] - rsse[0]) <= 1e-9 * w2
    assert abs(sse[1] - rsse[1]) <= 1e-9 * w2
    # fp16 coefficients: fp16(fp32(alpha)) of the oracle's refit, within one
    # unit in the last place (the two fp64 values may straddle a tie)
    h = u16(a16)
    want = oracle.f32_to_f16(ral.astype(np.float32))
    assert (np.abs(h[:r].astype(np.int32) - want.astype(np.int32)) <= 1).all()
    assert (h[r:] == 0).all()


@pytest.mark.parametrize("case", FIT_CASES, ids=lambda c: "M%d_N%d_r%d_rounds%d" % c)
def test_binlr_fit_matches_oracle(case):
    M, N, r, rounds = case
    say("binlr_fit", case)
    W = np.random.default_rng([4242, M, N, r]).standard_normal((M, N)).astype(np.float32) * 0.02
    got, ref = _fit_both(M, N, r, rounds, W)
    _check_fit(M, N, r, got, ref, W)


def test_binlr_fit_recovers_a_signed_rank_one_matrix():
    M, N, a = 70, 128, 0.375
    say("binlr_fit rank one", M, N)
    rng = np.random.default_rng(99)
    u = np.where(rng.integers(0, 2, M) == 1, 1.0, -1.0)
    v = np.where(rng.integers(0, 2, N) == 1, 1.0, -1.0)
    W = (a * np.outer(u, v)).astype(np.float32)
    got, ref = _fit_both(M, N, 1, 5, W)
    _check_fit(M, N, 1, got, ref, W)
    assert abs(got[4][0] - a) < 1e-12 and got[6][0] < 1e-20


def test_binlr_fit_feeds_binlr_apply():
    """The fitted correction, applied with binlr_apply, matches the oracle's
    product of the oracle's factors (fp16 coefficients on both sides)."""
    M, N, r = 200, 256, 48
    say("binlr_fit -> binlr_apply", M, N, r)
    W = np.random.default_rng(7).standard_normal((M, N)).astype(np.float32) * 0.02
    got, ref = _fit_both(M, N, r, 5, W)
    U, V, a16, rp = got[:4]
    x = synth.random_x(17, N, 3, "bf16")
    y = torch.zeros((M, 3), dtype=torch.float32, device=DEV)
    bsg.binlr_apply(U, V, a16, rp, M, N, x_dev(x, "bf16"), y)
    torch.cuda.synchronize()
    ub, vb = ref[0], ref[1]
    # the oracle's factors padded to rp components the same way
    ubp = np.full((M, rp // 32), 0xFFFFFFFF, np.uint32)
    for w in range(rp // 32):
        nfit = max(0, min(32, r - 32 * w))
        if nfit:
            mask = np.uint32((1 << nfit) - 1) if nfit < 32 else np.uint32(0xFFFFFFFF)
            ubp[:, w] = (ub[:, w] & mask) | ~mask
    vbp = np.full((rp, N // 32), 0xFFFFFFFF, np.uint32)
    vbp[:r] = vb
    a16p = np.zeros(rp, np.uint16)
    a16p[:r] = u16(a16)[:r]
    yref = oracle.binlr(ubp, vbp, a16p, rp, M, N, x)
    check_close(y.cpu().numpy(), yref, oracle.tolerance(x, alpha_r_f16=a16p, M=M) + 1e-9, "fit -> apply")
