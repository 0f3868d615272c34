"""GPU parity of the fused multi-projection launch (bs_gemv_multi): every
projection's y against the CPU oracle, within the bs_gemv bound.

Cases cover projections of different heights sharing x (query/key/value and
gated-MLP shapes, scaled down), ragged heights, an empty projection between
others, eight projections, column scales on every projection, K = 1..6,
batch width 1 (one fused launch), 2 and 6 (a launch per projection) and 4,
16 and 20 (fused on the matrix cores: a launch per 16 columns and 4 bases),
fp32/fp16/bf16 x, and accumulation.
"""
import numpy as np
import pytest

import oracle
from bit_gemv_packed_amd import synth
from gpu_util import check_close, f16_dev, say, to_dev, x_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import bit_gemv_packed_amd as bsg  # noqa: E402

MULTI_CASES = [
    # K, heights, N, B, colscale, x dtype
    (2, (256, 64, 64), 1024, 1, False, "bf16"),
    (2, (1000, 1000), 512, 1, True, "bf16"),
    (3, (70, 130, 33, 5), 544, 2, False, "f32"),
    (1, (64,) * 8, 256, 1, False, "f16"),
    (2, (300, 0, 200), 256, 1, False, "bf16"),
    (2, (128, 64), 256, 4, False, "bf16"),
    (6, (100, 50), 256, 1, True, "bf16"),
    (2, (4096, 1024, 1024), 4096, 1, False, "bf16"),
    (2, (300, 64, 64), 1024, 16, False, "bf16"),
    (6, (100, 40, 70), 512, 20, False, "f16"),
    (3, (90, 33), 256, 6, False, "bf16"),
]


def _proj_inputs(case, i, M):
    K, hs, N, B, cs, dt = case
    seed = 70000 + 131 * i + K * 7919 + M * 31 + N + B
    L = synth.random_bits(seed, K, M, N) if M else np.zeros((K, 0, N // 32), np.uint32)
    alpha, csb = synth.random_scales(seed, K, M, N, cs)
    return L, alpha, csb


def _run(case, accumulate):
    K, hs, N, B, cs, dt = case
    x = synth.random_x(80000 + N + B, N, B, dt, "normal")
    xd = x_dev(x, dt)
    projs, refs, y0s = [], [], []
    for i, M in enumerate(hs):
        L, alpha, csb = _proj_inputs(case, i, M)
        bits = bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N) if M else None
        ad = to_dev(alpha) if M else None
        cd = f16_dev(csb) if (cs and M) else None
        y0 = synth.random_x(90000 + i, M, B, "f32", "normal") if M else np.zeros((0, B), np.float32)
        y = torch.from_numpy(y0.copy()).to("cuda:0") if (accumulate and M) else None
        projs.append((bits, M, ad, cd, y))
        ref = oracle.sign_gemv(L, K, M, N, alpha, x, csb) if M else np.zeros((0, B))
        if accumulate:
            ref = ref + y0.astype(np.float64)
        refs.append((ref, oracle.tolerance(x, alpha=alpha, colscale_f16=csb, M=M) if M else None, y0))
        y0s.append(y0)
    ys = bsg.bs_gemv_multi(projs, K, N, xd, accumulate=accumulate)
    torch.cuda.synchronize()
    for i, (y, (ref, tol, y0)) in enumerate(zip(ys, refs)):
        if hs[i] == 0:
            continue
        if accumulate:
            tol = tol + 1e-6 * np.abs(y0)
        check_close(y.cpu().numpy(), ref, tol, "bs_gemv_multi %s projection %d" % (case, i))
    return projs, ys, xd


@pytest.mark.parametrize("case", MULTI_CASES, ids=lambda c: "K%d_M%s_N%d_B%d_cs%d_%s" % (
    c[0], "-".join(map(str, c[1])), c[2], c[3], c[4], c[5]))
def test_bs_gemv_multi_matches_oracle(case):
    say("bs_gemv_multi", case)
    projs, ys, xd = _run(case, accumulate=False)
    # fixed-order sums: a second call gives the same bits
    ys2 = bsg.bs_gemv_multi([(b, M, a, c, None) for (b, M, a, c, _) in projs], case[0], case[2], xd)
    torch.cuda.synchronize()
    for y, y2 in zip(ys, ys2):
        assert torch.equal(y, y2)


@pytest.mark.parametrize("case", [MULTI_CASES[0], MULTI_CASES[2], MULTI_CASES[5]],
                         ids=lambda c: "K%d_N%d_B%d" % (c[0], c[2], c[3]))
def test_bs_gemv_multi_accumulates(case):
    say("bs_gemv_multi accumulate", case)
    _run(case, accumulate=True)


def test_bs_gemv_multi_agrees_with_separate_calls():
    """The fused launch and one bs_gemv per projection compute the same
    products (the plans may sum in another order: compared to the bound)."""
    K, N = 2, 2048
    hs = (512, 128, 128)
    say("bs_gemv_multi vs bs_gemv", K, hs, N)
    x = synth.random_x(5, N, 1, "bf16")
    xd = x_dev(x, "bf16")
    projs = []
    for i, M in enumerate(hs):
        L = synth.random_bits(100 + i, K, M, N)
        alpha, _ = synth.random_scales(100 + i, K, M, N, False)
        projs.append((bsg.bsg_logical_to_layout(to_dev(L.view(np.int32)), K, M, N), M, to_dev(alpha), None, None,
                      alpha))
    ys = bsg.bs_gemv_multi([p[:5] for p in projs], K, N, xd)
    sep = [bsg.bs_gemv(b, K, M, N, a, xd) for (b, M, a, _, _, _) in projs]
    torch.cuda.synchronize()
    for (b, M, a, _, _, alpha), y, s in zip(projs, ys, sep):
        tol = oracle.tolerance(x, alpha=alpha, M=M)
        check_close(y.cpu().numpy(), s.cpu().numpy().astype(np.float64), tol, "fused vs separate")
