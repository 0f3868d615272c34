"""bs_gemv captured in a HIP graph (as the benchmark times it) gives, on every
replay, exactly what the same launch gives eagerly."""
import numpy as np
import pytest
import torch

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def test_bs_gemv_graph_replay_matches_eager():
    import bit_gemv_packed_amd as bsg
    from bit_gemv_packed_amd import synth
    M, N, K = 1024, 4096, 2
    say("graph replay", M, N, K)
    W = torch.from_numpy(synth.weights(2, 7, M, N)).to(DEV)
    bits, alpha, cs = bsg.bsq_pack(W, K, colscale=True)
    xs = [torch.randn(N, device=DEV).to(torch.bfloat16) for _ in range(3)]
    ys = [torch.empty(M, device=DEV) for _ in range(3)]
    ref = [bsg.bs_gemv(bits, K, M, N, alpha, x, colscale=cs).clone() for x in xs]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for x, y in zip(xs, ys):
            bsg.bs_gemv(bits, K, M, N, alpha, x, colscale=cs, y=y)
    for rep in range(4):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for y, r in zip(ys, ref):
            assert torch.equal(y, r.view_as(y)), "replay %d differs from the eager launch" % rep
        # eager work between replays
        bsg.bs_gemv(bits, K, M, N, alpha, xs[0], colscale=cs, y=ys[0])
        torch.cuda.synchronize()
