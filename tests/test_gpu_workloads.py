"""End-to-end parity on the full-size synthetic workloads (the shapes of the
pages' LLaMA-2/3.1 and Qwen3 projections), through the same calls and launch
plans the benchmark times.

Per workload shape: GPU packing must equal the oracle's packing bit for bit
(sign bits, row scales, column scales, protected rows and their int8 codes);
the full product  y = bases + binary low-rank + protected rows, computed both
by the separate calls and by the fused bsg_linear, must lie within the
per-output bound at every output for batch 1, and on a seeded sample of rows
for the larger batches.
"""
import numpy as np
import pytest

import oracle
from bit_gemv_packed_amd import synth
from gpu_util import check_close, f16_dev, say, to_dev, u16, u32, x_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import bit_gemv_packed_amd as bsg  # noqa: E402

CASES = [(1, 0), (2, 0), (3, 0)] + [(4, p) for p in range(7)] + [(5, p) for p in range(3)]


@pytest.mark.parametrize("wid,part", CASES, ids=lambda c: str(c))
def test_workload_end_to_end(wid, part):
    w = synth.WORKLOADS[wid]
    sh = w.shapes[part]
    M, N, K = sh.M, sh.N, w.K
    say("workload", w.name, sh.name, "M=%d N=%d K=%d" % (M, N, K))
    W = synth.weights(wid, part, M, N)
    Wd = to_dev(W)

    # ---- GPU packing
    bits, alpha, cs = bsg.bsq_pack(Wd, K, colscale=w.colscale)
    rows = q = s = None
    ns = synth.n_salient(M, w.salient_frac) if w.salient_frac else 0
    if ns:
        X = synth.calibration(w, part, N, 128)
        xbar = bsg.bsq_absmean(to_dev(X))
        rows, q, s = bsg.bsq_salient(Wd, xbar, ns, alpha)
    lr = synth.low_rank(w, part, M, N)
    if lr is not None:
        Ub = bsg.bsq_pack_signs(to_dev(lr.u))
        Vb = bsg.bsq_pack_signs(to_dev(lr.v))
        ard = f16_dev(lr.alpha_r_f16)
    torch.cuda.synchronize()
    del Wd

    # ---- oracle packing, compared bit for bit
    rb, ra, rc = oracle.pack(W, K, w.colscale)
    np.testing.assert_array_equal(u32(bsg.bsg_layout_to_logical(bits, K, M, N)).reshape(K, M, -1), rb)
    if w.colscale:
        np.testing.assert_array_equal(u16(cs), rc)
    orows = oq = os_ = None
    if ns:
        orows, oq, os_, ra = oracle.salient_select(W, oracle.absmean(X), ns, ra)
        np.testing.assert_array_equal(rows.cpu().numpy(), orows)
        np.testing.assert_array_equal(q.cpu().numpy(), oq)
        np.testing.assert_array_equal(u16(s), os_)
    np.testing.assert_array_equal(alpha.cpu().numpy().view(np.uint32), ra.view(np.uint32))
    del W
    if lr is not None:
        ub, vb = oracle.pack_signs(lr.u), oracle.pack_signs(lr.v)
        np.testing.assert_array_equal(u32(bsg.bsg_layout_to_logical(Vb, 1, lr.r, N)).reshape(lr.r, -1), vb)

    # ---- the product
    for B in w.batches:
        x = synth.activations(w, part, N, B)
        xd = x_dev(x, w.x_dtype)
        say("  batch", B)
        y = bsg.bs_gemv(bits, K, M, N, alpha, xd, colscale=cs)
        if lr is not None:
            bsg.binlr_apply(Ub, Vb, ard, lr.r, M, N, xd, y)
        if ns:
            bsg.salient_int8_apply(rows, q, s, M, N, xd, y)
        torch.cuda.synchronize()
        yh = y.cpu().numpy()
        if B == 1:
            sel = np.arange(M)
        else:
            sel = np.sort(np.random.default_rng([wid, part, B]).choice(M, min(M, 192), replace=False))
        ref = oracle.sign_gemv(np.ascontiguousarray(rb[:, sel]), K, len(sel), N, ra[:, sel], x, rc)
        tolkw = dict(alpha=ra[:, sel], colscale_f16=rc)
        if lr is not None:
            ref += oracle.binlr(np.ascontiguousarray(ub[sel]), vb, lr.alpha_r_f16, lr.r, len(sel), N, x)
            tolkw["alpha_r_f16"] = lr.alpha_r_f16
        if ns:
            full = oracle.salient(orows, oq, os_, M, N, x)
            ref += full[sel]
            # restrict the protected-row term of the bound to the sampled rows
            pos = {m: i for i, m in enumerate(sel)}
            keep = [i for i, m in enumerate(orows) if m in pos]
            tolkw.update(rows=np.array([pos[orows[i]] for i in keep], np.int64),
                         q=oq[keep], s_f16=os_[keep])
        tol = oracle.tolerance(x, M=len(sel), **tolkw)
        err, ratio = check_close(yh[sel], ref, tol, "%s/%s B=%d" % (w.name, sh.name, B))
        say("  max err %.3e, max err/tol %.3f" % (err, ratio))
        # the same layer through the fused entry point
        yf = bsg.bsg_linear(bits, K, M, N, alpha, xd, colscale=cs,
                            lowrank=(Ub, Vb, ard, lr.r) if lr is not None else None,
                            salient=(rows, q, s) if ns else None)
        torch.cuda.synchronize()
        err, ratio = check_close(yf.cpu().numpy()[sel], ref, tol, "fused %s/%s B=%d" % (w.name, sh.name, B))
        say("  fused: max err %.3e, max err/tol %.3f" % (err, ratio))
