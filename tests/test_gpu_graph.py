"""Hot calls under HIP graph capture, with caller-owned workspaces.

Nothing in a hot call allocates or synchronises, so the very first call of a
process can be captured; a captured call keeps using the workspace it was
given, whatever runs on the stream between replays.  Every replay is checked
against the oracle, with the program's own eager work and synchronisations
between the replays.
"""
from __future__ import annotations

import os
import subprocess
import sys
import textwrap

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_gemv, assert_within, down, note, require_gpu, up, GEMM_REL

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def torch():
    return require_gpu()


@pytest.fixture(scope="module")
def q4k(torch):
    import bit_block_quantized_gguf_amd as q4k
    return q4k


FIRST_CALL = textwrap.dedent("""
    import sys
    sys.path.insert(0, %r)
    import numpy as np, torch
    import bit_block_quantized_gguf_amd as q4k
    import oracle, synth
    M, K = 3000, 4096
    w = synth.q4k_weight(synth.key(14, 1), M, K)
    x = synth.normal(synth.key(14, 2), K)
    wd = torch.from_numpy(w).cuda(); xd = torch.from_numpy(x).cuda()
    y = torch.empty(M, device="cuda")
    ws = q4k.Workspace(q4k.workspace_size(q4k.OP_GEMV, M, K))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):          # the process's first q4k_gemv call
        q4k.gemv(wd, xd, y, ws=ws)
    yr, S = oracle.gemv(w, x, M, K)
    worst = 0.0
    for r in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy().astype(np.float64) - yr)
        worst = max(worst, float(np.max(err / (1e-4 * S + 1e-6))))
    print("WORST", worst)
""")


def test_first_call_of_a_process_captured():
    note("graph: first q4k_gemv call of a fresh process, captured")
    r = subprocess.run([sys.executable, "-c", FIRST_CALL % ROOT], capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    worst = float(r.stdout.split("WORST")[-1])
    assert worst <= 1.0, worst


def test_graph_keeps_its_workspace_across_other_calls(q4k, torch):
    """Capture a GEMV with workspace A; then run larger eager calls (GEMV and
    batched GEMV with other workspaces) on the same stream between replays."""
    M, K = 2048, 5120
    w = synth.q4k_weight(synth.key(14, 10), M, K)
    x = synth.normal(synth.key(14, 11), K)
    wd, xd = up(w), up(x)
    y = torch.empty(M, device="cuda")
    ws_a = q4k.Workspace(q4k.workspace_size(q4k.OP_GEMV, M, K))
    M2, K2, N2 = 17408, 5120, 16
    w2 = synth.q4k_weight(synth.key(14, 12), M2, K2)
    X2 = synth.activations(14, N2, K2)
    w2d, X2d = up(w2), up(X2)
    Y2 = torch.empty((N2, M2), device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q4k.gemv(wd, xd, y, ws=ws_a)
    yr, S = oracle.gemv(w, x, M, K)
    Y2r, S2 = oracle.gemv_batch(w2, X2, M2, K2, rows=np.arange(0, M2, 97))
    note("graph replays with larger eager calls between them")
    for r in range(3):
        q4k.gemv_batch(w2d, X2d, Y2)            # default workspace of this stream
        y.fill_(float("nan"))
        g.replay()
        got = down(y).astype(np.float64)
        assert_gemv(got, yr, S, "graph replay %d" % r)
        Yg = down(Y2)[:, ::97].astype(np.float64)
        for n in range(N2):
            assert_gemv(Yg[n], Y2r[n], S2[n], "eager batch between replays n=%d" % n)


def test_graph_of_gemm_and_mlp(q4k, torch):
    """The GEMM (bf16 copy of X and stream-K partials in the workspace) and the
    MLP block (its intermediates in the workspace), captured and replayed."""
    M, K, P = 1280, 1024, 96
    w = synth.q4k_weight(synth.key(14, 20), M, K)
    X = synth.activations(14, P, K, first=20)
    wd, Xd = up(w), up(X)
    Y = torch.empty((P, M), device="cuda")
    ws_g = q4k.Workspace(q4k.workspace_size(q4k.OP_GEMM, M, K, P))
    H, I = 512, 1024
    wg, wu = (synth.q4k_weight(synth.key(14, 21 + i), I, H) for i in (0, 1))
    wdn = synth.q4k_weight(synth.key(14, 23), H, I)
    xm = synth.normal(synth.key(14, 24), H)
    ym = torch.empty(H, device="cuda")
    ws_m = q4k.Workspace(q4k.workspace_size(q4k.OP_MLP, I, H))
    dev = [up(a) for a in (wg, wu, wdn, xm)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q4k.gemm(wd, Xd, Y, ws=ws_g)
        q4k.mlp(dev[0], dev[1], dev[2], dev[3], None, 1e-6, dev[3], ym, ws=ws_m)
    Yr, S = oracle.gemm(w, X, M, K)
    om = oracle.mlp(wg, wu, wdn, H, I, xm, None, 1e-6, xm)
    eager = down(q4k.mlp(dev[0], dev[1], dev[2], dev[3], None, 1e-6, dev[3])).copy()
    note("graph of gemm + mlp")
    for r in range(3):
        Y.fill_(float("nan"))
        ym.fill_(float("nan"))
        g.replay()
        assert_within(down(Y).astype(np.float64), Yr, S, GEMM_REL, "graph gemm %d" % r)
        got = down(ym)
        # same kernels, same launch shapes, same inputs: the same bits as eager
        assert np.array_equal(got.view(np.uint32), eager.view(np.uint32)), r
        c = float(got.astype(np.float64) @ om["y"] /
                  (np.linalg.norm(got.astype(np.float64)) * np.linalg.norm(om["y"])))
        assert c >= 0.999999, c


def test_one_workspace_serves_every_kind_of_call(q4k, torch):
    """Calls of different kinds ordered on one stream may share a workspace:
    a GEMM's partial tiles and bf16 X never land on the GEMV counters."""
    M, K, P = 2048, 5120, 200
    w = synth.q4k_weight(synth.key(14, 40), M, K)
    x = synth.normal(synth.key(14, 41), K)
    X = synth.activations(14, P, K, first=40)
    w8 = synth.q8_0_weight(synth.key(14, 42), M, K)
    w6 = synth.q6_k_weight(synth.key(14, 43), M, K)
    need = max(q4k.workspace_size(op, M, K, n) for op, n in
               ((q4k.OP_GEMV, 1), (q4k.OP_GEMM, P), (q4k.OP_GEMV_Q8_0, 1),
                (q4k.OP_GEMV_Q6_K, 1), (q4k.OP_GEMV_BATCH, 5)))
    ws = q4k.Workspace(need)
    wd, xd, Xd = up(w), up(x), up(X)
    yr, S = oracle.gemv(w, x, M, K)
    Yr, SY = oracle.gemm(w, X, M, K, toks=np.arange(0, P, 7))
    note("one workspace, every kind of call")
    for r in range(2):
        Y = down(q4k.gemm(wd, Xd, ws=ws))[::7].astype(np.float64)
        assert_within(Y, Yr, SY, GEMM_REL, "gemm %d" % r)
        assert_gemv(down(q4k.gemv(wd, xd, ws=ws)).astype(np.float64), yr, S, "gemv %d" % r)
        y8r, S8 = oracle.gemv_q8_0(w8, x, M, K)
        assert_gemv(down(q4k.gemv_q8_0(up(w8), xd, ws=ws)).astype(np.float64), y8r, S8, "q8 %d" % r)
        y6r, S6 = oracle.gemv_q6_k(w6, x, M, K)
        assert_gemv(down(q4k.gemv_q6_k(up(w6), xd, ws=ws)).astype(np.float64), y6r, S6, "q6 %d" % r)
        Yb = down(q4k.gemv_batch(wd, Xd[:5], ws=ws)).astype(np.float64)
        Ybr, Sb = oracle.gemv_batch(w, X[:5], M, K)
        for n in range(5):
            assert_gemv(Yb[n], Ybr[n], Sb[n], "batch %d n=%d" % (r, n))
