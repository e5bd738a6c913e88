"""GEMM calls captured in a HIP graph (torch.cuda.graph) and replayed.

The library launches only kernels on the caller's stream (arguments by value, no memset, no
host synchronisation), so a captured call replays the launch it recorded: w12_gemm, a grouped
launch in the kernel-argument form (up to GROUP_INLINE products), a larger group (whose argument
blocks are stored into the workspace by kernels taking them by value) and w12_gemm_noalloc.
Every replay is compared bit for bit with the eager result, with the outputs poisoned and other
eager GEMM work on the same workspace between the replays, and checked against the FP64 oracle.
"""
import numpy as np
import pytest
import torch

import lossless_bit_weight_encode_amd as w12
import w12_synth as S
from oracle import w12_oracle as O
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [("gauss", 300, 4096), ("heavy", 64, 2048), ("wide", 37, 1008), ("gauss", 130, 640), ("wide", 70, 272)]
_cache = {}


def weights(i):
    kind, n, k = SHAPES[i % len(SHAPES)]
    if i not in _cache:
        if kind == "gauss":
            w = S.layer_matrix(torch.Generator().manual_seed(60 + i), n, k)
        elif kind == "heavy":
            w = S.heavy_tail_weights(1100 + i, n, k)
        else:
            w = S.random_bits_matrix(np.random.default_rng(70 + i), n, k, "wide")
        _cache[i] = (w, w12.encode(to_dev(w)))
    return _cache[i]


def replay_and_check(graph, ys, ref, interleave, replays=4):
    for r in range(replays):
        for y in ys:
            y.fill_(float("nan"))
        interleave()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (y, y0) in enumerate(zip(ys, ref)):
            assert torch.equal(y, y0), f"replay {r}, output {i}: differs from the eager call"


def interleaved_gemm(ws, m):
    """Eager GEMM work between replays, on the same workspace (its counters must come back to
    zero for the next replay)."""
    w, t = weights(0)
    x = to_dev(S.activations(m, w.shape[1], 31))

    def run():
        w12.gemm(x, t, ws=ws)
    return run


@pytest.mark.parametrize("m", [1, 16, 33])
def test_graph_replays_single_gemm(m):
    w, t = weights(0)
    x = S.activations(m, w.shape[1], 100 + m)
    xd = to_dev(x)
    y = torch.empty(m, t.n, dtype=torch.float32, device="cuda")
    ws = w12.gemm_workspace(m, t.n, t.k)
    w12.gemm(xd, t, y=y, ws=ws)
    torch.cuda.synchronize()
    ref = [y.clone()]
    bad, worst = O.gemm_check(x, w, y.cpu().numpy())
    assert bad == 0, f"eager: {bad} outputs outside tolerance (worst rel {worst:.3g})"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w12.gemm(xd, t, y=y, ws=ws)
    say(f"[graph] single M={m} captured")
    replay_and_check(g, [y], ref, interleaved_gemm(ws, m))


@pytest.mark.parametrize("count", [3, 8, 9, 21])
@pytest.mark.parametrize("m", [1, 16])
def test_graph_replays_group(m, count):
    ws_, ts, xs = [], [], []
    for i in range(count):
        w, t = weights(i)
        ws_.append(w)
        ts.append(t)
        xs.append(S.activations(m, w.shape[1], 200 + 7 * i + m))
    xd = [to_dev(x) for x in xs]
    ys = [torch.empty(m, t.n, dtype=torch.float32, device="cuda") for t in ts]
    # the workspace also serves the interleaved single GEMM
    need = max(w12.gemm_group_workspace_size(m, ts), w12.gemm_workspace_size(m, ts[0].n, ts[0].k))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    w12.gemm_workspace_init(ws)
    w12.gemm_group(xd, ts, ys, ws=ws)
    torch.cuda.synchronize()
    ref = [y.clone() for y in ys]
    for i in range(count):
        bad, worst = O.gemm_check(xs[i], ws_[i], ys[i].cpu().numpy())
        assert bad == 0, f"eager item {i}: {bad} outputs outside tolerance (worst rel {worst:.3g})"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w12.gemm_group(xd, ts, ys, ws=ws)
    say(f"[graph] group of {count} M={m} captured")
    replay_and_check(g, ys, ref, interleaved_gemm(ws, m))
    assert int(ws[:w12.gemm_plan(1, 16, 16)["counter_bytes"]].count_nonzero()) == 0


def test_graph_replays_noalloc():
    m = 16
    w, t = weights(3)
    x = S.activations(m, w.shape[1], 300)
    xd = to_dev(x)
    y = torch.empty(m, t.n, dtype=torch.float32, device="cuda")
    w12.gemm_noalloc(xd, t, y)   # the first call on the device sets the library's array up
    torch.cuda.synchronize()
    ref = [y.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w12.gemm_noalloc(xd, t, y)
    say("[graph] noalloc captured")
    w2, t2 = weights(4)
    x2 = to_dev(S.activations(m, w2.shape[1], 301))
    y2 = torch.empty(m, t2.n, dtype=torch.float32, device="cuda")

    def between():
        w12.gemm_noalloc(x2, t2, y2)   # eager calls share the array with the replays
    replay_and_check(g, [y], ref, between)
    bad, worst = O.gemm_check(x, w, y.cpu().numpy())
    assert bad == 0, f"{bad} outputs outside tolerance (worst rel {worst:.3g})"
