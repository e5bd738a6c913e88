"""GPU tests of w12_gemm_noalloc, the GEMM entry point that allocates nothing and runs on the
library's own per-device scratch array: bitwise the same Y as w12_gemm (same kernels, same
plan) and within the oracle's tolerance, on consecutive calls whose second input is smaller
(the scratch keeps the first call's partial sums), and a clear error above its size limit.
"""
import numpy as np
import pytest
import torch

import lossless_bit_weight_encode_amd as w12
import w12_synth as S
from oracle import w12_oracle as O
from gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


def _weights(n, k, seed):
    return S.layer_matrix(torch.Generator().manual_seed(seed), n, k)


def _check_call(w, t, m, seed):
    n, k = w.shape
    x = S.activations(m, k, seed)
    xd = to_dev(x, (k + 7) // 8 * 8)
    canary = -777.25
    buf = torch.full((m + 2, n + 5), canary, dtype=torch.float32, device="cuda")
    y = buf[:m, :n]
    w12.gemm_noalloc(xd, t, y)
    ref = w12.gemm(xd, t)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.array_equal(yh.view(np.uint32), ref.cpu().numpy().view(np.uint32)), \
        f"M={m} N={n} K={k}: w12_gemm_noalloc differs from w12_gemm"
    bad, worst = O.gemm_check(x, w, yh)
    assert bad == 0, f"M={m} N={n} K={k}: {bad} outputs outside tolerance (worst rel {worst:.3g})"
    bh = buf.cpu().numpy()
    assert (bh[:m, n:] == np.float32(canary)).all() and (bh[m:, :] == np.float32(canary)).all(), "write outside Y"


@pytest.mark.parametrize("first,second", [((32, 1000, 4096), (5, 300, 1008)),
                                          ((16, 2048, 2048), (1, 200, 512)),
                                          ((64, 700, 3000), (17, 130, 640))])
def test_noalloc_matches_gemm_on_consecutive_calls(first, second):
    """Two calls in a row, the second on a smaller input; each is compared with w12_gemm."""
    for i, (m, n, k) in enumerate([first, second]):
        say(f"[noalloc] call {i}: M={m} N={n} K={k}")
        w = _weights(n, k, 40 + i + n)
        t = w12.encode(to_dev(w, (k + 7) // 8 * 8))
        plan = w12.gemm_plan(m, n, k)
        assert plan["splits"] > 1 or m == 1, "the case must exercise split-K"
        _check_call(w, t, m, 3000 + m + n)


def test_noalloc_repeats_bitwise():
    """Ten calls in a row on one input give the same bits (the counters return to zero)."""
    w = _weights(300, 4096, 7)
    t = w12.encode(to_dev(w))
    x = to_dev(S.activations(16, 4096, 99))
    y = torch.empty(16, 300, dtype=torch.float32, device="cuda")
    outs = []
    for _ in range(10):
        w12.gemm_noalloc(x, t, y)
        outs.append(y.cpu().numpy().view(np.uint32).copy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_noalloc_rejects_plans_above_its_scratch():
    """M = 256 on a 4096 x 4096 matrix (wide tiles) needs more workspace than the scratch holds:
    a clear error before any launch, and w12_gemm still serves it."""
    n, k, m = 4096, 4096, 256
    assert w12.gemm_workspace_size(m, n, k) > 32 << 20
    w = _weights(n, k, 11)
    t = w12.encode(to_dev(w))
    x = to_dev(S.activations(m, k, 5))
    y = torch.empty(m, n, dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="scratch"):
        w12.gemm_noalloc(x, t, y)
    # calls within the limit still work afterwards
    w_small = _weights(64, 512, 3)
    _check_call(w_small, w12.encode(to_dev(w_small)), 8, 17)
