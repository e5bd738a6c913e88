"""GPU parity on seeded random shapes: ragged N and K, several value mixes, M from 1 to 300.

Each case checks the encode (bases, records, escape pointers and list) against the oracle bit for
bit, the load-time check and the decode, and the GEMM (exact and Q pass) within the tolerance.
Grouped launches take random sets of products with K a multiple of 16."""
import numpy as np
import pytest
import torch

import lossless_bit_weight_encode_amd as w12
import w12_synth as S
from oracle import w12_oracle as O
from gpu_util import assert_encode_equal, say, to_dev, u16

pytestmark = pytest.mark.gpu

KINDS = ("gauss", "wide", "heavy", "zeros_mix")


def _weights(rng, kind, n, k):
    if kind == "gauss":
        return S.random_bits_matrix(rng, n, k, "gauss")
    if kind == "wide":
        return S.random_bits_matrix(rng, n, k, "wide")
    if kind == "heavy":
        return S.heavy_tail_weights(int(rng.integers(0, 1 << 30)), n, k)
    w = S.random_bits_matrix(rng, n, k, "gauss")
    w[rng.random((n, k)) < 0.2] = 0   # many zeros: long escape lists
    return w


def _case(seed):
    rng = np.random.default_rng(10_000 + seed)
    n = int(rng.integers(1, 300))
    k = int(rng.integers(1, 3000))
    kind = KINDS[seed % len(KINDS)]
    m = int(rng.choice([1, 2, 3, 7, 9, 16, 17, 31, 33, 48, 64, 65, 100, 129, 300]))
    return rng, n, k, kind, m


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_parity(seed):
    rng, n, k, kind, m = _case(seed)
    say(f"[random] seed={seed} N={n} K={k} kind={kind} M={m}")
    w = _weights(rng, kind, n, k)
    ref = O.encode(w)
    ld = (k + 7) // 8 * 8
    wd = to_dev(w, ld)
    t = w12.encode(wd)
    assert_encode_equal(t, ref)
    assert w12.verify(t, wd) == (0, -1)
    assert np.array_equal(u16(w12.decode(t)), w)
    x = S.activations(m, k, 20_000 + seed)
    xd = to_dev(x, ld)
    y = w12.gemm(xd, t).cpu().numpy()
    bad, worst = O.gemm_check(x, w, y)
    assert bad == 0, f"GEMM: {bad} outputs outside tolerance (worst {worst:.3g})"
    yq = w12.gemm(xd, t, qpass=True).cpu().numpy()
    bad, worst = O.gemm_q_check(x, ref, yq)
    assert bad == 0, f"Q pass: {bad} outputs outside tolerance (worst {worst:.3g})"


@pytest.mark.parametrize("seed", range(12))
def test_random_group_parity(seed):
    rng = np.random.default_rng(30_000 + seed)
    # both forms: arguments in the kernel arguments (<= GROUP_INLINE) and in the workspace
    count = int(rng.integers(1, 3 * w12.GROUP_INLINE + 1))
    m = int(rng.choice([1, 2, 5, 16, 24, 40, 64]))
    say(f"[random group] seed={seed} count={count} M={m}")
    ws_, ts, xs = [], [], []
    for i in range(count):
        n = int(rng.integers(1, 400))
        k = 16 * int(rng.integers(1, 200))
        w = _weights(rng, KINDS[(seed + i) % len(KINDS)], n, k)
        ws_.append(w)
        ts.append(w12.encode(to_dev(w)))
        xs.append(S.activations(m, k, 40_000 + 97 * seed + i))
    ys = w12.gemm_group([to_dev(x) for x in xs], ts)
    for i in range(count):
        bad, worst = O.gemm_check(xs[i], ws_[i], ys[i].cpu().numpy())
        assert bad == 0, f"item {i}: {bad} outputs outside tolerance (worst {worst:.3g})"
