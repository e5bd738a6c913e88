"""GPU parity at the full sizes of the five synthetic workloads, in the launch configuration
the benchmark uses (the default GEMM plan and a workspace from gemm_workspace()).

* Encode: full-tensor bit-identity with the oracle (window bases, escape pointers, escape
  list and logical records) for the dense-layer and heavy-tail matrices; sampled channels
  for the extra full-model layers.  The encode is per channel, so a sampled channel is
  checked exactly.
* Load-time check: w12_verify over the whole tensor reports zero mismatches.
* GEMM: every output of Y (the dense layer at M = 16, the tree-verify M sweep, the batched M
  = 256 / 512 and the heavy-tail matrices at M = 16, 256, 512) within 2^-12 * sum|x w| of the
  FP64 reference; for the extra full-model layers every output of a sample of channels.  The
  full Y is bitwise identical over repeated runs.
"""
import numpy as np
import pytest
import torch

import lossless_bit_weight_encode_amd as w12
import w12_synth as S
from oracle import w12_oracle as O
from gpu_util import assert_encode_equal, say, to_dev, u16, u32

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]

_layers = {}
_heavy = {}
_enc = {}


def layer(seed):
    if seed not in _layers:
        say(f"[configs] generating layer seed {seed}")
        _layers.clear()   # keep host memory bounded: one layer at a time
        _layers[seed] = S.layer(seed)
    return _layers[seed]


def heavy(name):
    """Heavy-tailed weights with 2% out-of-window values on the gate_up (seed 1000) and down
    (seed 1001) shapes."""
    if name not in _heavy:
        n, k = S.LAYER_SHAPES[name]
        seed = 1000 if name == "gate_up" else 1001
        say(f"[configs] generating heavy-tail {name} seed {seed}")
        _heavy[name] = S.heavy_tail_weights(seed, n, k)
    return _heavy[name]


def encoded(key, w):
    if key not in _enc:
        _enc.clear()
        t = w12.encode(to_dev(w))
        torch.cuda.synchronize()
        _enc[key] = t
    return _enc[key]


def sample_rows(n, count=192, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(range(min(64, n))) | set(range(max(0, n - 64), n))
    rows |= set(rng.choice(n, size=min(count, n), replace=False).tolist())
    return np.array(sorted(rows))


def check_verify(t, w):
    cnt, first = w12.verify(t, to_dev(w))
    assert (cnt, first) == (0, -1), f"load-time check found {cnt} mismatches (first {first})"


def check_encode_rows(t, w, rows):
    """Exact encode parity on the given channels (the oracle encodes them on their own)."""
    ref = O.encode(w[rows])
    base = t.base.cpu().numpy()
    ptr = u32(t.esc_ptr)
    esc = u32(t.esc) if t.num_escapes else np.zeros(0, np.uint32)
    assert np.array_equal(base[rows], ref.base)
    rec = u16(w12.unpack_records(t))
    assert np.array_equal(rec[rows], ref.rec)
    for i, r in enumerate(rows):
        got = esc[ptr[r]:ptr[r + 1]]
        want = ref.esc[ref.esc_ptr[i]:ref.esc_ptr[i + 1]]
        assert np.array_equal(got, want), f"escape list of channel {r} differs"


def check_gemm(t, w, m, x_seed, rows=None, repeats=2):
    """Y = X W^T on the GPU against the FP64 oracle: every output (rows=None) or the given
    output channels; bitwise repeatable."""
    n, k = w.shape
    x = S.activations(m, k, x_seed)
    xd = to_dev(x)
    ws = w12.gemm_workspace(m, n, k)
    y = w12.gemm(xd, t, ws=ws)
    torch.cuda.synchronize()
    for _ in range(repeats - 1):
        y2 = w12.gemm(xd, t, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, y2), "GEMM output is not bitwise repeatable"
    yh = y.cpu().numpy()
    if rows is None:
        bad, worst = O.gemm_check(x, w, yh)
        what = f"of all {m * n}"
    else:
        bad, worst = O.gemm_check(x, w[rows], yh[:, rows])
        what = f"of {m * len(rows)} sampled"
    assert bad == 0, f"M={m}: {bad} outputs {what} outside tolerance (worst rel {worst:.3g})"
    assert np.isfinite(yh).all()
    return y


# ---- config 1: the tiny round trip + GEMV, exhaustively -------------------------------------
def test_config1_tiny_roundtrip_and_gemv():
    w = S.tiny_weights(0)
    ref = O.encode(w)
    t = w12.encode(to_dev(w))
    assert_encode_equal(t, ref)
    check_verify(t, w)
    assert np.array_equal(u16(w12.decode(t))[:, :w.shape[1]], w)
    x = S.activations(1, 512, S.x_seed(1, 512))
    y = w12.gemm(to_dev(x), t, ws=w12.gemm_workspace(1, 256, 512)).cpu().numpy()
    bad, worst = O.gemm_check(x, w, y)
    assert bad == 0, f"{bad} outputs outside tolerance (worst {worst:.3g})"
    say(f"[configs] tiny: E={ref.num_escapes} bits/weight={O.bits_per_weight(256, 512, ref.num_escapes):.4f}")


# ---- config 2: one dense decoder layer, M = 16 ----------------------------------------------
@pytest.mark.parametrize("name", S.LAYER_ORDER)
def test_config2_layer_encode_verify_gemm(name):
    w = layer(0)[name]
    n, k = w.shape
    t = encoded(("layer0", name), w)
    ref = O.encode(w)
    assert_encode_equal(t, ref)
    bpw = t.bits_per_weight()
    say(f"[configs] layer0 {name}: E={t.num_escapes} bits/weight={bpw:.5f}")
    assert 12.0 < bpw < 12.03
    check_verify(t, w)
    check_gemm(t, w, 16, S.x_seed(16, k))


# ---- config 3: tree-verify M sweep on gate_up and down ------------------------------------
@pytest.mark.parametrize("name", ["gate_up", "down"])
@pytest.mark.parametrize("m", S.TREE_M_SWEEP)
def test_config3_m_sweep(name, m):
    w = layer(0)[name]
    n, k = w.shape
    t = encoded(("layer0", name), w)
    check_gemm(t, w, m, S.x_seed(m, k))


# ---- config 4: full-model layers (sampled: first, middle and last layer) -----------------------
@pytest.mark.parametrize("seed", [1, 31, 63])
def test_config4_model_layers(seed):
    lay = layer(seed)
    for name in S.LAYER_ORDER:
        w = lay[name]
        n, k = w.shape
        t = w12.encode(to_dev(w))
        rows = sample_rows(n, count=64, seed=seed)
        check_encode_rows(t, w, rows)
        check_verify(t, w)
        check_gemm(t, w, 32, S.x_seed(32, k), rows)
        del t
        torch.cuda.empty_cache()


# ---- config 5: batched verify (MFMA tiles) and escape stress ------------------------------------
@pytest.mark.parametrize("name", ["gate_up", "down"])
@pytest.mark.parametrize("m", S.BATCHED_M)
def test_config5_batched(name, m):
    w = layer(0)[name]
    n, k = w.shape
    t = encoded(("layer0", name), w)
    check_gemm(t, w, m, S.x_seed(m, k))


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_config5_heavy_tail(name):
    w = heavy(name)
    n, k = w.shape
    t = encoded(("heavy", name), w)
    ref = O.encode(w)
    assert_encode_equal(t, ref)
    frac = t.num_escapes / (n * k)
    say(f"[configs] heavy {name}: E={t.num_escapes} ({100 * frac:.3f}%) bits/weight={t.bits_per_weight():.4f}")
    assert 0.02 < frac < 0.03
    check_verify(t, w)
    for m in (16, 256, 512):
        check_gemm(t, w, m, S.x_seed(m, k))


# ---- the Q pass (nested 8-bit view) on the dense layer, M = 16, and the heavy tail ---------------
@pytest.mark.parametrize("name", S.LAYER_ORDER)
def test_config2_layer_qpass(name):
    w = layer(0)[name]
    n, k = w.shape
    t = encoded(("layer0", name), w)
    rows = sample_rows(n, count=96, seed=3)
    x = S.activations(16, k, S.x_seed(16, k))
    ws = w12.gemm_workspace(16, n, k)
    y = w12.gemm(to_dev(x), t, ws=ws, qpass=True)
    y2 = w12.gemm(to_dev(x), t, ws=ws, qpass=True)
    torch.cuda.synchronize()
    assert torch.equal(y, y2), "Q-pass GEMM is not bitwise repeatable"
    ref = O.encode(w[rows])
    bad, worst = O.gemm_q_check(x, ref, y.cpu().numpy()[:, rows])
    assert bad == 0, f"{bad} sampled Q-pass outputs outside tolerance (worst rel {worst:.3g})"


def test_config5_heavy_tail_qpass():
    w = heavy("down")
    n, k = w.shape
    t = encoded(("heavy", "down"), w)
    rows = sample_rows(n, count=48, seed=9)
    x = S.activations(16, k, S.x_seed(16, k))
    y = w12.gemm(to_dev(x), t, ws=w12.gemm_workspace(16, n, k), qpass=True)
    torch.cuda.synchronize()
    bad, worst = O.gemm_q_check(x, O.encode(w[rows]), y.cpu().numpy()[:, rows])
    assert bad == 0, f"{bad} sampled Q-pass outputs outside tolerance (worst rel {worst:.3g})"
