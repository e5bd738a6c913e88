"""Pins for the CPU oracle: checks against facts fixed by the definition, not by the oracle.

Each test names what pins it: a hand-derived fixture, a closed form, a brute force on
tiny inputs, an invariant or an exact summation.  None of these tests touches a GPU.
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import w12_oracle as O
import w12_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def all_bf16_patterns():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


# ---------------------------------------------------------------------------------------
# Hand-derived fixtures
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("ch", _load("w12_hand_channels.json")["channels"], ids=lambda c: c["name"])
def test_hand_channel(ch):
    w = np.array([ch["w"]], dtype=np.uint16)
    t = O.encode(w)
    assert int(t.base[0]) == ch["base"]
    assert t.rec[0].tolist() == ch["rec"]
    assert t.esc.tolist() == ch["esc"]
    assert t.esc_ptr.tolist() == [0, len(ch["esc"])]
    assert np.array_equal(O.decode(t), w)
    if "bits_per_weight" in ch:
        assert O.bits_per_weight(1, w.shape[1], t.num_escapes) == pytest.approx(ch["bits_per_weight"], abs=1e-12)


def test_hand_channels_stacked():
    """All hand channels in one matrix, padded with +0 (field 0 never joins a window, so
    every pad is one more escape (k << 16) | 0 and the windows are unchanged)."""
    chans = _load("w12_hand_channels.json")["channels"]
    k = max(len(c["w"]) for c in chans) + 2
    rows, exp_rec, exp_esc = [], [], []
    for c in chans:
        npad = k - len(c["w"])
        rows.append(c["w"] + [0] * npad)
        exp_rec.append(c["rec"] + [0] * npad)
        exp_esc.append(c["esc"] + [(kk << 16) for kk in range(len(c["w"]), k)])
    w = np.array(rows, dtype=np.uint16)
    t = O.encode(w)
    assert t.base.tolist() == [c["base"] for c in chans]
    assert t.rec.tolist() == exp_rec
    assert t.esc.tolist() == [e for row in exp_esc for e in row]
    assert t.esc_ptr.tolist() == np.concatenate([[0], np.cumsum([len(e) for e in exp_esc])]).tolist()
    assert np.array_equal(O.decode(t), w)


@pytest.mark.parametrize("case", _load("w12_hand_channels.json")["bits_per_weight_cases"])
def test_bits_per_weight_hand(case):
    assert O.bits_per_weight(case["n"], case["k"], case["e"]) == pytest.approx(case["bpw"], rel=0, abs=1e-12)


def _as_float(v):
    """A JSON number, or a string: "inf", "-inf", "nan", or an exact hexadecimal float."""
    if not isinstance(v, str):
        return float(v)
    return float.fromhex(v) if "0x" in v else float(v)


@pytest.mark.parametrize("case", _load("w12_hand_gemm.json")["cases"], ids=lambda c: c["name"])
def test_gemm_hand(case):
    x = np.array(case["x"], dtype=np.uint16)
    w = np.array(case["w"], dtype=np.uint16)
    y, a = O.gemm_reference(x, w)
    exp = np.array([[_as_float(v) for v in row] for row in case["y"]])
    assert y.shape == exp.shape
    fin = np.isfinite(exp)
    assert np.array_equal(y[fin], exp[fin])
    assert np.array_equal(np.isnan(y), np.isnan(exp))
    assert np.array_equal(y[np.isinf(exp)], exp[np.isinf(exp)])
    if "a" in case:
        assert np.array_equal(a, np.array([[_as_float(v) for v in row] for row in case["a"]], dtype=np.float64))


# ---------------------------------------------------------------------------------------
# The exhaustive channel: every BF16 pattern once in one channel of K = 65536
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("shuffle", [False, True])
def test_exhaustive_channel(shuffle):
    w = all_bf16_patterns()
    if shuffle:
        w = w[np.random.default_rng(0).permutation(w.size)]
    w = w[None, :]
    t = O.encode(w)
    # every exponent field occurs 256 times, so every window holds 16*256 = 4096: all tie, b = 1
    assert int(t.base[0]) == 1
    assert t.num_escapes == 65536 - 4096 == 61440
    e = (w[0].astype(np.int32) >> 7) & 0xFF
    esc_k = (t.esc >> 16).astype(np.int64)
    assert np.array_equal(esc_k, np.flatnonzero((e < 1) | (e > 16)))
    assert np.array_equal((t.esc & 0xFFFF).astype(np.uint16), w[0, esc_k])
    assert np.array_equal(O.decode(t), w)


def test_forced_window_sweep():
    """Any b in 1..239 encodes losslessly; the escapes are exactly the fields outside [b, b+15]."""
    w = all_bf16_patterns()[None, :]
    e = (w[0].astype(np.int32) >> 7) & 0xFF
    val = O.bf16_to_f64(w[0])
    for b in range(1, 240):
        t = O.encode(w, forced_base=np.array([b], dtype=np.uint8))
        out = (e < b) | (e > b + 15)
        assert t.num_escapes == 61440
        assert np.array_equal((t.esc >> 16).astype(np.int64), np.flatnonzero(out))
        assert np.array_equal(O.decode(t), w)
        # the records mean (-1)^s * 2^(off + b - 127) * (1 + m/128): check by float arithmetic
        r = t.rec[0, ~out].astype(np.int64)
        s = r >> 11
        off = (r >> 7) & 15
        m = r & 127
        v = np.where(s == 1, -1.0, 1.0) * np.ldexp(1.0 + m / 128.0, (off + b - 127).astype(np.int32))
        assert np.array_equal(v, val[~out])
        assert (t.rec[0, out] == 0).all()


# ---------------------------------------------------------------------------------------
# Brute force on tiny channels
# ---------------------------------------------------------------------------------------

def brute_force_window(row):
    best_b, best_c = None, -1
    for b in range(1, 240):
        c = 0
        for v in row:
            f = (int(v) >> 7) & 0xFF
            if b <= f <= b + 15:
                c += 1
        if c > best_c:
            best_b, best_c = b, c
    return best_b, best_c


def brute_force_encode_row(row, b):
    rec, esc = [], []
    for k, v in enumerate(int(x) for x in row):
        f = (v >> 7) & 0xFF
        if b <= f <= b + 15:
            rec.append(((v >> 15) << 11) | ((f - b) << 7) | (v & 0x7F))
        else:
            rec.append(0)
            esc.append((k << 16) | v)
    return rec, esc


@settings(max_examples=200, deadline=None)
@given(st.lists(st.integers(0, 0xFFFF), min_size=1, max_size=40))
def test_window_bruteforce_random_bits(vals):
    w = np.array([vals], dtype=np.uint16)
    b, c = brute_force_window(vals)
    t = O.encode(w)
    assert int(t.base[0]) == b
    assert t.num_escapes == len(vals) - c
    rec, esc = brute_force_encode_row(vals, b)
    assert t.rec[0].tolist() == rec
    assert t.esc.tolist() == esc


@settings(max_examples=150, deadline=None)
@given(st.lists(st.tuples(st.integers(0, 1), st.integers(90, 160), st.integers(0, 127)), min_size=1, max_size=48))
def test_window_bruteforce_clustered(fields):
    vals = [(s << 15) | (e << 7) | m for s, e, m in fields]
    w = np.array([vals], dtype=np.uint16)
    b, c = brute_force_window(vals)
    t = O.encode(w)
    assert int(t.base[0]) == b and t.num_escapes == len(vals) - c
    assert np.array_equal(O.decode(t), w)


def test_window_bruteforce_multirow():
    rng = np.random.default_rng(7)
    w = S.random_bits_matrix(rng, 12, 33, "wide")
    t = O.encode(w)
    for n in range(w.shape[0]):
        b, _ = brute_force_window(w[n].tolist())
        assert int(t.base[n]) == b
        rec, esc = brute_force_encode_row(w[n].tolist(), b)
        assert t.rec[n].tolist() == rec
        lo, hi = int(t.esc_ptr[n]), int(t.esc_ptr[n + 1])
        assert t.esc[lo:hi].tolist() == esc


# ---------------------------------------------------------------------------------------
# Closed forms and invariants
# ---------------------------------------------------------------------------------------

def test_span_at_most_16_closed_form():
    rng = np.random.default_rng(3)
    for _ in range(200):
        lo = int(rng.integers(1, 240))
        span = int(rng.integers(1, 17))
        hi = min(254, lo + span - 1)
        k = int(rng.integers(1, 64))
        e = rng.integers(lo, hi + 1, size=k)
        vals = (rng.integers(0, 2, k) << 15) | (e << 7) | rng.integers(0, 128, k)
        special = rng.random(k) < 0.2
        vals = np.where(special, rng.choice([0x0000, 0x8000, 0x0001, 0x7F80, 0xFFC0], k), vals)
        w = vals.astype(np.uint16)[None, :]
        t = O.encode(w)
        fields = (w[0].astype(np.int32) >> 7) & 0xFF
        normal = (fields >= 1) & (fields <= 254)
        if normal.any():
            assert int(t.base[0]) == max(1, int(fields[normal].max()) - 15)
        assert t.num_escapes == int((~normal).sum())


@pytest.mark.parametrize("kind", ["gauss", "uniform_bits", "wide"])
def test_invariants(kind):
    rng = np.random.default_rng(11)
    w = S.random_bits_matrix(rng, 37, 300, kind)
    t = O.encode(w)
    assert (t.rec < 4096).all()
    c = O.window_counts(O.exponent_histogram(w))
    assert t.num_escapes == int((w.shape[1] - c.max(axis=1)).sum())
    assert int(t.esc_ptr[-1]) == t.num_escapes and (np.diff(t.esc_ptr.astype(np.int64)) >= 0).all()
    for n in range(t.n):
        ks = (t.esc[t.esc_ptr[n]:t.esc_ptr[n + 1]] >> 16).astype(np.int64)
        assert (np.diff(ks) > 0).all()
        assert (t.rec[n, ks] == 0).all()
    assert np.array_equal(O.decode(t), w)


def test_tiny_config_round_trip():
    w = S.tiny_weights(0)
    t = O.encode(w)
    assert np.array_equal(O.decode(t), w)
    fields = (w.astype(np.int32) >> 7) & 0xFF
    esc_mask = np.zeros(w.shape, dtype=bool)
    for n in range(t.n):
        ks = (t.esc[t.esc_ptr[n]:t.esc_ptr[n + 1]] >> 16).astype(np.int64)
        esc_mask[n, ks] = True
    # zeros, denormals and infs (field 0 or 255) are always escapes
    assert esc_mask[(fields == 0) | (fields == 255)].all()
    assert 12.0 < O.bits_per_weight(t.n, t.k, t.num_escapes) < 12.6


def test_bits_per_weight_near_page_figure():
    """Gaussian x lognormal channels give ~12.01 bits/weight, the pages' 12.01-12.02 (S4.1 result)."""
    gen = __import__("torch").Generator().manual_seed(123)
    w = S.layer_matrix(gen, 512, 5120)
    t = O.encode(w)
    bpw = O.bits_per_weight(t.n, t.k, t.num_escapes)
    assert 12.005 < bpw < 12.03, bpw


# ---------------------------------------------------------------------------------------
# GEMM reference pins
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_gemm_reference_vs_fsum(seed):
    rng = np.random.default_rng(seed)
    m, n, k = int(rng.integers(1, 5)), int(rng.integers(1, 7)), int(rng.integers(1, 200))
    x = S.random_bits_matrix(rng, m, k, "wide")
    w = S.random_bits_matrix(rng, n, k, "wide")
    y, a = O.gemm_reference(x, w)
    xf, wf = O.bf16_to_f64(x), O.bf16_to_f64(w)
    for i in range(m):
        for j in range(n):
            prods = [float(xf[i, kk]) * float(wf[j, kk]) for kk in range(k)]
            exact = math.fsum(prods)
            assert abs(y[i, j] - exact) <= k * 2.0 ** -52 * math.fsum(abs(p) for p in prods)
            assert a[i, j] == pytest.approx(math.fsum(abs(p) for p in prods), rel=1e-13, abs=0)


def test_gemm_one_hot_picks_weights():
    rng = np.random.default_rng(5)
    w = S.random_bits_matrix(rng, 9, 40, "wide")
    w[w == 0] = 0x3F80
    ks = [0, 7, 39, 13]
    x = np.zeros((len(ks), 40), dtype=np.uint16)
    for i, kk in enumerate(ks):
        x[i, kk] = 0x3F80  # 1.0
    y, a = O.gemm_reference(x, w)
    for i, kk in enumerate(ks):
        assert np.array_equal(y[i], O.bf16_to_f64(w[:, kk]))
        assert np.array_equal(a[i], np.abs(O.bf16_to_f64(w[:, kk])))


def test_within_tolerance_boundaries():
    y_ref = np.array([[1.0, -2.0, np.inf, -np.inf, np.nan, 0.0]])
    a_ref = np.array([[4096.0, 4096.0, 1.0, 1.0, 1.0, 0.0]])
    good = np.array([[2.0, -1.0, np.inf, -np.inf, np.nan, 0.0]])    # errors exactly 1 = 2^-12 * 4096
    bad = np.array([[2.001, -3.5, -np.inf, np.inf, 1.0, 1e-30]])
    assert O.within_tolerance(good, y_ref, a_ref).all()
    assert not O.within_tolerance(bad, y_ref, a_ref).any()


# ---------------------------------------------------------------------------------------
# The load-time check catches corruption
# ---------------------------------------------------------------------------------------

def test_verify_catches_single_bit_flips():
    w = S.tiny_weights(0)
    t = O.encode(w)
    assert O.verify(t, w) == (0, -1)
    rng = np.random.default_rng(9)
    for _ in range(40):
        n, k = int(rng.integers(0, t.n)), int(rng.integers(0, t.k))
        bit = int(rng.integers(0, 12))
        bad = O.W12Logical(t.n, t.k, t.base.copy(), t.rec.copy(), t.esc_ptr.copy(), t.esc.copy())
        bad.rec[n, k] ^= np.uint16(1 << bit)
        ks = set((t.esc[t.esc_ptr[n]:t.esc_ptr[n + 1]] >> 16).tolist())
        cnt, first = O.verify(bad, w)
        if k in ks:      # a record under an escape is overwritten by the patch
            assert cnt == 0
        else:
            assert (cnt, first) == (1, n * t.k + k)
    # an escape value flip
    bad = O.W12Logical(t.n, t.k, t.base.copy(), t.rec.copy(), t.esc_ptr.copy(), t.esc.copy())
    bad.esc[5] ^= np.uint32(1)
    assert O.verify(bad, w)[0] == 1
    # a base flip corrupts every in-window weight of that channel
    bad = O.W12Logical(t.n, t.k, t.base.copy(), t.rec.copy(), t.esc_ptr.copy(), t.esc.copy())
    bad.base[3] ^= np.uint8(1)
    n_esc = int(t.esc_ptr[4] - t.esc_ptr[3])
    assert O.verify(bad, w)[0] == t.k - n_esc
