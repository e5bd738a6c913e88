"""Planted mistakes in the oracle (on the CPU): each one must be caught by the pins.

A plausible slip anywhere in the oracle (a narrower window, a shifted field, the wrong
tie-break, a transposed GEMM operand, a dropped term) is planted with monkeypatch, and
the pin checks below must reject it.  This shows that the pins constrain the oracle
rather than restate it.
"""
import json
import os

import numpy as np
import pytest

from oracle import w12_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(v):
    """A JSON number, or a string: "inf", "-inf", "nan", or an exact hexadecimal float."""
    if not isinstance(v, str):
        return float(v)
    return float.fromhex(v) if "0x" in v else float(v)


def pins_hold() -> bool:
    """Run a compact set of pins; False if any fails."""
    try:
        for ch in _load("w12_hand_channels.json")["channels"]:
            w = np.array([ch["w"]], dtype=np.uint16)
            t = O.encode(w)
            assert int(t.base[0]) == ch["base"]
            assert t.rec[0].tolist() == ch["rec"]
            assert t.esc.tolist() == ch["esc"]
            assert np.array_equal(O.decode(t), w)
        for case in _load("w12_hand_channels.json")["bits_per_weight_cases"]:
            assert abs(O.bits_per_weight(case["n"], case["k"], case["e"]) - case["bpw"]) < 1e-9
        w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)[None, :]
        t = O.encode(w)
        assert int(t.base[0]) == 1 and t.num_escapes == 61440
        assert np.array_equal(O.decode(t), w)
        for case in _load("w12_hand_gemm.json")["cases"]:
            x = np.array(case["x"], dtype=np.uint16)
            ww = np.array(case["w"], dtype=np.uint16)
            y, a = O.gemm_reference(x, ww)
            exp = np.array([[_num(v) for v in row] for row in case["y"]])
            assert y.shape == exp.shape
            fin = np.isfinite(exp)
            assert np.array_equal(y[fin], exp[fin])
            assert np.array_equal(np.isnan(y), np.isnan(exp))
            if "a" in case:
                assert np.array_equal(a, np.array([[_num(v) for v in row] for row in case["a"]], dtype=np.float64))
        return True
    except (AssertionError, ValueError, IndexError):
        return False


def test_unmutated_oracle_passes():
    assert pins_hold()


def _mut_window15(mp):
    mp.setattr(O, "WINDOW_BINADES", 15)


def _mut_bmax(mp):
    mp.setattr(O, "B_MAX", 238)


def _mut_tie_largest(mp):
    def choose(w):
        c = O.window_counts(O.exponent_histogram(w))
        last = c.shape[1] - 1 - np.argmax(c[:, ::-1], axis=1)
        return (last + O.B_MIN).astype(np.uint8)
    mp.setattr(O, "choose_window", choose)


def _mut_offset_off_by_one(mp):
    orig = O.decode

    def dec(t):
        t2 = O.W12Logical(t.n, t.k, (t.base.astype(np.int32) + 1).astype(np.uint8), t.rec, t.esc_ptr, t.esc)
        return orig(t2)
    mp.setattr(O, "decode", dec)


def _mut_sign_dropped(mp):
    orig = O.sign_field
    mp.setattr(O, "sign_field", lambda w: orig(w) * 0)


def _mut_gemm_transposed(mp):
    orig = O.gemm_reference

    def g(x, w):
        y, a = orig(x, w)
        return y.T, a.T
    mp.setattr(O, "gemm_reference", g)


def _mut_gemm_abs_dropped(mp):
    orig = O.gemm_reference

    def g(x, w):
        y, a = orig(x, w)
        return y, np.abs(y)
    mp.setattr(O, "gemm_reference", g)


def _mut_bpw_no_pointer(mp):
    mp.setattr(O, "bits_per_weight", lambda n, k, e: (1.5 * n * k + n + 4 * e) * 8.0 / (n * k))


def _mut_escape_order(mp):
    orig = O.encode

    def enc(w, forced_base=None):
        t = orig(w, forced_base)
        return O.W12Logical(t.n, t.k, t.base, t.rec, t.esc_ptr, t.esc[::-1].copy())
    mp.setattr(O, "encode", enc)


def _mut_subnormals_flushed(mp):
    orig = O.bf16_to_f64

    def conv(w):
        v = orig(w)
        return np.where((np.asarray(w, np.uint16) & 0x7F80) == 0, 0.0, v)
    mp.setattr(O, "bf16_to_f64", conv)


def _mut_subnormal_implicit_bit(mp):
    orig = O.bf16_to_f64

    def conv(w):
        w = np.asarray(w, np.uint16)
        sub = ((w & 0x7F80) == 0) & ((w & 0x7F) != 0)
        sign = np.where(w & 0x8000, -1.0, 1.0)
        return np.where(sub, sign * (1.0 + (w & 0x7F) / 128.0) * 2.0 ** -126, orig(w))
    mp.setattr(O, "bf16_to_f64", conv)


@pytest.mark.parametrize("mutation", [
    _mut_window15, _mut_bmax, _mut_tie_largest, _mut_offset_off_by_one, _mut_sign_dropped,
    _mut_gemm_transposed, _mut_gemm_abs_dropped, _mut_bpw_no_pointer, _mut_escape_order,
    _mut_subnormals_flushed, _mut_subnormal_implicit_bit,
], ids=lambda f: f.__name__)
def test_planted_mistake_is_caught(monkeypatch, mutation):
    mutation(monkeypatch)
    assert not pins_hold()
