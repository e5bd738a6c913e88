"""Pins for the oracle's Q-pass view (the nested 8-bit weights, R14/R15) and its GEMM.

The view is pinned by what defines it, not by re-typing it: a hand fixture, a numeric
characterisation of truncation toward zero to four significant bits (checked with float
arithmetic over all 65536 BF16 patterns in one channel), escapes kept exact, and the
Q-pass GEMM reference against a brute-force sum of values built from their fields with
math.ldexp.  Planted slips (rounding instead of truncation, escapes dropped, a shifted
mantissa) must fail these pins.  No GPU is touched.
"""
import math

import numpy as np
import pytest

from oracle import w12_oracle as O


def all_patterns_channel():
    return np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)[None, :]


def _value(bits: int) -> float:
    """A BF16 value from its fields (normal or zero/denormal), independent of the oracle."""
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        v = math.ldexp(m / 128.0, -126)
    elif e == 255:
        v = math.inf if m == 0 else math.nan
    else:
        v = math.ldexp(1.0 + m / 128.0, e - 127)
    return -v if s else v


# hand fixture: one channel, window chosen by the bulk (fields 125..128 -> base 128 - 15 = 113)
#   0x3F80 = 1.0        -> 1.0          (mantissa 0000000: nothing to clear)
#   0x3FFF = 1.9921875  -> 1.875        (mantissa 1111111 -> 1110000: 1 + 7/8)
#   0xBF8F = -1.1171875 -> -1.0         (mantissa 0001111 -> 0000000)
#   0x4049 = 3.140625   -> 3.0          (mantissa 1001001 -> 1000000: 2 * (1 + 4/8))
#   0x3E80 = 0.25       -> 0.25
#   0x0000 = +0         -> +0 (escape, exact)
#   0x0005 = denormal   -> 0x0005 (escape, exact: not truncated)
#   0x7FC1 = NaN        -> 0x7FC1 (escape, exact: clearing its low bits would change it)
HAND_W = [0x3F80, 0x3FFF, 0xBF8F, 0x4049, 0x3E80, 0x0000, 0x0005, 0x7FC1]
HAND_Q = [0x3F80, 0x3FF0, 0xBF80, 0x4040, 0x3E80, 0x0000, 0x0005, 0x7FC1]
HAND_QV = [1.0, 1.875, -1.0, 3.0, 0.25, 0.0]


def q_pins_hold() -> bool:
    try:
        t = O.encode(np.array([HAND_W], dtype=np.uint16))
        q = O.q_view(t)[0]
        assert q.tolist() == HAND_Q
        assert [_value(int(v)) for v in q[:6]] == HAND_QV
        # every pattern in one channel: truncation toward zero to four significant bits for
        # in-window weights (checked numerically), exact values for escapes
        w = all_patterns_channel()
        t = O.encode(w)
        q = O.q_view(t)[0]
        esc_pos = set((t.esc >> 16).tolist())
        b = int(t.base[0])
        for i in range(1 << 16):
            wi, qi = int(w[0, i]), int(q[i])
            if i in esc_pos:
                assert qi == wi
                continue
            e = (wi >> 7) & 0xFF
            assert b <= e <= b + 15
            vw, vq = _value(wi), _value(qi)
            assert (qi >> 15) == (wi >> 15)                      # same sign
            assert abs(vq) <= abs(vw)                             # toward zero
            assert abs(vw) - abs(vq) < math.ldexp(1.0, e - 127 - 3)   # within one 4-bit step
            assert ((qi >> 7) & 0xFF) == e                        # same binade
            assert (abs(vq) / math.ldexp(1.0, e - 127) * 8.0).is_integer()   # 4 significant bits
        # the Q-pass GEMM reference equals a brute-force FP64 sum of field-built values
        rng = np.random.default_rng(5)
        wsm = rng.integers(0x3C00, 0x4100, size=(3, 40)).astype(np.uint16)
        wsm[0, 3] = 0
        wsm[2, 7] = 0x5F00   # far above the bulk: an escape
        x = rng.integers(0x3E00, 0x4000, size=(2, 40)).astype(np.uint16)
        ts = O.encode(wsm)
        qs = O.q_view(ts)
        y, a = O.gemm_reference(x, qs)
        for m in range(2):
            for n in range(3):
                ref = math.fsum(_value(int(x[m, k])) * _value(int(qs[n, k])) for k in range(40))
                assert abs(y[m, n] - ref) <= 1e-12 * max(1.0, a[m, n])
        assert int(qs[2, 7]) == 0x5F00
        return True
    except (AssertionError, ValueError, IndexError):
        return False


def test_q_view_pins():
    assert q_pins_hold()


def test_q_gemm_check_uses_q_view():
    """gemm_q_check accepts the Q-view product and rejects the exact-weight product where
    the two differ by more than the tolerance."""
    rng = np.random.default_rng(11)
    w = rng.integers(0x3F80, 0x4000, size=(4, 64)).astype(np.uint16) | 0x000F   # low bits set
    t = O.encode(w)
    x = np.full((1, 64), 0x3F80, dtype=np.uint16)   # all ones: y = row sums
    yq, _ = O.gemm_reference(x, O.q_view(t))
    ye, _ = O.gemm_reference(x, w)
    assert O.gemm_q_check(x, t, yq.astype(np.float32))[0] == 0
    assert O.gemm_q_check(x, t, ye.astype(np.float32))[0] > 0
    rows = [1, 3]
    assert O.gemm_q_check(x, t, yq[:, rows].astype(np.float32), rows=rows)[0] == 0


def _mut_round(mp):
    real = O.q_view

    def rounded(t):
        q = real(t).astype(np.uint32)
        d = O.decode(t).astype(np.uint32)
        inwin = q != d
        q = np.where(inwin & ((d & 0xF) >= 8), q + 0x10, q)   # round half up instead of truncating
        return q.astype(np.uint16)
    mp.setattr(O, "q_view", rounded)


def _mut_drop_escapes(mp):
    def no_esc(t):
        top = (t.rec.astype(np.uint32) >> 4) & 0xFF
        e = ((top >> 3) & 0xF) + t.base.astype(np.uint32)[:, None]
        return (((top >> 7) << 15) | (e << 7) | ((top & 7) << 4)).astype(np.uint16)
    mp.setattr(O, "q_view", no_esc)


def _mut_shift(mp):
    real = O.q_view

    def shifted(t):
        q = real(t).astype(np.uint32)
        d = O.decode(t).astype(np.uint32)
        inwin = q != d
        return np.where(inwin, (q & 0xFF80) | ((q & 0x70) >> 1), q).astype(np.uint16)   # m3 one bit low
    mp.setattr(O, "q_view", shifted)


@pytest.mark.parametrize("mutate", [_mut_round, _mut_drop_escapes, _mut_shift])
def test_planted_q_slips_are_caught(monkeypatch, mutate):
    mutate(monkeypatch)
    assert not q_pins_hold()
