"""W12 reference oracle (CPU, numpy).  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never calls it, and it shares no code, tables or helpers with
that path: it works on the *logical* W12 format only, written out from the
definition so that a reader can check it against the pages by eye.

Sources (SpecPilot, arXiv 2611.02501, as summarised on its web pages):

* [S4.1-method]  summary page, method bullet of section 4.1.  Fixes the record: one
  sign bit, the exponent as a four-bit offset from a base chosen per output channel
  (so one channel's window spans sixteen binades), and the top seven mantissa bits.
  Exponents outside the window, zeros and subnormals are not representable there
  and go to an exact side list.  The GEMM decodes in registers and reduces its K
  split in a fixed order, which makes its result reproducible.
* [S4.1-result]  summary page, result bullet of section 4.1.  Gives the storage cost
  (a little over twelve bits per weight, averaged over eight dense models) and
  states that each decoded tensor is compared with its source bit for bit when it
  is loaded.
* [Article-W12]  news article, part "(1) W12".  Motivates the window (within one
  output channel the BF16 exponents sit close together), gives the same twelve-bit
  split, and says the side list restores the remaining weights exactly, so the
  source tensor comes back unchanged.
* [Article-TLV]  news article, part "(3) two-level verification".  The first of two
  verification passes runs on the eight-bit view contained in each W12 record and
  only proposes a chain of candidate tokens; tokens are accepted by the exact pass.

Readings where the pages are silent (each is also listed in the design notes):

* R1  window choice: the base b of the window [b, b+15] maximises the number of
      in-window weights of the channel (each escape costs a fixed 4 bytes, so this
      also minimises the encoded size);
* R2  ties go to the smallest b;
* R3  b ranges over 1..239, i.e. windows cover normal exponent fields 1..254 only;
      zeros and denormals (field 0) and inf/NaN (field 255) always escape;
* R4  record bit order is sign | offset | mantissa from bit 11 down to bit 0,
      mirroring BF16; offset = exponent field - b;
* R5  the record at an escaped position is 0;
* R6  escape entry = (k << 16) | bf16_bits, per channel in ascending k, channels
      concatenated in order with an (N+1)-entry exclusive prefix-sum pointer;
* R7  bits/weight = (1.5*N*K + N + 4*(N+1) + 4*E) * 8 / (N*K): 12 record bits per
      weight, one base byte per channel, the pointer array and 4 bytes per escape;
* R8  GEMM: Y = X @ W^T with FP32 outputs; the reference is the FP64 sum of the
      exact BF16 x BF16 products, and an output y passes when
      |y - y_ref| <= 2^-12 * sum_k |x_k * w_k|; where y_ref is +-inf, y must be the
      same infinity; where y_ref is NaN, y must be NaN.
* R14 the nested 8-bit view of a record is its top byte, sign | offset | top three
      mantissa bits; read as a weight it is the BF16 value with the four low mantissa
      bits cleared (truncation toward zero);
* R15 in the Q pass escaped weights keep their exact value (the escape list is the
      format's only copy of them); the Q-pass GEMM is the R8 GEMM on the Q-view
      weights, with the same tolerance.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

WINDOW_BINADES = 16          # [S4.1-method]: 16-binade window per output channel
B_MIN, B_MAX = 1, 239        # R3: the window [b, b+15] stays inside fields 1..254
TOL_EXP = -12                # R8: tolerance 2^-12 * sum |x w|


@dataclass
class W12Logical:
    """The logical W12 tensor: the form both sides are compared in."""
    n: int
    k: int
    base: np.ndarray      # uint8 [N]      window base exponent field b_n
    rec: np.ndarray       # uint16 [N, K]  12-bit records (R4), 0 at escapes (R5)
    esc_ptr: np.ndarray   # uint32 [N+1]   exclusive prefix sum of escape counts (R6)
    esc: np.ndarray       # uint32 [E]     (k << 16) | bf16 bits, ascending k per channel (R6)

    @property
    def num_escapes(self) -> int:
        return int(self.esc.shape[0])


# ----------------------------------------------------------------------------------------
# BF16 fields
# ----------------------------------------------------------------------------------------

def sign_field(w: np.ndarray) -> np.ndarray:
    return (w.astype(np.uint16) >> 15) & 0x1


def exponent_field(w: np.ndarray) -> np.ndarray:
    return (w.astype(np.uint16) >> 7) & 0xFF


def mantissa_field(w: np.ndarray) -> np.ndarray:
    return w.astype(np.uint16) & 0x7F


def bf16_to_f64(w: np.ndarray) -> np.ndarray:
    """Exact value of BF16 bit patterns (inf, NaN and denormals included)."""
    u32 = w.astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u32.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------------
# Step 1: per-channel window choice  ([S4.1-method], [Article-W12]; R1-R3)
# ----------------------------------------------------------------------------------------

def exponent_histogram(w: np.ndarray) -> np.ndarray:
    """H[n, e] = number of weights of channel n whose exponent field is e (0..255)."""
    n, k = w.shape
    e = exponent_field(w).astype(np.int64)
    flat = (np.arange(n, dtype=np.int64)[:, None] * 256 + e).reshape(-1)
    return np.bincount(flat, minlength=n * 256).reshape(n, 256)


def window_counts(hist: np.ndarray) -> np.ndarray:
    """c[n, b - 1] = sum_{e=b}^{b+15} H[n, e] for b = 1..239 (in-window weights)."""
    cols = [hist[:, b:b + WINDOW_BINADES].sum(axis=1) for b in range(B_MIN, B_MAX + 1)]
    return np.stack(cols, axis=1)


def choose_window(w: np.ndarray) -> np.ndarray:
    """b_n = the smallest b in 1..239 maximising the in-window count of channel n."""
    c = window_counts(exponent_histogram(w))
    # np.argmax returns the first (smallest-index) maximum: the smallest b (R2)
    return (np.argmax(c, axis=1) + B_MIN).astype(np.uint8)


# ----------------------------------------------------------------------------------------
# Step 2: records and the escape list  ([S4.1-method], [Article-W12]; R4-R6)
# ----------------------------------------------------------------------------------------

def in_window(w: np.ndarray, base: np.ndarray) -> np.ndarray:
    e = exponent_field(w).astype(np.int32)
    b = base.astype(np.int32)[:, None]
    return (e >= b) & (e <= b + WINDOW_BINADES - 1)


def encode(w: np.ndarray, forced_base: np.ndarray | None = None) -> W12Logical:
    """BF16 bits [N, K] -> logical W12.

    ``forced_base`` replaces the window search (a test hook: every b in 1..239 gives
    a lossless encoding, only the escape count changes).
    """
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n, k = w.shape
    base = choose_window(w) if forced_base is None else np.asarray(forced_base, dtype=np.uint8)
    if base.shape != (n,) or base.min(initial=B_MIN) < B_MIN or base.max(initial=B_MIN) > B_MAX:
        raise ValueError("base must hold N values in 1..239")
    inside = in_window(w, base)
    s = sign_field(w)
    off = (exponent_field(w).astype(np.int32) - base.astype(np.int32)[:, None])
    m = mantissa_field(w)
    rec_all = (s.astype(np.uint32) << 11) | (off.astype(np.uint32) << 7) | m.astype(np.uint32)
    rec = np.where(inside, rec_all, 0).astype(np.uint16)          # R5: 0 at escapes
    # escape list: channel-major, ascending k inside each channel (R6)
    rows, cols = np.nonzero(~inside)
    esc = ((cols.astype(np.uint32) << 16) | w[rows, cols].astype(np.uint32)).astype(np.uint32)
    counts = np.bincount(rows, minlength=n).astype(np.uint64)
    esc_ptr = np.zeros(n + 1, dtype=np.uint64)
    esc_ptr[1:] = np.cumsum(counts)
    return W12Logical(n, k, base, rec, esc_ptr.astype(np.uint32), esc)


# ----------------------------------------------------------------------------------------
# Step 3: decode and the load-time bit check  ([S4.1-result], [Article-W12])
# ----------------------------------------------------------------------------------------

def decode(t: W12Logical) -> np.ndarray:
    """Logical W12 -> BF16 bits: records re-biased by the channel base, escapes patched."""
    rec = t.rec.astype(np.uint32)
    s = rec >> 11
    off = (rec >> 7) & 0xF
    m = rec & 0x7F
    e = off + t.base.astype(np.uint32)[:, None]
    out = ((s << 15) | (e << 7) | m).astype(np.uint16)
    for row in range(t.n):
        lo, hi = int(t.esc_ptr[row]), int(t.esc_ptr[row + 1])
        if hi > lo:
            ent = t.esc[lo:hi]
            out[row, (ent >> 16).astype(np.int64)] = (ent & 0xFFFF).astype(np.uint16)
    return out


def verify(t: W12Logical, ref: np.ndarray) -> tuple[int, int]:
    """(mismatch count, first mismatching flat index or -1) of decode(t) against ref."""
    d = decode(t)
    bad = np.flatnonzero(d.reshape(-1) != np.asarray(ref, dtype=np.uint16).reshape(-1))
    return int(bad.size), (int(bad[0]) if bad.size else -1)


def q_view(t: W12Logical) -> np.ndarray:
    """R14/R15: the weights the Q pass reads, as BF16 bits.  In-window positions take the
    record's top byte (sign, offset, three mantissa bits) re-biased by the channel base, with
    the four low mantissa bits zero; escaped positions take their exact escape value."""
    top = (t.rec.astype(np.uint32) >> 4) & 0xFF
    s = top >> 7
    off = (top >> 3) & 0xF
    m3 = top & 0x7
    e = off + t.base.astype(np.uint32)[:, None]
    out = ((s << 15) | (e << 7) | (m3 << 4)).astype(np.uint16)
    for row in range(t.n):
        lo, hi = int(t.esc_ptr[row]), int(t.esc_ptr[row + 1])
        if hi > lo:
            ent = t.esc[lo:hi]
            out[row, (ent >> 16).astype(np.int64)] = (ent & 0xFFFF).astype(np.uint16)
    return out


def bits_per_weight(n: int, k: int, e: int) -> float:
    """R7: stored bits per weight of the logical format."""
    return (1.5 * n * k + n + 4 * (n + 1) + 4 * e) * 8.0 / (n * k)


# ----------------------------------------------------------------------------------------
# Step 4: the GEMM reference  (R8)
# ----------------------------------------------------------------------------------------

def gemm_reference(x: np.ndarray, w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """y[m, n] = sum_k x[m, k] * w[n, k] in FP64, and a[m, n] = sum_k |x[m, k] * w[n, k]|.

    Every BF16 x BF16 product is exact in FP64.  Rows with only finite values use an
    FP64 matrix product (error <= K * 2^-53 * a, negligible next to 2^-12 * a); rows
    holding inf or NaN are summed product by product so IEEE rules (0 * inf = NaN,
    inf - inf = NaN) apply exactly as written.
    """
    xf = bf16_to_f64(np.asarray(x, dtype=np.uint16))
    wf = bf16_to_f64(np.asarray(w, dtype=np.uint16))
    finite_rows = np.isfinite(wf).all(axis=1)
    x_finite = bool(np.isfinite(xf).all())
    y = np.empty((xf.shape[0], wf.shape[0]), dtype=np.float64)
    a = np.empty_like(y)
    sel = finite_rows if x_finite else np.zeros_like(finite_rows)
    if sel.any():
        y[:, sel] = xf @ wf[sel].T
        a[:, sel] = np.abs(xf) @ np.abs(wf[sel]).T
    rest = np.flatnonzero(~sel)
    with np.errstate(invalid="ignore", over="ignore"):
        for n in rest:
            p = xf * wf[n][None, :]
            y[:, n] = p.sum(axis=1)
            a[:, n] = np.abs(p).sum(axis=1)
    return y, a


def within_tolerance(y: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray) -> np.ndarray:
    """Elementwise R8 acceptance mask for an FP32 result y."""
    y = np.asarray(y, dtype=np.float64)
    ok = np.zeros(y_ref.shape, dtype=bool)
    fin = np.isfinite(y_ref)
    with np.errstate(invalid="ignore"):
        ok[fin] = np.isfinite(y[fin]) & (np.abs(y[fin] - y_ref[fin]) <= np.ldexp(a_ref[fin], TOL_EXP))
    nan = np.isnan(y_ref)
    ok[nan] = np.isnan(y[nan])
    inf = np.isinf(y_ref)
    ok[inf] = y[inf] == y_ref[inf]
    return ok


def gemm_check(x: np.ndarray, w: np.ndarray, y: np.ndarray) -> tuple[int, float]:
    """(number of failing outputs, worst |y - y_ref| / a_ref over finite outputs)."""
    y_ref, a_ref = gemm_reference(x, w)
    ok = within_tolerance(y, y_ref, a_ref)
    fin = np.isfinite(y_ref) & (a_ref > 0)
    worst = float(np.max(np.abs(np.asarray(y, np.float64)[fin] - y_ref[fin]) / a_ref[fin])) if fin.any() else 0.0
    return int((~ok).sum()), worst


def gemm_q_check(x: np.ndarray, t: W12Logical, y: np.ndarray, rows=None) -> tuple[int, float]:
    """R15: the Q-pass GEMM checked as the R8 GEMM on the Q-view weights (optionally on a
    subset of output channels: y then holds only those columns)."""
    wq = q_view(t)
    if rows is not None:
        wq = wq[np.asarray(rows)]
    return gemm_check(x, wq, y)
