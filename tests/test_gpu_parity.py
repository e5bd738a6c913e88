"""GPU parity on small and ragged inputs: the HIP path against the CPU oracle.

Encode: window bases, logical records (via w12_unpack_records), escape pointers and escape
list bit-identical.  Verify: zero mismatches on the source, exact counts on corrupted
copies.  Decode: bit-identical.  GEMM: every output within 2^-12 * sum|x w| of the FP64
reference, bitwise identical over repeated runs, nothing written outside Y.
"""
import numpy as np
import pytest
import torch

import lossless_bit_weight_encode_amd as w12
import w12_synth as S
from oracle import w12_oracle as O
from gpu_util import assert_encode_equal, say, to_dev, u16, u32

pytestmark = pytest.mark.gpu


def _exhaustive(shuffle):
    w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if shuffle:
        w = w[np.random.default_rng(0).permutation(w.size)]
    return w[None, :]


def _fields(seed, n, k, lo, hi, zero_frac=0.0, special_frac=0.0):
    """BF16 bit patterns with exponent fields drawn uniformly from lo..hi, random sign and
    mantissa; a fraction set to +-0 and a fraction to inf/NaN (field 255)."""
    rng = np.random.default_rng(seed)
    e = rng.integers(lo, hi + 1, size=(n, k)).astype(np.uint16)
    w = (rng.integers(0, 2, size=(n, k)).astype(np.uint16) << 15) | (e << 7) | rng.integers(0, 128, size=(n, k)).astype(np.uint16)
    u = rng.random((n, k))
    w[u < zero_frac] &= 0x8000
    w[(u >= zero_frac) & (u < zero_frac + special_frac)] |= 0x7F80
    return w


def _bimodal(seed, n, k, gap):
    """Half the weights of each row around field 100, half around field 100 + gap."""
    w = _fields(seed, n, k, 98, 102)
    hi = _fields(seed + 1, n, k, 98 + gap, 102 + gap)
    pick = np.random.default_rng(seed + 2).random((n, k)) < 0.5
    return np.where(pick, hi, w).astype(np.uint16)


def _outliers_first(seed, n, k):
    """Gaussian rows whose first 512 weights are 80 binades above the rest."""
    w = S.layer_matrix(torch.Generator().manual_seed(seed), n, k)
    w[:, :512] = _fields(seed, n, 512, 200, 205)
    return w


CASES = {
    "tiny_256x512": lambda: S.tiny_weights(0),
    # exponent counts: bulk at the top or bottom of the field range, zeros, inf/NaN, two modes
    # further apart than a window, outliers where each channel is first read, short rows
    "top_fields_48x4100": lambda: _fields(11, 48, 4100, 238, 254, special_frac=0.05),
    "bottom_fields_48x4100": lambda: _fields(12, 48, 4100, 1, 20, zero_frac=0.2),
    "half_zeros_32x5000": lambda: _fields(13, 32, 5000, 110, 125, zero_frac=0.5),
    "bimodal_32x5120": lambda: _bimodal(14, 32, 5120, 25),
    "bimodal_close_32x5120": lambda: _bimodal(15, 32, 5120, 13),
    "outliers_first_16x4096": lambda: _outliers_first(16, 16, 4096),
    "short_9x7": lambda: _fields(17, 9, 7, 100, 130, zero_frac=0.1),
    "multi_batch_5x8197": lambda: _fields(18, 5, 8197, 90, 140, zero_frac=0.01, special_frac=0.01),
    "exhaustive_1x65536": lambda: _exhaustive(False),
    "exhaustive_shuffled_1x65536": lambda: _exhaustive(True),
    "wide_37x1000": lambda: S.random_bits_matrix(np.random.default_rng(1), 37, 1000, "wide"),
    "gauss_300x4096": lambda: S.layer_matrix(torch.Generator().manual_seed(5), 300, 4096),
    "uniform_bits_100x520": lambda: S.random_bits_matrix(np.random.default_rng(2), 100, 520, "uniform_bits"),
    "ragged_17x33": lambda: S.random_bits_matrix(np.random.default_rng(3), 17, 33, "wide"),
    "single_1x16": lambda: S.random_bits_matrix(np.random.default_rng(4), 1, 16, "wide"),
    "heavy_64x2048": lambda: S.heavy_tail_weights(1000, 64, 2048),
    "all_escapes_20x96": lambda: np.zeros((20, 96), dtype=np.uint16),
    # more channels than one pass of the escape-count scan keeps in registers
    "tall_100003x16": lambda: S.random_bits_matrix(np.random.default_rng(6), 100003, 16, "wide"),
    # channel counts at the escape-count scan's chunk boundaries (32768 counts per chunk)
    "scan_edge_32767x24": lambda: S.random_bits_matrix(np.random.default_rng(21), 32767, 24, "wide"),
    "scan_edge_32768x24": lambda: S.random_bits_matrix(np.random.default_rng(22), 32768, 24, "wide"),
    "scan_edge_32769x24": lambda: S.random_bits_matrix(np.random.default_rng(23), 32769, 24, "wide"),
    "scan_edge_65537x8": lambda: S.random_bits_matrix(np.random.default_rng(24), 65537, 8, "wide"),
    # every weight in [1, 2): one binade, no escape at all (E = 0, no escape array)
    "no_escapes_64x512": lambda: S.to_bf16_bits(1.0 + torch.rand(64, 512, generator=torch.Generator().manual_seed(8))),
}

_cache = {}


def case(name):
    if name not in _cache:
        w = CASES[name]()
        _cache[name] = (w, O.encode(w))
    return _cache[name]


def dev_weights(w):
    k = w.shape[1]
    ld = (k + 7) // 8 * 8
    return to_dev(w, ld)


@pytest.mark.parametrize("name", list(CASES))
def test_encode_matches_oracle(name):
    w, ref = case(name)
    t = w12.encode(dev_weights(w))
    assert_encode_equal(t, ref)
    assert t.bits_per_weight() == pytest.approx(O.bits_per_weight(ref.n, ref.k, ref.num_escapes), rel=1e-15)


@pytest.mark.parametrize("name", list(CASES))
def test_verify_and_decode_bit_exact(name):
    w, _ = case(name)
    wd = dev_weights(w)
    t = w12.encode(wd)
    assert w12.verify(t, wd) == (0, -1)
    out = w12.decode(t)
    assert np.array_equal(u16(out), w)


@pytest.mark.parametrize("b", [1, 2, 17, 64, 112, 127, 200, 238, 239])
def test_forced_window_matches_oracle(b):
    w = _exhaustive(True)
    ref = O.encode(w, forced_base=np.array([b], dtype=np.uint8))
    wd = to_dev(w)
    base, hi, lo, esc_ptr = w12.alloc_planes(1, w.shape[1], wd.device)
    forced = torch.tensor([b], dtype=torch.uint8, device="cuda")
    w12.encode_count(wd, base, esc_ptr, forced)
    e = int(esc_ptr[1].item())
    t = w12.W12Tensor(1, w.shape[1], base, hi, lo, esc_ptr, torch.empty(e, dtype=torch.int32, device="cuda"))
    w12.encode_emit(wd, t)
    assert_encode_equal(t, ref)
    assert w12.verify(t, wd) == (0, -1)


def test_verify_reports_corruption():
    w, ref = case("tiny_256x512")
    wd = to_dev(w)
    t = w12.encode(wd)
    rng = np.random.default_rng(0)
    esc_pos = set()
    for n in range(ref.n):
        for e in ref.esc[ref.esc_ptr[n]:ref.esc_ptr[n + 1]]:
            esc_pos.add((n, int(e) >> 16))
    # 1) flip one bit of a hi byte at an in-window position
    hi0 = t.hi.clone()
    for _ in range(5):
        while True:
            n, k = int(rng.integers(0, ref.n)), int(rng.integers(0, ref.k))
            if (n, k) not in esc_pos:
                break
        off = (((n // 16) * ((ref.k + 15) // 16) + k // 16) * 16 + n % 16) * 16 + k % 16
        t.hi.copy_(hi0)
        t.hi[off] ^= 1 << int(rng.integers(0, 8))
        assert w12.verify(t, wd) == (1, n * ref.k + k)
    t.hi.copy_(hi0)
    assert w12.verify(t, wd) == (0, -1)
    # 2) flip a bit of an escape value
    esc0 = t.esc.clone()
    i = 17
    n = int(np.searchsorted(ref.esc_ptr, i, side="right") - 1)
    k = int(ref.esc[i]) >> 16
    t.esc[i] ^= 1
    assert w12.verify(t, wd) == (1, n * ref.k + k)
    t.esc.copy_(esc0)
    # 3) two escapes of a channel out of order: structural defect (and values land wrongly)
    n = int(np.argmax(np.diff(ref.esc_ptr.astype(np.int64)) >= 2))
    a = int(ref.esc_ptr[n])
    t.esc[a], t.esc[a + 1] = esc0[a + 1].clone(), esc0[a].clone()
    cnt, _ = w12.verify(t, wd)
    assert cnt >= 1
    t.esc.copy_(esc0)
    # 4) pointer total inconsistent with num_escapes
    p0 = t.esc_ptr.clone()
    t.esc_ptr[ref.n] -= 1
    cnt, _ = w12.verify(t, wd)
    assert cnt >= 1
    t.esc_ptr.copy_(p0)
    # 5) a window base off by one corrupts the channel's in-window weights
    t.base[3] ^= 1
    cnt, first = w12.verify(t, wd)
    n_esc = int(ref.esc_ptr[4] - ref.esc_ptr[3])
    assert cnt == ref.k - n_esc
    assert first // ref.k == 3
    t.base[3] ^= 1
    assert w12.verify(t, wd) == (0, -1)


# ---------------------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------------------

GEMM_SHAPES = ["tiny_256x512", "wide_37x1000", "gauss_300x4096", "uniform_bits_100x520", "ragged_17x33",
               "single_1x16", "heavy_64x2048", "all_escapes_20x96", "no_escapes_64x512"]
GEMM_M = [1, 2, 3, 5, 8, 9, 16, 17, 24, 32, 33, 48, 63, 64, 65, 100, 128]


RAW_BITS = "uniform_bits_100x520"   # every 16-bit pattern: NaN, inf and values near the FP32 limit


def check_raw_bits(x, w, y):
    """GEMM check for matrices of raw random bit patterns.  The FP64 reference never overflows,
    FP32 can: a product of two BF16 values near 2^127 is beyond the FP32 range.  So the outputs
    compared are the ones the reference fixes for FP32 too: NaN outputs (a NaN weight, or
    infinite products of both signs: NaN in any summation order, whatever overflows beside
    them) and outputs whose finite products sum in magnitude below 2^127 (then no FP32 product
    or partial sum overflows, and NaN / inf / the tolerance apply as for ordinary weights).
    Returns the number of outputs compared."""
    y_ref, a_ref = O.gemm_reference(x, w)
    w_fin = np.where((w & 0x7F80) == 0x7F80, np.uint16(0), w)   # inf and NaN patterns dropped
    _, a_fin = O.gemm_reference(x, w_fin)
    mask = np.isnan(y_ref) | (a_fin < 2.0 ** 127)
    ok = O.within_tolerance(y, y_ref, a_ref)
    bad = int((mask & ~ok).sum())
    assert bad == 0, f"{bad} of {int(mask.sum())} compared outputs differ from the reference"
    return int(mask.sum())


def test_raw_bits_check_compares_outputs():
    """The raw-bit GEMM case is not vacuous: most outputs are compared, NaN ones and finite
    overflow-free ones among them."""
    w, _ = case(RAW_BITS)
    x = S.activations(4, w.shape[1], 17)
    y_ref, _ = O.gemm_reference(x, w)
    with np.errstate(over="ignore"):
        y32 = y_ref.astype(np.float32)   # the reference rounded to FP32: overflowing outputs become inf
    n = check_raw_bits(x, w, y32)
    assert n >= y_ref.size // 2
    w_fin = np.where((w & 0x7F80) == 0x7F80, np.uint16(0), w)
    _, a_fin = O.gemm_reference(x, w_fin)
    assert np.isnan(y_ref).any() and (np.isfinite(y_ref) & (a_fin < 2.0 ** 127)).any()


def run_gemm_check(name, m, seed=0):
    w, _ = case(name)
    n, k = w.shape
    x = S.activations(m, k, 500 + seed + m)
    ld = (k + 7) // 8 * 8
    t = w12.encode(dev_weights(w))
    y = w12.gemm(to_dev(x, ld), t)
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    if name == RAW_BITS:
        check_raw_bits(x, w, yh)
        return 0.0
    bad, worst = O.gemm_check(x, w, yh)
    assert bad == 0, f"{bad} outputs outside tolerance (worst rel {worst:.3g})"
    return worst


@pytest.mark.parametrize("name", GEMM_SHAPES)
@pytest.mark.parametrize("m", GEMM_M)
def test_gemm_within_tolerance(name, m):
    run_gemm_check(name, m)


@pytest.mark.parametrize("name", GEMM_SHAPES)
@pytest.mark.parametrize("limit,ms", [(8, [3, 4, 5, 6, 7, 8]), (0, [1, 2])])
def test_gemm_other_path_within_tolerance(monkeypatch, name, limit, ms):
    """Both inner products serve every M <= 8: the wavefront GEMV at M = 3..8 and the MFMA
    tiles at M = 1, 2, selected with W12_GEMV_MAX_M."""
    monkeypatch.setenv("W12_GEMV_MAX_M", str(limit))
    w, _ = case(name)
    for m in ms:
        assert w12.gemm_plan(m, *w.shape)["path"] == (1 if limit else 2)
        run_gemm_check(name, m, seed=1000)


@pytest.mark.parametrize("name", GEMM_SHAPES)
def test_gemm_wide_tiles_every_m(monkeypatch, name):
    """The wide tiles serve any M (W12_WIDE_MIN_M = 3): 128-row tiles mostly padding at small M,
    256-row tiles above 128, several m tiles above 256."""
    monkeypatch.setenv("W12_WIDE_MIN_M", "3")
    w, _ = case(name)
    for m in (3, 16, 40, 64, 129, 300):
        assert w12.gemm_plan(m, *w.shape)["path"] == 3
        run_gemm_check(name, m, seed=2000)


@pytest.mark.parametrize("m", [65, 128, 256])
def test_gemm_wide_matches_streaming(monkeypatch, m):
    """Wide tiles and 64-row streaming tiles give the same Y up to the FP32 summation order."""
    w, _ = case("gauss_300x4096")
    n, k = w.shape
    t = w12.encode(dev_weights(w))
    x = S.activations(m, k, 4000 + m)
    xd = to_dev(x)
    ys = {}
    for limit in (m, 100000):
        monkeypatch.setenv("W12_WIDE_MIN_M", str(limit))
        ys[limit] = w12.gemm(xd, t).cpu().numpy()
    bad, _ = O.gemm_check(x, w, ys[m])
    assert bad == 0
    bad, _ = O.gemm_check(x, w, ys[100000])
    assert bad == 0
    _, a_ref = O.gemm_reference(x, w)   # sum |x w| per output: each side is within 2^-12 of it
    assert (np.abs(ys[m].astype(np.float64) - ys[100000]) <= 2.0 ** -11 * a_ref).all()


# ---------------------------------------------------------------------------------------
# GEMM, Q pass (nested 8-bit view: hi plane only, escapes exact)
# ---------------------------------------------------------------------------------------

QPASS_M = [1, 2, 3, 16, 24, 33, 64, 100, 256]


@pytest.mark.parametrize("name", GEMM_SHAPES)
@pytest.mark.parametrize("m", QPASS_M)
def test_gemm_qpass_within_tolerance(name, m):
    w, _ = case(name)
    n, k = w.shape
    x = S.activations(m, k, 700 + m)
    ld = (k + 7) // 8 * 8
    t = w12.encode(dev_weights(w))
    y = w12.gemm(to_dev(x, ld), t, qpass=True)
    torch.cuda.synchronize()
    if name == RAW_BITS:
        check_raw_bits(x, O.q_view(O.encode(w)), y.cpu().numpy())
        return
    bad, worst = O.gemm_q_check(x, O.encode(w), y.cpu().numpy())
    assert bad == 0, f"{bad} outputs outside tolerance of the Q-view product (worst rel {worst:.3g})"


@pytest.mark.parametrize("m", [1, 16, 32])
def test_gemm_qpass_bitwise_deterministic_and_differs_from_exact(m):
    """Q pass: bitwise repeatable, counters back at zero, and a different product from the
    exact pass (the weights have low mantissa bits set)."""
    w, _ = case("gauss_300x4096")
    n, k = w.shape
    t = w12.encode(dev_weights(w))
    x = to_dev(S.activations(m, k, 88 + m))
    plan = w12.gemm_plan(m, n, k)
    ws = w12.gemm_workspace(m, n, k)
    cb = plan["counter_bytes"]
    outs = []
    for _ in range(10):
        ws[cb:].view(torch.float32).fill_(float("nan"))
        outs.append(w12.gemm(x, t, ws=ws, qpass=True).cpu().numpy().view(np.uint32))
        assert (ws[:cb].cpu().numpy() == 0).all()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    exact = w12.gemm(x, t, ws=ws).cpu().numpy().view(np.uint32)
    assert not np.array_equal(exact, outs[0])


@pytest.mark.parametrize("m", [1, 4, 8, 16, 32, 64, 100])
def test_gemm_bitwise_deterministic(m):
    """20 runs bitwise identical; the partial region of the workspace is NaN-poisoned before
    every run so a read of a partial that was never written would show."""
    w, _ = case("gauss_300x4096")
    n, k = w.shape
    t = w12.encode(dev_weights(w))
    x = to_dev(S.activations(m, k, 77 + m))
    plan = w12.gemm_plan(m, n, k)
    assert plan["splits"] > 1, "the determinism test must exercise split-K"
    ws = w12.gemm_workspace(m, n, k)
    cb = plan["counter_bytes"]
    outs = []
    for i in range(20):
        ws[cb:].view(torch.float32).fill_(float("nan"))
        outs.append(w12.gemm(x, t, ws=ws).cpu().numpy().view(np.uint32))
        assert (ws[:cb].cpu().numpy() == 0).all(), "arrival counters must return to zero"
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    bad, _ = O.gemm_check(S.activations(m, k, 77 + m), w, outs[0].view(np.float32))
    assert bad == 0


@pytest.mark.parametrize("name,m,grid", [("gauss_300x4096", 1, 4), ("gauss_300x4096", 16, 3),
                                         ("heavy_64x2048", 100, 1), ("wide_37x1000", 100, 1),
                                         ("tiny_256x512", 64, 3), ("ragged_17x33", 70, 1),
                                         # grids that are not a multiple of the 8 XCDs: the logical
                                         # work-group order has full rounds and a remainder
                                         ("gauss_300x4096", 16, 13), ("gauss_300x4096", 2, 37),
                                         ("heavy_64x2048", 32, 7)])
def test_gemm_small_grid(monkeypatch, name, m, grid):
    """More tiles than work-groups (the grid capped with W12_MAX_GRID): work-group ranges span
    several tiles, with partial first and last segments and whole tiles between them.  Y is
    bitwise identical from run to run and within tolerance, and the arrival counters are back
    at zero after each call."""
    monkeypatch.setenv("W12_MAX_GRID", str(grid))
    w, _ = case(name)
    n, k = w.shape
    plan = w12.gemm_plan(m, n, k)
    assert plan["grid"] <= grid
    t = w12.encode(dev_weights(w))
    x = S.activations(m, k, 900 + m)
    ld = (k + 7) // 8 * 8
    xd = to_dev(x, ld)
    ws = w12.gemm_workspace(m, n, k)
    cb = plan["counter_bytes"]
    outs = []
    for _ in range(8):
        ws[cb:].view(torch.uint8).fill_(0xFF)   # NaN partials: a read of an unwritten slot shows
        outs.append(w12.gemm(xd, t, ws=ws).cpu().numpy().view(np.uint32))
        assert (ws[:cb].cpu().numpy() == 0).all(), "arrival counters must return to zero"
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    bad, worst = O.gemm_check(x, w, outs[0].view(np.float32))
    assert bad == 0, f"{bad} outputs outside tolerance (worst rel {worst:.3g})"


def test_gemm_workspace_reused_across_shapes():
    """One workspace, sized for the largest call, serves calls of different shapes in turn."""
    w, _ = case("gauss_300x4096")
    n, k = w.shape
    t = w12.encode(dev_weights(w))
    need = max(w12.gemm_workspace_size(m, n, k) for m in (1, 16, 100))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    w12.gemm_workspace_init(ws)
    for m in (16, 1, 100, 16, 3):
        x = S.activations(m, k, 300 + m)
        y = w12.gemm(to_dev(x), t, ws=ws).cpu().numpy()
        bad, _ = O.gemm_check(x, w, y)
        assert bad == 0


@pytest.mark.parametrize("m", [3, 24])
def test_gemm_writes_only_y(m):
    w, _ = case("wide_37x1000")
    n, k = w.shape
    t = w12.encode(dev_weights(w))
    x = to_dev(S.activations(m, k, 9), 1000)
    canary = -12345.678
    buf = torch.full((m + 3, n + 11), canary, dtype=torch.float32, device="cuda")
    y = buf[:m, :n]
    w12.gemm(x, t, y=y)
    b = buf.cpu().numpy()
    assert (b[:m, n:] == np.float32(canary)).all()
    assert (b[m:, :] == np.float32(canary)).all()
    bad, _ = O.gemm_check(S.activations(m, k, 9), w, b[:m, :n])
    assert bad == 0


@pytest.mark.parametrize("m", [1, 2, 16, 40, 100])
def test_gemm_max_k(m):
    """K = 65536 (the largest K: escape entries keep k in 16 bits), where a lane's serial chain of
    products is longest."""
    w = S.layer_matrix(torch.Generator().manual_seed(21), 40, 65536)
    x = S.activations(m, 65536, 700 + m)
    t = w12.encode(to_dev(w))
    y = w12.gemm(to_dev(x), t).cpu().numpy()
    bad, worst = O.gemm_check(x, w, y)
    assert bad == 0, f"{bad} outputs outside tolerance (worst rel {worst:.3g})"


@pytest.mark.parametrize("m", [1025, 4096])
def test_gemm_large_m(m):
    """Many m tiles of the wide kernel, up to the largest M the library accepts."""
    w, _ = case("heavy_64x2048")
    x = S.activations(m, w.shape[1], 800 + m)
    t = w12.encode(dev_weights(w))
    y = w12.gemm(to_dev(x), t).cpu().numpy()
    bad, worst = O.gemm_check(x, w, y)
    assert bad == 0, f"{bad} outputs outside tolerance (worst rel {worst:.3g})"



def test_verify_reports_corruption_escape_dense():
    """The structural check on an escape-dense tensor, where it walks each channel's list with
    64 lanes (entry i against entry i - 1): an entry moved past K and two entries swapped are
    both reported, with the first differing position where an escape went missing."""
    w, ref = case("all_escapes_20x96")
    wd = to_dev(w, 96)
    t = w12.encode(wd)
    assert w12.verify(t, wd) == (0, -1)
    esc0 = t.esc.clone()
    n = 10
    a, b = int(ref.esc_ptr[n]), int(ref.esc_ptr[n + 1])
    assert b - a > 70, "the channel must hold more entries than one round of its 64 lanes"
    i = a + 65   # the second entry of the second round of lanes
    k_orig = int(ref.esc[i]) >> 16
    t.esc[i] = int(((ref.k + 5) << 16) | (int(ref.esc[i]) & 0xFFFF))   # k past K
    cnt, first = w12.verify(t, wd)
    assert cnt >= 2 and first == n * ref.k + k_orig
    t.esc.copy_(esc0)
    t.esc[a + 64], t.esc[a + 65] = esc0[a + 65].clone(), esc0[a + 64].clone()   # out of order
    cnt, _ = w12.verify(t, wd)
    assert cnt >= 1
    t.esc.copy_(esc0)
    assert w12.verify(t, wd) == (0, -1)

def test_side_stream_encode_verify_gemm():
    """Every binding call on a non-default stream: encode (its read-back of the escape count),
    verify (its read-back of the result) and the GEMM with its own workspace all run on that
    stream and give the same results as on the default stream.  A long kernel queued on the
    default stream first would expose a read-back taken on the wrong stream."""
    w, _ = case("gauss_300x4096")
    n, k = w.shape
    wd = dev_weights(w)
    x = to_dev(S.activations(16, k, 4242))
    t_ref = w12.encode(wd)
    y_ref = w12.gemm(x, t_ref)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    # keep the default stream busy, so work that wrongly lands there would be visibly late
    busy = torch.empty(1 << 26, dtype=torch.float32, device="cuda")
    for _ in range(20):
        busy.mul_(1.0001)
    t = w12.encode(wd, stream=s)
    assert t.num_escapes == t_ref.num_escapes
    assert w12.verify(t, wd, stream=s) == (0, -1)
    y = w12.gemm(x, t, stream=s)
    s.synchronize()
    assert torch.equal(y, y_ref)
    for name in ("base", "hi", "lo", "esc_ptr", "esc"):
        assert torch.equal(getattr(t, name), getattr(t_ref, name)), name
    torch.cuda.synchronize()


def test_encode_many_matches_encode():
    """encode_many (one read-back of the escape counts for several matrices) gives, tensor for
    tensor, exactly what encode gives for each alone, also on a side stream, and an empty list
    gives an empty list."""
    names = ["gauss_300x4096", "ragged_17x33", "all_escapes_20x96", "no_escapes_64x512", "heavy_64x2048"]
    ws = [dev_weights(case(nm)[0]) for nm in names]
    refs = [w12.encode(w) for w in ws]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    for stream in (None, s):
        got = w12.encode_many(ws, stream=stream)
        if stream is not None:
            stream.synchronize()
        assert len(got) == len(refs)
        for nm, t, r in zip(names, got, refs):
            assert (t.n, t.k, t.num_escapes) == (r.n, r.k, r.num_escapes), nm
            for field in ("base", "hi", "lo", "esc_ptr", "esc"):
                assert torch.equal(getattr(t, field), getattr(r, field)), (nm, field)
        for nm, t in zip(names, got):
            assert_encode_equal(t, case(nm)[1])
    assert w12.encode_many([]) == []


# ---------------------------------------------------------------------------------------
# Escape-dense tensors: more escapes per 64-channel tile than its LDS slice holds, on average.
# The 16-row MFMA tiles and the GEMV (M <= 4) run an instantiation of their own for them that
# keeps the next four entries of each list in registers and reads past them one at a time.


def _dense_mix(seed, n, k):
    """Heavy-tail rows (about 2% escapes), Gaussian rows (almost none) and rows of zeros (all
    escapes): some tiles' lists fit a slice and some do not; n and k ragged."""
    g = torch.Generator().manual_seed(seed)
    w = S.layer_matrix(g, n, k)
    w[:64] = S.heavy_tail_weights(seed, 64, k)
    w[128:] = 0
    return w


def _window_edge(seed, n, k):
    """Gaussian rows with (n + c) % 7 zeros at the start of chunk c of channel n: chunks with
    0..6 escapes, i.e. inside, at and past a four-entry window."""
    w = S.layer_matrix(torch.Generator().manual_seed(seed), n, k)
    for r in range(n):
        for c in range(k // 16):
            w[r, 16 * c:16 * c + (r + c) % 7] = 0
    return w


DENSE = {
    "dense_mix_150x1000": lambda: _dense_mix(31, 150, 1000),
    "window_edge_64x512": lambda: _window_edge(32, 64, 512),
}
_dense_cache = {}


@pytest.mark.parametrize("name", list(DENSE))
@pytest.mark.parametrize("m,gemv_max,grid", [(1, 2, 0), (2, 2, 0), (3, 4, 0), (4, 4, 0), (8, 2, 0),
                                              (16, 2, 0), (16, 2, 3), (1, 2, 2), (4, 4, 5)])
def test_gemm_escape_dense(monkeypatch, name, m, gemv_max, grid):
    """Escape-dense tensors through the escape-window instantiation (GEMV and 16-row tiles, some
    with grids small enough that work-group ranges cross tiles): within tolerance of the FP64
    product and bitwise repeatable."""
    if name not in _dense_cache:
        w = DENSE[name]()
        _dense_cache[name] = (w, w12.encode(dev_weights(w)))
    w, t = _dense_cache[name]
    n, k = w.shape
    assert t.num_escapes * 64 > 1024 * n, "the tensor must be escape-dense"
    monkeypatch.setenv("W12_GEMV_MAX_M", str(gemv_max))
    if grid:
        monkeypatch.setenv("W12_MAX_GRID", str(grid))
    say(f"[dense] {name} M={m} gemv_max={gemv_max} grid={grid} E={t.num_escapes}")
    x = S.activations(m, k, 1300 + m)
    xd = to_dev(x, (k + 7) // 8 * 8)
    y1 = w12.gemm(xd, t).cpu().numpy()
    y2 = w12.gemm(xd, t).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "not bitwise repeatable"
    bad, worst = O.gemm_check(x, w, y1)
    assert bad == 0, f"{bad} outputs outside tolerance (worst rel {worst:.3g})"


@pytest.mark.parametrize("name", list(DENSE))
@pytest.mark.parametrize("m,grid", [(65, 0), (200, 0), (300, 0), (130, 1), (257, 2)])
def test_gemm_wide_escape_dense(monkeypatch, name, m, grid):
    """Escape-dense tensors through the wide tiles' escape-window instantiation (W12_WIDE_MIN_M = 3
    keeps every M on the wide tiles; small grids make work-group ranges cross tiles): within
    tolerance of the FP64 product and bitwise repeatable."""
    if name not in _dense_cache:
        w = DENSE[name]()
        _dense_cache[name] = (w, w12.encode(dev_weights(w)))
    w, t = _dense_cache[name]
    n, k = w.shape
    assert t.num_escapes * 256 > 2048 * n, "the tensor must be escape-dense for 256-channel tiles"
    monkeypatch.setenv("W12_WIDE_MIN_M", "3")
    if grid:
        monkeypatch.setenv("W12_MAX_GRID", str(grid))
    assert w12.gemm_plan(m, n, k)["path"] == 3
    say(f"[dense wide] {name} M={m} grid={grid} E={t.num_escapes}")
    x = S.activations(m, k, 1700 + m)
    xd = to_dev(x, (k + 7) // 8 * 8)
    y1 = w12.gemm(xd, t).cpu().numpy()
    y2 = w12.gemm(xd, t).cpu().numpy()
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32)), "not bitwise repeatable"
    bad, worst = O.gemm_check(x, w, y1)
    assert bad == 0, f"{bad} outputs outside tolerance (worst rel {worst:.3g})"
