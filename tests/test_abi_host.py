"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and
rejects bad arguments before touching a GPU.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

import lossless_bit_weight_encode_amd as w12
from lossless_bit_weight_encode_amd import _lib as L
from oracle import w12_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w12.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w12_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = w12.lib()
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(L.EXPORTED)


def test_status_strings():
    lib = w12.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.w12_status_string(code).decode() != "unknown status"
    assert lib.w12_status_string(7).decode() == "unknown status"


@pytest.mark.parametrize("n,k,e", [(1, 5, 2), (5120, 5120, 0), (34816, 5120, 29837), (7, 1000, 123)])
def test_bits_per_weight_matches_definition(n, k, e):
    assert w12.bits_per_weight(n, k, e) == pytest.approx(O.bits_per_weight(n, k, e), rel=1e-15)


@pytest.mark.parametrize("n,k,e", [(1, 16, 0), (34816, 5120, 29837), (3, 5, 7), (5120, 17408, 1800594)])
def test_tensor_bytes_matches_definition(n, k, e):
    """w12_tensor_bytes = the oracle's bits per weight x N K / 8 (rounded up to whole bytes)."""
    import math
    assert w12.tensor_bytes(n, k, e) == math.ceil(O.bits_per_weight(n, k, e) * n * k / 8 - 1e-6)
    assert w12.tensor_bytes(0, k, e) == 0 and w12.tensor_bytes(n, k, -1) == 0


@pytest.mark.parametrize("m,n", [(1, 64), (1, 65520), (16, 65520), (33, 4096), (100, 65520), (256, 65520)])
def test_long_k_is_always_split(m, n):
    """At K = 65,536 (256 units of 256 k per tile) no work-group range holds more than 250
    units, so a lane chains at most 4,000 products and the summation depth stays below 4,096."""
    k = 65536
    p = w12.gemm_plan(m, n, k)
    rb = 16 if p["path"] == 3 else 4
    tiles = ((n + 15) // 16 + rb - 1) // rb * ((m + p["m_tile"] - 1) // p["m_tile"])
    units = tiles * 256
    assert -(-units // p["grid"]) <= 250
    assert p["splits"] >= 2


def test_layout_bytes():
    assert w12.layout_bytes(256, 512) == (256 * 512, 256 * 512 // 2)
    # ragged N and K are padded to 16 rows x 16 k
    assert w12.layout_bytes(17, 33) == (32 * 48, 32 * 48 // 2)
    assert w12.layout_bytes(1, 65536) == (16 * 65536, 8 * 65536)


@pytest.mark.parametrize("n,k", [(0, 64), (-3, 64), (1, 0), (4, 65537), (1 << 25, 16), (70000, 65536)])
def test_bad_shapes_rejected(n, k):
    with pytest.raises(w12.W12Error) as ei:
        w12.layout_bytes(n, k)
    assert ei.value.status == -2


def _desc(n=64, k=64, e=0, **kw):
    d = L._Tensor()
    d.N, d.K, d.layout, d.reserved, d.num_escapes = n, k, L.W12_LAYOUT_RB16_K16, 0, e
    d.base, d.hi, d.lo, d.esc_ptr, d.esc = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000
    for key, v in kw.items():
        setattr(d, key, v)
    return d


def call_gemm(x=0x10000, m=4, ldx=64, d=None, y=0x20000, ldy=64, ws=None, ws_bytes=0):
    d = d or _desc()
    return w12.lib().w12_gemm(x, m, ldx, ctypes.byref(d), y, ldy, ws, ws_bytes, None)


def test_escape_count_limit():
    """E >= 2^30 is rejected before any launch (the kernels use 32-bit byte offsets into the
    escape list); E = 2^30 - 1 passes the tensor check and fails later on a NULL workspace."""
    big = dict(n=1 << 16, k=1 << 15)
    assert call_gemm(d=_desc(e=1 << 30, **big), ldx=1 << 15, ldy=1 << 16) == -2
    assert "2^30" in w12.lib().w12_last_error().decode()
    assert call_gemm(d=_desc(e=(1 << 30) - 1, **big), ldx=1 << 15, ldy=1 << 16, m=16) in (-1, -3)
    assert w12.lib().w12_decode(ctypes.byref(_desc(e=1 << 30, **big)), 0x10000, 1 << 15, None) == -2


def test_gemm_argument_validation():
    lib = w12.lib()
    assert call_gemm(x=None) == -1
    assert call_gemm(m=0) == -2
    assert call_gemm(m=5000) == -2
    assert call_gemm(ldx=32) == -1                 # pitch below K
    assert call_gemm(ldx=68) == -5                 # pitch not a multiple of 8
    assert call_gemm(x=0x10002) == -5              # X not 16-byte aligned
    assert call_gemm(y=None) == -1
    assert call_gemm(ldy=10) == -1
    assert call_gemm(d=_desc(layout=2)) == -1
    assert call_gemm(d=_desc(reserved=1)) == -1
    assert call_gemm(d=_desc(hi=0)) == -1
    assert call_gemm(d=_desc(hi=0x2008)) == -5
    assert call_gemm(d=_desc(e=5, esc=0)) == -1
    assert call_gemm(d=_desc(e=-1)) == -1
    assert call_gemm(d=_desc(n=0)) == -2
    assert "M=" in lib.w12_last_error().decode() or True
    # a case that needs a workspace must be refused when it is too small
    need = w12.gemm_workspace_size(16, 5120, 17408)
    assert need > 0
    d = _desc(n=5120, k=17408)
    assert call_gemm(m=16, ldx=17408, d=d, ldy=5120, ws=0x100000, ws_bytes=need - 1) == -3
    assert "workspace" in lib.w12_last_error().decode()
    assert call_gemm(m=16, ldx=17408, d=d, ldy=5120, ws=None, ws_bytes=need) == -1


def test_encode_decode_verify_validation():
    lib = w12.lib()
    d = _desc()
    assert lib.w12_encode_count(None, 4, 64, 64, None, 0x1000, 0x2000, None) == -1
    assert lib.w12_encode_count(0x1000, 4, 64, 60, None, 0x1000, 0x2000, None) == -1
    assert lib.w12_encode_count(0x1008, 4, 64, 64, None, 0x1000, 0x2000, None) == -5
    assert lib.w12_encode_count(0x1000, 4, 64, 64, None, None, 0x2000, None) == -1
    assert lib.w12_encode_count(0x1000, 4, 0, 64, None, 0x1000, 0x2000, None) == -2
    assert lib.w12_encode_emit(0x1000, 64, None, None) == -1
    assert lib.w12_encode_emit(0x1000, 63, ctypes.byref(d), None) == -1
    assert lib.w12_decode(ctypes.byref(d), None, 64, None) == -1
    assert lib.w12_decode(ctypes.byref(d), 0x1000, 72 + 4, None) == -5
    assert lib.w12_verify(ctypes.byref(d), 0x1000, 64, None, None) == -1
    assert lib.w12_verify(ctypes.byref(d), 0x1000, 64, 0x1004, None) == -5
    assert lib.w12_unpack_records(ctypes.byref(d), None, 64, None) == -1
    assert lib.w12_unpack_records(ctypes.byref(d), 0x1000, 10, None) == -1


@pytest.mark.parametrize("m,n,k", [(1, 256, 512), (8, 5120, 17408), (16, 34816, 5120), (63, 7168, 5120),
                                   (512, 34816, 5120), (256, 5120, 17408), (100, 300, 4096), (70, 17, 33),
                                   (9, 1, 16), (3, 17, 33)])
def test_gemm_plan_is_consistent(m, n, k):
    p = w12.gemm_plan(m, n, k)
    assert p["path"] == (1 if m <= 2 else (2 if m < 65 else 3))
    # streaming tiles: 4 row blocks (64 channels); wide tiles: 16 row blocks x 128 or 256 rows
    rb = 16 if p["path"] == 3 else 4
    assert p["rows_per_block"] == 16 * rb
    if p["path"] == 3:
        assert p["m_tile"] == (128 if m <= 128 else 256)
    assert p["splits"] >= 1
    kc = (k + 15) // 16
    upt = (kc + 15) // 16                       # stream-K units (16 chunks) per tile
    tiles = ((n + 15) // 16 + rb - 1) // rb * ((m + p["m_tile"] - 1) // p["m_tile"])
    assert 1 <= p["grid"] <= min(tiles * upt, 4096)   # never more work-groups than units (or counters)
    # one counter region for every plan: a counter per work-group, up to 4096 work-groups
    assert p["counter_bytes"] == 16384
    if tiles <= p["grid"]:
        # a whole multiple of the tiles when that keeps 3/4 of the grid: no range crosses a tile
        assert p["grid"] % tiles == 0 or p["grid"] * 3 > 4 * (p["grid"] // tiles) * tiles
    # counters + two partial tiles (tile channels x m tile) per work-group, + a copy of X: for
    # the wide tiles every m tile whole in operand order, otherwise X padded to whole 16-k
    # chunks when K is ragged
    if p["path"] == 3:
        mt = (m + p["m_tile"] - 1) // p["m_tile"]
        xpad = (mt * p["m_tile"] * kc * 16 * 2 + 255) // 256 * 256
    else:
        xpad = 0 if k % 16 == 0 else (m * kc * 16 * 2 + 255) // 256 * 256
    assert p["workspace_bytes"] == p["counter_bytes"] + 2 * p["grid"] * 16 * rb * p["m_tile"] * 4 + xpad
    assert w12.gemm_workspace_size(m, n, k) == p["workspace_bytes"]


@pytest.mark.parametrize("limit", [0, 1, 5, 8, 99, -3])
def test_gemm_gemv_boundary_env(monkeypatch, limit):
    """W12_GEMV_MAX_M moves the GEMV / MFMA boundary (clamped to 0..8) at each call."""
    monkeypatch.setenv("W12_GEMV_MAX_M", str(limit))
    eff = min(max(limit, 0), 8)
    for m in range(1, 17):
        p = w12.gemm_plan(m, 4096, 4096)
        assert p["path"] == (1 if m <= eff else 2), (limit, m)
        assert p["m_tile"] == (m if p["path"] == 1 else 16)


@pytest.mark.parametrize("limit", [3, 17, 65, 129, 100000])
def test_gemm_wide_boundary_env(monkeypatch, limit):
    """W12_WIDE_MIN_M moves the streaming / wide-tile boundary at each call."""
    monkeypatch.setenv("W12_WIDE_MIN_M", str(limit))
    for m in (3, 16, 64, 65, 100, 128, 129, 256, 512):
        p = w12.gemm_plan(m, 5120, 5120)
        assert p["path"] == (3 if m >= limit else 2), (limit, m)
        assert p["m_tile"] == ((128 if m <= 128 else 256) if m >= limit else min(64, (m + 15) // 16 * 16))


@pytest.mark.parametrize("cap", [1, 3, 100])
def test_gemm_grid_cap_env(monkeypatch, cap):
    """W12_MAX_GRID caps the work-groups of a GEMM (read at each call)."""
    monkeypatch.setenv("W12_MAX_GRID", str(cap))
    for m, n, k in [(1, 5120, 5120), (16, 34816, 5120), (64, 300, 4096)]:
        p = w12.gemm_plan(m, n, k)
        assert 1 <= p["grid"] <= cap
        assert w12.gemm_workspace_size(m, n, k) == p["workspace_bytes"]


def _items(descs, m, x=0x10000, y=0x20000):
    items = (L._GemmItem * len(descs))()
    for i, d in enumerate(descs):
        items[i].X, items[i].ldx = x, d.K
        items[i].t = ctypes.pointer(d)
        items[i].Y, items[i].ldy = y, d.N
    return items


def test_gemm_group_argument_validation():
    lib = w12.lib()
    d = [_desc(n=5120, k=5120), _desc(n=5120, k=17408)]
    items = _items(d, 16)
    need = L._c_u64()
    assert lib.w12_gemm_group_workspace_size(16, 2, items, ctypes.byref(need)) == 0
    assert need.value > 0
    assert lib.w12_gemm_group_workspace_size(16, 0, items, ctypes.byref(need)) == -2
    assert lib.w12_gemm_group_workspace_size(16, L.GROUP_MAX + 1, items, ctypes.byref(need)) == -2
    assert lib.w12_gemm_group_workspace_size(65, 2, items, ctypes.byref(need)) == -2
    assert lib.w12_gemm_group_workspace_size(0, 2, items, ctypes.byref(need)) == -2
    assert lib.w12_gemm_group_workspace_size(16, 2, None, ctypes.byref(need)) == -1
    # K not a multiple of 16
    bad = _items([_desc(n=64, k=1000)], 4)
    assert lib.w12_gemm_group_workspace_size(4, 1, bad, ctypes.byref(need)) == -2
    # a bad member descriptor names its item
    bad = _items([_desc(n=64, k=1024), _desc(n=64, k=1024, hi=0)], 4)
    assert lib.w12_gemm_group_workspace_size(4, 2, bad, ctypes.byref(need)) == -1
    assert "item 1" in lib.w12_last_error().decode()
    # operand checks, workspace size
    lib.w12_gemm_group_workspace_size(16, 2, items, ctypes.byref(need))
    assert lib.w12_gemm_group(16, 2, items, 0x100000, need.value - 1, None) == -3
    assert lib.w12_gemm_group(16, 2, items, None, need.value, None) == -1
    assert lib.w12_gemm_group(16, 2, items, 0x100008, need.value, None) == -5
    items[1].X = 0x10002
    assert lib.w12_gemm_group(16, 2, items, 0x100000, need.value, None) == -5
    assert "item 1" in lib.w12_last_error().decode()
    items[1].X = 0x10000
    items[0].Y = None
    assert lib.w12_gemm_group_q(16, 2, items, 0x100000, need.value, None) == -1
    items[0].Y = 0x20000
    items[0].ldy = 10
    assert lib.w12_gemm_group(16, 2, items, 0x100000, need.value, None) == -1


@pytest.mark.parametrize("m", [1, 16, 32, 64])
def test_gemm_group_workspace_covers_counters_and_partials(m):
    """The group workspace holds one counter per tile of every product and two partial tiles per
    work-group; a group of one needs no more than the single launch's counters and partials."""
    d = [_desc(n=7168, k=5120), _desc(n=5120, k=5120), _desc(n=34816, k=5120), _desc(n=5120, k=17408)]
    need = L._c_u64()
    assert w12.lib().w12_gemm_group_workspace_size(m, 4, _items(d, m), ctypes.byref(need)) == 0
    tiles = sum(-(-(-(-dd.N // 16)) // 4) for dd in d)
    assert need.value >= 4 * tiles
    one = L._c_u64()
    assert w12.lib().w12_gemm_group_workspace_size(m, 1, _items(d[2:3], m), ctypes.byref(one)) == 0
    assert one.value <= need.value


def test_group_constants_match_the_header():
    text = open(HEADER).read()
    assert int(re.search(r"#define W12_GROUP_MAX (\d+)", text).group(1)) == L.GROUP_MAX
    assert int(re.search(r"#define W12_GROUP_INLINE (\d+)", text).group(1)) == L.GROUP_INLINE
    assert L.GROUP_INLINE < L.GROUP_MAX


def _group_need(m, d):
    need = L._c_u64()
    rc = w12.lib().w12_gemm_group_workspace_size(m, len(d), _items(d, m), ctypes.byref(need))
    return rc, need.value


@pytest.mark.parametrize("m", [1, 16, 32])
def test_large_group_workspace_holds_the_argument_blocks(m, monkeypatch):
    """Past W12_GROUP_INLINE products the argument blocks (one per product) sit after the
    partials: the region grows with the count, on top of what the same launch shape needs."""
    monkeypatch.setenv("W12_MAX_GRID", "64")   # the same grid (and partial region) for every count
    d = [_desc(n=64, k=2048) for _ in range(L.GROUP_MAX)]
    sizes = {}
    for count in (L.GROUP_INLINE, L.GROUP_INLINE + 1, 100, L.GROUP_MAX):
        rc, sizes[count] = _group_need(m, d[:count])
        assert rc == 0, count
    inline = sizes[L.GROUP_INLINE]
    # about 200 bytes per product, rounded to 256 bytes
    for count in (L.GROUP_INLINE + 1, 100, L.GROUP_MAX):
        extra = sizes[count] - inline
        assert 64 * count <= extra <= 512 * count + 256, (count, extra)
    assert (sizes[L.GROUP_MAX] - inline) % 256 == 0
    rc, _ = _group_need(m, d + d[:1])
    assert rc == -2


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """Without libw12.so the binding raises; there is no other code path."""
    monkeypatch.setattr(L, "LIB_PATH", str(tmp_path / "absent" / "libw12.so"))
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        L.lib()


def test_binding_refuses_host_tensors():
    import torch
    w = torch.zeros(16, 16, dtype=torch.int16)
    with pytest.raises(ValueError, match="GPU"):
        w12.encode(w)
    with pytest.raises(ValueError, match="GPU"):
        w12.gemm(torch.zeros(1, 16, dtype=torch.int16), None)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
