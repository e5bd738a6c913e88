"""W12 checkpoint files on the host: the byte layout written by w12_file_write, read back with
numpy from the documented format (header, 128-byte index entries, 256-byte aligned sections),
and the index reader's error handling.  No GPU is used: the writer takes host arrays."""
import ctypes

import numpy as np
import pytest

import lossless_bit_weight_encode_amd as w12
from lossless_bit_weight_encode_amd import _lib as L


def _fake_tensor(rng, n, k, e):
    """Random host planes of the right sizes (the file layer does not interpret them)."""
    hib, lob = w12.layout_bytes(n, k)
    base = rng.integers(1, 240, n, dtype=np.uint8)
    hi = rng.integers(0, 256, hib, dtype=np.uint8)
    lo = rng.integers(0, 256, lob, dtype=np.uint8)
    esc_ptr = np.sort(rng.integers(0, e + 1, n + 1)).astype(np.uint32)
    esc_ptr[0], esc_ptr[-1] = 0, e
    esc = rng.integers(0, 1 << 32, e, dtype=np.uint64).astype(np.uint32)
    return dict(n=n, k=k, e=e, base=base, hi=hi, lo=lo, esc_ptr=esc_ptr, esc=esc)


def _write(path, named):
    descs = (L._Tensor * len(named))()
    for i, t in enumerate(named.values()):
        descs[i] = L._host_descriptor(t["n"], t["k"], t["e"], t["base"], t["hi"], t["lo"], t["esc_ptr"], t["esc"])
    names = (ctypes.c_char_p * len(named))(*[nm.encode() for nm in named])
    return w12.lib().w12_file_write(str(path).encode(), len(named), names, descs)


def test_file_layout_matches_format(tmp_path):
    rng = np.random.default_rng(0)
    named = {"a.qkv": _fake_tensor(rng, 37, 1000, 11), "b": _fake_tensor(rng, 300, 512, 0),
             "c" * 70: _fake_tensor(rng, 1, 16, 3)}
    path = tmp_path / "m.w12"
    assert _write(path, named) == 0
    raw = np.fromfile(path, dtype=np.uint8)
    assert raw[:8].tobytes() == b"W12CKPT1"
    assert int(raw[8:12].view(np.uint32)[0]) == 1
    assert int(raw[12:16].view(np.uint32)[0]) == 3
    assert not raw[16:64].any()
    idx = w12.file_index(str(path))
    assert [e["name"] for e in idx] == ["a.qkv", "b", "c" * 63]
    prev_end = 64 + 3 * 128
    for i, (nm, t) in enumerate(named.items()):
        ent = raw[64 + 128 * i: 64 + 128 * (i + 1)]
        n, k, layout, res = ent[64:80].view(np.int32)
        e, off, nbytes = ent[80:104].view(np.uint64)
        assert (n, k, layout, res, e) == (t["n"], t["k"], 1, 0, t["e"])
        assert idx[i]["offset"] == off and idx[i]["bytes"] == nbytes
        assert off % 256 == 0 and off >= prev_end
        o = int(off)
        for arr in (t["base"], t["esc_ptr"], t["esc"], t["hi"], t["lo"]):
            b = arr.view(np.uint8)
            assert o % 256 == 0
            assert np.array_equal(raw[o:o + b.size], b)
            o = (o + b.size + 255) // 256 * 256
        assert o == off + nbytes
        prev_end = o
    assert raw.size == prev_end


def test_file_index_errors(tmp_path):
    lib = w12.lib()
    n = L._c_i32()
    assert lib.w12_file_index(str(tmp_path / "missing.w12").encode(), ctypes.byref(n), None, 0) == -6
    bad = tmp_path / "bad.w12"
    bad.write_bytes(b"NOTW12\0\0" + bytes(56))
    assert lib.w12_file_index(str(bad).encode(), ctypes.byref(n), None, 0) == -6
    # a truncated index
    rng = np.random.default_rng(1)
    path = tmp_path / "t.w12"
    assert _write(path, {"x": _fake_tensor(rng, 20, 96, 2), "y": _fake_tensor(rng, 20, 96, 2)}) == 0
    data = path.read_bytes()
    cut = tmp_path / "cut.w12"
    cut.write_bytes(data[:64 + 128 + 40])
    entries = (L._FileEntry * 4)()
    assert lib.w12_file_index(str(cut).encode(), ctypes.byref(n), entries, 4) == -6
    # room for fewer entries than the file holds
    assert lib.w12_file_index(str(path).encode(), ctypes.byref(n), entries, 1) == -1
    assert lib.w12_file_index(str(path).encode(), ctypes.byref(n), entries, 4) == 0 and n.value == 2


def test_file_write_and_load_validation(tmp_path):
    lib = w12.lib()
    rng = np.random.default_rng(2)
    t = _fake_tensor(rng, 20, 96, 2)
    assert _write(tmp_path / "z.w12", {}) == -1                     # count 0
    bad = dict(t, n=0)
    assert _write(tmp_path / "z.w12", {"x": bad}) == -2              # shape
    assert _write(tmp_path / "nodir" / "z.w12", {"x": t}) == -6      # cannot open
    path = tmp_path / "ok.w12"
    assert _write(path, {"x": t}) == 0
    d = (L._Tensor * 1)()
    d[0] = L._host_descriptor(20, 96, 2, t["base"], t["hi"], t["lo"], t["esc_ptr"], t["esc"])
    which = (L._c_i32 * 1)(0)
    stage = ctypes.create_string_buffer(4096)
    # staging too small, index out of range, descriptor not matching the entry: refused before any copy
    assert lib.w12_file_load(str(path).encode(), 1, which, d, ctypes.addressof(stage), 100, None, None, None, None) == -1
    which[0] = 1
    assert lib.w12_file_load(str(path).encode(), 1, which, d, ctypes.addressof(stage), 4096, None, None, None, None) == -1
    which[0] = 0
    d[0].num_escapes = 3
    assert lib.w12_file_load(str(path).encode(), 1, which, d, ctypes.addressof(stage), 4096, None, None, None, None) == -1
    assert "does not match" in lib.w12_last_error().decode()
