"""ctypes binding of libw12.so: argument marshalling only.

Every step of encode / decode / verify / GEMM runs in the HIP kernels of libw12.so.
PyTorch provides device memory and the current stream.  If the library is not built, or
a tensor is not on a GPU, the calls raise: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libw12.so")

W12_OK = 0
W12_LAYOUT_RB16_K16 = 1

_c_i32, _c_i64, _c_u64, _c_p = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_void_p


class _Tensor(ctypes.Structure):
    _fields_ = [
        ("N", _c_i32), ("K", _c_i32), ("layout", _c_i32), ("reserved", _c_i32),
        ("num_escapes", _c_i64),
        ("base", _c_p), ("hi", _c_p), ("lo", _c_p), ("esc_ptr", _c_p), ("esc", _c_p),
    ]


class _GemmItem(ctypes.Structure):
    _fields_ = [("X", _c_p), ("ldx", _c_i64), ("t", ctypes.POINTER(_Tensor)), ("Y", _c_p), ("ldy", _c_i64)]


GROUP_MAX = 1024      # products per grouped launch
GROUP_INLINE = 8      # of which the kernel arguments hold this many; larger groups copy theirs to the workspace


class _FileEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("N", _c_i32), ("K", _c_i32), ("layout", _c_i32), ("reserved", _c_i32),
                ("num_escapes", _c_i64), ("offset", _c_u64), ("bytes", _c_u64)]


class _PlanInfo(ctypes.Structure):
    _fields_ = [
        ("path", _c_i32), ("splits", _c_i32), ("rows_per_block", _c_i32), ("m_tile", _c_i32),
        ("grid", _c_i64), ("workspace_bytes", _c_u64), ("counter_bytes", _c_u64),
    ]


_SIGNATURES = {
    "w12_layout_bytes": (ctypes.c_int, [_c_i32, _c_i32, ctypes.POINTER(_c_u64), ctypes.POINTER(_c_u64)]),
    "w12_encode_count": (ctypes.c_int, [_c_p, _c_i32, _c_i32, _c_i64, _c_p, _c_p, _c_p, _c_p]),
    "w12_encode_emit": (ctypes.c_int, [_c_p, _c_i64, ctypes.POINTER(_Tensor), _c_p]),
    "w12_decode": (ctypes.c_int, [ctypes.POINTER(_Tensor), _c_p, _c_i64, _c_p]),
    "w12_verify": (ctypes.c_int, [ctypes.POINTER(_Tensor), _c_p, _c_i64, _c_p, _c_p]),
    "w12_unpack_records": (ctypes.c_int, [ctypes.POINTER(_Tensor), _c_p, _c_i64, _c_p]),
    "w12_gemm_workspace_size": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_u64)]),
    "w12_gemm_workspace_init": (ctypes.c_int, [_c_p, _c_u64, _c_p]),
    "w12_gemm": (ctypes.c_int, [_c_p, _c_i32, _c_i64, ctypes.POINTER(_Tensor), _c_p, _c_i64, _c_p, _c_u64, _c_p]),
    "w12_gemm_q": (ctypes.c_int, [_c_p, _c_i32, _c_i64, ctypes.POINTER(_Tensor), _c_p, _c_i64, _c_p, _c_u64, _c_p]),
    "w12_gemm_noalloc": (ctypes.c_int, [_c_p, _c_i32, _c_i64, ctypes.POINTER(_Tensor), _c_p, _c_i64, _c_p]),
    "w12_gemm_plan": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, ctypes.POINTER(_PlanInfo)]),
    "w12_gemm_group_workspace_size": (ctypes.c_int, [_c_i32, _c_i32, ctypes.POINTER(_GemmItem), ctypes.POINTER(_c_u64)]),
    "w12_gemm_group": (ctypes.c_int, [_c_i32, _c_i32, ctypes.POINTER(_GemmItem), _c_p, _c_u64, _c_p]),
    "w12_gemm_group_q": (ctypes.c_int, [_c_i32, _c_i32, ctypes.POINTER(_GemmItem), _c_p, _c_u64, _c_p]),
    "w12_file_write": (ctypes.c_int, [ctypes.c_char_p, _c_i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_Tensor)]),
    "w12_file_index": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(_c_i32), ctypes.POINTER(_FileEntry), _c_i32]),
    "w12_file_load": (ctypes.c_int, [ctypes.c_char_p, _c_i32, ctypes.POINTER(_c_i32), ctypes.POINTER(_Tensor), _c_p,
                                     _c_u64, ctypes.POINTER(_c_p), ctypes.POINTER(_c_i64), _c_p, _c_p]),
    "w12_read_probe": (ctypes.c_int, [_c_p, _c_u64, _c_i32, _c_i32, _c_p, _c_p]),
    "w12_bits_per_weight": (ctypes.c_double, [_c_i32, _c_i32, _c_i64]),
    "w12_tensor_bytes": (_c_u64, [_c_i32, _c_i32, _c_i64]),
    "w12_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "w12_last_error": (ctypes.c_char_p, []),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


class W12Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libw12.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m lossless_bit_weight_encode_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != W12_OK:
        msg = lib().w12_last_error().decode()
        raise W12Error(fn, status, msg or lib().w12_status_string(status).decode())


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _pitch(t: torch.Tensor) -> int:
    """Row pitch in elements.  A single-row matrix is never stepped by its pitch, and torch
    may report any stride for a size-1 dimension, so it gets its padded width."""
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride 1 along k)")
    if t.shape[0] == 1:
        return (t.shape[1] + 7) // 8 * 8
    return t.stride(0)


def _require_cuda(*ts: torch.Tensor) -> None:
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU (libw12 has no CPU path)")


def _bits16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected BF16 bit patterns (bfloat16/int16/uint16), got {t.dtype}")
    return t


def layout_bytes(n: int, k: int) -> tuple[int, int]:
    hi, lo = _c_u64(), _c_u64()
    _check("w12_layout_bytes", lib().w12_layout_bytes(n, k, ctypes.byref(hi), ctypes.byref(lo)))
    return hi.value, lo.value


@dataclass
class W12Tensor:
    """An encoded tensor: the planes and escape list, all on the GPU."""
    n: int
    k: int
    base: torch.Tensor      # uint8 [N]
    hi: torch.Tensor        # uint8 [layout hi bytes]
    lo: torch.Tensor        # uint8 [layout lo bytes]
    esc_ptr: torch.Tensor   # int32 [N+1] (uint32 values)
    esc: torch.Tensor       # int32 [E]  (uint32 values)

    @property
    def num_escapes(self) -> int:
        return int(self.esc.numel())

    def descriptor(self) -> _Tensor:
        d = _Tensor()
        d.N, d.K, d.layout, d.reserved = self.n, self.k, W12_LAYOUT_RB16_K16, 0
        d.num_escapes = self.num_escapes
        d.base, d.hi, d.lo = _ptr(self.base), _ptr(self.hi), _ptr(self.lo)
        d.esc_ptr = _ptr(self.esc_ptr)
        d.esc = _ptr(self.esc) if self.num_escapes else None
        return d

    def bits_per_weight(self) -> float:
        return bits_per_weight(self.n, self.k, self.num_escapes)

    def nbytes(self) -> int:
        """Bytes of the logical format (w12_tensor_bytes)."""
        return tensor_bytes(self.n, self.k, self.num_escapes)


def alloc_planes(n: int, k: int, device) -> tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    hib, lob = layout_bytes(n, k)
    base = torch.empty(n, dtype=torch.uint8, device=device)
    hi = torch.empty(hib, dtype=torch.uint8, device=device)
    lo = torch.empty(lob, dtype=torch.uint8, device=device)
    esc_ptr = torch.empty(n + 1, dtype=torch.int32, device=device)
    return base, hi, lo, esc_ptr


def encode_count(w: torch.Tensor, base: torch.Tensor, esc_ptr: torch.Tensor, forced_base: torch.Tensor | None = None,
                 stream=None) -> None:
    _require_cuda(w, base, esc_ptr, forced_base)
    _bits16(w)
    n, k = w.shape
    _check("w12_encode_count", lib().w12_encode_count(_ptr(w), n, k, _pitch(w), _ptr(forced_base), _ptr(base),
                                                       _ptr(esc_ptr), _stream(stream)))


def encode_emit(w: torch.Tensor, t: W12Tensor, stream=None) -> None:
    _require_cuda(w)
    _bits16(w)
    d = t.descriptor()
    _check("w12_encode_emit", lib().w12_encode_emit(_ptr(w), _pitch(w), ctypes.byref(d), _stream(stream)))


def encode(w: torch.Tensor, forced_base: torch.Tensor | None = None, stream=None) -> W12Tensor:
    """BF16 [N, K] on the GPU -> W12Tensor.  Reads E back once (one synchronisation).

    With a stream, everything (allocations, kernels, the read-back of E) runs on that stream;
    w and forced_base must be ready on it."""
    _require_cuda(w)
    _bits16(w)
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        n, k = w.shape
        base, hi, lo, esc_ptr = alloc_planes(n, k, w.device)
        encode_count(w, base, esc_ptr, forced_base)
        e = int(esc_ptr[n].item()) & 0xFFFFFFFF   # copies and waits on the same stream
        esc = torch.empty(e, dtype=torch.int32, device=w.device)
        t = W12Tensor(n, k, base, hi, lo, esc_ptr, esc)
        encode_emit(w, t)
    return t


def encode_many(ws: list, stream=None) -> list:
    """encode() of several BF16 matrices with a single read-back: every count pass is launched,
    the escape counts E of all of them come back in one copy (one synchronisation), then every
    emit is launched.  Returns the W12Tensors in the order of ws."""
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        parts = []
        for w in ws:
            _require_cuda(w)
            _bits16(w)
            n, k = w.shape
            base, hi, lo, esc_ptr = alloc_planes(n, k, w.device)
            encode_count(w, base, esc_ptr)
            parts.append((w, n, k, base, hi, lo, esc_ptr))
        if not parts:
            return []
        es = torch.stack([p[6][p[1]] for p in parts]).cpu().tolist()   # copies and waits on the same stream
        out = []
        for (w, n, k, base, hi, lo, esc_ptr), e in zip(parts, es):
            esc = torch.empty(int(e) & 0xFFFFFFFF, dtype=torch.int32, device=w.device)
            t = W12Tensor(n, k, base, hi, lo, esc_ptr, esc)
            encode_emit(w, t)
            out.append(t)
    return out


def decode(t: W12Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if out is None:
        # rows padded to a multiple of 8 elements (the 16-byte store granule), viewed to K
        ld = (t.k + 7) // 8 * 8
        out = torch.empty(t.n, ld, dtype=torch.bfloat16, device=t.hi.device)[:, :t.k]
    _require_cuda(out)
    d = t.descriptor()
    _check("w12_decode", lib().w12_decode(ctypes.byref(d), _ptr(out), _pitch(out), _stream(stream)))
    return out


def verify_async(t: W12Tensor, ref: torch.Tensor, result: torch.Tensor, stream=None) -> None:
    _require_cuda(ref, result)
    d = t.descriptor()
    _check("w12_verify", lib().w12_verify(ctypes.byref(d), _ptr(ref), _pitch(ref), _ptr(result), _stream(stream)))


def verify(t: W12Tensor, ref: torch.Tensor, stream=None) -> tuple[int, int]:
    """(mismatch count, first bad flat index or -1); synchronises to read the result.  With a
    stream, the result buffer, the check and the read-back all run on that stream."""
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        result = torch.empty(2, dtype=torch.int64, device=ref.device)
        verify_async(t, ref, result)
        cnt, first = (int(v) for v in result.cpu().tolist())
    return cnt, (-1 if first == -1 else first)


def unpack_records(t: W12Tensor, stream=None) -> torch.Tensor:
    rec = torch.empty(t.n, t.k, dtype=torch.int16, device=t.hi.device)
    d = t.descriptor()
    _check("w12_unpack_records", lib().w12_unpack_records(ctypes.byref(d), _ptr(rec), _pitch(rec), _stream(stream)))
    return rec


def gemm_workspace_size(m: int, n: int, k: int) -> int:
    b = _c_u64()
    _check("w12_gemm_workspace_size", lib().w12_gemm_workspace_size(m, n, k, ctypes.byref(b)))
    return b.value


def gemm_plan(m: int, n: int, k: int) -> dict:
    info = _PlanInfo()
    _check("w12_gemm_plan", lib().w12_gemm_plan(m, n, k, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in _PlanInfo._fields_}


def gemm_workspace_init(ws: torch.Tensor, stream=None) -> None:
    _require_cuda(ws)
    _check("w12_gemm_workspace_init",
           lib().w12_gemm_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def gemm_workspace(m: int, n: int, k: int, device="cuda", stream=None) -> torch.Tensor | None:
    """A ready-to-use (zero-initialised) workspace for gemm() with M=m on W[n][k], or None."""
    need = gemm_workspace_size(m, n, k)
    if not need:
        return None
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    gemm_workspace_init(ws, stream)
    return ws


def gemm(x: torch.Tensor, t: W12Tensor, y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
         stream=None, qpass: bool = False) -> torch.Tensor:
    """Y[M, N] (FP32) = X[M, K] (BF16) @ W^T with W12 weights (qpass: the Q pass on the nested
    8-bit view, w12_gemm_q).

    ws: a workspace from gemm_workspace() (or any buffer of at least gemm_workspace_size bytes
    initialised once with gemm_workspace_init); one is allocated here when omitted.  With a
    stream, Y and the workspace allocated here belong to that stream."""
    _require_cuda(x)
    _bits16(x)
    m = x.shape[0]
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        if y is None:
            y = torch.empty(m, t.n, dtype=torch.float32, device=x.device)
        if ws is None:
            ws = gemm_workspace(m, t.n, t.k, x.device)
        wsb = 0 if ws is None else ws.numel() * ws.element_size()
        d = t.descriptor()
        name = "w12_gemm_q" if qpass else "w12_gemm"
        _check(name, getattr(lib(), name)(_ptr(x), m, _pitch(x), ctypes.byref(d), _ptr(y), _pitch(y), _ptr(ws), wsb,
                                          _stream()))
    return y


def gemm_noalloc(x: torch.Tensor, t: W12Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """w12_gemm_noalloc: the product of gemm() into a caller-provided Y, with the library's own
    per-device workspace (no device allocation)."""
    _require_cuda(x, y)
    _bits16(x)
    d = t.descriptor()
    _check("w12_gemm_noalloc", lib().w12_gemm_noalloc(_ptr(x), x.shape[0], _pitch(x), ctypes.byref(d), _ptr(y),
                                                       _pitch(y), _stream(stream)))
    return y


def read_probe(buf: torch.Tensor, nbytes: int, loads_per_lane: int, groups_per_cu: int, sink: torch.Tensor,
               offset: int = 0, stream=None) -> None:
    """A plain streaming read of nbytes bytes of buf starting at byte offset (w12_read_probe): the
    practical HBM read ceiling.  sink: a device buffer of at least groups_per_cu * CUs uint32."""
    _require_cuda(buf, sink)
    if offset < 0 or offset + nbytes > buf.numel() * buf.element_size():
        raise ValueError("read range outside the buffer")
    _check("w12_read_probe", lib().w12_read_probe(buf.data_ptr() + offset, nbytes, loads_per_lane, groups_per_cu,
                                                   _ptr(sink), _stream(stream)))


def bits_per_weight(n: int, k: int, e: int) -> float:
    return float(lib().w12_bits_per_weight(n, k, e))


def tensor_bytes(n: int, k: int, e: int) -> int:
    return int(lib().w12_tensor_bytes(n, k, e))


def _group_items(xs, ts, ys):
    """ctypes item array for a group (the descriptors are kept alive alongside it)."""
    n = len(ts)
    descs = [t.descriptor() for t in ts]
    items = (_GemmItem * max(n, 1))()
    for i in range(n):
        items[i].X = _ptr(xs[i])
        items[i].ldx = _pitch(xs[i])
        items[i].t = ctypes.pointer(descs[i])
        items[i].Y = _ptr(ys[i])
        items[i].ldy = _pitch(ys[i])
    return items, descs


def gemm_group_workspace_size(m: int, ts) -> int:
    descs = [t.descriptor() for t in ts]
    items = (_GemmItem * max(len(ts), 1))()
    for i, d in enumerate(descs):
        items[i].t = ctypes.pointer(d)
    b = _c_u64()
    _check("w12_gemm_group_workspace_size", lib().w12_gemm_group_workspace_size(m, len(ts), items, ctypes.byref(b)))
    return b.value


def gemm_group_workspace(m: int, ts, device="cuda", stream=None) -> torch.Tensor:
    """A ready-to-use (zero-initialised) workspace for gemm_group() with M=m on the tensors ts."""
    ws = torch.empty(gemm_group_workspace_size(m, ts), dtype=torch.uint8, device=device)
    gemm_workspace_init(ws, stream)
    return ws


def gemm_group(xs, ts, ys=None, ws: torch.Tensor | None = None, stream=None, qpass: bool = False):
    """Y_i = X_i @ W_i^T for independent products of one M in a single launch (w12_gemm_group,
    or w12_gemm_group_q with qpass).  Returns the list of Y_i (FP32 [M, N_i])."""
    if len(xs) != len(ts):
        raise ValueError("one X per tensor")
    _require_cuda(*xs)
    for x in xs:
        _bits16(x)
    m = xs[0].shape[0] if xs else 0
    if any(x.shape[0] != m for x in xs):
        raise ValueError("every X of a group has the same number of rows")
    with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
        if ys is None:
            ys = [torch.empty(m, t.n, dtype=torch.float32, device=xs[0].device) for t in ts]
        _require_cuda(*ys)
        if ws is None:
            ws = gemm_group_workspace(m, ts, xs[0].device)
        items, _descs = _group_items(xs, ts, ys)
        name = "w12_gemm_group_q" if qpass else "w12_gemm_group"
        _check(name, getattr(lib(), name)(m, len(ts), items, _ptr(ws), ws.numel() * ws.element_size(), _stream()))
    return ys


def _host_descriptor(n, k, e, base, hi, lo, esc_ptr, esc) -> _Tensor:
    d = _Tensor()
    d.N, d.K, d.layout, d.reserved, d.num_escapes = n, k, W12_LAYOUT_RB16_K16, 0, e
    d.base, d.hi, d.lo, d.esc_ptr = (a.ctypes.data for a in (base, hi, lo, esc_ptr))
    d.esc = esc.ctypes.data if e else None
    return d


def save(path: str, tensors: dict) -> None:
    """Write {name: W12Tensor} to a W12 checkpoint file (w12_file_write); the planes are copied
    to host memory first."""
    import numpy as np
    names = list(tensors)
    keep, descs = [], (_Tensor * len(names))()
    for i, nm in enumerate(names):
        t = tensors[nm]
        arrs = [x.cpu().contiguous().numpy() for x in (t.base, t.hi, t.lo, t.esc_ptr, t.esc)]
        arrs = [np.ascontiguousarray(a) for a in arrs]
        keep.append(arrs)
        descs[i] = _host_descriptor(t.n, t.k, t.num_escapes, arrs[0], arrs[1], arrs[2], arrs[3], arrs[4])
    cnames = (ctypes.c_char_p * len(names))(*[nm.encode() for nm in names])
    _check("w12_file_write", lib().w12_file_write(path.encode(), len(names), cnames, descs))


def file_index(path: str) -> list[dict]:
    """The index of a W12 checkpoint file (w12_file_index)."""
    n = _c_i32()
    _check("w12_file_index", lib().w12_file_index(path.encode(), ctypes.byref(n), None, 0))
    entries = (_FileEntry * max(n.value, 1))()
    _check("w12_file_index", lib().w12_file_index(path.encode(), ctypes.byref(n), entries, n.value))
    return [{"name": e.name.decode(), "n": e.N, "k": e.K, "num_escapes": e.num_escapes, "offset": e.offset,
             "bytes": e.bytes} for e in entries[:n.value]]


def load(path: str, refs: dict | None = None, device="cuda", staging: torch.Tensor | None = None,
         staging_bytes: int = 64 << 20, stream=None):
    """Stream every tensor of a W12 checkpoint file to the GPU (w12_file_load).  With refs
    ({name: BF16 [N, K] on the GPU}), the load-time bit-for-bit check of each named tensor is
    enqueued right after its copies.  Returns ({name: W12Tensor}, results) where results is an
    int64 [count, 2] device tensor of (mismatch count, first bad flat index) per tensor (zeros
    for tensors without a reference)."""
    idx = file_index(path)
    if staging is None:
        staging = torch.empty(staging_bytes, dtype=torch.uint8, pin_memory=True)
    out, descs = {}, (_Tensor * len(idx))()
    for i, e in enumerate(idx):
        base, hi, lo, esc_ptr = alloc_planes(e["n"], e["k"], device)
        esc = torch.empty(e["num_escapes"], dtype=torch.int32, device=device)
        t = W12Tensor(e["n"], e["k"], base, hi, lo, esc_ptr, esc)
        out[e["name"]] = t
        descs[i] = t.descriptor()
    which = (_c_i32 * len(idx))(*range(len(idx)))
    results = torch.zeros(len(idx), 2, dtype=torch.int64, device=device)
    refs_arr = ldr_arr = None
    keep = []
    if refs:
        refs_arr = (_c_p * len(idx))()
        ldr_arr = (_c_i64 * len(idx))()
        for i, e in enumerate(idx):
            r = refs.get(e["name"])
            if r is not None:
                _require_cuda(r)
                _bits16(r)
                keep.append(r)
                refs_arr[i] = r.data_ptr()
                ldr_arr[i] = _pitch(r)
    _check("w12_file_load", lib().w12_file_load(path.encode(), len(idx), which, descs, staging.data_ptr(),
                                                staging.numel(), refs_arr, ldr_arr, results.data_ptr(),
                                                _stream(stream)))
    return out, results
