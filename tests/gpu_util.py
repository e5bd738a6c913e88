"""Helpers for the GPU tests: move BF16 bit patterns between numpy and the GPU, and pull
the encoded arrays back for comparison with the oracle."""
import sys

import numpy as np
import torch

import lossless_bit_weight_encode_amd as w12


def say(*a):
    print(*a, file=sys.__stderr__, flush=True)


def to_dev(a: np.ndarray, ld: int | None = None) -> torch.Tensor:
    """uint16 [R, C] -> int16 CUDA tensor, optionally with a row pitch ld >= C."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    r, c = a.shape
    if ld is None or ld == c:
        return torch.from_numpy(a.view(np.int16)).cuda()
    buf = torch.full((r, ld), 0x7FC1, dtype=torch.int16)   # NaN-pattern filler in the pitch gap
    buf[:, :c] = torch.from_numpy(a.view(np.int16))
    return buf.cuda()[:, :c]


def u16(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().contiguous().numpy().view(np.uint16)


def u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def encoded_arrays(t: w12.W12Tensor) -> dict:
    torch.cuda.synchronize()
    return {
        "base": t.base.cpu().numpy(),
        "esc_ptr": u32(t.esc_ptr),
        "esc": u32(t.esc) if t.num_escapes else np.zeros(0, np.uint32),
        "rec": u16(w12.unpack_records(t)),
    }


def assert_encode_equal(t: w12.W12Tensor, ref) -> None:
    got = encoded_arrays(t)
    assert np.array_equal(got["base"], ref.base), "window bases differ"
    assert np.array_equal(got["esc_ptr"], ref.esc_ptr), "escape pointers differ"
    assert t.num_escapes == ref.num_escapes
    assert np.array_equal(got["esc"], ref.esc), "escape lists differ"
    assert np.array_equal(got["rec"], ref.rec), "records differ"
