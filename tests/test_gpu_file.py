"""GPU: W12 checkpoint round trip and the streamed load with the load-time check overlapped.

Encoded tensors written with save() and streamed back with load() (staging buffers from a
few hundred bytes up, so tensors cross many staging halves) have identical planes, decode to
their BF16 sources bit for bit, and the checks enqueued during the load report no mismatch.
A flipped byte in a file's record plane is caught by the load-time check."""
import numpy as np
import pytest
import torch

import lossless_bit_weight_encode_amd as w12
import w12_synth as S
from gpu_util import say, to_dev, u16

pytestmark = pytest.mark.gpu


def _sources():
    return {
        "tiny": S.tiny_weights(0),
        "gauss": S.layer_matrix(torch.Generator().manual_seed(5), 300, 4096),
        "heavy": S.heavy_tail_weights(1000, 64, 2048),
        "zeros": np.zeros((20, 96), dtype=np.uint16),
        "ragged": S.random_bits_matrix(np.random.default_rng(3), 17, 33, "wide"),
        "no_escapes": S.to_bf16_bits(1.0 + torch.rand(32, 256, generator=torch.Generator().manual_seed(8))),
    }


@pytest.mark.parametrize("staging", [512, 4096, 1 << 20])
def test_save_load_roundtrip_with_overlapped_check(tmp_path, staging):
    src = _sources()
    dev = {nm: to_dev(w, (w.shape[1] + 7) // 8 * 8) for nm, w in src.items()}
    enc = {nm: w12.encode(d) for nm, d in dev.items()}
    path = str(tmp_path / "layer.w12")
    w12.save(path, enc)
    say(f"[file] staging={staging}")
    st = torch.empty(staging, dtype=torch.uint8, pin_memory=True)
    got, res = w12.load(path, refs=dev, staging=st)
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [[0, -1]] * len(src)
    for nm, t in enc.items():
        g = got[nm]
        for a, b in ((t.base, g.base), (t.hi, g.hi), (t.lo, g.lo), (t.esc_ptr, g.esc_ptr), (t.esc, g.esc)):
            assert torch.equal(a, b), nm
        assert np.array_equal(u16(w12.decode(g)), src[nm])


def test_load_time_check_catches_corruption(tmp_path):
    src = _sources()
    dev = {nm: to_dev(w, (w.shape[1] + 7) // 8 * 8) for nm, w in src.items()}
    enc = {nm: w12.encode(d) for nm, d in dev.items()}
    path = tmp_path / "layer.w12"
    w12.save(str(path), enc)
    idx = {e["name"]: e for e in w12.file_index(str(path))}
    e = idx["gauss"]
    n = e["n"]
    hi_off = e["offset"] + sum(((b + 255) // 256) * 256 for b in (n, 4 * (n + 1), 4 * e["num_escapes"]))
    raw = bytearray(path.read_bytes())
    raw[hi_off + 1000] ^= 0x10
    path.write_bytes(bytes(raw))
    got, res = w12.load(str(path), refs=dev, staging_bytes=1 << 16)
    torch.cuda.synchronize()
    r = dict(zip(idx, res.cpu().tolist()))
    assert r["gauss"][0] == 1
    assert all(v == [0, -1] for nm, v in r.items() if nm != "gauss")


@pytest.mark.timeout(600)
def test_layer_file_full_size(tmp_path):
    """One dense decoder layer (495 MB of W12) through a file and back, checked at load."""
    lay = S.layer(0)
    dev = {nm: to_dev(lay[nm]) for nm in S.LAYER_ORDER}
    enc = {nm: w12.encode(dev[nm]) for nm in S.LAYER_ORDER}
    path = str(tmp_path / "layer0.w12")
    w12.save(path, enc)
    got, res = w12.load(path, refs=dev)
    torch.cuda.synchronize()
    assert res.cpu().tolist() == [[0, -1]] * 4
    for nm in S.LAYER_ORDER:
        assert torch.equal(got[nm].hi, enc[nm].hi) and torch.equal(got[nm].esc, enc[nm].esc)
