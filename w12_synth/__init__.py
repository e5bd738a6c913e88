"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module holds only random-number recipes and shapes.  It contains none of the
W12 arithmetic (no exponent windows, records, escapes or GEMM): both the CPU oracle
and the HIP path receive the BF16 bit patterns produced here and nothing else.

Every tensor is generated on the host with a seeded ``torch.Generator`` (CPU), so the
bits do not depend on the GPU, and is returned as a numpy ``uint16`` array of raw
BF16 bit patterns (row-major).  The one exception is ``layer_device``, the same layer
recipe drawn on the GPU for the 64-layer timing run.  ``to_bf16`` rounds float32 to BF16 with
round-to-nearest-even through ``torch.Tensor.to(torch.bfloat16)``.

Recipes (the pages give no weights, so these stand in for the dense 27B-class
target layers they evaluate on):

* layer matrices  W = bf16(0.02 * s_n * Z), Z ~ N(0,1) [N,K], s_n ~ lognormal(0, 0.5)
  per output channel, then round(1e-4 * N * K) positions (drawn with replacement)
  set to +0.
* tiny case       W = bf16(0.02 * Z) [256,512], then disjoint random positions set
  to +0 (0.5%), to BF16 denormals (0.1%), multiplied by 2^12 (0.1%) and to
  +inf, -inf, +inf, -inf.
* heavy tail      W = bf16(0.02 * t3), t3 = Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3), then
  2% of positions replaced by +-2^j * (1 + f/128), j uniform in 12..19,
  f uniform in 0..127.
* activations     X = bf16(Z) [M,K].
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np
import torch

# Shapes of one 27B-class dense decoder layer with hidden size 5120.
LAYER_SHAPES = {
    "qkv": (7168, 5120),
    "o_proj": (5120, 5120),
    "gate_up": (34816, 5120),
    "down": (5120, 17408),
}
LAYER_ORDER = ("qkv", "o_proj", "gate_up", "down")

TREE_M_SWEEP = (1, 8, 24, 32, 63, 64)
BATCHED_M = (256, 512)
FULL_MODEL_LAYERS = 64


def to_bf16_bits(x: torch.Tensor) -> np.ndarray:
    """float32 tensor -> BF16 (round to nearest even) -> raw uint16 bit patterns."""
    b = x.to(torch.bfloat16).contiguous()
    return b.view(torch.int16).numpy().view(np.uint16)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def layer_matrix(gen: torch.Generator, n: int, k: int, zero_frac: float = 1e-4) -> np.ndarray:
    """Gaussian x per-channel lognormal(0, 0.5) scale, with a few exact zeros."""
    z = torch.randn(n, k, generator=gen)
    s = torch.exp(0.5 * torch.randn(n, 1, generator=gen))
    w = to_bf16_bits(0.02 * s * z)
    nz = int(round(zero_frac * n * k))
    if nz:
        pos = torch.randint(0, n * k, (nz,), generator=gen).numpy()
        w.reshape(-1)[pos] = 0x0000
    return w


def layer(seed: int, which=LAYER_ORDER) -> dict:
    """One decoder layer's four matrices drawn in the fixed order qkv, o_proj, gate_up, down.

    Matrices not in ``which`` are still drawn (and discarded) so that every matrix of a
    layer has the same bits whichever subset is asked for.
    """
    gen = torch.Generator().manual_seed(seed)
    out = {}
    for name in LAYER_ORDER:
        n, k = LAYER_SHAPES[name]
        w = layer_matrix(gen, n, k)
        if name in which:
            out[name] = w
    return out


def tiny_weights(seed: int = 0, n: int = 256, k: int = 512) -> np.ndarray:
    """The tiny round-trip case: Gaussian weights with zeros, denormals, outliers and infs."""
    gen = torch.Generator().manual_seed(seed)
    w = to_bf16_bits(0.02 * torch.randn(n, k, generator=gen))
    flat = w.reshape(-1)
    total = n * k
    perm = torch.randperm(total, generator=gen).numpy()
    n_zero = int(round(0.005 * total))
    n_den = int(round(0.001 * total))
    n_out = int(round(0.001 * total))
    i = 0
    flat[perm[i:i + n_zero]] = 0x0000
    i += n_zero
    den_pos = perm[i:i + n_den]
    i += n_den
    sign = torch.randint(0, 2, (n_den,), generator=gen).numpy().astype(np.uint16)
    mant = torch.randint(1, 128, (n_den,), generator=gen).numpy().astype(np.uint16)
    flat[den_pos] = (sign << 15) | mant
    out_pos = perm[i:i + n_out]
    i += n_out
    # multiply by 2^12 exactly: add 12 to the exponent field (values stay normal and finite)
    flat[out_pos] = flat[out_pos] + np.uint16(12 << 7)
    inf_pos = perm[i:i + 4]
    flat[inf_pos] = np.array([0x7F80, 0xFF80, 0x7F80, 0xFF80], dtype=np.uint16)
    return w


def heavy_tail_weights(seed: int, n: int, k: int, outlier_frac: float = 0.02) -> np.ndarray:
    """Student-t (nu=3) weights at scale 0.02 plus 2% values 12..19 binades above the bulk."""
    gen = torch.Generator().manual_seed(seed)
    z0 = torch.randn(n, k, generator=gen)
    chi = torch.zeros(n, k)
    for _ in range(3):
        zi = torch.randn(n, k, generator=gen)
        chi += zi * zi
    t3 = z0 / torch.sqrt(chi / 3.0)
    w = to_bf16_bits(0.02 * t3)
    flat = w.reshape(-1)
    total = n * k
    n_out = int(round(outlier_frac * total))
    pos = torch.randint(0, total, (n_out,), generator=gen).numpy()
    j = torch.randint(12, 20, (n_out,), generator=gen).numpy().astype(np.uint16)
    f = torch.randint(0, 128, (n_out,), generator=gen).numpy().astype(np.uint16)
    s = torch.randint(0, 2, (n_out,), generator=gen).numpy().astype(np.uint16)
    # value = (-1)^s * 2^j * (1 + f/128): exponent field 127 + j, mantissa f
    flat[pos] = (s << 15) | ((127 + j) << 7) | f
    return w


def activations(m: int, k: int, seed: int) -> np.ndarray:
    gen = torch.Generator().manual_seed(seed)
    return to_bf16_bits(torch.randn(m, k, generator=gen))


def x_seed(m: int, k: int) -> int:
    return 10000 + 100000 * int(k == 17408) + m


@dataclass(frozen=True)
class Case:
    name: str
    n: int
    k: int
    m: int


def config_cases() -> dict:
    """The five synthetic configurations, as (matrix, M) cases."""
    cases = {
        "tiny": [Case("tiny", 256, 512, 1)],
        "layer_m16": [Case(nm, *LAYER_SHAPES[nm], 16) for nm in LAYER_ORDER],
        "tree_sweep": [Case(nm, *LAYER_SHAPES[nm], m) for nm in ("gate_up", "down") for m in TREE_M_SWEEP],
        "full_model_m32": [Case(nm, *LAYER_SHAPES[nm], 32) for nm in LAYER_ORDER],
        "batched": [Case(nm, *LAYER_SHAPES[nm], m) for nm in ("gate_up", "down") for m in BATCHED_M],
    }
    return cases


def random_bits_matrix(gen: np.random.Generator, n: int, k: int, kind: str = "gauss") -> np.ndarray:
    """Small assorted test matrices (raw BF16 bits) for property tests."""
    if kind == "gauss":
        x = torch.from_numpy(gen.standard_normal((n, k)).astype(np.float32) * 0.02)
        return to_bf16_bits(x)
    if kind == "uniform_bits":
        return gen.integers(0, 1 << 16, size=(n, k), dtype=np.uint16)
    if kind == "wide":
        # exponents spread over ~40 binades around 1.0, some zeros
        e = gen.integers(107, 147, size=(n, k)).astype(np.uint16)
        m = gen.integers(0, 128, size=(n, k)).astype(np.uint16)
        s = gen.integers(0, 2, size=(n, k)).astype(np.uint16)
        w = (s << 15) | (e << 7) | m
        w[gen.random((n, k)) < 0.01] = 0
        return w.astype(np.uint16)
    raise ValueError(kind)


def layer_device(seed: int, device) -> dict:
    """The layer recipe drawn on the GPU's own generator, for the full-model stream.

    Same shapes, order and distributions as ``layer`` (Gaussian x per-channel lognormal(0, 0.5)
    scale, round(1e-4 N K) exact zeros), but the bits come from the device generator, so they
    differ from the host recipe's.  Drawing 64 layers on the host would take minutes; the
    parity tests check sampled host-drawn layers of the same recipe.  Returns int16 tensors of
    raw BF16 bits on ``device``.
    """
    gen = torch.Generator(device=device).manual_seed(seed)
    out = {}
    for name in LAYER_ORDER:
        n, k = LAYER_SHAPES[name]
        z = torch.randn(n, k, generator=gen, device=device)
        s = torch.exp(0.5 * torch.randn(n, 1, generator=gen, device=device))
        z.mul_(s).mul_(0.02)
        w = z.to(torch.bfloat16).view(torch.int16)
        del z
        nz = int(round(1e-4 * n * k))
        pos = torch.randint(0, n * k, (nz,), generator=gen, device=device)
        w.view(-1)[pos] = 0
        out[name] = w
    return out
