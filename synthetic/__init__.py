"""Seeded synthetic inputs shaped like Llama-3.1-8B linear layers.

This module is shared by the tests, the benchmark and the oracle's callers.
It draws random numbers and rounds them to bf16; it holds none of the
method's arithmetic (no rotation, no scaling, no quantization).

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64, in the
order listed; normal draws are numpy's float32 ziggurat
(``standard_normal(dtype=float32)`` times sigma in fp32), the other
distributions are drawn in fp64 and rounded to fp32; every tensor is then
rounded to bf16 with round-to-nearest-even; row-major):

=====  ====  =============================================================
name   seed  tensors
=====  ====  =============================================================
tiny   0     X = normal(128x256); W = normal(256x256);
             idx = choice(256, 5, replace=False); X[:, idx] *= 40
quant  1     A = standard_t(3, 8192x4096) * lognormal(0, 1, 4096)[None, :]
qkv    2     Z = normal(8192x4096); idx = choice(4096, 41, replace=False);
             Z[:, idx] *= 50; X = Z / rms(Z, per row);
             W = normal(0, 0.02, 6144x4096)
mlp    3     X as in qkv; W_gu = normal(0, 0.02, 28672x4096);
             dY = normal(0, 1e-4, 8192x4096), dY[random(8192x4096) < 1e-3] *= 100;
             W_down = normal(0, 0.02, 4096x14336)
wgrad  4     dY as in mlp (8192x4096);
             X = silu(normal(8192x14336)) * |standard_cauchy(8192x14336)|
=====  ====  =============================================================

The five workloads stand in for Llama 3.1-8B pretraining on C4 (the data
set and the trained weights are not available): hidden 4096, fused QKV
6144, MLP intermediate 14336 (gate+up 28672), 8192 tokens.

Every function returns bf16 bit patterns as ``numpy.uint16`` arrays.
``scale`` shrinks the token count (rows of X / dY) and the weight rows for
quick tests while keeping the recipe; ``scale=1`` is the full workload.
"""
from __future__ import annotations

import numpy as np

__all__ = ["f64_to_bf16_bits", "bf16_bits_to_f32", "make", "WORKLOADS", "random_signs",
           "random_u32"]


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64/fp32 -> fp32 (RNE) -> bf16 (RNE) bit patterns. Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    sixteen = np.uint32(16)
    lsb = np.bitwise_and(np.right_shift(u, sixteen), np.uint32(1))
    return np.right_shift(u + np.uint32(0x7FFF) + lsb, sixteen).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return np.left_shift(np.asarray(b, dtype=np.uint16).astype(np.uint32),
                         np.uint32(16)).view(np.float32)


def _normal(rng, shape, sigma=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def _rms_rows_with_outliers(rng, t, k, frac_count, factor):
    z = _normal(rng, (t, k)).astype(np.float64)
    idx = rng.choice(k, frac_count, replace=False)
    z[:, idx] *= factor
    rms = np.sqrt(np.mean(z * z, axis=1, keepdims=True))
    return z / rms


def _grad_with_spikes(rng, t, n):
    g = _normal(rng, (t, n), 1e-4)
    mask = rng.random((t, n)) < 1e-3
    g[mask] *= np.float32(100.0)
    return g


def make(name: str, scale: int = 1) -> dict:
    """Return the named workload's tensors as bf16 bits (uint16 arrays).

    ``scale`` divides the token axis (and, for the big weights, the output
    axis) so that tests can run the same recipe at a fraction of the size.
    Reduction axes that the method blocks (multiples of 32) stay valid.
    """
    if name == "tiny":
        rng = np.random.default_rng(0)
        x = _normal(rng, (128, 256)).astype(np.float64)
        w = _normal(rng, (256, 256))
        idx = rng.choice(256, 5, replace=False)
        x[:, idx] *= 40.0
        return {"X": f64_to_bf16_bits(x), "W": f64_to_bf16_bits(w)}
    if name == "quant":
        rng = np.random.default_rng(1)
        r, c = 8192 // scale, 4096
        a = rng.standard_t(3, size=(r, c)) * rng.lognormal(0.0, 1.0, size=c)[None, :]
        return {"A": f64_to_bf16_bits(a)}
    if name == "qkv":
        rng = np.random.default_rng(2)
        t, k, n = 8192 // scale, 4096, 6144 // scale
        x = _rms_rows_with_outliers(rng, t, k, 41, 50.0)
        w = _normal(rng, (n, k), 0.02)
        return {"X": f64_to_bf16_bits(x), "W": f64_to_bf16_bits(w)}
    if name == "mlp":
        rng = np.random.default_rng(3)
        t, k, ngu, ni = 8192 // scale, 4096, 28672 // scale, 14336 // scale
        x = _rms_rows_with_outliers(rng, t, k, 41, 50.0)
        out = {"X": f64_to_bf16_bits(x)}
        del x
        out["W_gu"] = f64_to_bf16_bits(_normal(rng, (ngu, k), 0.02))
        out["dY"] = f64_to_bf16_bits(_grad_with_spikes(rng, t, k))
        out["W_down"] = f64_to_bf16_bits(_normal(rng, (k, ni), 0.02))
        return out
    if name == "wgrad":
        rng = np.random.default_rng(4)
        t, n, k = 8192 // scale, 4096, 14336 // scale
        out = {"dY": f64_to_bf16_bits(_grad_with_spikes(rng, t, n))}
        g = _normal(rng, (t, k))
        silu = g / (np.float32(1.0) + np.exp(-g))
        del g
        silu *= np.abs(rng.standard_cauchy(size=(t, k))).astype(np.float32)
        out["X"] = f64_to_bf16_bits(silu)
        return out
    raise KeyError(name)


# (T, N, K) of each product at full size; N and K follow Y = X W^T with
# X [T x K], W [N x K].
WORKLOADS = {
    "tiny_fprop": ("tiny", "fprop", 128, 256, 256),
    "qkv_fprop": ("qkv", "fprop", 8192, 6144, 4096),
    "mlp_gateup_fprop": ("mlp", "fprop", 8192, 28672, 4096),
    "mlp_down_dgrad": ("mlp", "dgrad", 8192, 4096, 14336),
    "down_wgrad": ("wgrad", "wgrad", 8192, 4096, 14336),
}


def random_signs(n: int, seed: int) -> np.ndarray:
    """n sign flags (uint8 0 or 1, equally likely) for the random-sign
    Hadamard comparison arm: ``default_rng(seed).integers(0, 2, n)``."""
    return np.random.default_rng(seed).integers(0, 2, size=n, dtype=np.uint8)


def random_u32(shape, seed: int) -> np.ndarray:
    """Uniform 32-bit integers (uint32) for the stochastic-rounding arm:
    ``default_rng(seed).integers(0, 2**32, shape)``."""
    return np.random.default_rng(seed).integers(0, 2 ** 32, size=shape, dtype=np.uint32)
