"""Seeded synthetic inputs for the Q4_K linear layer.

This module is shared by the tests, the smoke check and the benchmark, on both
sides of every parity check (the HIP path and the oracle).  It holds none of
the method's arithmetic: it never decodes a block, never dequantizes and never
multiplies a weight.  It only draws bytes and numbers.

Distributions (the workload of the pages: 4-bit quants uniform in 0..15,
6-bit sub-block scales and mins uniform in 0..63, fp16 super-block scales
d and dmin = |N(0,1)| * 0.01, activations N(0,1)):

* A super-block is 144 bytes: fp16 ``d`` at byte 0, fp16 ``dmin`` at byte 2,
  then 12 scale bytes and 128 quant bytes.  The 140 scale and quant bytes are
  drawn uniformly from 0..255.  Every bit of them is then an independent fair
  coin, so *any* 6-bit field is uniform in 0..63 and any 4-bit field uniform
  in 0..15 -- whatever packing a reader applies.  The generator therefore
  needs no knowledge of how the scales are packed.
* ``d`` and ``dmin`` are |N(0,1)| * 0.01 drawn in fp64 and rounded to fp16
  (round to nearest even, numpy's conversion).  About 0.5% of them land in
  the fp16 subnormal range; they are kept.
* Activations are fp32 N(0,1); bf16 activations are the fp32 draw rounded to
  bf16 (round to nearest even, torch's conversion).

A Q5_K super-block (176 bytes) is drawn the same way: fp16 ``d`` and ``dmin`` at
bytes 0 and 2, the other 172 bytes uniform.  A Q6_K block (210 bytes) has its
208 quant and scale bytes uniform (6-bit quants uniform in 0..63, signed 8-bit
sub-block scales uniform in -128..127) and fp16 ``d`` = |N(0,1)| * 1e-4 at byte
208, so weights have a spread like the Q4_K draws.  A Q3_K block (110 bytes) has
its 108 quant and scale bytes uniform and fp16 ``d`` = |N(0,1)| * 1e-3 at byte
108.

INT8 W8A8 inputs (the INT8 linear layer of the xpu-kernels page): int8 codes
are a normal draw with standard deviation 32, rounded and clipped to
[-127, 127] (the spread of per-row absmax codes of Gaussian rows at k in the
thousands); activation row scales are uniform in [0.01, 0.05], weight row
scales uniform in [2e-4, 1e-3] (absmax / 127 of N(0,1) activations and of
N(0, 0.02) weights) and the bias is N(0, 0.1), all fp32.  ``int8_uniform``
draws codes uniformly from the whole int8 range, -128 included, for extremes.

Random streams come from numpy's PCG64 seeded with ``SeedSequence([seed,
stream])``, so every tensor of a case has its own independent stream and a
case is reproducible from ``seed`` alone.
"""
from __future__ import annotations

import numpy as np

QK = 256            # weights per super-block
BLOCK_BYTES = 144   # bytes per Q4_K super-block
Q5K_BLOCK_BYTES = 176  # bytes per Q5_K super-block (Q4_K plus 32 high-bit bytes)
Q6K_BLOCK_BYTES = 210  # bytes per Q6_K block
Q3K_BLOCK_BYTES = 110  # bytes per Q3_K block

# stream ids: one per tensor role, so cases never share draws
W, X, W_GATE, W_UP, W_DOWN = 0, 1, 2, 3, 4
X_SCALE, W_SCALE, BIAS = 5, 6, 7


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(stream)])))


def q4k_weights(n: int, k: int, seed: int = 0, stream: int = W,
                scale: float = 0.01) -> np.ndarray:
    """Random Q4_K matrix W [n, k] as uint8 [n, (k/256)*144] (row-major blocks)."""
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nb = n * (k // QK)
    g = rng(seed, stream)
    blocks = np.empty((nb, BLOCK_BYTES), np.uint8)
    d = (np.abs(g.standard_normal(nb)) * scale).astype(np.float16)
    dmin = (np.abs(g.standard_normal(nb)) * scale).astype(np.float16)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    blocks[:, 4:] = g.integers(0, 256, size=(nb, BLOCK_BYTES - 4), dtype=np.uint8)
    return blocks.reshape(n, (k // QK) * BLOCK_BYTES)


def q5k_weights(n: int, k: int, seed: int = 0, stream: int = W,
                scale: float = 0.01) -> np.ndarray:
    """Random Q5_K matrix W [n, k] as uint8 [n, (k/256)*176]: fp16 d and dmin as for Q4_K,
    the other 172 bytes (scales, high bits, nibbles) uniform, so every 5-bit quant is
    uniform in 0..31 whatever the packing."""
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nb = n * (k // QK)
    g = rng(seed, stream)
    blocks = np.empty((nb, Q5K_BLOCK_BYTES), np.uint8)
    d = (np.abs(g.standard_normal(nb)) * scale).astype(np.float16)
    dmin = (np.abs(g.standard_normal(nb)) * scale).astype(np.float16)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    blocks[:, 4:] = g.integers(0, 256, size=(nb, Q5K_BLOCK_BYTES - 4), dtype=np.uint8)
    return blocks.reshape(n, (k // QK) * Q5K_BLOCK_BYTES)


def q6k_weights(n: int, k: int, seed: int = 0, stream: int = W,
                scale: float = 1e-4) -> np.ndarray:
    """Random Q6_K matrix W [n, k] as uint8 [n, (k/256)*210]: 208 uniform bytes and an fp16
    d per block."""
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nb = n * (k // QK)
    g = rng(seed, stream)
    blocks = np.empty((nb, Q6K_BLOCK_BYTES), np.uint8)
    blocks[:, :208] = g.integers(0, 256, size=(nb, 208), dtype=np.uint8)
    d = (np.abs(g.standard_normal(nb)) * scale).astype(np.float16)
    blocks[:, 208:210] = d.view(np.uint8).reshape(nb, 2)
    return blocks.reshape(n, (k // QK) * Q6K_BLOCK_BYTES)


def q3k_weights(n: int, k: int, seed: int = 0, stream: int = W,
                scale: float = 1e-3) -> np.ndarray:
    """Random Q3_K matrix W [n, k] as uint8 [n, (k/256)*110]: 108 uniform bytes and an fp16
    d per block."""
    if k % QK:
        raise ValueError("k must be a multiple of 256")
    nb = n * (k // QK)
    g = rng(seed, stream)
    blocks = np.empty((nb, Q3K_BLOCK_BYTES), np.uint8)
    blocks[:, :108] = g.integers(0, 256, size=(nb, 108), dtype=np.uint8)
    d = (np.abs(g.standard_normal(nb)) * scale).astype(np.float16)
    blocks[:, 108:110] = d.view(np.uint8).reshape(nb, 2)
    return blocks.reshape(n, (k // QK) * Q3K_BLOCK_BYTES)


def normal_f32(shape, seed: int = 0, stream: int = X) -> np.ndarray:
    """fp32 N(0,1) array."""
    return rng(seed, stream).standard_normal(shape, dtype=np.float32)


def bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 (nearest even) and return the uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, seed: int = 0, stream: int = X) -> np.ndarray:
    """bf16 bits of fp32 N(0,1) draws."""
    return bf16_bits(normal_f32(shape, seed, stream))


def int8_codes(shape, seed: int = 0, stream: int = X, std: float = 32.0) -> np.ndarray:
    """int8 codes: rint(N(0, std)) clipped to [-127, 127]."""
    v = np.rint(rng(seed, stream).standard_normal(shape) * std)
    return np.clip(v, -127, 127).astype(np.int8)


def int8_uniform(shape, seed: int = 0, stream: int = X) -> np.ndarray:
    """int8 codes uniform over -128..127."""
    return rng(seed, stream).integers(-128, 128, size=shape, dtype=np.int8)


def uniform_f32(shape, lo: float, hi: float, seed: int = 0, stream: int = X_SCALE) -> np.ndarray:
    """fp32 uniform in [lo, hi)."""
    return rng(seed, stream).uniform(lo, hi, size=shape).astype(np.float32)


def w8a8_case(m: int, n: int, k: int, seed: int = 0):
    """(x int8 [m,k], x_scale [m], w int8 [n,k], w_scale [n], bias [n]) of one seeded case."""
    x = int8_codes((m, k), seed, X)
    w = int8_codes((n, k), seed, W)
    xs = uniform_f32((m,), 0.01, 0.05, seed, X_SCALE)
    ws = uniform_f32((n,), 2e-4, 1e-3, seed, W_SCALE)
    bias = (rng(seed, BIAS).standard_normal(n) * 0.1).astype(np.float32)
    return x, xs, w, ws, bias
