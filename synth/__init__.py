"""Seeded synthetic inputs in canonical GGUF block bytes.

This module only draws random numbers and lays them out in the GGUF Q8_0 /
Q4_0 block byte format. It holds none of the arithmetic of the method (no
dequantisation, no dot products, no quantiser): both the fp64 oracle and the
HIP library consume what it returns, and neither imports the other.

Block byte layout (GGUF, little-endian), the layout the pages describe:
  * Q8_0: 2-byte IEEE binary16 scale ``d``, then 32 int8 quants
    (34 bytes per 32 weights);
  * Q4_0: 2-byte binary16 scale ``d``, then 16 bytes holding 32 4-bit quants
    (18 bytes per 32 weights; "Gem native architecture" page, section
    "M4 Max operating assumptions").

Draw order (fixed; a fresh ``numpy.random.default_rng(seed)`` per workload):
weights' quant bytes first, then the weight scales, then the activations.
Q4_0 quant bytes are drawn as uniform bytes 0..255, which makes both nibbles
of every byte independent and uniform on 0..15.
"""
from __future__ import annotations

import numpy as np

QK = 32
TYPE_Q4_0 = 2
TYPE_Q8_0 = 8

Q8_0_BLOCK = np.dtype([("d", "<u2"), ("qs", "i1", (32,))])
Q4_0_BLOCK = np.dtype([("d", "<u2"), ("qs", "u1", (16,))])
assert Q8_0_BLOCK.itemsize == 34 and Q4_0_BLOCK.itemsize == 18

# K-quant super-blocks of 256 elements (GGUF layout; the pages give only the
# arithmetic, see the oracle's header): Q4_K = binary16 d, binary16 dmin,
# 12 bytes of packed 6-bit sub-block scales and minimums, 128 quant bytes;
# Q5_K = the same header, 32 bytes of fifth quant bits, 128 quant bytes;
# Q6_K = 128 bytes of low quant bits, 64 bytes of high bits, 16 int8 scales,
# binary16 d.
QK_K = 256
TYPE_Q4_K = 12
TYPE_Q5_K = 13
TYPE_Q6_K = 14
Q4_K_BLOCK = np.dtype([("d", "<u2"), ("dmin", "<u2"), ("scales", "u1", (12,)), ("qs", "u1", (128,))])
Q5_K_BLOCK = np.dtype([("d", "<u2"), ("dmin", "<u2"), ("scales", "u1", (12,)), ("qh", "u1", (32,)),
                       ("qs", "u1", (128,))])
Q6_K_BLOCK = np.dtype([("ql", "u1", (128,)), ("qh", "u1", (64,)), ("scales", "i1", (16,)), ("d", "<u2")])
assert Q4_K_BLOCK.itemsize == 144 and Q5_K_BLOCK.itemsize == 176 and Q6_K_BLOCK.itemsize == 210

BLOCK_DTYPE = {TYPE_Q8_0: Q8_0_BLOCK, TYPE_Q4_0: Q4_0_BLOCK, TYPE_Q4_K: Q4_K_BLOCK, TYPE_Q5_K: Q5_K_BLOCK,
               TYPE_Q6_K: Q6_K_BLOCK}


def block_dtype(qtype: int) -> np.dtype:
    return BLOCK_DTYPE[qtype]


def as_bytes(blocks: np.ndarray) -> np.ndarray:
    """View an (n, k/32) structured block array as its raw uint8 bytes."""
    return np.ascontiguousarray(blocks).view(np.uint8).reshape(blocks.shape[0], -1)


def fp16_scales(rng, shape, lo=1e-3, hi=1e-2) -> np.ndarray:
    """Uniform scales in [lo, hi), rounded to binary16, returned as raw bits."""
    return rng.uniform(lo, hi, size=shape).astype(np.float16).view(np.uint16)


def q8_0_weights(rng, n: int, k: int, dist: str = "uniform", chunk_rows: int = 4096,
                 scale_lo=1e-3, scale_hi=1e-2) -> np.ndarray:
    """(n, k/32) Q8_0 blocks.

    dist="uniform": int8 quants uniform on [-127, 127].
    dist="normal40": quants round(N(0, 40)) clipped to [-127, 127], drawn in
    ``chunk_rows`` row chunks from the same stream (bounded host memory).
    """
    assert k % QK == 0
    nb = k // QK
    blocks = np.empty((n, nb), dtype=Q8_0_BLOCK)
    if dist == "uniform":
        blocks["qs"] = rng.integers(-127, 128, size=(n, nb, QK), dtype=np.int8)
    elif dist == "normal40":
        for r0 in range(0, n, chunk_rows):
            r1 = min(n, r0 + chunk_rows)
            v = rng.normal(0.0, 40.0, size=(r1 - r0, nb, QK))
            np.rint(v, out=v)
            np.clip(v, -127, 127, out=v)
            blocks["qs"][r0:r1] = v.astype(np.int8)
    else:
        raise ValueError(dist)
    blocks["d"] = fp16_scales(rng, (n, nb), scale_lo, scale_hi)
    return blocks


def q4_0_weights(rng, n: int, k: int, scale_lo=1e-3, scale_hi=1e-2) -> np.ndarray:
    """(n, k/32) Q4_0 blocks: uniform quant bytes, uniform binary16 scales."""
    assert k % QK == 0
    nb = k // QK
    blocks = np.empty((n, nb), dtype=Q4_0_BLOCK)
    blocks["qs"] = rng.integers(0, 256, size=(n, nb, 16), dtype=np.uint8)
    blocks["d"] = fp16_scales(rng, (n, nb), scale_lo, scale_hi)
    return blocks


def q4_k_weights(rng, n: int, k: int, scale_lo=1e-4, scale_hi=3e-4) -> np.ndarray:
    """(n, k/256) Q4_K super-blocks: uniform quant bytes (both nibbles uniform
    on 0..15), uniform bytes for the 12 packed scale/min bytes (every 6-bit
    field uniform on 0..63), then binary16 d and dmin uniform in
    [scale_lo, scale_hi] (so d sc and dmin m stay below about 0.02)."""
    assert k % QK_K == 0
    nsb = k // QK_K
    blocks = np.empty((n, nsb), dtype=Q4_K_BLOCK)
    blocks["qs"] = rng.integers(0, 256, size=(n, nsb, 128), dtype=np.uint8)
    blocks["scales"] = rng.integers(0, 256, size=(n, nsb, 12), dtype=np.uint8)
    blocks["d"] = fp16_scales(rng, (n, nsb), scale_lo, scale_hi)
    blocks["dmin"] = fp16_scales(rng, (n, nsb), scale_lo, scale_hi)
    return blocks


def q5_k_weights(rng, n: int, k: int, scale_lo=1e-4, scale_hi=2e-4) -> np.ndarray:
    """(n, k/256) Q5_K super-blocks: uniform quant bytes and fifth-bit bytes
    (every 5-bit quant uniform on 0..31), uniform bytes for the 12 packed
    scale/min bytes, then binary16 d and dmin uniform in [scale_lo,
    scale_hi]."""
    assert k % QK_K == 0
    nsb = k // QK_K
    blocks = np.empty((n, nsb), dtype=Q5_K_BLOCK)
    blocks["qs"] = rng.integers(0, 256, size=(n, nsb, 128), dtype=np.uint8)
    blocks["qh"] = rng.integers(0, 256, size=(n, nsb, 32), dtype=np.uint8)
    blocks["scales"] = rng.integers(0, 256, size=(n, nsb, 12), dtype=np.uint8)
    blocks["d"] = fp16_scales(rng, (n, nsb), scale_lo, scale_hi)
    blocks["dmin"] = fp16_scales(rng, (n, nsb), scale_lo, scale_hi)
    return blocks


def q6_k_weights(rng, n: int, k: int, scale_lo=1e-5, scale_hi=1e-4) -> np.ndarray:
    """(n, k/256) Q6_K super-blocks: uniform low-bit and high-bit bytes (every
    6-bit quant uniform on 0..63), int8 scales uniform on [-128, 127], then
    binary16 d uniform in [scale_lo, scale_hi]."""
    assert k % QK_K == 0
    nsb = k // QK_K
    blocks = np.empty((n, nsb), dtype=Q6_K_BLOCK)
    blocks["ql"] = rng.integers(0, 256, size=(n, nsb, 128), dtype=np.uint8)
    blocks["qh"] = rng.integers(0, 256, size=(n, nsb, 64), dtype=np.uint8)
    blocks["scales"] = rng.integers(-128, 128, size=(n, nsb, 16), dtype=np.int8)
    blocks["d"] = fp16_scales(rng, (n, nsb), scale_lo, scale_hi)
    return blocks


def weights(rng, qtype: int, n: int, k: int, **kw) -> np.ndarray:
    if qtype == TYPE_Q8_0:
        return q8_0_weights(rng, n, k, **kw)
    if qtype == TYPE_Q4_0:
        return q4_0_weights(rng, n, k, **kw)
    if qtype == TYPE_Q4_K:
        return q4_k_weights(rng, n, k, **kw)
    if qtype == TYPE_Q5_K:
        return q5_k_weights(rng, n, k, **kw)
    if qtype == TYPE_Q6_K:
        return q6_k_weights(rng, n, k, **kw)
    raise ValueError(qtype)


def activations(rng, shape) -> np.ndarray:
    """fp32 activations ~ N(0, 1)."""
    return rng.standard_normal(size=shape, dtype=np.float32)


def q8_0_activations(rng, m: int, k: int):
    """Activation rows generated already in Q8_0 form: int8 quants uniform on
    [-127, 127] and binary16 scales uniform in [1e-3, 1e-2] per 32-block.
    Returns (xq int8 [m][k], xd uint16 bits [m][k/32])."""
    assert k % QK == 0
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    xd = fp16_scales(rng, (m, k // QK))
    return xq, xd


# --------------------------------------------------------------------------
# The five workloads the library is sized for (seed 0 unless given).
# --------------------------------------------------------------------------

def workload_q8_0_small(seed=0):
    """Q8_0 matvec M=1, N=64, K=256; uniform int8 quants, fp32 x ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    w = q8_0_weights(rng, 64, 256)
    x = activations(rng, 256)
    return {"type": TYPE_Q8_0, "n": 64, "k": 256, "w": w, "x": x}


def workload_q4_0_2048(seed=0, n=2048, k=2048):
    """Q4_0 matvec M=1, N=K=2048, fp32 x ~ N(0,1) (plus a Q8_0-quantised
    variant of the same x, made by each side's own quantiser)."""
    rng = np.random.default_rng(seed)
    w = q4_0_weights(rng, n, k)
    x = activations(rng, k)
    return {"type": TYPE_Q4_0, "n": n, "k": k, "w": w, "x": x}


def workload_ffn(seed=0, n_ff=8192, k=2048):
    """Fused FFN decode: Q4_0 gate and up [n_ff][k], Q4_0 down [k][n_ff]."""
    rng = np.random.default_rng(seed)
    wg = q4_0_weights(rng, n_ff, k)
    wu = q4_0_weights(rng, n_ff, k)
    wd = q4_0_weights(rng, k, n_ff)
    x = activations(rng, k)
    return {"n_ff": n_ff, "k": k, "wg": wg, "wu": wu, "wd": wd, "x": x}


def workload_vocab(seed=0, n=262144, k=2048):
    """Q8_0 vocab projection: quants round(N(0,40)) clipped, fp32 x ~ N(0,1)."""
    rng = np.random.default_rng(seed)
    w = q8_0_weights(rng, n, k, dist="normal40")
    x = activations(rng, k)
    return {"type": TYPE_Q8_0, "n": n, "k": k, "w": w, "x": x}


def workload_tile(seed=0, n=8192, k=2048, ms=(8, 16, 32)):
    """Prefill tile: Q4_0 weights [n][k]; for each M in order, activation rows
    already in Q8_0 form (int8 uniform [-127,127], binary16 scales)."""
    rng = np.random.default_rng(seed)
    w = q4_0_weights(rng, n, k)
    acts = {}
    for m in ms:
        acts[m] = q8_0_activations(rng, m, k)
    return {"type": TYPE_Q4_0, "n": n, "k": k, "w": w, "acts": acts}
