"""Test-side encoders: integer weight codes -> canonical bytes.

Written from the encoding the workloads state (int4 in [-8, 7] packed two per
byte, int6 in [-32, 31] packed four per three bytes), in the encode direction,
so that they pin the oracle's decoder instead of repeating it.
"""
import numpy as np


def pack_w4(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    assert c.min() >= -8 and c.max() <= 7 and c.shape[-1] % 2 == 0
    u = (c & 0xF).astype(np.uint8)
    return (u[..., 0::2] | (u[..., 1::2] << 4)).astype(np.uint8)


def pack_w6(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    assert c.min() >= -32 and c.max() <= 31 and c.shape[-1] % 4 == 0
    u = c & 0x3F
    t = u[..., 0::4] | (u[..., 1::4] << 6) | (u[..., 2::4] << 12) | (u[..., 3::4] << 18)
    out = np.empty(c.shape[:-1] + (c.shape[-1] // 4, 3), np.uint8)
    out[..., 0] = t & 0xFF
    out[..., 1] = (t >> 8) & 0xFF
    out[..., 2] = (t >> 16) & 0xFF
    return out.reshape(c.shape[:-1] + (c.shape[-1] * 3 // 4,))


def pack(bits, codes):
    return pack_w4(codes) if bits == 4 else pack_w6(codes)


def random_codes(rng, bits, N, K):
    lo, hi = (-8, 7) if bits == 4 else (-32, 31)
    return rng.integers(lo, hi + 1, size=(N, K))


def bf16_to_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits_via_f32(v):
    """Nearest-even bf16 of values that are exactly representable in fp32."""
    f = np.asarray(v, np.float64).astype(np.float32)
    assert np.all(f.astype(np.float64) == np.asarray(v, np.float64))
    u = f.view(np.uint32)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
