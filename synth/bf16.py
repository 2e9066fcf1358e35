"""bfloat16 as raw uint16 bit patterns (numpy has no bf16 dtype).

fp32 -> bf16 uses round-to-nearest-even on the upper 16 bits; the
inverse is exact (bf16 is a truncated fp32).
"""
import numpy as np


def f32_to_bf16_bits(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b):
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)
