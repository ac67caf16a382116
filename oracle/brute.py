"""Exact brute force for tiny products -- TEST INFRASTRUCTURE ONLY.

Pure-Python i-j-k loops over exact rationals ("I Wrote a GPU Matmul Kernel
From Scratch in Triton", Step 1, the naive three-loop matmul). The inputs are
decoded with Python's own `struct` codecs, not with the C oracle's bit
decoding, so the two are independent.
"""
import struct
from fractions import Fraction


def value(bits: int, dtype: str) -> Fraction:
    """Exact value of one bit pattern (finite inputs only)."""
    if dtype == "f16":
        v = struct.unpack("<e", struct.pack("<H", bits))[0]
    elif dtype == "bf16":
        v = struct.unpack("<f", struct.pack("<I", bits << 16))[0]
    elif dtype == "f32":
        v = struct.unpack("<f", struct.pack("<I", bits))[0]
    else:
        raise ValueError(dtype)
    return Fraction(v)


def matmul(a, b):
    """Exact C = A @ B for nested lists of Fractions or ints."""
    M, K = len(a), len(a[0]) if a else 0
    K2 = len(b)
    N = len(b[0]) if b else 0
    if K != K2:
        raise ValueError("inner dimensions differ")
    c = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += a[i][k] * b[k][j]
            c[i][j] = s
    return c
