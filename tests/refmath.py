"""Test-side numerics used to pin the oracle: library routines (torch's bf16
conversion, numpy's fp64 matmul and stable sorts) and a round-to-odd
binary64 -> binary32 step, written independently of the oracle's code."""
import math
from fractions import Fraction

import numpy as np
import torch


def bf16_to_f32(a):
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_from_f32(a):
    """float32 -> bf16 bits via torch (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f64_to_f32_round_to_odd(d):
    """binary64 -> binary32 with round-to-odd (truncate, then set the last bit if inexact).
    Rounding that result to nearest bf16 equals rounding the binary64 value directly,
    since binary32 carries more than two extra bits over bf16."""
    d = np.asarray(d, dtype=np.float64)
    f = d.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(d)
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    inexact = f.astype(np.float64) != d
    u = f.view(np.uint32).copy()
    u[inexact] |= np.uint32(1)
    return u.view(np.float32)


def bf16_from_f64(d):
    return bf16_from_f32(f64_to_f32_round_to_odd(d))


def unpack_int4_np(packed, K):
    """[N, K/2] uint8 -> [N, K] int8 two's-complement nibbles, low nibble = even column."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    q = np.empty(p.shape[:-1] + (K,), dtype=np.int16)
    q[..., 0::2] = lo
    q[..., 1::2] = hi
    q = np.where(q >= 8, q - 16, q)
    return q.astype(np.int8)


def dequant_np(packed, scales, K):
    q = unpack_int4_np(packed, K).astype(np.float64)
    s = bf16_to_f32(scales).astype(np.float64)
    return q * np.repeat(s, 32, axis=-1)


def pack_int4_np(q):
    """[N, K] ints in [-8, 7] -> [N, K/2] packed bytes (low nibble = even column)."""
    q = np.asarray(q, dtype=np.int16) & 0xF
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def silu64(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def rn32(fr) -> float:
    """The binary32 value nearest to a rational (normal range, or zero), ties to
    even: the IEEE round-to-nearest of one exact result."""
    fr = Fraction(fr)
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = math.floor(math.log2(float(a)))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    scaled = a / Fraction(2) ** (e - 23)
    fl = math.floor(scaled)
    rem = scaled - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return float(sign * fl * Fraction(2) ** (e - 23))


def rint_half_even(fr) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fr = Fraction(fr)
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)
