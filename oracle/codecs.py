"""Exact decoders for the storage formats, written from the format definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* FP8 E4M3FN (OCP 8-bit floating point specification): 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6);
  S.1111.111 is NaN; there is no infinity; largest finite value 448.
* E2M1 (OCP Microscaling Formats v1.0, FP4): 1 sign bit (bit 3), 2 exponent
  bits with bias 1, 1 mantissa bit: magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
  Two elements per byte, element 2i in the low nibble (a reading: the pages
  give no packing, only "FP4", blog §"SWA bounded replay").
* E8M0 (OCP MX v1.0 shared scale): unsigned 8-bit exponent, value 2^(e-127),
  0xFF is NaN.
* bfloat16: the upper 16 bits of an IEEE binary32.

All tables are computed here from these definitions; nothing is read from the
GPU library.
"""
from __future__ import annotations

import numpy as np


def _e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** (1 - 7)
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def _e2m1_value(code: int) -> float:
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        v = m * 0.5                      # subnormal: m/2 * 2^(1-1)
    else:
        v = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -v if s else v


E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 array of E4M3FN codes -> float64 values (same shape)."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_unpack(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., D/2] packed E2M1 -> float64 [..., D]; element 2i = low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = E2M1_TABLE[p & 0x0F]
    hi = E2M1_TABLE[p >> 4]
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def e8m0(e: np.ndarray) -> np.ndarray:
    """uint8 E8M0 exponents -> float64 scales 2^(e-127); 255 -> NaN."""
    e = np.asarray(e, dtype=np.int64)
    out = np.ldexp(1.0, e - 127).astype(np.float64)
    return np.where(e == 255, np.nan, out)


def bf16(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float values -> uint16 bfloat16 bits, rounded once to the nearest bfloat16 (ties to the
    even significand).  bfloat16 keeps 8 significant bits: a value with binary exponent e
    (2^(e-1) <= |x| < 2^e) lies on a grid of spacing 2^(e-8), and below the smallest normal
    2^-126 on the subnormal grid of spacing 2^-133.  Scaling by a power of two is exact, so
    the rounding is numpy's round-half-to-even on the integer grid.  Overflow gives inf."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    y = np.ldexp(np.round(np.ldexp(x, -q)), q)
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)          # exact: y has at most 8 significant bits
    return (f.view(np.uint32) >> 16).astype(np.uint16)


_E4M3_POS = np.array([_e4m3_value(c) for c in range(0x7F)], dtype=np.float64)   # 0x00..0x7E


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float values -> OCP E4M3FN codes: the nearest finite value, ties to the even code (the
    one whose mantissa ends in 0), magnitudes above 448 saturated to 448; the sign bit is
    the input's (-0 and a negative value that rounds to zero give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def global_rows(codes: np.ndarray, e8: np.ndarray, rowscale) -> np.ndarray:
    """Decode global-latent rows: V[j,d] = e2m1(nib(j,d)) * 2^(E[j, d//32]-127) * rho_j.

    codes uint8 [R, D/2], e8 uint8 [R, D/32], rowscale float32 [R] or None (rho = 1).
    """
    vals = e2m1_unpack(codes)
    R, D = vals.shape
    scale = np.repeat(e8m0(e8), 32, axis=1)
    assert scale.shape == (R, D)
    v = vals * scale
    if rowscale is not None:
        v = v * np.asarray(rowscale, dtype=np.float64)[:, None]
    return v


def nvfp4_rows(codes: np.ndarray, scales: np.ndarray, rowscale, tensor_scale: float) -> np.ndarray:
    """Decode NVFP4 latent rows: V[j,d] = e2m1(nib(j,d)) * e4m3(S[j, d//16]) * rho_j * g.

    The NVFP4 layout: E2M1 elements with one E4M3 scale per 16 elements and one fp32 scale g
    for the whole tensor; rho (optional, None = 1) is an extra fp32 row scale.  codes uint8
    [R, D/2], scales uint8 [R, D/16].
    """
    vals = e2m1_unpack(codes)
    R, D = vals.shape
    sc = np.repeat(e4m3(scales), 16, axis=1)
    assert sc.shape == (R, D)
    v = vals * sc * float(tensor_scale)
    if rowscale is not None:
        v = v * np.asarray(rowscale, dtype=np.float64)[:, None]
    return v


def window_rows(codes: np.ndarray, scale) -> np.ndarray:
    """Decode sliding-window rows: X[u,d] = e4m3(byte) * sigma_u (sigma = 1 when None)."""
    x = e4m3(codes)
    if scale is not None:
        x = x * np.asarray(scale, dtype=np.float64)[..., None]
    return x


def mxfp8_quantize(x: np.ndarray):
    """OCP MX v1.0 MXFP8 (E4M3) quantisation along the last axis in blocks of 32: each block
    gets the shared exponent E = floor(log2(amax)) - emax + 127 with emax = 8 (E4M3's largest
    normal is 1.75 * 2^8), clamped to [0, 254] (0 for an all-zero block), and each element
    the E4M3 code of x / 2^(E - 127), nearest even, saturating at 448.  Returns (codes uint8
    [..., n], E uint8 [..., n/32]).  Dividing by a power of two is exact, so the only
    rounding is the E4M3 one."""
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] % 32 == 0
    blocks = x.reshape(x.shape[:-1] + (x.shape[-1] // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)                     # amax = m * 2^ex, m in [0.5, 1): floor(log2) = ex - 1
    E = np.where(amax > 0, np.clip(ex.astype(np.int64) - 1 - 8 + 127, 0, 254), 0)
    y = blocks / np.ldexp(1.0, E - 127)[..., None]
    codes = e4m3_encode(y).reshape(x.shape)
    return codes, E.astype(np.uint8)


def mxfp8_decode(codes: np.ndarray, E: np.ndarray) -> np.ndarray:
    """MXFP8 codes [..., n] with block exponents [..., n/32] -> float64 values."""
    v = e4m3(codes)
    return v * np.repeat(e8m0(E), 32, axis=-1)
