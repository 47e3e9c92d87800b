"""Pure-Python loop versions of the oracle for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

These repeat the definitions with scalar loops, exact summation (math.fsum)
and their own bit-level decoders (math.ldexp from the format fields), so that
``ref`` (NumPy, table decoders) is checked against an independent evaluation.
Use on inputs with at most a few thousand products.
"""
from __future__ import annotations

import math


def e4m3_scalar(code: int) -> float:
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 15
    man = code & 7
    if exp == 15 and man == 7:
        return math.nan
    if exp == 0:
        return sign * math.ldexp(man, -9)            # m * 2^-3 * 2^-6
    return sign * math.ldexp(8 + man, exp - 10)      # (8+m) * 2^-3 * 2^(e-7)


def e2m1_scalar(nib: int) -> float:
    sign = -1.0 if nib & 8 else 1.0
    exp = (nib >> 1) & 3
    man = nib & 1
    if exp == 0:
        return sign * 0.5 * man
    return sign * math.ldexp(2 + man, exp - 2)       # (1 + m/2) * 2^(e-1)


def bf16_scalar(bits: int) -> float:
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def global_row(codes_row, e8_row, rho) -> list:
    out = []
    D = 2 * len(codes_row)
    for d in range(D):
        byte = int(codes_row[d // 2])
        nib = (byte >> 4) if (d & 1) else (byte & 15)
        v = e2m1_scalar(nib) * math.ldexp(1.0, int(e8_row[d // 32]) - 127)
        out.append(v * (1.0 if rho is None else float(rho)))
    return out


def nvfp4_row(codes_row, scales_row, rho, g) -> list:
    out = []
    D = 2 * len(codes_row)
    for d in range(D):
        byte = int(codes_row[d // 2])
        nib = (byte >> 4) if (d & 1) else (byte & 15)
        v = e2m1_scalar(nib) * e4m3_scalar(int(scales_row[d // 16])) * float(g)
        out.append(v * (1.0 if rho is None else float(rho)))
    return out


def window_row(codes_row, sigma) -> list:
    return [e4m3_scalar(int(c)) * (1.0 if sigma is None else float(sigma)) for c in codes_row]


def score_one(qI_t, w_t, key_row, kappa=None) -> float:
    """S = sum_h w_h * max(0, kappa * sum_d q[h,d] k[d]) for one query and one position."""
    terms = []
    for h in range(len(qI_t)):
        dot = math.fsum(e4m3_scalar(int(qI_t[h][d])) * e4m3_scalar(int(key_row[d]))
                        for d in range(len(key_row)))
        if kappa is not None:
            dot *= float(kappa)
        terms.append(float(w_t[h]) * max(0.0, dot))
    return math.fsum(terms)


def topk_positions(scores: dict, k: int) -> list:
    """scores: {position: score}; returns the k best by (score desc, position asc), ascending."""
    order = sorted(scores, key=lambda j: (-scores[j], j))
    return sorted(order[:k])


def attend_one(q_h_bits, rows: list, sm_scale: float):
    """One query head over an explicit list of decoded rows -> (O list, LSE)."""
    q = [bf16_scalar(b) for b in q_h_bits]
    if not rows:
        return [0.0] * len(q), -math.inf
    logits = [sm_scale * math.fsum(a * b for a, b in zip(q, r)) for r in rows]
    m = max(logits)
    wts = [math.exp(l - m) for l in logits]
    Z = math.fsum(wts)
    D = len(q)
    O = [math.fsum(wts[x] * rows[x][d] for x in range(len(rows))) / Z for d in range(D)]
    return O, m + math.log(Z)
