"""Plain float64 definition of the FP8 LM-head projection.

TEST INFRASTRUCTURE ONLY (see the package docstring): slow, obviously
correct, written step by step from the definitions.

What it computes, and where it is stated:
  * The LM head projects the 2,560-wide hidden state onto the 157,184-token
    vocabulary ("3 Ways to Improve MoE Inference on NVIDIA DGX Spark" digest,
    section 2); it is, with the MoE layers, one of the two most expensive
    decode operations (digest, section 1).
  * Its BF16 checkpoint weights are quantised online to FP8 when the head is
    built, halving the bytes each decode step reads (digest, section 4; the
    Vietnamese rewrite, section 2).

Readings taken where the pages are silent:
  FP8 is OCP E4M3 (the "FN" variant: bias 7, no infinities, 0x7F/0xFF are
  NaN, largest finite 448); one fp32 scale per vocabulary row,
  s = amax(row) / 448 computed in fp32 (s = 1 for an all-zero row); a code is
  the E4M3 value nearest to the fp32 quotient w / s (ties to an even
  mantissa), the quotient first clamped to [-448, 448]; activations stay bf16
  (W8A16); a logit is sum_k x_k * e4m3(code_k) * s, here in float64.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """8-bit E4M3 code -> float64 from its bit fields: bit 7 sign, bits 6..3
    exponent (bias 7), bits 2..0 mantissa; exponent field 0 is subnormal
    (m/8 * 2^-6); exponent 15 with mantissa 7 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    out = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


# the 127 non-negative finite E4M3 values with their codes, ascending
_POS_CODES = np.arange(0, 127, dtype=np.int64)          # 0x00 .. 0x7E
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_round(q: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each finite value, ties to the even mantissa; the
    value is first clamped to [-448, 448].  The sign bit is the input's (so a
    negative value that rounds to zero, and -0 itself, give 0x80), as in IEEE
    conversions."""
    q = np.clip(np.asarray(q, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(q)
    # candidates: the largest value <= a and the next one up
    lo = np.searchsorted(_POS_VALUES, a, side="right") - 1
    hi = np.minimum(lo + 1, len(_POS_VALUES) - 1)
    dlo, dhi = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((_POS_CODES[lo] & 1) == 1))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    return np.where(np.signbit(q), code | 0x80, code).astype(np.uint8)


def lmhead_quantize(w_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """bf16 weights [V][H] (bit patterns) -> (E4M3 codes [V][H], fp32 row scales [V]).
    The scale and the quotient are computed in fp32, as the kernel does."""
    w = (np.asarray(w_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    amax = np.max(np.abs(w), axis=1).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    quotient = (w / scale[:, None]).astype(np.float32)
    return e4m3_round(quotient.astype(np.float64)), scale


def lmhead_logits(x_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """logits[t][v] = sum_k x[t][k] * e4m3(codes[v][k]) * scales[v], float64."""
    x = (np.asarray(x_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = e4m3_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]
    return x @ w.T
