"""Plain CPU reference of the fp8 tile codec: block-scaled E4M3 probabilities.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline import this module. It shares no code with the HIP library.

Why a codec: MapFlow ("Accelerating Cross-Model LLM Inference via Attention Map
Reuse"), §9 names quantised sparse representations of the maps as the next step
for cutting their size. The maps are probabilities, and inside a long row most
of them are far below the smallest normal E4M3 value (2^-6), so a plain fp8 cast
would zero most of the mass. The codec therefore scales every block of 32
consecutive keys of one row by its own power of two, as the OCP Microscaling
(MX) formats do (block size 32, E8M0 shared scale, E4M3 elements).

Definitions used here (all arithmetic in float64, exact where it matters):

* E4M3 (OCP 8-bit floating point, "E4M3FN"): sign, 4 exponent bits (bias 7), 3
  mantissa bits. Exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111 is
  NaN; there are no infinities; the largest finite value is 448.
* Encoding of a non-negative x <= 448: the nearest E4M3 value, ties to the code
  with an even mantissa (round to nearest even).
* Shared scale of a block with maximum a: e = floor(log2 a) - 7, clamped below
  at -126 (and e = -126 for an all-zero block); stored as the E8M0 byte e + 127.
  The block maximum then scales into [128, 256), so no element saturates.  (The
  OCP rule is floor(log2 a) - 8 with saturation at 448, which can clip the
  largest element of a block by up to 12.5%; here the block keeps its largest
  element to 3 mantissa bits at the cost of one binade at the bottom.)
* Element codes: E4M3 encoding of p * 2^-e; decoded value code_value * 2^e.

Error bound of one decoded element p' against p (block scale e): the E4M3 grid
spacing at a scaled value y = p * 2^-e is 2^(max(floor(log2 y), -6) - 3), so
|p' - p| <= max(2^-4 * p, 2^(e - 10)).
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

E4M3_MAX = 448.0
MX_BLOCK = 32
SCALE_BIAS = 127
SCALE_MIN = -126


def e4m3_value(code: int) -> float:
    """Value of an E4M3 byte (NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    ef = (code >> 3) & 0xF
    m = code & 0x7
    if ef == 0xF and m == 0x7:
        return math.nan
    if ef == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (ef - 7)


def e4m3_code(x: float) -> int:
    """Nearest-even E4M3 code of a finite non-negative x <= 448."""
    x = float(x)
    if not (0.0 <= x <= E4M3_MAX):
        raise ValueError(f"e4m3_code takes 0 <= x <= 448, got {x!r}")
    if x == 0.0:
        return 0
    _, E = math.frexp(x)          # x = f * 2^E with f in [0.5, 1)
    E -= 1                        # binade: x in [2^E, 2^(E+1))
    Eg = max(E, -6)               # subnormals share the spacing of binade -6
    spacing = 2.0 ** (Eg - 3)
    n = float(np.rint(x / spacing))  # x / spacing is exact; rint rounds half to even
    v = n * spacing
    if v == 0.0:
        return 0
    if v < 2.0 ** -6:             # subnormal: exponent field 0, mantissa n
        return int(n)
    _, Ev = math.frexp(v)
    Ev -= 1
    m = int(round((v / 2.0 ** Ev - 1.0) * 8.0))
    return ((Ev + 7) << 3) | m


def block_scale_exponent(amax: float) -> int:
    """Shared scale exponent e of a block whose largest element is amax >= 0."""
    if amax <= 0.0:
        return SCALE_MIN
    _, E = math.frexp(float(amax))
    return max(E - 1 - 7, SCALE_MIN)


def e4m3_codes(y: np.ndarray) -> np.ndarray:
    """e4m3_code over an array (same steps, elementwise)."""
    y = np.asarray(y, dtype=np.float64)
    if np.any(~(y >= 0.0)) or np.any(y > E4M3_MAX):
        raise ValueError("e4m3_codes takes 0 <= y <= 448")
    _, E = np.frexp(y)
    Eg = np.maximum(E - 1, -6)
    spacing = np.ldexp(1.0, Eg - 3)
    n = np.rint(y / spacing)
    v = n * spacing
    _, Ev = np.frexp(v)
    Ev = Ev - 1
    m = np.rint((np.ldexp(v, -Ev) - 1.0) * 8.0)
    normal = ((Ev + 7) << 3) + m.astype(np.int64)
    code = np.where(v < 2.0 ** -6, n.astype(np.int64), normal)
    return np.where(v == 0.0, 0, code).astype(np.uint8)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def encode_tile(P: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """[R, C] non-negative probabilities (C a multiple of 32) -> (codes uint8 [R, C],
    scale bytes uint8 [R, C/32]), one scale per 32 consecutive keys of a row."""
    P = np.asarray(P, dtype=np.float64)
    R, C = P.shape
    assert C % MX_BLOCK == 0
    blocks = P.reshape(R, C // MX_BLOCK, MX_BLOCK)
    amax = blocks.max(axis=2)
    _, E = np.frexp(amax)
    e = np.where(amax > 0.0, np.maximum(E - 1 - 7, SCALE_MIN), SCALE_MIN)
    codes = e4m3_codes(np.ldexp(blocks, -e[:, :, None]))
    return codes.reshape(R, C), (e + SCALE_BIAS).astype(np.uint8)


def decode_tile(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of encode_tile: code_value * 2^(scale - 127), float64."""
    codes = np.asarray(codes)
    R, C = codes.shape
    e = np.asarray(scales).astype(np.int64) - SCALE_BIAS
    vals = E4M3_TABLE[codes.astype(np.int64)].reshape(R, C // MX_BLOCK, MX_BLOCK)
    return np.ldexp(vals, e[:, :, None]).reshape(R, C)


def quantize(P: np.ndarray) -> np.ndarray:
    """Decoded values of encode_tile(P): what a receiver reads back."""
    return decode_tile(*encode_tile(P))


def error_bound(P: np.ndarray) -> np.ndarray:
    """Per-element bound max(2^-4 p, 2^(e - 10)) on |quantize(P) - P|."""
    P = np.asarray(P, dtype=np.float64)
    R, C = P.shape
    blocks = P.reshape(R, C // MX_BLOCK, MX_BLOCK)
    e = np.array([[block_scale_exponent(a) for a in row] for row in blocks.max(axis=2)],
                 dtype=np.int64)
    return np.maximum(2.0 ** -4 * blocks, np.ldexp(1.0, e - 10)[:, :, None]).reshape(R, C)
