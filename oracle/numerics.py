"""Storage-format helpers for the oracle: bf16 and OCP E4M3FN, written from the format definitions.

TEST INFRASTRUCTURE. Only tests/, the smoke check and the CPU-baseline leg of the benchmark may
import this package; the product path never does.

Formats
-------
* bf16: IEEE-754 binary32 with the low 16 bits of the fraction removed. 1 sign bit, 8 exponent
  bits (bias 127), 7 stored fraction bits. Rounding from a real number is round-to-nearest,
  ties-to-even (RNE); values at or beyond (2 - 2^-8) * 2^127 round to infinity.
* E4M3FN (OCP 8-bit floating point specification, "E4M3"): 1 sign bit, 4 exponent bits (bias 7),
  3 fraction bits. No infinities; the only NaN encodings are S.1111.111. Largest finite
  magnitude 1.75 * 2^8 = 448, smallest normal 2^-6, subnormal step 2^-9. Conversion here is
  RNE with saturation to +-448 ("satfinite"), the mode used for the fp8 KV cache rows.

* E2M1 (OCP Microscaling (MX) specification, "FP4"): 1 sign bit, 2 exponent bits (bias 1), 1
  fraction bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; no infinities or NaN. Two
  codes per byte, element 2i in the low nibble of byte i.
* E8M0 (the same specification's shared scale): an 8-bit biased exponent, value 2^(code - 127);
  code 255 is NaN. One scale multiplies each block of 32 consecutive E2M1 elements (MXFP4).

The mixed-precision cache row (RoPE dims in bf16, the rest in fp8) is described on
jaylab-temp.pages.dev "DeepSeek-V4 — 百万 Token 上下文的高效 MoE 模型", section 其他技术细节
(KV cache 混合精度); the per-row fp32 scale is this library's reading of that row format.

Everything here works in float64 on numpy arrays; no routine is shared with the GPU path.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_BF16_MIN_EXP = -133  # quantum of the smallest bf16 subnormal: 2^-126 * 2^-7
_E4M3_MIN_EXP = -9    # quantum of the smallest e4m3 subnormal: 2^-6 * 2^-3


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 codes -> float64 values (exact: every bf16 value is a float32 value)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def _quantum(x: np.ndarray, sig_bits: int, min_exp: int) -> np.ndarray:
    """Spacing of the target format at |x|: 2^(e - sig_bits) with x = f * 2^e, 0.5 <= |f| < 1,
    never below the subnormal spacing 2^min_exp."""
    _, e = np.frexp(x)
    q = np.maximum(e.astype(np.int64) - sig_bits, min_exp)
    return np.ldexp(1.0, q)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round real values (float64) to the nearest bf16 value, ties to even. Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    q = _quantum(x, 8, _BF16_MIN_EXP)
    # x / q is exact (q is a power of two and stays in range); rint is ties-to-even.
    y = np.rint(x / q) * q
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    y = np.where(np.abs(y) > big, np.copysign(np.inf, x), y)
    return np.where(np.isnan(x), np.nan, y)


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """Round float64 to bf16 (RNE) and return the uint16 codes."""
    y = bf16_round(x).astype(np.float32)  # exact: y is a bf16 value
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3FN codes (NaN for S.1111.111)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        f = code & 0x7
        if e == 0xF and f == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (f / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3FN codes -> float64."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3FN value, ties to even, saturating to +-448. Returns float64."""
    x = np.asarray(x, dtype=np.float64)
    q = _quantum(x, 4, _E4M3_MIN_EXP)
    y = np.rint(x / q) * q
    return np.clip(y, -E4M3_MAX, E4M3_MAX)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round float64 to E4M3FN (RNE, satfinite) and return uint8 codes."""
    y = e4m3_round(x)
    # Map each finite value to its code through the positive half of the table.
    pos_vals = E4M3_VALUES[:0x7F]  # codes 0x00..0x7E: 0 .. 448, strictly increasing
    mag = np.searchsorted(pos_vals, np.abs(y))
    assert np.all(pos_vals[mag] == np.abs(y)), "value not representable in E4M3"
    code = mag.astype(np.uint8)
    neg = np.signbit(y) & (y != 0)
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def f32_round(x: np.ndarray) -> np.ndarray:
    """Round float64 to the nearest float32 (RNE) and return it as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def _e2m1_table() -> np.ndarray:
    """Value of each of the 16 E2M1 codes."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        f = code & 0x1
        vals[code] = s * (f / 2.0) if e == 0 else s * (1.0 + f / 2.0) * 2.0 ** (e - 1)
    return vals


E2M1_VALUES = _e2m1_table()


def fp4_unpack(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., n] holding two E2M1 codes each -> codes uint8 [..., 2n] (low nibble first)."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & np.uint8(0x0F)
    out[..., 1::2] = p >> np.uint8(4)
    return out


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """uint8 E8M0 codes -> float64 2^(code - 127) (NaN for 255)."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray, block: int = 32) -> np.ndarray:
    """MXFP4 rows -> float64: packed E2M1 codes [..., d/2] and E8M0 scales [..., d/block]; element
    i of a row is E2M1(code_i) * 2^(scale[i // block] - 127)."""
    v = E2M1_VALUES[fp4_unpack(packed)]
    sc = e8m0_decode(scales)
    return v * np.repeat(sc, block, axis=-1)
