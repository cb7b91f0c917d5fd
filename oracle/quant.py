"""Residual quantizer of the per-loop KV store (oracle; test infrastructure only).

Basis: the FlashLoop abstract's third observation -- KV residuals between
adjacent loops become amenable to low-bit quantization -- so loop k's KV is
stored as loop k-1's reconstruction plus a quantized residual.  The pages
give no format; the format read here is:

* groups of ``group`` (32) consecutive elements along head_dim of one
  (token, KV head, K-or-V) row;
* symmetric, no zero point; qmax = 2**(bits-1) - 1 (127 for int8, 7 for int4;
  the int4 code -8 is never produced);
* scale: s32 = amax / qmax in IEEE float32, then s16 = float16(s32) rounded to
  nearest even and saturated at 65504;
* code = 0 when s16 == 0, else clamp(rint_half_even(r / float32(s16)), -qmax, qmax);
* dequantized value = code * float32(s16) (exact in float32: |code| < 2**7 and
  s16 has an 11-bit significand);
* int4 codes are packed two per byte, element 2j in the low nibble and 2j+1
  in the high nibble (two's complement nibbles).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
FP16_MAX = F32(65504.0)


def qmax_of(bits: int) -> int:
    if bits not in (4, 8):
        raise ValueError("quantized widths are 4 and 8 bits")
    return (1 << (bits - 1)) - 1


def quantize(r: np.ndarray, bits: int, group: int = 32):
    """Quantize float32 rows ``r[..., hd]`` group-wise.

    Returns ``(codes int8 [..., hd], scales float16 [..., hd // group])``.
    """
    r = np.asarray(r, dtype=F32)
    hd = r.shape[-1]
    if hd % group:
        raise ValueError("head_dim must be a multiple of the group size")
    qmax = qmax_of(bits)
    g = r.reshape(r.shape[:-1] + (hd // group, group))
    amax = np.max(np.abs(g), axis=-1)                     # float32, exact
    s32 = amax / F32(qmax)                                # IEEE float32 divide
    s16 = np.minimum(s32, FP16_MAX).astype(np.float16)    # round to nearest even
    s = s16.astype(F32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(g / s)                                # float32 divide, half to even
    q = np.clip(q, -qmax, qmax)
    q = np.where(s == 0, F32(0), q)
    codes = q.astype(np.int8).reshape(r.shape)
    return codes, s16


def dequantize(codes: np.ndarray, scales: np.ndarray, group: int = 32) -> np.ndarray:
    """codes int8 [..., hd], scales float16 [..., hd // group] -> float32 [..., hd]."""
    hd = codes.shape[-1]
    c = codes.astype(F32).reshape(codes.shape[:-1] + (hd // group, group))
    return (c * scales.astype(F32)[..., None]).reshape(codes.shape)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """int8 codes in [-8, 7], last dim even -> uint8 [..., hd // 2]."""
    c = codes.astype(np.int16) & 0xF
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    p = packed.astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out
