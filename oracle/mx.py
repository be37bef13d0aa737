"""MX element and scale codecs, fp64 (TEST INFRASTRUCTURE ONLY - see package docstring).

Everything here is written from the definitions, not from any kernel:

* E2M1 (FP4): 1 sign, 2 exponent, 1 mantissa bit [DS4-FP4 section 一]. Reading
  (the page gives only the bit budget): sign = bit 3, exponent = bits 2..1 with
  bias 1, mantissa = bit 0; exponent 0 is subnormal (value m * 0.5). That gives
  the magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}. Largest normal 6 = 1.5 * 2^2, so
  emax = 2 [OCP-MX].
* E4M3 (the OCP "E4M3FN" variant): 4 exponent + 3 mantissa bits [FP8-GGUF 一],
  bias 7, exponent 0 subnormal (m * 2^-9), S.1111.111 is NaN, no infinities.
  Largest normal 448 = 1.75 * 2^8, so emax = 8 [OCP-MX].
* UE8M0 block scale [DS4-FP4 section 一]: an unsigned biased exponent byte b
  with value 2^(b - 127); b = 255 is NaN [OCP-MX].
* Packed FP4: two codes per byte, even column in the low nibble, odd column in
  the high nibble [TRITON-FP4, "第二步：Fused Dequant+Matmul Kernel"].

Quantisation of one 32-element block (the OCP MX rule [OCP-MX]):
  1. amax = max |v| over the block;
  2. X = floor(log2 amax) - emax, found exactly with frexp;
  3. scale byte = clamp(X + 127, 0, 254), and 0 when amax == 0; X' = byte - 127;
  4. t = v * 2^-X' (exact in fp64);
  5. each |t| goes to the nearest value of the element grid (subnormals
     included); a value exactly half-way goes to the code whose mantissa LSB
     is 0 (round-to-nearest-even); |t| above the largest normal saturates to it;
  6. the sign bit of v is kept, so negative values that round to zero give -0.
Readings: saturation rather than NaN on overflow (the OCP rule clamps to the
largest normal); signed zero kept; non-finite inputs are not defined here.
"""

import numpy as np

E2M1_EMAX = 2
E4M3_EMAX = 8
FMT_E4M3 = "e4m3"
FMT_E2M1 = "e2m1"


def _e2m1_value(code):
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def _e4m3_value(code):
    s = (code >> 7) & 1
    e = (code >> 3) & 15
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


_E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)
_E4M3_TABLE = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e2m1_decode(codes):
    """FP4 E2M1 codes (uint8, one code per element, 0..15) -> fp64 values."""
    return _E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 15]


def e4m3_decode(codes):
    """FP8 E4M3FN codes (uint8) -> fp64 values (NaN for 0x7F / 0xFF)."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def ue8m0_decode(b):
    """UE8M0 scale bytes -> fp64 2^(b-127); 255 -> NaN."""
    b = np.asarray(b, dtype=np.int64)
    out = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, out)


def pack_e2m1(codes):
    """[rows][K] codes (0..15) -> [rows][K/2] bytes, even k in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] & 15) | ((codes[..., 1::2] & 15) << 4)


def unpack_e2m1(packed):
    """[rows][K/2] bytes -> [rows][K] codes, low nibble first."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> fp64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def _fmt_params(fmt):
    if fmt == FMT_E4M3:
        codes = np.arange(0, 0x7F, dtype=np.int64)  # 0x00 .. 0x7E, all finite
        return E4M3_EMAX, codes, _E4M3_TABLE[codes], 0x80
    if fmt == FMT_E2M1:
        codes = np.arange(0, 8, dtype=np.int64)
        return E2M1_EMAX, codes, _E2M1_TABLE[codes], 0x8
    raise ValueError(f"unknown element format {fmt!r}")


def mx_scale_byte(amax, fmt):
    """Step 2-3 of the block rule: UE8M0 byte from the block's max magnitude."""
    emax = _fmt_params(fmt)[0]
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)  # amax = f * 2^e with 0.5 <= f < 1, so floor(log2) = e - 1
    byte = np.clip(e - 1 - emax + 127, 0, 254)
    return np.where(amax == 0, 0, byte).astype(np.uint8)


def round_to_grid(t_abs, fmt):
    """Step 5: nearest grid code for |t| >= 0, ties to even mantissa, saturating."""
    _, codes, vals, _ = _fmt_params(fmt)
    a = np.minimum(np.asarray(t_abs, dtype=np.float64), vals[-1])
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, len(vals) - 1)
    hi = np.minimum(lo + 1, len(vals) - 1)
    mid = (vals[lo] + vals[hi]) / 2.0  # exact: grid values have few significant bits
    even_hi = (codes[hi] & 1) == 0
    pick_hi = (hi != lo) & ((a > mid) | ((a == mid) & even_hi))
    return np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)


def mx_quantize(v, fmt):
    """Quantise rows of fp64 values per 32-block along the last axis.

    Returns (codes [rows][K] uint8 - one code per element, E2M1 not packed,
             scales [rows][K/32] uint8).
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    _, _, _, sign_bit = _fmt_params(fmt)
    blk = v.reshape(v.shape[:-1] + (K // 32, 32))
    amax = np.max(np.abs(blk), axis=-1)
    byte = mx_scale_byte(amax, fmt)
    xp = byte.astype(np.int64) - 127
    t = np.ldexp(blk, -xp[..., None])
    mag = round_to_grid(np.abs(t), fmt)
    sign = np.signbit(blk)
    codes = np.where(sign, mag | sign_bit, mag).astype(np.uint8)
    return codes.reshape(v.shape), byte


def mx_dequantize(codes, scales, fmt):
    """codes [rows][K] (unpacked) + scales [rows][K/32] -> fp64 [rows][K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    vals = e4m3_decode(codes) if fmt == FMT_E4M3 else e2m1_decode(codes)
    sc = ue8m0_decode(scales)
    blk = vals.reshape(codes.shape[:-1] + (K // 32, 32)) * sc[..., None]
    return blk.reshape(codes.shape)


def dequant_weights(packed, scales):
    """MXFP4 weights [N][K/2] packed + [N][K/32] scales -> fp64 [N][K]."""
    return mx_dequantize(unpack_e2m1(packed), scales, FMT_E2M1)


def ue4m3_decode(b):
    """UE4M3 block-scale bytes -> fp64 [DS4-FP4 section 一: the NVFP4 (kind::mxf4nvf4)
    scale]. Reading (the page names the type only): an OCP E4M3FN byte with the sign
    bit clear - exponent 0 subnormal (m * 2^-9), otherwise 2^(e-7) (1 + m/8); 0x7F is
    NaN; bytes with the sign bit set are not UE4M3 and decode to NaN here."""
    b = np.asarray(b, dtype=np.uint8)
    v = _E4M3_TABLE[b & 0x7F]
    return np.where(b & 0x80, np.nan, v)


def dequant_nvfp4_weights(packed, scales16):
    """NVFP4 weights [N][K/2] packed E2M1 + [N][K/16] UE4M3 scales -> fp64 [N][K]:
    value = e2m1(code) * ue4m3(scale of its 16-element block)."""
    codes = unpack_e2m1(packed)
    K = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (K // 16, 16))
    return (vals * ue4m3_decode(scales16)[..., None]).reshape(codes.shape)
