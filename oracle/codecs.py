"""Number formats of the oracle: bfloat16, OCP FP8 E4M3 (the FN variant) and E8M0.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The boundary page (section ``empty_quantized_layer_input``) fixes the MXFP8
layer input as float8_e4m3fn data of shape [tokens, hidden] plus uint8 scales,
with bf16 as the original dtype. The arithmetic below is written from the
format definitions:

* bfloat16: fp32's sign and 8-bit exponent with 7 stored fraction bits
  (8 significant bits); subnormals below 2**-126 with quantum 2**-133.
* E4M3 (FN): bias 7, 3 fraction bits, subnormal quantum 2**-9, largest finite
  value 1.75 * 2**8 = 448, no infinities, the single NaN pattern S.1111.111.
* E8M0: an unsigned 8-bit biased power of two, 2**(byte - 127), byte 255 NaN.
"""

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits):
    """Decode bfloat16 bit patterns (uint16) to fp64 exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round fp64 values to bfloat16 ONCE, to nearest with ties to even.

    No detour through fp32 (which would round twice). Finite inputs only;
    values whose rounding reaches 2**128 become +-inf, as IEEE rounding does.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding: non-finite input")
    a = np.abs(x)
    _, e = np.frexp(a)           # a = f * 2**e with f in [0.5, 1)
    e = np.maximum(e - 1, -126)  # exponent of the leading bit, floored at fp32's min normal
    quantum = np.ldexp(1.0, e - 7)  # 8 significant bits
    q = np.rint(a / quantum) * quantum  # np.rint rounds half to even; both scalings are exact
    q = np.where(q >= 2.0 ** 128, np.inf, q)
    q = np.copysign(q, x)        # keeps -0.0
    f32 = q.astype(np.float32)   # exact: q has <= 8 significant bits
    u = f32.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise AssertionError("bf16 rounding left low bits set")
    return (u >> np.uint32(16)).astype(np.uint16)


def e4m3_decode(codes):
    """Decode E4M3 (FN) codes to fp64; the NaN pattern decodes to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    normal = (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7)
    sub = (mf / 8.0) * 2.0 ** -6
    v = np.where(ef == 0, sub, normal)
    v = np.where((ef == 15) & (mf == 7), np.nan, v)
    return sign * v


def e4m3_encode(v):
    """Encode fp64 values as E4M3 (FN), rounding to nearest with ties to the even code.

    Magnitudes at or above 448 saturate to 448 (code 0x7E); the sign of zero is
    kept (-0.0 -> 0x80, and negatives that round to zero keep the sign bit).
    Non-finite inputs are rejected.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encode: non-finite input")
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    small = a < 2.0 ** -6
    # subnormal range: code = round(a / 2**-9), which may reach 8 == the smallest normal
    code = np.where(small, np.rint(a / 2.0 ** -9).astype(np.int64), code)
    _, e = np.frexp(np.where(small, 1.0, a))
    e = e - 1                                   # a = m * 2**e, m in [1, 2)
    m = np.where(small, 1.0, a) / np.ldexp(1.0, e)
    frac = np.rint((m - 1.0) * 8.0).astype(np.int64)  # 0..8; 8 carries into the exponent
    normal_code = ((e + 7) << 3) + frac
    code = np.where(small, code, normal_code)
    code = np.where(a >= E4M3_MAX, 0x7E, code)
    code = np.minimum(code, 0x7E)
    code = code | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


def e8m0_exponent(amax):
    """Shared block exponent: the smallest integer e with amax <= 448 * 2**e.

    Written as amax = M * 2**E with M in [1, 2): e = E - 8 + [M > 1.75], since
    448 = 1.75 * 2**8. A zero block takes e = -127. The result is clamped to
    the E8M0 range [-127, 127] (byte 255 is NaN and never produced).
    """
    a = np.asarray(amax, dtype=np.float64)
    if np.any(a < 0) or not np.all(np.isfinite(a)):
        raise ValueError("E8M0: amax must be finite and non-negative")
    f, E = np.frexp(np.where(a == 0, 1.0, a))
    M = 2.0 * f
    E = E - 1
    e = E - 8 + (M > 1.75).astype(np.int64)
    e = np.where(a == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp8_quantize(layer_input_bits, block=32):
    """MXFP8 of a bf16 matrix [rows, hidden]: one E8M0 scale per `block` contiguous elements.

    Returns (codes uint8 [rows, hidden], scale bytes uint8 [rows, hidden // block]),
    scales plain row-major. Each element is encoded as E4M3(value * 2**-e); the
    power-of-two scaling is exact.
    """
    x = bf16_bits_to_f64(layer_input_bits)
    rows, hidden = x.shape
    if hidden % block:
        raise ValueError("MXFP8: hidden must be a multiple of the block size")
    xb = x.reshape(rows, hidden // block, block)
    e = e8m0_exponent(np.max(np.abs(xb), axis=2))
    scaled = xb * np.ldexp(1.0, -e)[:, :, None]
    codes = e4m3_encode(scaled).reshape(rows, hidden)
    return codes, (e + 127).astype(np.uint8)


def mxfp8_scales_swizzled_128x4(scales, fill=0):
    """Row-major E8M0 scales [rows, blocks] -> the swizzled 128x4 byte vector.

    The boundary page gives its MXFP8 layer input FlashInfer's swizzled 128x4
    scale layout (section ``empty_quantized_layer_input``) without spelling it
    out; this is that layout as the block-scaled GEMM interfaces publish it.
    Rows are padded to a multiple of 128 and blocks to a multiple of 4 (the
    padding holds ``fill``). The padded matrix is cut into 128 x 4 tiles stored
    one after another in row-major tile order, 512 bytes each. Inside a tile,
    row t = 32 * a + b (a in 0..3, b in 0..31) and block c (0..3) sit at byte
    16 * b + 4 * a + c: the 32 row groups of 16 bytes each hold rows b, b+32,
    b+64, b+96, four blocks per row.
    """
    s = np.asarray(scales, dtype=np.uint8)
    rows, blocks = s.shape
    rp = -(-rows // 128) * 128
    bp = -(-blocks // 4) * 4
    padded = np.full((rp, bp), fill, dtype=np.uint8)
    padded[:rows, :blocks] = s
    # axes: (row tile, a, b, block tile, c) -> (row tile, block tile, b, a, c)
    t = padded.reshape(rp // 128, 4, 32, bp // 4, 4)
    return np.ascontiguousarray(t.transpose(0, 3, 2, 1, 4)).reshape(-1)
