"""Element formats of the fused-MoE path, decoded and encoded in fp64 (oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Formats (b12x README, "What's in here": MXFP4 / NVFP4 weights, MXFP8 row
quantizer; "PCIe DMA wire modes": MXFP8 keeps one E8M0 scale per 32 values;
vLLM b12x page, "Supported Configurations": MXFP4 or NVFP4 weights with BF16
or MXFP8 activations).  The bit layouts are the public OCP MX v1.0 / OFP8 ones:

* E2M1 (FP4): sign | 2-bit exponent (bias 1) | 1-bit mantissa, no inf/NaN.
* E4M3 (FN):  sign | 4-bit exponent (bias 7) | 3-bit mantissa, S.1111.111 is
  NaN, no infinity, largest finite 448.
* E8M0:       unsigned power-of-two exponent, bias 127; 0xFF is NaN.
* bf16:       the top half of an IEEE binary32.

Readings where the pages are silent (each one is listed with its reason in
the design notes):

* FP4 packing: byte ``b`` of a row holds element ``2b`` in bits 0-3 and
  element ``2b+1`` in bits 4-7.
* MXFP8 scale rule: the OCP rule ``floor(log2(amax)) - 8`` (8 = largest E4M3
  exponent), clamped to [-127, 127]; an all-zero block takes code 0.
* MXFP8 element rounding: round half to even onto the E4M3 grid, subnormals
  kept, saturating at +-448, sign of zero kept (-0 encodes as 0x80).
* Non-finite inputs are outside the method's domain and raise.
"""
import numpy as np

_F64 = np.float64


def _codes(codes):
    return np.asarray(codes).astype(np.int64)


def e2m1_decode(codes):
    """Value of each 4-bit E2M1 code (OCP MX: exponent bias 1, e=0 subnormal).

    Closed form: s = c>>3, e = (c>>1)&3, m = c&1;
    value = (-1)^s * (0.5*m if e == 0 else (1 + m/2) * 2^(e-1)).
    """
    c = np.arange(16)
    s = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    values = np.where(s == 1, -mag, mag).astype(_F64)   # the closed form at each of the 16 codes
    return values[np.asarray(codes).astype(np.intp) & 0xF]


def e4m3_decode(codes):
    """Value of each 8-bit E4M3 (FN) code; NaN for S.1111.111 (OFP8)."""
    c = _codes(codes) & 0xFF
    s = c >> 7
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where(s == 1, -mag, mag).astype(_F64)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def e8m0_decode(codes):
    """Value of each E8M0 scale code: 2^(c-127); NaN for 0xFF (OCP MX)."""
    c = _codes(codes) & 0xFF
    val = np.exp2(c - 127.0)
    return np.where(c == 0xFF, np.nan, val).astype(_F64)


def unpack_fp4(packed):
    """uint8 [..., K/2] -> uint8 codes [..., K]; element 2b is the low nibble of byte b."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _fp4_values(packed):
    """E2M1 values of packed FP4 bytes [..., K/2] -> [..., K] (fp64): each byte
    decodes to (E2M1 of its low nibble, E2M1 of its high nibble)."""
    b = np.arange(256)
    pairs = np.stack([e2m1_decode(b & 0xF), e2m1_decode(b >> 4)], axis=-1)   # [256, 2]
    p = np.asarray(packed, dtype=np.uint8)
    return np.take(pairs, p.astype(np.intp), axis=0).reshape(p.shape[:-1] + (p.shape[-1] * 2,))


def _apply_block_scales(vals, sc, group):
    """vals [..., K] times one scale per `group` consecutive elements of the last axis."""
    k = vals.shape[-1]
    if sc.shape[-1] * group != k:
        raise ValueError(f"block scales must hold one code per {group} elements")
    blocks = vals.reshape(vals.shape[:-1] + (k // group, group))
    blocks *= sc[..., None]
    return vals


def dequant_mxfp4(packed, scales):
    """MXFP4 block [N, K]: E2M1(code[n,k]) * E8M0(scale[n, k//32]), exact in fp64.

    packed: uint8 [N, K/2]; scales: uint8 [N, K/32] along the contraction axis.
    """
    sc = e8m0_decode(scales)
    if np.isnan(sc).any():
        raise ValueError("E8M0 scale 0xFF (NaN) in MXFP4 weights")
    return _apply_block_scales(_fp4_values(packed), sc, 32)


def dequant_nvfp4(packed, scales, global_scale):
    """NVFP4 block [N, K]: E2M1(code) * E4M3(scale[n, k//16]) * g, exact in fp64.

    ``global_scale`` is the fp32 tensor scale of this matrix (one per expert
    and matrix here: the per-tensor scale broadcast).
    """
    sc = e4m3_decode(scales)
    if np.isnan(sc).any():
        raise ValueError("E4M3 NaN block scale in NVFP4 weights")
    g = _F64(np.float32(global_scale))
    return _apply_block_scales(_fp4_values(packed), sc, 16) * g


def bf16_decode(bits):
    """uint16 bf16 bit patterns -> fp64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(_F64)


def _round_to_grid(mag, mant_bits, emin):
    """Round non-negative fp64 magnitudes to the nearest value of a binary
    format with ``mant_bits`` stored mantissa bits and smallest normal
    exponent ``emin`` (subnormals below it), ties to even.  No overflow
    handling: callers clamp first."""
    mag = np.asarray(mag, dtype=_F64)
    _, ex = np.frexp(mag)                 # mag = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, emin)   # floor(log2 mag), floored at emin
    ulp_exp = e - mant_bits
    q = np.ldexp(mag, -ulp_exp)            # exact: power-of-two scaling
    return np.ldexp(np.rint(q), ulp_exp)   # np.rint rounds half to even


def round_to_bf16(v):
    """Nearest bf16 value of each fp64 input, ties to even (fp64 result)."""
    v = np.asarray(v, dtype=_F64)
    if not np.isfinite(v).all():
        raise ValueError("non-finite value rounded to bf16")
    r = _round_to_grid(np.abs(v), 7, -126)
    r = np.where(r >= 2.0 ** 128, np.inf, r)
    return np.copysign(r, v)


def bf16_encode(v):
    """fp64 -> uint16 bf16 bits, round to nearest even (via round_to_bf16)."""
    r = round_to_bf16(v)
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _e4m3_encode_sat(q):
    """fp64 -> E4M3 codes: RNE, subnormals kept, saturating at +-448, sign kept."""
    q = np.asarray(q, dtype=_F64)
    neg = np.signbit(q)
    a = np.abs(q)
    r = np.where(a >= 448.0, 448.0, _round_to_grid(np.minimum(a, 448.0), 3, -6))
    # encode the (exactly representable) magnitude r
    _, ex = np.frexp(r)
    e = ex.astype(np.int64) - 1
    normal = r >= 2.0 ** -6
    m_norm = np.ldexp(r, -np.where(normal, e, 0)) * 8.0 - 8.0
    code_norm = ((e + 7) << 3) + m_norm.astype(np.int64)
    code_sub = np.ldexp(r, 9).astype(np.int64)          # r / 2^-9
    mag_code = np.where(normal, code_norm, code_sub)
    return (mag_code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_mxfp8(v):
    """MXFP8 quantization along the last axis (length a multiple of 32).

    Per block of 32 values: amax = max|v|; shared exponent
    s = clamp(floor(log2 amax) - 8, -127, 127) (s = -127 when amax = 0);
    scale code = s + 127; element code = E4M3_RNE_sat(v / 2^s).
    Returns (codes uint8 [..., K], scales uint8 [..., K/32]).
    """
    v = np.asarray(v, dtype=_F64)
    if not np.isfinite(v).all():
        raise ValueError("MXFP8 quantization of a non-finite value")
    k = v.shape[-1]
    if k % 32:
        raise ValueError("MXFP8 rows must be a multiple of 32 long")
    blocks = v.reshape(v.shape[:-1] + (k // 32, 32))
    amax = np.abs(blocks).max(axis=-1)
    _, ex = np.frexp(amax)
    s = np.clip(ex.astype(np.int64) - 1 - 8, -127, 127)
    s = np.where(amax == 0, -127, s)
    q = np.ldexp(blocks, -s[..., None])
    codes = _e4m3_encode_sat(q).reshape(v.shape)
    return codes, (s + 127).astype(np.uint8)


def dequant_mxfp8(codes, scales):
    """E4M3(code) * E8M0(scale) with one scale per 32 codes along the last axis."""
    vals = e4m3_decode(codes)
    sc = e8m0_decode(scales)
    return vals * np.repeat(sc, 32, axis=-1)


# E2M1 magnitudes in code order (OCP MX v1.0) and the finite E4M3 magnitudes
# in code order (codes 0x00 .. 0x7E), with the midpoints between neighbours
_E2M1_MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E4M3_MAGS = e4m3_decode(np.arange(0x7F))
_E2M1_MIDS = (_E2M1_MAGS[:-1] + _E2M1_MAGS[1:]) / 2.0
_E4M3_MIDS = (_E4M3_MAGS[:-1] + _E4M3_MAGS[1:]) / 2.0


def _nearest_index(a, thresholds):
    """Index i of the nearest grid value, given non-negative magnitudes ``a``
    and the midpoints between consecutive grid values already multiplied by
    the unit (``thresholds[..., i]`` lies between grid values i and i+1):
    the number of thresholds below ``a``, plus one where ``a`` equals an odd
    threshold (a tie goes to the even index).  Above the last threshold the
    result is the last index (saturation).  Exact when every threshold is an
    exact fp64 value."""
    idx = np.zeros(np.shape(a), dtype=np.int64)
    for i in range(thresholds.shape[-1]):
        t = thresholds[..., i]
        idx += (a > t).astype(np.int64)
        if i % 2 == 1:
            idx += (a == t).astype(np.int64)
    return idx


def quantize_nvfp4(v, global_scale):
    """NVFP4 quantization of activations along the last axis (length a multiple of 16).

    The vLLM b12x page ("Supported Configurations") lists NVFP4 activations
    for NVFP4 MoE, and the README names an NVFP4 row quantizer
    (quantization.nvfp4); neither gives the rule.  Reading, the NVFP4 format
    written out: with g the fp32 per-tensor scale of the activations (the
    checkpoint's input scale), each block of 16 takes the block scale s =
    the E4M3 value nearest to amax / (6 g) (ties to the even code, saturating
    at 448), and each element the E2M1 value nearest to v / (s g) (ties to the
    even code, saturating at 6, sign kept); a block whose scale is 0 takes
    codes 0.  Both nearest-value decisions are taken on the exact quotients:
    a magnitude is compared with the midpoints of the grid multiplied by the
    unit (6 g, or s g), and those products are exact in fp64 (a midpoint has at
    most 5 significant bits, 6 two, an E4M3 value four and g 24, so at most 31
    together).
    Returns (codes uint8 [..., K] unpacked, scales uint8 [..., K/16]).
    """
    v = np.asarray(v, dtype=_F64)
    if not np.isfinite(v).all():
        raise ValueError("NVFP4 quantization of a non-finite value")
    g = _F64(np.float32(global_scale))
    if not (np.isfinite(g) and g > 0):
        raise ValueError("NVFP4 activation scale must be finite and positive")
    k = v.shape[-1]
    if k % 16:
        raise ValueError("NVFP4 rows must be a multiple of 16 long")
    blocks = v.reshape(v.shape[:-1] + (k // 16, 16))
    mag = np.abs(blocks)
    amax = mag.max(axis=-1)
    scodes = _nearest_index(amax, _E4M3_MIDS * (6.0 * g)).astype(np.uint8)
    s = _E4M3_MAGS[scodes]
    unit = s * g                                            # exact: at most 28 significant bits
    mag_codes = _nearest_index(mag, _E2M1_MIDS * unit[..., None, None])
    mag_codes = np.where(unit[..., None] > 0, mag_codes, 0)
    codes = (mag_codes | np.where(np.signbit(blocks), 0x8, 0)).astype(np.uint8)
    return codes.reshape(v.shape), scodes


def nvfp4_values(codes, scales):
    """E2M1(code) * E4M3(scale) with one scale per 16 codes along the last axis
    (the round trip without the per-tensor scale, exact in fp64)."""
    sc = e4m3_decode(scales)
    if np.isnan(sc).any():
        raise ValueError("E4M3 NaN block scale")
    return e2m1_decode(codes) * np.repeat(sc, 16, axis=-1)


def nvfp4_roundtrip(v, global_scale):
    """g * E2M1 * E4M3 of quantize_nvfp4(v, g): the values the GEMMs see."""
    codes, scales = quantize_nvfp4(v, global_scale)
    return nvfp4_values(codes, scales) * _F64(np.float32(global_scale))
