"""Number formats of the MoE layer step, decoded and encoded from their definitions.

Test infrastructure: this module belongs to the CPU oracle.  Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the GPU
library never does.

Formats (all decoded exactly into float64):

* bf16 -- the upper 16 bits of an IEEE-754 binary32.
* e4m3 -- OCP FP8 E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
  bits, no infinities, NaN only at S.1111.111, largest finite 448, smallest
  subnormal 2**-9.  The pages state the KV cache is stored in fp8
  ("Muse Spark Open Hits 433 tok/s Per User on TPU v7 Megakernel", opening
  paragraphs); the e4m3 flavour with no scale is this implementation's reading.
* e2m1 -- OCP FP4: 1 sign bit (bit 3), 2 exponent bits (bias 1), 1 mantissa
  bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
* NVFP4-style block format -- e2m1 elements, one e4m3 scale per 16 consecutive
  elements along the reduction dimension, one fp32 scale per matrix.  The
  pages give the one-scale-per-16-values rule ("Optimizing Muse Spark Open on
  TPU v7 with SGLang-TorchTPU", section "Expert Weight Quantization"); the
  per-matrix fp32 scale and the nibble order (even element in the low nibble)
  are this implementation's reading.
"""
import numpy as np


# ---------------------------------------------------------------- bf16 / f32

def bf16_bits_to_f64(u16):
    """bf16 bit patterns (uint16 array) -> float64, exact."""
    u16 = np.asarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_to_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even.

    Works directly from the float64 value (no detour through float32, so
    there is no double rounding).  Normal range only: |x| below 2**-126 is
    rounded on the subnormal grid 2**-133; overflow is not handled (the layer
    never produces values near 3.4e38)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                      # |x| in [2**(e-1), 2**e)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.round(x / ulp) * ulp          # np.round: half to even


def f64_to_bf16_bits(x):
    """Encode float64 -> bf16 bit patterns with round-to-nearest-even."""
    r = round_to_bf16(x).astype(np.float32)  # exact: r is a bf16 value
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------- e4m3

def _e4m3_value(b):
    s = -1.0 if (b & 0x80) else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return np.nan
    if e == 0:
        return s * (m / 8.0) * 2.0 ** -6
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([_e4m3_value(b) for b in range(256)], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_bits_to_f64(u8):
    """e4m3 bit patterns (uint8 array) -> float64, exact (NaN for 0x7F/0xFF)."""
    return E4M3_TABLE[np.asarray(u8, dtype=np.uint8)]


def round_to_e4m3(x):
    """Round float64 values to the nearest e4m3 value, ties to even,
    saturating to +-448 (the cache format has no infinity)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    # normals: |x| in [2**(e-1), 2**e) has 3 mantissa bits -> ulp 2**(e-4);
    # below 2**-6 the grid is the subnormal spacing 2**-9.
    ulp = np.ldexp(1.0, np.maximum(e - 4, -9))
    r = np.round(x / ulp) * ulp
    return np.clip(r, -E4M3_MAX, E4M3_MAX)


_E4M3_POS_VALUES = E4M3_TABLE[:0x7F]        # codes 0..126 are increasing


def f64_to_e4m3_bits(x):
    """Encode float64 -> e4m3 bit patterns (RNE, saturating)."""
    r = round_to_e4m3(x)
    mag = np.abs(r)
    code = np.searchsorted(_E4M3_POS_VALUES, mag).astype(np.uint8)
    assert np.all(_E4M3_POS_VALUES[code] == mag)
    sign = np.where(np.signbit(r), np.uint8(0x80), np.uint8(0))
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------------- e2m1

def _e2m1_value(c):
    s = -1.0 if (c & 0x8) else 1.0
    e = (c >> 1) & 0x3
    m = c & 0x1
    if e == 0:
        return s * 0.5 * m
    return s * (1.0 + 0.5 * m) * 2.0 ** (e - 1)


E2M1_TABLE = np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e2m1_codes_to_f64(codes):
    """4-bit codes (0..15, any integer array) -> float64."""
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def unpack_nibbles(packed):
    """uint8 [..., n/2] -> codes [..., n]; element 2i is the low nibble of
    byte i, element 2i+1 the high nibble."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def nvfp4_to_f64(packed, scales, gscale):
    """Decode one NVFP4-style matrix.

    packed: uint8 [rows][cols/2]; scales: uint8 e4m3 [rows][cols/16];
    gscale: the matrix's fp32 scale.  value = e2m1(code) * e4m3(scale) * g.
    """
    vals = e2m1_codes_to_f64(unpack_nibbles(packed))
    rows, cols = vals.shape
    s = e4m3_bits_to_f64(scales)
    assert s.shape == (rows, cols // 16)
    return vals * np.repeat(s, 16, axis=1) * np.float64(np.float32(gscale))


# ------------------------------------------------------- dispatch by dtype

def decode(raw, dtype):
    """Decode a dense tensor stored as 'f32' (float32), 'bf16' (uint16 bits)
    or 'e4m3' (uint8 bits)."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if dtype == "e4m3":
        return e4m3_bits_to_f64(raw)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_to_dtype(x, dtype):
    """Value of x after storing it in `dtype` (RNE; e4m3 saturates)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "e4m3":
        return round_to_e4m3(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def encode(x, dtype):
    """Bit patterns of x stored in `dtype` (float32 array for 'f32')."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    if dtype == "e4m3":
        return f64_to_e4m3_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")
