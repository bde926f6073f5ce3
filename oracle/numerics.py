"""Storage formats the oracle reads: bf16 bit patterns and FP8 E4M3FN codes.

TEST INFRASTRUCTURE (see the package docstring).

* bf16 is the dtype of the drafter weights, of the target's shared embedding
  and LM head, and of the captured hidden stack ([Head/atlas], fields ``fc``,
  ``lm_head_shared``; [DraftProposer], ``propose`` arguments). Widening a
  bf16 bit pattern to float is exact: the 16 bits are the top half of an
  IEEE binary32.
* FP8 E4M3 is the format of the optional LM-head mirror ([Head/atlas], field
  ``lm_head_shared_fp8``: E4M3 codes plus one f32 scale per vocab row) and of
  the paged KV cache ([Head/atlas], field ``kv_cache``). The pages do not say
  which E4M3 variant; the OCP "E4M3FN" encoding is taken (bias 7, no
  infinities, S.1111.111 is NaN, largest finite magnitude 448). Encoding
  rounds to nearest, ties to even, and saturates to +-448 (reading: the pages
  give no overflow rule).

Pinned by tests/test_oracle_numerics.py against ``torch.bfloat16`` and
``torch.float8_e4m3fn`` conversions and against hand-known codes.
"""
import numpy as np

E4M3_MAX = 448.0


def bf16_to_f64(bits):
    """Widen bf16 bit patterns (uint16 array) to float64, exactly."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_round(x):
    """Round to bf16 storage and widen back: the value passes through float32
    (the precision the cache's producer holds it in), then rounds to the
    nearest bf16, ties to even. Used for the paged bf16 KV cache
    ([Head/metrale], field ``kv_cache``)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    r = ((b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)).astype(np.uint16)
    return bf16_to_f64(r)


def stored_to_f64(x):
    """A stored tensor as float64.

    uint16 arrays are bf16 bit patterns; float32 / float64 arrays are used as
    given (the tiny workload's fp32 weights).
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return bf16_to_f64(x)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {x.dtype}")


def e4m3_decode(codes):
    """Decode E4M3FN codes (uint8 array) to float64.

    Value of a code with sign s, 4-bit exponent e and 3-bit mantissa m:
    e == 0 gives (-1)^s * m/8 * 2^-6 (subnormal); otherwise
    (-1)^s * (1 + m/8) * 2^(e-7); e == 15 and m == 7 is NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _e4m3_finite_table():
    """All non-negative finite E4M3FN values with their codes, ascending."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)  # 0x00..0x7E; 0x7F is NaN
    vals = e4m3_decode(codes)
    return codes, vals


_E4M3_CODES, _E4M3_VALS = _e4m3_finite_table()


def e4m3_encode(x):
    """Encode float values to E4M3FN codes: round to nearest, ties to even
    code (even mantissa), saturate to +-448. NaN input is not supported.

    Implemented as a nearest-value search over the 127 non-negative finite
    codes, so it follows the definition rather than bit tricks.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("NaN has no saturating E4M3 encoding here")
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # index of the largest table value <= a
    hi = np.searchsorted(_E4M3_VALS, a, side="right")
    lo = np.clip(hi - 1, 0, len(_E4M3_VALS) - 1)
    up = np.clip(hi, 0, len(_E4M3_VALS) - 1)
    dlo = a - _E4M3_VALS[lo]
    dup = _E4M3_VALS[up] - a
    code_lo = _E4M3_CODES[lo]
    code_up = _E4M3_CODES[up]
    # ties go to the even code (mantissa LSB clear)
    choose_up = (dup < dlo) | ((dup == dlo) & ((code_lo & 1) == 1))
    code = np.where(choose_up, code_up, code_lo).astype(np.uint8)
    # the sign bit follows the input's sign bit (so -0.0 encodes as 0x80)
    return np.where(sign, code | np.uint8(0x80), code).astype(np.uint8)
