"""Number formats of the FP4 microscaling path (oracle; test infrastructure).

E2M1  -- the 4-bit element: 1 sign, 2 exponent and 1 mantissa bit, bias 1,
         no Inf/NaN.  Non-negative magnitudes by code index 0..7:
         0, 0.5, 1, 1.5, 2, 3, 4, 6.  ("Resumo Técnico: ScaleSweep",
         Declaração do Problema, names FP4 E2M1 as the NVFP4 element type;
         "Resumo Técnico: TORQ", 1. Declaração do Problema, names e2m1 codes.)
E4M3  -- the NVFP4 block scale: FP8 with 4 exponent bits (bias 7) and 3
         mantissa bits, no Inf; 0x7F is NaN, so 126 positive finite values
         0x01..0x7E, the largest 448 ("Resumo Técnico: ScaleSweep",
         2. Limites Teóricos para Varredura Eficiente: the exhaustive sweep
         runs over the 126 positive finite FP8 values).
E8M0  -- the MXFP4 block scale: a power of two 2**(b-127), b in 0..254
         ("Bridging the Gap ... Microscaling FP4", 1. O Problema: MXFP4
         scales are powers of two in E8M0).

Every function here works from these definitions by nearest-value search
over the enumerated value set; nothing uses bit tricks.
"""

import numpy as np

# ---------------------------------------------------------------- E2M1 ----
# magnitudes by code index; the code of a signed value is (sign << 3) | index
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)
# decision points between neighbouring magnitudes (all exact in float32)
E2M1_MIDPOINTS = ((E2M1_VALUES[:-1].astype(np.float64) + E2M1_VALUES[1:]) / 2).astype(np.float32)


def e2m1_rne_index(y):
    """Index (0..7) of the E2M1 magnitude nearest to y >= 0.

    Round to nearest; a value exactly half-way between two magnitudes goes to
    the one with the even code index; values above 6 saturate to 6 (the format
    has no infinity).  ``y`` is float32; comparisons with the float32
    midpoints are exact.
    """
    y = np.asarray(y, dtype=np.float32)
    below = np.searchsorted(E2M1_MIDPOINTS, y, side="left")   # midpoints < y
    at_or_below = np.searchsorted(E2M1_MIDPOINTS, y, side="right")  # midpoints <= y
    tie = at_or_below != below  # y equals midpoint[below]: neighbours are below, below+1
    idx = np.where(tie, below + (below & 1), below)
    return idx.astype(np.uint8)


def e2m1_value(idx):
    """Magnitude of an E2M1 code index (float32)."""
    return E2M1_VALUES[np.asarray(idx, dtype=np.int64)]


# ---------------------------------------------------------------- E4M3 ----
def e4m3_decode_pattern(p):
    """Exact value (float64) of a non-negative E4M3 bit pattern 0..126."""
    p = int(p)
    if not 0 <= p <= 126:
        raise ValueError("pattern outside the non-negative finite E4M3 range")
    exp_field, man_field = p >> 3, p & 7
    if exp_field == 0:                      # subnormal: m/8 * 2**(1-7)
        return man_field / 8.0 * 2.0 ** -6
    return (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


# value of every non-negative pattern (index = pattern), exact in float64 and float32
E4M3_VALUES64 = np.array([e4m3_decode_pattern(p) for p in range(127)], dtype=np.float64)
E4M3_VALUES = E4M3_VALUES64.astype(np.float32)
E4M3_MAX_PATTERN = 126          # 0x7E = 448
_E4M3_MIDPOINTS64 = (E4M3_VALUES64[:-1] + E4M3_VALUES64[1:]) / 2


def e4m3_rne_pattern(t):
    """Non-negative E4M3 pattern (0..126) nearest to t >= 0.

    Ties go to the even pattern; values above 448 saturate to 0x7E.  The
    comparison runs in float64, where both t (a float32) and the midpoints of
    neighbouring E4M3 values are exact.
    """
    t = np.asarray(t, dtype=np.float32).astype(np.float64)
    below = np.searchsorted(_E4M3_MIDPOINTS64, t, side="left")
    at_or_below = np.searchsorted(_E4M3_MIDPOINTS64, t, side="right")
    tie = at_or_below != below
    return np.where(tie, below + (below & 1), below).astype(np.int64)


def e4m3_reciprocal_table():
    """fp32(1 / V[p]) for p = 1..126 (index 0 unused, set to 0).

    Each entry is one correctly rounded float32 division.
    """
    r = np.zeros(127, dtype=np.float32)
    r[1:] = np.float32(1.0) / E4M3_VALUES[1:]
    return r


# ---------------------------------------------------------------- E8M0 ----
def e8m0_decode(b):
    """Value of an E8M0 byte (0..254) as float64: 2**(b - 127)."""
    b = np.asarray(b, dtype=np.int64)
    if np.any((b < 0) | (b > 254)):
        raise ValueError("E8M0 byte outside 0..254 (255 is NaN)")
    return np.ldexp(1.0, b - 127)


def pow2_f32(e):
    """2**e as float32 for integer e in [-149, 127] (exact; subnormal below -126)."""
    e = np.asarray(e, dtype=np.int64)
    return np.ldexp(np.float64(1.0), e).astype(np.float32)
