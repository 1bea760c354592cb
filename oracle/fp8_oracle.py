"""Plain CPU oracle of the FP8 variant of the expert GEMMs.  TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module; the product never does.  It shares no code with
the GPU path.

What it computes (MaxText pull request "[Draft] Integrate TE/JAX GroupedGEMM
for MoE": the run's ``quantization=fp8`` option and the review of the
quantizer set-up, current-tensor scaling with e4m3 in the forward and e5m2
in the backward, two quantized copies of each operand; TransformerEngine MoE
block pull request, commit notes: per-expert amax of the expert weights):

  format       OCP FP8: E4M3FN (bias 7, 3 mantissa bits, largest finite 448,
               no infinities) and E5M2 (bias 15, 2 mantissa bits, largest
               finite 57344); both with subnormals.
  scaling      current scaling: amax = max |x| over the scaling unit (the
               whole tensor for activations and gradients, one expert's
               matrix for the expert weights); scale = fmax / amax (1 when
               amax is 0) and scale_inv = 1 / scale, both float32.
  quantize     q = fp8(float32(x) * scale): the float32 product rounded to
               the nearest FP8 value, ties to even, magnitudes above fmax
               saturate to fmax.  Where the pages leave the rounding open
               this takes round-to-nearest-even with saturation, and the
               float32 arithmetic of the scaled value, so that the GPU and
               the oracle decide every code in the same precision.
  dequantize   decode(q) * scale_inv, exact in float64.
  fp8 GEMMs    the grouped GEMMs of the block on dequantized operands,
               accumulated in float64.
"""
from __future__ import annotations

import numpy as np

E4M3 = "e4m3"
E5M2 = "e5m2"
# (exponent bias, mantissa bits, largest finite value)
_FMT = {E4M3: (7, 3, 448.0), E5M2: (15, 2, 57344.0)}


def fmax(fmt: str) -> float:
    return _FMT[fmt][2]


def decode(codes, fmt: str) -> np.ndarray:
    """float64 value of each FP8 code (uint8).  E4M3FN codes 0x7F/0xFF are
    NaN; E5M2 exponent 31 is infinity (mantissa 0) or NaN."""
    bias, mb, _ = _FMT[fmt]
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> mb) & ((0x80 >> mb) - 1)
    m = c & ((1 << mb) - 1)
    normal = np.ldexp(1.0 + m / (1 << mb), (e - bias).astype(np.int64))
    sub = np.ldexp(m / (1 << mb), 1 - bias)
    v = sign * np.where(e == 0, sub, normal)
    if fmt == E4M3:
        v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    else:
        emax = (0x80 >> mb) - 1
        v = np.where(e == emax, np.where(m == 0, sign * np.inf, np.nan), v)
    return v


def encode(v, fmt: str) -> np.ndarray:
    """FP8 codes (uint8) of finite values v: round to nearest, ties to even,
    saturating at the largest finite value; the sign is kept (also for a
    result of zero)."""
    bias, mb, top = _FMT[fmt]
    v = np.asarray(v, dtype=np.float64)
    assert np.isfinite(v).all()
    a = np.abs(v)
    emin = 1 - bias
    # binade exponent of |v| (frexp: a = f 2^x with f in [0.5, 1)), clamped to
    # the subnormal range; the spacing there is 2^(e - mb)
    _, x = np.frexp(a)
    e = np.maximum(x - 1, emin)
    quantum = np.ldexp(1.0, (e - mb).astype(np.int64))
    r = np.round(a / quantum) * quantum          # numpy rounds halves to even
    r = np.minimum(r, top)                       # saturate
    # encode the rounded magnitude
    _, xr = np.frexp(r)
    er = np.where(r >= np.ldexp(1.0, emin), xr - 1, emin - 1)   # emin - 1: subnormal/zero
    sub = r < np.ldexp(1.0, emin)
    mant_sub = np.round(r / np.ldexp(1.0, emin - mb)).astype(np.int64)
    mant_norm = np.round((r / np.ldexp(1.0, er.astype(np.int64)) - 1.0) * (1 << mb)).astype(np.int64)
    code = np.where(sub, mant_sub, ((er + bias).astype(np.int64) << mb) | mant_norm)
    code = code | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


def scales(amax, fmt: str):
    """(scale, scale_inv) float32 for amax (array or scalar): fmax / amax
    and 1 / scale in float32 arithmetic; amax 0 gives scale 1."""
    am = np.asarray(amax, dtype=np.float32)
    f = np.float32(fmax(fmt))
    with np.errstate(divide="ignore"):
        s = np.where(am > 0, f / np.where(am > 0, am, np.float32(1)), np.float32(1)).astype(np.float32)
    return s, (np.float32(1) / s).astype(np.float32)


def amax_groups(x, group_rows: int | None = None) -> np.ndarray:
    """max |x| of a 2-D float32 array, over all rows (one scaling unit) or
    over consecutive blocks of group_rows rows ([G] values)."""
    a = np.abs(np.asarray(x, dtype=np.float32))
    if group_rows is None:
        return np.array([a.max() if a.size else 0.0], dtype=np.float32)
    G = a.shape[0] // group_rows
    return np.array([a[g * group_rows:(g + 1) * group_rows].max() if group_rows * a.shape[1] else 0.0
                     for g in range(G)], dtype=np.float32)


def quantize(x, fmt: str, scale) -> np.ndarray:
    """FP8 codes of float32 x times a float32 scale (scalar, or one per
    leading-axis entry of a 3-D x), the product taken in float32."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(scale, dtype=np.float32)
    if s.ndim == 1 and x.ndim == 3:
        s = s[:, None, None]
    prod = (x * s).astype(np.float32)
    return encode(prod.astype(np.float64), fmt)


def dequantize(codes, fmt: str, scale_inv) -> np.ndarray:
    """decode(codes) * scale_inv in float64 (scalar, or one per leading-axis
    entry of a 3-D array)."""
    v = decode(codes, fmt)
    si = np.asarray(scale_inv, dtype=np.float64)
    if si.ndim == 1 and v.ndim == 3:
        si = si[:, None, None]
    return v * si


def quantize_tensor(x, fmt: str):
    """Current scaling of a whole activation or gradient tensor: returns
    (codes, scale_inv float32 scalar, dequantized float64)."""
    am = amax_groups(np.asarray(x, dtype=np.float32).reshape(np.shape(x)[0], -1))[0]
    s, si = scales(am, fmt)
    q = quantize(x, fmt, s)
    return q, si, dequantize(q, fmt, si)


def quantize_experts(w, fmt: str):
    """Current scaling per expert of a weight stack [E, a, b]: returns
    (codes, scale_inv float32 [E], dequantized float64)."""
    w = np.asarray(w, dtype=np.float32)
    E = w.shape[0]
    am = amax_groups(w.reshape(E * w.shape[1], w.shape[2]), w.shape[1]) if E else np.zeros(0, np.float32)
    s, si = scales(am, fmt)
    q = quantize(w, fmt, s)
    return q, si, dequantize(q, fmt, si)
