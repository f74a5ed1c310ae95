"""Number formats and the packed storage layout (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix the ingredients of the storage format but not their exact
rounding: BF16 centroids and BF16 principal basis, INT2 residual codes packed
four per byte, uint8 centroid indices, bit-packed INT2 zero-points, and
scales / PSAC coefficients "in quantized formats" (QuantWM v2, App. D.1;
rainbus digest, method steps (3) and (4)).  The readings implemented here:

  * bf16 values are produced by round-to-nearest-even;
  * a scale is the smallest binary16 value h with m*h >= x ("rounded up" so
    that m steps of h always cover the range x);
  * an integer code is the round-half-to-even of the *exact* quotient a/b.
All of this is plain float64 arithmetic on exactly representable operands.
"""
from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0


# --------------------------------------------------------------------------
# bfloat16
# --------------------------------------------------------------------------
def bf16_rne(x) -> np.ndarray:
    """Round float64 values to bfloat16 (8 significant bits), ties to even.

    x = m * 2**e with 0.5 <= |m| < 1; the bf16 quantum in that binade is
    2**(e-8) (never below the subnormal quantum 2**-133).  Scaling by a power
    of two and numpy.rint (half-to-even) are exact in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - 8, -133)
    return np.ldexp(np.rint(np.ldexp(x, -q)), q)


def bf16_to_bits(x) -> np.ndarray:
    """uint16 bit pattern of bf16-valued numbers."""
    a = np.asarray(x, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("value is not bf16-representable")
    return (u >> 16).astype(np.uint16)


def bits_to_bf16(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# binary16 helpers
# --------------------------------------------------------------------------
def fp16_up_div(x, m: float):
    """Smallest binary16 h >= 0 with m*h >= x (x >= 0), i.e. fp16 round-up of x/m.

    Returns (h as float64, saturated mask).  Values above the fp16 range
    saturate to 65504 and are flagged.  The first guess comes from numpy's
    float64->float16 conversion; it is then corrected with exact products
    m*h (an 11-bit h times a small integer m is exact in float64).
    """
    x = np.asarray(x, dtype=np.float64)
    sat = x > m * FP16_MAX
    y = np.where(sat, 0.0, x / m)
    h = y.astype(np.float16)
    inf16 = np.float16(np.inf)
    zero16 = np.float16(0)
    with np.errstate(over="ignore"):
        for _ in range(2):
            low = (m * h.astype(np.float64)) < x
            h = np.where(low, np.nextafter(h, inf16), h)
            prev = np.nextafter(h, zero16)
            down = (h > 0) & ((m * prev.astype(np.float64)) >= x)
            h = np.where(down, prev, h)
    h = np.where(sat, np.float16(FP16_MAX), h)
    return h.astype(np.float64), sat


def fp16_bits(h) -> np.ndarray:
    return np.asarray(h, dtype=np.float64).astype(np.float16).view(np.uint16)


def bits_to_fp16(b) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def rne_quotient(a, b) -> np.ndarray:
    """Round-half-to-even of the exact quotient a/b (b > 0 a binary16 value).

    A float64 division gives n0 within one of the answer; the decision is then
    made with the exact products (n +- 1/2) * b (at most 20 significant bits).
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    n = np.rint(a / b)
    n = n + (a > (n + 0.5) * b)
    n = n - (a < (n - 0.5) * b)
    up_tie = a == (n + 0.5) * b          # exactly halfway between n and n+1
    n = np.where(up_tie & (np.mod(n, 2) != 0), n + 1, n)
    dn_tie = a == (n - 0.5) * b          # exactly halfway between n-1 and n
    n = np.where(dn_tie & (np.mod(n, 2) != 0), n - 1, n)
    return n


# --------------------------------------------------------------------------
# packed layout (per head): codes [T][d/4] u8, idx [T] u8, scale [T][G] fp16,
# zeros [ceil(T/2)] u8, c [T][r] i8, c_scale [T] fp16
# --------------------------------------------------------------------------
def pack_codes(q: np.ndarray) -> np.ndarray:
    """q [T][d] in 0..3 -> [T][d/4] bytes; channel 4b+i sits at bits 2i..2i+1 of byte b."""
    q = np.asarray(q, dtype=np.uint8)
    T, d = q.shape
    q4 = q.reshape(T, d // 4, 4)
    return (q4[..., 0] | (q4[..., 1] << 2) | (q4[..., 2] << 4) | (q4[..., 3] << 6)).astype(np.uint8)


def unpack_codes(b: np.ndarray, d: int) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    T = b.shape[0]
    out = np.empty((T, d // 4, 4), np.uint8)
    for i in range(4):
        out[..., i] = (b >> (2 * i)) & 3
    return out.reshape(T, d)


def pack_zeros(z: np.ndarray) -> np.ndarray:
    """z [T][G=2] in 0..3 -> [ceil(T/2)] bytes.

    Per token a 4-bit field z0 | z1 << 2; token 2m in the low nibble of byte m,
    token 2m+1 in the high nibble.
    """
    z = np.asarray(z, dtype=np.uint8)
    T = z.shape[0]
    nib = (z[:, 0] | (z[:, 1] << 2)).astype(np.uint8)
    if T % 2:
        nib = np.concatenate([nib, np.zeros(1, np.uint8)])
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def unpack_zeros(b: np.ndarray, T: int) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    nib = np.empty(2 * b.shape[0], np.uint8)
    nib[0::2] = b & 0xF
    nib[1::2] = b >> 4
    nib = nib[:T]
    return np.stack([nib & 3, (nib >> 2) & 3], axis=1)
