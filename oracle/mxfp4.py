"""Plain float64 CPU oracle of MXFP4 expert weights: decoding, the expert block
layout and the quantiser.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: imported by tests,
never by the GPU library, and sharing no code with it.

The pages name the format and nothing more: the Kimi K3 engine streams its
experts as MXFP4 straight from the original checkpoint, with nothing to
convert (ssnai.com digest, "前置条件" (prerequisites) and the per-model notes
quoted under "Get started").  The encoding is the public OCP Microscaling
Formats (MX) v1.0 specification, which this module follows:

* a block of 32 consecutive elements shares one scale X, an E8M0 number:
  8 exponent bits E, no sign, no mantissa, X = 2^(E - 127); E = 255 is NaN;
* each element is FP4 E2M1: a sign bit, two exponent bits e (bias 1) and one
  mantissa bit m; e = 0 is subnormal, 0.m * 2^(1 - 1) = m / 2; otherwise
  1.m * 2^(e - 1).  The 16 codes give +-{0, 0.5, 1, 1.5, 2, 3, 4, 6};
* the element's value is X times the E2M1 value.

Quantising (the spec's conversion from higher precision): per block, the
shared exponent is floor(log2(max |v|)) - emax with emax = 2 (the largest
E2M1 exponent), clamped to the E8M0 range; every v / X is rounded to the
nearest E2M1 value, ties to the even mantissa, and values beyond 6 saturate
to +-6.  An all-zero block is given E = 0 and zero elements (the spec leaves
its scale open).

Readings (where neither the pages nor the spec fix a point):

* blocks run along the input dimension of each matrix (as the int4 container's
  64-column groups do);
* an expert block holds the three matrices' element nibbles in the int4
  container's order (element 2j in the low nibble of byte j, gate, up, down),
  then the three matrices' E8M0 scale bytes ([out][in / 32] each), so its size,
  3*d*f/2 + 3*d*f/32 bytes, equals the int4 gs64 block's;
* activations stay as they are (bf16 or float32): the weights are decoded
  exactly and the FFN is the same SwiGLU as for int4 experts.
"""
from __future__ import annotations

import numpy as np

MX_BLOCK = 32       # elements sharing one E8M0 scale
E2M1_EMAX = 2       # exponent of the largest E2M1 normal (6 = 1.5 * 2^2)
E8M0_BIAS = 127


def decode_e2m1(codes) -> np.ndarray:
    """FP4 E2M1 codes (0..15) -> float64 values, from the bit fields."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return sign * mag


def decode_e8m0(e) -> np.ndarray:
    """E8M0 scale bytes -> float64 2^(E - 127); 255 -> NaN."""
    e = np.asarray(e, dtype=np.int64)
    return np.where(e == 255, np.nan, np.exp2(e.astype(np.float64) - E8M0_BIAS))


def unpack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Bytes [rows, cols/2] -> nibbles [rows, cols]; element 2j in the low
    nibble of byte j."""
    codes = np.asarray(codes, dtype=np.uint8)
    out = np.empty((codes.shape[0], 2 * codes.shape[1]), dtype=np.int64)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Nibbles [rows, cols] -> bytes [rows, cols/2] (inverse of unpack_nibbles)."""
    q = np.asarray(q, dtype=np.int64).astype(np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """W[r, c] = E2M1(q[r, c]) * 2^(E[r, c // 32] - 127), float64 (exact)."""
    v = decode_e2m1(unpack_nibbles(codes))
    x = np.repeat(decode_e8m0(scales), MX_BLOCK, axis=1)
    assert x.shape == v.shape
    return v * x


def block_bytes(d: int, f: int) -> int:
    """3*d*f nibbles plus one scale byte per 32 elements."""
    n = 3 * d * f
    return n // 2 + n // MX_BLOCK


def split_block(block: np.ndarray, d: int, f: int):
    """One MXFP4 expert block -> (q_gate [f, d/2], q_up, q_down [d, f/2],
    x_gate [f, d/32] uint8, x_up, x_down [d, f/32])."""
    block = np.asarray(block, dtype=np.uint8)
    parts, pos = [], 0
    for rows, cols in ((f, d), (f, d), (d, f)):
        n = rows * cols // 2
        parts.append(block[pos:pos + n].reshape(rows, cols // 2))
        pos += n
    for rows, cols in ((f, d), (f, d), (d, f)):
        n = rows * (cols // MX_BLOCK)
        parts.append(block[pos:pos + n].reshape(rows, cols // MX_BLOCK))
        pos += n
    assert pos == block.size, "block size does not match (d, f)"
    return parts


def expert_weights(block: np.ndarray, d: int, f: int):
    """Decoded (W_gate [f, d], W_up [f, d], W_down [d, f]) of one block."""
    qg, qu, qd, xg, xu, xd = split_block(block, d, f)
    return dequant(qg, xg), dequant(qu, xu), dequant(qd, xd)


def shared_exponent(amax) -> np.ndarray:
    """E8M0 byte of a block with largest magnitude amax:
    floor(log2(amax)) - 2 + 127, clamped to [0, 254]; 0 for amax == 0.
    frexp gives amax = m * 2^k with m in [0.5, 1), so floor(log2 amax) = k - 1
    exactly (no logarithm rounding)."""
    a = np.asarray(amax, dtype=np.float64)
    _, k = np.frexp(a)
    e = (k.astype(np.int64) - 1) - E2M1_EMAX + E8M0_BIAS
    return np.where(a == 0.0, 0, np.clip(e, 0, 254)).astype(np.int64)


def round_e2m1(r) -> np.ndarray:
    """Nearest E2M1 code to r (float64), ties to the even mantissa (m = 0),
    saturating at +-6.  Written as a search over the eight magnitudes."""
    r = np.asarray(r, dtype=np.float64)
    mags = decode_e2m1(np.arange(8))                 # 0, .5, 1, 1.5, 2, 3, 4, 6
    a = np.minimum(np.abs(r), 6.0)
    dist = np.abs(a[..., None] - mags)               # [..., 8]
    best = np.min(dist, axis=-1, keepdims=True)
    tie_ok = dist == best
    # among the nearest magnitudes take the one with an even mantissa bit
    even = (np.arange(8) & 1) == 0
    pick = np.where(np.any(tie_ok & even, axis=-1), np.argmax(tie_ok & even, axis=-1),
                    np.argmax(tie_ok, axis=-1))
    neg = (r < 0) & (pick > 0)
    return (pick + np.where(neg, 8, 0)).astype(np.int64)


def quantize(w: np.ndarray):
    """Float weights w [N, K] (K a multiple of 32) -> (codes [N, K/2] uint8,
    scales [N, K/32] uint8)."""
    w = np.asarray(w, dtype=np.float64)
    n, k = w.shape
    g = w.reshape(n, k // MX_BLOCK, MX_BLOCK)
    e = shared_exponent(np.max(np.abs(g), axis=2))
    x = np.exp2(e.astype(np.float64) - E8M0_BIAS)
    q = round_e2m1(g / x[:, :, None]).reshape(n, k)
    return pack_nibbles(q), e.astype(np.uint8)
