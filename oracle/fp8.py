"""FP8 (E4M3) block quantisation and the FP8 forward, by their definitions.

TEST INFRASTRUCTURE ONLY, like the rest of this package: imported by the test suite,
the package smoke check and the benchmark's ``cpu_baseline`` leg, never by the HIP
library, with which it shares no code.

Source: the V2/V3 article (aiqz.cc), section FP8低精度 and its formula block: E4M3 is
the forward format, its largest value is 448; a first pass over each block finds
max|x| and sets the step Delta = max|x| / 448, a second pass stores round(x / Delta)
in FP8, and the Q K^T product runs on the FP8 values with an FP32 accumulator.

Readings taken where the article is silent:

* E4M3 is the OCP 8-bit format (1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits; subnormals; signed zero; no infinities; 448 is the largest finite value).  "round" is
  round to the nearest representable E4M3 value, ties to the even code; x / Delta
  never exceeds 448 in magnitude by more than rounding, and is clamped to it.
* x / Delta is one fp32 division (the precision the kernel uses), so both sides
  take the same rounding decisions; Delta is max|x| (fp32) / 448 in fp32.  A block
  of zeros has Delta = 1.
* Blocks are ``block`` consecutive rows of one head: for Q the rows of a query
  block, for K those of a key block.  Only Q and K are quantised (the article
  quantises those two); V and the probabilities stay in bf16, so P V is the bf16
  product of the plain forward.
* The forward attends with the dequantised values x_hat * Delta, exactly.
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .attention import attn_fwd

E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, indexed by code (0x00 .. 0x7E)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(2.0 ** -6 * (m / 8.0))          # subnormal
        else:
            vals.append(2.0 ** (e - 7) * (1.0 + m / 8.0))
    return np.array(vals, dtype=np.float64)


_VALS = e4m3_values()


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code of each (finite) value, ties to the even code; |x| > 448
    saturates to 448.  Returns uint8."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_VALS, a, side="left")       # first value >= a
    hi = np.minimum(hi, len(_VALS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _VALS[lo]
    d_hi = _VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _VALS[hi], hi, code).astype(np.uint8)   # exact hits
    sign = np.signbit(x).astype(np.uint8) << 7   # a negative value rounding to 0 is -0
    return code | sign


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 codes (uint8), float64."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = _VALS[np.minimum(c & 0x7F, 0x7E)]
    return np.where(c & 0x80, -mag, mag)


def quantize_blocks(x, block: int) -> Tuple[np.ndarray, np.ndarray]:
    """Two-pass block quantisation of x [B, H, N, D] (fp32 values).

    Pass 1: Delta[b, h, n // block] = max|x| over the block's rows / 448 (fp32).
    Pass 2: codes = E4M3(x / Delta) with one fp32 division per element.
    Returns (codes uint8 [B, H, N, D], Delta float32 [B, H, ceil(N / block)]).
    """
    x = np.asarray(x, dtype=np.float32)
    b_, h_, n, d = x.shape
    nb = (n + block - 1) // block
    delta = np.ones((b_, h_, nb), dtype=np.float32)
    codes = np.zeros(x.shape, dtype=np.uint8)
    for j in range(nb):
        xs = x[:, :, j * block:(j + 1) * block]
        amax = np.max(np.abs(xs), axis=(2, 3)) if xs.size else np.zeros((b_, h_), np.float32)
        dj = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        delta[:, :, j] = dj
        codes[:, :, j * block:(j + 1) * block] = e4m3_encode((xs / dj[:, :, None, None]).astype(np.float32))
    return codes, delta


def dequantize_blocks(codes, delta, block: int) -> np.ndarray:
    """x_hat * Delta per block, exactly (float64)."""
    vals = e4m3_decode(codes)
    rep = np.repeat(np.asarray(delta, dtype=np.float64), block, axis=2)[:, :, :vals.shape[2]]
    return vals * rep[..., None]


def attn_fwd_fp8(q_codes, q_delta, k_codes, k_delta, v, block: int, scale: Optional[float] = None,
                 causal: bool = False, rows=None):
    """The FP8 forward: S = scale * (Delta_q q_hat)(Delta_k k_hat)^T, then the plain
    softmax and P V with V as given.  Returns (O, LSE) as ``attn_fwd``."""
    qd = dequantize_blocks(q_codes, q_delta, block)
    kd = dequantize_blocks(k_codes, k_delta, block)
    if scale is None:
        scale = 1.0 / np.sqrt(qd.shape[-1])
    return attn_fwd(qd, kd, v, scale, causal, None, rows)
