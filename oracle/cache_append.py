"""Plain CPU oracle for appending one decoded token to the latent cache: the
step that writes what the decode path later reads.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code, table
or constant with the HIP path.

What it follows ("DeepSeek's KV Cache: From 3.9 MB to 890 B per Token"):
  * section "MLA: the cache holds one latent" (Figure 3): per token the cache
    keeps the latent C^KV, which gets no rotation, and one rotary key K^R with
    RoPE applied, shared by all heads;
  * section "Calculating V3.2's KV cache": the FP8 item stores the latent as
    E4M3 values with float32 scales (one per token, or one per 128 dimensions)
    and the rotary key unquantised in BF16;
  * "What attention stores, and what DeepSeek changed", section "The rotary
    complication": RoPE rotates a key by an angle that depends on its
    position.

Readings (the pages leave these open):
  * the rotation acts on consecutive pairs (2i, 2i+1) of K^R with the angles
    the caller's cos / sin tables give for the position: (x, y) ->
    (x cos - y sin, x sin + y cos), the form of the original RoPE definition;
  * FP8 scale = max |c| / 448 over the token (or its 128-channel group), 1
    when that maximum is 0; code = the E4M3 value nearest c / scale, ties to
    the even code, quotients clamped to +-448.  Both the scale and the
    quotient are float32 operations, so the codes -- integer decisions -- are
    taken in the precision the kernel uses;
  * BF16 storage rounds to nearest, ties to even.
"""

from __future__ import annotations

import numpy as np

from .mla_oracle import e4m3_to_f64

__all__ = ["rope_rotate", "encode_e4m3_nearest", "quantize_token", "bf16_round", "append_token"]


def rope_rotate(x, cos_row, sin_row) -> np.ndarray:
    """Rotate consecutive pairs of x [D_R] by the angles whose cosines and
    sines are cos_row, sin_row [D_R / 2] (float64)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos_row, dtype=np.float64)
    s = np.asarray(sin_row, dtype=np.float64)
    out = np.empty_like(x)
    out[0::2] = x[0::2] * c - x[1::2] * s
    out[1::2] = x[0::2] * s + x[1::2] * c
    return out


# the 127 finite non-negative E4M3 values by code 0x00 .. 0x7E, from the
# format definition (bias 7, 3 mantissa bits, subnormals below 2^-6)
_POS = e4m3_to_f64(np.arange(127, dtype=np.uint8))


def encode_e4m3_nearest(v) -> np.ndarray:
    """E4M3 code of the nearest representable value (|v| <= 448), ties to the
    code with an even mantissa; the sign goes to bit 7 (+0 for zero)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > 448.0) or np.any(np.isnan(v)):
        raise ValueError("values must be finite and within +-448")
    d = np.abs(a[..., None] - _POS)                     # distance to every value
    best = d.min(axis=-1, keepdims=True)
    cand = d == best
    # two candidates only at a midpoint: take the even code
    even = cand & ((np.arange(127) % 2) == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1)).astype(np.uint8)
    neg = (v < 0) & (code != 0)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def quantize_token(c, groups: int = 1):
    """FP8 codes and float32 scales of one token's latent c [D_C] (float32
    values): one scale, or one per `groups` equal channel groups."""
    c = np.asarray(c, dtype=np.float32)
    D = c.shape[0]
    w = D // groups
    codes = np.empty(D, dtype=np.uint8)
    scales = np.empty(groups, dtype=np.float32)
    for g in range(groups):
        part = c[g * w:(g + 1) * w]
        amax = np.max(np.abs(part))
        scale = np.float32(amax) / np.float32(448.0) if amax > 0 else np.float32(1.0)
        q = np.clip(part / scale, np.float32(-448.0), np.float32(448.0))   # float32 quotient
        codes[g * w:(g + 1) * w] = encode_e4m3_nearest(q)
        scales[g] = scale
    return codes, scales


def bf16_round(x) -> np.ndarray:
    """Nearest BF16 value of float32 inputs, ties to even, as float32."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return r.astype(np.uint32).view(np.float32)


def append_token(c_new, k_new, cos_row, sin_row, cache: str):
    """What one appended token stores: (latent payload, rotary key, scales).
    cache is 'f32', 'bf16', 'fp8' (one scale) or 'fp8_g128' (one scale per
    128 channels).  The latent payload is float32 values (f32 / bf16) or E4M3
    codes (fp8); the rotary key is the rotated key rounded to the storage type
    (float32, else BF16); scales are None for unquantised caches."""
    k_rot = rope_rotate(k_new, cos_row, sin_row) if cos_row is not None else np.asarray(k_new, np.float64)
    if cache == "f32":
        return np.asarray(c_new, np.float32), k_rot.astype(np.float32), None
    k_bf = bf16_round(k_rot.astype(np.float32))
    if cache == "bf16":
        return bf16_round(np.asarray(c_new, np.float32)), k_bf, None
    groups = 1 if cache == "fp8" else np.asarray(c_new).shape[0] // 128
    codes, scales = quantize_token(c_new, groups)
    return codes, k_bf, scales
