"""fp8 (E4M3) KV cache for the oracle (test infrastructure only).

The pages name an fp8 or int8 KV cache as a quantization that stores keys and
values in low precision while the products run in bf16, halving the KV bytes
read per decode step ("LLM serving: KV cache, batching, paged attention and
quantization", learn.mohebi.ai, section 3.7, the table of schemes), and E4M3
(largest magnitude 448) as the fp8 format for inference, with per-tensor,
per-channel or per-block scales ("07 - Inference", lourdhu02.github.io,
section 4.3).

Format (the OCP 8-bit floating point E4M3 encoding): bit 7 sign, bits 6..3 a
biased exponent (bias 7), bits 2..0 the mantissa.  Exponent field 0 encodes
subnormals m/8 * 2^-6; exponent 1..15 encodes (1 + m/8) * 2^(e-7), except
that e = 15 with m = 7 is NaN (there are no infinities).  Largest finite
magnitude: 1.75 * 2^8 = 448.

Readings (the pages fix neither):
* one fp32 scale per KV head for K and one for V (the per-channel granularity
  the pages list, taken over the head); a stored code c of head g means the
  value decode(c) * scale[g];
* quantization: q = fp32(x) / fp32(scale) in IEEE fp32 (the precision the
  kernel decides in), clamped to [-448, 448], rounded to the nearest code with
  ties to the even mantissa; NaN is stored as 0x7F.
"""

from __future__ import annotations

import math

import numpy as np

from .attention import BLOCK_SIZE, attend_row, gather_sequence, kv_head_of, to_f64, visible_tokens

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3_decode(code: int) -> float:
    """The value of one E4M3 code (float64; NaN for the two NaN codes)."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """decode() of all 256 codes, float64."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code to x (ties to the even mantissa), saturating at +-448; NaN -> 0x7F.

    Written as the rounding of the exact binary value: the step between
    neighbouring codes at |x| is 2^(max(e, -6) - 3) where 2^e <= |x| < 2^(e+1).
    """
    if math.isnan(x):
        return E4M3_NAN
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    if a >= E4M3_MAX:
        return sign | 0x7E
    if a == 0.0:
        return sign
    e = max(math.frexp(a)[1] - 1, -6)  # exponent of the leading bit, at least the subnormal one
    step = 2.0 ** (e - 3)
    n = a / step  # exact: a power-of-two division of a double
    k = math.floor(n)
    frac = n - k
    if frac > 0.5 or (frac == 0.5 and k % 2 == 1):
        k += 1
    value = k * step
    if value > E4M3_MAX:  # cannot happen below 448, kept for clarity
        return sign | 0x7E
    # value = k * 2^(e-3): back to (exponent field, mantissa)
    if value < 2.0 ** -6:
        return sign | int(k)  # subnormal: m = value / 2^-9
    ee = math.frexp(value)[1] - 1
    m = int(round((value / 2.0 ** ee - 1.0) * 8))
    return sign | ((ee + 7) << 3) | m


def quantize(x32: np.ndarray, scale32: float) -> np.ndarray:
    """Codes of fp32 values x32 for a scale: the quotient in IEEE fp32, then e4m3_encode."""
    x32 = np.asarray(x32, dtype=np.float32)
    q = (x32 / np.float32(scale32)).astype(np.float32)  # one correctly rounded fp32 division each
    flat = [e4m3_encode(float(v)) for v in q.ravel()]
    return np.array(flat, dtype=np.uint8).reshape(x32.shape)


def cache_write_fp8(k_codes, v_codes, k, v, slot_mapping, k_scale, v_scale, dtype: str,
                    block_size: int = BLOCK_SIZE):
    """Copies of the fp8 caches [NB, 16, n_kv, d] (uint8 codes) with token t's K/V
    rows, quantized with the per-head scales, at flat slot slot_mapping[t]
    (negative: not stored).  k, v are [T, n_kv, d] in the input dtype."""
    NB = k_codes.shape[0]
    n_kv = k_codes.shape[2]
    kc = k_codes.copy()
    vc = v_codes.copy()
    kf = kc.reshape(NB * block_size, *kc.shape[2:])
    vf = vc.reshape(NB * block_size, *vc.shape[2:])
    k32 = to_f64(k, dtype).astype(np.float32)  # exact: bf16 and f32 inputs are fp32 values
    v32 = to_f64(v, dtype).astype(np.float32)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        if slot >= NB * block_size:
            raise IndexError(f"slot {slot} outside a pool of {NB} blocks")
        for g in range(n_kv):
            kf[slot, g] = quantize(k32[t, g], float(k_scale[g]))
            vf[slot, g] = quantize(v32[t, g], float(v_scale[g]))
    return kc, vc


def paged_decode_fp8_rows(q, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, scale, q_len,
                          q_dtype, rows, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Attention over an fp8 cache for the listed (b, j, h) rows, [len(rows), d] float64.

    Paging and the attention are those of attention.paged_decode_rows; the keys
    and values are the decoded codes times their head's scale, exactly in fp64.
    """
    n_h = q.shape[1]
    n_kv = k_codes.shape[2]
    G = n_h // n_kv
    table = e4m3_table()
    scale64 = float(np.float32(scale))
    out = np.empty((len(rows), q.shape[2]), dtype=np.float64)
    cache = {}
    for i, (b, j, h) in enumerate(rows):
        L = int(context_lens[b])
        g = kv_head_of(h, G)
        if (b, g) not in cache:
            Kc = gather_sequence(k_codes, block_tables[b], L, block_size)[:, g, :]
            Vc = gather_sequence(v_codes, block_tables[b], L, block_size)[:, g, :]
            cache[(b, g)] = (table[Kc] * float(k_scale[g]), table[Vc] * float(v_scale[g]))
        K, V = cache[(b, g)]
        n = visible_tokens(L, q_len, j)
        out[i] = attend_row(to_f64(q[b * q_len + j, h], q_dtype), K[:n], V[:n], scale64)
    return out


def paged_decode_fp8(q, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, scale, q_len, q_dtype,
                     block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Full output [num_seqs * q_len, num_q_heads, head_dim] in float64."""
    S = block_tables.shape[0]
    n_h, d = q.shape[1], q.shape[2]
    rows = [(b, j, h) for b in range(S) for j in range(q_len) for h in range(n_h)]
    flat = paged_decode_fp8_rows(q, k_codes, v_codes, k_scale, v_scale, block_tables, context_lens, scale, q_len,
                                 q_dtype, rows, block_size)
    return flat.reshape(S * q_len, n_h, d)
