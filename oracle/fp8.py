"""Plain fp64 NumPy oracle of the FP8 (e4m3) KV cache — TEST INFRASTRUCTURE ONLY.

See the package docstring for what may import this module.

The pages list FP8 among the quantisation schemes the engine supports (page
"vLLM推理引擎深度实战", introduction) and name quantised inference as a way to cut
memory use (page "vLLM推理引擎深度解析", closing list of optimisation strategies);
they give no format, scale or rounding. The readings taken here:

* the element format is the OCP 8-bit floating point format E4M3 ("e4m3fn"):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
  infinities, the two codes S.1111.111 are NaN, largest finite value 448;
* one float32 scale per kv head for K and one for V, a stored element standing
  for ``value(code) * scale``;
* writing a token quantises each element ``x`` as ``y = fl32(x / scale)`` (x
  widened exactly to float32, one correctly rounded float32 division), then
  rounds ``y`` to the nearest e4m3 value, ties to the even mantissa; finite
  values beyond +-448 (and infinities) saturate to +-448; NaN stays NaN with
  its sign bit (the sign a division leaves on a NaN is not fixed by IEEE 754,
  so only NaN inputs of positive sign have a defined code); the sign of zero is
  kept;
* attention reads the dequantised cache: ``K = value(code) * k_scale[h]``,
  ``V = value(code) * v_scale[h]``, and is otherwise the attention of
  ``paged_attention``.
"""
from __future__ import annotations

import math

import numpy as np

from .paged_attention import BLOCK_SIZE, attend, gather, kv_head_of, scatter, to_f64, visible_keys, _scale64

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6          # 2^-6, exponent field 1
_SUB_STEP = 2.0 ** -9         # spacing of subnormals: 2^-6 / 8


def e4m3_value(code: int) -> float:
    """Value of one e4m3 code from the format's fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * _SUB_STEP                       # m/8 * 2^(1-7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """float64 values of the 256 codes."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def _round_half_even(x: float) -> int:
    f = math.floor(x)
    r = x - f
    if r > 0.5:
        return f + 1
    if r < 0.5:
        return f
    return f if f % 2 == 0 else f + 1


def e4m3_code(y: float) -> int:
    """Nearest e4m3 code of one value (ties to even mantissa, saturating to +-448)."""
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    if math.isnan(y):
        return sign | 0x7F                                # NaN keeps its sign bit
    a = abs(y)
    if a >= E4M3_MAX:                                     # includes infinity
        return sign | 0x7E
    if a < 2.0 ** _MIN_NORMAL_EXP:                        # subnormal range (and zero)
        k = _round_half_even(a / _SUB_STEP)               # exact: power-of-two scaling
        return sign | k                                   # k == 8 is the smallest normal
    mant, exp = math.frexp(a)                             # a = mant * 2^exp, mant in [0.5, 1)
    e = exp - 1                                           # a = (2 * mant) * 2^e, e >= -6
    k = _round_half_even((2.0 * mant - 1.0) * 8.0)        # mantissa steps of 1/8
    if k == 8:                                            # rounded up to the next power of two
        k, e = 0, e + 1
    if e > 8 or (e == 8 and k == 7):                      # only reachable at a >= 448
        return sign | 0x7E
    return sign | ((e + 7) << 3) | k


def quantize(x_storage: np.ndarray, dtype: str, scale) -> np.ndarray:
    """Codes of ``fl32(x / scale)`` for storage values ``x`` of ``dtype`` ("f32", "f16",
    "bf16" as uint16 bits); ``scale`` broadcasts against the values (one per kv head:
    shape ``[H_kv, 1]`` for rows ``[H_kv, D]``)."""
    x32 = to_f64(x_storage, dtype).astype(np.float32)     # exact widening
    y = x32 / np.asarray(scale, dtype=np.float32)          # one float32 division
    flat = np.asarray(y, dtype=np.float32).ravel()
    return np.array([e4m3_code(float(v)) for v in flat], dtype=np.uint8).reshape(y.shape)


def scatter_fp8(k_pool: np.ndarray, v_pool: np.ndarray, key, value, slot_mapping, k_scale, v_scale,
                dtype: str, block_size: int = BLOCK_SIZE):
    """Quantise each new token's K and V rows ``[H_kv, D]`` with their heads' scales, then
    write the codes at the token's slot (the write of page "vLLM推理引擎深度解析" §三/§五)."""
    ks = np.asarray(k_scale, np.float32)[:, None]
    vs = np.asarray(v_scale, np.float32)[:, None]
    kq = np.stack([quantize(key[t], dtype, ks) for t in range(len(key))]) if len(key) else key
    vq = np.stack([quantize(value[t], dtype, vs) for t in range(len(value))]) if len(value) else value
    return scatter(k_pool, v_pool, kq, vq, slot_mapping, block_size)


def dequantize(codes: np.ndarray, scale) -> np.ndarray:
    """float64 ``value(code) * scale[h]`` for codes ``[..., H_kv, D]`` (a pool or gathered rows)."""
    tab = e4m3_table()
    s = np.asarray(scale, np.float32).astype(np.float64)
    return tab[np.asarray(codes, np.uint8)] * s[:, None]


def paged_decode_fp8(query, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale,
                     num_kv_heads, dtype, block_size: int = BLOCK_SIZE) -> np.ndarray:
    """Decode attention over the dequantised cache; ``query`` in ``dtype`` storage.
    Same walk and softmax as ``paged_attention.paged_decode``. Returns float64 ``[B, H_q, D]``."""
    B, Hq, D = query.shape
    sc = _scale64(scale)
    q64 = to_f64(query, dtype)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = dequantize(gather(k_pool, block_tables[b], L, block_size), k_scale)    # [L, H_kv, D]
        V = dequantize(gather(v_pool, block_tables[b], L, block_size), v_scale)
        for h in range(Hq):
            g = kv_head_of(h, Hq, num_kv_heads)
            out[b, h] = attend(q64[b, h], K[:, g], V[:, g], sc)
    return out


def paged_prefill_fp8(query, k_pool, v_pool, block_tables, seq_lens, cu_q_lens, scale, k_scale, v_scale,
                      num_kv_heads, dtype, causal: bool = True, block_size: int = BLOCK_SIZE,
                      seqs=None, heads=None) -> np.ndarray:
    """Chunked prefill over the dequantised cache: the queries of ``paged_attention.paged_prefill``
    (row ranges from ``cu_q_lens``, causal positions ``seq_lens[b] - q_len + i``) attend over
    ``K = value(code) * k_scale[h]`` and ``V = value(code) * v_scale[h]`` gathered through the
    table. ``query`` in ``dtype`` storage; returns float64 ``[T, H_q, D]``, rows outside
    ``seqs``/``heads`` zero."""
    T, Hq, D = query.shape
    sc = _scale64(scale)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    seqs = range(len(seq_lens)) if seqs is None else seqs
    heads = range(Hq) if heads is None else heads
    for b in seqs:
        q0, q1 = int(cu_q_lens[b]), int(cu_q_lens[b + 1])
        qlen, L = q1 - q0, int(seq_lens[b])
        if qlen == 0 or L == 0:
            continue
        K = dequantize(gather(k_pool, block_tables[b], L, block_size), k_scale)    # [L, H_kv, D]
        V = dequantize(gather(v_pool, block_tables[b], L, block_size), v_scale)
        Q = to_f64(query[q0:q1], dtype)
        visible = visible_keys(L, qlen, causal)
        for h in heads:
            g = kv_head_of(h, Hq, num_kv_heads)
            S = sc * (Q[:, h] @ K[:, g].T)
            S = np.where(visible, S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            out[q0:q1, h] = (P @ V[:, g]) / P.sum(axis=1, keepdims=True)
    return out
