"""Pins of the FP8 (e4m3) KV-cache oracle (CPU only).

The format is pinned against values fixed by its definition (the OCP 8-bit
floating point format, E4M3: bias 7, 3 mantissa bits, subnormals, NaN at
S.1111.111, largest finite 448) and against torch's own float8_e4m3fn
conversion (a library routine, round to nearest even) wherever the two readings
agree (|y| <= 464; torch turns larger values into NaN where the oracle
saturates). The attention over a dequantised cache is pinned against the
16-bit oracle on caches whose values e4m3 holds exactly, and mutation tests plant
mistakes in the oracle to show that the pins catch them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F


def torch_codes(y32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(y32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_table_special_values():
    t = F.e4m3_table()
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3F: 1.875,
             0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0x81: -(2.0 ** -9), 0xB8: -1.0, 0xFE: -448.0}
    for c, v in fixed.items():
        assert t[c] == v, hex(c)
    assert math.copysign(1.0, t[0x80]) < 0 and t[0x80] == 0.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # codes 0..126 increase strictly


def test_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = F.e4m3_table()
    assert np.array_equal(np.isnan(codes), np.isnan(t))
    ok = ~np.isnan(t)
    assert np.array_equal(codes[ok], t[ok])
    assert np.array_equal(np.signbit(codes[ok]), np.signbit(t[ok]))


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    t = F.e4m3_table()
    fin = t[~np.isnan(t)]
    mids = ((np.sort(fin)[1:] + np.sort(fin)[:-1]) / 2).astype(np.float32)      # every tie
    near = np.concatenate([np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf))])
    wide = (rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 9, 4000))).astype(np.float32)
    y = np.concatenate([mids, near, wide, fin.astype(np.float32), np.float32([0.0, -0.0, 464.0, -464.0])])
    y = y[np.abs(y) <= 464.0]
    ours = np.array([F.e4m3_code(float(v)) for v in y], np.uint8)
    assert np.array_equal(ours, torch_codes(y))


def test_encode_saturates_and_keeps_nan_and_signed_zero():
    assert F.e4m3_code(448.0) == 0x7E
    for v in (448.5, 464.0, 465.0, 1e6, 3.4e38, math.inf):
        assert F.e4m3_code(v) == 0x7E and F.e4m3_code(-v) == 0xFE
    assert F.e4m3_code(math.nan) & 0x7F == 0x7F
    assert F.e4m3_code(0.0) == 0x00 and F.e4m3_code(-0.0) == 0x80
    assert F.e4m3_code(2.0 ** -10) == 0x00                  # tie between 0 and 2^-9: even
    assert F.e4m3_code(1.5 * 2.0 ** -9) == 0x02             # tie between 1 and 2 steps: even
    assert F.e4m3_code(2.5 * 2.0 ** -9) == 0x02
    assert F.e4m3_code(7.5 * 2.0 ** -9) == 0x08             # rounds up into the first normal
    assert F.e4m3_code(1.0625) == 0x38                      # tie 1 | 1.125: even mantissa 0
    assert F.e4m3_code(1.1875) == 0x3A                      # tie 1.125 | 1.25: even mantissa 2
    assert F.e4m3_code(15.5) == 0x58                        # tie 15 | 16 (0x57 | 0x58): carries into exponent


def test_encode_round_trip_and_error_bound():
    t = F.e4m3_table()
    for c in range(256):
        if not np.isnan(t[c]):
            assert F.e4m3_code(t[c]) == c
    rng = np.random.default_rng(9)
    y = (rng.uniform(-1, 1, 3000) * np.exp2(rng.uniform(-10, 8.8, 3000))).astype(np.float64)
    for v in y:
        q = t[F.e4m3_code(v)]
        e = max(math.frexp(abs(v))[1] - 1, -6)
        assert abs(q - v) <= 2.0 ** (e - 3) / 2 * (1 + 1e-12), v     # half a step of v's binade


def test_quantize_divides_in_float32_per_head():
    x = np.array([[1.0, 3.0], [3.0, -7.0]], np.float32)
    scale = np.array([[0.5], [3.0]], np.float32)            # one scale per row (kv head)
    codes = F.quantize(x, "f32", scale)
    want = [[F.e4m3_code(2.0), F.e4m3_code(6.0)], [F.e4m3_code(1.0), F.e4m3_code(float(np.float32(-7.0) / np.float32(3.0)))]]
    assert codes.tolist() == want
    # bf16 storage bits: 0x3F80 is 1.0
    assert F.quantize(np.array([0x3F80, 0xC0A0], np.uint16), "bf16", np.float32(1.0)).tolist() == [0x38, 0xCA]


def exact_case(rng, B=3, Hq=8, Hkv=2, D=64, nb=20):
    """Pools whose e4m3 values times power-of-two scales are exact in fp64 and f32."""
    t = F.e4m3_table()
    finite = np.array([c for c in range(256) if not np.isnan(t[c]) and abs(t[c]) <= 8], np.uint8)
    kc = rng.choice(finite, size=(nb, 16, Hkv, D))
    vc = rng.choice(finite, size=(nb, 16, Hkv, D))
    ks = np.array([0.25, 2.0], np.float32)[:Hkv]
    vs = np.array([0.5, 4.0], np.float32)[:Hkv]
    lens = np.array([1, 37, 80][:B], np.int32)
    tables = np.stack([rng.permutation(nb)[:5] for _ in range(B)]).astype(np.int32)
    q = rng.standard_normal((B, Hq, D)).astype(np.float32)
    return q, kc, vc, ks, vs, tables, lens


def test_fp8_decode_equals_decode_of_the_dequantised_cache():
    rng = np.random.default_rng(3)
    q, kc, vc, ks, vs, tables, lens = exact_case(rng)
    kf = (t := F.e4m3_table())[kc] * ks[None, None, :, None]
    vf = t[vc] * vs[None, None, :, None]
    ref = oracle.paged_decode(q, kf.astype(np.float32), vf.astype(np.float32), tables, lens, 0.125, 2, "f32")
    got = F.paged_decode_fp8(q, kc, vc, tables, lens, 0.125, ks, vs, 2, "f32")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_one_token_context_returns_the_dequantised_value_row():
    rng = np.random.default_rng(4)
    q, kc, vc, ks, vs, tables, lens = exact_case(rng)
    lens = np.array([1, 1, 1], np.int32)
    got = F.paged_decode_fp8(q, kc, vc, tables, lens, 0.125, ks, vs, 2, "f32")
    t = F.e4m3_table()
    for b in range(3):
        for h in range(8):
            g = h // 4
            assert np.array_equal(got[b, h], t[vc[tables[b, 0], 0, g]] * vs[g])


def _prefill_exact_case(rng):
    """Two sequences over FP8 pools whose dequantised values are exact in f32: 30 cached + 9
    new tokens and 0 cached + 21 new tokens, 8 query heads over 2 kv heads, head_dim 8."""
    q, kc, vc, ks, vs, tables, _ = exact_case(rng)
    seq_lens = np.array([39, 21], np.int32)
    cu = np.array([0, 9, 30], np.int32)
    query = rng.standard_normal((30, 8, kc.shape[-1])).astype(np.float32)
    return query, kc, vc, ks, vs, tables[:2], seq_lens, cu


def test_fp8_prefill_equals_prefill_of_the_dequantised_cache():
    rng = np.random.default_rng(11)
    query, kc, vc, ks, vs, tables, seq_lens, cu = _prefill_exact_case(rng)
    t = F.e4m3_table()
    kf = (t[kc] * ks[None, None, :, None]).astype(np.float32)
    vf = (t[vc] * vs[None, None, :, None]).astype(np.float32)
    for causal in (True, False):
        ref = oracle.paged_prefill(query, kf, vf, tables, seq_lens, cu, 0.3, 2, "f32", causal=causal)
        got = F.paged_prefill_fp8(query, kc, vc, tables, seq_lens, cu, 0.3, ks, vs, 2, "f32", causal=causal)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_fp8_prefill_last_chunk_row_equals_fp8_decode():
    """The last query of a chunk sits at position seq_len - 1 and sees every key: the decode
    of the same sequence over the same FP8 cache."""
    rng = np.random.default_rng(12)
    query, kc, vc, ks, vs, tables, seq_lens, cu = _prefill_exact_case(rng)
    got = F.paged_prefill_fp8(query, kc, vc, tables, seq_lens, cu, 0.3, ks, vs, 2, "f32")
    last = query[cu[1:] - 1]
    dec = F.paged_decode_fp8(last, kc, vc, tables, seq_lens, 0.3, ks, vs, 2, "f32")
    np.testing.assert_allclose(got[cu[1:] - 1], dec, rtol=0, atol=1e-13)


def test_scatter_fp8_writes_codes_at_slots():
    key = np.array([[[1.0, -2.0]], [[448.0, 1000.0]]], np.float32)       # [T=2, H_kv=1, D=2]
    value = -key
    kp = np.zeros((2, 16, 1, 2), np.uint8)
    k2, v2 = F.scatter_fp8(kp, kp.copy(), key, value, np.array([17, -1]), [2.0], [1.0], "f32")
    assert k2[1, 1, 0].tolist() == [F.e4m3_code(0.5), F.e4m3_code(-1.0)]
    assert v2[1, 1, 0].tolist() == [F.e4m3_code(-1.0), F.e4m3_code(2.0)]
    assert int(np.count_nonzero(k2)) == 2                                 # slot -1 skipped


# -- mutation tests: plant a mistake in the oracle, some pin must catch it --

def test_mutation_round_half_up_is_caught(monkeypatch):
    monkeypatch.setattr(F, "_round_half_even", lambda x: math.floor(x + 0.5))
    with pytest.raises(AssertionError):
        test_encode_matches_torch_in_range()


def test_mutation_wrong_bias_is_caught(monkeypatch):
    def value(code):
        code = int(code) & 0xFF
        e, m = (code >> 3) & 0xF, code & 7
        if e == 0xF and m == 7:
            return math.nan
        s = -1.0 if code & 0x80 else 1.0
        return s * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 8))
    monkeypatch.setattr(F, "e4m3_value", value)
    with pytest.raises(AssertionError):
        test_table_matches_torch()


def test_mutation_scales_of_swapped_heads_are_caught(monkeypatch):
    orig = F.dequantize
    monkeypatch.setattr(F, "dequantize", lambda pool, scale: orig(pool, np.asarray(scale)[::-1]))
    with pytest.raises(AssertionError):
        test_fp8_decode_equals_decode_of_the_dequantised_cache()


def test_mutation_no_saturation_is_caught(monkeypatch):
    orig = F.e4m3_code
    monkeypatch.setattr(F, "e4m3_code", lambda y: 0x7F if abs(y) > 464 and not math.isnan(y) else orig(y))
    with pytest.raises(AssertionError):
        test_encode_saturates_and_keeps_nan_and_signed_zero()


def test_mutation_prefill_scales_of_swapped_heads_are_caught(monkeypatch):
    orig = F.dequantize
    monkeypatch.setattr(F, "dequantize", lambda pool, scale: orig(pool, np.asarray(scale)[::-1]))
    with pytest.raises(AssertionError):
        test_fp8_prefill_equals_prefill_of_the_dequantised_cache()


def test_mutation_prefill_k_and_v_scales_exchanged_are_caught(monkeypatch):
    orig = F.paged_prefill_fp8

    def swapped(query, kp, vp, bt, sl, cu, scale, ks, vs, *a, **kw):
        return orig(query, kp, vp, bt, sl, cu, scale, vs, ks, *a, **kw)
    monkeypatch.setattr(F, "paged_prefill_fp8", swapped)
    with pytest.raises(AssertionError):
        test_fp8_prefill_equals_prefill_of_the_dequantised_cache()
