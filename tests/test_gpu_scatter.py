"""GPU reshape_and_cache: bit-exact against the oracle's scatter over the whole pool."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_463_amd as P
import workloads as W
from gpu_cases import assert_scatter_exact, dev, host, i32, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny", "llama2_7b_fp16", "llama3_8b_gqa_bf16"])
def test_named_decode_configs(name):
    case = W.NAMED[name]()
    say(f"case: scatter {case.name}")
    kp, vp = dev(case.k_pool, case.dtype), dev(case.v_pool, case.dtype)
    P.reshape_and_cache(dev(case.k_new, case.dtype), dev(case.v_new, case.dtype), kp, vp,
                        i32(case.slot_mapping))
    torch.cuda.synchronize()
    assert_scatter_exact(case, kp, vp)


def test_prefill_chunk_scatter():
    case = W.chunked_prefill_bf16()
    say(f"case: scatter {case.name} ({len(case.slot_mapping)} tokens)")
    kp, vp = dev(case.k_pool, "bf16"), dev(case.v_pool, "bf16")
    P.reshape_and_cache(dev(case.k_new, "bf16"), dev(case.v_new, "bf16"), kp, vp, i32(case.slot_mapping))
    torch.cuda.synchronize()
    assert_scatter_exact(case, kp, vp)


@pytest.mark.parametrize("dtype", W.DTYPES)
@pytest.mark.parametrize("D", [64, 128])
def test_padding_and_out_of_range_slots_are_skipped(dtype, D):
    rng = np.random.default_rng(D)
    nb, H = 12, 3
    kp_h = W.normal(rng, (nb, 16, H, D), dtype)
    vp_h = W.normal(rng, (nb, 16, H, D), dtype)
    T = 40
    slots = rng.choice(nb * 16, size=T, replace=False).astype(np.int32)
    slots[::7] = -1
    slots[5] = nb * 16 + 3             # out of range: skipped, never written
    key, val = W.normal(rng, (T, H, D), dtype), W.normal(rng, (T, H, D), dtype)
    kp, vp = dev(kp_h, dtype), dev(vp_h, dtype)
    P.reshape_and_cache(dev(key, dtype), dev(val, dtype), kp, vp, i32(slots))
    torch.cuda.synchronize()
    ok = slots.copy()
    ok[5] = -1
    rk, rv = oracle.scatter(kp_h, vp_h, key, val, ok)
    assert host(kp, dtype).tobytes() == rk.tobytes()
    assert host(vp, dtype).tobytes() == rv.tobytes()


def test_strided_key_rows():
    """K/V rows taken out of a fused [T, H_q + 2 H_kv, D] projection (row stride > H_kv*D)."""
    rng = np.random.default_rng(9)
    T, Hq, Hkv, D, nb = 20, 8, 2, 128, 6
    fused = W.normal(rng, (T, Hq + 2 * Hkv, D), "bf16")
    f = dev(fused, "bf16")
    key, val = f[:, Hq:Hq + Hkv], f[:, Hq + Hkv:]
    kp_h = np.full((nb, 16, Hkv, D), 0x7FC0, dtype=np.uint16)
    vp_h = kp_h.copy()
    kp, vp = dev(kp_h, "bf16"), dev(vp_h, "bf16")
    slots = np.arange(T, dtype=np.int32) * 3 % (nb * 16)
    P.reshape_and_cache(key, val, kp, vp, i32(slots))
    torch.cuda.synchronize()
    rk, rv = oracle.scatter(kp_h, vp_h, fused[:, Hq:Hq + Hkv], fused[:, Hq + Hkv:], slots)
    assert host(kp, "bf16").tobytes() == rk.tobytes()
    assert host(vp, "bf16").tobytes() == rv.tobytes()
