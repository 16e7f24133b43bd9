"""Host logic of bench.py (no GPU): the algorithmic work the roofline divides by, the one-GPU
guard, and the rule that stored HBM traffic is reported only for the kernel sources it was
measured on. Expected values are worked out by hand from the workload definitions."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_tiny_decode_bytes_by_hand():
    """Lengths 5, 16, 17, 40, 4 heads, head_dim 64, fp32: K and V rows of the 78 cached
    tokens, query and output rows, the 1 + 1 + 2 + 3 table entries read and the 4 lengths."""
    case = W.tiny_fp32(keep_dense=False)
    kv = 78 * 2 * 4 * 64 * 4
    qo = 2 * 4 * 4 * 64 * 4
    tables = 4 * (1 + 1 + 2 + 3) + 4 * 4
    assert bench.kv_bytes(case, unique=False) == kv == 159744
    assert bench.decode_bytes(case, unique=False) == kv + qo + tables == 167980
    # the FP8 cache holds one byte per element; queries and outputs keep their type
    assert bench.kv_bytes(case, unique=False, call="decode_fp8") == kv // 4
    # scatter: read the new rows and write them into the pool (K and V), plus the slots
    assert bench.scatter_bytes(case) == 2 * 4 * (4 * 64) * (4 + 4) + 4 * 4


def test_shared_prefix_counted_once_in_unique_bytes():
    """The GQA batch: 128 sequences share 32 blocks of 16 tokens; unique bytes count those
    512 tokens once instead of 128 times."""
    case = W.llama3_8b_gqa_bf16()
    row = 2 * 8 * 128 * 2
    logical = bench.kv_bytes(case, unique=False)
    unique = bench.kv_bytes(case, unique=True)
    assert logical == int(case.context_lens.sum()) * row
    assert logical - unique == 127 * 512 * row
    assert bench.decode_bytes(case, unique=False) - bench.decode_bytes(case, unique=True) == 127 * 512 * row


def test_chunked_prefill_flops_closed_form():
    """16 sequences of 2048 cached + 512 new tokens, 32 query heads, head_dim 128: query i of
    the chunk sees 2048 + i + 1 keys, so the causal pairs per sequence and head are
    sum_{k=2049}^{2560} k = (2049 + 2560) * 512 / 2."""
    case = W.chunked_prefill_bf16()
    pairs = (2049 + 2560) * 512 // 2
    assert bench.prefill_flops(case) == 4 * 128 * 32 * 16 * pairs == 309_304_754_176   # 3.093e11


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stored_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    """A traffic record is reported only while the kernel sources hash as when it was taken
    (and, for split-KV, at the partition size it was taken with)."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    rec = {"kernel_source_sha256": bench.kernel_source_sha256("decode"), "hbm_bytes_per_launch": 1234,
           "partition_size": None}
    (tmp_path / "decode_w.traffic.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("w", "decode", 512) == 1234
    rec["kernel_source_sha256"] = "0" * 64
    (tmp_path / "decode_w.traffic.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("w", "decode", 512) is None
    rec = {"kernel_source_sha256": bench.kernel_source_sha256("splitkv"), "hbm_bytes_per_launch": 99,
           "partition_size": 512}
    (tmp_path / "splitkv_w.traffic.json").write_text(json.dumps(rec))
    assert bench.stored_traffic("w", "splitkv", 512) == 99
    assert bench.stored_traffic("w", "splitkv", 256) is None
    assert bench.stored_traffic("absent", "decode", 512) is None


@pytest.mark.parametrize("workload", sorted(bench.WORKLOADS))
def test_committed_traffic_records_are_consistent(workload):
    """Every committed record names its workload and call, and its bytes are the counter
    readings times their calibration scales, summed over the call's kernels."""
    call = bench.WORKLOADS[workload][1]
    path = os.path.join(ROOT, "profiles", f"{call}_{workload}.traffic.json")
    if not os.path.exists(path):
        pytest.skip("no traffic record for this workload")
    rec = json.load(open(path))
    assert rec["workload"] == workload and rec["call"] == call
    total = sum(v * rec["fetch_scale"] * 1024 for v in rec["fetch_kib_per_dispatch"].values()) + \
        sum(v * rec["write_scale"] * 1024 for v in rec["write_kib_per_dispatch"].values())
    assert abs(total - rec["hbm_bytes_per_launch"]) <= 1e-6 * total + 2
    assert 1.9 < rec["fetch_scale"] < 2.1 and 0.95 < rec["write_scale"] < 1.05


@pytest.mark.parametrize("maker,call", [(lambda: W.make_decode("cb", "bf16", [5, 40, 300], 8, 2, 64, seed=3),
                                         "splitkv"),
                                        (lambda: W.make_prefill("cbp", "bf16", [20, 0], [9, 33], 8, 2, 64, seed=4),
                                         "prefill")])
def test_cpu_baseline_units_reassemble_the_oracle(maker, call):
    """The CPU baseline splits a step into (sequence, kv head) units, each the oracle on one kv
    head's slice of the pools; in two worker processes the units must cover the batch and
    reassemble the oracle's whole-batch output exactly, and the record must state the worker
    count that ran them."""
    import numpy as np
    import oracle
    case = maker()
    ctx = bench._unit_ctx(case, call)
    rec, units = bench.cpu_baseline(ctx, 0.5, 2)
    assert rec["cores"] == 2 and rec["kind"] == "oracle" and rec["value"] > 0
    assert set(units) == {(b, g) for b in range(case.num_seqs) for g in range(case.num_kv_heads)}
    if call == "prefill":
        full = oracle.paged_prefill(case.query, ctx["kp"], ctx["vp"], case.block_tables, case.seq_lens,
                                    case.cu_q_lens, case.scale, case.num_kv_heads, case.dtype)
    else:
        full = oracle.paged_decode(case.query, ctx["kp"], ctx["vp"], case.block_tables, case.context_lens,
                                   case.scale, case.num_kv_heads, case.dtype)
    assert bench.oracle_error(case, call == "prefill", units, full) == 0.0
    one, _ = bench.cpu_baseline(ctx, 0.2, 1)
    assert one["cores"] == 1


def test_default_run_has_the_headline_first():
    assert bench.DEFAULT_SET[0] == bench.HEADLINE == "long_ctx_bf16_splitkv_b8"
    assert set(bench.DEFAULT_SET[1:]) == {"tiny_fp32_decode_b4", "llama2_7b_fp16_decode_b64",
                                          "llama3_8b_gqa_bf16_decode_b256", "chunked_prefill_bf16_16x2048p512"}
