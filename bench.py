"""Throughput of the paged-attention hot path on one MI355X.

One step = one attention layer of one decode step (or one prefill chunk) over
the whole batch: ``pa_reshape_and_cache`` of the new tokens, then the attention
call, both on torch's current stream. The KV pool is replicated over
``--layers`` independent copies and steps rotate through them, the way a model
walks its layers, so repeated steps are not served from the 256 MB
last-level cache. Inputs are seeded synthetic tensors resident in HBM before
the timed region starts.

Prints ONE JSON line: value = sequence-steps per second (decode) or query
tokens per second (prefill) for the whole job, plus the roofline of the
dominant kernel (algorithmic bytes or flops per launch divided by its average
duration, measured with HIP events on the launch stream inside the timed
region) and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attn: KV GB/s, % of MI355X HBM peak, seq-steps/s"
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_463_amd", "csrc")
# sources that define each attention launch (a change to any of them makes a
# stored HBM-traffic measurement stale)
KERNEL_SOURCES = {
    "decode": ["decode.hip", "pa_device.h", "pa_launch.h"],
    "splitkv": ["decode.hip", "pa_device.h", "pa_launch.h"],
    "decode_fp8": ["decode.hip", "pa_device.h", "pa_launch.h"],
    "splitkv_fp8": ["decode.hip", "pa_device.h", "pa_launch.h"],
    "prefill": ["prefill.hip", "pa_device.h", "pa_launch.h"],
    "prefill_fp8": ["prefill.hip", "pa_device.h", "pa_launch.h"],
    "copy_blocks": ["block_copy.hip", "pa_device.h", "pa_launch.h"],
}
HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6    # dense, 256 CUs at 2.4 GHz
TORCH_DT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}

WORKLOADS = {
    # name -> (generator key in workloads.NAMED, attention call)
    "llama2_7b_fp16_decode_b64": ("llama2_7b_fp16", "decode"),
    "llama3_8b_gqa_bf16_decode_b256": ("llama3_8b_gqa_bf16", "decode"),
    "long_ctx_bf16_splitkv_b8": ("long_context_bf16", "splitkv"),
    "tiny_fp32_decode_b4": ("tiny", "decode"),
    "chunked_prefill_bf16_16x2048p512": ("chunked_prefill_bf16", "prefill"),
    # the same decode workloads over an FP8 (e4m3) KV cache
    "llama2_7b_fp8kv_decode_b64": ("llama2_7b_fp16", "decode_fp8"),
    "llama3_8b_gqa_fp8kv_decode_b256": ("llama3_8b_gqa_bf16", "decode_fp8"),
    "long_ctx_fp8kv_splitkv_b8": ("long_context_bf16", "splitkv_fp8"),
    "chunked_prefill_fp8kv_16x2048p512": ("chunked_prefill_bf16", "prefill_fp8"),
}
DEFAULT_WORKLOAD = "llama2_7b_fp16_decode_b64"
# block movement: name -> (pool blocks, kv heads, head_dim, copy pairs, swap blocks)
BLOCK_WORKLOADS = {
    "cow_copy_bf16_2048x32k": (8192, 8, 128, 2048, 512),
}
COPY_METRIC = "copy-on-write block copy: GB/s, % of MI355X HBM peak, blocks/s"


# ----------------------------------------------------------------------------
# algorithmic work (what the operation must touch, independent of the kernel)
# ----------------------------------------------------------------------------
def kv_elem_bytes(case, call: str) -> int:
    import workloads as W
    return 1 if call.endswith("_fp8") else W.ELEM_BYTES[case.dtype]


def decode_bytes(case, unique: bool, call: str = "decode") -> int:
    """KV rows of every cached token (shared prefix blocks once if ``unique``),
    plus query, output, the table entries read and the lengths."""
    import workloads as W
    e = W.ELEM_BYTES[case.dtype]
    row = 2 * case.num_kv_heads * case.head_dim * kv_elem_bytes(case, call)   # K and V of one token
    tokens = int(case.context_lens.astype(np.int64).sum())
    if unique and case.shared_blocks:
        tokens -= (len(case.sharers) - 1) * len(case.shared_blocks) * W.BLOCK_SIZE
    qo = 2 * case.num_seqs * case.num_q_heads * case.head_dim * e
    tables = 4 * sum(W.ceil_div(int(L), W.BLOCK_SIZE) for L in case.context_lens) + 4 * case.num_seqs
    return tokens * row + qo + tables


def kv_bytes(case, unique: bool, call: str = "decode") -> int:
    import workloads as W
    e = kv_elem_bytes(case, call)
    tokens = int(case.context_lens.astype(np.int64).sum())
    if unique and getattr(case, "shared_blocks", None):
        tokens -= (len(case.sharers) - 1) * len(case.shared_blocks) * W.BLOCK_SIZE
    return tokens * 2 * case.num_kv_heads * case.head_dim * e


def scatter_bytes(case, call: str = "decode") -> int:
    import workloads as W
    e = W.ELEM_BYTES[case.dtype]
    n = len(case.slot_mapping)
    row = case.num_kv_heads * case.head_dim
    return 2 * n * row * (e + kv_elem_bytes(case, call)) + 4 * n         # read + write, K and V


def prefill_flops(case) -> int:
    """4*D per (query head, visible key) pair: QK^T and PV, causal."""
    pairs = 0
    for b in range(case.num_seqs):
        ql, L = int(case.q_lens[b]), int(case.seq_lens[b])
        pos = L - ql + np.arange(ql)
        pairs += int((pos + 1).sum())
    return 4 * case.head_dim * case.num_q_heads * pairs


def kernel_source_sha256(call: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[call] + ["../build.py"]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload: str, call: str, partition: int):
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when there is none or the
    kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{call}_{workload}.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_sha256") != kernel_source_sha256(call):
        return None
    if call.startswith("splitkv") and rec.get("partition_size") != partition:
        return None
    return int(rec["hbm_bytes_per_launch"])


# ----------------------------------------------------------------------------
# device state and one step
# ----------------------------------------------------------------------------
class Runner:
    def __init__(self, case, call: str, layers: int, partition: int, step_mode: str = "separate"):
        import torch
        import paged_kv_cache_463_amd as P
        import workloads as W
        self.P, self.torch, self.case, self.call = P, torch, case, call
        self.partition = partition
        dt = getattr(torch, TORCH_DT[case.dtype])

        def dev(a):
            if case.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()

        def i32(a):
            return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()

        self.fp8 = call.endswith("_fp8")
        if self.fp8:                                # e4m3 codes and per-head scales
            f = W.fp8_pools(case, 0)
            k0, v0 = torch.from_numpy(f.k_pool).cuda(), torch.from_numpy(f.v_pool).cuda()
            self.ks, self.vs = torch.from_numpy(f.k_scale).cuda(), torch.from_numpy(f.v_scale).cuda()
            self.fp8_host = f
        else:
            k0, v0 = dev(case.k_pool), dev(case.v_pool)
        self.kp = [k0] + [k0.clone() for _ in range(layers - 1)]
        self.vp = [v0] + [v0.clone() for _ in range(layers - 1)]
        self.q = dev(case.query)
        self.kn, self.vn = dev(case.k_new), dev(case.v_new)
        self.slots = i32(case.slot_mapping)
        self.bt = i32(case.block_tables)
        self.out = torch.empty_like(self.q)
        self.layers = layers
        if call.startswith("prefill"):
            self.cu = i32(case.cu_q_lens)
            self.lens = i32(case.seq_lens)
            self.max_q = case.max_q_len
        else:
            self.lens = i32(case.context_lens)
            self.mcl = max(case.max_context_len, 1)
            need = P.splitkv_workspace_bytes(case.num_seqs, case.num_q_heads, case.head_dim, self.mcl, partition)
            self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        assert self.q.dtype == dt
        self.step_mode = step_mode
        self.graph = None
        if step_mode == "graph":                   # one recording of the fused step of every layer
            self.graph = P.StepGraph()
            with self.graph:
                for layer in range(layers):
                    self.fused(layer, stream=self.graph.stream)

    def fused(self, layer: int, stream=None):
        c, P = self.case, self.P
        if self.fp8:
            P.decode_step_fp8(self.out, self.q, self.kn, self.vn, self.kp[layer], self.vp[layer], self.bt,
                              self.lens, c.scale, self.ks, self.vs, stream=stream)
        else:
            P.decode_step(self.out, self.q, self.kn, self.vn, self.kp[layer], self.vp[layer], self.bt, self.lens,
                          c.scale, stream=stream)

    def step(self, layer: int, ev=None):
        """One step (graph mode: one replay = the steps of all layers); ``ev`` = (start, end)
        events recorded around the attention launch (the replay)."""
        stream = self.torch.cuda.current_stream()
        if self.step_mode == "separate":
            self.scatter(layer)
        if ev:
            ev[0].record(stream)
        if self.step_mode == "separate":
            self.attend(layer)
        elif self.step_mode == "fused":
            self.fused(layer)
        else:
            self.graph.replay()
        if ev:
            ev[1].record(stream)

    def scatter(self, layer: int):
        if self.fp8:
            self.P.reshape_and_cache_fp8(self.kn, self.vn, self.kp[layer], self.vp[layer], self.slots,
                                         self.ks, self.vs)
        else:
            self.P.reshape_and_cache(self.kn, self.vn, self.kp[layer], self.vp[layer], self.slots)

    def attend(self, layer: int):
        c, P = self.case, self.P
        if self.call == "decode":
            P.decode(self.out, self.q, self.kp[layer], self.vp[layer], self.bt, self.lens, c.scale)
        elif self.call == "splitkv":
            P.decode_splitkv(self.out, self.q, self.kp[layer], self.vp[layer], self.bt, self.lens, c.scale,
                             self.mcl, self.partition, self.ws)
        elif self.call == "decode_fp8":
            P.decode_fp8(self.out, self.q, self.kp[layer], self.vp[layer], self.bt, self.lens, c.scale,
                         self.ks, self.vs)
        elif self.call == "splitkv_fp8":
            P.decode_splitkv_fp8(self.out, self.q, self.kp[layer], self.vp[layer], self.bt, self.lens, c.scale,
                                 self.ks, self.vs, self.mcl, self.partition, self.ws)
        elif self.call == "prefill_fp8":
            P.prefill_chunked_fp8(self.out, self.q, self.cu, self.max_q, self.kp[layer], self.vp[layer], self.bt,
                                  self.lens, c.scale, self.ks, self.vs, True)
        else:
            P.prefill_chunked(self.out, self.q, self.cu, self.max_q, self.kp[layer], self.vp[layer], self.bt,
                              self.lens, c.scale, True)


class TimingEvent:
    """A HIP timing event on the launch stream, created with hipEventDisableSystemFence.
    Recording a default event performs a system-scope release and acquire, i.e. a cache
    write-back and invalidate, which then falls inside the interval being timed and slows the
    steps around it. The HIP runtime documents this flag for timing accuracy. Used only around
    work that stays on the device; results are read after a full device synchronisation."""
    _hip = None
    FLAGS = 0x20000000                     # hipEventDisableSystemFence

    @classmethod
    def _runtime(cls):
        if cls._hip is None:               # the runtime torch already loaded (one per process)
            import ctypes
            import re
            with open("/proc/self/maps") as fh:
                paths = re.findall(r"(/\S*/libamdhip64\.so[.\d]*)", fh.read())
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded")
            cls._hip = ctypes.CDLL(paths[0])
        return cls._hip

    def __init__(self):
        import ctypes
        self._c = ctypes
        self.e = ctypes.c_void_p()
        if self._runtime().hipEventCreateWithFlags(ctypes.byref(self.e), ctypes.c_uint(self.FLAGS)) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream) -> None:
        if self._hip.hipEventRecord(self.e, self._c.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end: "TimingEvent") -> float:
        """Milliseconds from this event to ``end``."""
        ms = self._c.c_float()
        if self._hip.hipEventSynchronize(end.e) != 0 or \
                self._hip.hipEventElapsedTime(self._c.byref(ms), self.e, end.e) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.e:
            self._hip.hipEventDestroy(self.e)


def time_steps(r: Runner, steps: int, warmup: int):
    """Warm up, then time exactly ``steps`` steps; HIP events bracket every attention
    call on the launch stream."""
    torch = r.torch
    per = r.layers if r.step_mode == "graph" else 1      # steps covered by one call of r.step
    for i in range(0, warmup, per):
        r.step(i % r.layers)
    torch.cuda.synchronize()
    n = steps // per
    ev = [(TimingEvent(), TimingEvent()) for _ in range(n)]
    t0 = time.perf_counter()
    for i in range(n):
        r.step((i * per) % r.layers, ev[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    attn_ms = [a.elapsed_time(b) / per for a, b in ev]
    return elapsed, attn_ms


# ----------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a bounded sample
# ----------------------------------------------------------------------------
def cpu_baseline(case, call: str, r: Runner, budget_s: float):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    if r.fp8:
        f = r.fp8_host
        kp, vp = oracle.fp8.scatter_fp8(f.k_pool, f.v_pool, case.k_new, case.v_new, case.slot_mapping,
                                        f.k_scale, f.v_scale, case.dtype)
    else:
        kp, vp = oracle.scatter(case.k_pool, case.v_pool, case.k_new, case.v_new, case.slot_mapping)
    gpu_out = r.out.float().cpu().double().numpy()
    order = np.random.default_rng(0).permutation(case.num_seqs)
    t0 = time.perf_counter()
    done, units, err, passes = [], 0, 0.0, 0
    while True:                                 # whole passes over the batch until the budget is spent
        for b in order:
            b = int(b)
            if call.startswith("prefill"):
                heads = list(range(case.num_q_heads))
                if r.fp8:
                    ref = oracle.fp8.paged_prefill_fp8(case.query, kp, vp, case.block_tables, case.seq_lens,
                                                       case.cu_q_lens, case.scale, f.k_scale, f.v_scale,
                                                       case.num_kv_heads, case.dtype, seqs=[b], heads=heads)
                else:
                    ref = oracle.paged_prefill(case.query, kp, vp, case.block_tables, case.seq_lens,
                                               case.cu_q_lens, case.scale, case.num_kv_heads, case.dtype,
                                               seqs=[b], heads=heads)
                q0, q1 = int(case.cu_q_lens[b]), int(case.cu_q_lens[b + 1])
                err = max(err, float(np.abs(ref[q0:q1] - gpu_out[q0:q1]).max()))
                units += q1 - q0
            elif r.fp8:
                ref = oracle.fp8.paged_decode_fp8(case.query[[b]], kp, vp, case.block_tables[[b]],
                                                  case.context_lens[[b]], case.scale, f.k_scale, f.v_scale,
                                                  case.num_kv_heads, case.dtype)
                err = max(err, float(np.abs(ref[0] - gpu_out[b]).max()))
                units += 1
            else:
                ref = oracle.paged_decode(case.query[[b]], kp, vp, case.block_tables[[b]], case.context_lens[[b]],
                                          case.scale, case.num_kv_heads, case.dtype)
                err = max(err, float(np.abs(ref[0] - gpu_out[b]).max()))
                units += 1
            done.append(b)
            if time.perf_counter() - t0 > budget_s:
                break
        else:
            passes += 1
            continue
        break
    secs = time.perf_counter() - t0
    unit = "query-tokens/s" if call.startswith("prefill") else "seq-steps/s"
    return {"value": units / secs, "unit": unit, "cores": int(threads), "kind": "oracle",
            "sample": f"{len(done)} sequence-steps ({passes} whole passes over the {case.num_seqs}-sequence batch "
                      f"plus {len(done) - passes * case.num_seqs} sequences), all heads, fp64 NumPy, {secs:.1f} s",
            "max_abs_err_vs_gpu": err}


# ----------------------------------------------------------------------------
def calibration_copy(mib: int) -> None:
    """A plain device-to-device copy of ``mib`` MiB, three times (HBM counter calibration);
    issued right before the timed steps, after every other copy of the set-up."""
    if not mib:
        return
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def bench_block_copy(args) -> int:
    """pa_copy_blocks over a batch of copy-on-write pairs (one launch = one step), plus the
    device <-> pinned-host swap rates of pa_swap_blocks (copy engine, host-link bound)."""
    import torch
    import paged_kv_cache_463_amd as P
    from oracle import block_manager as OBM
    nb, hkv, d, npairs, nswap = BLOCK_WORKLOADS[args.workload]
    rng = np.random.default_rng(23)
    shape = (nb, 16, hkv, d)
    base = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(torch.bfloat16)
    kp = [base.cuda() for _ in range(args.layers)]
    vp = [(-base).cuda() for _ in range(args.layers)]
    perm = rng.permutation(nb)
    pairs_np = np.stack([perm[:npairs], perm[npairs:2 * npairs]], axis=1).astype(np.int32)
    pairs = torch.from_numpy(pairs_np).cuda()
    block_bytes = 16 * hkv * d * 2
    alg = npairs * 2 * block_bytes * 2                  # K and V, read and write
    calibration_copy(args.copy_calibration_mib)
    for i in range(args.warmup):
        P.copy_blocks(kp[i % args.layers], vp[i % args.layers], pairs)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        P.copy_blocks(kp[i % args.layers], vp[i % args.layers], pairs)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    achieved = alg / (us * 1e-6) / 1e9
    # swap: nswap blocks of one pool out to pinned host memory and back, timed with events
    host = torch.empty((nswap,) + shape[1:], dtype=torch.bfloat16, pin_memory=True)
    sw_out = [(int(b), i) for i, b in enumerate(perm[:nswap])]
    sw_in = [(i, int(b)) for i, b in enumerate(perm[:nswap])]
    rates = {}
    for name, (dst, src, prs) in {"out": (host, kp[0], sw_out), "in": (kp[0], host, sw_in)}.items():
        P.swap_blocks(dst, src, prs)
        torch.cuda.synchronize()
        # default events: their system-scope release is what completes the writes to host memory
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            P.swap_blocks(dst, src, prs)
        b.record(stream)
        torch.cuda.synchronize()
        rates[name] = 5 * nswap * block_bytes / (a.elapsed_time(b) * 1e-3) / 1e9
    res = {"metric": COPY_METRIC, "value": npairs * args.steps / elapsed, "unit": "blocks/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": elapsed * 1e3 / args.steps,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) pools, random disjoint copy pairs)",
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBPS,
                        "traffic": stored_traffic(args.workload, "copy_blocks", 0)},
           "copy_us_per_launch": us, "algorithmic_bytes_per_launch": alg,
           "swap_gb_per_s": {"device_to_host": rates["out"], "host_to_device": rates["in"],
                             "blocks": nswap, "block_bytes": block_bytes},
           "config": {"workload": args.workload, "kernel": "copy_blocks", "pool_blocks": nb,
                      "num_kv_heads": hkv, "head_dim": d, "block_size": 16, "copy_pairs": npairs,
                      "pool_replicas": args.layers}}
    if args.no_cpu_baseline:
        res["cpu_baseline"] = None
    else:
        kh, vh = base.float().numpy(), (-base).float().numpy()
        t0, done = time.perf_counter(), 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 5.0):
            OBM.copy_blocks(kh, vh, pairs_np[:256].tolist())
            done += 256
        secs = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": done / secs, "unit": "blocks/s", "cores": 1, "kind": "oracle",
                               "sample": f"{done} block copies (256-pair batches of the same pairs on "
                                         f"fp32 copies of the pools), NumPy, {secs:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS) + sorted(BLOCK_WORKLOADS))
    ap.add_argument("--kernel", default=None,
                    choices=["decode", "splitkv", "prefill", "decode_fp8", "splitkv_fp8", "prefill_fp8"],
                    help="attention entry point (default: the workload's)")
    ap.add_argument("--partition", type=int, default=512, help="split-KV partition size (tokens)")
    ap.add_argument("--layers", type=int, default=4, help="KV pool replicas rotated over steps")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-mode", default="separate", choices=["separate", "fused", "graph"],
                    help="separate: scatter launch + attention launch; fused: one pa_decode_step launch; "
                         "graph: the fused step replayed from a HIP graph (single-pass decode only)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-attention path here is built and timed on a single "
              "MI355X; run it with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import workloads as W

    if args.workload in BLOCK_WORKLOADS:
        return bench_block_copy(args)
    gen_key, call = WORKLOADS[args.workload]
    call = args.kernel or call
    t_gen = time.perf_counter()
    case = W.NAMED[gen_key]()
    t_gen = time.perf_counter() - t_gen
    if args.step_mode != "separate" and call not in ("decode", "decode_fp8"):
        print("--step-mode fused/graph applies to the single-pass decode workloads", file=sys.stderr)
        return 2
    if args.step_mode == "graph" and args.steps % args.layers:
        print("--step-mode graph replays all layers at once: --steps must be a multiple of --layers",
              file=sys.stderr)
        return 2
    r = Runner(case, call, args.layers, args.partition, args.step_mode)
    print(f"# workload {args.workload}: generated in {t_gen:.1f} s, kernel {call}", file=sys.stderr, flush=True)
    calibration_copy(args.copy_calibration_mib)

    elapsed, attn_ms = time_steps(r, args.steps, args.warmup)
    attn_us = float(np.mean(attn_ms)) * 1e3
    step_ms = elapsed * 1e3 / args.steps

    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": step_ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": case.dtype, "data": "synthetic (seeded N(0,1) K/V/Q, shuffled physical blocks)"}
    cfg = {"workload": args.workload, "kernel": call, "step_mode": args.step_mode, "block_size": 16,
           "num_seqs": case.num_seqs,
           "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
           "kv_pool_replicas": args.layers}
    if call.startswith("prefill"):
        flops = prefill_flops(case)
        tokens = case.num_q_tokens
        res.update({"value": tokens * args.steps / elapsed, "unit": "query-tokens/s"})
        achieved = flops / (attn_us * 1e-6) / 1e12
        res["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                           "traffic": stored_traffic(args.workload, call, args.partition)}
        res["prefill_causal_flops_per_step"] = flops
        cfg.update({"prior_tokens": int(case.prior_lens[0]), "chunk_tokens": int(case.q_lens[0]), "causal": True})
    else:
        ab_unique = decode_bytes(case, True, call)
        kv_logical, kv_unique = kv_bytes(case, False, call), kv_bytes(case, True, call)
        res.update({"value": case.num_seqs * args.steps / elapsed, "unit": "seq-steps/s"})
        achieved = ab_unique / (attn_us * 1e-6) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBPS,
                           "traffic": stored_traffic(args.workload, call, args.partition)}
        res["kv_gb_per_s"] = {"logical": kv_logical / (attn_us * 1e-6) / 1e9,
                              "unique": kv_unique / (attn_us * 1e-6) / 1e9}
        res["hbm_peak_frac"] = achieved / HBM_PEAK_GBPS
        res["algorithmic_bytes_per_launch"] = ab_unique
        cfg.update({"context_tokens": int(case.context_lens.astype(np.int64).sum()),
                    "max_context_len": case.max_context_len})
        if call.startswith("splitkv"):
            cfg["partition_size"] = args.partition
        if call.endswith("_fp8"):
            cfg["kv_cache_dtype"] = "fp8_e4m3"
            res["data"] = ("synthetic (seeded N(0,1) queries and new K/V, uniform e4m3 cache codes with "
                           "per-head scales, shuffled physical blocks)")
    res["attention_us_per_launch"] = attn_us
    res["scatter_bytes_per_step"] = scatter_bytes(case, call)
    res["config"] = cfg
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(case, call, r, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
