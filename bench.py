"""Throughput of the paged-attention hot path on one MI355X.

One step = one attention layer of one decode step (or one prefill chunk) over
the whole batch: ``pa_reshape_and_cache`` of the new tokens, then the attention
call, both on torch's current stream. The KV pool is replicated over
``--layers`` independent copies and steps rotate through them, the way a model
walks its layers, so repeated steps are not served from the 256 MB
last-level cache. Inputs are seeded synthetic tensors resident in HBM before
the timed region starts.

Prints ONE JSON line. By default its headline is the long-context split-KV
decode (8 sequences of 32k-131k tokens, the largest decode workload on one
GPU), and the tiny fp32 decode, the Llama-2-7B-like fp16 decode, the
Llama-3-8B-like GQA decode and the chunked prefill ride along as records of
the same line (``configs``); ``--workload`` times one workload alone. Per
workload: value = sequence-steps per second (decode) or query tokens per
second (prefill) for the whole job, the roofline of the attention kernel
(algorithmic bytes or flops per launch divided by its average duration,
measured with HIP events on the launch stream inside the timed region), and
the CPU oracle timed on a bounded sample of the same workload (worker
processes over (sequence, kv head) units, one BLAS thread each, forked before
this process touches the GPU).
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
    def __init__(self, case, call: str, layers: int, partition: int, step_mode: str = "separate",
                 fp8_host=None):
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
            f = fp8_host if fp8_host is not None else W.fp8_pools(case, 0)
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
# CPU baseline: the oracle as it stands, over (sequence, kv head) units
# ----------------------------------------------------------------------------
# One unit = the oracle's decode (or prefill chunk) of one sequence restricted to one kv head's
# G query heads, on the head's slice of the scattered pools. The units run in worker processes
# forked before this process touches the GPU (so they share the host arrays and never open the
# device), one BLAS thread each; the sample is every unit of whole passes over the batch, in a
# seeded order, until a time budget is spent.
_UNITS = None            # the host context of the workload being timed, read by the workers


def _unit_ctx(case, call: str, fp8_host=None):
    """Scattered host pools (the oracle's own scatter) and what the units need."""
    import oracle
    if fp8_host is not None:
        kp, vp = oracle.fp8.scatter_fp8(fp8_host.k_pool, fp8_host.v_pool, case.k_new, case.v_new,
                                        case.slot_mapping, fp8_host.k_scale, fp8_host.v_scale, case.dtype)
    else:
        kp, vp = oracle.scatter(case.k_pool, case.v_pool, case.k_new, case.v_new, case.slot_mapping)
    return {"case": case, "prefill": call.startswith("prefill"), "fp8": fp8_host, "kp": kp, "vp": vp}


def _oracle_unit(bg):
    """The oracle on unit (b, g); returns (b, g, float64 output rows [rows, G, D])."""
    import oracle
    b, g = bg
    c = _UNITS
    case, f = c["case"], c["fp8"]
    G = case.num_q_heads // case.num_kv_heads
    hs = slice(g * G, (g + 1) * G)
    kp, vp = c["kp"][:, :, g:g + 1], c["vp"][:, :, g:g + 1]
    if c["prefill"]:
        q0, q1 = int(case.cu_q_lens[b]), int(case.cu_q_lens[b + 1])
        args = (case.query[q0:q1, hs], kp, vp, case.block_tables[b:b + 1], case.seq_lens[b:b + 1],
                np.array([0, q1 - q0], dtype=np.int32), case.scale)
        if f is not None:
            out = oracle.fp8.paged_prefill_fp8(*args, f.k_scale[g:g + 1], f.v_scale[g:g + 1], 1, case.dtype)
        else:
            out = oracle.paged_prefill(*args, 1, case.dtype)
    else:
        args = (case.query[b:b + 1, hs], kp, vp, case.block_tables[b:b + 1], case.context_lens[b:b + 1],
                case.scale)
        if f is not None:
            out = oracle.fp8.paged_decode_fp8(*args, f.k_scale[g:g + 1], f.v_scale[g:g + 1], 1, case.dtype)
        else:
            out = oracle.paged_decode(*args, 1, case.dtype)
    return b, g, out


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def cpu_baseline(ctx, budget_s: float, workers: int):
    """Time the oracle on a bounded sample of the workload: whole passes over the batch (every
    (sequence, kv head) unit once per pass, in a seeded order) until ``budget_s`` is spent, at
    least one pass. ``workers`` processes are forked now, before any GPU call in this process;
    each pass is one ``map`` over the pool, and the pool is closed and joined, never terminated
    with work in flight. Returns (record, {(b, g): rows}) for the parity check against the GPU
    output."""
    import multiprocessing as mp
    global _UNITS
    _UNITS = ctx
    case = ctx["case"]
    B, H = case.num_seqs, case.num_kv_heads
    order = [(int(b), g) for b in np.random.default_rng(0).permutation(B) for g in range(H)]
    units, passes = {}, 0
    t0 = time.perf_counter()
    if workers <= 1:
        while passes == 0 or time.perf_counter() - t0 < budget_s:
            for bg in order:
                b, g, out = _oracle_unit(bg)
                units[(b, g)] = out
            passes += 1
    else:
        pool = mp.get_context("fork").Pool(workers, initializer=_one_blas_thread)
        try:
            while passes == 0 or time.perf_counter() - t0 < budget_s:
                for b, g, out in pool.map(_oracle_unit, order, chunksize=1):
                    units[(b, g)] = out
                passes += 1
        finally:
            pool.close()
            pool.join()
    secs = time.perf_counter() - t0
    _UNITS = None
    prefill = ctx["prefill"]
    if prefill:
        value, unit = passes * int(case.q_lens.sum()) / secs, "query-tokens/s"
    else:
        value, unit = passes * B / secs, "seq-steps/s"
    rec = {"value": value, "unit": unit, "cores": int(workers), "kind": "oracle",
           "sample": f"{passes} whole pass{'es' if passes > 1 else ''} over the {B}-sequence batch "
                     f"({'prefill chunks' if prefill else 'decode steps'}) as {passes * len(order)} "
                     f"(sequence, kv head) units, fp64 NumPy, {workers} process{'es' if workers > 1 else ''} "
                     f"x 1 BLAS thread, {secs:.1f} s"}
    return rec, units


def oracle_error(case, prefill: bool, units: dict, gpu_out: np.ndarray) -> float:
    """Largest |gpu - oracle| over the rows the CPU baseline computed."""
    G = case.num_q_heads // case.num_kv_heads
    err = 0.0
    for (b, g), ref in units.items():
        if prefill:
            q0, q1 = int(case.cu_q_lens[b]), int(case.cu_q_lens[b + 1])
            got = gpu_out[q0:q1, g * G:(g + 1) * G]
        else:
            got = gpu_out[b:b + 1, g * G:(g + 1) * G]
        if got.size:
            err = max(err, float(np.abs(got - ref).max()))
    return err


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


# The default run: the long-context split-KV decode is the headline line (the largest
# single-GPU decode workload, 2.8 GB of KV per step), the other workloads are records in the
# same run.
HEADLINE = "long_ctx_bf16_splitkv_b8"
DEFAULT_SET = [HEADLINE, "tiny_fp32_decode_b4", "llama2_7b_fp16_decode_b64", "llama3_8b_gqa_bf16_decode_b256",
               "chunked_prefill_bf16_16x2048p512"]
# workloads that also get a single-core oracle figure
SINGLE_CORE = {"tiny_fp32_decode_b4", "llama2_7b_fp16_decode_b64", "llama3_8b_gqa_bf16_decode_b256"}


def time_read_probe(r: Runner, steps: int, warmup: int) -> dict:
    """Time pa_read_kv_rows over the same pools, tables and walk as the attention call (its
    K/V rows with the same loads and no arithmetic): the practical read ceiling of that access
    set. Bytes counted are those it reads: every table block of every sequence, whole."""
    import workloads as W
    torch, P, case = r.torch, r.P, r.case
    part = r.partition if r.call.startswith("splitkv") else 0
    waves = 4 * (case.num_kv_heads * case.num_seqs * (W.ceil_div(max(case.max_context_len, 1), part) if part else 1))
    sink = torch.zeros(max(waves, 1), dtype=torch.int32, device="cuda")
    mcl = max(case.max_context_len, 1)
    for i in range(warmup):
        P.read_kv_rows(r.kp[i % r.layers], r.vp[i % r.layers], r.bt, r.lens, mcl, part, sink)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(TimingEvent(), TimingEvent()) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        P.read_kv_rows(r.kp[i % r.layers], r.vp[i % r.layers], r.bt, r.lens, mcl, part, sink)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    blocks = sum(W.ceil_div(int(L), W.BLOCK_SIZE) for L in case.context_lens)
    nbytes = blocks * W.BLOCK_SIZE * 2 * case.num_kv_heads * case.head_dim * kv_elem_bytes(case, r.call)
    return {"us_per_launch": us, "bytes_per_launch": nbytes, "gb_per_s": nbytes / (us * 1e-6) / 1e9,
            "frac_of_hbm_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "walk": "split-KV" if part else "single pass"}


def time_workload(args, name: str, case, call: str, host: dict) -> dict:
    """Upload one workload, time ``args.steps`` steps and return its record."""
    import torch
    r = Runner(case, call, args.layers, args.partition, args.step_mode, host.get("fp8"))
    calibration_copy(args.copy_calibration_mib)
    elapsed, attn_ms = time_steps(r, args.steps, args.warmup)
    attn_us = float(np.mean(attn_ms)) * 1e3
    rec = {"workload": name, "kernel": call, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": elapsed * 1e3 / args.steps, "dtype": case.dtype}
    cfg = {"workload": name, "kernel": call, "step_mode": args.step_mode, "block_size": 16,
           "num_seqs": case.num_seqs, "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
           "head_dim": case.head_dim, "kv_pool_replicas": args.layers}
    if call.startswith("prefill"):
        flops = prefill_flops(case)
        rec.update({"value": case.num_q_tokens * args.steps / elapsed, "unit": "query-tokens/s"})
        achieved = flops / (attn_us * 1e-6) / 1e12
        rec["roofline"] = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                           "traffic": stored_traffic(name, call, args.partition)}
        rec["prefill_causal_flops_per_step"] = flops
        cfg.update({"prior_tokens": int(case.prior_lens[0]), "chunk_tokens": int(case.q_lens[0]), "causal": True})
    else:
        ab_unique = decode_bytes(case, True, call)
        kv_logical, kv_unique = kv_bytes(case, False, call), kv_bytes(case, True, call)
        rec.update({"value": case.num_seqs * args.steps / elapsed, "unit": "seq-steps/s"})
        achieved = ab_unique / (attn_us * 1e-6) / 1e9
        rec["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                           "frac": achieved / HBM_PEAK_GBPS,
                           "traffic": stored_traffic(name, call, args.partition)}
        rec["kv_gb_per_s"] = {"logical": kv_logical / (attn_us * 1e-6) / 1e9,
                              "unique": kv_unique / (attn_us * 1e-6) / 1e9}
        rec["hbm_peak_frac"] = achieved / HBM_PEAK_GBPS
        rec["algorithmic_bytes_per_launch"] = ab_unique
        cfg.update({"context_tokens": int(case.context_lens.astype(np.int64).sum()),
                    "max_context_len": case.max_context_len})
        if call.startswith("splitkv"):
            cfg["partition_size"] = args.partition
        if call.endswith("_fp8"):
            cfg["kv_cache_dtype"] = "fp8_e4m3"
        if not args.no_read_probe and args.step_mode == "separate":
            rp = time_read_probe(r, args.steps, args.warmup)
            rp["attention_time_over_probe"] = attn_us / rp["us_per_launch"]
            rec["read_probe"] = rp
    rec["attention_us_per_launch"] = attn_us
    rec["attention_us_stats"] = {"median": float(np.median(attn_ms)) * 1e3, "min": float(np.min(attn_ms)) * 1e3,
                                 "max": float(np.max(attn_ms)) * 1e3}
    rec["scatter_bytes_per_step"] = scatter_bytes(case, call)
    rec["config"] = cfg
    cb = host.get("cpu_baseline")
    if cb is not None:
        gpu_out = r.out.float().cpu().double().numpy()
        cb = dict(cb)
        cb["max_abs_err_vs_gpu"] = oracle_error(case, call.startswith("prefill"), host["units"], gpu_out)
    rec["cpu_baseline"] = cb
    del r
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS) + sorted(BLOCK_WORKLOADS),
                    help="time only this workload (default: the headline workload plus the other "
                         "configurations as records of the same line)")
    ap.add_argument("--kernel", default=None,
                    choices=["decode", "splitkv", "prefill", "decode_fp8", "splitkv_fp8", "prefill_fp8"],
                    help="attention entry point (default: the workload's; with --workload only)")
    ap.add_argument("--partition", type=int, default=512, help="split-KV partition size (tokens)")
    ap.add_argument("--layers", type=int, default=4, help="KV pool replicas rotated over steps")
    ap.add_argument("--cpu-budget", type=float, default=5.0,
                    help="seconds of oracle work per workload for cpu_baseline (and again for the "
                         "single-core figure where one is taken)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle worker processes (default: the CPUs this process may run on)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip timing the read-only pass over the same K/V rows (decode workloads)")
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

    import workloads as W

    if args.workload in BLOCK_WORKLOADS:
        return bench_block_copy(args)
    names = [args.workload] if args.workload else DEFAULT_SET
    if args.kernel and not args.workload:
        print("--kernel needs --workload", file=sys.stderr)
        return 2
    if args.step_mode != "separate" and not all(WORKLOADS[n][1] in ("decode", "decode_fp8") or args.kernel
                                                for n in names):
        print("--step-mode fused/graph applies to the single-pass decode workloads: pass --workload",
              file=sys.stderr)
        return 2
    if args.step_mode == "graph" and args.steps % args.layers:
        print("--step-mode graph replays all layers at once: --steps must be a multiple of --layers",
              file=sys.stderr)
        return 2
    workers = args.cpu_workers or len(os.sched_getaffinity(0))

    # host phase (no GPU call yet): inputs, and the oracle's CPU baseline on them. This
    # process keeps one BLAS thread, so the workers it forks inherit no BLAS thread pool.
    _one_blas_thread()
    hosts = {}
    for name in names:
        gen_key, call = WORKLOADS[name]
        call = args.kernel or call
        t_gen = time.perf_counter()
        case = W.NAMED[gen_key]()
        t_gen = time.perf_counter() - t_gen
        fp8_host = W.fp8_pools(case, 0) if call.endswith("_fp8") else None
        host = {"case": case, "call": call, "fp8": fp8_host, "cpu_baseline": None, "units": {}}
        if not args.no_cpu_baseline:
            ctx = _unit_ctx(case, call, fp8_host)
            rec, units = cpu_baseline(ctx, args.cpu_budget, workers)
            if name in SINGLE_CORE:
                one, _ = cpu_baseline(ctx, args.cpu_budget, 1)
                rec["single_core"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
            del ctx
            host.update(cpu_baseline=rec, units=units)
            print(f"# {name}: oracle baseline {rec['value']:.4g} {rec['unit']} ({rec['sample']})",
                  file=sys.stderr, flush=True)
        hosts[name] = host
        print(f"# workload {name}: generated in {t_gen:.1f} s, kernel {call}", file=sys.stderr, flush=True)

    records = {}
    for name in names:
        h = hosts.pop(name)
        records[name] = time_workload(args, name, h["case"], h["call"], h)
        print(f"# {name}: {records[name]['attention_us_per_launch']:.1f} us per launch, "
              f"roofline {records[name]['roofline']['frac']:.3f}", file=sys.stderr, flush=True)

    head = records[names[0]]
    res = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": head["dtype"],
           "data": "synthetic (seeded N(0,1) K/V/Q, shuffled physical blocks)",
           "value": head["value"], "unit": head["unit"], "roofline": head["roofline"]}
    for k in ("kv_gb_per_s", "hbm_peak_frac", "algorithmic_bytes_per_launch", "prefill_causal_flops_per_step",
              "attention_us_per_launch", "attention_us_stats", "scatter_bytes_per_step", "read_probe"):
        if k in head:
            res[k] = head[k]
    if head["kernel"].endswith("_fp8"):
        res["data"] = ("synthetic (seeded N(0,1) queries and new K/V, uniform e4m3 cache codes with "
                       "per-head scales, shuffled physical blocks)")
    res["config"] = head["config"]
    res["cpu_baseline"] = head["cpu_baseline"]
    if len(names) > 1:
        res["configs"] = {n: records[n] for n in names[1:]}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
