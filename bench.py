#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Workload: the Llama-3-8B-shaped decode layer in bf16 -- 64 requests with KV
lengths uniform in [512, 4096], 32 query heads over 8 KV heads (GQA 4:1),
head_dim 128, 16-token blocks, a pool 1.2x the blocks needed, shuffled block
tables. One step = the slot_mapping write of the 64 new tokens' K/V plus paged
GQA decode attention over every request's whole KV (split-K partials and the
LSE merge when the step uses them).

Inputs are synthetic and seeded, generated on the GPU, and resident in HBM
before timing. Steps rotate over several independent copies of the inputs so
no step finds the previous step's KV in the 256 MB last-level cache. Each step
is a prepared call of the binding (checked and marshalled once), so the timed
loop pays one ctypes call per step.

Printed: one JSON line. ``value`` is the step's algorithmic HBM traffic
divided by the step time (GB/s). ``roofline`` is for the attention call,
timed with HIP events recorded on the stream it is launched on (mean, median
and min over the steps). ``read_ceiling`` gives what loads-only kernels reach
on the same bytes. ``cpu_baseline`` is the fp64 CPU oracle on the same
workload; every secondary leg carries its own streamed oracle sample.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged GQA decode: achieved HBM GB/s (% of peak) + decode tokens/s per layer"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
ATTN_SOURCES = ["attention.hip", "balanced.hip", "attn_tile.h", "pa_launch.h", "pa_api.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in ATTN_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_221_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_bytes(layout, kv_elem_bytes=None) -> int:
    """Bytes decode attention must move: every request's K and V, Q in and O
    out, the block-table entries it follows and seq_lens. ``kv_elem_bytes``
    overrides the cache element size (1 for an E4M3 cache; q and out keep
    the layout's)."""
    e = layout.elem_bytes
    kvb = 2 * layout.num_kv_heads * layout.head_dim * (kv_elem_bytes or e)
    bs = layout.block_size
    lens = layout.seq_lens.astype("int64")
    blocks = (lens + bs - 1) // bs
    qo = 2 * layout.num_seqs * layout.num_heads * layout.head_dim * e
    return int(lens.sum() * kvb + qo + 4 * blocks.sum() + 4 * layout.num_seqs)


def write_bytes(layout) -> int:
    """Bytes the KV write must move: read and write K+V rows, read slots."""
    kvb = 2 * layout.num_kv_heads * layout.head_dim * layout.elem_bytes
    return int(2 * layout.num_tokens * kvb + 8 * layout.num_tokens)


def varlen_bytes(layout, kv_elem_bytes=None) -> int:
    """Per-request KV bytes of a varlen step (each request reads its KV once);
    ``kv_elem_bytes`` as in decode_bytes."""
    e = layout.elem_bytes
    kvb = 2 * layout.num_kv_heads * layout.head_dim * (kv_elem_bytes or e)
    lens = layout.seq_lens.astype("int64")
    qo = 2 * layout.num_tokens * layout.num_heads * layout.head_dim * e
    blocks = (lens + layout.block_size - 1) // layout.block_size
    return int(lens.sum() * kvb + qo + 4 * blocks.sum() + 4 * (2 * layout.num_seqs + 1))


def causal_flops(layout) -> int:
    """FLOPs of exact causal attention over a varlen step: query row i of a
    request with n rows and KV length L sees L - n + i + 1 keys, each costing
    2 D FLOPs for QK and 2 D for PV, per query head."""
    pairs = 0
    for n, length in zip(layout.query_lens.tolist(), layout.seq_lens.tolist()):
        pairs += n * (length - n) + n * (n + 1) // 2
    return int(pairs * layout.num_heads * layout.head_dim * 4)


def shared_prefix_bytes(layout, kv_elem_bytes=None) -> int:
    """KV bytes a varlen step reads more than once: every sharer after the
    first reads the shared prefix blocks again."""
    sharers = int((layout.block_table[:, :1] == layout.shared_blocks[:1]).sum()) \
        if len(layout.shared_blocks) else 0
    kvb = 2 * layout.num_kv_heads * layout.head_dim * (kv_elem_bytes or layout.elem_bytes)
    return max(sharers - 1, 0) * len(layout.shared_blocks) * layout.block_size * kvb


# Kernels launched by the timed attention call of each path.
PATH_KERNELS = {
    "decode": "paged_attention_kernel",
    "balanced": "balanced_decode_kernel + balanced_merge_kernel",
    "fused": "balanced_decode_kernel with the KV write fused in + balanced_merge_kernel",
    "splitk": "paged_attention_kernel (split-K partials) + lse_merge_kernel",
}


def load_traffic(src_hash: str, path_name: str):
    """HBM bytes per attention call from the committed counter summary, if it
    was taken on the current kernel sources and the same path."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != src_hash or t.get("path") != path_name:
        return None
    return t.get("bytes_per_launch")


def host_info():
    """Host cores: the machine's count and the ones this process may use."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_count": os.cpu_count(), "sched_getaffinity": affinity}


def blas_threads() -> int:
    from threadpoolctl import threadpool_info
    return max([x.get("num_threads", 1) for x in threadpool_info()] or [1])


class DecodeStep:
    """One step on one copy of the inputs: write, then attention; each call
    of the library prepared once (tensors checked, arguments marshalled)."""

    def __init__(self, st, path: str, split_tokens: int, kv_scales=None):
        import torch
        import paged_kv_cache_221_amd as pa
        self.st, self.path = st, path
        kw = {} if kv_scales is None else {"k_scale": kv_scales[0], "v_scale": kv_scales[1]}
        lay = st.layout
        out = torch.empty_like(st.q)
        self.out = out
        common = (st.block_table, st.seq_lens, lay.max_seq_len)
        self.write = None
        self.after = None
        if path in ("balanced", "fused"):
            n = pa.pa_decode_balanced_workspace_bytes(st.k_cache, st.v_cache, lay.num_seqs,
                                                      lay.num_heads)
            ws = torch.zeros(n, dtype=torch.uint8, device=st.q.device)
        if path != "fused":
            self.write = pa.pa_write_kv(st.k_cache, st.v_cache, st.k_new, st.v_new,
                                        st.slot_mapping, prepared=True, **kw)
        if path == "fused":
            self.attn = pa.pa_write_decode_balanced(
                st.k_cache, st.v_cache, st.q, st.k_new, st.v_new, st.slot_mapping, *common,
                lay.scale, workspace=ws, out=out, prepared=True, **kw)
        elif path == "balanced":
            self.attn = pa.pa_decode_balanced(st.k_cache, st.v_cache, st.q, *common, lay.scale,
                                              workspace=ws, out=out, prepared=True, **kw)
        elif path == "decode":
            self.attn = pa.pa_decode(st.k_cache, st.v_cache, st.q, *common, lay.scale, out=out,
                                     prepared=True, **kw)
        else:
            s = pa.pa_splitk_num_splits(lay.max_seq_len, split_tokens)
            b, hq, d = st.q.shape
            o_part = torch.empty((b, hq, s, d), dtype=torch.float32, device=st.q.device)
            lse_part = torch.empty((b, hq, s), dtype=torch.float32, device=st.q.device)
            self.attn = pa.pa_decode_splitk(st.k_cache, st.v_cache, st.q, *common, split_tokens,
                                            lay.scale, o_part=o_part, lse_part=lse_part,
                                            prepared=True, **kw)
            # the merge belongs to the split-K attention call [P1 §07]
            self.after = pa.pa_lse_merge(o_part, lse_part, st.seq_lens, lay.max_seq_len,
                                         split_tokens, out_dtype=st.q.dtype, out=out,
                                         prepared=True)

    def __call__(self, ev=None):
        if self.write is not None:
            self.write()
        if ev is not None:
            ev[0].record()
        self.attn()
        if self.after is not None:
            self.after()
        if ev is not None:
            ev[1].record()


def _stats(vals):
    return {"mean": statistics.fmean(vals), "median": statistics.median(vals), "min": min(vals)}


def time_steps(steps_fns, k: int, w: int, kernel_events: bool):
    """Eager timing: W warmup steps, then K timed steps between two
    synchronisations. Returns the step time (ms), the host's launch time per
    step (us: until the last launch returned), and with ``kernel_events``
    the per-step event times of the attention call (ms) instead."""
    import torch
    n = len(steps_fns)
    for i in range(w):
        steps_fns[i % n]()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(k)] if kernel_events else [None] * k
    t0 = time.perf_counter()
    for i in range(k):
        steps_fns[i % n](evs[i])
    t_launch = time.perf_counter()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = [a.elapsed_time(b) for a, b in evs] if kernel_events else None
    return (t1 - t0) * 1e3 / k, (t_launch - t0) * 1e6 / k, kern


def time_graph(steps_fns, k: int, w: int):
    """Graph timing: the steps of every input copy, in turn, captured as one
    HIP graph (a graph launch costs ~8 us of its own per replay, more than a
    kernel launch, so one step per graph would time the launches), replayed
    until exactly K steps ran; a remainder of K is a graph of its first K mod
    n steps."""
    import torch
    n = len(steps_fns)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for fn in steps_fns:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    def capture(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in fns:
                fn()
        return g
    whole = capture(steps_fns)
    rest = capture(steps_fns[:k % n]) if k % n else None
    for _ in range(max(1, -(-w // n))):
        whole.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(k // n):
        whole.replay()
    if rest is not None:
        rest.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / k


def timed_leg(nbytes, kern, step_ms=None, extra=None):
    """A secondary leg's entry: attention call time (event mean, median,
    min) and GB/s and fraction of 8 TB/s at the median."""
    s = _stats(kern)
    med = s["median"]
    out = {"attention_kernel_ms": round(s["mean"], 4),
           "attention_ms_median": round(med, 4), "attention_ms_min": round(s["min"], 4),
           "attention_GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
           "attention_frac_of_8TBps": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "algorithmic_bytes": nbytes}
    if step_ms is not None:
        out = {"step_ms": round(step_ms, 4), **out}
    if extra:
        out.update(extra)
    return out


# ---------------------------------------------------------------- oracle legs
def cpu_baseline(st, layout, budget_s: float):
    """The fp64 oracle on the whole headline step (write + decode of all
    requests), repeated until ``budget_s`` of CPU time has been spent."""
    import oracle
    from workloads.tensors import raw_bits
    dt = layout.dtype
    k0, v0 = raw_bits(st.k_cache, dt).copy(), raw_bits(st.v_cache, dt).copy()
    q, kn, vn = raw_bits(st.q, dt), raw_bits(st.k_new, dt), raw_bits(st.v_new, dt)
    reps, spent = 0, 0.0
    while spent < budget_s or reps == 0:
        t = time.perf_counter()
        oracle.write_kv(k0, v0, kn, vn, layout.slot_mapping, layout.block_size)
        oracle.paged_decode(q, k0, v0, layout.block_table, layout.seq_lens, layout.scale,
                            layout.block_size, dt)
        spent += time.perf_counter() - t
        reps += 1
    per_step = spent / reps
    threads = blas_threads()
    gbs = (decode_bytes(layout) + write_bytes(layout)) / per_step / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"whole step ({layout.num_seqs} requests, {int(layout.seq_lens.sum())} "
                      f"KV tokens) repeated {reps}x, {per_step:.2f} s per step; numpy fp64 "
                      f"with BLAS on {threads} threads",
            **host_info()}


def oracle_sample(st, layout, requests, kind: str, split_tokens=None, kv=None):
    """The oracle timed on a few requests of a leg's workload, streaming only
    their blocks to the host: GB/s of those requests' algorithmic bytes."""
    import numpy as np
    import oracle
    from workloads.tensors import blocks_as_dict, raw_bits
    dt = layout.dtype
    bs = layout.block_size
    ids = set()
    for r in requests:
        ids.update(int(b) for b in layout.block_table[r, :-(-int(layout.seq_lens[r]) // bs)])
    kdt = kv["dtype"] if kv else dt
    k = blocks_as_dict(st.k_cache, ids, kdt)
    v = blocks_as_dict(st.v_cache, ids, kdt)
    q = raw_bits(st.q, dt)
    extra = {} if kv is None else dict(kv_dtype=kv["dtype"], k_scale=kv["k_scale"],
                                       v_scale=kv["v_scale"])
    t0 = time.perf_counter()
    if kind == "decode":
        oracle.paged_decode(q, k, v, layout.block_table, layout.seq_lens, layout.scale, bs, dt,
                            requests=requests, **extra)
    elif kind == "splitk":
        s = -(-layout.max_seq_len // split_tokens)
        o, lse = oracle.splitk_partials(q, k, v, layout.block_table, layout.seq_lens,
                                        layout.scale, bs, dt, split_tokens, s,
                                        requests=requests)
        oracle.lse_merge(o[requests], lse[requests])
    else:
        oracle.paged_varlen(q, k, v, layout.cu_seqlens_q, layout.seq_lens, layout.block_table,
                            layout.scale, bs, dt, requests=requests, **extra)
    dt_s = time.perf_counter() - t0
    kvb = 2 * layout.num_kv_heads * layout.head_dim * (1 if kv else layout.elem_bytes)
    toks = int(np.asarray(layout.seq_lens)[requests].sum())
    rows = int(sum(int(layout.query_lens[r]) for r in requests))
    nbytes = toks * kvb + 2 * rows * layout.num_heads * layout.head_dim * layout.elem_bytes
    return {"GBps": round(nbytes / dt_s / 1e9, 4), "seconds": round(dt_s, 3),
            "sample": f"{len(requests)} of {layout.num_seqs} requests ({toks} KV tokens, "
                      f"{rows} query rows), numpy fp64 with BLAS on {blas_threads()} threads",
            "kind": "oracle"}


# ---------------------------------------------------------------- read ceiling
def read_ceiling(copies, layout, k: int):
    """Loads-only kernels (libpa_probe.so) over the headline's bytes: the
    decode call's block walk (every request's blocks in table order, K and V,
    the input copies in turn) and a contiguous sweep of as many bytes."""
    import ctypes
    import numpy as np
    import torch
    from paged_kv_cache_221_amd import build as pa_build
    if not os.path.exists(pa_build.PROBE_LIB_PATH):
        return {"error": "libpa_probe.so is not built"}
    lib = ctypes.CDLL(pa_build.PROBE_LIB_PATH)
    lib.pa_probe_read_linear.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]
    lib.pa_probe_read_blocks.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    bs = layout.block_size
    lens = layout.seq_lens.astype("int64")
    walk = np.concatenate([layout.block_table[r, :-(-int(lens[r]) // bs)]
                           for r in range(layout.num_seqs)]).astype(np.int32)
    dev_walk = torch.from_numpy(walk).cuda()
    block_bytes = copies[0].k_cache[0].numel() * copies[0].k_cache.element_size()
    nbytes = 2 * len(walk) * block_bytes
    props = torch.cuda.get_device_properties(0)
    grid = props.multi_processor_count
    sink = torch.empty(grid * 512, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(len(copies))]
    for b in bufs:
        b.fill_(1)

    def run(launch):
        n = max(k, 20)
        for i in range(5):
            launch(i)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i in range(n):
            evs[i][0].record()
            if launch(i) != 0:
                raise RuntimeError("probe launch failed")
            evs[i][1].record()
        torch.cuda.synchronize()
        return _stats([a.elapsed_time(b) for a, b in evs])

    walk_t = run(lambda i: lib.pa_probe_read_blocks(
        copies[i % len(copies)].k_cache.data_ptr(), copies[i % len(copies)].v_cache.data_ptr(),
        layout.num_blocks, block_bytes, dev_walk.data_ptr(), len(walk), sink.data_ptr(), grid,
        stream))
    lin_t = run(lambda i: lib.pa_probe_read_linear(bufs[i % len(bufs)].data_ptr(), nbytes,
                                                   sink.data_ptr(), grid, stream))
    del bufs

    def entry(t):
        return {"ms_median": round(t["median"], 4), "ms_min": round(t["min"], 4),
                "GBps": round(nbytes / (t["median"] * 1e-3) / 1e9, 1),
                "frac_of_8TBps": round(nbytes / (t["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    return {"bytes": nbytes, "workgroups": grid,
            "paged_block_walk": entry(walk_t), "linear_sweep": entry(lin_t),
            "note": "loads only (nt), no attention: the decode call's K and V blocks in "
                    "table order, and a contiguous read of as many bytes"}


# ---------------------------------------------------------------- secondary legs
SECONDARY_LEGS = ("tiny-decode-fp32", "long-context-splitk-bf16", "llama2-7b-mha-decode-fp16",
                  "mixed-step-bf16", "mixed-step-prefill-chunks-bf16",
                  "mixed-step-prefill-chunks-e4m3-cache", "mixed-step-e4m3-cache",
                  "llama3-8b-decode-e4m3-cache", "long-context-splitk-e4m3-cache",
                  "llama3-8b-spec-verify-q4-bf16",
                  "rope-write-kv-mixed-step-bf16", "copy-on-write-blocks-bf16",
                  "block-manager-host")


def secondary_isolated(args):
    """Every secondary leg in a child process of its own (``--only``), as a
    serving process would allocate its pool once: run in this process after
    the headline's inputs and the earlier legs' pools, the 16 GiB MHA leg
    measured 4-8% slower (2.90-3.03 ms against 2.79 ms alone). The children
    print their progress on stderr; each prints one JSON line on stdout."""
    res = {}
    for leg in SECONDARY_LEGS:
        cmd = [sys.executable, os.path.abspath(__file__), "--only", leg,
               "--steps", str(args.steps), "--warmup", str(args.warmup)]
        try:
            p = subprocess.run(cmd, stdout=subprocess.PIPE, text=True, timeout=900)
        except subprocess.TimeoutExpired:
            res[leg] = {"error": "timed out after 900 s"}
            continue
        if p.returncode != 0 or not p.stdout.strip():
            # a failed leg is reported, and the headline line still printed
            print(f"[bench] secondary leg {leg} failed with status {p.returncode}",
                  file=sys.stderr, flush=True)
            res[leg] = {"error": f"exit status {p.returncode}"}
            continue
        res.update(json.loads(p.stdout.strip().splitlines()[-1])["secondary"])
    return res


def secondary(args, only=None):
    """Per-config attention timings on the other step shapes (not the metric);
    with ``only``, just that leg (for profiling one workload)."""
    import torch
    import paged_kv_cache_221_amd as pa
    from workloads import llama2_7b_mha_decode, long_context_splitk, mixed_step
    from workloads.tensors import materialize
    res = {}
    k = max(5, min(args.steps, 20))
    for name, fn in (("long-context-splitk-bf16", long_context_splitk),
                     ("llama2-7b-mha-decode-fp16", llama2_7b_mha_decode),
                     ("mixed-step-bf16", mixed_step)):
        if only is not None and name != only:
            continue
        lay = fn()
        st = materialize(lay, "cuda", poison=False)
        if name.startswith("long"):
            step = DecodeStep(st, "splitk", lay.split_tokens)
            nbytes = decode_bytes(lay)
            sample = dict(requests=[0], kind="splitk", split_tokens=lay.split_tokens)
        elif name.startswith("llama2"):
            step = DecodeStep(st, "decode", 0)
            nbytes = decode_bytes(lay)
            sample = dict(requests=[0, lay.num_seqs - 1], kind="decode")
        else:
            out = torch.empty_like(st.q)
            ws = torch.empty(pa.pa_varlen_workspace_bytes(st.k_cache, st.v_cache, lay.num_seqs,
                                                          st.q.shape[0], lay.num_heads,
                                                          st.block_table.shape[1]),
                             dtype=torch.uint8, device="cuda")
            write = pa.pa_write_kv(st.k_cache, st.v_cache, st.k_new, st.v_new, st.slot_mapping,
                                   prepared=True)
            attn = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                                st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                                out=out, workspace=ws, prepared=True)

            def step(ev=None, write=write, attn=attn):
                write()
                if ev is not None:
                    ev[0].record()
                attn()
                if ev is not None:
                    ev[1].record()
            nbytes = varlen_bytes(lay)
            dec = [r for r in range(lay.num_seqs) if lay.query_lens[r] == 1]
            sample = dict(requests=[1] + dec[:4], kind="varlen")
        ms, _, kern = time_steps([step], k, 3, True)
        extra = {}
        if name.startswith("mixed"):
            uniq = nbytes - shared_prefix_bytes(lay)
            extra = {"unique_bytes": uniq,
                     "attention_unique_GBps": round(uniq / (statistics.median(kern) * 1e-3)
                                                    / 1e9, 1)}
        if name.startswith("long"):
            extra = {"includes": "split-K partials and the LSE merge"}
        res[name] = timed_leg(nbytes, kern, ms, extra)
        res[name]["cpu_oracle"] = oracle_sample(st, lay, **sample)
        print(f"[bench] {name}: attention median {statistics.median(kern):.4f} ms",
              file=sys.stderr, flush=True)
        del st, step
        torch.cuda.empty_cache()
    for name, leg in (("tiny-decode-fp32", bench_tiny),
                      ("mixed-step-prefill-chunks-bf16", bench_prefill_only),
                      ("mixed-step-prefill-chunks-e4m3-cache", bench_prefill_only_fp8),
                      ("mixed-step-e4m3-cache", bench_mixed_fp8),
                      ("llama3-8b-decode-e4m3-cache", bench_fp8_decode),
                      ("long-context-splitk-e4m3-cache", bench_splitk_fp8),
                      ("llama3-8b-spec-verify-q4-bf16", bench_spec_verify),
                      ("rope-write-kv-mixed-step-bf16", bench_rope_write),
                      ("copy-on-write-blocks-bf16", bench_copy_blocks)):
        if only is None or name == only:
            res[name] = leg(k)
    if only is None or only == "block-manager-host":
        res["block-manager-host"] = bench_block_manager()
    return res


def bench_tiny(k: int):
    """The tiny fp32 decode (4 requests, 119 KB of KV: cache-resident, a
    latency figure, not a bandwidth one): write, then decode."""
    import torch
    from workloads import tiny_decode_fp32
    from workloads.tensors import materialize
    lay = tiny_decode_fp32()
    st = materialize(lay, "cuda")
    step = DecodeStep(st, "decode", 0)
    ms, host_us, kern = time_steps([step], max(k, 20), 5, True)
    s = _stats(kern)
    res = {"step_ms": round(ms, 4), "attention_kernel_ms": round(s["mean"], 4),
           "attention_ms_median": round(s["median"], 4), "attention_ms_min": round(s["min"], 4),
           "algorithmic_bytes": decode_bytes(lay),
           "note": "KV resident in the caches; correctness workload, timing for reference",
           "cpu_oracle": oracle_sample(st, lay, list(range(lay.num_seqs)), "decode")}
    del st, step
    torch.cuda.empty_cache()
    print(f"[bench] tiny decode: attention median {s['median']:.4f} ms", file=sys.stderr,
          flush=True)
    return res


def bench_prefill_only(k: int, kv=None):
    """pa_varlen on the mixed step's 4 prefill chunks alone: the compute rate
    of the prefill rows, exact causal FLOPs against the bf16 MFMA peak. With
    ``kv`` (dtype "e4m3" and the two scales) the cache holds E4M3 codes."""
    import torch
    import paged_kv_cache_221_amd as pa
    from workloads import mixed_step_prefill_only
    from workloads.tensors import materialize, materialize_e4m3
    lay = mixed_step_prefill_only()
    if kv is None:
        st = materialize(lay, "cuda", poison=False)
        scales = {}
    else:
        st = materialize_e4m3(lay, "cuda", kv["k_scale"], kv["v_scale"], poison=False)
        scales = dict(k_scale=kv["k_scale"], v_scale=kv["v_scale"])
    out = torch.empty_like(st.q)
    ws = torch.empty(pa.pa_varlen_workspace_bytes(st.k_cache, st.v_cache, lay.num_seqs,
                                                  st.q.shape[0], lay.num_heads,
                                                  st.block_table.shape[1]),
                     dtype=torch.uint8, device="cuda")
    attn = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                        st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale, out=out,
                        workspace=ws, prepared=True, **scales)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        attn()
        if ev is not None:
            ev[1].record()
    _, _, kern = time_steps([step], max(k, 10), 3, True)
    s = _stats(kern)
    flops = causal_flops(lay)
    print(f"[bench] prefill chunks{'' if kv is None else ' (e4m3)'}: median {s['median']:.4f} ms",
          file=sys.stderr, flush=True)
    sample = oracle_sample(st, lay, [0], "varlen", kv=kv)
    del st, out, ws, attn
    torch.cuda.empty_cache()
    tflops = flops / (s["median"] * 1e-3) / 1e12
    return {"kernel_ms": round(s["mean"], 4), "kernel_ms_median": round(s["median"], 4),
            "kernel_ms_min": round(s["min"], 4), "flops": flops, "TFLOPs": round(tflops, 1),
            "frac_of_bf16_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "cpu_oracle": sample}


def bench_prefill_only_fp8(k: int):
    """The mixed step's 4 prefill chunks on an E4M3 cache (bf16 q and
    output): the same FLOPs, with the KV codes widened to bf16 operands."""
    return bench_prefill_only(k, kv=dict(dtype="e4m3", k_scale=0.0625, v_scale=0.0625))


def bench_mixed_fp8(k: int):
    """The whole mixed step (4 prefill chunks, 120 decode rows, the shared
    prefix) on an E4M3 cache, bf16 q and output: write of the step's 2,168
    tokens (quantising), then pa_varlen with a workspace. Algorithmic bytes
    as the bf16 leg's with one byte per cached K/V element."""
    import torch
    import paged_kv_cache_221_amd as pa
    from workloads import mixed_step
    from workloads.tensors import materialize_e4m3
    lay = mixed_step()
    ks = vs = 0.0625
    st = materialize_e4m3(lay, "cuda", ks, vs, poison=False)
    out = torch.empty_like(st.q)
    ws = torch.empty(pa.pa_varlen_workspace_bytes(st.k_cache, st.v_cache, lay.num_seqs,
                                                  st.q.shape[0], lay.num_heads,
                                                  st.block_table.shape[1]),
                     dtype=torch.uint8, device="cuda")
    write = pa.pa_write_kv(st.k_cache, st.v_cache, st.k_new, st.v_new, st.slot_mapping,
                           k_scale=ks, v_scale=vs, prepared=True)
    attn = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                        st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale, out=out,
                        workspace=ws, k_scale=ks, v_scale=vs, prepared=True)

    def step(ev=None):
        write()
        if ev is not None:
            ev[0].record()
        attn()
        if ev is not None:
            ev[1].record()
    ms, _, kern = time_steps([step], max(k, 10), 3, True)
    nbytes = varlen_bytes(lay, kv_elem_bytes=1)
    uniq = nbytes - shared_prefix_bytes(lay, kv_elem_bytes=1)
    med = statistics.median(kern)
    print(f"[bench] mixed step (e4m3): attention median {med:.4f} ms", file=sys.stderr,
          flush=True)
    res = timed_leg(nbytes, kern, ms, {"unique_bytes": uniq,
                                       "attention_unique_GBps": round(uniq / (med * 1e-3) / 1e9,
                                                                      1)})
    dec = [r for r in range(lay.num_seqs) if lay.query_lens[r] == 1]
    res["cpu_oracle"] = oracle_sample(st, lay, [1] + dec[:4], "varlen",
                                      kv=dict(dtype="e4m3", k_scale=ks, v_scale=vs))
    del st, out, ws, write, attn
    torch.cuda.empty_cache()
    return res


def bench_splitk_fp8(k: int):
    """The long-context batch (8 requests of 32k-128k tokens) on an E4M3
    cache: write, then split-K partials and the LSE merge (bf16 q and
    output). Algorithmic bytes as the bf16 leg's with one byte per cached
    K/V element."""
    import torch
    from workloads import long_context_splitk
    from workloads.tensors import materialize_e4m3
    lay = long_context_splitk()
    scales = (0.0625, 0.0625)
    st = materialize_e4m3(lay, "cuda", *scales, poison=False)
    step = DecodeStep(st, "splitk", lay.split_tokens, kv_scales=scales)
    ms, _, kern = time_steps([step], max(k, 10), 3, True)
    nbytes = decode_bytes(lay, kv_elem_bytes=1)
    print(f"[bench] long-context split-K (e4m3): attention median "
          f"{statistics.median(kern):.4f} ms", file=sys.stderr, flush=True)
    res = timed_leg(nbytes, kern, ms, {"includes": "split-K partials and the LSE merge"})
    res["cpu_oracle"] = oracle_sample(st, lay, [0], "decode",
                                      kv=dict(dtype="e4m3", k_scale=scales[0],
                                              v_scale=scales[1]))
    del st, step
    torch.cuda.empty_cache()
    return res


def bench_fp8_decode(k: int, copies: int = 4):
    """The Llama-3-8B decode batch with an E4M3 KV cache (bf16 q and output):
    write, then the balanced decode. Algorithmic bytes: one byte per cached
    K/V element, bf16 q in and out, block-table entries and seq_lens."""
    import torch
    from workloads import llama3_8b_decode
    from workloads.tensors import materialize_e4m3
    lay = llama3_8b_decode()
    scales = (0.0625, 0.0625)
    sts = [materialize_e4m3(lay, "cuda", *scales, poison=False, seed_offset=i)
           for i in range(copies)]
    steps = [DecodeStep(st, "balanced", 0, kv_scales=scales) for st in sts]
    ms, _, kern = time_steps(steps, max(k, 10), 3, True)
    nbytes = decode_bytes(lay, kv_elem_bytes=1)
    print(f"[bench] e4m3 decode: attention median {statistics.median(kern):.4f} ms",
          file=sys.stderr, flush=True)
    res = timed_leg(nbytes, kern, ms, {"decode_tokens_per_s_per_layer":
                                       round(lay.num_seqs / (statistics.median(kern) * 1e-3),
                                             1)})
    res["cpu_oracle"] = oracle_sample(sts[0], lay, [0, 1], "decode",
                                      kv=dict(dtype="e4m3", k_scale=scales[0],
                                              v_scale=scales[1]))
    del sts, steps
    torch.cuda.empty_cache()
    return res


def bench_spec_verify(k: int, copies: int = 4):
    """The Llama-3-8B decode batch (same lengths and KV bytes) with every
    request verifying 4 tokens at once, as speculative decoding does: the
    step writes the 256 new tokens' K/V, then pa_varlen with a workspace (GQA
    group 4 x 4 tokens = one 16-row tile, the balanced kernel). Input copies
    rotate as in the decode bench. Algorithmic bytes: per-request KV, q and
    out, tables; FLOPs: exact causal pairs."""
    import torch
    import paged_kv_cache_221_amd as pa
    from workloads import llama3_8b_spec_verify
    from workloads.tensors import materialize
    lay = llama3_8b_spec_verify()
    sts = [materialize(lay, "cuda", poison=False, seed_offset=i) for i in range(copies)]
    ws = torch.zeros(pa.pa_varlen_workspace_bytes(sts[0].k_cache, sts[0].v_cache, lay.num_seqs,
                                                  sts[0].q.shape[0], lay.num_heads,
                                                  sts[0].block_table.shape[1]),
                     dtype=torch.uint8, device="cuda")

    def make(st):
        out = torch.empty_like(st.q)
        write = pa.pa_write_kv(st.k_cache, st.v_cache, st.k_new, st.v_new, st.slot_mapping,
                               prepared=True)
        attn = pa.pa_varlen(st.k_cache, st.v_cache, st.q, st.cu_seqlens_q, st.seq_lens,
                            st.block_table, lay.max_query_len, lay.max_seq_len, lay.scale,
                            out=out, workspace=ws, prepared=True)

        def step(ev=None):
            write()
            if ev is not None:
                ev[0].record()
            attn()
            if ev is not None:
                ev[1].record()
        return step
    ms, _, kern = time_steps([make(st) for st in sts], max(k, 10), 3, True)
    nbytes, flops = varlen_bytes(lay), causal_flops(lay)
    tokens = int(lay.query_lens.sum())
    med = statistics.median(kern)
    print(f"[bench] spec verify q4: attention median {med:.4f} ms", file=sys.stderr, flush=True)
    res = timed_leg(nbytes, kern, ms, {
        "query_len": 4, "flops": flops, "TFLOPs": round(flops / (med * 1e-3) / 1e12, 1),
        "verified_tokens_per_s_per_layer": round(tokens / (med * 1e-3), 1)})
    res["cpu_oracle"] = oracle_sample(sts[0], lay, [0, 1], "varlen")
    del sts, ws
    torch.cuda.empty_cache()
    return res


def bench_rope_write(k: int):
    """pa_rope_write_kv on the mixed step's 2,168 new tokens (32 query / 8 KV
    heads, head_dim 128, bf16, full rotary_dim, NeoX pairs). Algorithmic
    bytes: q read and written, new K and V read and written to the cache,
    positions, slots and each token's cos/sin row read."""
    import torch
    import paged_kv_cache_221_amd as pa
    from workloads import mixed_step
    from workloads.tensors import materialize
    lay = mixed_step()
    st = materialize(lay, "cuda", poison=False)
    t = st.q.shape[0]
    maxpos = int(lay.max_seq_len)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    ang = torch.rand((maxpos, 64), generator=gen, device="cuda") * 100
    cos_sin = torch.cat([ang.cos(), ang.sin()], dim=1).contiguous()
    positions = (torch.arange(t, device="cuda", dtype=torch.int32) % maxpos).contiguous()
    # 12 copies of the new tokens' q, K and V (~320 MB) rotate, so no call
    # finds its inputs in the 256 MB last-level cache; one pair of events
    # around a run of calls, as a single ~10 us call would be mostly event
    # overhead
    calls = [pa.pa_rope_write_kv(st.k_cache, st.v_cache, st.q.clone(), st.k_new.clone(),
                                 st.v_new.clone(), st.slot_mapping, positions, cos_sin, 128,
                                 True, prepared=True) for _ in range(12)]
    for c in calls:
        c()
    torch.cuda.synchronize()
    n = 4 * len(calls)
    runs = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            calls[i % len(calls)]()
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / n)
    s = _stats(runs)
    e = 2
    nbytes = t * (2 * lay.num_heads * lay.head_dim * e + 4 * lay.num_kv_heads * lay.head_dim * e
                  + 4 + 8 + 128 * 4)
    print(f"[bench] rope + write: {s['median']:.4f} ms", file=sys.stderr, flush=True)
    del st, calls
    torch.cuda.empty_cache()
    cp = _device_copy_ms(nbytes)
    return {"tokens": t, "kernel_ms": round(s["mean"], 4),
            "device_copy_ms": round(cp, 4),
            "frac_of_device_copy": round(cp / s["median"], 4),
            "kernel_ms_median": round(s["median"], 4), "kernel_ms_min": round(s["min"], 4),
            "GBps": round(nbytes / (s["median"] * 1e-3) / 1e9, 1),
            "frac_of_8TBps": round(nbytes / (s["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes,
            "timing": "5 runs of 48 back-to-back calls, one pair of events per run"}


def _device_copy_ms(nbytes: int) -> float:
    """Median time (ms) of torch's device-to-device copy of ``nbytes / 2``
    bytes (so ``nbytes`` of read plus write traffic, like the legs it sits
    beside), rotating over copies that together exceed the 256 MB last-level
    cache: the rate a plain copy of the same traffic reaches on this GPU."""
    import torch
    half = max(16, (nbytes // 2) // 16 * 16)
    n = max(2, (1200 << 20) // (2 * half))
    srcs = [torch.empty(half, dtype=torch.uint8, device="cuda").random_() for _ in range(n)]
    dsts = [torch.empty_like(x) for x in srcs]
    for i in range(n):
        dsts[i].copy_(srcs[i])
    torch.cuda.synchronize()
    runs, calls = [], 4 * n
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            dsts[i % n].copy_(srcs[i % n])
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / calls)
    del srcs, dsts
    torch.cuda.empty_cache()
    return statistics.median(runs)


def bench_copy_blocks(k: int, pairs: int = 4096):
    """pa_copy_blocks on Llama-3-8B-shaped blocks (16 tokens x 8 KV heads x 128,
    bf16: 32 KB per block per cache): `pairs` disjoint (source, destination)
    pairs, as a batch of copy-on-write forks would queue. Algorithmic bytes:
    every pair reads and writes one K and one V block."""
    import torch
    import paged_kv_cache_221_amd as pa
    nb = 2 * pairs
    kc = torch.zeros((nb, 16, 8, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    perm = torch.randperm(nb, generator=gen, device="cuda").to(torch.int32)
    src_dst = torch.stack([perm[:pairs], perm[pairs:]], dim=1).contiguous()
    copy = pa.pa_copy_blocks(kc, vc, src_dst, prepared=True)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        copy()
        if ev is not None:
            ev[1].record()
    _, _, kern = time_steps([step], max(k, 10), 3, True)
    s = _stats(kern)
    nbytes = pairs * 2 * kc[0].numel() * 2 * 2
    print(f"[bench] copy-on-write blocks: median {s['median']:.4f} ms", file=sys.stderr,
          flush=True)
    del kc, vc, copy
    torch.cuda.empty_cache()
    cp = _device_copy_ms(nbytes)
    return {"pairs": pairs, "kernel_ms": round(s["mean"], 4),
            "device_copy_ms": round(cp, 4),
            "frac_of_device_copy": round(cp / s["median"], 4),
            "kernel_ms_median": round(s["median"], 4), "kernel_ms_min": round(s["min"], 4),
            "GBps": round(nbytes / (s["median"] * 1e-3) / 1e9, 1),
            "frac_of_8TBps": round(nbytes / (s["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes}


def bench_block_manager(steps: int = 2000):
    """Host block-manager cost of one decode step of the Llama-3-8B batch (64
    sequences of the bench lengths, pool of its size): every sequence appends
    one token in one batched call, every 16th sequence also forks and frees a
    candidate (copy-on-write), the queued copies are taken and the step's
    block table is filled. Called through the Python binding, so ctypes
    overhead is included."""
    import numpy as np
    import paged_kv_cache_221_amd as pa
    from workloads import llama3_8b_decode
    lay = llama3_8b_decode()
    bm = pa.BlockManager(lay.num_blocks, lay.block_size)
    for r in range(lay.num_seqs):
        bm.append(r, int(lay.seq_lens[r]) - 1)
    seqs = np.arange(lay.num_seqs, dtype=np.int64)
    ones = np.ones(lay.num_seqs, dtype=np.int64)
    width = int(lay.block_table.shape[1]) + 64
    per = []
    for it in range(steps):
        t0 = time.perf_counter()
        bm.append_batch(seqs, ones)
        for r in range(it % 16, lay.num_seqs, 16):   # 4 candidates fork, write, end
            bm.fork(r, 1000 + r)
            bm.append(1000 + r, 1)
            bm.free(1000 + r)
        bm.take_copies()
        bm.block_tables(seqs, width)
        per.append(time.perf_counter() - t0)
        if it % 64 == 63:   # untimed: bring the batch back to its lengths
            for r in range(lay.num_seqs):
                bm.free(r)
                bm.append(r, int(lay.seq_lens[r]) - 1)
    bm.close()
    s = _stats(per)
    return {"sequences": lay.num_seqs, "us_per_step": round(s["mean"] * 1e6, 2),
            "us_median": round(s["median"] * 1e6, 2), "us_min": round(s["min"] * 1e6, 2),
            "note": "one batched append of 64 sequences, 4 fork/append/free, the copy "
                    "queue and the [64, width] block table per step, via ctypes"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--path", choices=["decode", "balanced", "fused", "splitk"],
                    default="fused")
    ap.add_argument("--split-tokens", type=int, default=512)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--only", choices=SECONDARY_LEGS, default=None,
                    help="run only this secondary workload and print its line (for profiling)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run torch's elementwise negation over this many MiB of "
                         "fp32 (3 times): a kernel that reads and writes a known number of "
                         "bytes, for scaling HBM counter readings")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from paged_kv_cache_221_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    import paged_kv_cache_221_amd as pa
    from workloads import llama3_8b_decode
    from workloads.tensors import materialize
    pa.load()
    torch.cuda.set_device(0)

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.only is not None:
        print(json.dumps({"secondary": secondary(args, args.only)}), flush=True)
        return

    layout = llama3_8b_decode()
    copies = [materialize(layout, "cuda", seed_offset=i) for i in range(args.copies)]
    steps = [DecodeStep(st, args.path, args.split_tokens) for st in copies]
    print(f"[bench] {layout.name}: {layout.num_seqs} requests, "
          f"{int(layout.seq_lens.sum())} KV tokens, path={args.path}", file=sys.stderr,
          flush=True)

    # step time without per-kernel events (recording them costs a few us per
    # step), then a second pass with events around the attention call
    eager_ms, host_us, _ = time_steps(steps, args.steps, args.warmup, False)
    _, _, kern = time_steps(steps, args.steps, args.warmup, True)
    kstat = _stats(kern)
    # The step time is the eager one: back-to-back launches on one stream.
    # A HIP-graph replay of the same steps is reported beside it.
    graph_ms = None if args.no_graph else time_graph(steps, args.steps, args.warmup)
    step_ms = eager_ms
    print(f"[bench] step {step_ms * 1e3:.1f} us eager, attention call median "
          f"{kstat['median'] * 1e3:.1f} us", file=sys.stderr, flush=True)

    dec_b, wr_b = decode_bytes(layout), write_bytes(layout)
    step_bytes = dec_b + wr_b
    value = step_bytes / (step_ms * 1e-3) / 1e9
    # the timed launch moves the attention's bytes, and the write's when fused
    launch_b = step_bytes if args.path == "fused" else dec_b
    achieved = launch_b / (kstat["mean"] * 1e-3) / 1e9
    src_hash = kernel_source_hash()
    traffic = load_traffic(src_hash, args.path)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, generated on the GPU; no weights)",
        "config": {"workload": layout.name, "num_seqs": layout.num_seqs,
                   "seq_len_range": [512, 4096], "total_kv_tokens": int(layout.seq_lens.sum()),
                   "num_heads": layout.num_heads, "num_kv_heads": layout.num_kv_heads,
                   "head_dim": layout.head_dim, "block_size": layout.block_size,
                   "num_blocks": layout.num_blocks, "path": args.path,
                   "split_tokens": args.split_tokens if args.path == "splitk" else None,
                   "input_copies": args.copies,
                   "timing": "eager, back-to-back launches of prepared calls"},
        "hbm_frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "decode_tokens_per_s_per_layer": round(layout.num_seqs / (step_ms * 1e-3), 1),
        "graph_ms_per_step": round(graph_ms, 5) if graph_ms is not None else None,
        "host_launch_us_per_step": round(host_us, 2),
        "step_algorithmic_bytes": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "kernel": PATH_KERNELS[args.path],
                     "kernel_ms": round(kstat["mean"], 5),
                     "kernel_ms_median": round(kstat["median"], 5),
                     "kernel_ms_min": round(kstat["min"], 5),
                     "algorithmic_bytes_per_launch": launch_b,
                     "kernel_source_hash": src_hash},
    }
    if not args.no_ceiling:
        line["read_ceiling"] = read_ceiling(copies, layout, args.steps)
    cpu = None if args.no_cpu_baseline else cpu_baseline(copies[0], layout, args.cpu_budget)
    # the secondary legs run in child processes on a GPU this process no
    # longer holds memory on
    del copies, steps
    torch.cuda.empty_cache()
    if not args.no_secondary:
        line["secondary"] = secondary_isolated(args)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
