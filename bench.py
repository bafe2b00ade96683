#!/usr/bin/env python3
"""Benchmark of the mixed-batch quantized-KV attention step on one MI355X.

A step is one pass of the whole hot path over the workload's batch:
kv_append_quant of the step's new K/V rows, then mixed_attention_fwd over the
paged cache (every layer, for the multi-layer workload).  Inputs are resident
in HBM before timing; the cached prefix is written beforehand by the same
append kernel.  To keep the Infinity Cache from serving repeated reads of a
working set near its 256 MB size, the timed steps rotate over several
identical copies of the pools (enough copies to exceed 1 GiB).

Prints one JSON line.  ``value`` is the effective KV bandwidth of the step:
the bytes of every visible cached position (prefix and new rows, K and V, in
their block format) read once per KV head, divided by the step time.  The
attention launches are timed separately with HIP events on the stream they
run on, for the roofline figure.  The oracle is timed on the host on a bounded
sample of the same workload for the cpu_baseline figure.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mixed-batch quantized-KV attention: effective KV GB/s and query tok/s per step"
HBM_PEAK_GBS = 8000.0
CLOCK_WARMUP_S = 0.5  # matrix-core work before the warm-up steps (not timed)
MFMA_F16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    "decode16": "16 decode rows, 24 q heads / 4 KV heads, head_dim 128, q8 34-byte blocks, "
                "page 256, contexts uniform in [1024, 32768], 2% K outlier channels x20, 1 layer",
    "mixed16_chunk2k": "16 decode rows (contexts uniform in [2048, 65536]) + one 2048-row chunk at "
                       "position 131072, 24/4 heads, head_dim 128, q8, page 256, K outliers, 1 layer",
    "decode16_f16": "the decode16 batch (16 decode rows, contexts uniform in [1024, 32768], 24/4 heads, "
                    "head_dim 128, page 256) over an unquantized f16 cache (64-byte blocks), 1 layer",
    "verify16": "16 verify rows of 4 tokens each (contexts of the last token uniform in [1024, 32768]), "
                "24/4 heads, head_dim 128, q8 34-byte blocks, page 256, 2% K outlier channels x20, 1 layer",
    "long_q8": "one decode row at context 262144, 24/4 heads, head_dim 128, q8, page 256, 1 layer",
    "long_k4v4": "one decode row at context 262144, 24/4 heads, head_dim 128, K4V4 18-byte blocks, "
                 "page 256, 1 layer",
    "step_k4v4": "12 attention layers, each: 16 decode rows (contexts log-uniform in [512, 262144]) + "
                 "a 2048-row chunk at 131072, 24/4 heads, head_dim 128, K4V4, page 256, K outliers",
}
SEEDS = {"decode16": 2, "decode16_f16": 2, "verify16": 6, "mixed16_chunk2k": 3, "long_q8": 4, "long_k4v4": 4,
         "step_k4v4": 5}


POISON = 0x7E  # bytes of pool space no append has written (fp16 NaN scales)


class DeviceCase:
    """One layer's device state: pools written by kv_append_quant (the cached
    prefix first, then the step's rows at their own positions), the batch
    descriptor, the step's inputs, an output buffer and the workspace.
    ``flags``: the attention batch's flags (0, or MAB_BATCH_INVARIANT)."""

    def __init__(self, case, flags=0):
        import torch
        import mixed_attention_block_amd as mab

        lay = case.layout
        self.case = case
        self.layout = mab.make_layout(lay["num_q_heads"], lay["num_kv_heads"], lay["head_dim"],
                                      lay["page_size"], lay["num_pages"], lay["k_format"], lay["v_format"])
        self.k_pool = torch.full((mab.kv_pool_bytes(self.layout, lay["k_format"]),), POISON,
                                 dtype=torch.uint8, device="cuda")
        self.v_pool = torch.full((mab.kv_pool_bytes(self.layout, lay["v_format"]),), POISON,
                                 dtype=torch.uint8, device="cuda")
        self.batch = self._batch(case.q_start, case.prefix_len, case.block_table, flags)
        # the cached prefix: one append over every sequence that has one
        keep = [s for s in range(case.num_seqs) if case.prefix_len[s] > 0]
        if keep:
            rows = case.prefix_len[keep].astype(np.int64)
            fill = self._batch(np.concatenate([[0], np.cumsum(rows)]), np.zeros(len(keep)),
                               case.block_table[keep])
            k = torch.cat([case.k_prefix[s] for s in keep]).cuda().contiguous()
            v = torch.cat([case.v_prefix[s] for s in keep]).cuda().contiguous()
            mab.kv_append_quant(self.layout, fill, k, v, self.k_pool, self.v_pool)
            del k, v
        self.q = case.q.cuda().contiguous()
        self.k_new = case.k_new.cuda().contiguous()
        self.v_new = case.v_new.cuda().contiguous()
        mab.kv_append_quant(self.layout, self.batch, self.k_new, self.v_new, self.k_pool, self.v_pool)
        self.out = torch.empty((case.num_rows, lay["num_q_heads"], lay["head_dim"]), dtype=torch.float32,
                               device="cuda")
        n = mab.attention_workspace_bytes(self.layout, self.batch)
        self.ws = torch.empty((max(n, 256),), dtype=torch.uint8, device="cuda")

    @staticmethod
    def _batch(q_start, prefix_len, block_table, flags=0):
        import torch
        import mixed_attention_block_amd as mab

        qs = np.ascontiguousarray(q_start, dtype=np.int32)
        pl = np.ascontiguousarray(prefix_len, dtype=np.int32)
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        return mab.BatchDesc(torch.from_numpy(qs).cuda(), torch.from_numpy(pl).cuda(),
                             torch.from_numpy(bt).cuda(), qs, pl, flags=flags)


def realism_probes(stream):
    """What this device reaches on plain work: a 4 GiB stream read (GB/s) and
    dense 16x16x32 fp16 matrix-core products (TFLOP/s), each the best of
    five runs timed with events on the benchmark's stream."""
    import torch
    import mixed_attention_block_amd as mab

    buf = torch.empty((4 << 30,), dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_rd = best_mf = 0.0
    mab.mab_probe_stream_read(buf, sink, stream)  # warm-up
    mab.mab_probe_mfma_f16(2000, sink, stream)
    for _ in range(5):
        e0.record(stream)
        n = mab.mab_probe_stream_read(buf, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        best_rd = max(best_rd, n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        e0.record(stream)
        f = mab.mab_probe_mfma_f16(20000, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        best_mf = max(best_mf, f / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    del buf
    return {"stream_read_gbs": round(best_rd, 1), "stream_read_bytes": 4 << 30,
            "mfma_f16_tflops": round(best_mf, 1),
            "note": "mab_probe_stream_read (16-byte non-temporal loads over 4 GiB) and "
                    "mab_probe_mfma_f16 (independent 16x16x32 fp16 products, 2 waves per SIMD), "
                    "best of 5"}


def kv_bytes_per_position(layout):
    from mixed_attention_block_amd import kv_block_bytes
    nb = layout["head_dim"] // 32
    return layout["num_kv_heads"] * nb * (kv_block_bytes(layout["k_format"]) +
                                          kv_block_bytes(layout["v_format"]))


def chunk_flops(case):
    """QK^T and PV flops of the prefill-chunk rows (sequences of more than 16
    rows, the ones on the matrix-core tiles) over their visible keys (unmasked
    pairs)."""
    lay = case.layout
    f = 0
    for s in range(case.num_seqs):
        n = case.q_len(s)
        if n > 16:
            p = int(case.prefix_len[s])
            f += 4 * lay["head_dim"] * lay["num_q_heads"] * (n * (p + 1) + n * (n - 1) // 2)
    return f


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None where it is not readable."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def chunk_only_launch(st, stream, n):
    """The first layer's prefill chunks alone (its sequences of more than 16
    rows, no decode rows) in one mixed_attention_fwd_timed call, n times: the
    attention kernel's average duration and its fraction of the fp16 peak."""
    import torch
    import mixed_attention_block_amd as mab

    case = st.case
    seqs = [s for s in range(case.num_seqs) if case.q_len(s) > 16]
    lens = np.array([case.q_len(s) for s in seqs], np.int64)
    qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    batch = DeviceCase._batch(qs, case.prefix_len[seqs], case.block_table[seqs])
    q = torch.cat([st.q[case.q_start[s]:case.q_start[s + 1]] for s in seqs]).contiguous()
    out = torch.empty((int(qs[-1]),) + tuple(st.out.shape[1:]), dtype=torch.float32, device="cuda")
    ws = torch.empty((max(mab.attention_workspace_bytes(st.layout, batch), 256),), dtype=torch.uint8,
                     device="cuda")
    flops = chunk_flops(case)  # counts exactly these sequences
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n + 2)]
    for e0, e1 in evs:
        mab.mixed_attention_fwd_timed(st.layout, batch, q, st.k_pool, st.v_pool, case.sm_scale, out, ws, e0, e1,
                                      stream)
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs[2:]]))
    tf = flops / (ms * 1e-3) / 1e12
    return {"kernel_ms_avg": round(ms, 6), "algorithmic_flops_per_launch": int(flops),
            "achieved": round(tf, 2), "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "note": "the first layer's prefill chunk alone (no decode rows), attention kernel only"}


def clock_warmup(stream, seconds=0.5):
    """Keeps the matrix cores busy for about `seconds` before a sweep's first
    point, so that the first points are not timed while the clock ramps up."""
    import torch
    import mixed_attention_block_amd as mab

    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    t = time.time()
    while time.time() - t < seconds:
        mab.mab_probe_mfma_f16(20000, sink, stream)
        torch.cuda.synchronize()


def decode_sweep(n=30):
    """Decode-only batches of growing size: 16 and 64 rows with decode16's
    heads (24/4, head_dim 128, page 256) and contexts uniform in
    [1024*m, 32768*m] (capped at 262144) for m = 1, 2, 4, 8, over q8, K4V4,
    K8V4 and K4V8 pools.  Per point: the attention kernel's average duration over n timed
    calls (the library's event pair around its launch), the whole call's
    (back-to-back calls), and the KV bytes each moves per launch.  One JSON
    line per point, then a fit of kernel time = fixed + bytes / rate."""
    import torch
    import mixed_attention_block_amd as mab
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    clock_warmup(stream)
    pts = []
    for kf, vf in (("q8", "q8"), ("q4", "q4"), ("q8", "q4"), ("q4", "q8")):
        for rows in (16, 64):
            for m in (1, 2, 4, 8):
                rng = np.random.Generator(np.random.PCG64(1000 * rows + m))
                ctx = np.minimum(rng.integers(1024 * m, 32768 * m, size=rows, endpoint=True), 262144)
                case = synth.make_case("decode16", 2, device="cuda", seqs=[(int(c) - 1, 1) for c in ctx],
                                       kf=kf, vf=vf, outliers=0.02)
                st = DeviceCase(case)
                case.k_prefix = case.v_prefix = None
                kv = int(ctx.sum()) * kv_bytes_per_position(case.layout)
                # identical pool copies rotated, as in the timed steps, so that
                # repeated calls do not find a small batch in the Infinity Cache
                copies = max(1, min(16, math.ceil((1 << 30) / (st.k_pool.numel() + st.v_pool.numel()))))
                pools = [(st.k_pool, st.v_pool)] + [(st.k_pool.clone(), st.v_pool.clone())
                                                    for _ in range(copies - 1)]
                call = lambda i: mab.mixed_attention_fwd(st.layout, st.batch, st.q, *pools[i % copies],
                                                         case.sm_scale, st.out, st.ws, stream)
                clock_warmup(stream, 0.25)  # the set-up above left the device idle
                for i in range(3):
                    call(i)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(n):
                    call(i)
                e1.record(stream)
                kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(n)]
                for i, (a, b) in enumerate(kev):
                    mab.mixed_attention_fwd_timed(st.layout, st.batch, st.q, *pools[i % copies], case.sm_scale,
                                                  st.out, st.ws, a, b, stream)
                torch.cuda.synchronize()
                call_us = e0.elapsed_time(e1) / n * 1e3
                kern_us = float(np.mean([a.elapsed_time(b) for a, b in kev])) * 1e3
                pt = {"format": f"K{kf}/V{vf}", "rows": rows, "ctx_scale": m, "kv_bytes": kv, "pool_copies": copies,
                      "kernel_us": round(kern_us, 2), "call_us": round(call_us, 2),
                      "kernel_tbs": round(kv / kern_us / 1e6, 3),
                      "kernel_frac": round(kv / kern_us / 1e6 / (HBM_PEAK_GBS / 1e3), 4),
                      "call_frac": round(kv / call_us / 1e6 / (HBM_PEAK_GBS / 1e3), 4)}
                print(json.dumps(pt), flush=True)
                pts.append(pt)
                del st, case, pools, call
                torch.cuda.empty_cache()
    for fmt in ("Kq8/Vq8", "Kq4/Vq4", "Kq8/Vq4", "Kq4/Vq8"):
        p = [q for q in pts if q["format"] == fmt]
        x = np.array([q["kv_bytes"] for q in p], np.float64)
        y = np.array([q["kernel_us"] for q in p], np.float64)
        slope, icpt = np.polyfit(x, y, 1)
        print(json.dumps({"format": fmt, "fit": "kernel_us = fixed_us + kv_bytes / rate",
                          "fixed_us": round(float(icpt), 2), "rate_tbs": round(1 / float(slope) / 1e6, 3)}),
              flush=True)


def chunk_sweep(n=10):
    """Prefill-chunk-only batches: one sequence of C new rows after a cached
    prefix of P tokens (C = 512, 2048, 4096; P = 8192, 32768, 131072) with
    24/4 heads, head_dim 128, page 256, K outliers, over q8, K4V4, K8V4 and
    K4V8 pools.
    Per point: the attention kernel's average duration over n timed calls and
    its fraction of the 2.5 PFLOP/s fp16 peak over the chunk's visible
    (row, key) pairs, and the whole call's.  One JSON line per point."""
    import torch
    import mixed_attention_block_amd as mab
    import synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    clock_warmup(stream)
    for kf, vf in (("q8", "q8"), ("q4", "q4"), ("q8", "q4"), ("q4", "q8")):
        for prefix in (8192, 32768, 131072):
            for rows in (512, 2048, 4096):
                case = synth.make_case("mixed16_chunk2k", 3, device="cuda", seqs=[(prefix, rows)], kf=kf, vf=vf)
                st = DeviceCase(case)
                case.k_prefix = case.v_prefix = None
                flops = chunk_flops(case)
                call = lambda: mab.mixed_attention_fwd(st.layout, st.batch, st.q, st.k_pool, st.v_pool,
                                                       case.sm_scale, st.out, st.ws, stream)
                clock_warmup(stream, 0.25)  # the set-up above left the device idle
                for _ in range(2):
                    call()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(n):
                    call()
                e1.record(stream)
                kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(n)]
                for a, b in kev:
                    mab.mixed_attention_fwd_timed(st.layout, st.batch, st.q, st.k_pool, st.v_pool, case.sm_scale,
                                                  st.out, st.ws, a, b, stream)
                torch.cuda.synchronize()
                call_ms = e0.elapsed_time(e1) / n
                kern_ms = float(np.mean([a.elapsed_time(b) for a, b in kev]))
                tf = flops / (kern_ms * 1e-3) / 1e12
                print(json.dumps({"format": f"K{kf}/V{vf}", "prefix": prefix, "rows": rows, "flops": int(flops),
                                  "kernel_ms": round(kern_ms, 4), "call_ms": round(call_ms, 4),
                                  "kernel_tflops": round(tf, 1),
                                  "kernel_frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                                  "call_frac": round(flops / (call_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)}),
                      flush=True)
                del st, case, call
                torch.cuda.empty_cache()


def cpu_baseline(case, budget_s=12.0, cap_s=30.0):
    """The oracle on whole sequences of the case, shortest first, until the
    budget is spent.  A sequence whose predicted time (from the rate so far per
    row-key pair and per key) would take the total past cap_s is not started
    whole: its first rows are run instead, as many as the budget left allows
    (at least one), and its KV bytes are counted in proportion to them."""
    import torch
    from threadpoolctl import threadpool_info

    from oracle import attention as oattn
    from oracle import cache as ocache

    lay = case.layout
    bpp = kv_bytes_per_position(lay)
    kp = ocache.new_pool(lay, lay["k_format"])
    vp = ocache.new_pool(lay, lay["v_format"])
    order = sorted(range(case.num_seqs), key=lambda s: case.context(s))  # short first
    done, nbytes, rows, elapsed, work = [], 0.0, 0, 0.0, 0.0
    part = None  # (sequence, rows run of its rows) of a sequence run in part
    flops = 0
    for s in order:
        r0, r1 = int(case.q_start[s]), int(case.q_start[s + 1])
        ctx = float(case.context(s))
        w = (r1 - r0 + 1) * ctx  # attention pairs plus the keys encoded
        if done and elapsed + elapsed / work * w > cap_s:
            rate = elapsed / work
            n_rows = int(max(1, min(r1 - r0, (budget_s - elapsed) / (rate * ctx) - 1)))
            if n_rows >= r1 - r0:
                break
            part = (s, n_rows)
            r1 = r0 + n_rows
            w = (n_rows + 1) * ctx
        work += w
        k = torch.cat([case.k_prefix[s].cpu(), case.k_new[int(case.q_start[s]):int(case.q_start[s + 1])].cpu()]).numpy()
        v = torch.cat([case.v_prefix[s].cpu(), case.v_new[int(case.q_start[s]):int(case.q_start[s + 1])].cpu()]).numpy()
        q = case.q.cpu().numpy()
        t0 = time.perf_counter()
        pos = np.arange(case.context(s))
        ocache.write_tokens(kp, lay, lay["k_format"], case.block_table[s], pos, k)
        ocache.write_tokens(vp, lay, lay["v_format"], case.block_table[s], pos, v)
        oattn.attention(q, kp, vp, lay, case.q_start, case.prefix_len, case.block_table,
                        case.sm_scale, rows=list(range(r0, r1)))
        elapsed += time.perf_counter() - t0
        if part is not None:  # more rows of the same sequence (its keys are encoded) while the budget lasts
            end = int(case.q_start[s + 1])
            while r1 < end and elapsed < budget_s:
                t1 = time.perf_counter()
                oattn.attention(q, kp, vp, lay, case.q_start, case.prefix_len, case.block_table,
                                case.sm_scale, rows=[r1])
                dt = time.perf_counter() - t1
                elapsed += dt
                r1 += 1
                n_more = int(min(end - r1, (budget_s - elapsed) / dt))
                if n_more > 0:
                    t1 = time.perf_counter()
                    oattn.attention(q, kp, vp, lay, case.q_start, case.prefix_len, case.block_table,
                                    case.sm_scale, rows=list(range(r1, r1 + n_more)))
                    elapsed += time.perf_counter() - t1
                    r1 += n_more
            part = (s, r1 - r0) if r1 < end else None  # all its rows ran: a whole sequence
            if part is None:
                done.append(s)
                nbytes += ctx * bpp
                rows += r1 - r0
                if int(case.q_start[s + 1]) - int(case.q_start[s]) > 16:
                    p = int(case.prefix_len[s])
                    flops += sum(4 * lay["head_dim"] * lay["num_q_heads"] * (p + 1 + i) for i in range(r1 - r0))
                break
        done.append(s)
        n_seq = int(case.q_start[s + 1]) - int(case.q_start[s])
        nbytes += ctx * bpp * (r1 - r0) / n_seq
        rows += r1 - r0
        if n_seq > 16:  # a prefill chunk: its QK^T and PV flops over the visible keys of the rows run
            p = int(case.prefix_len[s])
            flops += sum(4 * lay["head_dim"] * lay["num_q_heads"] * (p + 1 + i) for i in range(r1 - r0))
        if part is not None or elapsed >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    whole = len(done) - (1 if part else 0)
    sample = (f"{whole} of {case.num_seqs} sequences of this workload whole (shortest first)"
              + (f" and the first {part[1]} of the {int(case.q_start[part[0] + 1] - case.q_start[part[0]])} rows "
                 f"of the next" if part else "")
              + f"; {rows} rows, {nbytes / 1e6:.1f} MB of KV: encode + fp64 attention, {elapsed:.1f} s")
    out = {"value": round(nbytes / elapsed / 1e9, 6), "unit": "GB/s", "cores": int(threads),
           "cpu_model": cpu_model(), "kind": "oracle", "sample": sample,
           "query_tok_s": round(rows / elapsed, 3)}
    if flops:
        out["chunk_gflops"] = round(flops / elapsed / 1e9, 3)
    return out


# ---- HBM traffic from hardware counters ---------------------------------------
# Two rocprofv3 --pmc runs of this script per workload (FETCH_SIZE, then
# WRITE_SIZE, KiB per dispatch) and two of its --copy-probe mode (an
# elementwise kernel reading and writing COPY_PROBE_BYTES) give the counters;
# --ingest-pmc scales each kernel's average by what the counter reads for the
# probe and stores the result in profiles/traffic_<workload>.json together with
# a digest of the kernel source, so that a later change of the kernels turns
# the stored figure off (traffic null).

COPY_PROBE_BYTES = 512 << 20
LIB_KERNELS = ("mixed_attention_kernel", "decode_attention_kernel", "chunk_combine_kernel",
               "combine_kernel", "plan_kernel", "append_kernel")


def source_digest():
    import hashlib
    with open(os.path.join(ROOT, "mixed_attention_block_amd", "csrc", "mab.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def stored_traffic(name):
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    return d if d.get("source_digest") == source_digest() else None


def copy_probe():
    """An elementwise kernel that reads and writes COPY_PROBE_BYTES each (the
    calibration dispatches of the counter runs)."""
    import torch
    n = COPY_PROBE_BYTES // 4
    src = torch.randn((n,), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": COPY_PROBE_BYTES, "dispatches": 5}))


def _pmc_rows(d):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def _lib_kernel(name):
    for k in LIB_KERNELS:
        if k in name:
            return k
    return None


def ingest_pmc(workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir):
    def probe_avg(d, counter):
        vals = [float(r["Counter_Value"]) for r in _pmc_rows(d)
                if r["Counter_Name"] == counter and "neg" in r["Kernel_Name"].lower()]
        if not vals:
            raise SystemExit(f"no copy-probe dispatch in {d}")
        return sum(vals) / len(vals)

    def per_kernel(d, counter):
        acc = {}
        for r in _pmc_rows(d):
            k = _lib_kernel(r["Kernel_Name"])
            if k and r["Counter_Name"] == counter:
                acc.setdefault(k, []).append(float(r["Counter_Value"]))
        return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}

    scale_f = COPY_PROBE_BYTES / (probe_avg(copy_fetch_dir, "FETCH_SIZE") * 1024)
    scale_w = COPY_PROBE_BYTES / (probe_avg(copy_write_dir, "WRITE_SIZE") * 1024)
    fk, wk = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fk) | set(wk)):
        f_kib, n = fk.get(k, (0.0, 0))
        w_kib, _ = wk.get(k, (0.0, 0))
        kernels[k] = {"dispatches": n, "fetch_kib_avg": round(f_kib, 1), "write_kib_avg": round(w_kib, 1),
                      "bytes": int(f_kib * 1024 * scale_f + w_kib * 1024 * scale_w)}
    call = [k for k in kernels if k not in ("append_kernel",)]
    out = {"workload": workload, "source_digest": source_digest(),
           "copy_probe_bytes": COPY_PROBE_BYTES,
           "scale_fetch": round(scale_f, 4), "scale_write": round(scale_w, 4),
           "kernels": kernels,
           "bytes_per_call": int(sum(kernels[k]["bytes"] for k in call)),
           "note": "bytes = FETCH_SIZE*1024*scale_fetch + WRITE_SIZE*1024*scale_write per dispatch; "
                   "bytes_per_call sums the kernels of one mixed_attention_fwd call"}
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def main():
    if "--copy-probe" in sys.argv:
        copy_probe()
        return
    if "--decode-sweep" in sys.argv:
        decode_sweep()
        return
    if "--chunk-sweep" in sys.argv:
        chunk_sweep()
        return
    if "--ingest-pmc" in sys.argv:
        ap = argparse.ArgumentParser()
        ap.add_argument("--ingest-pmc", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                          "COPY_WRITE_DIR"))
        ap.add_argument("--workload", required=True, choices=sorted(WORKLOADS))
        args = ap.parse_args()
        ingest_pmc(args.workload, *args.ingest_pmc)
        return
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="step_k4v4", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=0, help="pool copies rotated (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--batch-invariant", action="store_true",
                    help="attention batches with MAB_BATCH_INVARIANT (decode rows cut from their own first key)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; runs on more than one GPU are not supported (the path "
              "shards by KV head, sequence or key range without kernel changes).", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixed_attention_block_amd as mab
    import synth

    torch.cuda.set_device(0)
    name = args.workload
    layers = 12 if name == "step_k4v4" else 1
    seed = SEEDS[name]

    # ---- set-up (untimed): cases, pools, prefix fill, pool copies -----------------
    states = []
    kv_bytes = 0
    rows = 0
    flops = 0
    first_case = None
    for layer in range(layers):
        case = synth.make_case(name, seed, device="cuda",
                               value_seed=seed * 100 + layer if layers > 1 else None)
        st = DeviceCase(case, mab.MAB_BATCH_INVARIANT if args.batch_invariant else 0)
        bpp = kv_bytes_per_position(case.layout)
        kv_bytes += sum(case.context(s) for s in range(case.num_seqs)) * bpp
        rows = case.num_rows  # the layers share one batch
        flops += chunk_flops(case)
        if first_case is None:
            first_case = case
        else:  # keep only what the timed loop needs
            case.k_prefix = case.v_prefix = None
        states.append(st)
    per_layer_pool = states[0].k_pool.numel() + states[0].v_pool.numel()
    copies = args.copies or (max(1, min(16, math.ceil((1 << 30) / (per_layer_pool * layers))))
                             if layers == 1 else 1)
    pools = [[(st.k_pool, st.v_pool)] for st in states]
    for i, st in enumerate(states):
        for _ in range(copies - 1):
            pools[i].append((st.k_pool.clone(), st.v_pool.clone()))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(it, ev=None):
        for i, st in enumerate(states):
            kp, vp = pools[i][it % copies]
            if ev is not None:
                ev[0].record(stream)
            mab.kv_append_quant(st.layout, st.batch, st.k_new, st.v_new, kp, vp, stream)
            if ev is not None:
                ev[1].record(stream)
            mab.mixed_attention_fwd(st.layout, st.batch, st.q, kp, vp, st.case.sm_scale, st.out,
                                    st.ws, stream)
            if ev is not None:
                ev[2].record(stream)
                ev = ev[3:]

    # the set-up left the device idle: half a second of matrix-core work first,
    # so that the W warm-up steps and the timed region run at the sustained
    # clock rather than while it ramps up (a short decode step is over in
    # well under a millisecond)
    clock_warmup(stream, CLOCK_WARMUP_S)
    for it in range(args.warmup):
        step(it)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, nothing else on the stream ---------------
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for it in range(args.steps):
        step(args.warmup + it)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # ---- breakdown pass (after the timed region): the same steps with events
    # around each call, which cost the stream a few us per step and so stay out
    # of the timed region -----------------------------------------------------------
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3 * layers)] for _ in range(args.steps)]
    for it in range(args.steps):
        step(args.warmup + args.steps + it, evs[it])
    torch.cuda.synchronize()
    attn_ms = [e[3 * l + 1].elapsed_time(e[3 * l + 2]) for e in evs for l in range(layers)]
    app_ms = [e[3 * l].elapsed_time(e[3 * l + 1]) for e in evs for l in range(layers)]
    attn_avg = float(np.mean(attn_ms))

    # ---- roofline pass (after the timed region): back-to-back attention calls
    # between two events on their stream, so per-call launch gaps are not
    # charged to the kernels ------------------------------------------------------
    n_rf = max(20, args.steps)
    rf0 = torch.cuda.Event(enable_timing=True)
    rf1 = torch.cuda.Event(enable_timing=True)
    rf0.record(stream)
    for it in range(n_rf):
        for i, st in enumerate(states):
            kp, vp = pools[i][it % copies]
            mab.mixed_attention_fwd(st.layout, st.batch, st.q, kp, vp, st.case.sm_scale, st.out,
                                    st.ws, stream)
    rf1.record(stream)
    torch.cuda.synchronize()
    call_ms = rf0.elapsed_time(rf1) / (n_rf * layers)
    # the dominant kernel alone: the same calls again, each with the library's
    # event pair around its attention kernel (the merge kernels excluded)
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_rf * layers)]
    for it in range(n_rf):
        for i, st in enumerate(states):
            kp, vp = pools[i][it % copies]
            e0, e1 = kev[it * layers + i]
            mab.mixed_attention_fwd_timed(st.layout, st.batch, st.q, kp, vp, st.case.sm_scale, st.out,
                                          st.ws, e0, e1, stream)
    torch.cuda.synchronize()
    kernel_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in kev]))
    kv_per_launch = kv_bytes / layers
    achieved = kv_per_launch / (kernel_ms * 1e-3) / 1e9
    call_achieved = kv_per_launch / (call_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"{name}: {WORKLOADS[name]}",
            "seed": seed,
            "layers": layers,
            "query_rows_per_step": rows,
            "kv_bytes_per_step": int(kv_bytes),
            "kv_format": f"K{first_case.layout['k_format']}/V{first_case.layout['v_format']}",
            "pool_copies_rotated": copies,
            "clock_warmup_s": CLOCK_WARMUP_S,
            "batch_invariant": bool(args.batch_invariant),
        },
        "query_tok_s": round(rows / (ms_per_step * 1e-3), 1),
        "attention_ms_avg": round(attn_avg, 6),
        "attention_ms_p10_p90": [round(float(np.percentile(attn_ms, 10)), 6),
                                 round(float(np.percentile(attn_ms, 90)), 6)],
        "append_ms_avg": round(float(np.mean(app_ms)), 6),
        "roofline": {
            "bound": "hbm",
            "kernel": ("the attention kernel of each mixed_attention_fwd call (HIP events the library "
                       "records around its launch, on its stream); call_* figures: the whole call "
                       "(attention kernel + its merge kernels), back-to-back calls"),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel_ms_avg": round(kernel_ms, 6),
            "call_ms_avg": round(call_ms, 6),
            "call_achieved": round(call_achieved, 2),
            "call_frac": round(call_achieved / HBM_PEAK_GBS, 4),
            "algorithmic_bytes_per_launch": int(kv_per_launch),
        },
    }
    traffic = stored_traffic(name)
    if traffic is not None:
        # the attention kernel's own bytes per launch (the kernel `achieved` is
        # measured on); the whole call's bytes beside them
        main = [k for k in ("mixed_attention_kernel", "decode_attention_kernel") if k in traffic["kernels"]]
        result["roofline"]["traffic"] = traffic["kernels"][main[0]]["bytes"] if main else None
        result["roofline"]["traffic_call"] = traffic["bytes_per_call"]
        result["roofline"]["traffic_detail"] = traffic
    if flops:
        # a batch with a prefill chunk is bound by the chunk's matrix products:
        # the roofline is the fp16 MFMA one (QK^T and PV flops of the visible
        # pairs per call); the KV bandwidth figure stays beside it
        tf = flops / layers / (kernel_ms * 1e-3) / 1e12
        call_tf = flops / layers / (call_ms * 1e-3) / 1e12
        hbm = result["roofline"]
        result["roofline"] = {
            "bound": "mfma",
            "kernel": hbm["kernel"],
            "achieved": round(tf, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": hbm["traffic"],
            "traffic_call": hbm.get("traffic_call"),
            "kernel_ms_avg": hbm["kernel_ms_avg"],
            "call_ms_avg": hbm["call_ms_avg"],
            "call_achieved": round(call_tf, 2),
            "call_frac": round(call_tf / MFMA_F16_PEAK_TFLOPS, 4),
            "algorithmic_flops_per_launch": int(flops / layers),
            "algorithmic_bytes_per_launch": hbm["algorithmic_bytes_per_launch"],
            "kv_gbs": hbm["achieved"],
            "kv_frac_of_hbm_peak": hbm["frac"],
        }
        if "traffic_detail" in hbm:
            result["roofline"]["traffic_detail"] = hbm["traffic_detail"]
        result["roofline"]["chunk_only"] = chunk_only_launch(states[0], stream, n_rf)
    result["roofline"]["realism"] = realism_probes(stream)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(first_case)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
