"""Serving loop: the step scheduler's batches run through the kernels.

Each tick, ``mab_sched_step`` picks the rows: decoders plus at most one prefill
chunk slice.  ``kv_append_quant`` then writes the rows' new K/V into the paged
pools, and ``mixed_attention_fwd`` computes their attention, both on the
current stream.  The rules are those of the MBufo page ("自研RDNA高併發推論引擎
以AI Max+ 395為範例"), section 1.

The simulator drives it with timed arrivals.  Its clock advances by the
measured GPU time of each tick (append + attention of one layer, HIP events
around them); when nothing can run it jumps to the next arrival.  From the
times at which rows emit tokens it reports time-to-first-token and
inter-token-latency proxies.  These are attention-only proxies: no weight
GEMMs, one layer, no sampling.

    python -m mixed_attention_block_amd.serve --scenario chat16_long250k
"""

import argparse
import json
import sys
import time

import numpy as np
import torch

from . import (Scheduler, attention_workspace_bytes, kv_append_quant, kv_pool_bytes, make_layout,
               mixed_attention_fwd)


class ServingLoop:
    """Device pools for one attention layer plus the scheduler that fills them."""

    def __init__(self, layout, scheduler, sm_scale, device="cuda"):
        self.layout = layout
        self.sched = scheduler
        self.sm_scale = sm_scale
        self.device = device
        self.k_pool = torch.zeros(kv_pool_bytes(layout, layout.k_format), dtype=torch.uint8, device=device)
        self.v_pool = torch.zeros(kv_pool_bytes(layout, layout.v_format), dtype=torch.uint8, device=device)
        self.workspace = torch.empty(1 << 20, dtype=torch.uint8, device=device)

    def prepare(self, step):
        """The step's device descriptor, with the workspace grown to fit it."""
        batch = step.batch(self.device)
        need = attention_workspace_bytes(self.layout, batch)
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.device)
        return batch

    def launch(self, batch, q, k, v, out):
        """Appends the step's K/V rows, then writes the rows' attention into
        ``out`` (fp32 [rows, Hq, D]).  q, k, v: fp16 device tensors."""
        kv_append_quant(self.layout, batch, k, v, self.k_pool, self.v_pool)
        mixed_attention_fwd(self.layout, batch, q, self.k_pool, self.v_pool, self.sm_scale, out, self.workspace)


def warm_up(loop):
    """One untimed decode step and one untimed 32-row chunk step on page 0, as
    an engine runs before it serves: the library's first launches (code
    object load and set-up) stay out of the first measured tick.  The rows'
    K/V land in slots that any request using page 0 writes before it reads.
    Then half a second of matrix-core work lets the clock settle."""
    from . import BatchDesc
    hq, hkv, d = loop.layout.num_q_heads, loop.layout.num_kv_heads, loop.layout.head_dim
    for rows in (1, 32):
        qs, pl = np.array([0, rows], np.int32), np.zeros(1, np.int32)
        bt = torch.zeros((1, 1), dtype=torch.int32, device=loop.device)
        batch = BatchDesc(torch.from_numpy(qs).to(loop.device), torch.from_numpy(pl).to(loop.device), bt, qs, pl)
        q = torch.zeros((rows, hq, d), dtype=torch.float16, device=loop.device)
        kv = torch.zeros((rows, hkv, d), dtype=torch.float16, device=loop.device)
        out = torch.empty((rows, hq, d), dtype=torch.float32, device=loop.device)
        need = attention_workspace_bytes(loop.layout, batch)
        if need > loop.workspace.numel():
            loop.workspace = torch.empty(need, dtype=torch.uint8, device=loop.device)
        loop.launch(batch, q, kv, kv, out)
    torch.cuda.synchronize()
    # half a second of matrix-core work, so that the first ticks run at the
    # sustained clock rather than while it ramps up from the idle set-up
    from . import mab_probe_mfma_f16
    sink = torch.zeros(4, dtype=torch.float32, device=loop.device)
    t = time.time()
    while time.time() - t < 0.5:
        mab_probe_mfma_f16(20000, sink)
        torch.cuda.synchronize()


def simulate(loop, arrivals, seed=0, max_ticks=1_000_000):
    """Runs ``arrivals`` [(time s, client, prompt, limit)] to completion.
    Returns (per-request records, per-tick records)."""
    gen = torch.Generator(device=loop.device)
    gen.manual_seed(seed)
    hq, hkv, d = loop.layout.num_q_heads, loop.layout.num_kv_heads, loop.layout.head_dim
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reqs, ticks = {}, []
    clock, i = 0.0, 0
    while len(ticks) < max_ticks:
        while i < len(arrivals) and arrivals[i][0] <= clock:
            t, client, prompt, limit = arrivals[i]
            status, rid = loop.sched.submit(client, prompt, limit)
            if rid >= 0:
                reqs[rid] = dict(client=client, prompt=prompt, limit=limit, arrival=t, tokens=[])
            else:
                reqs[f"rejected{i}"] = dict(client=client, prompt=prompt, limit=limit, arrival=t,
                                            status=status, tokens=[])
            i += 1
        step = loop.sched.step()
        if step is None:
            if i == len(arrivals):
                break
            clock = max(clock, arrivals[i][0])
            continue
        rows = int(step.q_start[-1])
        q = torch.randn((rows, hq, d), generator=gen, device=loop.device).to(torch.float16)
        k = torch.randn((rows, hkv, d), generator=gen, device=loop.device).to(torch.float16)
        v = torch.randn((rows, hkv, d), generator=gen, device=loop.device).to(torch.float16)
        batch = loop.prepare(step)
        out = torch.empty((rows, hq, d), dtype=torch.float32, device=loop.device)
        start.record()
        loop.launch(batch, q, k, v, out)
        stop.record()
        stop.synchronize()
        dt = start.elapsed_time(stop) / 1e3
        clock += dt
        q_len = np.diff(step.q_start)
        ticks.append(dict(kind=step.kind, seqs=step.num_seqs, rows=rows,
                          chunk=int(q_len[-1]) if step.kind == "merged" and q_len[-1] > 1 else 0,
                          max_context=int((step.prefix_len + q_len).max()), ms=dt * 1e3))
        for rid, e in zip(step.request_id, step.emit):
            if e:
                reqs[int(rid)]["tokens"].append(clock)
    return reqs, ticks


def _pct(x, p):
    return float(np.percentile(np.asarray(x), p)) if len(x) else None


def summarize(reqs, ticks, long_prompt=10000):
    """TTFT and ITL proxies (ms), for short requests and long prompts apart."""
    def group(sel):
        rs = [r for r in reqs.values() if r["tokens"] and sel(r)]
        ttft = [1e3 * (r["tokens"][0] - r["arrival"]) for r in rs]
        itl = [1e3 * g for r in rs for g in np.diff(r["tokens"])]
        return dict(requests=len(rs), ttft_ms_p50=_pct(ttft, 50), ttft_ms_max=_pct(ttft, 100),
                    itl_ms_p50=_pct(itl, 50), itl_ms_p99=_pct(itl, 99), itl_ms_max=_pct(itl, 100))
    kinds = [t["kind"] for t in ticks]
    return dict(ticks=len(ticks), decode_ticks=kinds.count("decode"), merged_ticks=kinds.count("merged"),
                gpu_ms=sum(t["ms"] for t in ticks),
                rejected=sum(1 for k in reqs if isinstance(k, str)),
                short=group(lambda r: r["prompt"] < long_prompt),
                long=group(lambda r: r["prompt"] >= long_prompt))


def scenario_loop(name, chunk=512, gate=64, sessions=None, device="cuda"):
    """The layout and scheduler for one of ``synth.SCENARIOS``: 24 query heads,
    4 KV heads, head_dim 128, q8 pools with 256-token pages, sized for every
    request of the scenario at once."""
    import synth
    arrivals = synth.serving_arrivals(name, 0)
    ps = 256
    pages = sum(-(-(p + l - 1) // ps) for _, _, p, l in arrivals)
    widest = max(-(-(p + l - 1) // ps) for _, _, p, l in arrivals)
    if sessions is None:
        sessions = 4 if name == "five_into_four" else len(arrivals)
    layout = make_layout(24, 4, 128, ps, pages, "q8", "q8")
    sched = Scheduler(sessions, chunk, 4, gate, ps, pages, widest)
    return ServingLoop(layout, sched, float(np.float32(1 / np.sqrt(128))), device), arrivals


def main(argv=None):
    ap = argparse.ArgumentParser(description="serving-loop simulator over the library's kernels")
    ap.add_argument("--scenario", default="chat16_long250k")
    ap.add_argument("--chunk", type=int, default=512)
    ap.add_argument("--gate", type=int, default=64)
    ap.add_argument("--sessions", type=int, default=None)
    args = ap.parse_args(argv)
    loop, arrivals = scenario_loop(args.scenario, args.chunk, args.gate, args.sessions)
    warm_up(loop)
    reqs, ticks = simulate(loop, arrivals)
    out = dict(scenario=args.scenario, prefill_chunk=args.chunk, near_done_gate=args.gate,
               sessions=loop.sched.config.sessions, **summarize(reqs, ticks))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
