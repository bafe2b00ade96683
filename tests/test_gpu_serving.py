"""The serving loop on the GPU: the library's step scheduler picks each tick's
rows, the kernels append and attend, and every tick's output is checked
against the oracle.  The oracle appends and attends on the same batch with the
same token values.  At the end the pools must be byte-identical.  The
scheduler's batches are also checked tick by tick against the scheduler
oracle."""

import sys

import numpy as np
import pytest
import torch

import mixed_attention_block_amd as mab
import synth
from gpu_harness import POISON, assert_close
from mixed_attention_block_amd.serve import ServingLoop, scenario_loop, simulate, summarize
from oracle import attention as oracle_attention
from oracle import cache as oracle_cache
from oracle import scheduler as oracle_sched

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # (name, layout, scheduler config, seed)
    ("q8_g4_p16", dict(hq=8, hkv=2, d=64, ps=16, kf="q8", vf="q8"),
     dict(sessions=4, prefill_chunk=40, max_pending_per_client=4, near_done_gate=6), 71),
    ("k4v4_g6_p32", dict(hq=12, hkv=2, d=128, ps=32, kf="q4", vf="q4"),
     dict(sessions=3, prefill_chunk=24, max_pending_per_client=2, near_done_gate=3, max_decode_rows=2), 72),
    ("f16_g8_p64", dict(hq=8, hkv=1, d=128, ps=64, kf="f16", vf="f16"),
     dict(sessions=5, prefill_chunk=33, max_pending_per_client=3, near_done_gate=5), 73),
    ("k8v4_g2_p48", dict(hq=4, hkv=2, d=64, ps=48, kf="q8", vf="q4"),
     dict(sessions=4, prefill_chunk=17, max_pending_per_client=4, near_done_gate=2, max_decode_rows=3), 74),
]


@pytest.mark.parametrize("name,lay,cfg,seed", CASES, ids=[c[0] for c in CASES])
def test_serving_loop_matches_oracle(name, lay, cfg, seed):
    rng = np.random.default_rng(seed)
    num_pages, width = 160, 16
    cfg = dict(cfg, page_size=lay["ps"], num_pages=num_pages, max_pages_per_seq=width)
    layout = mab.make_layout(lay["hq"], lay["hkv"], lay["d"], lay["ps"], num_pages, lay["kf"], lay["vf"])
    olay = dict(num_q_heads=lay["hq"], num_kv_heads=lay["hkv"], head_dim=lay["d"], page_size=lay["ps"],
                num_pages=num_pages, k_format=lay["kf"], v_format=lay["vf"])
    sm_scale = float(np.float32(1 / np.sqrt(lay["d"])))
    lib_sched = mab.Scheduler(**dict(cfg, max_decode_rows=cfg.get("max_decode_rows", 0)))
    ref_sched = oracle_sched.Scheduler(**cfg)
    loop = ServingLoop(layout, lib_sched, sm_scale)
    loop.k_pool.fill_(POISON)
    loop.v_pool.fill_(POISON)
    kp = oracle_cache.new_pool(olay, lay["kf"], fill=POISON)
    vp = oracle_cache.new_pool(olay, lay["vf"], fill=POISON)
    arrivals = {}
    for _ in range(10):
        t = int(rng.integers(0, 30))
        arrivals.setdefault(t, []).append((int(rng.integers(0, 3)), int(rng.integers(1, 90)),
                                           int(rng.integers(1, 20))))
    kinds = {"decode": 0, "merged": 0}
    verify_rows = chunk_rows = 0
    for tick in range(400):
        for client, prompt, limit in arrivals.get(tick, []):
            assert lib_sched.submit(client, prompt, limit) == ref_sched.submit(client, prompt, limit)
        step = lib_sched.step()
        want = ref_sched.step()
        if step is None:
            assert want is None
            if tick > max(arrivals):
                break
            continue
        q_len = np.diff(step.q_start)
        assert want["ids"] == list(step.request_id) and want["q_len"] == list(q_len)
        assert want["prefix_len"] == list(step.prefix_len)
        kinds[step.kind] += 1
        verify_rows += int(((q_len > 1) & (q_len <= 16)).sum())
        chunk_rows += int((q_len > 16).sum())
        rids = np.repeat(step.request_id, q_len)
        pos = np.concatenate([p + np.arange(n) for p, n in zip(step.prefix_len, q_len)])
        q, k, v = synth.token_values(seed, rids, pos, lay["hq"], lay["hkv"], lay["d"])
        _say(f"{name} tick {tick}: {step.kind}, {step.num_seqs} seqs, {int(q_len.sum())} rows")
        batch = loop.prepare(step)
        out = torch.full((len(pos), lay["hq"], lay["d"]), float("nan"), dtype=torch.float32, device="cuda")
        loop.launch(batch, torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), out)
        oracle_cache.append(kp, vp, olay, step.q_start, step.prefix_len, step.block_table, k, v)
        ref = oracle_attention.attention(q, kp, vp, olay, step.q_start, step.prefix_len, step.block_table, sm_scale)
        assert_close(out.cpu().numpy(), ref, f"{name} tick {tick}")
    else:
        pytest.fail("the trace did not drain")
    assert kinds["decode"] > 5 and kinds["merged"] > 5 and chunk_rows > 0 and verify_rows > 0, (kinds, chunk_rows,
                                                                                               verify_rows)
    assert np.array_equal(loop.k_pool.cpu().numpy(), kp.reshape(-1))
    assert np.array_equal(loop.v_pool.cpu().numpy(), vp.reshape(-1))


def test_simulator_runs_a_scenario():
    """The five-into-four scenario at a smaller scale of time: every request
    finishes with its token limit, the waiting request is admitted, and the
    clock only moves forward."""
    loop, arrivals = scenario_loop("five_into_four", chunk=512, gate=64)
    arrivals = [(t, c, min(p, 20000), min(l, 200)) for t, c, p, l in arrivals]
    _say(f"simulate five_into_four (shortened): {arrivals}")
    reqs, ticks = simulate(loop, arrivals)
    assert len(reqs) == 5
    for r in reqs.values():
        assert len(r["tokens"]) == r["limit"]
        assert all(b >= a for a, b in zip(r["tokens"], r["tokens"][1:]))
        assert r["tokens"][0] >= r["arrival"]
    s = summarize(reqs, ticks)
    assert s["ticks"] == s["decode_ticks"] + s["merged_ticks"] and s["gpu_ms"] > 0
