"""GPU parity at the benchmark workloads' full sizes, in the launch
configuration bench.py times.  The whole batch runs on the GPU; the oracle
recomputes a sample of rows (decode rows incl. the longest, and chunk rows at
tile and split boundaries) and the KV bytes of the sampled sequences' pages."""

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_harness import GpuState, assert_close, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

WORKLOADS = [("decode16", 2), ("decode16_f16", 2), ("verify16", 6), ("mixed16_chunk2k", 3), ("long_q8", 4),
             ("long_k4v4", 4), ("step_k4v4", 5)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _sample(case):
    seqs, rows = [], []
    dec = [s for s in range(case.num_seqs) if case.q_len(s) == 1]
    if dec:
        longest = max(dec, key=case.context)
        shortest = min(dec, key=case.context)
        for s in dict.fromkeys([longest, shortest, dec[len(dec) // 2]]):
            seqs.append(s)
            rows.append(int(case.q_start[s]))
    for s in range(case.num_seqs):
        n = case.q_len(s)
        if n > 1:
            seqs.append(s)
            r0 = int(case.q_start[s])
            for i in sorted({0, 1, 31, 32, 33, n // 2, n - 33, n - 2, n - 1}):
                if 0 <= i < n:
                    rows.append(r0 + i)
    return seqs, rows


def _pages_of(case, seqs):
    ps = case.layout["page_size"]
    out = []
    for s in seqs:
        npg = -(-case.context(s) // ps)
        out.extend(int(p) for p in case.block_table[s, :npg])
    return np.array(sorted(out))


@pytest.mark.parametrize("name,seed", WORKLOADS, ids=[w[0] for w in WORKLOADS])
def test_fullsize_sampled(name, seed):
    _say(f"fullsize workload={name} seed={seed}: building on GPU")
    case = synth.make_case(name, seed, device="cuda",
                           value_seed=seed * 100 if name == "step_k4v4" else None)
    st = GpuState(case)
    st.append_step()
    out = st.attention()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "non-finite output"
    seqs, rows = _sample(case)
    _say(f"  oracle on {len(seqs)} sequences, {len(rows)} rows")
    kp, vp = oracle_pools(case, seqs=seqs)
    gk, gv = st.pools_host()
    pages = _pages_of(case, seqs)
    assert np.array_equal(gk[pages], kp[pages]), "K bytes differ"
    assert np.array_equal(gv[pages], vp[pages]), "V bytes differ"
    want = oracle_out(case, kp, vp, rows=rows)
    got = out.cpu().numpy()
    mx, mean = assert_close(got[rows], want[rows], name)
    _say(f"  max abs {mx:.2e} mean abs {mean:.2e}")
