"""GPU: a batch at the sequence-count limit (4096 sequences: decode rows,
verify rows of 2-16 tokens and a few prefill chunks, K4V4 on 16-key pages),
whose launch-order tables the planning kernel writes on the device.  The KV
bytes of sampled sequences are bit-identical to the oracle's and the outputs
of their rows are within the oracle tolerance."""

import sys

import numpy as np
import pytest

import synth
from gpu_harness import GpuState, assert_close, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu


def test_sequence_count_limit_batch():
    rng = np.random.default_rng(53)
    seqs = [(int(rng.integers(0, 200)), 1) for _ in range(4000)]
    seqs += [(int(rng.integers(0, 150)), int(rng.integers(2, 17))) for _ in range(90)]
    seqs += [(int(rng.integers(0, 120)), int(rng.integers(17, 70))) for _ in range(6)]
    seqs = [seqs[i] for i in rng.permutation(len(seqs))]
    assert len(seqs) == 4096
    case = synth.make_case("small_mixed", 54, device="cuda", seqs=seqs, ps=16, kf="q4", vf="q4")
    print(f"max-size batch: {case.num_seqs} sequences, {case.num_rows} rows", flush=True)
    sys.stdout.flush()
    st = GpuState(case)
    st.append_step()
    out = st.attention().cpu().numpy()
    # every chunk and verify sequence, and a sample of the decode rows
    sample = sorted({s for s in range(case.num_seqs) if case.q_len(s) > 1}
                    | set(int(s) for s in rng.choice(case.num_seqs, 300, replace=False)))
    kp, vp = oracle_pools(case, sample)
    gk, gv = st.pools_host()
    for s in sample:  # the pages of each sampled sequence, byte for byte
        pages = case.block_table[s][case.block_table[s] >= 0]
        assert np.array_equal(gk[pages], kp[pages]) and np.array_equal(gv[pages], vp[pages]), f"sequence {s}"
    rows = [r for s in sample for r in range(int(case.q_start[s]), int(case.q_start[s + 1]))]
    assert_close(out[rows], oracle_out(case, kp, vp, rows=rows)[rows], "max-size batch")
