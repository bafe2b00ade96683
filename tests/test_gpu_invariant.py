"""GPU: the MAB_BATCH_INVARIANT batch flag.

With the flag, every decode and verify row is cut into 512-key pieces from
its own first key, so its output is bit-identical whatever else shares the
batch (the MBufo page's three-numbers table asks greedy output to stay
bit-identical; its section 1 fairness part checks a prompt by hash alone and
under load).  Prefill-chunk rows are batch-independent with or without it.
The outputs still meet the oracle tolerance (max abs 4e-3, mean abs 1e-3).
"""

import sys

import numpy as np
import pytest

import mixed_attention_block_amd as mab
import synth
from gpu_harness import GpuState, assert_close, batch_of, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

INV = mab.MAB_BATCH_INVARIANT

# decode rows longer than one piece, verify rows, a chunk; contexts span piece edges
SEQS = [(3000, 1), (511, 1), (512, 1), (1023, 1), (700, 4), (64, 40), (9000, 1), (2047, 16), (0, 2), (5, 1)]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inv_batch(case):
    return batch_of(case.q_start, case.prefix_len, case.block_table, flags=INV)


@pytest.mark.parametrize("kf,vf,hq,hkv,ps", [("q8", "q8", 24, 4, 32), ("q4", "q4", 24, 4, 64),
                                             ("q8", "q4", 8, 1, 48), ("q4", "q8", 14, 2, 16)],
                         ids=["q8_g6_p32", "k4v4_g6_p64", "k8v4_g8_p48", "k4v8_g7_p16"])
def test_invariant_matches_oracle(kf, vf, hq, hkv, ps):
    case = synth.make_case("small_mixed", 71, device="cuda", seqs=SEQS, kf=kf, vf=vf, hq=hq, hkv=hkv, ps=ps)
    _say(f"invariant vs oracle {kf}/{vf} hq={hq} hkv={hkv} ps={ps}")
    st = GpuState(case)
    st.append_step()
    out = st.attention(batch=_inv_batch(case)).cpu().numpy()
    kp, vp = oracle_pools(case)
    assert_close(out, oracle_out(case, kp, vp), f"invariant {kf}{vf}")
    default = st.attention().cpu().numpy()
    d = float(np.abs(out - default).max())
    assert d <= 1e-3, f"invariant vs default cut: {d:.3g}"


@pytest.mark.parametrize("key", ["q8", "k4v4"])
def test_invariant_mixed_equals_separate(key):
    """One mixed launch versus launches of its parts, every row bit-identical."""
    kw = dict(kf="q4", vf="q4") if key == "k4v4" else {}
    case = synth.make_case("small_mixed", 72, device="cuda", seqs=SEQS, ps=32, **kw)
    st = GpuState(case)
    st.append_step()
    full = st.attention(batch=_inv_batch(case)).cpu().numpy()
    chunks = [s for s in range(case.num_seqs) if case.q_len(s) > 16]
    decodes = [s for s in range(case.num_seqs) if case.q_len(s) <= 16]
    for seqs in (chunks, decodes, [decodes[-1], chunks[0]], [decodes[0]], decodes[::-1]):
        _say(f"invariant {key}: subset {seqs}")
        sub, rows = synth.subset(case, seqs)
        b = batch_of(sub.q_start, sub.prefix_len, sub.block_table, flags=INV)
        part = st.attention(batch=b, q=sub.q).cpu().numpy()
        for k, s in enumerate(seqs):
            r_full = np.arange(case.q_start[s], case.q_start[s + 1])
            r_part = np.arange(sub.q_start[k], sub.q_start[k + 1])
            assert np.array_equal(part[r_part], full[r_full]), f"seq {s} of {seqs}"


def test_invariant_large_batch_vs_single_row():
    """A batch beyond the kernel-argument tables (launch tables built on the
    device) and each of a few of its decode and verify rows alone: bit-identical."""
    rng = np.random.default_rng(73)
    seqs = [(int(rng.integers(0, 3000)), 1) for _ in range(110)]
    seqs += [(int(rng.integers(0, 2000)), int(rng.integers(2, 24))) for _ in range(20)]
    seqs = [seqs[i] for i in rng.permutation(len(seqs))]
    case = synth.make_case("small_mixed", 74, device="cuda", seqs=seqs, ps=16, spare_pages=8)
    _say(f"invariant large batch: {len(seqs)} sequences, {case.num_rows} rows")
    st = GpuState(case)
    st.append_step()
    out = st.attention(batch=_inv_batch(case)).cpu().numpy()
    kp, vp = oracle_pools(case)
    assert_close(out, oracle_out(case, kp, vp), "invariant large batch")
    picks = [s for s in range(case.num_seqs) if case.q_len(s) <= 16][:6]
    for s in picks:
        sub, rows = synth.subset(case, [s])
        one = st.attention(batch=batch_of(sub.q_start, sub.prefix_len, sub.block_table, flags=INV),
                           q=sub.q).cpu().numpy()
        assert np.array_equal(one, out[rows]), f"seq {s} (q_len {case.q_len(s)}, prefix {case.prefix_len[s]})"
