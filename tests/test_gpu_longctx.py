"""GPU: one decode row at context 1048576, four times the longest benchmark
context: positions near 2^20, 32768 stages per segment cut over the whole
device, and a combine of about 2048 pieces per segment.  K4V4, 8 query heads
over 1 KV head, 256-token pages.  Compared with the oracle element by
element; the pages the step appended are compared bit for bit."""

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_harness import GpuState, assert_close, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

CTX = 1 << 20


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_decode_row_at_1m_context():
    case = synth.make_case("tiny_mixed", 41, device="cuda", hq=8, hkv=1, d=128, ps=256, kf="q4", vf="q4",
                           seqs=[(CTX - 1, 1)])
    # a sharp softmax (logits with a standard deviation near 8): a few keys
    # out of 2^20 carry the output, so a piece left out of the merge, or one
    # merged twice, changes it by O(1) rather than by the noise of a mean
    case.q = (case.q.float() * 8).half()
    _say(f"decode row at context {CTX}: GPU")
    st = GpuState(case)
    st.append_step()
    out = st.attention().cpu().numpy()
    _say("  oracle (encode and fp64 attention over 2^20 keys)")
    kp, vp = oracle_pools(case)
    want = oracle_out(case, kp, vp)
    mx, mean = assert_close(out, want, "decode row at 1M context")
    _say(f"  max abs {mx:.2e} mean abs {mean:.2e}, max |out| {np.abs(want).max():.2f}")
    assert np.abs(want).max() > 0.5  # the softmax is sharp enough for the check to bite
    last = int(case.block_table[0][(CTX - 1) // case.layout["page_size"]])
    gk, gv = st.pools_host()
    assert np.array_equal(gk[last], kp[last]) and np.array_equal(gv[last], vp[last]), "appended page"
    del st
    torch.cuda.empty_cache()
