"""The no-allocation entry point against mixed_attention_fwd.

mixed_attention_fwd_noalloc takes its workspace from the library's fixed
per-device array instead of a caller buffer.  Two calls in a row (the second
on a smaller batch, so that it runs over what the first left in the array)
must each give outputs bit-identical to mixed_attention_fwd on the same batch
with a fresh caller workspace: the same kernels, launch shapes and
arithmetic.  A batch needing more workspace than the array is refused with
MAB_ERR_SCRATCH before anything runs.
"""

import sys

import numpy as np
import pytest
import torch

import mixed_attention_block_amd as mab
import synth
from gpu_harness import GpuState, assert_close, batch_of, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _noalloc(st, batch, q):
    c = st.case
    out = torch.full((q.shape[0], c.layout["num_q_heads"], c.layout["head_dim"]), float("nan"),
                     dtype=torch.float32, device="cuda")
    mab.mixed_attention_fwd_noalloc(st.layout, batch, q.contiguous(), st.k_pool, st.v_pool, c.sm_scale, out)
    return out


def test_noalloc_matches_caller_workspace():
    seqs = [(700, 40), (3000, 1), (129, 4), (5000, 1), (31, 1), (2047, 16), (64, 17), (1500, 1)]
    case = synth.make_case("small_mixed", 91, device="cuda", seqs=seqs, ps=32)
    _say(f"noalloc: {case.num_seqs} sequences, {case.num_rows} rows")
    st = GpuState(case)
    st.append_step()
    assert mab.attention_workspace_bytes(st.layout, st.batch) <= mab.NOALLOC_SCRATCH_BYTES
    # call 1: the whole batch
    got1 = _noalloc(st, st.batch, case.q).cpu().numpy()
    want1 = st.attention().cpu().numpy()
    assert np.array_equal(got1, want1), "call 1 differs from mixed_attention_fwd"
    kp, vp = oracle_pools(case)
    assert_close(got1, oracle_out(case, kp, vp), "noalloc call 1")
    # call 2: a smaller batch over what call 1 left in the array
    sub, rows = synth.subset(case, [1, 2, 4])
    b = batch_of(sub.q_start, sub.prefix_len, sub.block_table)
    got2 = _noalloc(st, b, sub.q).cpu().numpy()
    want2 = st.attention(batch=b, q=sub.q).cpu().numpy()
    assert np.array_equal(got2, want2), "call 2 differs from mixed_attention_fwd"
    _say("  both calls bit-identical to the caller-workspace call")


def test_noalloc_rejects_batches_beyond_the_array():
    case = synth.make_case("mixed16_chunk2k", 3, device="cuda", with_values=False)
    lay = case.layout
    layout = mab.make_layout(lay["num_q_heads"], lay["num_kv_heads"], lay["head_dim"], lay["page_size"],
                             lay["num_pages"], lay["k_format"], lay["v_format"])
    # the same sequences four times over: more split partials than the array holds
    reps = 4
    qs = np.concatenate([[0], np.cumsum(np.tile(np.diff(case.q_start), reps))]).astype(np.int32)
    pl = np.tile(case.prefix_len, reps).astype(np.int32)
    bt = np.tile(case.block_table, (reps, 1)).astype(np.int32)
    b = batch_of(qs, pl, bt)
    need = mab.attention_workspace_bytes(layout, b)
    _say(f"noalloc refusal: batch needs {need / 2**20:.1f} MiB")
    assert need > mab.NOALLOC_SCRATCH_BYTES
    small = torch.zeros(16, dtype=torch.uint8, device="cuda")
    q = torch.zeros((int(qs[-1]), lay["num_q_heads"], lay["head_dim"]), dtype=torch.float16, device="cuda")
    out = torch.zeros((int(qs[-1]), lay["num_q_heads"], lay["head_dim"]), dtype=torch.float32, device="cuda")
    with pytest.raises(mab.MabError) as e:
        mab.mixed_attention_fwd_noalloc(layout, b, q, small, small, case.sm_scale, out)
    assert e.value.status == 8
    torch.cuda.synchronize()
    assert float(out.abs().sum()) == 0.0  # nothing ran
