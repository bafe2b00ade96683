"""GPU: mixed_attention_fwd_timed, the measurement variant of the attention
call.  Its outputs must be bit-identical to mixed_attention_fwd's on the same
inputs (the call is the same; only two event records are added), and the
interval between its two events (the attention kernel alone) must lie
within the interval of the whole call."""

import sys

import pytest
import torch

import mixed_attention_block_amd as mab
import synth
from gpu_harness import GpuState

pytestmark = pytest.mark.gpu


# a mixed batch (chunk + decode + verify rows), and a decode-only K4V4 batch
CASES = {"small_mixed_q8": dict(name="small_mixed"),
         "decode_k4v4": dict(name="small_mixed", kf="q4", vf="q4", seqs=[(900, 1), (3000, 1), (40, 4), (7, 1)])}


@pytest.mark.parametrize("cid", sorted(CASES))
def test_timed_call_matches_and_brackets_the_kernel(cid):
    print(f"timed call: case {cid} seed 7", flush=True)
    sys.stdout.flush()
    kw = dict(CASES[cid])
    case = synth.make_case(kw.pop("name"), seed=7, device="cuda", **kw)
    st = GpuState(case)
    st.append_step()
    ref = st.attention()
    q = case.q.cuda().contiguous()
    ws = st.workspace()
    stream = torch.cuda.current_stream()
    for _ in range(2):  # the second call reuses events the first created
        out = torch.full_like(ref, float("nan"))
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        mab.mixed_attention_fwd_timed(st.layout, st.batch, q, st.k_pool, st.v_pool, case.sm_scale, out, ws,
                                      k0, k1, stream)
        c1.record(stream)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "timed call differs from mixed_attention_fwd"
        kernel_ms, call_ms = k0.elapsed_time(k1), c0.elapsed_time(c1)
        assert 0.0 < kernel_ms <= call_ms, (kernel_ms, call_ms)
