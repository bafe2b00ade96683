"""GPU: one step (kv_append_quant + mixed_attention_fwd) captured in a HIP
graph through torch.cuda.graph and replayed.  The library enqueues kernels
only (no memset, no allocation, no host synchronisation) and the per-step
batch travels in device arrays and kernel arguments, so every replay must
give the eager step's output bit for bit.  Replays are interleaved with the
program's own eager work and synchronisations, and each one is checked."""

import sys

import pytest
import torch

import mixed_attention_block_amd as mab
import synth
from gpu_harness import GpuState

pytestmark = pytest.mark.gpu

# a mixed batch (chunk, verify and decode rows), and a K4V4 batch with more
# decode sub-rows than the kernel arguments hold (launch tables written by a
# planning kernel inside the captured step)
CASES = {"small_mixed_q8": dict(name="small_mixed"),
         "many_decode_k4v4": dict(name="small_mixed", kf="q4", vf="q4",
                                  seqs=[(37 * i % 900 + 5, 1) for i in range(130)] + [(300, 40)])}


@pytest.mark.parametrize("cid", sorted(CASES))
@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_captured_step_replays_bitwise(cid, noalloc):
    print(f"graph: case {cid} noalloc={noalloc} seed 31", flush=True)
    sys.stdout.flush()
    kw = dict(CASES[cid])
    case = synth.make_case(kw.pop("name"), seed=31, device="cuda", **kw)
    st = GpuState(case)
    q = case.q.cuda().contiguous()
    kn, vn = case.k_new.cuda().contiguous(), case.v_new.cuda().contiguous()
    out = torch.empty((q.shape[0], case.layout["num_q_heads"], case.layout["head_dim"]), dtype=torch.float32,
                      device="cuda")
    ws = st.workspace()

    def step():
        mab.kv_append_quant(st.layout, st.batch, kn, vn, st.k_pool, st.v_pool)
        if noalloc:
            mab.mixed_attention_fwd_noalloc(st.layout, st.batch, q, st.k_pool, st.v_pool, case.sm_scale, out)
        else:
            mab.mixed_attention_fwd(st.layout, st.batch, q, st.k_pool, st.v_pool, case.sm_scale, out, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # eager, on the stream that will capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        noise = torch.randn(1 << 20, device="cuda")  # the program's own eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager step"
        del noise
