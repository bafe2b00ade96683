"""GPU: calls are stream-ordered with no implicit synchronisation, and calls
on different streams with distinct workspaces do not interfere.  Two batches
(different formats and shapes) run their steps on two streams at once, from
two host threads, several times over; every output must equal the same step
run alone on the default stream, bit for bit (the arithmetic of a call does
not depend on what else runs on the device)."""

import sys
import threading

import pytest
import torch

import mixed_attention_block_amd as mab
import synth
from gpu_harness import GpuState

pytestmark = pytest.mark.gpu


def _state(seed, **kw):
    case = synth.make_case("small_mixed", seed=seed, device="cuda", **kw)
    st = GpuState(case)
    st.q = case.q.cuda().contiguous()
    st.kn, st.vn = case.k_new.cuda().contiguous(), case.v_new.cuda().contiguous()
    st.out = torch.empty((st.q.shape[0], case.layout["num_q_heads"], case.layout["head_dim"]),
                         dtype=torch.float32, device="cuda")
    st.ws = st.workspace()
    return st


def _step(st, stream):
    mab.kv_append_quant(st.layout, st.batch, st.kn, st.vn, st.k_pool, st.v_pool, stream)
    mab.mixed_attention_fwd(st.layout, st.batch, st.q, st.k_pool, st.v_pool, st.case.sm_scale, st.out, st.ws,
                            stream)


def test_two_streams_two_threads():
    print("streams: small_mixed q8 seed 41 and K4V4 seed 42", flush=True)
    sys.stdout.flush()
    a = _state(41)
    b = _state(42, kf="q4", vf="q4", seqs=[(3000, 1), (700, 1), (40, 4), (128, 200), (9, 1)])
    refs = []
    for st in (a, b):
        _step(st, torch.cuda.current_stream())
        torch.cuda.synchronize()
        refs.append(st.out.clone())
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    errors = []

    def run(st, stream, n):
        try:
            for _ in range(n):
                _step(st, stream)
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    for rep in range(3):
        for st in (a, b):
            st.out.fill_(float("nan"))
        torch.cuda.synchronize()
        threads = [threading.Thread(target=run, args=(st, s, 4)) for st, s in zip((a, b), streams)]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        torch.cuda.synchronize()
        assert not errors, errors
        assert torch.equal(a.out, refs[0]), f"round {rep}: batch A differs"
        assert torch.equal(b.out, refs[1]), f"round {rep}: batch B differs"
