"""Debug mode (MAB_DEBUG=1): the kernels check every page id they read from
the block table and flag an out-of-range one, reading or writing page 0 in its
place.

The pools here hold 8 pages beyond the layout's num_pages, and the planted ids
point into them: an id the kernels failed to check would still address memory
inside the allocation, and shows up as a mismatch, not as a fault."""

import sys

import numpy as np
import pytest
import torch

import mixed_attention_block_amd as mab
import synth
from gpu_harness import POISON, GpuState, batch_of

pytestmark = pytest.mark.gpu

EXTRA_PAGES = 8

# tiny_mixed has 16-key pages (chunk rows take the per-lane page walk); the
# 64-key pages take the wave-uniform walk
CASES = [("tiny_mixed", 61, {}), ("tiny_mixed", 62, dict(ps=64, kf="q4", vf="q8"))]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _padded(pool, page_bytes):
    out = torch.full((pool.numel() + EXTRA_PAGES * page_bytes,), POISON, dtype=torch.uint8, device="cuda")
    out[:pool.numel()] = pool
    return out


def _page_bytes(case, fmt):
    lay = case.layout
    return lay["num_kv_heads"] * lay["page_size"] * (lay["head_dim"] // 32) * mab.kv_block_bytes(fmt)


def _sub_batch(case, seqs, table):
    sub, _ = synth.subset(case, seqs)
    return sub, batch_of(sub.q_start, sub.prefix_len, table[seqs])


@pytest.mark.parametrize("name,seed,kw", CASES)
def test_debug_mode_flags_and_clamps_page_ids(name, seed, kw, monkeypatch):
    case = synth.make_case(name, seed, device="cuda", **kw)
    lay = case.layout
    P = lay["num_pages"]
    _say(f"debug mode case={name} seed={seed} pages={P}")
    monkeypatch.delenv("MAB_DEBUG", raising=False)
    st = GpuState(case)
    st.append_step()
    plain = st.attention().cpu().numpy()

    monkeypatch.setenv("MAB_DEBUG", "1")
    mab.mab_debug_status(reset=True)
    checked = st.attention().cpu().numpy()
    torch.cuda.synchronize()
    assert mab.mab_debug_status(reset=True) == 0, "flag set on a valid batch"
    assert np.array_equal(plain, checked), "debug mode changed the outputs"

    kb, vb = _page_bytes(case, lay["k_format"]), _page_bytes(case, lay["v_format"])
    st.k_pool, st.v_pool = _padded(st.k_pool, kb), _padded(st.v_pool, vb)
    decodes = [s for s in range(case.num_seqs) if case.q_len(s) == 1 and case.prefix_len[s] > 0]
    chunks = [s for s in range(case.num_seqs) if case.q_len(s) > 16]
    assert decodes and chunks
    for kind, seqs in (("decode", decodes), ("chunk", chunks)):
        s = seqs[0]
        bad = case.block_table.copy()
        zero = case.block_table.copy()
        bad[s, 0], zero[s, 0] = P + 2, 0
        sub, b_bad = _sub_batch(case, seqs, bad)
        _, b_zero = _sub_batch(case, seqs, zero)
        _say(f"  {kind}: sequence {s} page 0 -> id {P + 2}")
        got = st.attention(batch=b_bad, q=sub.q).cpu().numpy()
        torch.cuda.synchronize()
        assert mab.mab_debug_status(reset=True) == 1, f"{kind}: out-of-range id not flagged"
        want = st.attention(batch=b_zero, q=sub.q).cpu().numpy()
        torch.cuda.synchronize()
        assert mab.mab_debug_status(reset=True) == 0
        assert np.array_equal(got, want, equal_nan=True), f"{kind}: id not replaced by page 0"

    # append: one sequence whose new rows do not land on page 0 (two writers
    # of one block would race), its first append page replaced
    ps = lay["page_size"]

    def append_pages(q):
        return case.block_table[q, case.prefix_len[q] // ps:(case.prefix_len[q] + case.q_len(q) - 1) // ps + 1]

    s = next(q for q in range(case.num_seqs) if 0 not in append_pages(q))
    pi = int(case.prefix_len[s]) // ps
    bad = case.block_table.copy()
    zero = case.block_table.copy()
    bad[s, pi], zero[s, pi] = P + EXTRA_PAGES - 1, 0
    sub, b_bad = _sub_batch(case, [s], bad)
    _, b_zero = _sub_batch(case, [s], zero)
    _say(f"  append: sequence {s} page {pi} -> id {P + EXTRA_PAGES - 1}")
    k0, v0 = st.k_pool.clone(), st.v_pool.clone()
    mab.kv_append_quant(st.layout, b_bad, sub.k_new.contiguous(), sub.v_new.contiguous(), st.k_pool, st.v_pool)
    torch.cuda.synchronize()
    assert mab.mab_debug_status(reset=True) == 1, "append: out-of-range id not flagged"
    mab.kv_append_quant(st.layout, b_zero, sub.k_new.contiguous(), sub.v_new.contiguous(), k0, v0)
    torch.cuda.synchronize()
    assert mab.mab_debug_status(reset=True) == 0
    assert torch.equal(st.k_pool, k0) and torch.equal(st.v_pool, v0), "append: id not replaced by page 0"
    assert bool((st.k_pool[P * kb:] == POISON).all()) and bool((st.v_pool[P * vb:] == POISON).all())
