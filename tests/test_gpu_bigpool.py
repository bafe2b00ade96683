"""GPU: pools larger than 4 GiB, with every page of a batch placed past the
first 4 GiB of each pool, so that the append, decode, verify and chunk kernels
all form byte offsets above 2^32.  Expected values come from the oracle on
the same case with a compact pool: the physical page assignment is invisible
(pinned for the oracle by the page-permutation test, and checked bitwise on
the GPU by test_page_permutation_is_bitwise_invisible)."""

import sys

import numpy as np
import pytest
import torch

import mixed_attention_block_amd as mab
import synth
from gpu_harness import GpuState, assert_close, layout_of, oracle_out, oracle_pools

pytestmark = pytest.mark.gpu

FOUR_GIB = 1 << 32


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _moved(case, shift, num_pages):
    """The case with every block-table page id moved up by `shift` in a pool
    of `num_pages` pages."""
    big = synth.Case(**{**case.__dict__})
    big.layout = dict(case.layout, num_pages=num_pages)
    big.block_table = np.where(case.block_table >= 0, case.block_table + shift, -1).astype(np.int32)
    return big


@pytest.mark.parametrize("kf,vf", [("q4", "q4"), ("q8", "q8")])
def test_pools_beyond_4gib(kf, vf):
    # a decode row, a verify row (5 tokens, G = 4: one wide sub-row over
    # quantized pools), two prefill chunks and a short verify row
    case = synth.make_case("tiny_mixed", 31, device="cuda", hq=8, hkv=2, d=128, ps=64, kf=kf, vf=vf,
                           seqs=[(2999, 1), (500, 100), (1000, 5), (70, 17), (0, 3)])
    kp, vp = oracle_pools(case)
    want = oracle_out(case, kp, vp)
    small = case.layout["num_pages"]
    page_k = mab.kv_pool_bytes(layout_of(case), kf) // small
    page_v = mab.kv_pool_bytes(layout_of(case), vf) // small
    shift = -(-(FOUR_GIB + (1 << 28)) // min(page_k, page_v))  # every used page starts past 4.25 GiB
    big = _moved(case, shift, shift + small)
    _say(f"pools beyond 4 GiB {kf}/{vf}: pages {shift + small}, page bytes {page_k}/{page_v}")
    st = GpuState(big)
    assert st.k_pool.numel() > FOUR_GIB and st.v_pool.numel() > FOUR_GIB
    st.append_step()
    out = st.attention().cpu().numpy()
    mx, mean = assert_close(out, want, f"pools beyond 4 GiB {kf}/{vf}")
    _say(f"  max abs {mx:.2e} mean abs {mean:.2e}")
    # every page the batch wrote holds the oracle's bytes
    for p in np.unique(case.block_table[case.block_table >= 0]):
        q = int(p) + shift
        gk = st.k_pool[q * page_k:(q + 1) * page_k].cpu().numpy()
        gv = st.v_pool[q * page_v:(q + 1) * page_v].cpu().numpy()
        assert np.array_equal(gk, kp[p].reshape(-1)), f"K page {p}"
        assert np.array_equal(gv, vp[p].reshape(-1)), f"V page {p}"
    del st
    torch.cuda.empty_cache()
