"""GPU parity: the HIP path (through the C ABI) against the oracle.

* KV bytes written by kv_append_quant are bit-identical to the oracle's.
* Attention outputs are within max abs 4e-3 and mean abs 1e-3 of the fp64
  oracle.
* Outputs are bit-identical under a permutation of physical pages and from run
  to run; chunk rows are bit-identical between one mixed launch and separate
  launches of its parts (decode rows agree to fp32 reassociation noise).
"""

import sys

import numpy as np
import pytest
import torch

import synth
from gpu_harness import (GpuState, assert_close, batch_of, oracle_out, oracle_pools)
from oracle import cache as oracle_cache

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = {
    "tiny_mixed": ("tiny_mixed", 1, {}),
    "small_q8": ("small_mixed", 2, {}),
    "small_k4v4": ("small_mixed", 3, dict(kf="q4", vf="q4")),
    "small_k8v4": ("small_mixed", 4, dict(kf="q8", vf="q4")),
    "small_k4v8": ("small_mixed", 5, dict(kf="q4", vf="q8")),
    "g6_d128_p16": ("tiny_mixed", 6, dict(hq=12, hkv=2, d=128, ps=16)),
    "g8_d64": ("tiny_mixed", 7, dict(hq=8, hkv=1)),
    "g1_d64_p48": ("tiny_mixed", 8, dict(hq=2, hkv=2, ps=48)),
    "small_f16": ("small_mixed", 9, dict(kf="f16", vf="f16")),
    "tiny_f16_p48": ("tiny_mixed", 10, dict(kf="f16", vf="f16", ps=48)),
    # verify rows (2-16 tokens) run on the decode path in sub-rows of 16/G
    # rows (of 32/G rows over quantized pools when the sequence has more than
    # 16/G rows); 17 rows is the shortest prefill chunk
    "verify_g6": ("small_mixed", 11, dict(seqs=[(300, 2), (1000, 4), (5, 16), (0, 3), (77, 1), (2000, 7),
                                                 (64, 17)])),
    "verify_g1_p48": ("tiny_mixed", 12, dict(hq=2, hkv=2, ps=48, seqs=[(100, 16), (31, 5), (0, 2), (500, 1),
                                                                          (47, 9)])),
    "verify_g8_k4v4": ("tiny_mixed", 13, dict(hq=8, hkv=1, kf="q4", vf="q4", seqs=[(200, 9), (40, 2), (1, 1),
                                                                                      (0, 16)])),
    "verify_f16": ("small_mixed", 14, dict(kf="f16", vf="f16", seqs=[(129, 5), (0, 2), (640, 16), (33, 1)])),
    # over quantized pools a sequence with more than 16/G rows takes sub-rows
    # of 32/G rows (two slot groups per wave, stages loaded straight into
    # LDS run by run): G = 4 on 16-key pages (every stage spans two pages),
    # D = 64, K8V4; and G = 2 at D = 128 on 48-key pages, K4V8
    "verify_g4_p16_k8v4": ("tiny_mixed", 15, dict(hq=8, hkv=2, ps=16, kf="q8", vf="q4",
                                                  seqs=[(100, 16), (31, 5), (0, 7), (250, 9), (3, 1), (60, 4)])),
    "verify_g2_d128_p48_k4v8": ("tiny_mixed", 16, dict(hq=4, hkv=2, d=128, ps=48, kf="q4", vf="q8",
                                                       seqs=[(700, 16), (47, 9), (0, 12), (95, 8), (1, 1)])),
    # odd groups above 1 leave MFMA slots idle: sub-rows of 16/G rows (5 at
    # G = 3, 3 at G = 5, 2 at G = 7) or 32/G over quantized pools (10, 6, 4),
    # and chunk tiles of one head (256 rows); row counts on both sides of
    # each sub-row size
    "g3_d128_p32_k4v4": ("tiny_mixed", 17, dict(hq=6, hkv=2, d=128, ps=32, kf="q4", vf="q4",
                                                seqs=[(100, 40), (300, 5), (64, 6), (0, 10), (777, 11), (5, 1),
                                                      (1500, 16)])),
    "g5_d64_p16_q8": ("tiny_mixed", 18, dict(hq=10, hkv=2, ps=16,
                                             seqs=[(200, 16), (50, 3), (0, 25), (10, 1), (333, 4), (77, 6),
                                                   (90, 7)])),
    "g7_d128_p48_k8v4": ("tiny_mixed", 19, dict(hq=14, hkv=2, d=128, ps=48, kf="q8", vf="q4",
                                                seqs=[(300, 2), (40, 16), (0, 17), (129, 1), (1000, 3), (61, 4),
                                                      (7, 5)])),
    "g7_d64_p64_f16": ("tiny_mixed", 20, dict(hq=7, hkv=1, ps=64, kf="f16", vf="f16",
                                              seqs=[(100, 9), (33, 1), (0, 20), (250, 2), (64, 3)])),
    # more KV heads than the benchmark shapes: eight (G = 8, 64 query heads)
    # and sixteen without grouping (G = 1), so that a chunk's work items span
    # many (KV head, key split) pairs
    "g8_hkv8_d128_p64_k4v4": ("tiny_mixed", 21, dict(hq=64, hkv=8, d=128, ps=64, kf="q4", vf="q4",
                                                     seqs=[(300, 70), (1000, 1), (77, 4), (0, 33), (5, 16)])),
    "g1_hkv16_d64_p32_q8": ("tiny_mixed", 22, dict(hq=16, hkv=16, ps=32,
                                                   seqs=[(200, 300), (4000, 1), (31, 2), (0, 17), (64, 12)])),
}


def _case(key):
    name, seed, kw = CASES[key]
    return synth.make_case(name, seed, device="cuda", **kw)


@pytest.mark.parametrize("key", list(CASES))
def test_append_bitexact(key):
    case = _case(key)
    _say(f"append case={key} seed={case.seed}")
    st = GpuState(case)
    st.append_step()
    torch.cuda.synchronize()
    gk, gv = st.pools_host()
    ok, ov = oracle_pools(case)
    assert np.array_equal(gk, ok), "K pool bytes differ"
    assert np.array_equal(gv, ov), "V pool bytes differ"


@pytest.mark.parametrize("key", list(CASES))
def test_attention_matches_oracle(key):
    case = _case(key)
    _say(f"attention case={key} seed={case.seed}")
    st = GpuState(case)
    st.append_step()
    out = st.attention().cpu().numpy()
    kp, vp = oracle_pools(case)
    want = oracle_out(case, kp, vp)
    mx, mean = assert_close(out, want, key)
    _say(f"  max abs {mx:.2e} mean abs {mean:.2e}")


def test_page_permutation_is_bitwise_invisible():
    case = _case("small_q8")
    other = synth.repage(case, seed=1234)
    outs = []
    for c in (case, other):
        st = GpuState(c)
        st.append_step()
        outs.append(st.attention().cpu().numpy())
    assert np.array_equal(outs[0], outs[1])


def test_run_to_run_bitwise():
    case = _case("small_k4v4")
    st = GpuState(case)
    st.append_step()
    a = st.attention().cpu().numpy()
    b = st.attention().cpu().numpy()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("key", ["tiny_mixed", "small_q8", "verify_g6", "g5_d64_p16_q8"])
def test_mixed_equals_separate(key):
    """One mixed launch versus launches of its parts.  Chunk rows are computed
    by work items that depend only on their own sequence: bitwise equal.  Decode
    rows are cut into stream ranges that depend on the whole batch (and run on
    8-wave work-groups in a mixed launch, 4-wave ones in a decode-only launch),
    so the per-wave maxima that P and P*scale are rounded to fp16 against
    differ, as does the summation order: equal to 1e-3 (a quarter of the oracle
    tolerance), and each within the oracle tolerance (checked by the other
    tests)."""
    case = _case(key)
    st = GpuState(case)
    st.append_step()
    full = st.attention().cpu().numpy()
    chunks = [s for s in range(case.num_seqs) if case.q_len(s) > 16]
    decodes = [s for s in range(case.num_seqs) if case.q_len(s) <= 16]
    for seqs in (chunks, decodes, [decodes[-1], chunks[0]]):
        sub, rows = synth.subset(case, seqs)
        b = batch_of(sub.q_start, sub.prefix_len, sub.block_table)
        part = st.attention(batch=b, q=sub.q).cpu().numpy()
        for k, s in enumerate(seqs):
            r_full = np.arange(case.q_start[s], case.q_start[s + 1])
            r_part = np.arange(sub.q_start[k], sub.q_start[k + 1])
            if case.q_len(s) > 16:
                assert np.array_equal(part[r_part], full[r_full]), f"chunk seq {s} of {seqs}"
            else:
                d = float(np.abs(part[r_part] - full[r_full]).max())
                assert d <= 1e-3, f"decode seq {s} of {seqs}: {d:.3g}"


BOUNDARY_SEQS = [(0, 1), (1, 1), (30, 1), (31, 1), (32, 1), (510, 1), (511, 1), (512, 1),
                 (1023, 1), (1024, 1), (0, 2), (0, 33), (7, 65), (32750, 40), (511, 3)]


@pytest.mark.parametrize("kf,vf", [("q8", "q8"), ("q4", "q4")])
def test_split_and_tile_boundaries(kf, vf):
    case = synth.make_case("small_mixed", 21, device="cuda", seqs=BOUNDARY_SEQS, kf=kf, vf=vf,
                           ps=64)
    _say(f"boundaries {kf}/{vf}")
    st = GpuState(case)
    st.append_step()
    out = st.attention().cpu().numpy()
    kp, vp = oracle_pools(case)
    want = oracle_out(case, kp, vp)
    assert_close(out, want, f"boundaries {kf}{vf}")


def test_verify_rows_with_stage_aligned_limits():
    """Verify rows whose first row sees exactly m whole stages: the stage after
    them is visible only to the later rows, so a decode worker whose range
    starts there has slots with no visible key in its piece.  Many such
    segments of different lengths make the cut land there; the outputs must
    match the oracle (no NaN from an empty piece)."""
    rng = np.random.default_rng(51)
    seqs = [(32 * int(rng.integers(1, 40)) - 1, int(rng.integers(2, 6))) for _ in range(40)]
    seqs += [(int(rng.integers(0, 300)), 1) for _ in range(8)]
    case = synth.make_case("small_mixed", 52, device="cuda", seqs=seqs, ps=32, spare_pages=4)
    _say(f"stage-aligned verify rows: {len(seqs)} sequences, {case.num_rows} rows")
    st = GpuState(case)
    st.append_step()
    out = st.attention().cpu().numpy()
    assert np.isfinite(out).all()
    kp, vp = oracle_pools(case)
    assert_close(out, oracle_out(case, kp, vp), "stage-aligned verify rows")


def test_large_batch_tables_in_workspace():
    """More decode (> 96) and chunk (> 16) sequences than the kernel arguments
    hold: the launch-order tables are built on the device (plan_kernel); the
    outputs must still match the oracle, and a single decode row must match
    its own launch to 1e-3 (different cuts and work-group sizes round P
    differently)."""
    rng = np.random.default_rng(41)
    seqs = [(int(rng.integers(0, 400)), 1) for _ in range(110)]
    seqs += [(int(rng.integers(0, 200)), int(rng.integers(2, 24))) for _ in range(20)]
    order = rng.permutation(len(seqs))
    seqs = [seqs[i] for i in order]
    case = synth.make_case("small_mixed", 42, device="cuda", seqs=seqs, ps=16, spare_pages=8)
    _say(f"large batch: {len(seqs)} sequences, {case.num_rows} rows")
    st = GpuState(case)
    st.append_step()
    out = st.attention().cpu().numpy()
    kp, vp = oracle_pools(case)
    assert_close(out, oracle_out(case, kp, vp), "large batch")
    s = next(i for i in range(case.num_seqs) if case.q_len(i) == 1 and case.prefix_len[i] > 64)
    sub, rows = synth.subset(case, [s])
    one = st.attention(batch=batch_of(sub.q_start, sub.prefix_len, sub.block_table), q=sub.q).cpu().numpy()
    d = float(np.abs(one - out[rows]).max())
    assert d <= 1e-3, f"single decode row vs the large batch: {d:.3g}"


def _sweep_values(gen, n, hkv, d, kind):
    x = torch.randn((n, hkv, d), generator=gen, device="cuda")
    if kind == "outliers":
        x = x * torch.where(torch.rand((n, hkv, d), generator=gen, device="cuda") < 0.05, 20.0, 1.0)
    elif kind == "subnormal_scales":
        x = x * 1e-4
    elif kind == "underflow":
        x = x * 3e-7
    elif kind == "ties":
        x = torch.round(x * 8) / 2
    elif kind == "wide":
        x = x * torch.exp(torch.randn((n, hkv, 1), generator=gen, device="cuda") * 4)
        x = x.clamp(-65504, 65504)
    elif kind == "sparse":
        x = x * (torch.rand((n, hkv, d), generator=gen, device="cuda") < 0.05)
    x = x.to(torch.float16)
    if kind == "sparse":
        x[::7, :, :32] = 0          # whole zero blocks
        x[1::11, 0, 0] = -0.0       # negative zero
        x[2::13, 1, :] = 65504.0    # fp16 maximum
    return x


@pytest.mark.parametrize("fmt", ["q8", "q4"])
def test_append_random_sweep(fmt):
    """11M blocks per format (K and V, seven distributions of 49152 rows x 4
    heads x 4 blocks each), bit-exact against the oracle."""
    n, hkv, d = 49152, 4, 128
    kinds = ["normal", "outliers", "subnormal_scales", "underflow", "ties", "wide", "sparse"]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77)
    for kind in kinds:
        _say(f"sweep fmt={fmt} kind={kind}")
        case = synth.make_case("small_mixed", 31, device="cuda", seqs=[(0, n)], kf=fmt, vf=fmt,
                               ps=256, hkv=hkv, hq=hkv, d=d, with_values=False)
        case.k_new = _sweep_values(gen, n, hkv, d, kind)
        case.v_new = _sweep_values(gen, n, hkv, d, kind)
        case.k_prefix = [case.k_new[:0]]
        case.v_prefix = [case.v_new[:0]]
        st = GpuState(case, fill_prefix=False)
        st.append_step()
        torch.cuda.synchronize()
        gk, gv = st.pools_host()
        ok, ov = oracle_pools(case)
        assert np.array_equal(gk, ok), kind
        assert np.array_equal(gv, ov), kind
