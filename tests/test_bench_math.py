"""The benchmark's accounting, checked on the CPU: bytes per cached position
(against the KV modes table of the MBufo page, section 2) and the chunk flop
count (prefill chunks only, every visible (row, key) pair once)."""

import numpy as np

import bench
import synth


def test_bytes_per_position_match_the_kv_modes_table():
    # 4 KV heads x 128 dims per layer: 2048 (fp16), 1088 (q8), 832 (K8V4), 576 (K4V4) bytes
    lay = dict(num_kv_heads=4, head_dim=128)
    for kf, vf, want in (("f16", "f16", 2048), ("q8", "q8", 1088), ("q8", "q4", 832), ("q4", "q4", 576)):
        assert bench.kv_bytes_per_position(dict(lay, k_format=kf, v_format=vf)) == want


def test_chunk_flops_count_visible_pairs_of_prefill_chunks_only():
    seqs = [(100, 17), (50, 16), (7, 1), (0, 40)]   # a 17-row chunk, a verify row, a decode row, a chunk
    case = synth.make_case("tiny_mixed", 3, seqs=seqs, with_values=False)
    lay = case.layout
    pairs = 0
    for s, (prefix, q_len) in enumerate(seqs):
        if q_len <= 16:
            continue  # decode and verify rows are counted as KV bytes, not matrix-core flops
        for i in range(q_len):
            pairs += prefix + i + 1   # keys 0 .. prefix + i
    assert bench.chunk_flops(case) == 4 * lay["head_dim"] * lay["num_q_heads"] * pairs
