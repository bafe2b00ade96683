"""Pins of the oracle's paged, mixed-batch attention: pure-Python brute force,
a library routine on the codec-free special case, closed forms, and the
invariants the pages state (mixed batch == separate passes; the physical page
assignment is invisible)."""

import math
import struct

import numpy as np
import pytest
import torch

import synth
from oracle import attention, cache, codec


def build_oracle_pools(case):
    """Oracle pools holding every sequence's prefix, then the step's rows (the
    append step runs before attention)."""
    lay = case.layout
    kp = cache.new_pool(lay, lay["k_format"])
    vp = cache.new_pool(lay, lay["v_format"])
    qs, pl, k, v = synth.prefix_fill_batch(case)
    if k is not None and k.shape[0]:
        cache.append(kp, vp, lay, qs, pl, case.block_table, k.cpu().numpy(), v.cpu().numpy())
    cache.append(kp, vp, lay, case.q_start, case.prefix_len, case.block_table,
                 case.k_new.cpu().numpy(), case.v_new.cpu().numpy())
    return kp, vp


def run_oracle(case, kp=None, vp=None, rows=None):
    if kp is None:
        kp, vp = build_oracle_pools(case)
    return attention.attention(case.q.cpu().numpy(), kp, vp, case.layout, case.q_start,
                               case.prefix_len, case.block_table, case.sm_scale, rows=rows)


# ---- pure-Python brute force (no numpy arithmetic, no vectorisation) --------------------

def _py_decode_block(raw, fmt):
    if fmt == "f16":  # 32 little-endian IEEE halves
        return list(struct.unpack("<32e", bytes(int(b) for b in raw)))
    d = struct.unpack("<e", bytes([int(raw[0]), int(raw[1])]))[0]
    vals = []
    if fmt == "q8":
        for byte in raw[2:]:
            c = int(byte)
            vals.append((c - 256 if c >= 128 else c) * d)
    else:
        for byte in raw[2:]:
            for nib in (int(byte) & 0xF, int(byte) >> 4):
                vals.append((nib - 16 if nib >= 8 else nib) * d)
    return vals


def _py_token(pool, fmt, table_row, ps, t, g, nblk):
    page = int(table_row[t // ps])
    out = []
    for b in range(nblk):
        out.extend(_py_decode_block(pool[page, g, t % ps, b], fmt))
    return out


def brute_force(case, kp, vp):
    lay = case.layout
    hq, hkv, dim, ps = lay["num_q_heads"], lay["num_kv_heads"], lay["head_dim"], lay["page_size"]
    grp = hq // hkv
    q = case.q.cpu().numpy().astype(float).tolist()
    out = [[None] * hq for _ in range(case.num_rows)]
    for s in range(case.num_seqs):
        for i in range(case.q_len(s)):
            r = int(case.q_start[s]) + i
            t = int(case.prefix_len[s]) + i
            for h in range(hq):
                g = h // grp
                z = []
                for j in range(t + 1):
                    kj = _py_token(kp, lay["k_format"], case.block_table[s], ps, j, g, dim // 32)
                    z.append(case.sm_scale * sum(a * b for a, b in zip(q[r][h], kj)))
                m = max(z)
                w = [math.exp(x - m) for x in z]
                acc = [0.0] * dim
                for j in range(t + 1):
                    vj = _py_token(vp, lay["v_format"], case.block_table[s], ps, j, g, dim // 32)
                    acc = [a + w[j] * b for a, b in zip(acc, vj)]
                tot = sum(w)
                out[r][h] = [a / tot for a in acc]
    return np.array(out, dtype=np.float64)


@pytest.mark.parametrize("kf,vf", [("q8", "q8"), ("q4", "q4"), ("q8", "q4"), ("q4", "q8"), ("f16", "f16")])
def test_brute_force_tiny(kf, vf):
    case = synth.make_case("tiny_mixed", seed=5, seqs=[(5, 3), (0, 2), (20, 1), (16, 1), (31, 1)],
                           hq=4, hkv=2, d=64, ps=16, kf=kf, vf=vf, outliers=0.05)
    kp, vp = build_oracle_pools(case)
    got = run_oracle(case, kp, vp)
    want = brute_force(case, kp, vp)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_codec_free_case_matches_torch_sdpa():
    rng = np.random.default_rng(3)
    hq, hkv, dim, length, n = 6, 2, 64, 70, 9
    q = rng.standard_normal((n, hq, dim)).astype(np.float16)
    k = rng.standard_normal((length, hkv, dim)).astype(np.float16).astype(np.float64)
    v = rng.standard_normal((length, hkv, dim)).astype(np.float16).astype(np.float64)
    pos = np.array([0, 3, 17, 40, 60, 61, 62, 68, 69])
    sm = float(np.float32(1 / np.sqrt(dim)))
    got = attention.attend(q, k, v, pos, sm)
    tq = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)[None]            # [1,Hq,n,D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, 0)[None]
    mask = torch.from_numpy(np.arange(length)[None, :] <= pos[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=sm)
    np.testing.assert_allclose(got, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-10)


def test_f16_cache_matches_torch_sdpa_on_the_raw_values():
    # The unquantized f16 format through the whole paged, mixed-batch path
    # (append, block table, causal chunk rows, decode rows) equals a library
    # attention over the case's own fp16 K/V, with no codec in between.
    case = synth.make_case("tiny_mixed", seed=9, seqs=[(40, 24), (0, 5), (77, 1), (15, 1)],
                           hq=6, hkv=2, d=64, ps=16, kf="f16", vf="f16", outliers=0.05)
    got = run_oracle(case)
    lay = case.layout
    hq, hkv = lay["num_q_heads"], lay["num_kv_heads"]
    want = np.empty_like(got)
    for s in range(case.num_seqs):
        r0, r1 = int(case.q_start[s]), int(case.q_start[s + 1])
        k = torch.cat([case.k_prefix[s].cpu(), case.k_new[r0:r1].cpu()]).double()   # [L, Hkv, D]
        v = torch.cat([case.v_prefix[s].cpu(), case.v_new[r0:r1].cpu()]).double()
        q = case.q[r0:r1].cpu().double()
        pos = int(case.prefix_len[s]) + np.arange(r1 - r0)
        mask = torch.from_numpy(np.arange(k.shape[0])[None, :] <= pos[:, None])
        ref = torch.nn.functional.scaled_dot_product_attention(
            q.permute(1, 0, 2)[None], k.permute(1, 0, 2).repeat_interleave(hq // hkv, 0)[None],
            v.permute(1, 0, 2).repeat_interleave(hq // hkv, 0)[None], attn_mask=mask, scale=case.sm_scale)
        want[r0:r1] = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


def test_closed_forms():
    rng = np.random.default_rng(4)
    hq, hkv, dim, length = 4, 2, 32, 50
    k = rng.standard_normal((length, hkv, dim))
    v = rng.standard_normal((length, hkv, dim))
    q = rng.standard_normal((3, hq, dim)).astype(np.float16)
    # one visible key: the output is that key's value
    out = attention.attend(q[:1], k, v, np.array([0]), 0.125)
    for h in range(hq):
        assert np.array_equal(out[0, h], v[0, h // 2])
    # zero query: the mean of the visible values
    out = attention.attend(np.zeros((1, hq, dim), np.float16), k, v, np.array([29]), 0.125)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], v[:30, h // 2].mean(axis=0), rtol=0, atol=1e-13)
    # identical keys: the mean of the visible values whatever the query
    kk = np.repeat(k[:1], length, axis=0)
    out = attention.attend(q[1:2], kk, v, np.array([44]), 0.125)
    for h in range(hq):
        np.testing.assert_allclose(out[0, h], v[:45, h // 2].mean(axis=0), rtol=0, atol=1e-13)


def test_mixed_batch_equals_separate_passes():
    case = synth.make_case("tiny_mixed", seed=1)
    kp, vp = build_oracle_pools(case)
    full = run_oracle(case, kp, vp)
    for seqs in ([0], [1, 2, 3], [2], [3, 0]):
        sub, rows = synth.subset(case, seqs)
        part = attention.attention(sub.q.cpu().numpy(), kp, vp, sub.layout, sub.q_start,
                                   sub.prefix_len, sub.block_table, sub.sm_scale)
        assert np.array_equal(part, full[rows])


def test_page_permutation_is_invisible():
    case = synth.make_case("tiny_mixed", seed=2)
    other = synth.repage(case, seed=99)
    assert not np.array_equal(case.block_table, other.block_table)
    a = run_oracle(case)
    b = run_oracle(other)
    assert np.array_equal(a, b)


def test_cache_placement_by_hand():
    case = synth.make_case("tiny_mixed", seed=3, seqs=[(40, 2), (0, 5)], d=64, ps=16)
    kp, vp = build_oracle_pools(case)
    lay = case.layout
    ks = [torch.cat([case.k_prefix[s], case.k_new[case.q_start[s]:case.q_start[s + 1]]]).numpy()
          for s in range(case.num_seqs)]
    written = set()
    for s in range(case.num_seqs):
        for t in range(case.context(s)):
            page, slot = int(case.block_table[s][t // 16]), t % 16
            written.add(page)
            for g in range(2):
                want = codec.encode_blocks(ks[s][t, g].reshape(2, 32), "q8")
                assert np.array_equal(kp[page, g, slot], want)
    for page in range(lay["num_pages"]):
        if page not in written:                            # untouched pages keep the poison
            assert (kp[page] == 0x7E).all() and (vp[page] == 0x7E).all()


def test_row_sampling_matches_full():
    case = synth.make_case("tiny_mixed", seed=4)
    kp, vp = build_oracle_pools(case)
    full = run_oracle(case, kp, vp)
    rows = [0, 17, 47, 48, 50]
    part = run_oracle(case, kp, vp, rows=rows)
    assert np.array_equal(part[rows], full[rows])
    assert np.isnan(part[1]).all()


def test_pool_size_closed_form():
    # pages x KV heads x page slots x blocks per token x block bytes (the pool
    # layout of the paged cache; 34/18/64-byte blocks from the modes table)
    for fmt, bb in (("q8", 34), ("q4", 18), ("f16", 64)):
        lay = dict(num_q_heads=24, num_kv_heads=4, head_dim=128, page_size=256, num_pages=7)
        assert cache.pool_shape(lay, fmt) == (7, 4, 256, 4, bb)
        assert cache.pool_bytes(lay, fmt) == 7 * 4 * 256 * 4 * bb
        assert cache.new_pool(lay, fmt).nbytes == cache.pool_bytes(lay, fmt)
