"""C ABI checks that need no GPU: the library loads, exports every function
that include/mab.h declares, sizes pools and workspaces by the closed forms,
and rejects malformed calls with a status before touching the device."""

import ctypes
import os
import re

import numpy as np
import pytest

import mixed_attention_block_amd as mab
from oracle import cache as oracle_cache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mab.h")
FAKE_DEV = 0x7F0000000000  # never dereferenced on the host paths exercised here


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"kv_append_quant", "mixed_attention_fwd", "attention_workspace_bytes",
            "kv_pool_bytes", "kv_block_bytes", "mab_status_string", "mab_debug_status"} <= set(names)
    lib = ctypes.CDLL(mab.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_block_and_pool_sizes():
    assert mab.kv_block_bytes("q8") == 34 and mab.kv_block_bytes("q4") == 18
    assert mab.kv_block_bytes("f16") == 64
    assert mab.kv_block_bytes(99) == 0
    for kf, vf in (("q8", "q8"), ("q4", "q4"), ("q8", "q4"), ("f16", "f16")):
        lay = mab.make_layout(24, 4, 128, 256, 77, kf, vf)
        d = dict(num_q_heads=24, num_kv_heads=4, head_dim=128, page_size=256, num_pages=77)
        assert mab.kv_pool_bytes(lay, kf) == oracle_cache.pool_bytes(d, kf)
        assert mab.kv_pool_bytes(lay, vf) == oracle_cache.pool_bytes(d, vf)
    assert mab.kv_pool_bytes(mab.make_layout(24, 4, 100, 256, 77), "q8") == -1


def test_status_strings():
    for st in range(7):
        assert mab.mab_status_string(st)
    assert "unknown" in mab.mab_status_string(1234)


class _HostBatch:
    def __init__(self, q_start, prefix_len, max_pages=64, dev_ptrs=True, flags=0):
        self.qs = np.ascontiguousarray(q_start, np.int32)
        self.pl = np.ascontiguousarray(prefix_len, np.int32)
        ptr = FAKE_DEV if dev_ptrs else 0
        self.struct = mab.Batch(len(self.pl), int(self.qs[-1]), max_pages, flags, ptr, ptr, ptr,
                                self.qs.ctypes.data, self.pl.ctypes.data)


def _ws(layout, batch):
    return mab._lib().attention_workspace_bytes(ctypes.byref(layout), ctypes.byref(batch.struct))


def _decode_plan(ctxs, hkv, cus=256):
    """The decode stream's cut, restated from its rule: the segments (one per
    decode row and KV head, ceil(ctx/32) stages each) laid end to end, cut into
    equal ranges, one per worker (a wave), at most 8 per compute unit and at
    least 4 stages each; pieces per range = 1 + segment starts strictly inside
    it.  Returns (workers, range, pieces per worker at most)."""
    units = sum(hkv * -(-c // 32) for c in ctxs)
    wgs = min(8 * cus, max(1, units // 4))
    rng = -(-units // wgs)
    wgs = -(-units // rng)
    pieces = [1] * wgs
    x = 0
    for c in ctxs:
        for _ in range(hkv):
            if x % rng:
                pieces[x // rng] += 1
            x += -(-c // 32)
    return wgs, rng, max(pieces)


def _chunk_plan(q_len, hkv, group, cus=256):
    """Chunk tiles and key splits, restated from their rule: a tile is H heads
    (largest of 4, 2, 1 dividing G) x 256/H rows; the split F in 1..8 makes
    tiles*F fill whole rounds of one work-group per compute unit best."""
    h = 4 if group % 4 == 0 else 2 if group % 2 == 0 else 1
    rows = 256 // h
    tiles = -(-q_len // rows) * hkv * (group // h)
    slots = cus
    best, eff = 1, 0.0
    for f in range(1, 9):
        e = tiles * f / (-(-(tiles * f) // slots) * slots)
        if e > eff:
            best, eff = f, e
    return tiles, best, h, rows


def test_workspace_closed_form():
    lay = mab.make_layout(24, 4, 128, 256, 1000)
    b = _HostBatch([0, 1, 2, 50], [1000, 70000, 300], max_pages=400)  # 2 decode rows + 48-row chunk
    n = _ws(lay, b)
    wgs, rng, pmax = _decode_plan([1001, 70001], 4)
    assert (wgs, rng, pmax) == (1776, 5, 2)
    tiles, f, h, rows = _chunk_plan(48, 4, 6)
    assert (tiles, f, h, rows) == (12, 8, 2, 128)
    slots = wgs * pmax
    align = lambda x: -(-x // 256) * 256
    o = align(slots * 6 * 128 * 4)
    ml = align(slots * 6 * 8)
    cho = align(tiles * f * h * rows * 128 * 4)
    chml = align(tiles * f * h * rows * 8)
    dirs = align(2 * 4 * 16)
    assert n == o + ml + cho + chml + dirs


@pytest.mark.parametrize("fmt", ["f16", "q8"])
def test_workspace_closed_form_verify_rows(fmt):
    # A 5-row verify sequence at G = 6.  Over f16 pools it runs as decode
    # sub-rows of 16 // 6 = 2 rows (2, 2, 1: contexts prefix + 2, + 4, + 5),
    # so a partial holds 2 * 6 = 12 (row, head) slots.  Over quantized pools a
    # sequence with more than 16 // 6 rows takes two slot groups per wave:
    # sub-rows of 32 // 6 = 5 rows, one sub-row (context prefix + 5) and
    # 5 * 6 = 30 slots.  17 rows are the shortest prefill chunk.
    lay = mab.make_layout(24, 4, 128, 256, 1000, fmt, fmt)
    b = _HostBatch([0, 5, 6, 23], [300, 1000, 50], max_pages=400)
    n = _ws(lay, b)
    ctxs, T = ([302, 304, 305, 1001], 2) if fmt == "f16" else ([305, 1001], 5)
    wgs, rng, pmax = _decode_plan(ctxs, 4)
    tiles, f, h, rows = _chunk_plan(17, 4, 6)
    slots = wgs * pmax
    align = lambda x: -(-x // 256) * 256
    o = align(slots * T * 6 * 128 * 4)
    ml = align(slots * T * 6 * 8)
    cho = align(tiles * f * h * rows * 128 * 4) if f > 1 else 0
    chml = align(tiles * f * h * rows * 8) if f > 1 else 0
    dirs = align(len(ctxs) * 4 * 16)
    assert n == o + ml + cho + chml + dirs


def test_workspace_large_batch_holds_tables():
    """Batches beyond the kernel-argument tables (96 decode / 16 chunk
    sequences) keep the launch-order tables in the workspace."""
    lay = mab.make_layout(8, 2, 64, 16, 4000)
    small = _HostBatch(list(range(97)), [100] * 96, max_pages=16)
    big = _HostBatch(list(range(98)), [100] * 97, max_pages=16)
    assert _ws(lay, big) - _ws(lay, small) >= 4 * (4 * 97 + 1 + 1)


def test_workspace_closed_form_batch_invariant():
    """With MAB_BATCH_INVARIANT every decode segment (row x KV head) is cut
    into pieces of 512 keys (16 stages) from its own first key, one piece per
    worker: a partial slot per piece, whatever else is in the batch."""
    lay = mab.make_layout(24, 4, 128, 256, 1000)
    ctxs = [1, 511, 512, 513, 5000, 40000]
    b = _HostBatch(list(range(len(ctxs) + 1)), [c - 1 for c in ctxs], max_pages=200,
                   flags=mab.MAB_BATCH_INVARIANT)
    pieces = sum(4 * -(-(-(-c // 32)) // 16) for c in ctxs)
    align = lambda x: -(-x // 256) * 256
    assert _ws(lay, b) == align(pieces * 6 * 128 * 4) + align(pieces * 6 * 8) + align(len(ctxs) * 4 * 16)
    # the same rows in another batch take the same pieces: the slots add up
    b1 = _HostBatch([0, 1], [ctxs[-1] - 1], max_pages=200, flags=mab.MAB_BATCH_INVARIANT)
    assert _ws(lay, b1) == align(4 * 79 * 6 * 128 * 4) + align(4 * 79 * 6 * 8) + align(4 * 16)


@pytest.mark.parametrize("flags", [2, 3, 1 << 30, -1])
def test_unknown_batch_flags_are_refused(flags):
    lay = mab.make_layout(24, 4, 128, 256, 100)
    assert _ws(lay, _HostBatch([0, 1], [5], flags=flags)) == -2


@pytest.mark.parametrize("mutate,status", [
    (dict(num_q_heads=25), 2), (dict(head_dim=96), 3), (dict(head_dim=48), 2),
    (dict(page_size=24), 2), (dict(page_size=0), 2), (dict(k_format=4), 2),
    (dict(k_format=3), 3), (dict(v_format=3), 3),    # f16 on one side only
    (dict(num_q_heads=36, num_kv_heads=2), 3), (dict(num_pages=0), 2), (dict(reserved=1), 2),
])
def test_layout_errors(mutate, status):
    base = dict(num_q_heads=24, num_kv_heads=4, head_dim=128, page_size=256, num_pages=100,
                k_format=1, v_format=1, reserved=0)
    base.update(mutate)
    lay = mab.KVLayout(**base)
    assert _ws(lay, _HostBatch([0, 1], [5])) == -status


@pytest.mark.parametrize("q_start,prefix,max_pages,status", [
    ([0, 1, 1], [5, 6], 64, 2),          # a sequence with no rows
    ([1, 2], [5], 64, 2),                # q_start[0] != 0
    ([0, 1], [-1], 64, 2),               # negative prefix
    ([0, 1], [256 * 64], 64, 2),         # context beyond the block-table row
    ([0, 3, 2], [0, 0], 64, 2),          # decreasing q_start
])
def test_batch_errors(q_start, prefix, max_pages, status):
    lay = mab.make_layout(24, 4, 128, 256, 100)
    assert _ws(lay, _HostBatch(q_start, prefix, max_pages)) == -status


def test_null_and_alignment_and_workspace_errors():
    lib = mab._lib()
    lay = mab.make_layout(24, 4, 128, 256, 100)
    b = _HostBatch([0, 1, 2], [10, 20])
    L, B = ctypes.byref(lay), ctypes.byref(b.struct)
    d = FAKE_DEV
    assert lib.kv_append_quant(L, B, 0, d, d, d, None) == 1
    assert lib.kv_append_quant(L, B, d + 2, d, d, d, None) == 5
    assert lib.mixed_attention_fwd(L, B, d, d, d, 0.1, 0, d, 1 << 30, None) == 1
    assert lib.mixed_attention_fwd(L, B, d, d + 8, d, 0.1, d, d, 1 << 30, None) == 5
    assert lib.mixed_attention_fwd(L, B, d, d, d, 0.1, d, d, 16, None) == 4
    for bad_scale in (0.0, -0.1, float("inf"), float("nan")):  # softmax scale must be positive, finite
        assert lib.mixed_attention_fwd(L, B, d, d, d, bad_scale, d, d, 1 << 30, None) == 3
    nb = _HostBatch([0, 1, 2], [10, 20], dev_ptrs=False)
    assert lib.mixed_attention_fwd(L, ctypes.byref(nb.struct), d, d, d, 0.1, d, d, 1 << 30, None) == 1
    assert lib.kv_append_quant(None, B, d, d, d, d, None) == 1


def test_empty_batch_is_a_no_op():
    lib = mab._lib()
    lay = mab.make_layout(24, 4, 128, 256, 100)
    b = mab.Batch(0, 0, 1, 0, 0, 0, 0, 0, 0)
    assert lib.kv_append_quant(ctypes.byref(lay), ctypes.byref(b), 0, 0, 0, 0, None) == 0
    assert lib.mixed_attention_fwd(ctypes.byref(lay), ctypes.byref(b), 0, 0, 0, 0.1, 0, 0, 0, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(mab, "LIB_PATH", "/nonexistent/libmab.so")
    monkeypatch.setattr(mab, "_lib_handle", None)
    with pytest.raises(RuntimeError, match="missing"):
        mab.kv_block_bytes("q8")


def test_sequence_count_limit():
    """4096 sequences per batch (the launch-table limit) are accepted; one
    more is refused as unsupported before anything is enqueued."""
    lay = mab.make_layout(24, 4, 128, 256, 100)
    for n, ok in ((4096, True), (4097, False)):
        q_start = np.arange(n + 1, dtype=np.int32)  # one decode row each
        ws = _ws(lay, _HostBatch(q_start, np.full(n, 7, np.int32), 1))
        assert (ws > 0) if ok else ws == -3, (n, ws)
