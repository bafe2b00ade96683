"""Oracle: the paged KV cache (test infrastructure only).

A pool holds ``num_pages`` pages.  One page holds ``page_size`` consecutive
token positions of one sequence for every KV head; within a page, the data of
one KV head is contiguous.  Byte layout of a pool::

    pool[num_pages][num_kv_heads][page_size][head_dim / 32][B]      B = 34, 18 or 64 (f16)

The token at absolute position t of sequence s, KV head g, block b lives at
``pool[block_table[s][t // page_size], g, t % page_size, b]``.  Physical page
ids are arbitrary: the attention result must not depend on them.

The pages describe a paged, blocked cache but not its byte order; the order
above is this design's choice (one contiguous run per page and KV head), and
the product path uses the same byte order so that pools can be compared byte
for byte.

Pinned by: the page-permutation invariance test (output independent of the
physical ids), the pool-size closed forms, and the append/gather round trip.
"""

import numpy as np

from . import codec


def pool_shape(layout, fmt):
    """Shape of a byte pool: [num_pages, Hkv, page_size, head_dim/32, B]."""
    return (
        layout["num_pages"],
        layout["num_kv_heads"],
        layout["page_size"],
        layout["head_dim"] // codec.VALUES_PER_BLOCK,
        codec.block_bytes(fmt),
    )


def pool_bytes(layout, fmt):
    """Total bytes of one pool (K or V) = num_pages*Hkv*page_size*(D/32)*B."""
    return int(np.prod(pool_shape(layout, fmt)))


def new_pool(layout, fmt, fill=0x7E):
    """A pool filled with ``fill``.  The default 0x7E makes every unwritten
    block's scale the fp16 NaN 0x7E7E, so reading one poisons the result."""
    return np.full(pool_shape(layout, fmt), fill, dtype=np.uint8)


def write_tokens(pool, layout, fmt, table_row, positions, x):
    """Encode ``x[n, Hkv, D]`` (fp16) and store token i at ``positions[i]``
    of the sequence whose block-table row is ``table_row``."""
    ps = layout["page_size"]
    hkv, d = layout["num_kv_heads"], layout["head_dim"]
    x = np.asarray(x, dtype=np.float16)
    positions = np.asarray(positions, dtype=np.int64)
    assert x.shape == (len(positions), hkv, d)
    blocks = codec.encode_blocks(x.reshape(len(positions), hkv, d // 32, 32), fmt)
    pages = np.asarray(table_row, dtype=np.int64)[positions // ps]
    slots = positions % ps
    for g in range(hkv):
        pool[pages, g, slots] = blocks[:, g]


def gather_tokens(pool, layout, fmt, table_row, length):
    """Dequantized keys or values of positions [0, length): float64 [length, Hkv, D]."""
    ps = layout["page_size"]
    hkv, d = layout["num_kv_heads"], layout["head_dim"]
    pos = np.arange(length, dtype=np.int64)
    pages = np.asarray(table_row, dtype=np.int64)[pos // ps]
    slots = pos % ps
    out = np.empty((length, hkv, d), dtype=np.float64)
    for g in range(hkv):
        out[:, g] = codec.decode_blocks(pool[pages, g, slots], fmt).reshape(length, d)
    return out


def append(k_pool, v_pool, layout, q_start, prefix_len, block_table, k_new, v_new):
    """The append step: row i of sequence s is written at position
    ``prefix_len[s] + i`` (its own position), keys to ``k_pool`` and values to
    ``v_pool``, each in its own format."""
    for s in range(len(prefix_len)):
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        if r1 == r0:
            continue
        pos = int(prefix_len[s]) + np.arange(r1 - r0)
        write_tokens(k_pool, layout, layout["k_format"], block_table[s], pos, k_new[r0:r1])
        write_tokens(v_pool, layout, layout["v_format"], block_table[s], pos, v_new[r0:r1])
