"""Oracle: causal softmax attention of a mixed batch over the paged cache, in
binary64 (test infrastructure only).

MBufo page ("自研RDNA高併發推論引擎 以AI Max+ 395為範例"), section 1: the rows
of a bounded prefill chunk and the single-token decode rows ride in one
ForwardBatch and go through the same attention.  A chunk row attends its whole
cached prefix and, causally, the chunk rows up to and including itself; a
decode row attends every cached position of its sequence.  Both are one rule:

    row i of sequence s sits at position t = prefix_len[s] + i and attends the
    keys at positions 0 .. t of sequence s.

For a query head h the KV head is g = h // (Hq / Hkv) (consecutive grouping).
With K_hat and V_hat the dequantized cache (see ``codec``):

    z_j  = sm_scale * sum_d Q[r, h, d] * K_hat[s, j, g, d]       j = 0 .. t
    O    = sum_j exp(z_j - max z) V_hat[s, j, g, :] / sum_j exp(z_j - max z)

``sm_scale`` is the binary32 value handed to the kernel, widened to binary64.
The row's own key is read back from the cache, that is quantized: the append
step runs before attention in the same step.  No row depends on another row, so
the mixed-batch result is the concatenation of per-row results.

Pinned by: pure-Python brute force on tiny inputs; the codec-free special case
against ``torch.nn.functional.scaled_dot_product_attention`` in float64; closed
forms (one visible key, zero query, identical keys); mixed batch == chunk-only
and decode-only batches; invariance under permutation of physical pages.
"""

import numpy as np

from . import cache

_ROW_BLOCK = 64  # rows per matmul block; only bounds memory, not arithmetic order


def attend(q, k, v, positions, sm_scale):
    """Attention of rows ``q[n, Hq, D]`` over dense ``k, v[L, Hkv, D]``.

    Row i attends keys 0 .. positions[i].  Returns float64 [n, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    positions = np.asarray(positions, dtype=np.int64)
    n, hq, d = q.shape
    length, hkv, _ = k.shape
    assert hq % hkv == 0 and positions.shape == (n,)
    assert n == 0 or (positions.min() >= 0 and positions.max() < length)
    group = hq // hkv
    scale = float(np.float32(sm_scale))
    out = np.empty((n, hq, d), dtype=np.float64)
    key_pos = np.arange(length)
    for h in range(hq):
        g = h // group
        for r0 in range(0, n, _ROW_BLOCK):
            r1 = min(n, r0 + _ROW_BLOCK)
            z = scale * (q[r0:r1, h, :] @ k[:, g, :].T)           # [rows, L]
            visible = key_pos[None, :] <= positions[r0:r1, None]
            z = np.where(visible, z, -np.inf)
            m = np.max(z, axis=1, keepdims=True)
            p = np.exp(z - m)                                      # masked -> 0
            out[r0:r1, h, :] = (p @ v[:, g, :]) / np.sum(p, axis=1, keepdims=True)
    return out


def attention(q, k_pool, v_pool, layout, q_start, prefix_len, block_table, sm_scale,
              rows=None):
    """Mixed-batch attention over the paged, quantized cache.

    ``q``: fp16 [num_rows, Hq, D]; ``q_start``: int [S+1]; ``prefix_len``:
    int [S]; ``block_table``: int [S, max_pages].  Returns float64
    [num_rows, Hq, D].  With ``rows`` (global row indices), only those rows
    are computed and the others are NaN.
    """
    q = np.asarray(q)
    num_rows, hq, d = q.shape
    out = np.full((num_rows, hq, d), np.nan, dtype=np.float64)
    wanted = None if rows is None else set(int(r) for r in rows)
    for s in range(len(prefix_len)):
        r0, r1 = int(q_start[s]), int(q_start[s + 1])
        sel = [r for r in range(r0, r1) if wanted is None or r in wanted]
        if not sel:
            continue
        length = int(prefix_len[s]) + (r1 - r0)
        kh = cache.gather_tokens(k_pool, layout, layout["k_format"], block_table[s], length)
        vh = cache.gather_tokens(v_pool, layout, layout["v_format"], block_table[s], length)
        sel = np.asarray(sel)
        pos = int(prefix_len[s]) + (sel - r0)
        out[sel] = attend(q[sel], kh, vh, pos, sm_scale)
    return out
