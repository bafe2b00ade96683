"""Oracle: the 32-value KV block codec (test infrastructure only).

MBufo page ("自研RDNA高併發推論引擎 以AI Max+ 395為範例"), section 2, KV modes
table: the q8 mode keeps one f16 scale for every 32 elements, 34 bytes per
block; the 4-bit modes pack 32 values into 18 bytes.  The same section says the
blocked modes are bit-exact at the codec level, so the encoder below is an
exact, step-by-step emulation of one fixed arithmetic:

    xf    = float32(x)                       (x is fp16; exact)
    amax  = max_i |xf_i|
    s     = fl32(amax / QMAX)                QMAX = 127 (8-bit) or 7 (4-bit);
                                             IEEE binary32 divide, nearest-even
    q_i   = clamp(rint_even(fl32(xf_i / s)), -QMAX, QMAX)
    d     = fp16_rne(s)                      gradual underflow, no flush
    bytes = [d as little-endian fp16] + payload

An all-zero block stores d = +0 and q = 0.  The payload of the 8-bit block is
the 32 values as two's-complement bytes.  The payload of the 4-bit block is 16
bytes; byte j holds value 2j in its low nibble and value 2j+1 in its high
nibble, each as a two's-complement nibble.  Decoding is x_hat_i = q_i * d.

The unquantized f16 mode of the same table (2 bytes per value; 2048 bytes per
position in the occupancy table) is stored in the same block structure: a
"block" is the 32 values themselves, 64 bytes of little-endian IEEE halves, with
no scale; encoding and decoding are the identity on the fp16 values.

Readings taken where the page is silent (each also listed in the design notes):
the block runs along head_dim of one token and one KV head; the quantizing
scale is the binary32 value s while the stored (and decoding) scale is its
fp16 rounding; rounding to integer is half-to-even; the scale comes first in
the block; 4-bit values are two's-complement nibbles, even element low.

numpy's float32 arithmetic is IEEE binary32 with round-to-nearest-even, its
``rint`` rounds half to even and its float32 -> float16 cast rounds to nearest
even with subnormals; the tests pin each of these against independent exact
arithmetic (``fractions.Fraction`` and ``struct``'s 'e' format).
"""

import numpy as np

VALUES_PER_BLOCK = 32

#: format name -> (bytes per block, largest code magnitude; None: unquantized)
_FORMATS = {
    "q8": (2 + 32, 127),
    "q4": (2 + 16, 7),
    "f16": (2 * 32, None),
}


def block_bytes(fmt):
    """Bytes of one 32-value block: 34 for q8, 18 for q4 (MBufo page, section 2,
    KV modes table), 64 for the unquantized f16 mode (2 bytes per value).
    Pinned by the closed forms in the modes table and the occupancy table."""
    return _FORMATS[fmt][0]


def qmax(fmt):
    """Largest code magnitude: 127 for 8-bit blocks, 7 for 4-bit blocks."""
    return _FORMATS[fmt][1]


def bytes_per_position(num_kv_heads, head_dim, k_fmt, v_fmt):
    """KV bytes per token position per layer (K plus V).

    MBufo page, section 2, occupancy table ("佔用"): with 4 KV heads of 128
    dims this is 2048 (f16), 1088 (q8), 832 (one side 4-bit) and 576 (K4V4).
    """
    total = 0
    for fmt in (k_fmt, v_fmt):
        if fmt == "f16":
            total += num_kv_heads * head_dim * 2
        else:
            assert head_dim % VALUES_PER_BLOCK == 0
            total += num_kv_heads * (head_dim // VALUES_PER_BLOCK) * block_bytes(fmt)
    return total


def session_bytes(context, layers, num_kv_heads, head_dim, k_fmt, v_fmt):
    """KV bytes held by one session of ``context`` positions over ``layers``
    attention layers (MBufo page, section 2 occupancy table, -c 262144 with 12
    attention layers: 6.44 / 3.42 / 2.62 / 1.81 GB, GB = 1e9 bytes)."""
    return context * layers * bytes_per_position(num_kv_heads, head_dim, k_fmt, v_fmt)


def encode_blocks(x, fmt):
    """Encode fp16 values ``x[..., 32]`` into blocks ``uint8[..., B]``.

    Follows the arithmetic in the module docstring in the order written there.
    Pinned by: worked examples in ``tests/golden``; exact-rational checks of
    the binary32 divide and the fp16 rounding; the invariants max|q| == QMAX,
    |xf/s - q| <= 1/2 and decode(encode) within half a step.
    """
    x = np.asarray(x)
    assert x.dtype == np.float16 and x.shape[-1] == VALUES_PER_BLOCK
    nbytes, qm = _FORMATS[fmt]
    if fmt == "f16":  # the values themselves, little-endian halves
        return np.ascontiguousarray(x).astype("<f2").view(np.uint8).reshape(x.shape[:-1] + (nbytes,))
    qm32 = np.float32(qm)

    xf = x.astype(np.float32)                               # exact widening
    amax = np.max(np.abs(xf), axis=-1)                      # float32
    s = np.divide(amax, qm32, dtype=np.float32)             # fl32(amax / QMAX)
    nonzero = amax > np.float32(0)
    s_safe = np.where(nonzero, s, np.float32(1)).astype(np.float32)
    r = np.divide(xf, s_safe[..., None], dtype=np.float32)  # fl32(x / s)
    q = np.rint(r)                                          # half to even
    q = np.clip(q, -qm32, qm32)
    q = np.where(nonzero[..., None], q, np.float32(0)).astype(np.int8)
    d = s.astype(np.float16)                                # fp16 RNE, subnormals kept
    d = np.where(nonzero, d, np.float16(0)).astype(np.float16)

    out = np.empty(x.shape[:-1] + (nbytes,), dtype=np.uint8)
    dbits = d.view(np.uint16)
    out[..., 0] = (dbits & 0xFF).astype(np.uint8)           # little-endian scale
    out[..., 1] = (dbits >> 8).astype(np.uint8)
    qb = q.view(np.uint8)                                   # two's complement
    if fmt == "q8":
        out[..., 2:] = qb
    else:
        lo = qb[..., 0::2] & 0x0F
        hi = qb[..., 1::2] & 0x0F
        out[..., 2:] = lo | (hi << 4)
    return out


def decode_codes(blocks, fmt):
    """Split blocks ``uint8[..., B]`` into (scale fp16[...], codes int8[..., 32])."""
    blocks = np.asarray(blocks, dtype=np.uint8)
    nbytes, _ = _FORMATS[fmt]
    assert blocks.shape[-1] == nbytes and fmt != "f16"
    dbits = blocks[..., 0].astype(np.uint16) | (blocks[..., 1].astype(np.uint16) << 8)
    d = dbits.view(np.float16)
    payload = blocks[..., 2:]
    if fmt == "q8":
        q = payload.view(np.int8)
    else:
        lo = (payload & 0x0F).astype(np.int16)
        hi = (payload >> 4).astype(np.int16)
        lo = np.where(lo >= 8, lo - 16, lo)                 # two's-complement nibble
        hi = np.where(hi >= 8, hi - 16, hi)
        q = np.empty(payload.shape[:-1] + (VALUES_PER_BLOCK,), dtype=np.int8)
        q[..., 0::2] = lo
        q[..., 1::2] = hi
    return d, q


def decode_blocks(blocks, fmt):
    """Decode blocks ``uint8[..., B]`` to float64 ``[..., 32]``: x_hat = q * d.

    The product of a code of at most 7 magnitude bits and an 11-bit fp16
    significand is exact in binary64 (and in binary32).  Pinned by the worked
    examples and by the half-step bound against the encoder's input.
    """
    if fmt == "f16":
        blocks = np.ascontiguousarray(np.asarray(blocks, dtype=np.uint8))
        assert blocks.shape[-1] == block_bytes("f16")
        return blocks.view("<f2").astype(np.float64)
    d, q = decode_codes(blocks, fmt)
    return q.astype(np.float64) * d.astype(np.float64)[..., None]
