"""Oracle for mixed-batch attention over a block-quantized, paged KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this package.
The product path (``mixed_attention_block_amd``) never imports it, and this
package never imports the product path: the two share no code, tables or
helpers.  Inputs come from ``synth`` (seeded generators that hold none of the
method's arithmetic) or from the tests themselves.

Everything here is plain, slow and written to be checked by eye:

* ``codec``      -- the 34-byte (8-bit) and 18-byte (4-bit) KV blocks, with the
                    encoder emulated step by step in IEEE binary32 and the
                    decoder in binary64.
* ``cache``      -- placement of blocks in page pools through a block table,
                    and gathering them back by logical position.
* ``attention``  -- causal softmax attention in binary64 over the dequantized
                    cache, for a mixed batch of chunk rows and decode rows.
* ``scheduler``  -- the fair scheduler that decides each step's rows (bounded
                    prefill chunk, decode first, decoder rotation, per-client
                    quota, SRTF, starving-decode preemption, near-done gate)
                    and builds the step's batch descriptor.

Source pages (cited by title and section):

* MBufo page -- "自研RDNA高併發推論引擎 以AI Max+ 395為範例" (lcz.me, topic 2938).
  Section 1 ("高併發（架構差異）") states that chunk rows and decode rows share
  one ForwardBatch and one attention kernel.  Section 2 ("提供更多壓縮精度")
  gives the KV modes table (q8: one f16 scale per 32 elements, 34 bytes; 4-bit
  values packed into 18 bytes), the codec bit-exactness statement, and the
  occupancy table ("佔用": bytes per position and per 262144-token session).
  Section 1 also holds the scheduler rules: the table "排程器保證什麼" and the
  fairness part "公平性：排隊不插隊".

Parity status of each function is given in its docstring.  Every function here
is pinned by a ``-m "not gpu"`` test against something other than itself
(closed forms, worked examples, brute force, a library routine on a special
case, or invariants), except where a docstring says "parity unpinned".
"""

from . import codec, cache, attention, scheduler  # noqa: F401
