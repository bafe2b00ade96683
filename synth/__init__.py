"""Seeded synthetic inputs for the mixed-batch quantized-KV attention step.

This module only draws inputs: batch structure (context lengths, chunk
position, shuffled physical pages) and fp16 values.  It holds none of the
method's arithmetic (no quantization, no attention), so both the HIP path and
the oracle can consume what it produces without sharing code.

Integer structure (contexts, page permutation, outlier channels) comes from
``numpy.random.Generator(PCG64(seed))`` and is the same on every device.
Values are N(0, 1) drawn in float32 by a ``torch.Generator`` seeded from the
same seed on the requested device, optionally multiplied by 20 on a fixed set
of "outlier" K channels, then rounded to fp16.  A case is therefore defined by
(name, seed, device); tests that compare two implementations give both the
same tensors.

Workloads (one attention layer each unless stated):

* ``tiny_mixed``      -- 4 q heads / 2 KV heads, head_dim 64, q8, page 16.  One
                         48-row chunk over an 80-token prefix plus decode rows
                         with contexts 100, 257, 511.
* ``decode16``        -- 16 decode rows, 24 q heads / 4 KV heads (GQA 6:1),
                         head_dim 128, q8, page 256, contexts uniform in
                         [1024, 32768], 2% of K channels x20.
* ``mixed16_chunk2k`` -- same heads and format: 16 decode rows with contexts in
                         [2048, 65536] plus a 2048-row chunk at position 131072
                         (of a 250000-token prompt); K outliers.
* ``decode16_f16``    -- the decode16 batch (same seed, same contexts) over an
                         unquantized f16 cache.
* ``verify16``        -- 16 verify rows of 4 tokens (speculative verify), the
                         last token's context uniform in [1024, 32768]; decode16's
                         heads and format, K outliers.
* ``long_q8`` / ``long_k4v4`` -- one decode row at context 262144.
* ``step_k4v4``       -- one layer of the full-step stress: K4V4, 16 decode rows
                         with contexts log-uniform in [512, 262144] and a
                         2048-row chunk at 131072; K outliers.  The step has 12
                         such layers sharing one batch; layer l draws its values
                         with ``value_seed = seed * 100 + l``.
* ``small_mixed``     -- a mid-size parity case: 24/4 heads, head_dim 128,
                         page 32, several chunks and decode rows with ragged
                         lengths (not a benchmark workload).
"""

from dataclasses import dataclass, field

import numpy as np
import torch

OUTLIER_FRACTION = 0.02
OUTLIER_GAIN = 20.0


@dataclass
class Case:
    name: str
    seed: int
    layout: dict               # num_q_heads, num_kv_heads, head_dim, page_size, num_pages, k_format, v_format
    q_start: np.ndarray        # int32 [S+1]
    prefix_len: np.ndarray     # int32 [S]   cached positions before the step's rows
    block_table: np.ndarray    # int32 [S, max_pages]; -1 where unused
    q: torch.Tensor            # fp16 [rows, Hq, D]
    k_new: torch.Tensor        # fp16 [rows, Hkv, D]   the step's own keys
    v_new: torch.Tensor        # fp16 [rows, Hkv, D]
    k_prefix: list = field(default_factory=list)   # per seq fp16 [P_s, Hkv, D]
    v_prefix: list = field(default_factory=list)
    sm_scale: float = 0.0      # a binary32 value
    outlier_channels: np.ndarray = None  # int [n, 2] of (kv head, dim)

    @property
    def num_seqs(self):
        return len(self.prefix_len)

    @property
    def num_rows(self):
        return int(self.q_start[-1])

    def q_len(self, s):
        return int(self.q_start[s + 1] - self.q_start[s])

    def context(self, s):
        """Keys visible to the last row of sequence s (prefix + own rows)."""
        return int(self.prefix_len[s]) + self.q_len(s)


def _spec(name):
    if name == "tiny_mixed":
        return dict(hq=4, hkv=2, d=64, kf="q8", vf="q8", ps=16, outliers=0.0,
                    seqs=[(80, 48), (99, 1), (256, 1), (510, 1)])
    if name == "small_mixed":
        return dict(hq=24, hkv=4, d=128, kf="q8", vf="q8", ps=32, outliers=OUTLIER_FRACTION,
                    seqs=[(0, 37), (5, 1), (300, 70), (1, 1), (777, 1), (64, 33), (2000, 1)])
    raise KeyError(name)


def _draw_seqs(name, rng):
    """(prefix_len, q_len) per sequence for the named workload."""
    if name in ("decode16", "decode16_f16"):
        ctx = rng.integers(1024, 32768, size=16, endpoint=True)
        return [(int(c) - 1, 1) for c in ctx]
    if name == "verify16":
        ctx = rng.integers(1024, 32768, size=16, endpoint=True)
        return [(int(c) - 4, 4) for c in ctx]
    if name == "mixed16_chunk2k":
        ctx = rng.integers(2048, 65536, size=16, endpoint=True)
        return [(131072, 2048)] + [(int(c) - 1, 1) for c in ctx]
    if name in ("long_q8", "long_k4v4"):
        return [(262144 - 1, 1)]
    if name == "step_k4v4":
        ctx = np.round(np.exp(rng.uniform(np.log(512), np.log(262144), size=16))).astype(np.int64)
        return [(131072, 2048)] + [(int(c) - 1, 1) for c in ctx]
    raise KeyError(name)


def _heads_format(name):
    if name in ("decode16", "verify16", "mixed16_chunk2k", "long_q8"):
        return dict(hq=24, hkv=4, d=128, kf="q8", vf="q8", ps=256)
    if name in ("long_k4v4", "step_k4v4"):
        return dict(hq=24, hkv=4, d=128, kf="q4", vf="q4", ps=256)
    if name == "decode16_f16":
        return dict(hq=24, hkv=4, d=128, kf="f16", vf="f16", ps=256)
    raise KeyError(name)


def _outlier_fraction(name):
    return 0.0 if name in ("long_q8", "long_k4v4") else OUTLIER_FRACTION


WORKLOADS = ("tiny_mixed", "small_mixed", "decode16", "decode16_f16", "verify16", "mixed16_chunk2k",
             "long_q8", "long_k4v4", "step_k4v4")


def make_case(name, seed, device="cpu", seqs=None, spare_pages=3, with_values=True,
              value_seed=None, **overrides):
    """Build a seeded case.  ``seqs`` (list of (prefix_len, q_len)) and the
    keyword overrides (hq, hkv, d, kf, vf, ps, outliers) allow custom shapes
    for edge-case tests.  The batch structure comes from ``seed``; values come
    from ``value_seed`` (default ``seed``), so the layers of one step share a
    batch and differ in their values."""
    rng = np.random.Generator(np.random.PCG64(seed))
    try:
        spec = _spec(name)
        drawn = spec.pop("seqs")
    except KeyError:
        spec = _heads_format(name)
        spec["outliers"] = _outlier_fraction(name)
        drawn = _draw_seqs(name, rng)
    spec.update(overrides)
    if seqs is not None:
        drawn = list(seqs)
    hq, hkv, d, ps = spec["hq"], spec["hkv"], spec["d"], spec["ps"]

    prefix_len = np.array([p for p, _ in drawn], dtype=np.int32)
    q_len = np.array([n for _, n in drawn], dtype=np.int32)
    q_start = np.zeros(len(drawn) + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(q_len)
    ctx = prefix_len.astype(np.int64) + q_len
    pages_per_seq = (ctx + ps - 1) // ps
    max_pages = int(max(1, pages_per_seq.max()))
    num_pages = int(pages_per_seq.sum()) + spare_pages
    perm = rng.permutation(num_pages).astype(np.int32)
    block_table = np.full((len(drawn), max_pages), -1, dtype=np.int32)
    cur = 0
    for s, npg in enumerate(pages_per_seq):
        block_table[s, :npg] = perm[cur:cur + npg]
        cur += npg

    n_out = int(round(spec["outliers"] * hkv * d))
    chan = rng.choice(hkv * d, size=n_out, replace=False) if n_out else np.zeros(0, np.int64)
    outlier_channels = np.stack([chan // d, chan % d], axis=1) if n_out else np.zeros((0, 2), np.int64)

    layout = dict(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
                  num_pages=num_pages, k_format=spec["kf"], v_format=spec["vf"])
    sm_scale = float(np.float32(1.0 / np.sqrt(d)))
    case = Case(name=name, seed=seed if value_seed is None else value_seed, layout=layout, q_start=q_start, prefix_len=prefix_len,
                block_table=block_table, q=None, k_new=None, v_new=None,
                sm_scale=sm_scale, outlier_channels=outlier_channels)
    if with_values:
        fill_values(case, device)
    return case


def _normal(gen, shape, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _k_values(gen, n, hkv, d, chan, device):
    x = _normal(gen, (n, hkv, d), device)
    if len(chan):
        x[:, torch.as_tensor(chan[:, 0], device=device), torch.as_tensor(chan[:, 1], device=device)] *= OUTLIER_GAIN
    return x.to(torch.float16)


def fill_values(case, device="cpu"):
    """Draw Q, the step's K/V and every sequence's prefix K/V."""
    lay = case.layout
    hq, hkv, d = lay["num_q_heads"], lay["num_kv_heads"], lay["head_dim"]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(case.seed) * 7919 + 17)
    rows = case.num_rows
    chan = case.outlier_channels
    case.q = _normal(gen, (rows, hq, d), device).to(torch.float16)
    case.k_new = _k_values(gen, rows, hkv, d, chan, device)
    case.v_new = _normal(gen, (rows, hkv, d), device).to(torch.float16)
    case.k_prefix, case.v_prefix = [], []
    for s in range(case.num_seqs):
        p = int(case.prefix_len[s])
        case.k_prefix.append(_k_values(gen, p, hkv, d, chan, device))
        case.v_prefix.append(_normal(gen, (p, hkv, d), device).to(torch.float16))
    return case


def prefix_fill_batch(case):
    """A batch that writes every sequence's cached prefix: sequence s gets rows
    for positions [0, prefix_len[s]).  Returns (q_start, prefix_len, k, v)
    with prefix_len all zero."""
    plen = case.prefix_len.astype(np.int64)
    q_start = np.zeros(case.num_seqs + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(plen)
    zeros = np.zeros(case.num_seqs, dtype=np.int32)
    k = torch.cat(case.k_prefix, dim=0) if case.k_prefix else None
    v = torch.cat(case.v_prefix, dim=0) if case.v_prefix else None
    return q_start, zeros, k, v


def repage(case, seed):
    """The same case with a different physical page assignment."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ctx = case.prefix_len.astype(np.int64) + np.diff(case.q_start)
    ps = case.layout["page_size"]
    pages_per_seq = (ctx + ps - 1) // ps
    perm = rng.permutation(case.layout["num_pages"]).astype(np.int32)
    bt = np.full_like(case.block_table, -1)
    cur = 0
    for s, npg in enumerate(pages_per_seq):
        bt[s, :npg] = perm[cur:cur + npg]
        cur += npg
    other = Case(**{**case.__dict__})
    other.block_table = bt
    return other


def subset(case, seqs):
    """The sub-batch holding only the sequences ``seqs`` (same block table rows,
    same pools), for the mixed == separate comparison."""
    seqs = list(seqs)
    q_len = np.diff(case.q_start)[seqs]
    q_start = np.zeros(len(seqs) + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(q_len)
    rows = np.concatenate([np.arange(case.q_start[s], case.q_start[s + 1]) for s in seqs])
    idx = torch.as_tensor(rows, device=case.q.device)
    other = Case(**{**case.__dict__})
    other.q_start = q_start
    other.prefix_len = case.prefix_len[seqs].copy()
    other.block_table = case.block_table[seqs].copy()
    other.q = case.q.index_select(0, idx)
    other.k_new = case.k_new.index_select(0, idx)
    other.v_new = case.v_new.index_select(0, idx)
    other.k_prefix = [case.k_prefix[s] for s in seqs]
    other.v_prefix = [case.v_prefix[s] for s in seqs]
    return other, rows


# --- serving-loop inputs ------------------------------------------------------

def token_values(seed, request_ids, positions, hq, hkv, d):
    """Query, key and value of the token at ``positions[i]`` of request
    ``request_ids[i]``: fp16 numpy arrays [n, Hq, D], [n, Hkv, D], [n, Hkv, D].
    Each token's values depend only on (seed, request, position), so a serving
    loop and a checker that see the same tokens in different batches draw the
    same numbers."""
    n = len(positions)
    q = np.empty((n, hq, d), np.float16)
    k = np.empty((n, hkv, d), np.float16)
    v = np.empty((n, hkv, d), np.float16)
    for i, (rid, pos) in enumerate(zip(request_ids, positions)):
        rng = np.random.default_rng([seed, int(rid), int(pos)])
        x = rng.standard_normal((hq + 2 * hkv, d), dtype=np.float32).astype(np.float16)
        q[i], k[i], v[i] = x[:hq], x[hq:hq + hkv], x[hq + hkv:]
    return q, k, v


SCENARIOS = ("chat16_long250k", "five_into_four")


def serving_arrivals(name, seed):
    """Arrivals (time in s, client, prompt tokens, token limit), sorted by time.

    * ``chat16_long250k`` -- 16 clients chatting (prompts uniform in
      [200, 2000] tokens, 64-256 output tokens, arrivals uniform over the
      first 50 ms) while a 250000-token prompt (16 output tokens) arrives at
      10 ms from client 16: the long-prompt-in-the-middle case.
    * ``five_into_four`` -- four slots, five requests: a 120000-token prompt
      and three chats at t = 0 (500-token prompts, 400 / 800 / 1600 output
      tokens), then a short request (300 tokens, 64 out) at 20 ms that must
      wait for a slot."""
    rng = np.random.default_rng(seed)
    if name == "chat16_long250k":
        out = [(float(rng.uniform(0, 0.05)), c, int(rng.integers(200, 2001)), int(rng.integers(64, 257)))
               for c in range(16)]
        out.append((0.01, 16, 250000, 16))
    elif name == "five_into_four":
        out = [(0.0, 0, 120000, 32), (0.0, 1, 500, 400), (0.0, 2, 500, 800), (0.0, 3, 500, 1600),
               (0.02, 4, 300, 64)]
    else:
        raise KeyError(name)
    return sorted(out, key=lambda a: (a[0], a[1]))
