"""Runs a synth case through the HIP library (via the C ABI binding) and
through the oracle, for the GPU parity tests and the smoke check."""

import numpy as np
import torch

import mixed_attention_block_amd as mab
import synth
from oracle import attention as oracle_attention
from oracle import cache as oracle_cache

MAX_ABS = 4e-3   # attention output tolerance vs the fp64 oracle (max abs error)
MEAN_ABS = 1e-3  # (mean abs error)
POISON = 0x7E    # unwritten bytes: every unwritten block has the fp16 NaN scale 0x7E7E


def layout_of(case):
    lay = case.layout
    return mab.make_layout(lay["num_q_heads"], lay["num_kv_heads"], lay["head_dim"],
                           lay["page_size"], lay["num_pages"], lay["k_format"], lay["v_format"])


def batch_of(q_start, prefix_len, block_table, device="cuda", flags=0):
    qs = np.ascontiguousarray(q_start, dtype=np.int32)
    pl = np.ascontiguousarray(prefix_len, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    return mab.BatchDesc(torch.from_numpy(qs).to(device), torch.from_numpy(pl).to(device),
                         torch.from_numpy(bt).to(device), qs, pl, flags=flags)


class GpuState:
    """Device pools for a case, filled with the prefix through kv_append_quant."""

    def __init__(self, case, fill_prefix=True):
        self.case = case
        self.layout = layout_of(case)
        lay = case.layout
        self.k_pool = torch.full((mab.kv_pool_bytes(self.layout, lay["k_format"]),), POISON,
                                 dtype=torch.uint8, device="cuda")
        self.v_pool = torch.full((mab.kv_pool_bytes(self.layout, lay["v_format"]),), POISON,
                                 dtype=torch.uint8, device="cuda")
        self.batch = batch_of(case.q_start, case.prefix_len, case.block_table)
        if fill_prefix:
            self.fill_prefix()

    def fill_prefix(self):
        qs, pl, k, v = synth.prefix_fill_batch(self.case)
        if k is None or k.shape[0] == 0:
            return
        # sequences without a prefix would have zero rows; drop them from the fill batch
        keep = [s for s in range(self.case.num_seqs) if self.case.prefix_len[s] > 0]
        rows = np.diff(qs)[keep]
        q_start = np.zeros(len(keep) + 1, np.int32)
        q_start[1:] = np.cumsum(rows)
        fill = batch_of(q_start, np.zeros(len(keep), np.int32), self.case.block_table[keep])
        mab.kv_append_quant(self.layout, fill, k.cuda().contiguous(), v.cuda().contiguous(),
                            self.k_pool, self.v_pool)

    def append_step(self):
        c = self.case
        mab.kv_append_quant(self.layout, self.batch, c.k_new.cuda().contiguous(),
                            c.v_new.cuda().contiguous(), self.k_pool, self.v_pool)

    def workspace(self, batch=None):
        n = mab.attention_workspace_bytes(self.layout, batch or self.batch)
        return torch.empty((max(n, 256),), dtype=torch.uint8, device="cuda")

    def attention(self, batch=None, q=None, workspace=None):
        c = self.case
        batch = batch or self.batch
        q = (c.q if q is None else q).cuda().contiguous()
        out = torch.full((q.shape[0], c.layout["num_q_heads"], c.layout["head_dim"]), float("nan"),
                         dtype=torch.float32, device="cuda")
        ws = self.workspace(batch) if workspace is None else workspace
        mab.mixed_attention_fwd(self.layout, batch, q, self.k_pool, self.v_pool, c.sm_scale, out, ws)
        return out

    def pools_host(self):
        lay = self.case.layout
        return (self.k_pool.cpu().numpy().reshape(oracle_cache.pool_shape(lay, lay["k_format"])),
                self.v_pool.cpu().numpy().reshape(oracle_cache.pool_shape(lay, lay["v_format"])))


def oracle_pools(case, seqs=None):
    """Oracle-encoded pools holding the prefix and the step rows of ``seqs``
    (all sequences by default); other pages keep the poison bytes."""
    lay = case.layout
    kp = oracle_cache.new_pool(lay, lay["k_format"], fill=POISON)
    vp = oracle_cache.new_pool(lay, lay["v_format"], fill=POISON)
    seqs = range(case.num_seqs) if seqs is None else seqs
    for s in seqs:
        p = int(case.prefix_len[s])
        r0, r1 = int(case.q_start[s]), int(case.q_start[s + 1])
        k = torch.cat([case.k_prefix[s].cpu(), case.k_new[r0:r1].cpu()]).numpy()
        v = torch.cat([case.v_prefix[s].cpu(), case.v_new[r0:r1].cpu()]).numpy()
        pos = np.arange(p + (r1 - r0))
        oracle_cache.write_tokens(kp, lay, lay["k_format"], case.block_table[s], pos, k)
        oracle_cache.write_tokens(vp, lay, lay["v_format"], case.block_table[s], pos, v)
    return kp, vp


def oracle_out(case, kp, vp, rows=None):
    return oracle_attention.attention(case.q.cpu().numpy(), kp, vp, case.layout, case.q_start,
                                      case.prefix_len, case.block_table, case.sm_scale, rows=rows)


def error_stats(got, want):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    return float(err.max()), float(err.mean())


def assert_close(got, want, what=""):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = error_stats(got, want)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, f"{what}: max abs {mx:.3g}, mean abs {mean:.3g}"
    return mx, mean
