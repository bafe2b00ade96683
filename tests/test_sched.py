"""The library's step scheduler (mab_sched_*, host C++) against the scheduler
oracle, CPU only: every submit status and every tick's batch (kind, request
ids, q_start, prefix_len, block-table rows, emit and finished flags) must be
identical on the hand-derived traces and on seeded random traces."""

import ctypes

import numpy as np
import pytest

import mixed_attention_block_amd as mab
import test_oracle_scheduler as ts
from oracle import scheduler as oracle_sched


def _cfg_args(cfg):
    c = dict(cfg)
    c.setdefault("max_decode_rows", 0)
    return c


def _as_rows(step, width):
    """A library Step in the oracle's form."""
    if step is None:
        return None
    q = np.diff(step.q_start)
    return dict(kind=step.kind, ids=[int(x) for x in step.request_id],
                prefix_len=[int(x) for x in step.prefix_len], q_len=[int(x) for x in q],
                emit=[int(x) for x in step.emit], finished=[int(x) for x in step.finished],
                block_table=[[int(x) for x in row] for row in step.block_table])


def _oracle_rows(st):
    if st is None:
        return None
    return dict(st)


def _compare(cfg, arrivals):
    o = oracle_sched.Scheduler(**cfg)
    c = mab.Scheduler(**_cfg_args(cfg))
    t = 0
    while True:
        for client, prompt, limit in (arrivals[t] if t < len(arrivals) else []):
            assert c.submit(client, prompt, limit) == o.submit(client, prompt, limit), (t, client, prompt, limit)
        want = _oracle_rows(o.step())
        got = _as_rows(c.step(), cfg["max_pages_per_seq"])
        assert got == want, f"tick {t}: {got} != {want}"
        t += 1
        if want is None and t >= len(arrivals) and not o.any_pending():
            return t
        assert t < 20000


@pytest.mark.parametrize("trace", ts.golden_traces(), ids=lambda t: t["name"])
def test_golden_trace(trace):
    got, pages = ts.run_golden(trace, make=_LibAsOracle)
    assert got == trace["steps"]
    assert pages == trace["pages"]


class _LibAsOracle:
    """The library scheduler behind the oracle's interface (for the golden runner)."""

    def __init__(self, **cfg):
        self.width = cfg["max_pages_per_seq"]
        self.s = mab.Scheduler(**_cfg_args(cfg))

    def submit(self, client, prompt, limit):
        return self.s.submit(client, prompt, limit)

    def step(self):
        return _as_rows(self.s.step(), self.width)


@pytest.mark.parametrize("seed", range(200))
def test_random_traces_match_oracle(seed):
    rng = np.random.default_rng(5000 + seed)
    cfg = ts.random_config(rng)
    if seed % 4 == 0:
        cfg["num_pages"] = int(rng.integers(8, 30))   # admission blocked by pages
        cfg["max_pages_per_seq"] = cfg["num_pages"]
    arrivals = ts.random_arrivals(rng, int(rng.integers(20, 150)), int(rng.integers(1, 6)))
    _compare(cfg, arrivals)


def test_max_decode_rows_zero_means_sessions():
    cfg = dict(sessions=3, prefill_chunk=4, max_pending_per_client=4, near_done_gate=2, page_size=4,
               num_pages=64, max_pages_per_seq=16)
    rng = np.random.default_rng(9)
    arrivals = ts.random_arrivals(rng, 60, 3)
    o = oracle_sched.Scheduler(**cfg)            # default: sessions
    c = mab.Scheduler(**cfg)                     # 0: sessions
    for t in range(400):
        for client, prompt, limit in (arrivals[t] if t < len(arrivals) else []):
            assert c.submit(client, prompt, limit) == o.submit(client, prompt, limit)
        assert _as_rows(c.step(), 16) == _oracle_rows(o.step())


def test_errors():
    lib = mab._lib()
    cfg = mab.SchedConfig(2, 8, 2, 4, 0, 16, 10, 4)
    h = ctypes.c_void_p()
    assert lib.mab_sched_create(None, ctypes.byref(h)) == 1
    for field, bad in (("sessions", 0), ("prefill_chunk", 0), ("max_pending_per_client", 0),
                       ("near_done_gate", -1), ("max_decode_rows", -1), ("page_size", 0),
                       ("num_pages", 0), ("max_pages_per_seq", 0)):
        c = mab.SchedConfig(2, 8, 2, 4, 0, 16, 10, 4)
        setattr(c, field, bad)
        assert lib.mab_sched_create(ctypes.byref(c), ctypes.byref(h)) == 2, field
        assert not h.value
    s = mab.Scheduler(2, 8, 2, 4, page_size=16, num_pages=10, max_pages_per_seq=4)
    assert s.submit(-1, 4, 4) == (2, -1)
    assert s.submit(0, 0, 4) == (2, -1)
    assert s.submit(0, 60, 6) == (2, -1)          # 65 positions: 5 pages > 4
    big = mab.Scheduler(2, 8, 2, 4, page_size=1 << 20, num_pages=1 << 12, max_pages_per_seq=1 << 12)
    assert big.submit(0, 2**31 - 1, 2) == (2, -1)  # positions past int32
    assert s.submit(0, 60, 5) == (0, 0)
    assert s.submit(0, 1, 1) == (0, 1)
    assert s.submit(0, 1, 1) == (mab.MAB_ERR_QUOTA, -1)
    assert "client_quota" in mab.mab_status_string(mab.MAB_ERR_QUOTA)
    info = mab.StepInfo()
    small = np.zeros(64, np.int32)
    ids = np.zeros(64, np.int64)
    args = [s._h, ctypes.byref(info), ids.ctypes.data] + [small.ctypes.data] * 5
    assert lib.mab_sched_step(*args, 2) == 2      # capacity below max_decode_rows + 1
    assert lib.mab_sched_step(s._h, ctypes.byref(info), None, *([small.ctypes.data] * 5), 8) == 1
    assert lib.mab_sched_step(*args, 3) == 0 and info.kind == 2
    lib.mab_sched_destroy(None)


def test_step_batch_descriptor_matches_its_rows():
    s = mab.Scheduler(4, 16, 8, 4, page_size=16, num_pages=200, max_pages_per_seq=32)
    rng = np.random.default_rng(3)
    for _ in range(6):
        s.submit(int(rng.integers(0, 3)), int(rng.integers(1, 100)), int(rng.integers(1, 30)))
    seen = 0
    while (st := s.step()) is not None:
        q = st.q_len
        assert st.q_start[0] == 0 and (q >= 1).all()
        assert (q[:-1] == 1).all() or st.num_seqs == 1 or (q == 1).all()
        for i in range(st.num_seqs):
            used = -(-(st.prefix_len[i] + q[i]) // 16)
            assert (st.block_table[i, :used] >= 0).all()
        seen += 1
    assert seen > 10
