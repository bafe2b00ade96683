"""Pins of the scheduler oracle (CPU only).

* Three traces whose every step was derived by hand from the rules
  (tests/golden/sched_traces.json).
* The guarantees of the MBufo page's scheduler table and fairness part, checked
  from the outside on seeded random traces: decode first, every decoder served
  between two merged steps, bounded chunks, decoder rotation, per-client quota
  and admission rotation, SRTF with the near-done gate, and every accepted
  request finishing with exactly its token limit.
"""

import json
import os

import numpy as np
import pytest

from oracle import scheduler as sched

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "sched_traces.json")


def golden_traces():
    return json.load(open(GOLDEN, encoding="utf-8"))["traces"]


def run_golden(trace, make=sched.Scheduler):
    s = make(**trace["config"])
    for client, prompt, limit, status, rid in trace["submit"]:
        assert s.submit(client, prompt, limit) == (status, rid), (trace["name"], client, prompt, limit)
    got, pages = [], {}
    for _ in trace["steps"]:
        st = s.step()
        if st is None:
            got.append(None)
            continue
        rows = [list(r) for r in zip(st["ids"], st["prefix_len"], st["q_len"], st["emit"], st["finished"])]
        got.append([st["kind"], rows])
        for rid, row in zip(st["ids"], st["block_table"]):
            pages[str(rid)] = [p for p in row if p >= 0]
    return got, pages


@pytest.mark.parametrize("trace", golden_traces(), ids=lambda t: t["name"])
def test_golden_trace(trace):
    got, pages = run_golden(trace)
    for t, (g, w) in enumerate(zip(got, trace["steps"])):
        assert g == w, f"{trace['name']} tick {t + 1}: {g} != {w}"
    assert pages == trace["pages"]


def random_config(rng):
    sessions = int(rng.integers(1, 7))
    return dict(sessions=sessions, prefill_chunk=int(rng.choice([4, 8, 16, 64])),
                max_pending_per_client=int(rng.integers(1, 4)), near_done_gate=int(rng.integers(0, 9)),
                page_size=int(rng.choice([4, 16])), num_pages=int(rng.integers(40, 200)),
                max_pages_per_seq=64, max_decode_rows=int(rng.integers(1, sessions + 1)))


def random_arrivals(rng, ticks, clients):
    """Per tick, a list of (client, prompt, limit): short and long prompts,
    short and long outputs."""
    out = []
    for _ in range(ticks):
        k = int(rng.poisson(0.6))
        reqs = []
        for _ in range(k):
            prompt = int(rng.integers(1, 12)) if rng.random() < 0.6 else int(rng.integers(12, 200))
            limit = int(rng.integers(1, 6)) if rng.random() < 0.5 else int(rng.integers(6, 40))
            reqs.append((int(rng.integers(0, clients)), prompt, limit))
        out.append(reqs)
    return out


class Observer:
    """Checks the guarantees from the submissions and the step outputs (plus,
    where a rule needs them, the pending queue and the admitted prefills read
    after the tick's admission)."""

    def __init__(self, cfg):
        self.cfg = cfg
        self.info = {}          # rid -> [client, prompt, limit]
        self.prefilled = {}
        self.generated = {}
        self.finished = set()
        self.due = set()
        self.decoder_since = {}  # rid -> step at which it became a decoder
        self.served_at = {}      # rid -> (index in log, step) of its last decode row
        self.log = []            # decode rows' request ids, in the order served
        self.last_merged = None
        self.must_serve = set()  # decoders due since the last merged step, not yet served
        self.steps = 0
        self.admissions = []     # (step, client) in admission order
        self.entered = {}        # client -> step at which it last entered the rotation

    def submitted(self, s, client, prompt, limit, status, rid):
        pending_before = len(s.pending.get(client, [])) - (1 if status == sched.OK else 0)
        if status == sched.QUOTA:
            assert pending_before == self.cfg["max_pending_per_client"]
            return
        if status != sched.OK:
            return
        assert pending_before < self.cfg["max_pending_per_client"]
        if pending_before == 0:
            self.entered[client] = self.steps
        self.info[rid] = [client, prompt, limit]
        self.prefilled[rid] = 0
        self.generated[rid] = 0

    def admitted(self, s, before):
        new = [r for r in s.resident if r.rid not in before]
        for r in new:
            self.admissions.append((self.steps, r.client, r.rid))
        # what the tick's chunk choice sees: the admitted prefills, the queue
        self.pre_prefills = sorted(r.rid for r in s.resident if r.state == "prefill")
        self.pre_pending = s.any_pending()
        assert len(s.resident) <= self.cfg["sessions"]
        held = [p for r in s.resident for p in r.pages]
        assert len(held) == len(set(held)), "a page is held twice"
        assert all(0 <= p < self.cfg["num_pages"] for p in held)

    def check_chunk_choice(self, s, chunk_rid):
        cfg = self.cfg
        prefills = self.pre_prefills
        rem = {rid: self.info[rid][1] - self.prefilled[rid] for rid in prefills}
        near = [rid for rid in prefills if rem[rid] <= cfg["prefill_chunk"]]
        far = [rid for rid in prefills if rem[rid] > cfg["prefill_chunk"]]
        # fewest slices left first, the earlier request within a count
        far.sort(key=lambda rid: (-(-rem[rid] // cfg["prefill_chunk"]), rid))
        decoders = [rid for rid in self.generated if self.is_decoder(rid)]
        starving = self.pre_pending and any(self.info[d][2] - self.generated[d] <= cfg["near_done_gate"]
                                           for d in decoders)
        if chunk_rid is None:
            assert not near and (starving or not far), "a prefill was left without a chunk"
        elif near:
            assert chunk_rid == near[0], "SRTF: the earliest near-done prefill goes first"
        else:
            assert not starving, "a far prefill ran while a waiting request starved"
            assert chunk_rid == far[0], "SRTF among longer prefills (fewest slices left, then FIFO)"

    def is_decoder(self, rid):
        return (rid not in self.finished and self.prefilled[rid] == self.info[rid][1]
                and self.generated[rid] >= 1)

    def stepped(self, s, st):
        cfg = self.cfg
        self.steps += 1
        t = self.steps
        decoders_before = [rid for rid in self.generated if self.is_decoder(rid)]
        if st is None:
            assert not decoders_before and not self.pre_prefills
            return
        rows = list(zip(st["ids"], st["prefix_len"], st["q_len"], st["emit"], st["finished"]))
        dec_rows = [r for r in rows if self.prefilled[r[0]] == self.info[r[0]][1]]
        chunk_rows = [r for r in rows if self.prefilled[r[0]] < self.info[r[0]][1]]
        assert len(chunk_rows) <= 1
        assert rows == dec_rows + chunk_rows, "decode rows come first"
        assert len(dec_rows) <= cfg["max_decode_rows"]
        if self.due:
            assert st["kind"] == "decode", "decode first: a chunk ran while a decoder was due"
            assert all(r[0] in self.due for r in dec_rows)
        if st["kind"] == "decode":
            assert not chunk_rows
        else:
            assert len(dec_rows) == min(cfg["max_decode_rows"], len(decoders_before))
            self.check_chunk_choice(s, chunk_rows[0][0] if chunk_rows else None)
        for rid, prefix, q, emit, fin in dec_rows:
            client, prompt, limit = self.info[rid]
            assert q == 1 and prefix == prompt + self.generated[rid] - 1 and emit == 1
            self.generated[rid] += 1
            assert fin == (self.generated[rid] == limit)
            # rotation: between two services of rid (in the order rows are
            # served), every decoder that already was one at the first of them
            # is served
            last = self.served_at.get(rid)
            if last is not None:
                i1, t1 = last
                between = set(self.log[i1 + 1:])
                for other in decoders_before:
                    if other != rid and self.decoder_since[other] < t1:
                        assert other in between, f"{rid} served twice before {other}"
            self.served_at[rid] = (len(self.log), t)
            self.log.append(rid)
            self.due.discard(rid)
            self.must_serve.discard(rid)
            if fin:
                self.finished.add(rid)
        for rid, prefix, q, emit, fin in chunk_rows:
            client, prompt, limit = self.info[rid]
            assert 1 <= q <= cfg["prefill_chunk"] and prefix == self.prefilled[rid]
            self.prefilled[rid] += q
            assert emit == (self.prefilled[rid] == prompt)
            if emit:
                self.generated[rid] = 1
                self.decoder_since[rid] = t
                assert fin == (limit == 1)
                if fin:
                    self.finished.add(rid)
        for row, (rid, prefix, q, _, _) in zip(st["block_table"], rows):
            used = -(-(prefix + q) // cfg["page_size"])
            assert all(p >= 0 for p in row[:used])
        if st["kind"] == "merged":
            assert not self.must_serve, "a decoder was pushed out of the rotation by a chunk"
            self.due = {rid for rid in self.generated if self.is_decoder(rid)}
            self.must_serve = set(self.due)
            self.last_merged = t

    def check_admission_rotation(self):
        for (t1, c1, r1), (t2, c2, r2) in zip(self.admissions, self.admissions[1:]):
            if c1 != c2:
                continue
            # another client waiting since before the first of two admissions
            # of one client would have been admitted between them
            for c, since in self.entered.items():
                if c != c1 and since < t1:
                    waiting = [rid for rid, inf in self.info.items()
                               if inf[0] == c and rid < r2 and not any(a[2] == rid for a in self.admissions[:self.admissions.index((t2, c2, r2))])]
                    assert not waiting or min(waiting) > r1, f"client {c} skipped between admissions {r1}, {r2}"

    def check_all_finished(self):
        for rid, (client, prompt, limit) in self.info.items():
            assert rid in self.finished, f"request {rid} never finished"
            assert self.prefilled[rid] == prompt and self.generated[rid] == limit


def drive(s, cfg, arrivals, observer=None, record=None, max_ticks=20000):
    """Runs the arrivals (one list per tick) and then drains the scheduler."""
    ticks = 0
    while True:
        reqs = arrivals[ticks] if ticks < len(arrivals) else []
        for client, prompt, limit in reqs:
            status, rid = s.submit(client, prompt, limit)
            if record is not None:
                record.append(("submit", client, prompt, limit, status, rid))
            if observer:
                observer.submitted(s, client, prompt, limit, status, rid)
        if observer:
            before = {r.rid for r in s.resident}
            s.admit()
            observer.admitted(s, before)
        st = s.step()
        if record is not None:
            record.append(("step", st))
        if observer:
            observer.stepped(s, st)
        ticks += 1
        if st is None and ticks >= len(arrivals) and not s.any_pending():
            return ticks
        assert ticks < max_ticks, "the scheduler did not drain"


@pytest.mark.parametrize("seed", range(40))
def test_guarantees_on_random_traces(seed):
    rng = np.random.default_rng(1000 + seed)
    cfg = random_config(rng)
    arrivals = random_arrivals(rng, int(rng.integers(20, 120)), int(rng.integers(1, 5)))
    s = sched.Scheduler(**cfg)
    obs = Observer(cfg)
    drive(s, cfg, arrivals, obs)
    obs.check_all_finished()
    obs.check_admission_rotation()
    assert sorted(s.free_pages) == list(range(cfg["num_pages"])), "pages leaked"


def test_submit_rejects_impossible_requests():
    s = sched.Scheduler(2, 8, 2, 4, page_size=16, num_pages=10, max_pages_per_seq=4)
    assert s.submit(0, 0, 4)[0] == sched.INVALID
    assert s.submit(0, 4, 0)[0] == sched.INVALID
    assert s.submit(0, 60, 6)[0] == sched.INVALID      # 65 positions > 4 pages of 16
    assert s.submit(0, 60, 5) == (sched.OK, 0)         # 64 positions fit exactly
    assert s.submit(0, 1, 1) == (sched.OK, 1)
    assert s.submit(0, 1, 1)[0] == sched.QUOTA
    assert s.submit(1, 1, 1) == (sched.OK, 2)
