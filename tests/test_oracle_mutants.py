"""Planted mistakes in the oracle (CPU only): each plausible slip must make at
least one pin fail, or the pins would not be worth trusting."""

import numpy as np
import pytest

import test_oracle_attention as ta
import test_oracle_codec as tc
from oracle import attention, codec
from oracle_pins import parse_worked_examples

_orig_encode = codec.encode_blocks
_orig_attend = attention.attend


def _swap_nibbles(x, fmt):
    out = _orig_encode(x, fmt)
    if fmt == "q4":
        out[..., 2:] = ((out[..., 2:] & 0x0F) << 4) | (out[..., 2:] >> 4)
    return out


def _big_endian_scale(x, fmt):
    out = _orig_encode(x, fmt)
    out[..., [0, 1]] = out[..., [1, 0]]
    return out


def _quantize_with_stored_scale(x, fmt):
    # quantizes with the fp16 scale d instead of the binary32 scale s
    qm = np.float32(codec.qmax(fmt))
    xf = x.astype(np.float32)
    amax = np.abs(xf).max(axis=-1)
    d = (amax / qm).astype(np.float16)
    ds = np.where(d > 0, d.astype(np.float32), np.float32(1))
    q = np.clip(np.rint(xf / ds[..., None]), -qm, qm)
    q = np.where((d > 0)[..., None], q, 0).astype(np.int8)
    out = _orig_encode(x, fmt)
    qb = q.view(np.uint8)
    out[..., 2:] = qb if fmt == "q8" else (qb[..., 0::2] & 0xF) | ((qb[..., 1::2] & 0xF) << 4)
    return out


def _round_half_up(monkeypatch):
    floor = np.floor
    monkeypatch.setattr(np, "rint", lambda a: floor(np.asarray(a) + np.float32(0.5)))


def _codec_pins():
    for ex in parse_worked_examples():
        tc.test_worked_examples_encode(ex)
    tc.test_codec_invariants("q8")
    tc.test_codec_invariants("q4")


@pytest.mark.parametrize("mutant", [_swap_nibbles, _big_endian_scale, _quantize_with_stored_scale])
def test_codec_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(codec, "encode_blocks", mutant)
    with pytest.raises(AssertionError):
        _codec_pins()


def test_round_half_up_is_caught(monkeypatch):
    _round_half_up(monkeypatch)
    with pytest.raises(AssertionError):
        _codec_pins()


def _sees_one_future_key(q, k, v, positions, sm_scale):
    return _orig_attend(q, k, v, np.minimum(np.asarray(positions) + 1, k.shape[0] - 1), sm_scale)


def _wrong_group_mapping(q, k, v, positions, sm_scale):
    return _orig_attend(q, k[:, ::-1], v[:, ::-1], positions, sm_scale)


def _keys_and_values_swapped(q, k, v, positions, sm_scale):
    return _orig_attend(q, v, k, positions, sm_scale)


def _scale_dropped(q, k, v, positions, sm_scale):
    return _orig_attend(q, k, v, positions, 1.0)


@pytest.mark.parametrize("mutant", [_sees_one_future_key, _wrong_group_mapping,
                                    _keys_and_values_swapped, _scale_dropped])
def test_attention_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(attention, "attend", mutant)
    with pytest.raises(AssertionError):
        ta.test_brute_force_tiny("q8", "q4")
    with pytest.raises(AssertionError):
        ta.test_codec_free_case_matches_torch_sdpa()


# --- scheduler oracle -------------------------------------------------------

import numpy as np  # noqa: E402

import test_oracle_scheduler as ts  # noqa: E402
from oracle import scheduler as sched  # noqa: E402


class _NoMarkAllDue(sched.Scheduler):
    def step(self):
        st = super().step()
        if st is not None and st["kind"] == "merged":
            for r in self.decode_queue:
                r.due = False
        return st


class _FifoPrefill(sched.Scheduler):
    def pick_chunk(self):
        prefills = sorted((r for r in self.resident if r.state == "prefill"), key=lambda r: r.rid)
        return prefills[0] if prefills else None


class _NoGate(sched.Scheduler):
    def pick_chunk(self):
        prefills = sorted((r for r in self.resident if r.state == "prefill"),
                          key=lambda r: (self.slices_left(r), r.rid))
        return prefills[0] if prefills else None


class _TwoClassSrtf(sched.Scheduler):
    """Near done first, then first come first served among the others."""

    def pick_chunk(self):
        prefills = sorted((r for r in self.resident if r.state == "prefill"), key=lambda r: r.rid)
        near = [r for r in prefills if r.prompt - r.prefilled <= self.chunk]
        far = [r for r in prefills if r.prompt - r.prefilled > self.chunk]
        starving = self.any_pending() and any(r.limit - r.generated <= self.gate for r in self.decode_queue)
        choices = near if starving else near + far
        return choices[0] if choices else None


class _NoRotation(sched.Scheduler):
    def step(self):
        st = super().step()
        self.decode_queue.sort(key=lambda r: r.rid)
        return st


class _ChunkFirst(sched.Scheduler):
    def step(self):
        st = super().step()
        if st is not None and st["kind"] == "merged" and len(st["ids"]) > 1:
            chunk_row = [i for i, rid in enumerate(st["ids"]) if st["q_len"][i] > 1 or self.requests[rid].generated <= 1]
            if chunk_row and chunk_row[-1] == len(st["ids"]) - 1:
                for k in st:
                    if k != "kind":
                        st[k] = st[k][-1:] + st[k][:-1]
        return st


class _GlobalFifoAdmission(sched.Scheduler):
    def admit(self):
        while len(self.resident) < self.sessions and self.rotation:
            waiting = sorted((q[0] for q in self.pending.values() if q), key=lambda r: r.rid)
            r = waiting[0]
            need = self.pages_needed(r.prompt, r.limit)
            if need > len(self.free_pages):
                break
            self.pending[r.client].popleft()
            self.free_pages.sort()
            r.pages, self.free_pages = self.free_pages[:need], self.free_pages[need:]
            r.state = "prefill"
            self.resident.append(r)
            self.rotation = [c for c in self.rotation if self.pending[c]]


class _DecodePrefixOffByOne(sched.Scheduler):
    def step(self):
        st = super().step()
        if st is not None:
            st["prefix_len"] = [p + 1 if q == 1 and self.requests[rid].prefilled == self.requests[rid].prompt
                                and p >= self.requests[rid].prompt - 1 else p
                                for rid, p, q in zip(st["ids"], st["prefix_len"], st["q_len"])]
        return st


def _scheduler_pins(make):
    for trace in ts.golden_traces():
        got, pages = ts.run_golden(trace, make)
        assert got == trace["steps"] and pages == trace["pages"]
    for seed in range(40):
        rng = np.random.default_rng(1000 + seed)
        cfg = ts.random_config(rng)
        arrivals = ts.random_arrivals(rng, int(rng.integers(20, 120)), int(rng.integers(1, 5)))
        obs = ts.Observer(cfg)
        ts.drive(make(**cfg), cfg, arrivals, obs)
        obs.check_all_finished()
        obs.check_admission_rotation()


@pytest.mark.parametrize("mutant", [_NoMarkAllDue, _FifoPrefill, _NoGate, _TwoClassSrtf, _NoRotation, _ChunkFirst,
                                    _GlobalFifoAdmission, _DecodePrefixOffByOne], ids=lambda m: m.__name__)
def test_scheduler_mutants_are_caught(mutant):
    with pytest.raises(AssertionError):
        _scheduler_pins(mutant)


def test_scheduler_pins_pass_unmutated():
    _scheduler_pins(sched.Scheduler)
