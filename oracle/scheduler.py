"""Fair scheduler and ForwardBatch builder: which rows go into each engine step.

TEST INFRASTRUCTURE ONLY: only ``tests/`` may import this module.  It shares no
code with the library's scheduler (``mixed_attention_block_amd/csrc/sched.cpp``).

Source: MBufo page, "自研RDNA高併發推論引擎 以AI Max+ 395為範例" (lcz.me, topic
2938), section 1.  Three parts of it apply:

* the opening of section 1, which sets out what the scheduler was already
  doing: a bounded prefill chunk, decode served before prefill, and a
  per-client cap on admission;
* the table "排程器保證什麼" (what the scheduler guarantees);
* the part "公平性：排隊不插隊（SRTF＋飢餓 decode 優先搶佔＋near-done 閘門）" (SRTF
  prefill choice, starving-decode preemption, near-done gate).

The pages list the rules but not a tick-by-tick algorithm.  Where they leave a
step open, this module takes the plain reading below (R-S1 .. R-S9):

R-S1  A tick first admits pending requests into free session slots.  A
      request's KV pages, ceil((prompt + limit - 1) / page_size) of them, are
      reserved at admission.  The lowest-numbered free pages are taken, in
      increasing order.  Admission stops at the first request that does not
      fit.
R-S2  Pending requests leave the queue by client rotation.  Clients take turns
      in the order they entered the rotation, FIFO within a client.  After a
      client's request is admitted, the client goes to the back of the
      rotation if it still has requests pending.
R-S3  If a resident decoder is due, the step is a decode step.  It serves the
      due decoders in decode-queue order, at most max_decode_rows of them.
      Otherwise the step is a merged step: at most one prefill chunk slice,
      plus the first max_decode_rows decoders in queue order.
R-S4  PopDecoder rotation: the decoders a step serves move to the back of
      the decode queue, in their relative order.  A new decoder joins at the
      back.
R-S5  MarkAllDecodersDue: after a merged step, every resident decoder is due,
      including one whose prefill finished in that step.  A decode step
      clears the flag of the decoders it served.
R-S6  SRTF: prefills are ordered by the chunk slices they still need,
      ceil(remaining / prefill_chunk), fewest first; within a class (the same
      count) the earlier request goes first.  A prefill with one slice left
      (remaining <= prefill_chunk) is "near done" and so goes before every
      longer prefill continuation, and a prompt of a few slices goes before a
      long prompt's continuation slices.
R-S7  Starving-decode preemption with the near-done gate: while some request
      is pending, and some resident decoder has at most near_done_gate tokens
      left, prefills that are not near done get no chunk.
R-S8  Rows and positions.  A chunk row covers prompt positions [done,
      done + n) with n = min(prefill_chunk, remaining); its prefix is done.
      A decoder that has produced g tokens feeds token g at position
      prompt + g - 1.  That is a row with prefix prompt + g - 1 and one
      query.  The last chunk of a prompt yields the first token.  A request
      is finished when it has produced `limit` tokens, and its slot and
      pages free at the end of that step.
R-S9  Batch order: the decoders in the order served, then the chunk.  Block
      table rows are the request's reserved pages, padded with -1.

Parity: pinned by hand-derived step sequences of three small traces
(tests/golden/sched_traces.json) and by the guarantees checked on seeded
random traces (tests/test_oracle_scheduler.py).
"""

from collections import deque

OK, INVALID, QUOTA = 0, 2, 7


class Request:
    def __init__(self, rid, client, prompt, limit):
        self.rid = rid
        self.client = client
        self.prompt = prompt
        self.limit = limit
        self.state = "pending"     # pending -> prefill -> decode -> done
        self.prefilled = 0
        self.generated = 0
        self.pages = []
        self.due = False


class Scheduler:
    def __init__(self, sessions, prefill_chunk, max_pending_per_client, near_done_gate,
                 page_size, num_pages, max_pages_per_seq, max_decode_rows=None):
        self.sessions = sessions
        self.chunk = prefill_chunk
        self.quota = max_pending_per_client
        self.gate = near_done_gate
        self.page_size = page_size
        self.num_pages = num_pages
        self.max_pages = max_pages_per_seq
        self.max_decode_rows = sessions if max_decode_rows is None else max_decode_rows
        self.requests = []
        self.pending = {}          # client -> deque of requests
        self.rotation = []         # clients with pending requests, in turn order
        self.resident = []         # admitted requests, in admission order
        self.decode_queue = []     # resident decoders, in rotation order
        self.free_pages = list(range(num_pages))

    def pages_needed(self, prompt, limit):
        return -(-(prompt + limit - 1) // self.page_size)

    def submit(self, client, prompt, limit):
        """Returns (status, request id or -1)."""
        if prompt < 1 or limit < 1 or client < 0:
            return INVALID, -1
        need = self.pages_needed(prompt, limit)
        if need > self.max_pages or need > self.num_pages:
            return INVALID, -1
        waiting = self.pending.get(client, deque())
        if len(waiting) >= self.quota:
            return QUOTA, -1
        r = Request(len(self.requests), client, prompt, limit)
        self.requests.append(r)
        waiting.append(r)
        self.pending[client] = waiting
        if client not in self.rotation:
            self.rotation.append(client)
        return OK, r.rid

    def any_pending(self):
        return len(self.rotation) > 0

    def admit(self):
        while len(self.resident) < self.sessions and self.rotation:
            client = self.rotation[0]
            r = self.pending[client][0]
            need = self.pages_needed(r.prompt, r.limit)
            if need > len(self.free_pages):
                break
            self.pending[client].popleft()
            self.free_pages.sort()
            r.pages = self.free_pages[:need]
            self.free_pages = self.free_pages[need:]
            r.state = "prefill"
            self.resident.append(r)
            self.rotation.pop(0)
            if self.pending[client]:
                self.rotation.append(client)

    def slices_left(self, r):
        return -(-(r.prompt - r.prefilled) // self.chunk)

    def pick_chunk(self):
        prefills = sorted((r for r in self.resident if r.state == "prefill"),
                          key=lambda r: (self.slices_left(r), r.rid))
        near = [r for r in prefills if self.slices_left(r) == 1]
        starving = self.any_pending() and any(r.limit - r.generated <= self.gate for r in self.decode_queue)
        choices = near if starving else prefills
        return choices[0] if choices else None

    def step(self):
        """One tick.  Returns None when there is nothing to run, else a dict:
        kind ("decode" | "merged"), ids, prefix_len, q_len, emit, finished,
        block_table (one row per sequence)."""
        self.admit()
        due = [r for r in self.decode_queue if r.due]
        if due:
            kind = "decode"
            served = due[:self.max_decode_rows]
            chunk = None
        else:
            kind = "merged"
            served = self.decode_queue[:self.max_decode_rows]
            chunk = self.pick_chunk()
        if not served and chunk is None:
            return None
        rest = [r for r in self.decode_queue if r not in served]
        self.decode_queue = rest + served

        ids, prefix, qlen, emit, finished, table = [], [], [], [], [], []

        def add_row(r, p, n, emits):
            ids.append(r.rid)
            prefix.append(p)
            qlen.append(n)
            emit.append(1 if emits else 0)
            table.append(r.pages + [-1] * (self.max_pages - len(r.pages)))

        for r in served:
            add_row(r, r.prompt + r.generated - 1, 1, True)
        if chunk is not None:
            n = min(self.chunk, chunk.prompt - chunk.prefilled)
            add_row(chunk, chunk.prefilled, n, chunk.prefilled + n == chunk.prompt)

        done = []
        for r in served:
            r.generated += 1
            if kind == "decode":
                r.due = False
            if r.generated == r.limit:
                done.append(r)
        if chunk is not None:
            chunk.prefilled += n
            if chunk.prefilled == chunk.prompt:
                chunk.generated = 1
                if chunk.limit == 1:
                    done.append(chunk)
                else:
                    chunk.state = "decode"
                    self.decode_queue.append(chunk)
        for r in done:
            r.state = "done"
            r.due = False
            self.resident.remove(r)
            if r in self.decode_queue:
                self.decode_queue.remove(r)
            self.free_pages.extend(r.pages)
        finished = [1 if self.requests[i] in done else 0 for i in ids]
        if kind == "merged":
            for r in self.decode_queue:
                r.due = True
        return dict(kind=kind, ids=ids, prefix_len=prefix, q_len=qlen, emit=emit, finished=finished,
                    block_table=table)
