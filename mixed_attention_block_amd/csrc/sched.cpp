// Step scheduler and batch builder for a serving loop over the paged cache.
//
// Each call to mab_sched_step decides one engine tick: which decode rows and
// which prefill chunk slice go into the step's ForwardBatch.  It then writes
// that batch's descriptor (q_start, prefix_len, block-table rows) for
// kv_append_quant and mixed_attention_fwd.  The rules are those of the MBufo
// page ("自研RDNA高併發推論引擎 以AI Max+ 395為範例", section 1: the scheduler
// guarantees table and the fairness part on SRTF, starving-decode preemption
// and the near-done gate):
//
//  * Admission.  Pending requests take free session slots.  Clients take
//    turns, FIFO within a client, and each client holds at most
//    max_pending_per_client waiting requests.  A request's KV pages,
//    ceil((prompt + limit - 1) / page_size) of them, are reserved at
//    admission: the lowest-numbered free pages, in increasing order.
//    Admission stops at the first request that does not fit.
//  * Decode first.  While a decoder is due, the tick is a decode step over
//    the due decoders in queue order, at most max_decode_rows of them.
//    Otherwise it is a merged step: at most one chunk slice of at most
//    prefill_chunk tokens, plus the first max_decode_rows decoders.
//  * Served decoders move to the back of the decode queue, in their order
//    (PopDecoder rotation).  After a merged step every resident decoder is
//    due (MarkAllDecodersDue).
//  * Chunk choice (SRTF).  Prefills are ordered by the chunk slices they
//    still need, fewest first, earliest request first within a count: one
//    with a single slice left ("near done") goes before every longer one,
//    and a short prompt before a long prompt's continuation slices.  While a
//    request waits for a slot, prefills with more than one slice left get
//    no chunk if some resident decoder is within near_done_gate tokens of
//    its limit.
//
// The state is plain arrays indexed by request id, with a min-heap of free
// pages.  A tick costs O(resident + decoders + rows * max_pages_per_seq).
#include <stdint.h>

#include <algorithm>
#include <climits>
#include <deque>
#include <functional>
#include <new>
#include <queue>
#include <unordered_map>
#include <vector>

#include "mab.h"

namespace {

enum Phase : uint8_t { kPending, kPrefill, kDecode, kDone };

struct Req {
  int32_t client, prompt, limit;
  int32_t prefilled, generated;
  Phase phase;
  bool due;
  bool served;  // picked for the current tick
  std::vector<int32_t> pages;
};

int64_t pages_for(int64_t prompt, int64_t limit, int64_t page_size) {
  return (prompt + limit - 1 + page_size - 1) / page_size;
}

}  // namespace

struct mab_sched {
  mab_sched_config cfg;
  int32_t max_decode;
  std::vector<Req> req;                                      // by request id
  std::unordered_map<int32_t, std::deque<int64_t>> waiting;  // client -> its pending requests
  std::deque<int32_t> turns;                                 // clients with pending requests, in turn order
  int64_t n_pending = 0;
  std::vector<int64_t> resident;                             // in admission order
  std::deque<int64_t> queue;                                 // decoders, in rotation order
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_pages;
  std::vector<int64_t> picked;                               // scratch: the tick's decoders

  void admit() {
    while ((int64_t)resident.size() < cfg.sessions && !turns.empty()) {
      const int32_t client = turns.front();
      std::deque<int64_t>& w = waiting[client];
      Req& r = req[w.front()];
      const int64_t need = pages_for(r.prompt, r.limit, cfg.page_size);
      if (need > (int64_t)free_pages.size()) break;
      r.pages.resize(need);
      for (int64_t i = 0; i < need; ++i) {
        r.pages[i] = free_pages.top();
        free_pages.pop();
      }
      r.phase = kPrefill;
      resident.push_back(w.front());
      w.pop_front();
      --n_pending;
      turns.pop_front();
      if (!w.empty()) turns.push_back(client);
    }
  }

  // the prefill that gets this tick's chunk, or -1
  int64_t choose_chunk() const {
    bool starving = false;
    if (n_pending > 0)
      for (int64_t d : queue)
        if (req[d].limit - req[d].generated <= cfg.near_done_gate) starving = true;
    int64_t best = -1, best_slices = 0;
    for (int64_t id : resident) {
      const Req& r = req[id];
      if (r.phase != kPrefill) continue;
      const int64_t slices = ((int64_t)r.prompt - r.prefilled + cfg.prefill_chunk - 1) / cfg.prefill_chunk;
      if (best < 0 || slices < best_slices || (slices == best_slices && id < best)) {
        best = id;
        best_slices = slices;
      }
    }
    if (best >= 0 && best_slices > 1 && starving) return -1;  // only a near-done prefill may run
    return best;
  }

  void release(int64_t id) {
    Req& r = req[id];
    r.phase = kDone;
    r.due = false;
    for (int32_t p : r.pages) free_pages.push(p);
    resident.erase(std::find(resident.begin(), resident.end(), id));
    auto it = std::find(queue.begin(), queue.end(), id);
    if (it != queue.end()) queue.erase(it);
  }
};

extern "C" {

int32_t mab_sched_create(const mab_sched_config* cfg, mab_sched** out) {
  if (!cfg || !out) return MAB_ERR_NULL;
  *out = nullptr;
  if (cfg->sessions < 1 || cfg->prefill_chunk < 1 || cfg->max_pending_per_client < 1 ||
      cfg->near_done_gate < 0 || cfg->max_decode_rows < 0 || cfg->page_size < 1 || cfg->num_pages < 1 ||
      cfg->max_pages_per_seq < 1)
    return MAB_ERR_SHAPE;
  mab_sched* s = new (std::nothrow) mab_sched();
  if (!s) return MAB_ERR_NULL;
  s->cfg = *cfg;
  s->max_decode = cfg->max_decode_rows > 0 ? cfg->max_decode_rows : cfg->sessions;
  std::vector<int32_t> pages(cfg->num_pages);
  for (int32_t i = 0; i < cfg->num_pages; ++i) pages[i] = i;
  s->free_pages = decltype(s->free_pages)(std::greater<int32_t>(), std::move(pages));
  *out = s;
  return MAB_OK;
}

void mab_sched_destroy(mab_sched* s) { delete s; }

int32_t mab_sched_submit(mab_sched* s, int32_t client, int32_t prompt_len, int32_t token_limit,
                         int64_t* request_id) {
  if (!s || !request_id) return MAB_ERR_NULL;
  *request_id = -1;
  if (client < 0 || prompt_len < 1 || token_limit < 1) return MAB_ERR_SHAPE;
  if ((int64_t)prompt_len + token_limit - 1 > INT32_MAX) return MAB_ERR_SHAPE;  // positions are int32
  const int64_t need = pages_for(prompt_len, token_limit, s->cfg.page_size);
  if (need > s->cfg.max_pages_per_seq || need > s->cfg.num_pages) return MAB_ERR_SHAPE;
  std::deque<int64_t>& w = s->waiting[client];
  if ((int64_t)w.size() >= s->cfg.max_pending_per_client) return MAB_ERR_QUOTA;
  const int64_t id = (int64_t)s->req.size();
  s->req.push_back(Req{client, prompt_len, token_limit, 0, 0, kPending, false, false, {}});
  if (w.empty()) s->turns.push_back(client);
  w.push_back(id);
  ++s->n_pending;
  *request_id = id;
  return MAB_OK;
}

int32_t mab_sched_step(mab_sched* s, mab_step_info* info, int64_t* request_id, int32_t* q_start,
                       int32_t* prefix_len, int32_t* block_table, int32_t* emit, int32_t* finished,
                       int32_t capacity) {
  if (!s || !info || !request_id || !q_start || !prefix_len || !block_table || !emit || !finished)
    return MAB_ERR_NULL;
  if (capacity < s->max_decode + 1) return MAB_ERR_SHAPE;
  s->admit();

  // the tick's decoders: the due ones (decode step) or the queue's head (merged step)
  bool any_due = false;
  for (int64_t d : s->queue) any_due |= s->req[d].due;
  s->picked.clear();
  for (int64_t d : s->queue) {
    if ((int32_t)s->picked.size() == s->max_decode) break;
    if (!any_due || s->req[d].due) s->picked.push_back(d);
  }
  const int64_t chunk = any_due ? -1 : s->choose_chunk();
  info->kind = s->picked.empty() && chunk < 0 ? 0 : any_due ? 1 : 2;
  info->num_seqs = 0;
  info->num_rows = 0;
  if (info->kind == 0) {
    q_start[0] = 0;
    info->pending = (int32_t)s->n_pending;
    return MAB_OK;
  }

  // PopDecoder: the picked decoders go to the back, in their order
  for (int64_t d : s->picked) s->req[d].served = true;
  std::deque<int64_t> rotated;
  for (int64_t d : s->queue)
    if (!s->req[d].served) rotated.push_back(d);
  for (int64_t d : s->picked) {
    rotated.push_back(d);
    s->req[d].served = false;
  }
  s->queue.swap(rotated);

  const int32_t width = s->cfg.max_pages_per_seq;
  int32_t n = 0, rows = 0;
  auto put_row = [&](int64_t id, int32_t prefix, int32_t q) {
    const Req& r = s->req[id];
    request_id[n] = id;
    q_start[n] = rows;
    prefix_len[n] = prefix;
    int32_t* bt = block_table + (int64_t)n * width;
    std::copy(r.pages.begin(), r.pages.end(), bt);
    std::fill(bt + r.pages.size(), bt + width, -1);
    rows += q;
    ++n;
  };
  for (int64_t d : s->picked) {
    const Req& r = s->req[d];
    put_row(d, r.prompt + r.generated - 1, 1);
  }
  int32_t slice = 0;
  if (chunk >= 0) {
    const Req& r = s->req[chunk];
    slice = std::min(s->cfg.prefill_chunk, r.prompt - r.prefilled);
    put_row(chunk, r.prefilled, slice);
  }
  q_start[n] = rows;

  // advance: one token per decoder, the slice for the chunk
  std::vector<int64_t> done;
  for (int32_t i = 0; i < (int32_t)s->picked.size(); ++i) {
    Req& r = s->req[s->picked[i]];
    ++r.generated;
    if (info->kind == 1) r.due = false;
    emit[i] = 1;
    finished[i] = r.generated == r.limit;
    if (finished[i]) done.push_back(s->picked[i]);
  }
  if (chunk >= 0) {
    Req& r = s->req[chunk];
    r.prefilled += slice;
    const int32_t i = n - 1;
    emit[i] = r.prefilled == r.prompt;
    finished[i] = 0;
    if (emit[i]) {
      r.generated = 1;
      if (r.limit == 1) {
        finished[i] = 1;
        done.push_back(chunk);
      } else {
        r.phase = kDecode;
        s->queue.push_back(chunk);
      }
    }
  }
  for (int64_t id : done) s->release(id);
  if (info->kind == 2)
    for (int64_t d : s->queue) s->req[d].due = true;  // MarkAllDecodersDue

  info->num_seqs = n;
  info->num_rows = rows;
  info->pending = (int32_t)s->n_pending;
  return MAB_OK;
}

}  // extern "C"
