// Interleaved span-prefill scheduling (host code).
//
// MiniPIC §2 (the scheduling paragraph that follows §2.2) and §3,
// contribution 4: span prefills are not all batched ahead of a barrier that
// holds back the final prompts; each engine step mixes the running requests'
// decode tokens, final-prompt chunks and span-prefill chunks under one token
// budget, so that one mixed attention launch (pic_attn_prefill) serves them
// all.  The barrier-separated policy the page compares against runs a single
// kind of work per step: span prefills while any admitted request still waits
// for one, then final prompts, then decodes.
//
// Model of the work (lengths in tokens):
//   span     shared by id, a whole number of KV blocks (the Padding primitive
//            of §2.2 aligns spans to block boundaries).  Its KV is prefilled
//            once, on its own (causal within the span, positions 0..len-1),
//            stored position-free and reused by every request that lists it.
//   request  arrival step, list of spans, final-prompt length, output length.
//            The final prompt attends to the request's spans in the listed
//            order followed by its own tokens (causal); then one decode token
//            per step.  Key slot j of a request is the j-th token of that
//            composed sequence (its spans' blocks, then private blocks) and
//            its logical position is j.
// Admission is first come, first served by (arrival, id), bounded by the
// number of running requests and by free blocks; a request's blocks (private
// blocks for prompt + output, blocks of its spans that are not resident) are
// reserved when it is admitted, so a running request never waits for memory.
// Resident spans that no running request uses are evicted, oldest use first,
// when an admission needs their blocks (they are prefilled again if needed).
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "pic.h"
#include "pic_common.hpp"

namespace pic {

namespace {

enum Phase { kWaiting = 0, kSpans, kPrompt, kDecode, kFinished };

struct SSpan {
  int len = 0;
  int nblk = 0;
  std::vector<int32_t> blocks;  // empty while not resident
  int done = 0;                 // tokens prefilled into `blocks`
  int running_users = 0;        // running requests that list it
  long long last_use = -1;      // last step that referenced it
  bool in_step = false;         // a chunk of it is in the step being built
};

struct SReq {
  long long arrival = 0;
  std::vector<int> spans;
  int prompt_len = 0, out_len = 0;
  int span_tokens = 0;  // composed offset of the final prompt
  Phase phase = kWaiting;
  int prompt_done = 0, decoded = 0;
  std::vector<int32_t> priv;  // private blocks (prompt + output tokens)
};

struct Entry {
  int kind, id, q_begin, q_len;
};

}  // namespace

struct Sched {
  int policy, budget, max_running, num_blocks, bs;
  std::vector<int32_t> free_blocks;
  std::vector<SSpan> spans;
  std::vector<SReq> reqs;
  std::vector<int> waiting;  // request ids not yet admitted, in (arrival, id) order once sorted
  std::vector<int> running;  // admitted, unfinished, in admission order
  bool started = false;
  long long step = 0;
  long long finished = 0;

  int priv_blocks(const SReq& r) const { return cdiv(r.prompt_len + r.out_len, bs); }

  // blocks an admission of r needs beyond what is free now
  long long admission_need(const SReq& r) const {
    long long need = priv_blocks(r);
    std::vector<int> seen;
    for (int s : r.spans) {
      if (!spans[s].blocks.empty() || std::find(seen.begin(), seen.end(), s) != seen.end())
        continue;
      seen.push_back(s);
      need += spans[s].nblk;
    }
    return need;
  }

  std::vector<int32_t> take(int n) {
    std::vector<int32_t> b(free_blocks.end() - n, free_blocks.end());
    std::reverse(b.begin(), b.end());
    free_blocks.resize(free_blocks.size() - (size_t)n);
    return b;
  }
  void give(std::vector<int32_t>& b) {
    for (size_t i = b.size(); i-- > 0;) free_blocks.push_back(b[i]);
    b.clear();
  }

  // Evict resident spans that no running request (and not `keep`) uses,
  // least recently used first, until `need` blocks are free.
  void evict_for(long long need, const SReq& keep) {
    while ((long long)free_blocks.size() < need) {
      int victim = -1;
      for (int s = 0; s < (int)spans.size(); ++s) {
        const SSpan& sp = spans[s];
        if (sp.blocks.empty() || sp.running_users > 0) continue;
        if (std::find(keep.spans.begin(), keep.spans.end(), s) != keep.spans.end()) continue;
        if (victim < 0 || sp.last_use < spans[victim].last_use) victim = s;
      }
      if (victim < 0) return;
      give(spans[victim].blocks);
      spans[victim].done = 0;
    }
  }

  void finish(int id) {
    SReq& r = reqs[id];
    r.phase = kFinished;
    give(r.priv);
    for (int s : r.spans) spans[s].running_users--;
    ++finished;
  }

  // phase after spans / prompt progress (kFinished handled by the caller)
  void advance(int id) {
    SReq& r = reqs[id];
    if (r.phase == kSpans) {
      bool all = true;
      for (int s : r.spans) all = all && spans[s].done == spans[s].len;
      if (all) r.phase = kPrompt;
    }
    if (r.phase == kPrompt && r.prompt_done == r.prompt_len) r.phase = kDecode;
    if (r.phase == kDecode && r.decoded == r.out_len) finish(id);
  }

  void admit() {
    size_t w = 0;
    while (w < waiting.size() && (int)running.size() < max_running) {
      const int id = waiting[w];
      SReq& r = reqs[id];
      if (r.arrival > step) break;
      const long long need = admission_need(r);
      if ((long long)free_blocks.size() < need) evict_for(need, r);
      if ((long long)free_blocks.size() < need) break;  // first come, first served
      for (int s : r.spans) {
        SSpan& sp = spans[s];
        if (sp.blocks.empty()) {
          sp.blocks = take(sp.nblk);
          sp.done = 0;
        }
        sp.running_users++;
      }
      r.priv = take(priv_blocks(r));
      r.phase = kSpans;
      running.push_back(id);
      ++w;
      advance(id);
    }
    waiting.erase(waiting.begin(), waiting.begin() + (long)w);
    running.erase(std::remove_if(running.begin(), running.end(),
                                 [&](int id) { return reqs[id].phase == kFinished; }),
                  running.end());
  }

  void add_decodes(std::vector<Entry>& e, int& left) {
    for (int id : running) {
      const SReq& r = reqs[id];
      if (r.phase != kDecode || left <= 0) continue;
      e.push_back({PIC_SEQ_DECODE, id, r.span_tokens + r.prompt_len + r.decoded, 1});
      --left;
    }
  }
  void add_prompts(std::vector<Entry>& e, int& left) {
    for (int id : running) {
      const SReq& r = reqs[id];
      if (r.phase != kPrompt || left <= 0) continue;
      const int n = std::min(r.prompt_len - r.prompt_done, left);
      e.push_back({PIC_SEQ_PROMPT, id, r.span_tokens + r.prompt_done, n});
      left -= n;
    }
  }
  void add_spans(std::vector<Entry>& e, int& left) {
    for (int id : running) {
      const SReq& r = reqs[id];
      if (r.phase != kSpans) continue;
      for (int s : r.spans) {
        SSpan& sp = spans[s];
        if (left <= 0) return;
        if (sp.done == sp.len || sp.in_step) continue;
        const int n = std::min(sp.len - sp.done, left);
        e.push_back({PIC_SEQ_SPAN, s, sp.done, n});
        sp.in_step = true;
        left -= n;
      }
    }
  }

  std::vector<Entry> build() {
    std::vector<Entry> e;
    int left = budget;
    bool spans_wait = false, prompts_wait = false;
    for (int id : running) {
      spans_wait = spans_wait || reqs[id].phase == kSpans;
      prompts_wait = prompts_wait || reqs[id].phase == kPrompt;
    }
    if (policy == PIC_SCHED_ISPS) {
      add_decodes(e, left);
      add_prompts(e, left);
      add_spans(e, left);
    } else if (spans_wait) {
      add_spans(e, left);
    } else if (prompts_wait) {
      add_prompts(e, left);
    } else {
      add_decodes(e, left);
    }
    for (SSpan& sp : spans) sp.in_step = false;
    return e;
  }

  int seq_len_blocks(const Entry& x) const { return cdiv(x.q_begin + x.q_len, bs); }

  // block id of key slot j of the entry's sequence
  int32_t block_of(const Entry& x, int blk) const {
    if (x.kind == PIC_SEQ_SPAN) return spans[x.id].blocks[(size_t)blk];
    const SReq& r = reqs[x.id];
    for (int s : r.spans) {
      if (blk < spans[s].nblk) return spans[s].blocks[(size_t)blk];
      blk -= spans[s].nblk;
    }
    return r.priv[(size_t)blk];
  }
};

}  // namespace pic

using pic::Sched;

extern "C" int pic_sched_create(int policy, int token_budget, int max_running, int num_blocks,
                                int block_size, pic_sched** out) {
  if (!out) return PIC_EINVAL;
  *out = nullptr;
  if ((policy != PIC_SCHED_ISPS && policy != PIC_SCHED_BARRIER) || token_budget <= 0 ||
      max_running <= 0 || num_blocks <= 0 || block_size != pic::kBlockSize)
    return PIC_EINVAL;
  Sched* s = new (std::nothrow) Sched();
  if (!s) return PIC_EINVAL;
  s->policy = policy;
  s->budget = token_budget;
  s->max_running = max_running;
  s->num_blocks = num_blocks;
  s->bs = block_size;
  try {
    s->free_blocks.reserve((size_t)num_blocks);
    for (int b = num_blocks - 1; b >= 0; --b) s->free_blocks.push_back(b);
  } catch (...) {
    delete s;
    return PIC_EINVAL;
  }
  *out = reinterpret_cast<pic_sched*>(s);
  return PIC_OK;
}

extern "C" void pic_sched_destroy(pic_sched* h) { delete reinterpret_cast<Sched*>(h); }

extern "C" int pic_sched_add_span(pic_sched* h, int length) {
  Sched* s = reinterpret_cast<Sched*>(h);
  if (!s || s->started || length <= 0 || length % s->bs != 0) return PIC_EINVAL;
  try {
    pic::SSpan sp;
    sp.len = length;
    sp.nblk = length / s->bs;
    s->spans.push_back(sp);
  } catch (...) {
    return PIC_EINVAL;
  }
  return (int)s->spans.size() - 1;
}

extern "C" int pic_sched_add_request(pic_sched* h, long long arrival_step, const int32_t* span_ids,
                                     int num_spans, int prompt_len, int output_len) {
  Sched* s = reinterpret_cast<Sched*>(h);
  if (!s || s->started || arrival_step < 0 || num_spans < 0 || prompt_len < 0 ||
      output_len < 0 || (num_spans > 0 && !span_ids))
    return PIC_EINVAL;
  if (num_spans == 0 && prompt_len == 0) return PIC_EINVAL;  // nothing to attend to
  try {
    pic::SReq r;
    r.arrival = arrival_step;
    long long tokens = 0;
    for (int i = 0; i < num_spans; ++i) {
      const int id = span_ids[i];
      if (id < 0 || id >= (int)s->spans.size()) return PIC_EINVAL;
      r.spans.push_back(id);
      tokens += s->spans[(size_t)id].len;
    }
    tokens += (long long)prompt_len + output_len;
    if (tokens > (1LL << 30)) return PIC_EINVAL;
    r.span_tokens = (int)(tokens - prompt_len - output_len);
    r.prompt_len = prompt_len;
    r.out_len = output_len;
    // it must fit the pool on its own (then it is admitted at the latest
    // once nothing else runs)
    if (s->admission_need(r) > s->num_blocks) return PIC_EINVAL;
    s->reqs.push_back(r);
    s->waiting.push_back((int)s->reqs.size() - 1);
  } catch (...) {
    return PIC_EINVAL;
  }
  return (int)s->reqs.size() - 1;
}

extern "C" int pic_sched_step(pic_sched* h, pic_sched_batch* b) {
  Sched* s = reinterpret_cast<Sched*>(h);
  if (!s || !b) return PIC_EINVAL;
  if (!s->started) {
    std::stable_sort(s->waiting.begin(), s->waiting.end(), [&](int x, int y) {
      return s->reqs[(size_t)x].arrival < s->reqs[(size_t)y].arrival;
    });
    s->started = true;
  }
  if (s->waiting.empty() && s->running.empty()) return 0;
  if (!b->cu_seqlens_q || !b->q_pos || !b->slot_mapping || !b->seq_lens || !b->cu_seqlens_k ||
      !b->k_pos || !b->block_table || !b->seq_kind || !b->seq_id || !b->q_begin ||
      b->max_seqs < 0 || b->max_rows < 0 || b->max_keys < 0 || b->block_table_stride < 0)
    return PIC_EINVAL;
  std::vector<pic::Entry> e;
  const long long fin0 = s->finished;
  // Everything up to here leaves the state unchanged when a capacity check
  // below fails; admission does not, so it runs on a copy first.
  try {
    Sched trial = *s;
    trial.admit();
    e = trial.build();
    long long rows = 0, keys = 0;
    for (const auto& x : e) {
      rows += x.q_len;
      keys += x.q_begin + x.q_len;
      if (trial.seq_len_blocks(x) > b->block_table_stride) return PIC_EINVAL;
    }
    if ((long long)e.size() > b->max_seqs || rows > b->max_rows || keys > b->max_keys)
      return PIC_EINVAL;
    *s = std::move(trial);
  } catch (...) {
    return PIC_EINVAL;
  }
  // metadata of the step
  int row = 0, max_q = 0, max_k = 0;
  long long key = 0;
  b->cu_seqlens_q[0] = 0;
  b->cu_seqlens_k[0] = 0;
  for (size_t i = 0; i < e.size(); ++i) {
    const pic::Entry& x = e[i];
    const int L = x.q_begin + x.q_len;
    int32_t* bt = b->block_table + i * (size_t)b->block_table_stride;
    const int nblk = s->seq_len_blocks(x);
    for (int k = 0; k < b->block_table_stride; ++k) bt[k] = k < nblk ? s->block_of(x, k) : 0;
    for (int j = 0; j < L; ++j) b->k_pos[key + j] = j;
    for (int t = 0; t < x.q_len; ++t) {
      const int c = x.q_begin + t;  // slot index of the token in its sequence
      b->q_pos[row + t] = c;
      b->slot_mapping[row + t] = bt[c / s->bs] * s->bs + c % s->bs;
    }
    b->seq_kind[i] = x.kind;
    b->seq_id[i] = x.id;
    b->q_begin[i] = x.q_begin;
    b->seq_lens[i] = L;
    row += x.q_len;
    key += L;
    b->cu_seqlens_q[i + 1] = row;
    b->cu_seqlens_k[i + 1] = (int32_t)key;
    max_q = std::max(max_q, x.q_len);
    max_k = std::max(max_k, L);
  }
  b->step = s->step;
  b->num_seqs = (int)e.size();
  b->total_q = row;
  b->max_q_len = max_q;
  b->max_seq_len = max_k;
  b->total_keys = key;
  // commit the step's progress, then move phases on
  for (const auto& x : e) {
    if (x.kind == PIC_SEQ_SPAN) {
      s->spans[(size_t)x.id].done += x.q_len;
    } else if (x.kind == PIC_SEQ_PROMPT) {
      s->reqs[(size_t)x.id].prompt_done += x.q_len;
    } else {
      s->reqs[(size_t)x.id].decoded += 1;
    }
  }
  for (int id : s->running) {
    for (int sp : s->reqs[(size_t)id].spans) s->spans[(size_t)sp].last_use = s->step;
    s->advance(id);
  }
  s->running.erase(std::remove_if(s->running.begin(), s->running.end(),
                                  [&](int id) { return s->reqs[(size_t)id].phase == pic::kFinished; }),
                   s->running.end());
  b->num_finished = (int)(s->finished - fin0);
  s->step++;
  return 1;
}
