// Token-budget scheduler of chunked prefill (host code).
//
// Every iteration fills a token budget in a fixed priority order ("Chunked prefill (stall-free
// batching), explained", "How it works, step by step"): one token for every running decode; then
// the next chunk of the prompt already being prefilled, min(budget left, p - p_done) tokens from
// offset p_done; then waiting requests in arrival order while budget, sequence slots and KV blocks
// remain, each given as many prompt tokens as fit. A request whose last prompt chunk completes
// takes its first token from that iteration and decodes from the next one. The budget is fixed,
// or the iteration's prompt share follows chapter 7.8's dynamic chunk sizing ("Priority and
// Preemption Policies"): the largest chunk while nothing decodes, the smallest once decodes reach
// a pressure threshold, the straight line from the base chunk down to the smallest in between
// (rounded down to whole tokens); decode tokens come on top of that share.
//
// KV blocks (16 tokens each) come from one free pool shared by all layers' pools, lowest free id
// first. Reading of "the request can be allocated": a request is admitted only if blocks for its
// whole lifetime (prompt plus outputs) are free, and they are taken at admission, so no running
// request is ever preempted; they return to the pool when it finishes.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <functional>
#include <new>
#include <queue>
#include <vector>

#include "hybrid_layer.h"

namespace {

enum State { kWaiting, kPrefill, kDecode, kFinished };

struct Req {
  int32_t id, prompt_len, max_new;
  int32_t prefilled = 0, generated = 0, last_token = -1;
  State state = kWaiting;
  std::vector<int32_t> blocks;
};

int32_t blocks_for(int64_t tokens) { return (int32_t)((tokens + HL_BLOCK_SIZE - 1) / HL_BLOCK_SIZE); }

}  // namespace

struct hl_sched {
  hl_sched_params p;
  std::vector<Req> reqs;          // by handle (submission order)
  std::deque<int32_t> waiting;    // handles, arrival order
  std::vector<int32_t> prefill;   // handles being prefilled, admission order
  std::vector<int32_t> decoding;  // handles decoding, admission order
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_blocks;
  int64_t iteration = 0;
  // the last batch
  std::vector<int32_t> b_handle, q_start, num_cached, req_id, table, token, emits, n_new;
};

extern "C" {

hl_sched* hl_sched_create(const hl_sched_params* p) {
  if (!p || p->max_seqs < 1 || p->num_blocks < 1 || p->max_blocks_per_seq < 1) return nullptr;
  if (p->adaptive) {
    if (p->min_chunk < 1 || p->base_chunk < p->min_chunk || p->max_chunk < p->base_chunk ||
        p->pressure_threshold < 1)
      return nullptr;
  } else if (p->budget < 1) {
    return nullptr;
  }
  hl_sched* s = new (std::nothrow) hl_sched;
  if (!s) return nullptr;
  s->p = *p;
  for (int32_t i = 0; i < p->num_blocks; ++i) s->free_blocks.push(i);
  return s;
}

void hl_sched_destroy(hl_sched* s) { delete s; }

int hl_sched_submit(hl_sched* s, int32_t request_id, int32_t prompt_len, int32_t max_new_tokens,
                    int32_t* handle) {
  if (!s || !handle) return HL_ERR_NULL;
  if (prompt_len < 1 || max_new_tokens < 1) return HL_ERR_ARG;
  // a request whose lifetime outgrows its table row or the whole pool could never be admitted,
  // and arrival-order admission would then hold back every later request behind it
  const int32_t need = blocks_for((int64_t)prompt_len + max_new_tokens - 1);
  if (need > s->p.max_blocks_per_seq || need > s->p.num_blocks) return HL_ERR_BLOCK;
  Req r;
  r.id = request_id;
  r.prompt_len = prompt_len;
  r.max_new = max_new_tokens;
  *handle = (int32_t)s->reqs.size();
  s->reqs.push_back(std::move(r));
  s->waiting.push_back(*handle);
  return HL_OK;
}

// Prompt tokens the next iteration may carry after every decode has its one token. Adaptive:
// max_chunk at no decode load, min_chunk at or past the pressure threshold, and in between
// floor(base - d (base - min) / threshold) = base - ceil(d (base - min) / threshold), in exact
// integer arithmetic.
static int64_t prompt_share(const hl_sched* s) {
  const int64_t d = (int64_t)s->decoding.size();
  if (!s->p.adaptive) return (int64_t)s->p.budget - d;
  const hl_sched_params& p = s->p;
  if (d == 0) return p.max_chunk;
  if (d >= p.pressure_threshold) return p.min_chunk;
  const int64_t span = (int64_t)p.base_chunk - p.min_chunk;
  return p.base_chunk - (d * span + p.pressure_threshold - 1) / p.pressure_threshold;
}

int hl_sched_next(hl_sched* s, hl_sched_batch* out) {
  if (!s || !out) return HL_ERR_NULL;
  s->b_handle.clear();
  s->n_new.clear();
  int64_t left = prompt_share(s);
  // 1. every running decode: one token (on top of the prompt share)
  for (int32_t h : s->decoding) {
    s->b_handle.push_back(h);
    s->n_new.push_back(1);
  }
  // 2. prompts already being prefilled, then 3. admissions in arrival order
  for (int32_t h : s->prefill) {
    if (left <= 0) break;
    const Req& r = s->reqs[h];
    const int32_t n = (int32_t)std::min<int64_t>(left, r.prompt_len - r.prefilled);
    s->b_handle.push_back(h);
    s->n_new.push_back(n);
    left -= n;
  }
  while (left > 0 && !s->waiting.empty()) {
    const int32_t h = s->waiting.front();
    Req& r = s->reqs[h];
    if ((int32_t)(s->decoding.size() + s->prefill.size()) >= s->p.max_seqs) break;
    const int32_t need = blocks_for((int64_t)r.prompt_len + r.max_new - 1);
    if (need > (int32_t)s->free_blocks.size()) break;
    s->waiting.pop_front();
    for (int32_t i = 0; i < need; ++i) {
      r.blocks.push_back(s->free_blocks.top());
      s->free_blocks.pop();
    }
    r.state = kPrefill;
    s->prefill.push_back(h);
    const int32_t n = (int32_t)std::min<int64_t>(left, r.prompt_len);
    s->b_handle.push_back(h);
    s->n_new.push_back(n);
    left -= n;
  }
  // the batch in host arrays
  const size_t S = s->b_handle.size();
  const int32_t mb = s->p.max_blocks_per_seq;
  s->q_start.assign(S + 1, 0);
  s->num_cached.assign(S, 0);
  s->req_id.assign(S, 0);
  s->token.assign(S, -1);
  s->emits.assign(S, 0);
  s->table.assign(S * (size_t)mb, 0);
  for (size_t i = 0; i < S; ++i) {
    const Req& r = s->reqs[s->b_handle[i]];
    const int32_t n = s->n_new[i];
    s->q_start[i + 1] = s->q_start[i] + n;
    s->req_id[i] = r.id;
    if (r.state == kDecode) {
      s->num_cached[i] = r.prompt_len + r.generated - 1;
      s->token[i] = r.last_token;
      s->emits[i] = 1;
    } else {
      s->num_cached[i] = r.prefilled;
      s->emits[i] = (r.prefilled + n == r.prompt_len) ? 1 : 0;
    }
    std::copy(r.blocks.begin(), r.blocks.end(), s->table.begin() + i * mb);
  }
  out->num_seqs = (int32_t)S;
  out->num_tokens = s->q_start[S];
  out->q_start = s->q_start.data();
  out->num_cached = s->num_cached.data();
  out->request_ids = s->req_id.data();
  out->table = s->table.data();
  out->decode_tokens = s->token.data();
  out->emits = s->emits.data();
  out->max_blocks_per_seq = mb;
  return HL_OK;
}

int hl_sched_complete(hl_sched* s, const int32_t* next_tokens, int32_t* finished_ids,
                      int32_t* num_finished) {
  if (!s || !num_finished) return HL_ERR_NULL;
  const size_t S = s->b_handle.size();
  if (S && !next_tokens) return HL_ERR_NULL;
  int32_t nf = 0;
  for (size_t i = 0; i < S; ++i) {
    Req& r = s->reqs[s->b_handle[i]];
    if (r.state == kPrefill) {
      r.prefilled += s->n_new[i];
      if (r.prefilled < r.prompt_len) continue;
      r.generated = 1;  // first token from this pass
      r.last_token = next_tokens[i];
      s->prefill.erase(std::find(s->prefill.begin(), s->prefill.end(), s->b_handle[i]));
      r.state = kDecode;
      s->decoding.push_back(s->b_handle[i]);
    } else {
      r.generated += 1;
      r.last_token = next_tokens[i];
    }
    if (r.generated >= r.max_new) {
      r.state = kFinished;
      s->decoding.erase(std::find(s->decoding.begin(), s->decoding.end(), s->b_handle[i]));
      for (int32_t b : r.blocks) s->free_blocks.push(b);
      r.blocks.clear();
      if (finished_ids) finished_ids[nf] = r.id;
      ++nf;
    }
  }
  s->b_handle.clear();
  ++s->iteration;
  *num_finished = nf;
  return HL_OK;
}

int hl_sched_counts(const hl_sched* s, int32_t* waiting, int32_t* prefilling, int32_t* decoding,
                    int32_t* free_blocks) {
  if (!s) return HL_ERR_NULL;
  if (waiting) *waiting = (int32_t)s->waiting.size();
  if (prefilling) *prefilling = (int32_t)s->prefill.size();
  if (decoding) *decoding = (int32_t)s->decoding.size();
  if (free_blocks) *free_blocks = (int32_t)s->free_blocks.size();
  return HL_OK;
}

}  // extern "C"
