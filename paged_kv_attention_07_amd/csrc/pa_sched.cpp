// Host-side KV block manager and step scheduler (the model and its sources
// are documented in include/pa_sched.h).
//
// Data structures are sized once from the pool and kept flat: per-block
// arrays for reference counts, hashes and the free queue's links (an
// intrusive doubly linked list, so a prefix-cache hit is pulled out of the
// middle in O(1), "vllm v1 源码精读（三）" §3.3), an open hash map from block
// hash to block id, and per-request token / block vectors with their block
// hashes memoised (a block's tokens never change once it is full).
#include <stdint.h>
#include <string.h>

#include <deque>
#include <memory>
#include <unordered_map>
#include <vector>

#include "pa.h"
#include "pa_sched.h"

// ---------------------------------------------------------------------------
// XXH64, written from the published xxHash specification (64-bit variant).
// ---------------------------------------------------------------------------
namespace {

constexpr uint64_t kP1 = 0x9E3779B185EBCA87ull;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4Full;
constexpr uint64_t kP3 = 0x165667B19E3779F9ull;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ull;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ull;

inline uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

inline uint64_t read_le64(const uint8_t* p) {
  uint64_t v;
  memcpy(&v, p, 8);  // x86-64 and the GPU hosts are little-endian
  return v;
}

inline uint32_t read_le32(const uint8_t* p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}

inline uint64_t xxh_round(uint64_t acc, uint64_t lane) {
  acc += lane * kP2;
  acc = rotl64(acc, 31);
  return acc * kP1;
}

inline uint64_t xxh_merge(uint64_t acc, uint64_t v) {
  acc ^= xxh_round(0, v);
  return acc * kP1 + kP4;
}

uint64_t xxh64(const uint8_t* p, size_t len, uint64_t seed) {
  const uint8_t* const end = p + len;
  uint64_t acc;
  if (len >= 32) {
    uint64_t v[4] = {seed + kP1 + kP2, seed + kP2, seed, seed - kP1};
    const uint8_t* const limit = end - 32;
    do {
      for (int i = 0; i < 4; ++i) v[i] = xxh_round(v[i], read_le64(p + 8 * i));
      p += 32;
    } while (p <= limit);
    acc = rotl64(v[0], 1) + rotl64(v[1], 7) + rotl64(v[2], 12) + rotl64(v[3], 18);
    for (int i = 0; i < 4; ++i) acc = xxh_merge(acc, v[i]);
  } else {
    acc = seed + kP5;
  }
  acc += (uint64_t)len;
  for (; p + 8 <= end; p += 8) {
    acc ^= xxh_round(0, read_le64(p));
    acc = rotl64(acc, 27) * kP1 + kP4;
  }
  if (p + 4 <= end) {
    acc ^= (uint64_t)read_le32(p) * kP1;
    acc = rotl64(acc, 23) * kP2 + kP3;
    p += 4;
  }
  for (; p < end; ++p) {
    acc ^= (uint64_t)(*p) * kP5;
    acc = rotl64(acc, 11) * kP1;
  }
  acc ^= acc >> 33;
  acc *= kP2;
  acc ^= acc >> 29;
  acc *= kP3;
  acc ^= acc >> 32;
  return acc;
}

// Test builds narrow the hash (e.g. -DPA_SCHED_HASH_MASK=0x3f) so that
// different blocks collide often; the product keeps all 64 bits.
#ifndef PA_SCHED_HASH_MASK
#define PA_SCHED_HASH_MASK (~(uint64_t)0)
#endif

uint64_t block_hash(uint64_t parent, bool has_parent, const int32_t* tokens, int n) {
  // parent (8 bytes) + the block's tokens; blocks are small, so one buffer
  uint8_t stack_buf[8 + 4 * 64];
  std::vector<uint8_t> heap;
  uint8_t* buf = stack_buf;
  const size_t bytes = (has_parent ? 8 : 0) + 4 * (size_t)n;
  if (bytes > sizeof(stack_buf)) {
    heap.resize(bytes);
    buf = heap.data();
  }
  size_t o = 0;
  if (has_parent) {
    memcpy(buf, &parent, 8);
    o = 8;
  }
  memcpy(buf + o, tokens, 4 * (size_t)n);
  return xxh64(buf, bytes, 0) & (uint64_t)PA_SCHED_HASH_MASK;
}

// ---------------------------------------------------------------------------
// scheduler state
// ---------------------------------------------------------------------------
enum Status { kWaiting = 0, kRunning = 1, kFinished = 2 };

struct Request {
  int64_t id;
  std::vector<int32_t> tokens;
  int32_t prompt_len, max_new, num_generated = 0, num_computed = 0;
  std::vector<int32_t> blocks;
  std::vector<uint64_t> hashes;  // memoised hashes of the first full blocks
  int32_t num_hashed = 0;        // table prefix known to carry hashes
  Status status = kWaiting;
};

struct Scheduled {
  Request* r;
  int32_t before, num_new;
};

}  // namespace

struct pa_sched {
  pa_sched_config cfg;
  // block pool
  std::vector<int32_t> ref, prev, next;
  std::vector<uint64_t> hash;
  std::vector<int32_t> tok;  // token ids of each hashed block (block_size per block)
  std::vector<uint8_t> has_hash, in_free;
  int32_t head = -1, tail = -1, num_free = 0;
  std::unordered_map<uint64_t, int32_t> cached;
  // requests
  std::unordered_map<int64_t, std::unique_ptr<Request>> requests;
  std::vector<Request*> running;
  std::deque<Request*> waiting;
  std::vector<Scheduled> sched;
  bool planned = false;
  // statistics
  int64_t preemptions = 0, prefix_hit_tokens = 0, scheduled_tokens = 0, steps = 0;
  int32_t finished = 0;

  // ---- free queue (intrusive doubly linked list over block ids)
  void unlink(int32_t b) {
    const int32_t p = prev[b], n = next[b];
    (p >= 0 ? next[p] : head) = n;
    (n >= 0 ? prev[n] : tail) = p;
    prev[b] = next[b] = -1;
    in_free[b] = 0;
    --num_free;
  }
  void push_front(int32_t b) {
    prev[b] = -1;
    next[b] = head;
    (head >= 0 ? prev[head] : tail) = b;
    head = b;
    in_free[b] = 1;
    ++num_free;
  }
  void push_back(int32_t b) {
    next[b] = -1;
    prev[b] = tail;
    (tail >= 0 ? next[tail] : head) = b;
    tail = b;
    in_free[b] = 1;
    ++num_free;
  }

  // a block for new content: the head of the free queue; its cached
  // content (if any) is evicted
  int32_t take_fresh() {
    const int32_t b = head;
    unlink(b);
    if (has_hash[b]) {
      auto it = cached.find(hash[b]);
      if (it != cached.end() && it->second == b) cached.erase(it);
      has_hash[b] = 0;
    }
    ref[b] = 1;
    return b;
  }
  void take_cached(int32_t b) {
    if (ref[b] == 0) unlink(b);
    ++ref[b];
  }
  void release(std::vector<int32_t>& blocks) {
    for (auto it = blocks.rbegin(); it != blocks.rend(); ++it) {
      const int32_t b = *it;
      if (--ref[b] == 0) {
        if (has_hash[b]) push_back(b); else push_front(b);
      }
    }
    blocks.clear();
  }

  // ---- hashing
  uint64_t hash_of(Request* r, int k) {
    const int B = cfg.block_size;
    while ((int)r->hashes.size() <= k) {
      const int j = (int)r->hashes.size();
      const uint64_t parent = j ? r->hashes[j - 1] : 0;
      r->hashes.push_back(block_hash(parent, j > 0, r->tokens.data() + (size_t)j * B, B));
    }
    return r->hashes[k];
  }

  // ---- one step
  int32_t cap(int32_t computed, int32_t num_new, int32_t budget) const {
    if (cfg.long_prefill_token_threshold > 0 && cfg.long_prefill_token_threshold < num_new)
      num_new = cfg.long_prefill_token_threshold;
    if (num_new > budget) num_new = budget;
    const int32_t room = cfg.max_model_len - computed;
    return num_new < room ? num_new : room;
  }

  bool allocate_slots(Request* r, int32_t num_new, std::vector<int32_t>& copies) {
    const int B = cfg.block_size;
    const int32_t need_total = (r->num_computed + num_new + B - 1) / B;
    const int32_t need_new = need_total - (int32_t)r->blocks.size();
    int32_t shared = 0;
    for (size_t j = r->num_computed / B; j < r->blocks.size(); ++j) shared += ref[r->blocks[j]] > 1;
    if (num_free < need_new + shared) return false;
    if (shared) {
      for (size_t j = r->num_computed / B; j < r->blocks.size(); ++j) {
        const int32_t src = r->blocks[j];
        if (ref[src] <= 1) continue;
        const int32_t dst = take_fresh();
        --ref[src];
        r->blocks[j] = dst;
        copies.push_back(src);
        copies.push_back(dst);
      }
    }
    for (int32_t i = 0; i < need_new; ++i) r->blocks.push_back(take_fresh());
    return true;
  }

  void preempt(Request* r) {
    release(r->blocks);
    r->num_computed = 0;
    r->num_hashed = 0;
    r->status = kWaiting;
    waiting.push_front(r);
    ++preemptions;
  }

  // leading run of cached full blocks, leaving at least one token to compute;
  // a hit needs the hash and the block's own token ids to match, so two
  // blocks whose hashes collide are never mistaken for one another (the
  // chain is taken on the hash alone: a cached block's parent is the block
  // with the parent's hash)
  void prefix_hits(Request* r, std::vector<int32_t>& hits) {
    hits.clear();
    const int B = cfg.block_size;
    const int usable = ((int)r->tokens.size() - 1) / B;
    for (int k = 0; k < usable; ++k) {
      auto it = cached.find(hash_of(r, k));
      if (it == cached.end() ||
          memcmp(tok.data() + (size_t)it->second * B, r->tokens.data() + (size_t)k * B,
                 sizeof(int32_t) * B) != 0)
        break;
      hits.push_back(it->second);
    }
  }

  void cache_blocks(Request* r) {
    const int full = r->num_computed / cfg.block_size;
    for (int k = r->num_hashed; k < full; ++k) {
      const int32_t b = r->blocks[k];
      if (has_hash[b]) continue;
      const uint64_t h = hash_of(r, k);
      hash[b] = h;
      has_hash[b] = 1;
      memcpy(tok.data() + (size_t)b * cfg.block_size, r->tokens.data() + (size_t)k * cfg.block_size,
             sizeof(int32_t) * cfg.block_size);
      cached.emplace(h, b);  // an existing entry keeps its block
    }
    if (full > r->num_hashed) r->num_hashed = full;
  }
};

namespace {

bool config_ok(const pa_sched_config& c) {
  return c.num_blocks >= 1 && c.block_size >= 1 && c.block_size <= 4096 &&
         c.max_num_batched_tokens >= 1 && c.max_num_seqs >= 1 && c.max_model_len >= 1 &&
         c.long_prefill_token_threshold >= 0;
}

}  // namespace

extern "C" {

int pa_sched_create(const pa_sched_config* config, pa_sched** out) {
  if (!config || !out || !config_ok(*config)) return PA_ERR_INVALID_ARG;
  std::unique_ptr<pa_sched> s(new pa_sched());
  s->cfg = *config;
  const int32_t n = config->num_blocks;
  s->ref.assign(n, 0);
  s->prev.assign(n, -1);
  s->next.assign(n, -1);
  s->hash.assign(n, 0);
  s->tok.assign((size_t)n * config->block_size, 0);
  s->has_hash.assign(n, 0);
  s->in_free.assign(n, 0);
  for (int32_t b = 0; b < n; ++b) s->push_back(b);
  s->cached.reserve((size_t)n * 2);
  *out = s.release();
  return PA_OK;
}

void pa_sched_destroy(pa_sched* s) { delete s; }

int pa_sched_add_request(pa_sched* s, int64_t request_id, const int32_t* prompt,
                         int32_t prompt_len, int32_t max_new_tokens) {
  if (!s || !prompt || prompt_len < 1 || max_new_tokens < 1) return PA_ERR_INVALID_ARG;
  if ((int64_t)prompt_len + max_new_tokens - 1 > s->cfg.max_model_len) return PA_ERR_INVALID_ARG;
  if (s->requests.count(request_id)) return PA_SCHED_ERR_DUPLICATE;
  std::unique_ptr<Request> r(new Request());
  r->id = request_id;
  r->tokens.assign(prompt, prompt + prompt_len);
  r->tokens.reserve((size_t)prompt_len + max_new_tokens);
  r->prompt_len = prompt_len;
  r->max_new = max_new_tokens;
  s->waiting.push_back(r.get());
  s->requests.emplace(request_id, std::move(r));
  return PA_OK;
}

int pa_sched_fork(pa_sched* s, int64_t parent_id, int64_t child_id, int32_t max_new_tokens) {
  if (!s || max_new_tokens < 1) return PA_ERR_INVALID_ARG;
  if (s->planned) return PA_SCHED_ERR_ORDER;
  if (s->requests.count(child_id)) return PA_SCHED_ERR_DUPLICATE;
  auto it = s->requests.find(parent_id);
  if (it == s->requests.end()) return 0;
  Request* p = it->second.get();
  if (p->status != kRunning || p->num_computed != (int32_t)p->tokens.size() - 1 ||
      p->num_generated >= max_new_tokens || (int32_t)s->running.size() >= s->cfg.max_num_seqs)
    return 0;
  if ((int64_t)p->prompt_len + max_new_tokens - 1 > s->cfg.max_model_len)
    return PA_ERR_INVALID_ARG;
  std::unique_ptr<Request> c(new Request(*p));
  c->id = child_id;
  c->max_new = max_new_tokens;
  for (int32_t b : c->blocks) ++s->ref[b];
  s->running.push_back(c.get());
  s->requests.emplace(child_id, std::move(c));
  return 1;
}

int pa_sched_schedule(pa_sched* s, pa_sched_step* st) {
  if (!s || !st) return PA_ERR_INVALID_ARG;
  if (s->planned) return PA_SCHED_ERR_ORDER;
  const pa_sched_config& c = s->cfg;
  const int B = c.block_size;
  const int32_t width = (c.max_model_len + B - 1) / B;
  if (!st->request_ids || !st->query_start_loc || !st->num_computed || !st->seq_lens ||
      !st->block_table || !st->token_ids || !st->copy_pairs || !st->preempted_ids ||
      st->block_table_stride < width)
    return PA_ERR_INVALID_ARG;

  int32_t budget = c.max_num_batched_tokens;
  std::vector<Scheduled>& sched = s->sched;
  sched.clear();
  std::vector<int32_t> copies;
  int32_t npre = 0;

  // running requests first, in order
  for (size_t i = 0; i < s->running.size() && budget > 0;) {
    Request* r = s->running[i];
    const int32_t num_new = s->cap(r->num_computed, (int32_t)r->tokens.size() - r->num_computed,
                                   budget);
    if (num_new <= 0) {
      ++i;
      continue;
    }
    bool self_preempted = false;
    while (!s->allocate_slots(r, num_new, copies)) {
      Request* victim = s->running.back();
      s->running.pop_back();
      s->preempt(victim);
      st->preempted_ids[npre++] = victim->id;
      if (victim == r) {
        self_preempted = true;
        break;
      }
    }
    if (self_preempted) break;
    sched.push_back({r, r->num_computed, num_new});
    budget -= num_new;
    ++i;
  }
  // then waiting requests, unless this step preempted
  if (npre == 0) {
    std::vector<int32_t> hits;
    while (!s->waiting.empty() && budget > 0 && (int32_t)s->running.size() < c.max_num_seqs) {
      Request* r = s->waiting.front();
      hits.clear();
      if (c.enable_prefix_caching && r->num_computed == 0) s->prefix_hits(r, hits);
      const int32_t start = (int32_t)hits.size() * B;
      const int32_t remaining = (int32_t)r->tokens.size() - start;
      const int32_t num_new = s->cap(start, remaining, budget);
      if (num_new <= 0 || (!c.enable_chunked_prefill && num_new < remaining)) break;
      const int32_t need_new = (start + num_new + B - 1) / B - (int32_t)hits.size();
      int32_t free_hits = 0;
      for (int32_t b : hits) free_hits += s->ref[b] == 0;
      if (s->num_free - free_hits < need_new) break;
      for (int32_t b : hits) s->take_cached(b);
      r->blocks.assign(hits.begin(), hits.end());
      r->num_computed = start;
      r->num_hashed = (int32_t)hits.size();
      s->prefix_hit_tokens += start;
      for (int32_t i = 0; i < need_new; ++i) r->blocks.push_back(s->take_fresh());
      s->waiting.pop_front();
      r->status = kRunning;
      s->running.push_back(r);
      sched.push_back({r, start, num_new});
      budget -= num_new;
    }
  }

  // step metadata
  int32_t t = 0, max_q = 0, max_L = 0;
  st->query_start_loc[0] = 0;
  for (size_t i = 0; i < sched.size(); ++i) {
    const Scheduled& e = sched[i];
    st->request_ids[i] = e.r->id;
    st->num_computed[i] = e.before;
    st->seq_lens[i] = e.before + e.num_new;
    if (e.num_new > 0)
      memcpy(st->token_ids + t, e.r->tokens.data() + e.before, sizeof(int32_t) * e.num_new);
    t += e.num_new;
    st->query_start_loc[i + 1] = t;
    int32_t* row = st->block_table + (int64_t)i * st->block_table_stride;
    const size_t nb = e.r->blocks.size();
    if (nb > 0) memcpy(row, e.r->blocks.data(), sizeof(int32_t) * nb);
    for (int32_t j = (int32_t)nb; j < st->block_table_stride; ++j) row[j] = -1;
    if (e.num_new > max_q) max_q = e.num_new;
    if (e.before + e.num_new > max_L) max_L = e.before + e.num_new;
  }
  // (an empty vector's data() may be null, and memcpy from null is undefined
  // even for zero bytes)
  if (!copies.empty()) memcpy(st->copy_pairs, copies.data(), sizeof(int32_t) * copies.size());
  st->num_seqs = (int32_t)sched.size();
  st->num_tokens = t;
  st->max_query_len = max_q;
  st->max_seq_len = max_L;
  st->num_copies = (int32_t)(copies.size() / 2);
  st->num_preempted = npre;
  s->scheduled_tokens += t;
  ++s->steps;
  s->planned = true;
  return PA_OK;
}

int pa_sched_update(pa_sched* s, const int32_t* sampled, int32_t num_seqs, int64_t* finished_ids,
                    int32_t* num_finished) {
  if (!s || !num_finished) return PA_ERR_INVALID_ARG;
  if (!s->planned) return PA_SCHED_ERR_ORDER;
  if (num_seqs != (int32_t)s->sched.size()) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!sampled || !finished_ids)) return PA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Request* r = s->sched[i].r;
    r->num_computed = s->sched[i].before + s->sched[i].num_new;
    if (r->num_computed == (int32_t)r->tokens.size()) {
      r->tokens.push_back(sampled[i]);
      if (++r->num_generated >= r->max_new) r->status = kFinished;
    }
    if (s->cfg.enable_prefix_caching) s->cache_blocks(r);
  }
  int32_t nf = 0;
  for (int32_t i = 0; i < num_seqs; ++i) {
    Request* r = s->sched[i].r;
    if (r->status != kFinished || r->blocks.empty()) continue;
    for (size_t j = 0; j < s->running.size(); ++j)
      if (s->running[j] == r) {
        s->running.erase(s->running.begin() + j);
        break;
      }
    s->release(r->blocks);
    r->hashes.clear();
    r->hashes.shrink_to_fit();
    finished_ids[nf++] = r->id;
    ++s->finished;
  }
  *num_finished = nf;
  s->sched.clear();
  s->planned = false;
  return PA_OK;
}

int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* out) {
  if (!s || !out) return PA_ERR_INVALID_ARG;
  out->num_free_blocks = s->num_free;
  out->num_cached_blocks = (int32_t)s->cached.size();
  out->num_running = (int32_t)s->running.size();
  out->num_waiting = (int32_t)s->waiting.size();
  out->num_finished = s->finished;
  out->total_preemptions = s->preemptions;
  out->total_prefix_hit_tokens = s->prefix_hit_tokens;
  out->total_scheduled_tokens = s->scheduled_tokens;
  out->total_steps = s->steps;
  return PA_OK;
}

int pa_sched_get_request(const pa_sched* s, int64_t request_id, pa_sched_request_info* out,
                         int32_t* blocks, int32_t blocks_capacity) {
  if (!s || !out) return PA_ERR_INVALID_ARG;
  auto it = s->requests.find(request_id);
  if (it == s->requests.end()) return PA_SCHED_ERR_UNKNOWN_REQUEST;
  const Request* r = it->second.get();
  out->status = r->status;
  out->num_tokens = (int32_t)r->tokens.size();
  out->num_computed = r->num_computed;
  out->num_generated = r->num_generated;
  out->num_blocks = (int32_t)r->blocks.size();
  out->prompt_len = r->prompt_len;
  if (blocks) {
    if (blocks_capacity < out->num_blocks) return PA_ERR_INVALID_ARG;
    if (!r->blocks.empty())
      memcpy(blocks, r->blocks.data(), sizeof(int32_t) * r->blocks.size());
  }
  return PA_OK;
}

int pa_sched_get_free_queue(const pa_sched* s, int32_t* out, int32_t capacity, int32_t* count) {
  if (!s || !count) return PA_ERR_INVALID_ARG;
  *count = s->num_free;
  if (!out) return PA_OK;
  if (capacity < s->num_free) return PA_ERR_INVALID_ARG;
  int32_t i = 0;
  for (int32_t b = s->head; b >= 0; b = s->next[b]) out[i++] = b;
  return PA_OK;
}

int pa_sched_get_block(const pa_sched* s, int32_t block_id, int32_t* ref_cnt, uint64_t* hash,
                       int32_t* has_hash) {
  if (!s || !ref_cnt || !hash || !has_hash) return PA_ERR_INVALID_ARG;
  if (block_id < 0 || block_id >= s->cfg.num_blocks) return PA_ERR_INVALID_ARG;
  *ref_cnt = s->ref[block_id];
  *has_hash = s->has_hash[block_id];
  *hash = s->has_hash[block_id] ? s->hash[block_id] : 0;
  return PA_OK;
}

uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed) {
  return xxh64(static_cast<const uint8_t*>(data), data ? len : 0, seed);
}

uint64_t pa_block_hash(uint64_t parent, int32_t has_parent, const int32_t* tokens,
                       int32_t num_tokens) {
  if (!tokens || num_tokens < 0) return 0;
  return block_hash(parent, has_parent != 0, tokens, num_tokens);
}

}  // extern "C"
