/*
 * pa_sched.h -- C ABI of the host-side KV block manager and step scheduler
 * in libpa.so (plain C++ on the CPU; no GPU call is made by anything here).
 *
 * It produces, step by step, the metadata the attention entry points of
 * pa.h consume (query_start_loc, num_computed_tokens, seq_lens, block_table,
 * plus the block copies pa_copy_blocks must run first), from a stream of
 * requests, following the pages' V1-style engine:
 *   [P1] "vLLM 架构源码解析（一）：从 API 请求到 Token 生成" §3.2, §4.3
 *   [P2] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
 *        §3.3, §3.5, §3.6
 *   [P3] the nano-vllm walk-through on blog.mospan.cn, block manager section
 *   [P4] "vllm v1 源码精读（三）：KV Cache 管理、Chunked Prefill 与异步架构"
 *        §3.3 - §3.6, §4.2, §4.3
 *
 * Model (each rule with its source):
 *   - Block pool: every block has a reference count and, once it is full and
 *     computed, a content hash ([P4] §3.3).  Unreferenced blocks sit in one
 *     free queue, unhashed ones toward the head, hashed ones (prefix-cache
 *     candidates) toward the tail; new blocks come from the head, which
 *     evicts a hashed block's cache entry ([P4] §3.3, §3.6).  A request's
 *     blocks are released last block first.
 *   - Block hash k = XXH64 (seed 0) of [hash k-1 as 8 little-endian bytes,
 *     omitted for k = 0] followed by the block's token ids as 4-byte
 *     little-endian integers; full blocks only ([P4] §3.5; [P2] §3.6;
 *     XXH64 as named by [P3]).
 *   - Prefix caching: at admission, a request's full blocks are looked up in
 *     order until the first miss; hits are shared (reference + 1) and
 *     num_computed_tokens starts at hits * block_size ([P4] §3.5).  At least
 *     one prompt token is always left to compute.  A hit needs the block's
 *     hash and its own token ids (kept with each hashed block) to match, so
 *     two blocks whose 64-bit hashes collide are never shared by mistake;
 *     the parent chain is followed through the hashes.
 *   - A step ([P4] §4.2; [P2] §3.3; [P1] §3.2): one token budget
 *     (max_num_batched_tokens) shared by all requests.  Running requests
 *     first, in order: new tokens = min(remaining, threshold if set, budget,
 *     max_model_len - computed); blocks = ceil((computed + new) / block_size)
 *     ([P2] §3.3); if the pool cannot cover them the newest running request
 *     is preempted (blocks freed, computed reset to 0, front of the waiting
 *     queue: [P1] §3.2, [P4] §4.3) and allocation is retried.  Then, if no
 *     request was preempted, waiting requests in arrival order while budget
 *     and sequence slots remain; without chunked prefill a request that does
 *     not fit whole ends admission for the step ([P4] §4.2).
 *   - Copy-on-write ([P1] §4.3.2): before a request writes into a block that
 *     another request shares, it gets a fresh copy (reported as a (src, dst)
 *     pair for pa_copy_blocks).
 *   - After the step ([P4] §3.6): computed counts advance; a request whose
 *     step reached the end of its tokens appends the sampled token; full
 *     computed blocks get their hashes registered; finished requests
 *     (max_new_tokens generated) release their blocks.
 *
 * Conventions: all pointers are HOST pointers owned by the caller; calls
 * are not thread-safe on one handle (one scheduler per engine thread);
 * status codes are pa_status values from pa.h, plus PA_SCHED_* below.
 */
#ifndef PA_SCHED_H_
#define PA_SCHED_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched; /* opaque */

#define PA_SCHED_ERR_UNKNOWN_REQUEST (-10) /* no request with that id        */
#define PA_SCHED_ERR_DUPLICATE (-11)       /* request id already in use      */
#define PA_SCHED_ERR_ORDER (-12)           /* update without schedule, etc.  */

typedef struct {
  int32_t num_blocks;                   /* blocks in the pool (>= 1)         */
  int32_t block_size;                   /* tokens per block (>= 1)           */
  int32_t max_num_batched_tokens;       /* token budget per step (>= 1)      */
  int32_t max_num_seqs;                 /* running requests at most (>= 1)   */
  int32_t max_model_len;                /* positions per request (>= 1)      */
  int32_t long_prefill_token_threshold; /* per-request chunk cap; 0 = none   */
  int32_t enable_chunked_prefill;       /* 0 / 1                             */
  int32_t enable_prefix_caching;        /* 0 / 1                             */
} pa_sched_config;

/* Output buffers of one step, allocated by the caller with at least the
 * capacities named (checked by pa_sched_schedule before anything changes). */
typedef struct {
  /* in: buffers */
  int64_t* request_ids;     /* [max_num_seqs] scheduled requests, batch order */
  int32_t* query_start_loc; /* [max_num_seqs + 1] prefix sums of new tokens    */
  int32_t* num_computed;    /* [max_num_seqs] tokens cached before this step   */
  int32_t* seq_lens;        /* [max_num_seqs] num_computed + new tokens        */
  int32_t* block_table;     /* [max_num_seqs * block_table_stride], -1 padded  */
  int32_t* token_ids;       /* [max_num_batched_tokens] the step's input ids   */
  int32_t* copy_pairs;      /* [max_num_seqs * 2] (src, dst) block copies      */
  int64_t* preempted_ids;   /* [max_num_seqs] requests preempted this step     */
  int32_t block_table_stride; /* >= ceil(max_model_len / block_size)           */
  /* out: sizes */
  int32_t num_seqs, num_tokens, max_query_len, max_seq_len;
  int32_t num_copies, num_preempted;
} pa_sched_step;

typedef struct {
  int32_t num_free_blocks, num_cached_blocks;
  int32_t num_running, num_waiting, num_finished;
  int64_t total_preemptions, total_prefix_hit_tokens, total_scheduled_tokens;
  int64_t total_steps;
} pa_sched_stats;

typedef struct {
  int32_t status;          /* 0 waiting, 1 running, 2 finished */
  int32_t num_tokens;      /* prompt + generated               */
  int32_t num_computed;
  int32_t num_generated;
  int32_t num_blocks;
  int32_t prompt_len;
} pa_sched_request_info;

/* Create / destroy a scheduler.  *out receives the handle. */
int pa_sched_create(const pa_sched_config* config, pa_sched** out);
void pa_sched_destroy(pa_sched* s);

/* Queue a request (its prompt is copied).  Requires prompt_len >= 1,
 * max_new_tokens >= 1 and prompt_len + max_new_tokens - 1 <= max_model_len
 * (the last sampled token is never written to the cache). */
int pa_sched_add_request(pa_sched* s, int64_t request_id, const int32_t* prompt,
                         int32_t prompt_len, int32_t max_new_tokens);

/* Parallel sampling ([P1] §4.3.2): start request child_id as another sample
 * of running request parent_id, sharing all its blocks.  Returns 1 if forked;
 * 0 (nothing changes) if the parent is not running, still prefilling, has
 * already generated max_new_tokens, or max_num_seqs requests are running. */
int pa_sched_fork(pa_sched* s, int64_t parent_id, int64_t child_id, int32_t max_new_tokens);

/* Plan one step into *step (see pa_sched_step).  A step with no work has
 * num_seqs = 0.  Every call must be followed by pa_sched_update. */
int pa_sched_schedule(pa_sched* s, pa_sched_step* step);

/* Finish the planned step.  sampled[i] is the token the i-th scheduled
 * request samples if the step reached the end of its tokens (ignored for
 * requests still prefilling).  Ids of requests that finished are written to
 * finished_ids (capacity >= the step's num_seqs), their count to
 * *num_finished. */
int pa_sched_update(pa_sched* s, const int32_t* sampled, int32_t num_seqs,
                    int64_t* finished_ids, int32_t* num_finished);

/* Inspection (tests, monitoring). */
int pa_sched_get_stats(const pa_sched* s, pa_sched_stats* out);
int pa_sched_get_request(const pa_sched* s, int64_t request_id, pa_sched_request_info* out,
                         int32_t* blocks, int32_t blocks_capacity);
/* Free queue from head to tail into out[capacity]; *count = its length. */
int pa_sched_get_free_queue(const pa_sched* s, int32_t* out, int32_t capacity,
                            int32_t* count);
/* Reference count and hash of one block (*has_hash = 0 if it has none). */
int pa_sched_get_block(const pa_sched* s, int32_t block_id, int32_t* ref_cnt, uint64_t* hash,
                       int32_t* has_hash);

/* XXH64 of len bytes (the published xxHash 64-bit algorithm). */
uint64_t pa_xxh64(const void* data, size_t len, uint64_t seed);
/* Chained block hash as above: parent is ignored when has_parent == 0. */
uint64_t pa_block_hash(uint64_t parent, int32_t has_parent, const int32_t* tokens,
                       int32_t num_tokens);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H_ */
