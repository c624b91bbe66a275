/*
 * pa_engine.h -- C ABI of the multi-step driver in libpa.so: the scheduler
 * of pa_sched.h planning each step and the kernels of pa.h executing it, in
 * one native call per step.
 *
 * One step ("vllm v1 源码精读（三）" §3.6 steps 2-3; "Inside vLLM" §3.3-§3.4),
 * all on the caller's stream:
 *   1. pa_sched_schedule into one of two page-locked metadata arenas owned by
 *      the engine (the arena is reused only after its previous copy ended);
 *   2. one asynchronous host-to-device copy of the arena's used prefix:
 *      [query_start_loc | num_computed | seq_lens | copy pairs | block table];
 *   3. pa_copy_blocks for the step's copy-on-write pairs, if any
 *      ("vLLM 架构源码解析（一）" §4.3.2);
 *   4. pa_cache_and_attend_mixed over the packed batch: the slot of every
 *      new token and the store of its K/V ("vllm v1 源码精读（三）" §3.4) in
 *      the same launch as the attention (same page, §4.2), which reads the
 *      new rows from k / v; the slots land in the device scratch.
 * The caller owns the KV cache and one device scratch buffer (sized by
 * pa_engine_device_bytes); the engine owns its scheduler, its page-locked
 * host arenas (allocated at creation) and two HIP events.  After each step
 * the caller reports the sampled tokens with pa_engine_update.  All steps of
 * one engine go to the same stream: the device copy of the metadata is
 * reused in stream order.  An engine is not thread-safe.
 */
#ifndef PA_ENGINE_H_
#define PA_ENGINE_H_

#include <stddef.h>
#include <stdint.h>

#include "pa_sched.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_engine pa_engine; /* opaque */

typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;    /* 64 or 128 */
  int32_t dtype;       /* pa_dtype; PA_F32 has no prefill path */
  float scale;         /* softmax scale, > 0 */
  int32_t num_splits;  /* decode partitions, 0 = library choice */
} pa_engine_geometry;

/* Bytes of device scratch an engine needs: the metadata arena, the slot
 * mapping and the attention workspace at the configuration's bounds.
 * 0 if the configuration or geometry is invalid. */
size_t pa_engine_device_bytes(const pa_sched_config* config, const pa_engine_geometry* geometry);

/* kv_cache: [config->num_blocks, 2, block_size, num_kv_heads, head_dim]
 * device memory (block_size must be 16); device_scratch: >= the bytes above,
 * 256-byte aligned.  Both stay owned by the caller and must outlive the
 * engine. */
int pa_engine_create(const pa_sched_config* config, const pa_engine_geometry* geometry,
                     void* kv_cache, void* device_scratch, size_t device_scratch_bytes,
                     pa_engine** out);
void pa_engine_destroy(pa_engine* e);

/* The engine's scheduler, for pa_sched_add_request / pa_sched_fork /
 * pa_sched_get_*.  Do not call pa_sched_schedule / pa_sched_update on it
 * directly. */
pa_sched* pa_engine_scheduler(pa_engine* e);

/* Plan and launch one step.  q [>= T, Hq, D], k and v [>= T, Hkv, D] and
 * out [>= T, Hq, D] are device buffers whose first T = step->num_tokens rows
 * are used (T <= max_num_batched_tokens).  On return *step describes the
 * plan: its pointers point into the engine's host arena and stay valid until
 * the step after next.  A step with num_seqs = 0 launches nothing. */
int pa_engine_step(pa_engine* e, const void* q, const void* k, const void* v, void* out,
                   void* stream, pa_sched_step* step);

/* pa_sched_update for the last step (same arguments). */
int pa_engine_update(pa_engine* e, const int32_t* sampled, int32_t num_seqs,
                     int64_t* finished_ids, int32_t* num_finished);

#ifdef __cplusplus
}
#endif

#endif /* PA_ENGINE_H_ */
