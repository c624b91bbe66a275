/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-KV-attention library (libpa.so).
 *
 * Sources for what each call computes (web pages, cited by title + section):
 *   [P1] "vLLM 架构源码解析（一）：从 API 请求到 Token 生成"
 *   [P2] "Inside vLLM: Anatomy of a High-Throughput LLM Inference System"
 *   [P4] "vllm v1 源码精读（三）：KV Cache 管理、Chunked Prefill 与异步架构"
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers owned by the caller unless marked (host).
 *     The library keeps no pointer after a call returns and never allocates.
 *     (The one exception, pa_cache_and_attend_mixed_no_workspace, uses a
 *     fixed-size scratch array the library holds in device memory instead of
 *     a caller's workspace.)
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and never synchronises.
 *   - Tensors are dense, row-major, with the shapes given below.
 *   - KV cache: one tensor [num_blocks, 2, block_size, num_kv_heads, head_dim]
 *     ([P4] §3.2/§3.3); kv_cache[b][0] is block b's K, kv_cache[b][1] its V.
 *     block_size must be 16; head_dim 64 or 128; dtype one of pa_dtype.
 *     Queries, new keys/values and outputs have the cache's dtype.
 *   - `scale` (the softmax scale, 1/sqrt(head_dim) on the pages) must be a
 *     finite number > 0; zero, negative or non-finite scales return
 *     PA_ERR_INVALID_ARG.
 *   - Host-visible arguments (sizes, dtype, alignment, workspace size) are
 *     checked before anything is launched; a failed check launches nothing
 *     and returns a negative pa_status.  Device-resident metadata (tables,
 *     lengths, slots) is trusted, as the pages' model runner trusts its
 *     scheduler: preconditions are listed per call; violating them gives
 *     unspecified results (never a write outside `out`/`kv_cache`/workspace,
 *     as long as table entries for positions < seq_len are valid block ids).
 *   - Thread safety: no global mutable state besides that scratch array;
 *     concurrent calls on different streams must not share `out`, `kv_cache`
 *     slots being written, or `workspace`.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_F16 = 2 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad stride/shape,
                              scale not finite and > 0                        */
  PA_ERR_UNSUPPORTED = -2, /* block_size != 16, head_dim, dtype, head grouping */
  PA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required      */
  PA_ERR_HIP = -4,         /* a HIP launch reported an error                  */
  PA_ERR_SCRATCH = -5      /* the call needs more scratch than the library's
                              built-in array holds (no-workspace entry only)  */
} pa_status;

/* Static, NUL-terminated description of a status code. */
const char* pa_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int pa_version(void);

/*
 * pa_compute_slot_mapping -- physical slot of every query token of a step.
 *   [P4] §3.4: slot = block_table[r][pos / block_size] * block_size
 *                     + pos % block_size,
 *   with pos = num_computed_tokens[r] + i for the i-th new token of request r
 *   ([P1] §3.3.2: prefill positions start at the computed count).
 *
 *   slot_mapping        out [num_tokens] int64, varlen token order.
 *   block_table         [num_seqs, block_table_stride] int32, -1 = unused.
 *   query_start_loc     [num_seqs + 1] int32, prefix sums of per-request
 *                       query counts; precondition qsl[0] = 0,
 *                       qsl[num_seqs] = num_tokens, non-decreasing.
 *   num_computed_tokens [num_seqs] int32.
 *   A token whose table entry is -1 gets a negative slot (skipped by
 *   pa_reshape_and_cache).
 */
int pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                            int32_t block_table_stride,
                            const int32_t* query_start_loc,
                            const int32_t* num_computed_tokens, int32_t num_seqs,
                            int32_t num_tokens, int32_t block_size, void* stream);

/*
 * pa_reshape_and_cache -- scatter this step's K/V rows into their slots.
 *   [P1] §3.3.3 (write into the KV cache by slot_mapping before attention),
 *   [P4] §3.4 (reshape_and_cache_flash: key/value scattered to physical slots).
 *   For every t with s = slot_mapping[t] >= 0:
 *     kv_cache[s / 16][0][s % 16][:][:] = key[t][:][:]
 *     kv_cache[s / 16][1][s % 16][:][:] = value[t][:][:]
 *   The copy is bit-exact; nothing else in the cache changes.
 *
 *   key, value    [num_tokens, num_kv_heads, head_dim], cache dtype.
 *   kv_cache      [num_blocks, 2, block_size, num_kv_heads, head_dim].
 *   slot_mapping  [num_tokens] int64; negative = padding token, skipped.
 *   Preconditions: 0 <= slot < num_blocks * block_size or slot < 0; slots
 *   distinct within one call.  All three tensors 16-byte aligned.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* kv_cache,
                         const int64_t* slot_mapping, int32_t num_tokens,
                         int64_t num_blocks, int32_t block_size,
                         int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         void* stream);

/*
 * pa_copy_blocks -- copy whole KV-cache blocks inside the cache.
 *   [P1] §4.3.2 (copy-on-write: samples of one prompt share its blocks; a
 *   sample that is about to write into a shared block first gets a private
 *   copy of it).  For every pair p with src = block_pairs[2p] >= 0 and
 *   dst = block_pairs[2p + 1] >= 0:
 *     kv_cache[dst][0 | 1][:][:][:] = kv_cache[src][0 | 1][:][:][:]
 *   bit-exact; a pair with a negative entry is skipped; nothing else in the
 *   cache changes.
 *
 *   kv_cache     [num_blocks, 2, block_size, num_kv_heads, head_dim].
 *   block_pairs  [num_pairs, 2] int32 (src, dst), device memory.
 *   Preconditions: ids < num_blocks; destinations distinct; no destination is
 *   also a source in the same call (the copies run in parallel, in no order).
 */
int pa_copy_blocks(void* kv_cache, const int32_t* block_pairs, int32_t num_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, int32_t dtype, void* stream);

/*
 * pa_attention_workspace_size -- bytes of fp32 scratch the attention calls
 * need for their split-KV partial results (max, sum, unnormalised output per
 * query head and partition).  A function of its arguments and of the current
 * device's CU count (see pa_plan_decode_ranges); returns 0 for arguments the
 * attention calls would reject.  `num_splits` = 0 selects the
 * library's own partition count; the size covers every plan the attention
 * calls may choose for these arguments.
 */
size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens,
                                   int32_t num_q_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t max_seq_len,
                                   int32_t max_query_len, int32_t num_splits);

/*
 * pa_attention_decode -- paged attention for one new query token per request.
 *   [P1] §3.3.3 / §4.2 (paged_attention(q, kv_cache, block_tables,
 *   context_lens)), [P2] §3.3 (decode reads the cached history).
 *   For request r and query head h (kv head g = h / (num_q_heads /
 *   num_kv_heads)), with L = seq_lens[r] keys at positions 0..L-1 stored at
 *   kv_cache[block_table[r][j/16]][.][j%16][g]:
 *     out[r][h] = sum_j softmax_j(scale * <q[r][h], K_j>) * V_j.
 *   Long contexts are split over work-groups and merged exactly
 *   (partition-and-reduce); the split is balanced over the whole batch.
 *
 *   out, q        [num_seqs, num_q_heads, head_dim], cache dtype.
 *   block_table   [num_seqs, block_table_stride] int32.
 *   seq_lens      [num_seqs] int32; precondition 1 <= seq_lens[r] <=
 *                 max_seq_len (a 0 length leaves that row unwritten).
 *   max_seq_len   (host) bound used to size the split.
 *   num_q_heads   multiple of num_kv_heads, group size 1, 2, 4 or 8.
 *   workspace     >= pa_attention_workspace_size(num_seqs, num_seqs, ...,
 *                 max_seq_len, 1, num_splits) bytes, 256-byte aligned; its
 *                 contents on entry do not matter.
 *   num_splits    partitions of the batch per kv head; 0 = library choice.
 */
int pa_attention_decode(void* out, const void* q, const void* kv_cache,
                        int64_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        const int32_t* block_table, int32_t block_table_stride,
                        const int32_t* seq_lens, int32_t num_seqs,
                        int32_t max_seq_len, int32_t num_q_heads, float scale,
                        void* workspace, size_t workspace_bytes,
                        int32_t num_splits, void* stream);

/*
 * pa_attention_decode_shared_prefix -- decode for a batch whose requests all
 * start with the same physical blocks (a common prompt prefix shared through
 * prefix caching: [P4] §3.5, [P1] §4.3.1).  Same result as
 * pa_attention_decode; the prefix's keys are read once for the whole batch:
 *   - a matrix-core pass attends every request's query to the prefix keys
 *     (one virtual request whose queries are all the rows), producing a
 *     partial (max, sum, output) per row and query head;
 *   - the split decode attends each request's keys after the prefix, in the
 *     same launch as the pass (work-groups of both kinds);
 *   - a merge combines both with the online-softmax identity.
 *
 *   shared_prefix_blocks  (host) P: block_table[r][0 .. P-1] are the same
 *                         physical blocks for every r (precondition, not
 *                         checked on the device), and 16 P <= seq_lens[r]
 *                         <= max_seq_len.  P = 0, fp32, or a head shape
 *                         without a matrix-core path runs pa_attention_decode.
 *   workspace             >= pa_attention_decode_shared_prefix_workspace_size
 *                         (same arguments) bytes, 256-byte aligned.
 *   Other arguments as pa_attention_decode.
 */
size_t pa_attention_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                        int32_t num_kv_heads, int32_t head_dim,
                                                        int32_t max_seq_len,
                                                        int32_t shared_prefix_blocks,
                                                        int32_t num_splits);

int pa_attention_decode_shared_prefix(void* out, const void* q, const void* kv_cache,
                                      int64_t num_blocks, int32_t block_size,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                      const int32_t* block_table, int32_t block_table_stride,
                                      const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t max_seq_len, int32_t num_q_heads, float scale,
                                      int32_t shared_prefix_blocks, void* workspace,
                                      size_t workspace_bytes, int32_t num_splits, void* stream);

/*
 * pa_cache_and_attend_decode_shared_prefix -- the decode step of a batch
 * sharing prefix blocks in one attention launch (plus the merge): each
 * request's new token gets its slot ([P4] §3.4), its K/V row is stored into
 * the cache and the attention reads it from key / value, as in
 * pa_cache_and_attend_decode; the prefix is attended once, as in
 * pa_attention_decode_shared_prefix.  Results are those of
 *     pa_compute_slot_mapping -> pa_reshape_and_cache ->
 *     pa_attention_decode_shared_prefix
 * with the same arguments (out, cache and slots bit for bit).
 *
 *   key, value, slot_mapping  as pa_cache_and_attend_decode.
 *   Preconditions, besides those of pa_attention_decode_shared_prefix:
 *   16 P < seq_lens[r] for every request (its new token, at position
 *   seq_lens[r] - 1, lies past the prefix: shared blocks are never written,
 *   [P4] §3.5), and the conditions of pa_cache_and_attend_decode.
 *   P = 0, fp32, or a head shape without a matrix-core path runs
 *   pa_cache_and_attend_decode.
 */
int pa_cache_and_attend_decode_shared_prefix(
    void* out, const void* q, const void* key, const void* value, void* kv_cache,
    int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
    int32_t dtype, const int32_t* block_table, int32_t block_table_stride,
    const int32_t* seq_lens, int64_t* slot_mapping, int32_t num_seqs, int32_t max_seq_len,
    int32_t num_q_heads, float scale, int32_t shared_prefix_blocks, void* workspace,
    size_t workspace_bytes, int32_t num_splits, void* stream);

/*
 * pa_attention_mixed -- attention for a chunked-prefill mixed batch.
 *   [P4] §4.2 (prefill chunks and decodes packed in one 1-D varlen batch;
 *   each sequence handled by its own bounds; a chunk attends its cached
 *   history plus the earlier tokens of the chunk), [P2] §3.4 step 3
 *   (each sequence attends only to its own tokens).
 *   Token i of request r is row t = query_start_loc[r] + i at absolute
 *   position pos = num_computed_tokens[r] + i; it attends keys 0..pos:
 *     out[t][h] = sum_{j<=pos} softmax_j(scale * <q[t][h], K_j>) * V_j.
 *   Requests with one query take the decode path; longer ones the MFMA
 *   tile path with a causal mask.  When the batch has a chunk and at least
 *   one other request, the tiles and the decode ranges are work-groups of
 *   one launch (one tile wave and one decode wave per SIMD), so the
 *   compute-bound and the bandwidth-bound halves overlap; the decode merge
 *   follows (pa_attention_mixed_planned can keep them apart).  An fp32 cache
 *   has no matrix-core tiles: its chunks
 *   are attended in fp32 on the vector ALU (16-token tiles), in a launch
 *   before the decode rows.
 *
 *   out, q              [num_tokens, num_q_heads, head_dim], cache dtype.
 *   seq_lens            [num_seqs]: keys of the request's last query,
 *                       = num_computed_tokens[r] + q_len[r].
 *   query_start_loc     [num_seqs + 1]: qsl[0] = 0, qsl[num_seqs] =
 *                       num_tokens; q_len = 0 requests produce no rows.
 *   num_computed_tokens [num_seqs].
 *   max_query_len, max_seq_len (host) bounds.
 *   workspace           >= pa_attention_workspace_size(num_seqs, num_tokens,
 *                       ..., max_seq_len, max_query_len, num_splits) bytes.
 *   The new tokens' K/V must already be in the cache (pa_reshape_and_cache
 *   on the same stream first, as in [P1] §3.3.3), or use
 *   pa_cache_and_attend_mixed, which stores them in the same launch.
 */
int pa_attention_mixed(void* out, const void* q, const void* kv_cache,
                       int64_t num_blocks, int32_t block_size,
                       int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                       const int32_t* block_table, int32_t block_table_stride,
                       const int32_t* seq_lens, const int32_t* query_start_loc,
                       const int32_t* num_computed_tokens, int32_t num_seqs,
                       int32_t num_tokens, int32_t max_query_len,
                       int32_t max_seq_len, int32_t num_q_heads, float scale,
                       void* workspace, size_t workspace_bytes,
                       int32_t num_splits, void* stream);

/*
 * pa_cache_and_attend_decode / pa_cache_and_attend_mixed -- one layer's
 * step in one attention launch: the slot of every new token ([P4] §3.4), the
 * store of its K/V into the cache by that slot, and the attention that reads
 * it ([P1] §3.3.3: the new keys/values are written before attention uses
 * them).  Results are those of the three calls on one stream
 *     pa_compute_slot_mapping -> pa_reshape_and_cache -> pa_attention_decode
 *                                                        (or _mixed)
 * with the same arguments: `out` as the attention call, kv_cache holding
 * key[t] / value[t] at token t's position (bit-exact), and slot_mapping[t]
 * (when not NULL) the slot written.  Inside the launch the new rows are read
 * from key / value directly and each is stored into the cache once, so the
 * stores and the reads do not depend on each other.
 *
 *   key, value     [rows, num_kv_heads, head_dim], cache dtype, 16-byte
 *                  aligned; rows = num_seqs (decode) or num_tokens (mixed).
 *   slot_mapping   out [rows] int64, or NULL.
 *   Decode: request r's new token is row r at position seq_lens[r] - 1
 *   (num_computed = seq_lens - 1); a row with seq_lens[r] = 0 has none.
 *   Mixed: token t = query_start_loc[r] + i sits at num_computed_tokens[r] + i.
 *   Preconditions, besides the attention call's: table entries for every new
 *   position are valid block ids; the new tokens' slots are distinct and none
 *   is a key that another request reads in the same call (a request writes
 *   only into blocks it does not share, as copy-on-write guarantees).
 *   Workspace and other arguments as the attention calls.
 */
int pa_cache_and_attend_decode(void* out, const void* q, const void* key, const void* value,
                               void* kv_cache, int64_t num_blocks, int32_t block_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                               const int32_t* block_table, int32_t block_table_stride,
                               const int32_t* seq_lens, int64_t* slot_mapping,
                               int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                               float scale, void* workspace, size_t workspace_bytes,
                               int32_t num_splits, void* stream);

int pa_cache_and_attend_mixed(void* out, const void* q, const void* key, const void* value,
                              void* kv_cache, int64_t num_blocks, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                              const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, const int32_t* query_start_loc,
                              const int32_t* num_computed_tokens, int64_t* slot_mapping,
                              int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                              int32_t max_seq_len, int32_t num_q_heads, float scale,
                              void* workspace, size_t workspace_bytes, int32_t num_splits,
                              void* stream);

/*
 * pa_cache_and_attend_mixed_no_workspace -- for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): pa_cache_and_attend_mixed without the workspace
 * arguments.  Same kernels, same plan, same results bit for bit; the split-KV
 * partials go to a scratch array of PA_NO_WORKSPACE_MAX_BYTES that the
 * library holds in device memory (one per GPU it runs on, kept until the
 * process ends).
 *   - The call allocates nothing: no hipMalloc, no hipFree.  Its first call
 *     on a device looks up that device's copy of the array (the current HIP
 *     device must be the one `stream` belongs to).
 *   - Sizes: a call whose pa_attention_workspace_size(num_seqs, num_tokens,
 *     ..., max_seq_len, max_query_len, num_splits) exceeds
 *     PA_NO_WORKSPACE_MAX_BYTES returns PA_ERR_SCRATCH and launches nothing
 *     (e.g. 32 query heads of 128 dims: about 1,900 requests).
 *   - Every call on a GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (different streams, or different threads without an
 *     ordering between their streams) race and give unspecified results.
 *     Calls on one stream are ordered and safe.  Nothing in the array needs
 *     to be cleared between calls.
 *   Other arguments, preconditions and errors as pa_cache_and_attend_mixed.
 */
#define PA_NO_WORKSPACE_MAX_BYTES ((size_t)32 << 20)

int pa_cache_and_attend_mixed_no_workspace(
    void* out, const void* q, const void* key, const void* value, void* kv_cache,
    int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
    int32_t dtype, const int32_t* block_table, int32_t block_table_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    const int32_t* num_computed_tokens, int64_t* slot_mapping, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
    float scale, int32_t num_splits, void* stream);

/*
 * pa_attention_mixed_planned / pa_cache_and_attend_mixed_planned -- the
 * mixed-batch calls with the work plan spelled out instead of chosen by the
 * library (plan = NULL: the library's choice, as the plain calls).  Results
 * are the same whatever the plan (to the tolerance of the attention; the
 * cache and slots bit for bit); it changes only how the work is cut:
 *   num_splits           as the plain calls' argument.
 *   tile_shape           -1: library choice; 0: 16 query tokens per wave and
 *                        two key parts per tile (short chunks); 1: 32 tokens
 *                        per wave (long chunks).  Used when the tiles run in a
 *                        launch of their own.
 *   tiles_beside_decode  -1: library choice (one launch of tiles and decode
 *                        ranges when the batch has both); 0: the tiles, then
 *                        the decode rows, in launches of their own.
 * Other fields out of range return PA_ERR_INVALID_ARG.  Other arguments as
 * pa_attention_mixed / pa_cache_and_attend_mixed (whose num_splits the plan
 * carries).
 */
typedef struct {
  int32_t num_splits;
  int32_t tile_shape;
  int32_t tiles_beside_decode;
} pa_mixed_plan;

int pa_attention_mixed_planned(void* out, const void* q, const void* kv_cache,
                               int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype, const int32_t* block_table,
                               int32_t block_table_stride, const int32_t* seq_lens,
                               const int32_t* query_start_loc,
                               const int32_t* num_computed_tokens, int32_t num_seqs,
                               int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                               int32_t num_q_heads, float scale, void* workspace,
                               size_t workspace_bytes, const pa_mixed_plan* plan, void* stream);

int pa_cache_and_attend_mixed_planned(
    void* out, const void* q, const void* key, const void* value, void* kv_cache,
    int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
    int32_t dtype, const int32_t* block_table, int32_t block_table_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    const int32_t* num_computed_tokens, int64_t* slot_mapping, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
    float scale, void* workspace, size_t workspace_bytes, const pa_mixed_plan* plan,
    void* stream);

/*
 * pa_plan_decode_ranges -- the split the attention calls would plan on a
 * device with `num_cus` compute units: key ranges per KV head for the decode
 * rows (3 wavefronts per CU, i.e. one 4-wave work-group on three CUs in
 * four; beside concurrent prefill tiles, the wave slots those leave, 4-6 per
 * CU; no range shorter than 4 blocks).  The
 * calls themselves read the current device's CU and XCD counts (hipGetDevice,
 * hipDeviceGetAttribute; 256 and 8 when no device answers), and so does
 * pa_attention_workspace_size: compute a workspace size with the device
 * current that the calls will run on.  Pure function; returns the range
 * count, or a negative pa_status for arguments the calls would reject.
 */
int pa_plan_decode_ranges(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t dtype, int32_t max_seq_len,
                          int32_t max_query_len, int32_t num_splits, int32_t num_cus);

/*
 * pa_check_metadata -- check, on the device, the step metadata the calls
 * above trust (the pages' model runner takes it from its scheduler
 * unchecked: [P4] §3.4 block tables and slots, §4.2 packed query offsets and
 * computed counts, §3.5 shared prefix blocks).  For a caller debugging its
 * own scheduler: run it on the same stream before the attention call, then
 * read *flags whenever convenient (it is not synchronised here).
 *
 *   flags                 [1] uint32, caller-zeroed; each violated condition
 *                         ORs its pa_meta_flag bit (device atomics).
 *   block_table, block_table_stride, seq_lens, num_seqs, max_seq_len,
 *   num_blocks            as the attention calls.
 *   query_start_loc, num_computed_tokens
 *                         [num_seqs + 1], [num_seqs] for a mixed batch, or
 *                         both null for a decode batch (one query per
 *                         request, seq_lens >= 1).
 *   slot_mapping          [num_tokens] int64 or null: checked inside the pool
 *                         and distinct (negative = skipped token); the
 *                         distinctness test compares all pairs, O(T^2).
 *   num_tokens, max_query_len
 *                         (host) as pa_attention_mixed (decode: num_seqs, 1).
 *   shared_prefix_blocks  (host) P >= 0: also check that every row's first P
 *                         entries equal row 0's and 16 P <= seq_lens[r];
 *                         P <= block_table_stride.
 *   Only the metadata is read, each array within its given extent whatever
 *   its contents.  Host argument errors return PA_ERR_INVALID_ARG.
 */
typedef enum {
  PA_META_SEQ_LEN = 1u << 0,       /* seq_len < 0 or > max_seq_len (decode: < 1) */
  PA_META_TABLE_WIDTH = 1u << 1,   /* ceil(seq_len / 16) > block_table_stride */
  PA_META_BLOCK_ID = 1u << 2,      /* a table entry read by attention not in [0, num_blocks) */
  PA_META_QUERY_START = 1u << 3,   /* qsl[0] != 0, qsl decreasing, or qsl[R] != num_tokens */
  PA_META_COMPUTED = 1u << 4,      /* num_computed < 0 or != seq_len - q_len */
  PA_META_QUERY_LEN = 1u << 5,     /* q_len > max_query_len */
  PA_META_SLOT_RANGE = 1u << 6,    /* slot >= num_blocks * 16 */
  PA_META_SLOT_DUP = 1u << 7,      /* two tokens of the call share a slot */
  PA_META_SHARED_PREFIX = 1u << 8  /* rows differ in the prefix blocks, or too short */
} pa_meta_flag;

int pa_check_metadata(uint32_t* flags, const int32_t* block_table, int32_t block_table_stride,
                      const int32_t* seq_lens, const int32_t* query_start_loc,
                      const int32_t* num_computed_tokens, const int64_t* slot_mapping,
                      int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                      int32_t max_seq_len, int64_t num_blocks, int32_t block_size,
                      int32_t shared_prefix_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
