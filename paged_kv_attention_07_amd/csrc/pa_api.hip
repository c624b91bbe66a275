// C-ABI front end of libpa.so: argument checks, work planning and dispatch.
// The public contract of every function is documented in include/pa.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "pa.h"
#include "pa_kernels.h"

namespace {

constexpr int kVersion = 100;  // 0.1.0

// Geometry of the device a call runs on: compute units and XCDs (dies, each
// with its own L2).  The kernels hold 4 waves per work-group and at most two
// waves per SIMD (their register budget), so a CU has 4 SIMDs x 2 = 8 wave
// slots.
struct Geometry {
  int cus, xcds;
};
constexpr Geometry kDefaultGeometry = {256, 8};  // MI355X, used when no device answers

std::mutex g_geo_mu;
Geometry g_geo[64];
bool g_geo_known[64];

// The current device's geometry, read once per device.
Geometry device_geometry() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kDefaultGeometry;
  std::lock_guard<std::mutex> lock(g_geo_mu);
  if (!g_geo_known[dev]) {
    Geometry g = kDefaultGeometry;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        v > 0)
      g.cus = v;
    v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess && v > 0)
      g.xcds = v;
    g_geo[dev] = g;
    g_geo_known[dev] = true;
  }
  return g_geo[dev];
}

// A caller's plan for a mixed batch (pa_mixed_plan); -1 fields are the
// library's choice.
struct Plan {
  int num_splits = 0;
  int tile_shape = -1;
  int tiles_beside_decode = -1;
};

Plan splits_plan(int num_splits) {
  Plan p;
  p.num_splits = num_splits;
  return p;
}

// Partition plan for the balanced split: three wavefronts per CU (one
// work-group of 4 waves on three CUs in four), but no range shorter than a
// few blocks.  With each wave keeping its next block in flight this reads
// HBM faster than one wave per SIMD (~2%), which beat two per SIMD on every
// batch of private sequences measured (16-512 requests, 256-8192 keys:
// 2-4%); more waves paid only on a batch whose blocks are mostly shared,
// i.e. read from cache, which the shared-prefix entry plans for itself.
// Beside concurrent prefill tiles the decode rows
// take the slots the tiles leave: the chip's wave slots (8 per CU) minus the
// tiles of the longest chunk (a lower bound on the tile count), between one
// and one and a half waves per SIMD.
constexpr int kMinBlocksPerRange = 4;

// query heads per wave of the matrix-core prefill tiles
int heads_per_wave(int group) { return group < 4 ? group : 4; }

bool group_ok(int group) { return group == 1 || group == 2 || group == 4 || group == 8; }

bool dtype_ok(int dtype) { return dtype == PA_F32 || dtype == PA_BF16 || dtype == PA_F16; }

int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Matrix-core prefill tiles run beside the decode rows when the batch can
// hold both (a chunk, max_query_len > 1, and at least one other request) and
// the plan does not keep them apart.  fp32 tiles (vector ALU) run before the
// decode rows instead.
bool tiles_beside_decode(int num_seqs, int max_query_len, int dtype, const Plan& plan) {
  return max_query_len > 1 && num_seqs >= 2 && dtype != PA_F32 && plan.tiles_beside_decode != 0;
}

// Decode waves beside the tiles of a chunk of up to max_query_len tokens
// (tile shape of the fused launch: 4 waves per tile, 32 * 4 / group-per-wave
// tokens per tile).  With exact_tiles (the shared-prefix pass: one virtual
// request of exactly max_query_len rows) the tiles and the decode waves fill
// the chip's wave slots exactly, so every CU holds the same number of
// work-groups (slots - tile waves, at least 4 per CU); otherwise the tile
// count is only a lower bound and the decode waves stay within 4-6 per CU.
int64_t waves_beside_prefill(int num_kv_heads, int group, int max_query_len, bool exact_tiles,
                             int cus) {
  const int wpw = heads_per_wave(group);
  const int64_t qt = 32 * (4 / wpw);
  const int64_t tile_waves = 4 * ceil_div(max_query_len, qt) * num_kv_heads * (group / wpw);
  int64_t w = (int64_t)cus * 8 - tile_waves;
  if (w < (int64_t)cus * 4) w = (int64_t)cus * 4;
  if (!exact_tiles && w > (int64_t)cus * 6) w = (int64_t)cus * 6;
  return w;
}

// Ranges per KV head on a device of `cus` compute units.  dtype and head_dim
// set the waves per GQA group; the workspace-size queries, which have no
// dtype, plan with PA_BF16: its waves serve the most heads each, so its plan
// has the most ranges and bounds the others.
int plan_chunks(int num_seqs, int num_kv_heads, int group, int max_seq_len, int num_splits,
                bool beside_prefill, int max_query_len, int dtype, int head_dim, int cus,
                bool exact_tiles = false) {
  if (num_splits > 0) return num_splits;
  const int hg = group / pa::decode_heads_per_wave(dtype, head_dim, group);
  const int64_t blocks_upper = (int64_t)num_seqs * ceil_div(max_seq_len, pa::kBlockSize);
  // decode rows alone: 3 waves per CU (one 4-wave work-group on each of
  // three CUs in four); measured faster than one wave per SIMD on the bf16
  // decode batches tried (64 requests: 116.2 -> 114.1 us; 16 x 32K: 359 ->
  // 352 us), and both beat two per SIMD
  const int64_t waves = beside_prefill
                            ? waves_beside_prefill(num_kv_heads, group, max_query_len,
                                                   exact_tiles, cus)
                            : (int64_t)cus * 3;
  int64_t n = ceil_div(waves, (int64_t)num_kv_heads * hg);
  const int64_t cap = ceil_div(blocks_upper, kMinBlocksPerRange);
  if (n > cap) n = cap;
  if (n < 1) n = 1;
  return (int)n;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// workspace: [R] x int4 request metadata, then [(R + N) * Hq * 2] floats of
// (max, sum), then [(R + N) * Hq * D] floats of partial outputs
struct WsLayout {
  size_t meta, ml, o, total;
};

WsLayout workspace_layout(int num_seqs, int num_q_heads, int head_dim, int chunks) {
  const size_t slots = (size_t)num_seqs + (size_t)chunks;
  WsLayout w;
  w.meta = 0;
  w.ml = align256((size_t)num_seqs * 4 * sizeof(int32_t));
  w.o = w.ml + align256(slots * num_q_heads * 2 * sizeof(float));
  w.total = w.o + align256(slots * num_q_heads * (size_t)head_dim * sizeof(float));
  return w;
}

int check_cache(const void* kv_cache, int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                int32_t head_dim, int32_t dtype) {
  if (!kv_cache || num_blocks <= 0 || num_kv_heads <= 0) return PA_ERR_INVALID_ARG;
  if (block_size != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (!aligned16(kv_cache)) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (!group_ok(num_q_heads / num_kv_heads)) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }


}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch error";
    case PA_ERR_SCRATCH: return "call needs more than the built-in scratch array";
    default: return "unknown status";
  }
}

int pa_version(void) { return kVersion; }

int pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                            int32_t block_table_stride, const int32_t* query_start_loc,
                            const int32_t* num_computed_tokens, int32_t num_seqs,
                            int32_t num_tokens, int32_t block_size, void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || block_table_stride < 0) return PA_ERR_INVALID_ARG;
  if (block_size != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (num_seqs == 0) return PA_ERR_INVALID_ARG;
  if (!slot_mapping || !block_table || !query_start_loc || !num_computed_tokens)
    return PA_ERR_INVALID_ARG;
  return hip_status(pa::launch_slot_mapping(slot_mapping, block_table, block_table_stride,
                                            query_start_loc, num_computed_tokens, num_seqs,
                                            num_tokens, static_cast<hipStream_t>(stream)));
}

int pa_reshape_and_cache(const void* key, const void* value, void* kv_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int64_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                         int32_t dtype, void* stream) {
  int st = check_cache(kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return PA_ERR_INVALID_ARG;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_INVALID_ARG;
  const int row_bytes = num_kv_heads * head_dim * elem_bytes(dtype);
  return hip_status(pa::launch_reshape_and_cache(key, value, kv_cache, slot_mapping, num_tokens,
                                                 row_bytes, static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* kv_cache, const int32_t* block_pairs, int32_t num_pairs,
                   int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, int32_t dtype, void* stream) {
  int st = check_cache(kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return PA_ERR_INVALID_ARG;
  if (num_pairs == 0) return PA_OK;
  if (!block_pairs) return PA_ERR_INVALID_ARG;
  const int64_t block_bytes =
      (int64_t)2 * block_size * num_kv_heads * head_dim * elem_bytes(dtype);
  return hip_status(pa::launch_copy_blocks(kv_cache, block_pairs, num_pairs, block_bytes,
                                           static_cast<hipStream_t>(stream)));
}

size_t pa_attention_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t max_seq_len,
                                   int32_t max_query_len, int32_t num_splits) {
  (void)num_tokens;
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_seq_len <= 0 || num_splits < 0) return 0;
  if (head_dim != 64 && head_dim != 128) return 0;
  if (check_heads(num_q_heads, num_kv_heads) != PA_OK) return 0;
  const int group = num_q_heads / num_kv_heads;
  // size for the larger of the plans with and without concurrent tiles, so
  // the buffer serves either call; beside tiles, for the shortest chunk (2
  // tokens), which leaves the decode rows the most waves: a call may pass any
  // max_query_len up to the one given here
  const int cus = device_geometry().cus;
  const int alone = plan_chunks(num_seqs, num_kv_heads, group, max_seq_len, num_splits, false,
                                0, PA_BF16, head_dim, cus);
  const int beside =
      max_query_len > 1 ? plan_chunks(num_seqs, num_kv_heads, group, max_seq_len, num_splits,
                                      true, 2, PA_BF16, head_dim, cus)
                        : 0;
  const int chunks = alone > beside ? alone : beside;
  return workspace_layout(num_seqs, num_q_heads, head_dim, chunks).total;
}

static int attention_common(void* out, const void* q, const void* kv_cache, int64_t num_blocks,
                            int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                            int32_t dtype, const int32_t* block_table, int32_t bt_stride,
                            const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                            int32_t num_q_heads, float scale, void* workspace,
                            size_t workspace_bytes, const Plan& plan, int32_t max_query_len,
                            int32_t shared_prefix_blocks, pa::DecodeArgs* a,
                            int (*scratch)(void**, size_t*) = nullptr,
                            bool launches = true) {
  int st = check_cache(kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype);
  if (st != PA_OK) return st;
  st = check_heads(num_q_heads, num_kv_heads);
  if (st != PA_OK) return st;
  const int num_splits = plan.num_splits;
  if (num_seqs < 0 || max_seq_len < 0 || bt_stride < 0 || num_splits < 0) return PA_ERR_INVALID_ARG;
  if (!isfinite(scale) || !(scale > 0.f)) return PA_ERR_INVALID_ARG;  // a softmax temperature
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !block_table || !seq_lens) return PA_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q)) return PA_ERR_INVALID_ARG;
  if (max_seq_len == 0) return PA_OK;
  if (bt_stride < ceil_div(max_seq_len, pa::kBlockSize)) return PA_ERR_INVALID_ARG;
  const int group = num_q_heads / num_kv_heads;
  // with a shared prefix the split covers the keys after it, beside the
  // prefix pass, and R more slots hold the prefix partials
  const int P = shared_prefix_blocks;
  const int chunks =
      plan_chunks(num_seqs, num_kv_heads, group,
                  P > 0 ? max(max_seq_len - P * pa::kBlockSize, 1) : max_seq_len, num_splits,
                  P > 0 || tiles_beside_decode(num_seqs, max_query_len, dtype, plan),
                  P > 0 ? num_seqs : max_query_len, dtype, head_dim, device_geometry().cus,
                  P > 0);
  const WsLayout lay = workspace_layout(num_seqs, num_q_heads, head_dim,
                                        chunks + (P > 0 ? num_seqs : 0));
  if (launches) {
    // no workspace given: the library's own scratch array, looked up only
    // now that every host check has passed
    if (!workspace && scratch) {
      const int sst = scratch(&workspace, &workspace_bytes);
      if (sst != PA_OK) return sst;
    }
    if (!workspace || workspace_bytes < lay.total) return PA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PA_ERR_WORKSPACE;
  }

  a->out = out;
  a->q = q;
  a->kv = kv_cache;
  a->block_table = block_table;
  a->bt_stride = bt_stride;
  a->seq_lens = seq_lens;
  a->qsl = nullptr;
  a->num_seqs = num_seqs;
  a->num_kv_heads = num_kv_heads;
  a->num_q_heads = num_q_heads;
  a->num_chunks = chunks;
  a->head_groups = group / pa::decode_heads_per_wave(dtype, head_dim, group);
  a->scale_log2 = scale * 1.4426950408889634f;
  char* ws = static_cast<char*>(workspace);
  a->ws_meta = reinterpret_cast<int32_t*>(ws + lay.meta);
  a->ws_ml = reinterpret_cast<float*>(ws + lay.ml);
  a->ws_o = reinterpret_cast<float*>(ws + lay.o);
  a->skip_blocks = P;
  a->prefix_slot0 = P > 0 ? num_seqs + chunks : -1;
  return 1;  // proceed
}

}  // extern "C"

namespace {

// New-token rows handed to an attention launch that also stores them; null
// pointers when the caller scattered them beforehand.
int fresh_tokens(const void* key, const void* value, void* kv_cache, int64_t* slot_mapping,
                 pa::NewTokens* f) {
  if (!key || !value) return PA_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value)) return PA_ERR_INVALID_ARG;
  f->k = key;
  f->v = value;
  f->kv = kv_cache;
  f->slot_out = slot_mapping;
  return PA_OK;
}

int decode_impl(void* out, const void* q, const void* kv_cache, int64_t num_blocks,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
                int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads, float scale,
                void* workspace, size_t workspace_bytes, int32_t num_splits,
                const pa::NewTokens& fresh, void* stream) {
  Plan plan;
  plan.num_splits = num_splits;
  pa::DecodeArgs a{};
  const int st = attention_common(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim,
                                  dtype, block_table, block_table_stride, seq_lens, num_seqs,
                                  max_seq_len, num_q_heads, scale, workspace, workspace_bytes,
                                  plan, 1, 0, &a);
  if (st <= 0) return st;
  a.fresh = fresh;
  return hip_status(pa::launch_decode(a, dtype, head_dim, num_q_heads / num_kv_heads,
                                      static_cast<hipStream_t>(stream)));
}

int mixed_impl(void* out, const void* q, const void* kv_cache, int64_t num_blocks,
               int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
               const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
               const int32_t* query_start_loc, const int32_t* num_computed_tokens,
               int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
               int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
               const Plan& plan, const pa::NewTokens& fresh, void* stream,
               int (*scratch)(void**, size_t*) = nullptr) {
  if (plan.tile_shape < -1 || plan.tile_shape > 1 || plan.tiles_beside_decode < -1 ||
      plan.tiles_beside_decode > 1)
    return PA_ERR_INVALID_ARG;
  if (num_tokens < 0 || max_query_len < 0) return PA_ERR_INVALID_ARG;
  // metadata pointers are checked before the workspace, whichever supplies it
  if (num_seqs > 0 && num_tokens > 0 && (!query_start_loc || !num_computed_tokens))
    return PA_ERR_INVALID_ARG;
  pa::DecodeArgs a{};
  const int st = attention_common(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim,
                                  dtype, block_table, block_table_stride, seq_lens, num_seqs,
                                  max_seq_len, num_q_heads, scale, workspace, workspace_bytes,
                                  plan, max_query_len, 0, &a, scratch, num_tokens > 0);
  if (st <= 0) return st;
  if (num_tokens == 0) return PA_OK;
  if (!query_start_loc || !num_computed_tokens) return PA_ERR_INVALID_ARG;
  a.fresh = fresh;
  const int group = num_q_heads / num_kv_heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  a.qsl = query_start_loc;
  if (max_query_len > 1) {
    pa::PrefillArgs p{};
    p.out = out;
    p.q = q;
    p.kv = kv_cache;
    p.block_table = block_table;
    p.bt_stride = block_table_stride;
    p.seq_lens = seq_lens;
    p.qsl = query_start_loc;
    p.num_computed = num_computed_tokens;
    p.num_seqs = num_seqs;
    p.num_kv_heads = num_kv_heads;
    p.num_q_heads = num_q_heads;
    p.max_tiles = (int)(ceil_div(num_tokens, pa::kQueriesPerTile) + num_seqs);
    p.max_query_len = max_query_len;
    p.tile_shape = plan.tile_shape;
    p.num_xcds = device_geometry().xcds;
    p.cus_per_xcd = std::max(1, device_geometry().cus / p.num_xcds);
    p.scale_log2 = a.scale_log2;
    p.fresh = fresh;
    if (tiles_beside_decode(num_seqs, max_query_len, dtype, plan)) {
      // tiles and decode ranges in one launch, then the merge
      p.beside_decode = 1;
      const hipError_t e = pa::launch_fused(a, p, dtype, head_dim, group, s);
      if (e != hipSuccess) return PA_ERR_HIP;
      return hip_status(pa::launch_decode_merge(a, dtype, head_dim, group, s));
    }
    const hipError_t e = dtype == PA_F32 ? pa::launch_prefill_f32(p, head_dim, group, s)
                                         : pa::launch_prefill(p, dtype, head_dim, group, s);
    if (e != hipSuccess) return PA_ERR_HIP;
    if (num_seqs == 1) return PA_OK;  // the one request is the chunk: no decode rows
  }
  return hip_status(pa::launch_decode(a, dtype, head_dim, group, s));
}

}  // namespace

extern "C" {

int pa_attention_decode(void* out, const void* q, const void* kv_cache, int64_t num_blocks,
                        int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        const int32_t* block_table, int32_t block_table_stride,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                        int32_t num_q_heads, float scale, void* workspace, size_t workspace_bytes,
                        int32_t num_splits, void* stream) {
  return decode_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                     block_table, block_table_stride, seq_lens, num_seqs, max_seq_len,
                     num_q_heads, scale, workspace, workspace_bytes, num_splits, pa::NewTokens{},
                     stream);
}

int pa_attention_mixed(void* out, const void* q, const void* kv_cache, int64_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                       const int32_t* block_table, int32_t block_table_stride,
                       const int32_t* seq_lens, const int32_t* query_start_loc,
                       const int32_t* num_computed_tokens, int32_t num_seqs, int32_t num_tokens,
                       int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                       float scale, void* workspace, size_t workspace_bytes, int32_t num_splits,
                       void* stream) {
  return mixed_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                    block_table, block_table_stride, seq_lens, query_start_loc,
                    num_computed_tokens, num_seqs, num_tokens, max_query_len, max_seq_len,
                    num_q_heads, scale, workspace, workspace_bytes, splits_plan(num_splits),
                    pa::NewTokens{}, stream);
}

int pa_cache_and_attend_decode(void* out, const void* q, const void* key, const void* value,
                               void* kv_cache, int64_t num_blocks, int32_t block_size,
                               int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                               const int32_t* block_table, int32_t block_table_stride,
                               const int32_t* seq_lens, int64_t* slot_mapping,
                               int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                               float scale, void* workspace, size_t workspace_bytes,
                               int32_t num_splits, void* stream) {
  if (num_seqs > 0 && max_seq_len > 0 && !(key && value)) return PA_ERR_INVALID_ARG;
  pa::NewTokens f{};
  if (key || value) {
    const int st = fresh_tokens(key, value, kv_cache, slot_mapping, &f);
    if (st != PA_OK) return st;
  }
  return decode_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                     block_table, block_table_stride, seq_lens, num_seqs, max_seq_len,
                     num_q_heads, scale, workspace, workspace_bytes, num_splits, f, stream);
}

int pa_cache_and_attend_mixed(void* out, const void* q, const void* key, const void* value,
                              void* kv_cache, int64_t num_blocks, int32_t block_size,
                              int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                              const int32_t* block_table, int32_t block_table_stride,
                              const int32_t* seq_lens, const int32_t* query_start_loc,
                              const int32_t* num_computed_tokens, int64_t* slot_mapping,
                              int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                              int32_t max_seq_len, int32_t num_q_heads, float scale,
                              void* workspace, size_t workspace_bytes, int32_t num_splits,
                              void* stream) {
  if (num_tokens > 0 && !(key && value)) return PA_ERR_INVALID_ARG;
  pa::NewTokens f{};
  if (key || value) {
    const int st = fresh_tokens(key, value, kv_cache, slot_mapping, &f);
    if (st != PA_OK) return st;
  }
  return mixed_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                    block_table, block_table_stride, seq_lens, query_start_loc,
                    num_computed_tokens, num_seqs, num_tokens, max_query_len, max_seq_len,
                    num_q_heads, scale, workspace, workspace_bytes, splits_plan(num_splits), f,
                    stream);
}

static int plan_from(const pa_mixed_plan* plan, Plan* out) {
  if (plan) {
    out->num_splits = plan->num_splits;
    out->tile_shape = plan->tile_shape;
    out->tiles_beside_decode = plan->tiles_beside_decode;
  }
  return PA_OK;
}

int pa_attention_mixed_planned(void* out, const void* q, const void* kv_cache,
                               int64_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype, const int32_t* block_table,
                               int32_t block_table_stride, const int32_t* seq_lens,
                               const int32_t* query_start_loc,
                               const int32_t* num_computed_tokens, int32_t num_seqs,
                               int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                               int32_t num_q_heads, float scale, void* workspace,
                               size_t workspace_bytes, const pa_mixed_plan* plan,
                               void* stream) {
  Plan p;
  plan_from(plan, &p);
  return mixed_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                    block_table, block_table_stride, seq_lens, query_start_loc,
                    num_computed_tokens, num_seqs, num_tokens, max_query_len, max_seq_len,
                    num_q_heads, scale, workspace, workspace_bytes, p, pa::NewTokens{}, stream);
}

int pa_cache_and_attend_mixed_planned(
    void* out, const void* q, const void* key, const void* value, void* kv_cache,
    int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
    int32_t dtype, const int32_t* block_table, int32_t block_table_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    const int32_t* num_computed_tokens, int64_t* slot_mapping, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
    float scale, void* workspace, size_t workspace_bytes, const pa_mixed_plan* plan,
    void* stream) {
  if (num_tokens > 0 && !(key && value)) return PA_ERR_INVALID_ARG;
  pa::NewTokens f{};
  if (key || value) {
    const int st = fresh_tokens(key, value, kv_cache, slot_mapping, &f);
    if (st != PA_OK) return st;
  }
  Plan p;
  plan_from(plan, &p);
  return mixed_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                    block_table, block_table_stride, seq_lens, query_start_loc,
                    num_computed_tokens, num_seqs, num_tokens, max_query_len, max_seq_len,
                    num_q_heads, scale, workspace, workspace_bytes, p, f, stream);
}

int pa_plan_decode_ranges(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t dtype, int32_t max_seq_len,
                          int32_t max_query_len, int32_t num_splits, int32_t num_cus) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_seq_len <= 0 || max_query_len < 0 ||
      num_splits < 0 || num_cus <= 0)
    return PA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  const int st = check_heads(num_q_heads, num_kv_heads);
  if (st != PA_OK) return st;
  const int group = num_q_heads / num_kv_heads;
  return plan_chunks(num_seqs, num_kv_heads, group, max_seq_len, num_splits,
                     tiles_beside_decode(num_seqs, max_query_len, dtype, Plan{}), max_query_len,
                     dtype, head_dim, num_cus);
}

int pa_check_metadata(uint32_t* flags, const int32_t* block_table, int32_t block_table_stride,
                      const int32_t* seq_lens, const int32_t* query_start_loc,
                      const int32_t* num_computed_tokens, const int64_t* slot_mapping,
                      int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                      int32_t max_seq_len, int64_t num_blocks, int32_t block_size,
                      int32_t shared_prefix_blocks, void* stream) {
  if (block_size != pa::kBlockSize) return PA_ERR_UNSUPPORTED;
  if (!flags || num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || max_seq_len < 0 ||
      block_table_stride < 0 || num_blocks < 0 || shared_prefix_blocks < 0 ||
      shared_prefix_blocks > block_table_stride)
    return PA_ERR_INVALID_ARG;
  if ((query_start_loc == nullptr) != (num_computed_tokens == nullptr)) return PA_ERR_INVALID_ARG;
  if (!query_start_loc && num_tokens != num_seqs) return PA_ERR_INVALID_ARG;  // decode: T = R
  if (num_seqs > 0 && (!block_table || !seq_lens)) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0 && num_tokens == 0) return PA_OK;
  if (num_seqs == 0 && query_start_loc) return PA_ERR_INVALID_ARG;  // tokens without requests
  pa::MetaCheckArgs a{};
  a.flags = flags;
  a.block_table = block_table;
  a.bt_stride = block_table_stride;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.num_computed = num_computed_tokens;
  a.slots = slot_mapping;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.max_seq_len = max_seq_len;
  a.num_blocks = num_blocks;
  a.shared_prefix_blocks = num_seqs > 0 ? shared_prefix_blocks : 0;
  return hip_status(pa::launch_check_metadata(a, static_cast<hipStream_t>(stream)));
}

size_t pa_attention_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                        int32_t num_kv_heads, int32_t head_dim,
                                                        int32_t max_seq_len,
                                                        int32_t shared_prefix_blocks,
                                                        int32_t num_splits) {
  const size_t plain = pa_attention_workspace_size(num_seqs, num_seqs, num_q_heads, num_kv_heads,
                                                   head_dim, max_seq_len, 1, num_splits);
  if (plain == 0 || shared_prefix_blocks < 0 ||
      (int64_t)shared_prefix_blocks * pa::kBlockSize > max_seq_len)
    return 0;
  if (shared_prefix_blocks == 0) return plain;
  const int group = num_q_heads / num_kv_heads;
  const int rest = max(max_seq_len - shared_prefix_blocks * pa::kBlockSize, 1);
  const int chunks = plan_chunks(num_seqs, num_kv_heads, group, rest, num_splits, true, num_seqs,
                                 PA_BF16, head_dim, device_geometry().cus, true);
  const size_t casc = workspace_layout(num_seqs, num_q_heads, head_dim, chunks + num_seqs).total;
  return casc > plain ? casc : plain;
}

}  // extern "C"

namespace {

int shared_prefix_impl(void* out, const void* q, const void* kv_cache, int64_t num_blocks,
                       int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                       const int32_t* block_table, int32_t block_table_stride,
                       const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                       int32_t num_q_heads, float scale, int32_t shared_prefix_blocks,
                       void* workspace, size_t workspace_bytes, int32_t num_splits,
                       const pa::NewTokens& fresh, void* stream) {
  const int P = shared_prefix_blocks;
  if (P < 0 || (int64_t)P * pa::kBlockSize > max_seq_len) return PA_ERR_INVALID_ARG;
  const int group = num_kv_heads > 0 && num_q_heads % num_kv_heads == 0
                        ? num_q_heads / num_kv_heads : 0;
  // no prefix, or no matrix-core path for this configuration: plain decode
  if (P == 0 || !pa::prefill_supported(dtype, head_dim, group))
    return decode_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                       block_table, block_table_stride, seq_lens, num_seqs, max_seq_len,
                       num_q_heads, scale, workspace, workspace_bytes, num_splits, fresh,
                       stream);
  pa::DecodeArgs a{};
  const int st = attention_common(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim,
                                  dtype, block_table, block_table_stride, seq_lens, num_seqs,
                                  max_seq_len, num_q_heads, scale, workspace, workspace_bytes,
                                  splits_plan(num_splits), 1, P, &a);
  if (st <= 0) return st;
  // the new tokens sit past the prefix: the split over each request's
  // suffix reads them from the input and stores them (the prefix pass reads
  // prefix keys only)
  a.fresh = fresh;
  pa::PrefillArgs p{};
  p.q = q;
  p.kv = kv_cache;
  p.block_table = block_table;  // row 0 holds the shared prefix like every row
  p.bt_stride = block_table_stride;
  p.num_seqs = 1;
  p.num_kv_heads = num_kv_heads;
  p.num_q_heads = num_q_heads;
  p.max_tiles = (int)ceil_div(num_seqs, pa::kQueriesPerTile) + 1;
  p.max_query_len = num_seqs;
  p.beside_decode = 1;
  p.tile_shape = -1;
  p.num_xcds = device_geometry().xcds;
  p.cus_per_xcd = std::max(1, device_geometry().cus / p.num_xcds);
  p.scale_log2 = a.scale_log2;
  p.cascade_rows = num_seqs;
  p.cascade_keys = P * pa::kBlockSize;
  p.prefix_slot0 = a.prefix_slot0;
  p.ws_ml = a.ws_ml;
  p.ws_o = a.ws_o;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the prefix pass and the split over the suffixes in one launch, then the
  // merge of prefix and suffix partials
  const hipError_t e = pa::launch_fused(a, p, dtype, head_dim, group, s);
  if (e != hipSuccess) return PA_ERR_HIP;
  return hip_status(pa::launch_decode_merge(a, dtype, head_dim, group, s));
}

}  // namespace

extern "C" {

int pa_attention_decode_shared_prefix(void* out, const void* q, const void* kv_cache,
                                      int64_t num_blocks, int32_t block_size,
                                      int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                      const int32_t* block_table, int32_t block_table_stride,
                                      const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t max_seq_len, int32_t num_q_heads, float scale,
                                      int32_t shared_prefix_blocks, void* workspace,
                                      size_t workspace_bytes, int32_t num_splits, void* stream) {
  return shared_prefix_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim,
                            dtype, block_table, block_table_stride, seq_lens, num_seqs,
                            max_seq_len, num_q_heads, scale, shared_prefix_blocks, workspace,
                            workspace_bytes, num_splits, pa::NewTokens{}, stream);
}

int pa_cache_and_attend_decode_shared_prefix(
    void* out, const void* q, const void* key, const void* value, void* kv_cache,
    int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
    const int32_t* block_table, int32_t block_table_stride, const int32_t* seq_lens,
    int64_t* slot_mapping, int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
    float scale, int32_t shared_prefix_blocks, void* workspace, size_t workspace_bytes,
    int32_t num_splits, void* stream) {
  if (num_seqs > 0 && max_seq_len > 0 && !(key && value)) return PA_ERR_INVALID_ARG;
  pa::NewTokens f{};
  if (key || value) {
    const int st = fresh_tokens(key, value, kv_cache, slot_mapping, &f);
    if (st != PA_OK) return st;
  }
  return shared_prefix_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim,
                            dtype, block_table, block_table_stride, seq_lens, num_seqs,
                            max_seq_len, num_q_heads, scale, shared_prefix_blocks, workspace,
                            workspace_bytes, num_splits, f, stream);
}

}  // extern "C"

// ---- pa_cache_and_attend_mixed_no_workspace ---------------------------------
// The split-KV partials of callers that cannot allocate live in this array.
// Host code never passes `scratch` itself to a kernel (in host code the name
// is only a stand-in for the symbol): each device's copy is looked up once
// with hipGetSymbolAddress and that address is what the kernels receive.
static __device__ __align__(256) unsigned char scratch[PA_NO_WORKSPACE_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per device, filled on the device's first call

// Address and size of the current device's copy of `scratch` (looked up on
// the first call with that device current, then cached).
int scratch_address(void** out, size_t* bytes) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  *bytes = PA_NO_WORKSPACE_MAX_BYTES;
  return PA_OK;
}

}  // namespace

extern "C" int pa_cache_and_attend_mixed_no_workspace(
    void* out, const void* q, const void* key, const void* value, void* kv_cache,
    int64_t num_blocks, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
    int32_t dtype, const int32_t* block_table, int32_t block_table_stride,
    const int32_t* seq_lens, const int32_t* query_start_loc,
    const int32_t* num_computed_tokens, int64_t* slot_mapping, int32_t num_seqs,
    int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
    float scale, int32_t num_splits, void* stream) {
  // the bound the workspace query gives for these arguments (it covers every
  // plan the call may choose) must fit the array
  const size_t need = pa_attention_workspace_size(num_seqs, num_tokens, num_q_heads,
                                                  num_kv_heads, head_dim, max_seq_len,
                                                  max_query_len, num_splits);
  if (need > PA_NO_WORKSPACE_MAX_BYTES) return PA_ERR_SCRATCH;
  if (num_tokens > 0 && !(key && value)) return PA_ERR_INVALID_ARG;
  pa::NewTokens f{};
  if (key || value) {
    const int st = fresh_tokens(key, value, kv_cache, slot_mapping, &f);
    if (st != PA_OK) return st;
  }
  return mixed_impl(out, q, kv_cache, num_blocks, block_size, num_kv_heads, head_dim, dtype,
                    block_table, block_table_stride, seq_lens, query_start_loc,
                    num_computed_tokens, num_seqs, num_tokens, max_query_len, max_seq_len,
                    num_q_heads, scale, nullptr, 0, splits_plan(num_splits), f, stream,
                    scratch_address);
}
