// Internal launch interface between the C-ABI front end (pa_api.cpp) and the
// HIP kernels.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlockSize = 16;  // tokens per paged block
constexpr int F32_KIND = 0;     // pa_dtype value of fp32

// The step's new tokens when the attention launch also stores them into the
// cache (k == null: the caller scattered them beforehand).  Token t of the
// step (row t of k and v) sits at position num_computed + (t - qsl[r]) of its
// request r -- for a decode row, seq_len - 1.  Every reader of such a key row
// in the launch takes it from k / v, and exactly one work-group writes it to
// the cache, so no access in the launch depends on another's store.
struct NewTokens {
  const void* k;              // [rows, Hkv, D], cache dtype
  const void* v;
  void* kv;                   // the cache (writable view of DecodeArgs::kv)
  int64_t* slot_out;          // [rows] or null: the cache slot of each new token
};

// Arguments shared by the decode (split-KV) kernel and its merge kernel.
struct DecodeArgs {
  void* out;                  // [rows, Hq, D]
  const void* q;              // [rows, Hq, D]
  const void* kv;             // [NB, 2, 16, Hkv, D]
  const int32_t* block_table; // [R, bt_stride]
  int32_t bt_stride;
  const int32_t* seq_lens;    // [R]
  const int32_t* qsl;         // [R+1] or null: row r = request r, all decode
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t num_chunks;         // partitions of the flattened block list per kv head
  int32_t head_groups;        // waves per kv head (query heads split in groups)
  float scale_log2;           // softmax scale * log2(e)
  float* ws_ml;               // [(R + num_chunks), Hq, 2]  (max, sum) per partial
  float* ws_o;                // [(R + num_chunks), Hq, D]  unnormalised partial outputs
  int32_t* ws_meta;           // [R, 4]: first range, last range (-1: no merge), W, 0
  // Shared prefix (0 / -1 when absent): the first skip_blocks table entries
  // of every row are one common prefix, attended separately; request r's
  // prefix partial (max, sum, output) is in workspace slot prefix_slot0 + r.
  int32_t skip_blocks;
  int32_t prefix_slot0;
  NewTokens fresh;
};

// Arguments of the MFMA prefill-tile kernel.
struct PrefillArgs {
  void* out;                  // [T, Hq, D]
  const void* q;              // [T, Hq, D]
  const void* kv;
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  const int32_t* num_computed;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t max_tiles;          // upper bound on the tile count (grid size)
  int32_t max_query_len;      // (host) longest chunk: picks the tile shape
  int32_t beside_decode;      // (host) 1: runs concurrently with decode rows
  int32_t tile_shape;         // (host) -1: chosen from the chunk; 0 | 1: forced
  int32_t num_xcds;           // dies of the device, each with its own L2 (>= 1)
  int32_t cus_per_xcd;        // compute units of one die (>= 1)
  float scale_log2;
  // Shared-prefix pass (cascade_rows > 0): one virtual request whose queries
  // are rows 0 .. cascade_rows - 1 of q and whose keys are the first
  // cascade_keys positions of block_table row 0, all visible; each row's
  // partial (max, sum, unnormalised output) goes to workspace slot
  // prefix_slot0 + row instead of `out`.
  int32_t cascade_rows;
  int32_t cascade_keys;
  int32_t prefix_slot0;
  float* ws_ml;
  float* ws_o;
  NewTokens fresh;
};

// Arguments of the metadata check (pa_check_metadata).
struct MetaCheckArgs {
  uint32_t* flags;            // OR of pa_meta_flag bits
  const int32_t* block_table;
  int32_t bt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;         // null: a decode batch (one query per request)
  const int32_t* num_computed;
  const int64_t* slots;       // or null
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_query_len;
  int32_t max_seq_len;
  int64_t num_blocks;
  int32_t shared_prefix_blocks;  // 0: no shared prefix to check
};

hipError_t launch_check_metadata(const MetaCheckArgs& a, hipStream_t stream);

constexpr int kQueriesPerTile = 16;  // fewest query tokens per prefill tile (grid bound)

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               int32_t bt_stride, const int32_t* qsl,
                               const int32_t* num_computed, int32_t num_seqs,
                               int32_t num_tokens, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kv_cache,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    int32_t row_bytes, hipStream_t stream);

hipError_t launch_copy_blocks(void* kv_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, hipStream_t stream);

// Query heads one decode wave serves (the rest of a GQA group goes to more
// waves): up to 4, and 2 for fp32 rows of 128 dims, whose four heads of
// queries, accumulators and two in-flight blocks do not fit 256 VGPRs.
inline int decode_heads_per_wave(int dtype, int head_dim, int group) {
  const int h = group < 4 ? group : 4;
  return (dtype == F32_KIND && head_dim == 128 && h > 2) ? 2 : h;
}

// dtype: pa_dtype value; head_dim 64 | 128; group = Hq / Hkv in {1,2,4,8}.
// launch_decode = launch_decode_split then launch_decode_merge.
hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group,
                         hipStream_t stream);
hipError_t launch_decode_split(const DecodeArgs& a, int dtype, int head_dim, int group,
                               hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, int dtype, int head_dim, int group,
                               hipStream_t stream);

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int group,
                          hipStream_t stream);

bool prefill_supported(int dtype, int head_dim, int group);

// fp32 cache: the same prefill-chunk attention on the vector ALU (16-token
// tiles, grid max_tiles x num_kv_heads); head_dim 64 | 128, group 1|2|4|8.
hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, int group, hipStream_t stream);

// Prefill tiles (32 tokens per wave) and the decode split in one launch; the
// caller launches the decode merge afterwards on the same stream.
hipError_t launch_fused(const DecodeArgs& da, const PrefillArgs& p, int dtype, int head_dim,
                        int group, hipStream_t stream);

}  // namespace pa
