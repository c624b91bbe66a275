// KV-cache write path on gfx950: slot computation, the reshape_and_cache
// scatter and whole-block copies.
//
//   slot = block_table[r][pos / 16] * 16 + pos % 16, pos = num_computed[r] + i
//     ("vllm v1 源码精读（三）" §3.4, Block Table 和 slot_mapping)
//   kv_cache[slot / 16][0 | 1][slot % 16] = key[t] | value[t]
//     ("vLLM 架构源码解析（一）" §3.3.3; "vllm v1 源码精读（三）" §3.4)
//   kv_cache[dst] = kv_cache[src] for each (src, dst) pair
//     (copy-on-write fork: "vLLM 架构源码解析（一）" §4.3.2)
//
// Both are pure data movement, bound by launch latency at serving sizes
// (a 593-token step moves 2.4 MB).  The scatter copies each token's K and V
// rows (num_kv_heads * head_dim elements, contiguous in both source and
// destination) with 16-byte vector loads/stores, one vector per lane, so a
// wavefront moves 1 KiB per instruction and every access is fully coalesced.
#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {

__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int64_t* __restrict__ slot_mapping, const int32_t* __restrict__ block_table,
    int32_t bt_stride, const int32_t* __restrict__ qsl,
    const int32_t* __restrict__ num_computed, int32_t num_seqs, int32_t num_tokens) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  // request owning token t: the last r with qsl[r] <= t (empty requests skip)
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int64_t pos = (int64_t)num_computed[r] + (t - qsl[r]);
  const int64_t lb = pos / kBlockSize;
  int64_t slot = -1;
  if (pos >= 0 && lb < bt_stride) {
    const int32_t phys = block_table[(int64_t)r * bt_stride + lb];
    if (phys >= 0) slot = (int64_t)phys * kBlockSize + pos % kBlockSize;
  }
  slot_mapping[t] = slot;
}

__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const uint8_t* __restrict__ key, const uint8_t* __restrict__ value,
    uint8_t* __restrict__ kv_cache, const int64_t* __restrict__ slot_mapping,
    int32_t num_tokens, int32_t row_vecs /* 16-byte vectors per K row */) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_token = 2 * (int64_t)row_vecs;
  const int64_t t = g / per_token;
  if (t >= num_tokens) return;
  const int rem = (int)(g - t * per_token);
  const int half = rem / row_vecs;  // 0 = K, 1 = V
  const int v = rem - half * row_vecs;
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;
  const int64_t row_bytes = (int64_t)row_vecs * 16;
  const int64_t blk = slot / kBlockSize, off = slot % kBlockSize;
  const int64_t dst = blk * (2 * kBlockSize * row_bytes) + half * (kBlockSize * row_bytes) +
                      off * row_bytes + (int64_t)v * 16;
  const uint8_t* src = (half ? value : key) + t * row_bytes + (int64_t)v * 16;
  store16(kv_cache + dst, load16(src));
}

// Whole-block copy.  A block is one contiguous run of block_bytes (K half
// then V half), so a copy is a flat 16-byte-vector stream.  Each work-group
// moves one 16 KiB piece of one pair: four 16-byte loads per lane issued
// before any store, so a wavefront keeps 4 KiB in flight.  Grid: x = piece
// index over all pairs (pair-major), so consecutive work-groups read
// consecutive addresses of one block.
constexpr int kCopyVecsPerLane = 4;
constexpr int kCopyPieceBytes = 256 * 16 * kCopyVecsPerLane;

__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ kv_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int32_t pieces_per_block,
                                                          int64_t block_bytes) {
  const int pair = uniform((int)(blockIdx.x / (unsigned)pieces_per_block));
  const int piece = uniform((int)(blockIdx.x - (unsigned)pair * (unsigned)pieces_per_block));
  const int32_t src = load_scalar(pairs + 2 * pair);
  const int32_t dst = load_scalar(pairs + 2 * pair + 1);
  if (src < 0 || dst < 0) return;
  const uint8_t* s = kv_cache + (int64_t)src * block_bytes;
  uint8_t* d = kv_cache + (int64_t)dst * block_bytes;
  const int64_t base = (int64_t)piece * kCopyPieceBytes;
  u32x4_t v[kCopyVecsPerLane];
#pragma unroll
  for (int i = 0; i < kCopyVecsPerLane; ++i) {
    const int64_t off = base + (int64_t)(i * 256 + (int)threadIdx.x) * 16;
    if (off < block_bytes) v[i] = load16(s + off);
  }
#pragma unroll
  for (int i = 0; i < kCopyVecsPerLane; ++i) {
    const int64_t off = base + (int64_t)(i * 256 + (int)threadIdx.x) * 16;
    if (off < block_bytes) store16(d + off, v[i]);
  }
}

hipError_t launch_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                               int32_t bt_stride, const int32_t* qsl,
                               const int32_t* num_computed, int32_t num_seqs,
                               int32_t num_tokens, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (num_tokens + threads - 1) / threads;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(threads), 0, stream, slot_mapping,
                     block_table, bt_stride, qsl, num_computed, num_seqs, num_tokens);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kv_cache,
                                    const int64_t* slot_mapping, int32_t num_tokens,
                                    int32_t row_bytes, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int row_vecs = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * 2 * row_vecs;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value),
                     static_cast<uint8_t*>(kv_cache), slot_mapping, num_tokens, row_vecs);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* kv_cache, const int32_t* pairs, int32_t num_pairs,
                              int64_t block_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const int64_t pieces = (block_bytes + kCopyPieceBytes - 1) / kCopyPieceBytes;
  const int64_t grid = pieces * num_pairs;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     static_cast<uint8_t*>(kv_cache), pairs, (int32_t)pieces, block_bytes);
  return hipGetLastError();
}

}  // namespace pa
