// One launch holding two kinds of work-group: prefill tiles (compute-bound,
// matrix cores) and decode split ranges (bandwidth-bound).  Both are 4 waves
// of at most 256 VGPRs (two waves per SIMD), so a SIMD runs a tile wave
// beside a decode wave and the two kinds overlap without a second stream.
// The decode merge follows as its own launch on the same stream.
//
// Order.  The decode work-groups come first, so the dispatcher spreads them
// one per SIMD before any tile is placed; the tile work-groups follow with
// the head index fastest, so the live tiles (the grid is sized for an upper
// bound on the tile count) come before the empty ones, which exit at once at
// the end of the grid.  Tile waves raise their issue priority: on a SIMD
// shared with a decode wave, the latency-bound decode wave loses little and
// the tile's critical path shortens.
//
// Used for mixed chunked-prefill batches ("vllm v1 源码精读（三）" §4.2) and
// for the shared-prefix pass of a decode batch ("vllm v1 源码精读（三）"
// §3.5: requests sharing cached prefix blocks).
#include "pa_decode_impl.h"
#include "pa_prefill_impl.h"

namespace pa {
namespace {

template <typename E, int D, int HPW, int WPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void fused_attention_kernel(
    DecodeArgs da, PrefillArgs pa, int decode_wgs, int tile_heads) {
  const int b = blockIdx.x;  // work-group-uniform: the branch never splits a group
  if (b < decode_wgs) {
    decode_split_body<E, D, HPW>(da, b);
  } else {
    __builtin_amdgcn_s_setprio(3);
    const int t = b - decode_wgs;
    prefill_tile_body<E, D, WPW, 2, 1, true>(pa, t / tile_heads, t % tile_heads);
  }
}

template <typename E, int D, int HPW, int WPW>
hipError_t launch_typed(const DecodeArgs& da, const PrefillArgs& p, hipStream_t stream) {
  // tiles of 32 tokens per wave (4 waves, one key part), as the standalone
  // tile launch sizes them
  constexpr int QT = 16 * 2 * (4 / WPW);
  const int group = p.num_q_heads / p.num_kv_heads;
  const int tiles_x = ((p.max_tiles - p.num_seqs) * kQueriesPerTile + QT - 1) / QT + p.num_seqs;
  const int tile_heads = p.num_kv_heads * (group / WPW);
  const int64_t tile_wgs = (int64_t)tiles_x * tile_heads;
  const int64_t items = (int64_t)da.num_chunks * da.num_kv_heads * da.head_groups;
  const int64_t decode_wgs = (items + 3) / 4;
  const int64_t wgs = tile_wgs + decode_wgs;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fused_attention_kernel<E, D, HPW, WPW>), dim3((unsigned)wgs), dim3(256), 0,
                     stream, da, p, (int)decode_wgs, tile_heads);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_group(const DecodeArgs& da, const PrefillArgs& p, int group,
                        hipStream_t stream) {
  switch (group) {
    case 1: return launch_typed<E, D, 1, 1>(da, p, stream);
    case 2: return launch_typed<E, D, 2, 2>(da, p, stream);
    case 4:
    case 8: return launch_typed<E, D, 4, 4>(da, p, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename E>
hipError_t launch_dim(const DecodeArgs& da, const PrefillArgs& p, int head_dim, int group,
                      hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_group<E, 64>(da, p, group, stream);
    case 128: return launch_group<E, 128>(da, p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fused(const DecodeArgs& da, const PrefillArgs& p, int dtype, int head_dim,
                        int group, hipStream_t stream) {
  if (da.num_chunks <= 0 || da.num_seqs <= 0 || p.max_tiles <= 0) return hipErrorInvalidValue;
  switch (dtype) {
    case BF16::kind: return launch_dim<BF16>(da, p, head_dim, group, stream);
    case F16::kind: return launch_dim<F16>(da, p, head_dim, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
