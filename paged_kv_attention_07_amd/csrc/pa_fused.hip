// One launch holding two kinds of work-group: prefill tiles (compute-bound,
// matrix cores) and decode split ranges (bandwidth-bound).  Work-groups
// 0 .. tile_wgs - 1 are tiles, the rest decode ranges; both are 4 waves of at
// most 246 VGPRs, so each SIMD runs a tile wave beside a decode wave and the
// two kinds overlap without a second stream.  The decode merge follows as
// its own launch on the same stream.
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
    DecodeArgs da, PrefillArgs pa, int tile_wgs, int tiles_x) {
  const int b = blockIdx.x;  // work-group-uniform: the branch never splits a group
  if (b < tile_wgs)
    prefill_tile_body<E, D, WPW, 2, 1>(pa, b % tiles_x, b / tiles_x);
  else
    decode_split_body<E, D, HPW>(da, b - tile_wgs);
}

template <typename E, int D, int HPW, int WPW>
hipError_t launch_typed(const DecodeArgs& da, const PrefillArgs& p, hipStream_t stream) {
  // tiles of 32 tokens per wave (4 waves, one key part), as the standalone
  // tile launch sizes them
  constexpr int QT = 16 * 2 * (4 / WPW);
  const int group = p.num_q_heads / p.num_kv_heads;
  const int tiles_x = ((p.max_tiles - p.num_seqs) * kQueriesPerTile + QT - 1) / QT + p.num_seqs;
  const int64_t tile_wgs = (int64_t)tiles_x * p.num_kv_heads * (group / WPW);
  const int64_t items = (int64_t)da.num_chunks * da.num_kv_heads * da.head_groups;
  const int64_t wgs = tile_wgs + (items + 3) / 4;
  if (wgs > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fused_attention_kernel<E, D, HPW, WPW>), dim3((unsigned)wgs), dim3(256), 0,
                     stream, da, p, (int)tile_wgs, tiles_x);
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
