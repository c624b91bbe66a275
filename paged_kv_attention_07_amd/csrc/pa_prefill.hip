// Tile-shape choice and launchers of the prefill tile kernel (device code
// in pa_prefill_impl.h).
#include "pa_prefill_impl.h"

namespace pa {
namespace {

// Tile shape of a launch.
//   0: 16 tokens per wave, two key parts of 4 waves: short chunks alone, which
//      would leave most of the chip idle with fewer, larger tiles;
//   1: 32 tokens per wave, one part of 4 waves: long chunks (each K and V
//      fragment read from LDS feeds two products), and tiles running beside
//      concurrent decode rows (a 4-wave work-group fits next to one decode
//      wave per SIMD).
// A caller's plan may force either (tile_shape 0 | 1).
int choose_shape(const PrefillArgs& a) {
  if (a.tile_shape == 0 || a.tile_shape == 1) return a.tile_shape;
  return (a.beside_decode || a.max_query_len >= 1024) ? 1 : 0;
}

template <typename E, int D, int WPW, int NT, int KSPLIT>
hipError_t launch_shape(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  // max_tiles bounds the tile count for 16-token tiles; scale it to this shape
  constexpr int QT = tile_tokens<WPW, NT>();
  const int tiles = ((a.max_tiles - a.num_seqs) * kQueriesPerTile + QT - 1) / QT + a.num_seqs;
  const dim3 grid((unsigned)tiles, (unsigned)(a.num_kv_heads * (group / WPW)));
  hipLaunchKernelGGL((prefill_tile_kernel<E, D, WPW, NT, KSPLIT>), grid, dim3(256 * KSPLIT), 0,
                     stream, a);
  return hipGetLastError();
}

template <typename E, int D, int WPW>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
  return choose_shape(a) == 1 ? launch_shape<E, D, WPW, 2, 1>(a, stream)
                              : launch_shape<E, D, WPW, 1, 2>(a, stream);
}

template <typename E, int D>
hipError_t launch_group(const PrefillArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_typed<E, D, 1>(a, stream);
    case 2: return launch_typed<E, D, 2>(a, stream);
    case 4:
    case 8: return launch_typed<E, D, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename E>
hipError_t launch_dim(const PrefillArgs& a, int head_dim, int group, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_group<E, 64>(a, group, stream);
    case 128: return launch_group<E, 128>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int group) {
  return (dtype == BF16::kind || dtype == F16::kind) && (head_dim == 64 || head_dim == 128) &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}

hipError_t launch_prefill(const PrefillArgs& a, int dtype, int head_dim, int group,
                          hipStream_t stream) {
  if (a.max_tiles <= 0) return hipSuccess;
  switch (dtype) {
    case BF16::kind: return launch_dim<BF16>(a, head_dim, group, stream);
    case F16::kind: return launch_dim<F16>(a, head_dim, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
