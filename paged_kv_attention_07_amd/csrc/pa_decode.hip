// Launchers of the decode split and merge kernels (device code in
// pa_decode_impl.h).
#include "pa_decode_impl.h"

namespace pa {
namespace {

template <typename E, int D, int HPW>
hipError_t launch_split_typed(const DecodeArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.num_chunks * a.num_kv_heads * a.head_groups;
  const unsigned wgs = (unsigned)((items + 3) / 4);
  hipLaunchKernelGGL((decode_split_kernel<E, D, HPW>), dim3(wgs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_merge_typed(const DecodeArgs& a, hipStream_t stream) {
  const unsigned merges = (unsigned)a.num_seqs * (unsigned)a.num_q_heads;
  if ((a.num_chunks > 1 || a.prefix_slot0 >= 0) && merges > 0) {
    hipLaunchKernelGGL((decode_merge_kernel<E, D>), dim3(merges), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename E, int D>
hipError_t launch_hpw(const DecodeArgs& a, int group, bool split, hipStream_t stream) {
  if (!split) return launch_merge_typed<E, D>(a, stream);
  if (group != 1 && group != 2 && group != 4 && group != 8) return hipErrorInvalidValue;
  switch (decode_heads_per_wave(E::kind, D, group)) {
    case 1: return launch_split_typed<E, D, 1>(a, stream);
    case 2: return launch_split_typed<E, D, 2>(a, stream);
    case 4:
      if constexpr (E::kind == F32::kind && D == 128) return hipErrorInvalidValue;  // never chosen
      else return launch_split_typed<E, D, 4>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename E>
hipError_t launch_dim(const DecodeArgs& a, int head_dim, int group, bool split,
                      hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_hpw<E, 64>(a, group, split, stream);
    case 128: return launch_hpw<E, 128>(a, group, split, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_part(const DecodeArgs& a, int dtype, int head_dim, int group, bool split,
                       hipStream_t stream) {
  if (a.num_chunks <= 0 || a.num_seqs <= 0) return hipSuccess;
  switch (dtype) {
    case F32::kind: return launch_dim<F32>(a, head_dim, group, split, stream);
    case BF16::kind: return launch_dim<BF16>(a, head_dim, group, split, stream);
    case F16::kind: return launch_dim<F16>(a, head_dim, group, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, int dtype, int head_dim, int group,
                               hipStream_t stream) {
  return launch_part(a, dtype, head_dim, group, true, stream);
}

hipError_t launch_decode_merge(const DecodeArgs& a, int dtype, int head_dim, int group,
                               hipStream_t stream) {
  return launch_part(a, dtype, head_dim, group, false, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int head_dim, int group,
                         hipStream_t stream) {
  const hipError_t e = launch_decode_split(a, dtype, head_dim, group, stream);
  return e != hipSuccess ? e : launch_decode_merge(a, dtype, head_dim, group, stream);
}

}  // namespace pa
