// Device-side check of the step metadata that the attention launches trust:
// request lengths, query offsets, computed counts, block-table entries and
// slots.  The pages' model runner takes this metadata from its scheduler
// unchecked ("vllm v1 源码精读（三）" §3.4 builds block tables and slots, §4.2
// the packed query offsets and computed counts); a caller debugging its own
// scheduler runs this check on the same stream before the attention call.
//
// One launch, three grid-stride passes over (request), (request, table
// entry) and (token); with a shared prefix of P blocks ("vllm v1 源码精读（三）"
// §3.5), also that every row starts with row 0's P block ids and holds at
// least 16 P keys; each violated condition sets its bit in *flags with a
// vector atomic OR.  Every read is inside the arrays' declared extents
// whatever their contents: a length or offset is only ever compared, and a
// table entry is read only at j < block_table_stride.
#include "pa.h"
#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {
namespace {

__device__ __forceinline__ void set_flag(uint32_t* flags, uint32_t bit) { atomicOr(flags, bit); }

__global__ __launch_bounds__(256) void check_metadata_kernel(MetaCheckArgs a) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  const bool decode = a.qsl == nullptr;

  // ---- per request: lengths, offsets, computed counts
  for (int64_t r = gid; r < a.num_seqs; r += nthr) {
    const int L = a.seq_lens[r];
    if (L < 0 || L > a.max_seq_len || (decode && L < 1)) set_flag(a.flags, PA_META_SEQ_LEN);
    if (L > 0 && ((int64_t)L + kBlockSize - 1) / kBlockSize > a.bt_stride)
      set_flag(a.flags, PA_META_TABLE_WIDTH);
    if ((int64_t)a.shared_prefix_blocks * kBlockSize > L) set_flag(a.flags, PA_META_SHARED_PREFIX);
    if (!decode) {
      const int64_t ql = (int64_t)a.qsl[r + 1] - a.qsl[r];
      if (ql < 0) set_flag(a.flags, PA_META_QUERY_START);
      if (ql > a.max_query_len) set_flag(a.flags, PA_META_QUERY_LEN);
      const int nc = a.num_computed[r];
      if (nc < 0 || (int64_t)nc + ql != L) set_flag(a.flags, PA_META_COMPUTED);
    }
  }
  if (gid == 0 && !decode && (a.qsl[0] != 0 || a.qsl[a.num_seqs] != a.num_tokens))
    set_flag(a.flags, PA_META_QUERY_START);

  // ---- per table entry read by attention: a valid block id
  const int64_t entries = (int64_t)a.num_seqs * a.bt_stride;
  for (int64_t x = gid; x < entries; x += nthr) {
    const int64_t r = x / a.bt_stride;
    const int j = (int)(x - r * a.bt_stride);
    const int L = a.seq_lens[r];
    if (L > 0 && j < ((int64_t)L + kBlockSize - 1) / kBlockSize) {
      const int32_t id = a.block_table[x];
      if (id < 0 || id >= a.num_blocks) set_flag(a.flags, PA_META_BLOCK_ID);
    }
    // a shared prefix: the same physical blocks at the head of every row
    if (j < a.shared_prefix_blocks && a.block_table[x] != a.block_table[j])
      set_flag(a.flags, PA_META_SHARED_PREFIX);
  }

  // ---- per token: slot inside the pool and not shared with a later token
  if (a.slots) {
    const int64_t pool_slots = a.num_blocks * kBlockSize;
    for (int64_t t = gid; t < a.num_tokens; t += nthr) {
      const int64_t s = a.slots[t];
      if (s < 0) continue;  // skipped token
      if (s >= pool_slots) set_flag(a.flags, PA_META_SLOT_RANGE);
      bool dup = false;
      for (int64_t u = t + 1; u < a.num_tokens; ++u) dup |= a.slots[u] == s;
      if (dup) set_flag(a.flags, PA_META_SLOT_DUP);
    }
  }
}

}  // namespace

hipError_t launch_check_metadata(const MetaCheckArgs& a, hipStream_t stream) {
  int64_t work = (int64_t)a.num_seqs * a.bt_stride;
  if (a.num_tokens > work) work = a.num_tokens;
  if (a.num_seqs > work) work = a.num_seqs;
  int64_t blocks = (work + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(check_metadata_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
