// Prefill-chunk attention over an fp32 paged KV cache on gfx950 (vector ALU).
//
// Same operation as the matrix-core tile kernel ("vllm v1 源码精读（三）" §4.2;
// "Inside vLLM" §3.4): token i of a request's chunk (absolute position
// pos = num_computed + i) attends keys 0..pos of its own request through the
// request's block table, with the causal mask inside the chunk.  gfx950 has
// no fp32-input matrix-core product at a useful rate for this (fp32 data would
// have to be rounded to a 16-bit type first, changing the result), so an fp32
// cache is attended with fp32 fused multiply-adds: the result matches the
// plain definition to fp32 rounding.
//
// Tiling.  A work-group (4 waves) owns 16 query tokens of one request and one
// KV head, i.e. 16 * G query rows (G = query heads per KV head), row
// tok * G + g.  The rows' queries (times the softmax scale, in the log2
// domain) stay in LDS; each 16-key paged block of K and V is staged through
// LDS once and used by all rows.  Per block:
//   scores   thread (slot, key): key = tid % 16, rows slot + 16 k, k < G;
//            the 16 scores of a row sit in 16 adjacent lanes, so the row max
//            and sum are 4-step butterflies inside the lane group;
//   softmax  online (running max m and sum l per row, rescale by
//            exp2(m_old - m_new)); probabilities go to LDS;
//   output   thread (column group, row group): 4 consecutive head dims of
//            G * D / 64 rows, accumulated from the 16 probabilities and V rows.
// Q and K rows in LDS are padded by 16 bytes, so the 16 key rows (and the 4
// query rows) a wave reads at one column fall on distinct banks.
//
// New tokens.  When the launch also stores the step's new tokens (fresh.k !=
// null), keys at positions >= num_computed come from the new-token input
// (row q0 + key - num_computed) instead of the cache, and each work-group
// stores its own tokens' K and V rows of its KV head into the cache after its
// key loop; the work-groups of KV head 0 also write the tokens' slots.  No
// access of the launch then depends on another work-group's store.
#include <math.h>

#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {
namespace {

constexpr int kTileTokens = 16;  // query tokens per work-group

// Request and tile (index within the request) owned by work-group `bx`:
// requests with more than one query token contribute ceil(qlen / 16) tiles
// each, in request order; -1 past the last tile (the grid is an upper bound).
__device__ void find_tile(const PrefillArgs& a, int bx, int* req, int* tile) {
  int found_r = -1, found_t = 0, running = 0;
  for (int base = 0; base < a.num_seqs && found_r < 0; base += kWave) {
    const int r = base + lane_id();
    int nt = 0;
    if (r < a.num_seqs) {
      const int ql = a.qsl[r + 1] - a.qsl[r];
      nt = ql > 1 ? (ql + kTileTokens - 1) / kTileTokens : 0;
    }
    const int incl = wave_incl_scan(nt) + running;
    const uint64_t hit = __ballot(nt > 0 && bx >= incl - nt && bx < incl);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      found_r = base + src;
      found_t = bx - (readlane(incl, src) - readlane(nt, src));
    }
    running = readlane(incl, kWave - 1);
  }
  *req = found_r;
  *tile = found_t;
}

template <int D, int G>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int NR = kTileTokens * G;  // query rows of the tile
  constexpr int QS = D + 4;            // LDS row stride (floats) of Q and K
  constexpr int CG = D / 4;            // 4-float columns of a row
  constexpr int RG = 256 / CG;         // row groups of the output mapping
  constexpr int ORPT = NR / RG;        // output rows per thread
  static_assert(NR % RG == 0, "unsupported tile");

  __shared__ __attribute__((aligned(16))) float sq[NR * QS];
  __shared__ __attribute__((aligned(16))) float sk[kBlockSize * QS];
  __shared__ __attribute__((aligned(16))) float sv[kBlockSize * D];
  __shared__ __attribute__((aligned(16))) float sp[NR * kBlockSize];
  __shared__ float salpha[NR];
  __shared__ float sl[NR];
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  // XCD-aware numbering: work-groups go to the 8 XCDs in turn; renumber them
  // (a bijection of the grid) so each XCD runs a contiguous block of (head,
  // tile) pairs and the keys a head's tiles all re-read stay in one L2
  const int tiles = gridDim.x;
  const int total = tiles * gridDim.y;
  const int lin = blockIdx.y * tiles + blockIdx.x;
  const int nx = a.num_xcds;       // the device's dies, each with its own L2
  const int xcd = lin % nx, local = lin / nx;
  const int idx = xcd * (total / nx) + min(xcd, total % nx) + local;
  const int h = idx / tiles;
  if (tid < kWave) {
    int r, t;
    find_tile(a, idx % tiles, &r, &t);
    if (tid == 0) {
      s_tile[0] = r;
      s_tile[1] = t;
    }
  }
  __syncthreads();
  const int r = s_tile[0];
  if (r < 0) return;  // work-group-uniform
  const int tile_start = s_tile[1] * kTileTokens;
  const int q0 = a.qsl[r];
  const int qlen = a.qsl[r + 1] - q0;
  const int nc = a.num_computed[r];
  const int tile_valid = min(kTileTokens, qlen - tile_start);
  const int kend = min(a.seq_lens[r], nc + tile_start + tile_valid);  // keys the tile needs
  const int nblk = (kend + kBlockSize - 1) / kBlockSize;
  const int Hq = a.num_q_heads;
  const int64_t tok_stride = (int64_t)a.num_kv_heads * D;  // floats
  const int64_t half_stride = kBlockSize * tok_stride;
  const float* kv = static_cast<const float*>(a.kv);
  const int32_t* bt = a.block_table + (int64_t)r * a.bt_stride;
  const bool fresh = a.fresh.k != nullptr;
  const int nfresh = fresh ? nc : 0x7fffffff;  // first key taken from the input rows

  // queries of the tile, scaled into the log2 domain; rows past the chunk are 0
  const float* qg = static_cast<const float*>(a.q);
  for (int x = tid; x < NR * CG; x += 256) {
    const int row = x / CG, c = x % CG;
    const int tok = row / G, g = row % G;
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
    if (tok < tile_valid)
      v = *reinterpret_cast<const f32x4_t*>(
              qg + ((int64_t)(q0 + tile_start + tok) * Hq + h * G + g) * D + 4 * c) *
          a.scale_log2;
    *reinterpret_cast<f32x4_t*>(&sq[row * QS + 4 * c]) = v;
  }

  const int key = tid % kBlockSize;  // score mapping
  const int slot = tid / kBlockSize;
  const int col = tid % CG;          // output mapping
  const int rgrp = tid / CG;
  float m[G], l[G];
#pragma unroll
  for (int k = 0; k < G; ++k) {
    m[k] = -INFINITY;
    l[k] = 0.f;
  }
  f32x4_t o[ORPT];
#pragma unroll
  for (int k = 0; k < ORPT; ++k) o[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int lb = 0; lb < nblk; ++lb) {
    __syncthreads();  // the previous block's K, V and probabilities are used up
    const int64_t phys = bt[lb];
    for (int x = tid; x < 2 * kBlockSize * CG; x += 256) {
      const int hv = x / (kBlockSize * CG);
      const int kr = (x / CG) % kBlockSize;
      const int c = x % CG;
      const int j = lb * kBlockSize + kr;
      f32x4_t v = {0.f, 0.f, 0.f, 0.f};  // keys past the tile's last one: zero rows
      if (j < kend) {
        const float* src;
        if (j >= nfresh)
          src = static_cast<const float*>(hv ? a.fresh.v : a.fresh.k) +
                (int64_t)(q0 + j - nc) * tok_stride;
        else
          src = kv + phys * 2 * half_stride + hv * half_stride + kr * tok_stride;
        v = *reinterpret_cast<const f32x4_t*>(src + h * D + 4 * c);
      }
      float* dst = hv ? &sv[kr * D + 4 * c] : &sk[kr * QS + 4 * c];
      *reinterpret_cast<f32x4_t*>(dst) = v;
    }
    __syncthreads();

    // scores of rows slot + 16 k against key `key` of the block
    float s[G];
#pragma unroll
    for (int k = 0; k < G; ++k) s[k] = 0.f;
#pragma unroll 2
    for (int c = 0; c < CG; ++c) {
      const f32x4_t kk = *reinterpret_cast<const f32x4_t*>(&sk[key * QS + 4 * c]);
#pragma unroll
      for (int k = 0; k < G; ++k) {
        const f32x4_t qq =
            *reinterpret_cast<const f32x4_t*>(&sq[(slot + kBlockSize * k) * QS + 4 * c]);
        s[k] = fmaf(qq[0], kk[0], s[k]);
        s[k] = fmaf(qq[1], kk[1], s[k]);
        s[k] = fmaf(qq[2], kk[2], s[k]);
        s[k] = fmaf(qq[3], kk[3], s[k]);
      }
    }
    const int j = lb * kBlockSize + key;
#pragma unroll
    for (int k = 0; k < G; ++k) {
      const int row = slot + kBlockSize * k;
      const int tok = row / G;
      const bool vis = tok < tile_valid && j <= nc + tile_start + tok && j < kend;
      const float sv_ = vis ? s[k] : -INFINITY;
      float mx = sv_;
      mx = row_max16(mx);
      const float mn = fmaxf(m[k], mx);
      float alpha = 1.f, p = 0.f;
      if (mn != -INFINITY) {  // row has a visible key so far
        alpha = __builtin_amdgcn_exp2f(m[k] - mn);
        p = vis ? __builtin_amdgcn_exp2f(sv_ - mn) : 0.f;
      }
      float ps = p;
      ps = row_sum16(ps);
      l[k] = l[k] * alpha + ps;
      m[k] = mn;
      sp[row * kBlockSize + key] = p;
      if (key == 0) salpha[row] = alpha;
    }
    __syncthreads();

    // output rows rgrp + RG k, head dims 4 col .. 4 col + 3
#pragma unroll
    for (int k = 0; k < ORPT; ++k) o[k] *= salpha[rgrp + RG * k];
#pragma unroll 1
    for (int kr = 0; kr < kBlockSize; kr += 4) {
      f32x4_t vv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        vv[u] = *reinterpret_cast<const f32x4_t*>(&sv[(kr + u) * D + 4 * col]);
#pragma unroll
      for (int k = 0; k < ORPT; ++k) {
        const f32x4_t pp =
            *reinterpret_cast<const f32x4_t*>(&sp[(rgrp + RG * k) * kBlockSize + kr]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          o[k][0] = fmaf(pp[u], vv[u][0], o[k][0]);
          o[k][1] = fmaf(pp[u], vv[u][1], o[k][1]);
          o[k][2] = fmaf(pp[u], vv[u][2], o[k][2]);
          o[k][3] = fmaf(pp[u], vv[u][3], o[k][3]);
        }
      }
    }
  }

  if (key == 0) {
#pragma unroll
    for (int k = 0; k < G; ++k) sl[slot + kBlockSize * k] = l[k];
  }
  __syncthreads();
  float* og = static_cast<float*>(a.out);
#pragma unroll
  for (int k = 0; k < ORPT; ++k) {
    const int row = rgrp + RG * k;
    const int tok = row / G, g = row % G;
    if (tok < tile_valid) {
      const float lsum = sl[row];
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      *reinterpret_cast<f32x4_t*>(og + ((int64_t)(q0 + tile_start + tok) * Hq + h * G + g) * D +
                                  4 * col) = o[k] * inv;
    }
  }

  // this tile's new tokens into the cache (KV head h), after every read
  if (fresh) {
    float* kvw = static_cast<float*>(a.fresh.kv);
    for (int x = tid; x < tile_valid * 2 * CG; x += 256) {
      const int i = x / (2 * CG);
      const int hv = (x / CG) & 1;
      const int c = x % CG;
      const int p = nc + tile_start + i;  // position in the request
      const int64_t id = bt[p / kBlockSize];
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(
          static_cast<const float*>(hv ? a.fresh.v : a.fresh.k) +
          (int64_t)(q0 + tile_start + i) * tok_stride + h * D + 4 * c);
      *reinterpret_cast<f32x4_t*>(kvw + id * 2 * half_stride + hv * half_stride +
                                  (int64_t)(p % kBlockSize) * tok_stride + h * D + 4 * c) = v;
      if (h == 0 && hv == 0 && c == 0 && a.fresh.slot_out)
        a.fresh.slot_out[q0 + tile_start + i] = id * kBlockSize + p % kBlockSize;
    }
  }
}

template <int D, int G>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
  // max_tiles bounds the number of 16-token tiles
  const dim3 grid((unsigned)a.max_tiles, (unsigned)a.num_kv_heads);
  hipLaunchKernelGGL((prefill_f32_kernel<D, G>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_group(const PrefillArgs& a, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_typed<D, 1>(a, stream);
    case 2: return launch_typed<D, 2>(a, stream);
    case 4: return launch_typed<D, 4>(a, stream);
    case 8: return launch_typed<D, 8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, int head_dim, int group, hipStream_t stream) {
  if (a.max_tiles <= 0 || a.num_kv_heads <= 0) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_group<64>(a, group, stream);
    case 128: return launch_group<128>(a, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
