// Prefill-chunk attention over a paged KV cache on gfx950 (MFMA tiles).
//
// What it computes ("vllm v1 源码精读（三）" §4.2; "Inside vLLM" §3.4): for a
// request with q_len > 1 new tokens on top of num_computed cached ones, token
// i (absolute position pos = num_computed + i) attends keys 0..pos of its own
// request -- the cached history plus the earlier tokens of the chunk (causal
// inside the chunk).  Keys are read through the request's block table; the
// new tokens' K/V were scattered into the cache beforehand.
//
// Tiling.  A work-group (4 wavefronts) owns one tile of query tokens of one
// request and one group of query heads sharing a KV head: for GQA group 4 the
// 4 waves are the 4 query heads of a KV head over the same 16 tokens, so each
// K/V tile staged in LDS feeds 4 heads.  Keys are processed 64 at a time
// (four 16-token blocks looked up in the block table).
//
// Matrix-core mapping (v_mfma_f32_16x16x32_{bf16,f16}).  Scores are formed
// transposed, S^T = K Q^T (keys x tokens), because the accumulator layout of
// a 16x16 tile gives each lane 4 consecutive keys of ONE token: exactly the
// operand layout the second product O^T = V^T P^T needs for P^T, so the
// probabilities go from the softmax to the matrix core without moving across
// lanes.  Each lane then holds the output of one token, so the online-softmax
// rescale is a per-lane scalar.  V is written transposed into LDS (pairs of
// keys per 32-bit word) while it is staged.  The contraction order inside an
// MFMA is a permutation of the keys; A and B use the same permutation.
#include <math.h>

#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {
namespace {

template <typename E>
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (E::kind == BF16::kind) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

template <typename E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return E::kind == BF16::kind ? pack_bf16(lo, hi) : pack_f16(lo, hi);
}

constexpr int kKeysPerIter = 64;  // keys staged per iteration (4 paged blocks)


template <int D>
struct TileShape {
  static constexpr int ROWB = D * 2;              // bytes of one token's head row
  static constexpr int KROW = ROWB + 16;          // padded LDS row of K
  static constexpr int VROW = kKeysPerIter * 2 + 8;  // padded LDS row of V^T
  static constexpr int NKS = D / 32;              // MFMA k-steps of Q K^T
  static constexpr int NMT = D / 16;              // 16-dim tiles of the output
};

// One work-group = 4 waves = WPW query heads x (4 / WPW) token sub-tiles of 16.
template <typename E, int D, int WPW>
__global__ __launch_bounds__(256) void prefill_tile_kernel(PrefillArgs a) {
  using S = TileShape<D>;
  constexpr int NQS = 4 / WPW;       // 16-token sub-tiles per work-group
  constexpr int QT = 16 * NQS;       // tokens per tile
  // two stages: the next 64 keys are staged while the current ones are used
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][kKeysPerIter * S::KROW];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][D * S::VROW];
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hg = group / WPW;
  const int h = blockIdx.y / hg;
  const int hs = blockIdx.y - h * hg;

  // ---- which request / tile this work-group owns
  if (wave == 0) {
    int found_r = -1, found_t = 0, running = 0;
    const int want = blockIdx.x;
    for (int base = 0; base < a.num_seqs && found_r < 0; base += kWave) {
      const int r = base + lane;
      int nt = 0;
      if (r < a.num_seqs) {
        const int ql = a.qsl[r + 1] - a.qsl[r];
        nt = ql > 1 ? (ql + QT - 1) / QT : 0;
      }
      const int incl = wave_incl_scan(nt) + running;
      const int excl = incl - nt;
      const uint64_t hit = __ballot(nt > 0 && want >= excl && want < incl);
      if (hit) {
        const int src = __builtin_ctzll(hit);
        found_r = base + src;
        found_t = want - readlane(excl, src);
      }
      running = readlane(incl, kWave - 1);
    }
    if (lane == 0) {
      s_tile[0] = found_r;
      s_tile[1] = found_t;
    }
  }
  __syncthreads();
  const int r = uniform(s_tile[0]);
  if (r < 0) return;
  const int tile = uniform(s_tile[1]);

  const int q0 = a.qsl[r];
  const int qlen = a.qsl[r + 1] - q0;
  const int nc = a.num_computed[r];
  const int L = a.seq_lens[r];
  const int tile_start = tile * QT;
  const int tile_valid = min(QT, qlen - tile_start);
  const int kend = min(L, nc + tile_start + tile_valid);  // keys this tile needs
  const int niter = (kend + kKeysPerIter - 1) / kKeysPerIter;

  const int hw = wave % WPW;                 // head within the group
  const int sub = wave / WPW;                // 16-token sub-tile
  const int hq = h * group + hs * WPW + hw;
  const int n = lane & 15;                   // token column of this lane
  const int g = lane >> 4;                   // lane group
  const int sub_start = tile_start + sub * 16;
  const int sub_valid = max(0, min(16, qlen - sub_start));
  const int my_tok = min(n, max(sub_valid - 1, 0));
  const int pos = nc + sub_start + my_tok;   // this column's last visible key

  // Q^T fragments: token n, dims 32s + 8g .. +8
  u32x4_t qf[S::NKS];
  {
    const bool ok = n < sub_valid;
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                        ((int64_t)(q0 + sub_start + n) * a.num_q_heads + hq) * S::ROWB + g * 16;
#pragma unroll
    for (int s = 0; s < S::NKS; ++s) {
      u32x4_t z = {0u, 0u, 0u, 0u};
      qf[s] = ok ? load16(qp + s * 64) : z;
    }
  }

  const int64_t tok_stride = (int64_t)a.num_kv_heads * S::ROWB;
  const int64_t half_stride = kBlockSize * tok_stride;
  const int64_t blk_stride = 2 * half_stride;
  const uint8_t* kvh = static_cast<const uint8_t*>(a.kv) + (int64_t)h * S::ROWB;
  const int32_t* bt = a.block_table + (int64_t)r * a.bt_stride;

  // Physical ids of the 4 blocks holding keys [64 it, 64 it + 64): uniform
  // across the work-group (scalar loads), fetched two iterations ahead of use.
  const int nb_need = (kend + kBlockSize - 1) / kBlockSize;
  // id of the paged block this wavefront stages in iteration it (scalar load)
  auto block_id = [&](int it) {
    const int lb = it * 4 + wave;
    return lb < nb_need ? load_scalar(bt + lb) : 0;
  };

  // Staging: wavefront w moves paged block w of the iteration (keys
  // 16w .. 16w+15), so the block id it needs is wave-uniform.  K rows go to
  // LDS as they are; V goes in transposed, two keys per 32-bit word.
  // K: lane l, step i -> key 4i + l/16 (D=128) or 8i + l/8 (D=64), 16-byte
  // column l % CPR.  V: lane l, step i -> key pair 4i + l/16 (D=128) or l/8.
  constexpr int CPR = S::ROWB / 16;          // 16-byte columns per row
  constexpr int KPT = 16 * CPR / kWave;      // K pieces per lane per block
  constexpr int VPT = 8 * (D / 8) / kWave;   // V key-pair items per lane per block
  u32x4_t kreg[KPT], vreg[VPT][2];
  auto fetch = [&](int it, int phys) {
    const int key0 = it * kKeysPerIter + 16 * wave;
    const uint8_t* blk = kvh + (int64_t)phys * blk_stride;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = i * kWave + lane;
      const int kb = c / CPR, dc = c % CPR;
      u32x4_t z = {0u, 0u, 0u, 0u};
      kreg[i] = z;
      if (key0 + kb < kend)  // keys past the tile's last query are never visible
        kreg[i] = load16(blk + kb * tok_stride + dc * 16);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = i * kWave + lane;
      const int kp = c / (D / 8), dc = c % (D / 8);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kb = 2 * kp + e;
        u32x4_t z = {0u, 0u, 0u, 0u};
        vreg[i][e] = z;
        if (key0 + kb < kend)
          vreg[i][e] = load16(blk + half_stride + kb * tok_stride + dc * 16);
      }
    }
  };
  auto stage = [&](int buf) {
    uint8_t* lk = lds_k[buf];
    uint8_t* lv = lds_v[buf];
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = i * kWave + lane;
      const int kb = c / CPR, dc = c % CPR;
      *reinterpret_cast<u32x4_t*>(lk + (16 * wave + kb) * S::KROW + dc * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = i * kWave + lane;
      const int kp = 8 * wave + c / (D / 8), dc = c % (D / 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims 8dc + 2w (lo) and 8dc + 2w + 1 (hi), keys 2kp and 2kp + 1
        const uint32_t lo = pair_lo(vreg[i][0][w], vreg[i][1][w]);
        const uint32_t hi = pair_hi(vreg[i][0][w], vreg[i][1][w]);
        *reinterpret_cast<uint32_t*>(lv + (8 * dc + 2 * w) * S::VROW + 4 * kp) = lo;
        *reinterpret_cast<uint32_t*>(lv + (8 * dc + 2 * w + 1) * S::VROW + 4 * kp) = hi;
      }
    }
  };

  f32x4_t acc[S::NMT];
#pragma unroll
  for (int mt = 0; mt < S::NMT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  // id_cur: block of iteration it + 1 (fetched during iteration it); id_nxt:
  // iteration it + 2 -- block-table reads run two iterations ahead.
  int id_cur = block_id(0), id_nxt;
  fetch(0, id_cur);
  stage(0);
  id_cur = block_id(1);
  id_nxt = block_id(2);
  __syncthreads();
  for (int it = 0; it < niter; ++it) {
    const int buf = it & 1;
    if (it + 1 < niter) fetch(it + 1, id_cur);
    const uint8_t* lds_kc = lds_k[buf];
    const uint8_t* lds_vc = lds_v[buf];

    // ---- S^T for 64 keys x 16 tokens: 4 tiles of 16 keys
    f32x4_t st[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      st[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S::NKS; ++s) {
        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(lds_kc + (16 * t + n) * S::KROW +
                                                              s * 64 + g * 16);
        st[t] = mfma16x16x32<E>(ka, qf[s], st[t]);
      }
    }
    // ---- scale to log2 units and apply the causal mask on diagonal tiles
    const int key0 = it * kKeysPerIter;
    float x[4][4];
    const bool diag = key0 + kKeysPerIter - 1 > nc + sub_start;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[t][i] = st[t][i] * a.scale_log2;
        if (diag) {
          const int key = key0 + 16 * t + 4 * g + i;
          x[t][i] = key <= pos ? x[t][i] : -INFINITY;
        }
      }
    float mx = x[0][0];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[t][i]);
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx);
    const bool grow = mn > m + 8.f;
    if (__any(grow)) {
      const float mu = grow ? mn : m;
      const float alpha = (mu == m) ? 1.f : __builtin_amdgcn_exp2f(m - mu);
      lsum *= alpha;
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt) acc[mt] *= alpha;
      m = mu;
    }
    const float ms = (m == -INFINITY) ? 0.f : m;
    float p[4][4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[t][i] = __builtin_amdgcn_exp2f(x[t][i] - ms);
        lsum += p[t][i];
      }
    // ---- O^T += V^T P^T, 32 keys per MFMA: lane group g holds keys
    // 32s2 + 4g + (0..3) and 32s2 + 16 + 4g + (0..3)
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4_t pb;
      pb[0] = pack2<E>(p[2 * s2][0], p[2 * s2][1]);
      pb[1] = pack2<E>(p[2 * s2][2], p[2 * s2][3]);
      pb[2] = pack2<E>(p[2 * s2 + 1][0], p[2 * s2 + 1][1]);
      pb[3] = pack2<E>(p[2 * s2 + 1][2], p[2 * s2 + 1][3]);
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt) {
        const uint8_t* vp = lds_vc + (16 * mt + n) * S::VROW + (32 * s2 + 4 * g) * 2;
        const uint2 lo = *reinterpret_cast<const uint2*>(vp);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 32);
        u32x4_t va = {lo.x, lo.y, hi.x, hi.y};
        acc[mt] = mfma16x16x32<E>(va, pb, acc[mt]);
      }
    }
    if (it + 1 < niter) {
      stage(buf ^ 1);
      id_cur = id_nxt;
      id_nxt = block_id(it + 3);
    }
    __syncthreads();
  }

  // ---- normalise and store: lane holds dims 16mt + 4g + (0..3) of token n
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  if (n < sub_valid) {
    const float inv = 1.f / lsum;
    uint8_t* op = static_cast<uint8_t*>(a.out) +
                  ((int64_t)(q0 + sub_start + n) * a.num_q_heads + hq) * S::ROWB + g * 8;
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt) {
      uint2 w;
      w.x = pack2<E>(acc[mt][0] * inv, acc[mt][1] * inv);
      w.y = pack2<E>(acc[mt][2] * inv, acc[mt][3] * inv);
      *reinterpret_cast<uint2*>(op + mt * 32) = w;
    }
  }
}

template <typename E, int D, int WPW>
hipError_t launch_typed(const PrefillArgs& a, hipStream_t stream) {
  const int group = a.num_q_heads / a.num_kv_heads;
  const dim3 grid((unsigned)a.max_tiles, (unsigned)(a.num_kv_heads * (group / WPW)));
  hipLaunchKernelGGL((prefill_tile_kernel<E, D, WPW>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
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
