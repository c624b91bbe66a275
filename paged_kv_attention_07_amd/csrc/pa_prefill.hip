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

// One work-group = 8 waves = 2 key halves x 4 waves; the 4 waves of a half
// are WPW query heads x (4 / WPW) token sub-tiles of 16.  The two halves
// split the tile's key range (iterations [0, n0) and [n0, n)), each with its
// own double-buffered LDS stages, and are merged through LDS at the end.
template <typename E, int D, int WPW>
__global__ __launch_bounds__(512) void prefill_tile_kernel(PrefillArgs a) {
  using S = TileShape<D>;
  constexpr int NQS = 4 / WPW;       // 16-token sub-tiles per work-group
  constexpr int QT = 16 * NQS;       // tokens per tile
  constexpr int KBUF = kKeysPerIter * S::KROW;
  constexpr int VBUF = D * S::VROW;
  // [half][stage]: the next 64 keys of each half are staged while the
  // current ones are used
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[2][2][KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[2][2][VBUF];
  __shared__ int s_tile[2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int half = wave >> 2;                // key half
  const int w4 = wave & 3;                   // wave within the half
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
  const int n0 = (niter + 1) / 2;            // iterations of half 0
  const int it_begin = half ? n0 : 0;
  const int my_iters = half ? niter - n0 : n0;  // n0 or n0 - 1 (or 0)

  const int hw = w4 % WPW;                   // head within the group
  const int sub = w4 / WPW;                  // 16-token sub-tile
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

  // id of the paged block this wavefront stages in (global) iteration it
  const int nb_need = (kend + kBlockSize - 1) / kBlockSize;
  auto block_id = [&](int it) {
    const int lb = it * 4 + w4;
    return lb < nb_need ? load_scalar(bt + lb) : 0;
  };

  // Staging: wavefront w4 of a half moves paged block w4 of the half's
  // iteration (keys 16 w4 .. 16 w4 + 15), so its block id is wave-uniform.
  // K rows go to LDS unchanged (lane l, step i: key (64 i + l) / CPR, 16-byte
  // column l % CPR).  V goes in transposed, two keys per 32-bit word: lane l,
  // step i handles key pair l % 8 and 8-dim column 8 i + l / 8, so the lanes
  // of one store write consecutive words.
  constexpr int CPR = S::ROWB / 16;          // 16-byte columns per row
  constexpr int KPT = 16 * CPR / kWave;      // K pieces per lane per block
  constexpr int VPT = (D / 8) / 8;           // V column groups per lane per block
  struct Regs {
    u32x4_t k[KPT], v[VPT][2];
  };
  // Loads are issued unconditionally (every address stays inside a real
  // block: ids past the table's end read block 0, rows past kend read their
  // own block) and keys past kend are zeroed when staged, so the compiler can
  // wait for exactly the loads a stage needs.
  // Per-lane byte offsets inside a block (32-bit): with the block base
  // wave-uniform, every load is scalar base + vector offset.
  uint32_t koff[KPT], voff[VPT][2];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int c = i * kWave + lane;
    koff[i] = (uint32_t)((c / CPR) * tok_stride + (c % CPR) * 16);
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i)
#pragma unroll
    for (int e = 0; e < 2; ++e)
      voff[i][e] = (uint32_t)(half_stride + (2 * (lane & 7) + e) * tok_stride +
                              (8 * i + (lane >> 3)) * 16);
  auto fetch = [&](Regs& R, int phys) {
    const uint8_t* blk = kvh + (int64_t)phys * blk_stride;
#pragma unroll
    for (int i = 0; i < KPT; ++i) R.k[i] = load16(blk + koff[i]);
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
      for (int e = 0; e < 2; ++e) R.v[i][e] = load16(blk + voff[i][e]);
  };
  // LDS offsets of this lane's staged pieces
  uint32_t kdst[KPT], vdst[VPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int c = i * kWave + lane;
    kdst[i] = (uint32_t)((16 * w4 + c / CPR) * S::KROW + (c % CPR) * 16);
  }
#pragma unroll
  for (int i = 0; i < VPT; ++i)
    vdst[i] = (uint32_t)((8 * (8 * i + (lane >> 3))) * S::VROW + 4 * (8 * w4 + (lane & 7)));
  auto stage = [&](Regs& R, int it, int buf) {
    uint8_t* lk = lds_k[half][buf];
    uint8_t* lv = lds_v[half][buf];
    const int key0 = it * kKeysPerIter + 16 * w4;
    if (key0 + 16 > kend) {
      // the block crosses the tile's last visible key: zero what lies past it
      const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        R.k[i] = key0 + (i * kWave + lane) / CPR < kend ? R.k[i] : z;
      const bool ok0 = key0 + 2 * (lane & 7) < kend, ok1 = key0 + 2 * (lane & 7) + 1 < kend;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        R.v[i][0] = ok0 ? R.v[i][0] : z;
        R.v[i][1] = ok1 ? R.v[i][1] : z;
      }
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) *reinterpret_cast<u32x4_t*>(lk + kdst[i]) = R.k[i];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // dims 8dc + 2w (lo) and 8dc + 2w + 1 (hi), keys 2kp and 2kp + 1
        *reinterpret_cast<uint32_t*>(lv + vdst[i] + (2 * w) * S::VROW) =
            pair_lo(R.v[i][0][w], R.v[i][1][w]);
        *reinterpret_cast<uint32_t*>(lv + vdst[i] + (2 * w + 1) * S::VROW) =
            pair_hi(R.v[i][0][w], R.v[i][1][w]);
      }
  };

  f32x4_t acc[S::NMT];
#pragma unroll
  for (int mt = 0; mt < S::NMT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;

  // One 64-key iteration from LDS stage `buf`: S^T, online softmax, O^T.
  auto compute = [&](int it, int buf) {
    const uint8_t* lds_kc = lds_k[half][buf];
    const uint8_t* lds_vc = lds_v[half][buf];
    // ---- S^T for 64 keys x 16 tokens: 4 tiles of 16 keys
    f32x4_t st[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      st[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < S::NKS; ++s) {
        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(
            lds_kc + (16 * tt + n) * S::KROW + s * 64 + g * 16);
        st[tt] = mfma16x16x32<E>(ka, qf[s], st[tt]);
      }
    }
    // ---- causal mask on diagonal tiles; scores stay unscaled (the scale,
    // with log2(e) folded in, is applied inside the exponent below)
    const int key0 = it * kKeysPerIter;
    float (&x)[4][4] = *reinterpret_cast<float (*)[4][4]>(&st[0]);
    if (key0 + kKeysPerIter - 1 > nc + sub_start) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = key0 + 16 * tt + 4 * g + i;
          x[tt][i] = key <= pos ? x[tt][i] : -INFINITY;
        }
    }
    float mx = x[0][0];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[tt][i]);
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    mx *= a.scale_log2;  // scale > 0: max of scaled = scaled max
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
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[tt][i] = __builtin_amdgcn_exp2f(fmaf(x[tt][i], a.scale_log2, -ms));
        lsum += p[tt][i];
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
  };

  // Both halves run n0 loop trips in lockstep (one barrier per trip); a half
  // with fewer iterations idles on its last trip.  Trip t computes iteration
  // it_begin + t from LDS stage t & 1, issues the loads of iteration
  // it_begin + t + 2 into register set t & 1, and stages iteration
  // it_begin + t + 1 from the other set (loaded one trip earlier).
  Regs R0, R1;
  fetch(R0, block_id(it_begin));
  if (my_iters > 0) stage(R0, it_begin, 0);
  fetch(R1, block_id(it_begin + 1));
  int id_ahead = block_id(it_begin + 2);
  __syncthreads();
  auto trip = [&](int t, Regs& Rload, Regs& Rstage) {
    const int buf = t & 1;
    const int it = it_begin + t;
    fetch(Rload, id_ahead);  // unconditional: past the range it reads block 0, never staged
    id_ahead = block_id(it + 3);
    if (t < my_iters) compute(it, buf);
    if (t + 1 < my_iters) stage(Rstage, it + 1, buf ^ 1);
    __syncthreads();
  };
  for (int t = 0; t < n0; t += 2) {
    trip(t, R0, R1);
    if (t + 1 < n0) trip(t + 1, R1, R0);
  }

  // ---- merge the halves: half 1 leaves (max, row sum, O^T) in LDS
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);
  constexpr int NF = S::NMT * 4 + 2;         // floats per lane
  static_assert(4 * kWave * NF * 4 <= 2 * KBUF, "merge buffer must fit in half 1's K stages");
  float* xch = reinterpret_cast<float*>(&lds_k[1][0][0]);  // half 1's stages, now free
  if (half == 1) {
    float* dst = xch + (w4 * kWave + lane) * NF;
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[4 * mt + i] = acc[mt][i];
    dst[NF - 2] = m;
    dst[NF - 1] = lsum;
  }
  __syncthreads();
  if (half == 1) return;
  {
    const float* src = xch + (w4 * kWave + lane) * NF;
    const float m1 = src[NF - 2], l1 = src[NF - 1];
    const float M = fmaxf(m, m1);            // m is finite: key 0 is visible
    const float a0 = __builtin_amdgcn_exp2f(m - M);
    const float a1 = (m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    lsum = lsum * a0 + l1 * a1;
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][i] = acc[mt][i] * a0 + src[4 * mt + i] * a1;
  }

  // ---- normalise and store: lane holds dims 16mt + 4g + (0..3) of token n
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
  hipLaunchKernelGGL((prefill_tile_kernel<E, D, WPW>), grid, dim3(512), 0, stream, a);
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
