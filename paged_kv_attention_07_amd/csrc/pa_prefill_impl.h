// Prefill-chunk attention over a paged KV cache on gfx950 (MFMA tiles):
// device code (kernel and the tile body that the fused launch reuses).
//
// What it computes ("vllm v1 源码精读（三）" §4.2; "Inside vLLM" §3.4): for a
// request with q_len > 1 new tokens on top of num_computed cached ones, token
// i (absolute position pos = num_computed + i) attends keys 0..pos of its own
// request -- the cached history plus the earlier tokens of the chunk (causal
// inside the chunk).  Keys are read through the request's block table.  The
// new tokens' K/V were either scattered into the cache beforehand, or come
// with the launch: then the chunk's keys are read from the new-token input
// and each tile stores its own tokens' rows into the cache.
//
// Tiling.  A work-group owns one tile of query tokens of one request and one
// group of query heads sharing a KV head.  Its waves form KSPLIT key parts of
// 4 waves; within a part, for GQA group 4, the 4 waves are the 4 query heads
// of the KV head over the same tokens, so each K/V tile staged in LDS feeds 4
// heads.  A wave covers NT sub-tiles of 16 tokens: with NT = 2 every K and V
// fragment read from LDS feeds two matrix-core products.  Keys are processed
// 64 at a time (four 16-token blocks looked up in the block table), copied
// from HBM straight into double-buffered LDS by the load unit (16 bytes per
// lane, no registers), one iteration ahead.  With KSPLIT = 2 the parts split
// the tile's key range and are merged through LDS at the end (more waves for
// chunks too short to fill the chip).
//
// Matrix-core mapping (v_mfma_f32_16x16x32_{bf16,f16}).  Scores are formed
// transposed, S^T = K Q^T (keys x tokens), because the accumulator layout of
// a 16x16 tile gives each lane 4 consecutive keys of ONE token: exactly the
// operand layout the second product O^T = V^T P^T needs for P^T, so the
// probabilities go from the softmax to the matrix core without moving across
// lanes.  Each lane then holds the output of one token, so the online-softmax
// rescale is a per-lane scalar.  K and V keep their cache layout in LDS
// (a 16-byte column swizzle per row keeps the reads free of bank
// conflicts); V^T fragments are read with the transposing LDS read
// (ds_read_b64_tr_b16: each lane gets 4 keys of one head dimension).  The
// contraction order inside an MFMA is a permutation of the keys; A and B
// use the same permutation.
#pragma once

#include <math.h>
#include <stdlib.h>

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
  static constexpr int ROWB = D * 2;                 // bytes of one token's head row
  static constexpr int CPR = ROWB / 16;              // 16-byte columns per row
  static constexpr int RPG = 256 / ROWB;             // rows per 256 bytes (64 banks)
  static constexpr int RPI = 1024 / ROWB;            // rows per 1 KiB wave copy
  static constexpr int NKS = D / 32;                 // MFMA k-steps of Q K^T
  static constexpr int NMT = D / 16;                 // 16-dim tiles of the output
  static constexpr int KBUF = kKeysPerIter * ROWB;
  static constexpr int STAGE = 2 * KBUF;             // one LDS stage: K rows then V rows
  // Physical 16-byte column of logical column c in LDS row `row`.  K is read
  // 16 rows x one column at a time (16 bytes per lane): fk spreads those 16
  // reads over all 64 banks.  V is read 8 rows x two adjacent columns at a
  // time (8 bytes per lane): fv spreads those 16 pieces over all banks.
  static __device__ __forceinline__ int fk(int row) { return (row / RPG) % CPR; }
  static __device__ __forceinline__ int fv(int row) { return 2 * ((row / RPG) % (CPR / 2)); }
};

// Zero row: the copy source for key rows past the tile's last key, so that
// those rows hold zeros (V must not carry a stale NaN into a product with a
// zero probability).
__device__ __attribute__((aligned(256))) uint8_t g_zero_row[256];

// Tokens per tile for a launch configuration.
template <int WPW, int NT>
constexpr int tile_tokens() {
  return 16 * NT * (4 / WPW);
}

// One work-group of tiles: tile slot bx (over requests' tiles), head group by.
// BESIDE_DECODE: the work-group shares the launch with decode work-groups
// (the fused mixed-step launch).
template <typename E, int D, int WPW, int NT, int KSPLIT, bool BESIDE_DECODE = false>
__device__ __forceinline__ void prefill_tile_body(const PrefillArgs& a, int bx, int by) {
  using S = TileShape<D>;
  constexpr int QT = tile_tokens<WPW, NT>();   // tokens per tile
  // Two stages per part: each part's next 64 keys are copied in while the
  // current ones are used.  Two stages keep a 4-wave work-group at 64 KiB of
  // LDS, so two work-groups share a CU and their barriers do not couple (a
  // third stage, or 8-wave groups sharing the stages, left one group per CU
  // and measured slower).  The stages are two separate LDS arrays, and every
  // trip names the one it reads and the one it fills at compile time (the
  // trip loop is unrolled by two): the compiler then knows a trip's reads
  // cannot touch the bytes its copies are filling and does not wait for
  // those copies before the reads (with one array indexed at run time it
  // waited, and every trip paid the full copy latency).
  __shared__ __attribute__((aligned(16))) uint8_t lds0[KSPLIT][S::STAGE];  // even trips
  __shared__ __attribute__((aligned(16))) uint8_t lds1[KSPLIT][S::STAGE];  // odd trips
  __shared__ int s_tile[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uniform(tid >> 6);
  const int part = wave >> 2;                  // key part
  const int w4 = wave & 3;                     // wave within the part
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hg = group / WPW;
  const int h = by / hg;
  const int hs = by - h * hg;

  // ---- which request / tile this work-group owns (a shared-prefix pass has
  // one virtual request: tile = work-group index)
  // Beside decode rows the work-group also notes whether the batch has any
  // (a request with one query token): then its copies are waited for before
  // each trip's reads rather than overlapped with them, leaving the memory
  // system to the decode reads that bound such a launch (overlapping them
  // made the mixed step ~1% slower; a batch of chunks alone gains 10%).
  const bool cascade = a.cascade_rows > 0;
  if (cascade) {
    if (lane == 0 && wave == 0) {
      const bool live = bx * QT < a.cascade_rows;
      s_tile[0] = live ? 0 : -1;
      s_tile[1] = bx;
      s_tile[2] = 1;                           // the shared-prefix pass runs beside decode
    }
  } else if (wave == 0) {
    int found_r = -1, found_t = 0, running = 0;
    bool decode_rows = false;
    const int want = bx;
    for (int base = 0; base < a.num_seqs && (BESIDE_DECODE || found_r < 0); base += kWave) {
      const int r = base + lane;
      int nt = 0, ql = 0;
      if (r < a.num_seqs) {
        ql = a.qsl[r + 1] - a.qsl[r];
        nt = ql > 1 ? (ql + QT - 1) / QT : 0;
      }
      decode_rows = decode_rows || __ballot(ql == 1) != 0;
      const int incl = wave_incl_scan(nt) + running;
      const int excl = incl - nt;
      const uint64_t hit = __ballot(nt > 0 && want >= excl && want < incl);
      if (hit && found_r < 0) {
        const int src = __builtin_ctzll(hit);
        found_r = base + src;
        // a request's tiles are handed out last-first: the tiles with the
        // most keys start early and the short ones fill in behind them
        found_t = readlane(incl, src) - 1 - want;
      }
      running = readlane(incl, kWave - 1);
    }
    if (lane == 0) {
      s_tile[0] = found_r;
      s_tile[1] = found_t;
      s_tile[2] = BESIDE_DECODE && decode_rows;
    }
  }
  __syncthreads();
  const int r = uniform(s_tile[0]);
  if (r < 0) return;
  const int tile = uniform(s_tile[1]);
  const bool wait_copies = uniform(s_tile[2]) != 0;

  // a shared-prefix pass: rows 0 .. cascade_rows - 1 all placed after the
  // cascade_keys prefix keys, so every prefix key is visible to every row
  const int q0 = cascade ? 0 : a.qsl[r];
  const int qlen = cascade ? a.cascade_rows : a.qsl[r + 1] - q0;
  const int nc = cascade ? a.cascade_keys : a.num_computed[r];
  const int L = cascade ? a.cascade_keys : a.seq_lens[r];
  const int tile_start = tile * QT;
  const int tile_valid = min(QT, qlen - tile_start);
  const int kend = min(L, nc + tile_start + tile_valid);  // keys this tile needs
  const int niter = (kend + kKeysPerIter - 1) / kKeysPerIter;
  const int n0 = (niter + KSPLIT - 1) / KSPLIT;           // trips of every part
  const int it_begin = part * n0;
  const int my_iters = max(0, min(n0, niter - it_begin));

  const int hw = w4 % WPW;                     // head within the group
  const int sub = w4 / WPW;                    // token group of this wave
  const int hq = h * group + hs * WPW + hw;
  const int n = lane & 15;                     // token column of this lane
  const int g = lane >> 4;                     // lane group

  // NT sub-tiles of 16 tokens: sub-tile j starts at token sub_start[j]
  int sub_start[NT], sub_valid[NT], pos[NT];
  u32x4_t qf[NT][S::NKS];                      // Q^T fragments: token n, dims 32s + 8g .. +8
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    sub_start[j] = tile_start + (sub * NT + j) * 16;
    sub_valid[j] = max(0, min(16, qlen - sub_start[j]));
    // last visible key; at most the tile's last key (a shared-prefix pass
    // places its rows after the keys it may see)
    pos[j] = min(nc + sub_start[j] + min(n, max(sub_valid[j] - 1, 0)), kend - 1);
    const bool ok = n < sub_valid[j];
    const uint8_t* qp = static_cast<const uint8_t*>(a.q) +
                        ((int64_t)(q0 + sub_start[j] + n) * a.num_q_heads + hq) * S::ROWB +
                        g * 16;
#pragma unroll
    for (int s = 0; s < S::NKS; ++s) {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      qf[j][s] = ok ? load16(qp + s * 64) : z;
    }
  }

  const int64_t tok_stride = (int64_t)a.num_kv_heads * S::ROWB;
  const int64_t half_stride = kBlockSize * tok_stride;
  const int64_t blk_stride = 2 * half_stride;
  const uint8_t* kvh = static_cast<const uint8_t*>(a.kv) + (int64_t)h * S::ROWB;
  const int32_t* bt = a.block_table + (int64_t)r * a.bt_stride;

  // Ids of the paged blocks this wavefront stages: one vector load per 64 of
  // its trips (lane l holds the id for trip t0 + l, i.e. iteration
  // it_begin + t0 + l), picked per trip with a lane read.  A scalar load per
  // trip would put its latency before every barrier: scalar loads share the
  // counter that the barrier's LDS wait drains.
  const int nb_need = (kend + kBlockSize - 1) / kBlockSize;
  auto load_ids = [&](int t0) {
    const int lb = (it_begin + t0 + lane) * 4 + w4;
    return (t0 + lane < my_iters && lb < nb_need) ? bt[lb] : 0;
  };

  // Staging: wavefront w4 of a part copies paged block w4 of the part's
  // iteration (keys 16 w4 .. 16 w4 + 15), so its block id is wave-uniform.
  // Each 1 KiB copy moves RPI rows: lane l lands at LDS byte 16 l of the
  // copy, so it fetches row l / CPR at the global column that the row's
  // swizzle puts in slot l % CPR.
  constexpr int CPB = 16 * S::ROWB / 1024;     // copies per block half
  uint32_t goff[2][CPB];                       // per-lane byte offset inside a block
  uint32_t zoff[2][CPB];                       // the same column in the zero row
#pragma unroll
  for (int hv = 0; hv < 2; ++hv)
#pragma unroll
    for (int i = 0; i < CPB; ++i) {
      const int rib = S::RPI * i + lane / S::CPR;       // row in block
      const int row = 16 * w4 + rib;                    // row in stage
      const int col = (lane % S::CPR) ^ (hv ? S::fv(row) : S::fk(row));
      goff[hv][i] = (uint32_t)(hv * half_stride + rib * tok_stride + col * 16);
      zoff[hv][i] = (uint32_t)(col * 16);
    }
  // Keys at positions >= nfresh are this step's new tokens when the launch
  // also stores them: their cache rows are being written in this launch, so
  // they are copied from the new-token input (row q0 + key - nc) instead.
  // The new-token rows are laid out like the cache's token rows (stride
  // tok_stride, head h at h * ROWB), so row key of a block comes from
  // fresh base + (key - nc) * tok_stride + the same in-block offset goff.
  const bool fresh = a.fresh.k != nullptr && !cascade;
  const int nfresh = fresh ? nc : 0x7fffffff;
  const uint8_t* fbase[2] = {
      static_cast<const uint8_t*>(a.fresh.k) + (int64_t)q0 * tok_stride + (int64_t)h * S::ROWB,
      static_cast<const uint8_t*>(a.fresh.v) + (int64_t)q0 * tok_stride + (int64_t)h * S::ROWB -
          half_stride};
  // the wave's 16 rows of an iteration start at key0: all cached, all new,
  // or (at most twice per tile) mixed / past the tile's last key, which is
  // the only case that selects a source per lane
  auto dma = [&](int it, int phys, uint8_t* stage) {
    const uint8_t* blk = kvh + (int64_t)phys * blk_stride;
    const int key0 = it * kKeysPerIter + 16 * w4;
    const uint8_t* fblk[2] = {fbase[0] + (int64_t)(key0 - nc) * tok_stride,
                              fbase[1] + (int64_t)(key0 - nc) * tok_stride};
    const bool cached = key0 + 15 < min(kend, nfresh);
    const bool all_new = key0 >= nfresh && key0 + 15 < kend;
    if (cached || all_new) {
      // the common cases, with one branch for all copies: a wave-uniform
      // base (the cache block, or the new-token rows) plus a 32-bit
      // per-lane offset
      const uint8_t* base[2] = {cached ? blk : fblk[0], cached ? blk : fblk[1]};
#pragma unroll
      for (int hv = 0; hv < 2; ++hv)
#pragma unroll
        for (int i = 0; i < CPB; ++i)
          __builtin_amdgcn_global_load_lds(base[hv] + goff[hv][i],
                                           stage + hv * S::KBUF + (16 * w4 + S::RPI * i) * S::ROWB,
                                           16, 0, 0);
      return;
    }
#pragma unroll
    for (int hv = 0; hv < 2; ++hv) {
#pragma unroll
      for (int i = 0; i < CPB; ++i) {
        const int rib = S::RPI * i + lane / S::CPR;
        const int key = key0 + rib;
        const uint8_t* src = key >= kend     ? g_zero_row + zoff[hv][i]
                             : key >= nfresh ? fblk[hv] + goff[hv][i]
                                             : blk + goff[hv][i];
        uint8_t* dst = stage + hv * S::KBUF + (16 * w4 + S::RPI * i) * S::ROWB;
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      }
    }
  };

  // Running max m of each token's raw scores <q, k>.  The score product
  // starts its accumulator at -m (negm holds -m in all four elements), so the
  // scores come out as s - m; the exponent is (s - m) * scale * log2(e),
  // formed in fp32 (Q stays as given: a Q pre-multiplied by the scale and
  // rounded to 16 bits would err in proportion to the score's size).  m is
  // set exactly from the part's first trip (every token that sees any key
  // of the part sees its first one) and afterwards moves only when a score
  // passes it by more than 8 / (scale * log2(e)) (lazy rescale:
  // probabilities stay below 2^8 and the largest so far at least 1).  A
  // token that sees no key of the part keeps m = 0 and zero sums.  The
  // scale is positive (checked by the caller).
  f32x4_t acc[NT][S::NMT];
  f32x4_t negm[NT];
  float lsum[NT];
  const float c = a.scale_log2;
  const float thr = 8.f / c;                   // a lazy-rescale step in raw score units
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    negm[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    lsum[j] = 0.f;
#pragma unroll
    for (int mt = 0; mt < S::NMT; ++mt) acc[j][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // One 64-key iteration from LDS stage `stage`: S^T, online softmax, O^T.
  auto compute = [&](int it, const uint8_t* stage) {
    // LLVM's single-wave MFMA interleaving strategy for this scheduling
    // region: measured ~2% faster on long prompts than the default schedule
    // (the small-GEMM strategy is equal, the exp-interleaving ones slower)
    __builtin_amdgcn_iglp_opt(1);
    const uint8_t* lds_kc = stage;
    const uint8_t* lds_vc = stage + S::KBUF;
    // ---- S^T for 64 keys x 16 tokens per sub-tile: 4 tiles of 16 keys
    f32x4_t st[NT][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int j = 0; j < NT; ++j) st[j][tt] = negm[j];
#pragma unroll
      for (int s = 0; s < S::NKS; ++s) {
        const int row = 16 * tt + n;
        const u32x4_t ka = *reinterpret_cast<const u32x4_t*>(
            lds_kc + row * S::ROWB + (((4 * s + g) ^ S::fk(row)) << 4));
#pragma unroll
        for (int j = 0; j < NT; ++j) st[j][tt] = mfma16x16x32<E>(ka, qf[j][s], st[j][tt]);
      }
    }
    const int key0 = it * kKeysPerIter;
    const bool first = it == it_begin;         // the part's first trip
    u32x4_t pb[NT][2];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      // ---- causal mask on diagonal tiles (x: the raw score less m)
      float (&x)[4][4] = *reinterpret_cast<float (*)[4][4]>(&st[j][0]);
      if (key0 + kKeysPerIter - 1 > min(nc + sub_start[j], kend - 1)) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = key0 + 16 * tt + 4 * g + i;
            x[tt][i] = key <= pos[j] ? x[tt][i] : -INFINITY;
          }
      }
      float mx = x[0][0];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, x[tt][i]);
      // A token's 64 scores of the trip sit in lanes l, l ^ 16, l ^ 32, l ^ 48
      // (16 each).  m has to move when the token's max passes it by more
      // than thr, which happens iff one of the four lanes' own max does: so
      // the lanes test their own max, and the max over the four lanes is
      // formed only in the (rare) trips where some lane of the wavefront
      // passes, and in the part's first trip, which sets m (the branch is
      // wavefront-uniform, so every lane takes part in the exchange).
      if (first || __any(mx > thr)) {
        const float cmx = max_over_rows(mx);    // the same in the token's four lanes
        const float d = first ? (cmx == -INFINITY ? 0.f : cmx) : (cmx > thr ? cmx : 0.f);
        if (!first) {                           // first trip: sums and outputs are still 0
          const float alpha = __builtin_amdgcn_exp2f(-d * c);
          lsum[j] *= alpha;
#pragma unroll
          for (int mt = 0; mt < S::NMT; ++mt) acc[j][mt] *= alpha;
        }
        negm[j] -= d;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[tt][i] -= d;
      }
      float p[4][4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[tt][i] = __builtin_amdgcn_exp2f(x[tt][i] * c);
          lsum[j] += p[tt][i];
        }
      // lane group g holds keys 32s2 + 4g + (0..3) and 32s2 + 16 + 4g + (0..3)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        pb[j][s2][0] = pack2<E>(p[2 * s2][0], p[2 * s2][1]);
        pb[j][s2][1] = pack2<E>(p[2 * s2][2], p[2 * s2][3]);
        pb[j][s2][2] = pack2<E>(p[2 * s2 + 1][0], p[2 * s2 + 1][1]);
        pb[j][s2][3] = pack2<E>(p[2 * s2 + 1][2], p[2 * s2 + 1][3]);
      }
    }
    // ---- O^T += V^T P^T, 32 keys per MFMA
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt) {
        // lane (n, g): dim 16 mt + n, keys 32 s2 + 4 g + (0..3) and
        // 32 s2 + 16 + 4 g + (0..3); the transposing read hands lane
        // 4 q + c of each 16-lane group element c of the 8 bytes that lane
        // 4 i + q points at, for i = 0..3 (i = key, q = dim quad)
        const int e = 4 * mt + (n & 3);                  // 8-byte piece (4 dims)
        u32x4_t va;
#pragma unroll
        for (int hv = 0; hv < 2; ++hv) {
          const int row = 32 * s2 + 16 * hv + 4 * g + (n >> 2);
          const uint8_t* vp = lds_vc + row * S::ROWB + ((((e >> 1) ^ S::fv(row)) << 4) | ((e & 1) << 3));
          typedef short v4s_t __attribute__((ext_vector_type(4)));
          const v4s_t t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) v4s_t*)(vp));
          const uint2 w = __builtin_bit_cast(uint2, t);
          va[2 * hv] = w.x;
          va[2 * hv + 1] = w.y;
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j][mt] = mfma16x16x32<E>(va, pb[j][s2], acc[j][mt]);
      }
  };

  // Every part runs n0 loop trips in lockstep, one barrier per trip; a part
  // with fewer iterations idles on its last trips.  Trip t waits for its own
  // copies of iteration it_begin + t (the only loads in flight), meets the
  // other waves at the barrier (after which every copy of that iteration has
  // landed and every wave is done with the other stage), starts the copies
  // of the next iteration into the other stage, and computes.
  int ids = load_ids(0);                       // trips 0 .. 63
  int ids_ahead = my_iters > 64 ? load_ids(64) : 0;  // trips 64 .. 127
  uint8_t* const st0 = lds0[part];
  uint8_t* const st1 = lds1[part];
  if (my_iters > 0) dma(it_begin, readlane(ids, 0), st0);

  auto trip = [&](int t, const uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
    const int tn = t + 1;                      // trip whose copies start now
    const bool wrap = (tn & 63) == 0 && tn < my_iters;
    if (wrap) ids = ids_ahead;                 // next window of ids
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tn < my_iters) dma(it_begin + tn, readlane(ids, tn & 63), nxt);
    // the window after it, loaded beside this trip's copies
    if (wrap) ids_ahead = tn + 64 < my_iters ? load_ids(tn + 64) : 0;
    if (wait_copies) __builtin_amdgcn_s_waitcnt(0);
    if (t < my_iters) compute(it_begin + t, cur);
  };
  for (int t = 0; t < n0; t += 2) {
    trip(t, st0, st1);
    if (t + 1 < n0) trip(t + 1, st1, st0);
  }
  // ---- store the tile's new tokens into the cache: one work-group per KV
  // head (the first query-head group) writes the K and V rows of tokens
  // tile_start .. tile_start + tile_valid - 1 (step rows q0 + ...), which no
  // work-group of this launch reads from the cache.  It runs after the key
  // loop (whose waits would otherwise also wait for these stores), all loads
  // issued before any store.
  if (fresh && hs == 0) {
    constexpr int NL = S::ROWB / 16;           // 16-byte pieces per row
    constexpr int NTH = 256 * KSPLIT;
    constexpr int PER = (QT * 2 * NL + NTH - 1) / NTH;
    u32x4_t val[PER];
    int64_t id[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int x = tid + k * NTH;
      const int i = x / (2 * NL);
      if (x < tile_valid * 2 * NL) {
        const int hv = (x / NL) & 1;
        const int64_t piece = (int64_t)h * S::ROWB + (x % NL) * 16;
        id[k] = bt[(nc + tile_start + i) / kBlockSize];
        val[k] = load16(static_cast<const uint8_t*>(hv ? a.fresh.v : a.fresh.k) +
                        (int64_t)(q0 + tile_start + i) * tok_stride + piece);
      }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int x = tid + k * NTH;
      if (x < tile_valid * 2 * NL) {
        const int i = x / (2 * NL);
        const int hv = (x / NL) & 1;
        const int col = x % NL;
        const int p = nc + tile_start + i;     // position in the request
        const int64_t piece = (int64_t)h * S::ROWB + col * 16;
        store16(static_cast<uint8_t*>(a.fresh.kv) + id[k] * blk_stride + hv * half_stride +
                    (int64_t)(p % kBlockSize) * tok_stride + piece,
                val[k]);
        if (h == 0 && hv == 0 && col == 0 && a.fresh.slot_out)
          a.fresh.slot_out[q0 + tile_start + i] = id[k] * kBlockSize + p % kBlockSize;
      }
    }
  }
  if constexpr (KSPLIT == 2) __syncthreads();  // stages are reused for the merge

  float m[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    lsum[j] = sum_over_rows(lsum[j]);
    m[j] = -negm[j][0] * c;                    // in log2 units, as the partials carry it
  }
  if constexpr (KSPLIT == 2) {
    // ---- merge the parts: part 1 leaves (max, row sum, O^T) in its LDS stages
    // the accumulators go to part 1's first stage, (max, sum) to its second
    constexpr int NA = NT * S::NMT * 4;        // accumulator floats per lane
    static_assert(4 * kWave * NA * 4 <= S::STAGE, "merge buffer must fit in part 1's stage");
    float* xa = reinterpret_cast<float*>(lds0[1]) + (w4 * kWave + lane) * NA;
    float* xm = reinterpret_cast<float*>(lds1[1]) + (w4 * kWave + lane) * 2 * NT;
    if (part == 1) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xa[j * S::NMT * 4 + 4 * mt + i] = acc[j][mt][i];
        xm[2 * j] = m[j];
        xm[2 * j + 1] = lsum[j];
      }
    }
    __syncthreads();
    if (part == 1) return;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const float* src = xa + j * S::NMT * 4;
      // part 0 holds key 0, which every token sees; part 1 may hold none of
      // a token's keys (then its sum is 0 and its m a placeholder)
      const float m1 = xm[2 * j], l1 = xm[2 * j + 1];
      const bool has1 = l1 > 0.f;
      const float M = has1 ? fmaxf(m[j], m1) : m[j];
      const float a0 = __builtin_amdgcn_exp2f(m[j] - M);
      const float a1 = has1 ? __builtin_amdgcn_exp2f(m1 - M) : 0.f;
      lsum[j] = lsum[j] * a0 + l1 * a1;
      m[j] = M;
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][mt][i] = acc[j][mt][i] * a0 + src[4 * mt + i] * a1;
    }
  }

  // ---- normalise and store: lane holds dims 16mt + 4g + (0..3) of token n
  if (cascade) {
    // partial (max, sum, unnormalised output) of row q0 + token, fp32
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (n < sub_valid[j]) {
        const int64_t ps = ((int64_t)a.prefix_slot0 + sub_start[j] + n) * a.num_q_heads + hq;
        float* po = a.ws_o + ps * D + 4 * g;
#pragma unroll
        for (int mt = 0; mt < S::NMT; ++mt)
          *reinterpret_cast<f32x4_t*>(po + 16 * mt) = acc[j][mt];
        if (g == 0) {
          const f32x2_t ml = {m[j], lsum[j]};
          *reinterpret_cast<f32x2_t*>(a.ws_ml + ps * 2) = ml;
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (n < sub_valid[j]) {
      const float inv = 1.f / lsum[j];
      uint8_t* op = static_cast<uint8_t*>(a.out) +
                    ((int64_t)(q0 + sub_start[j] + n) * a.num_q_heads + hq) * S::ROWB + g * 8;
#pragma unroll
      for (int mt = 0; mt < S::NMT; ++mt) {
        uint2 w;
        w.x = pack2<E>(acc[j][mt][0] * inv, acc[j][mt][1] * inv);
        w.y = pack2<E>(acc[j][mt][2] * inv, acc[j][mt][3] * inv);
        *reinterpret_cast<uint2*>(op + mt * 32) = w;
      }
    }
  }
}

template <typename E, int D, int WPW, int NT, int KSPLIT>
__global__ __launch_bounds__(256 * KSPLIT) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_tile_kernel(PrefillArgs a) {
  // XCD-aware numbering.  Work-groups are handed to the device's XCDs in
  // turn (linear index x fastest); renumber them so that each XCD runs one
  // contiguous block of (head group, tile) pairs, head-major: the tiles of a
  // KV head then share one XCD's L2, where the keys they all re-read stay.
  const int tiles = gridDim.x;
  const int total = tiles * gridDim.y;
  const int lin = blockIdx.y * tiles + blockIdx.x;
  const int nx = a.num_xcds;
  const int xcd = lin % nx, local = lin / nx;
  const int full = total / nx, rem = total % nx;
  // Pairing.  A die's dispatcher hands its work-groups to its C compute units
  // in turn; with D = 128 and one key part two fit on a CU (LDS and
  // registers), so local k and local k + C run side by side.  The die's
  // block is heaviest-first, and taken in order CU k would hold the k-th
  // and the (k + C)-th heaviest: the first CUs get the two heaviest loads
  // and the last the two lightest.  Taking the second C in reverse gives
  // CU k the k-th heaviest beside the k-th lightest of the first 2C, and the
  // CUs' loads even out (the 2048-token chunk's slowest CU finishes ~9%
  // sooner).  Only where the die's block fits that one round of two slots
  // per CU (the grid holds up to one empty slot per request beyond the
  // tiles): with more work-groups the later ones go wherever a slot frees,
  // heaviest first, and the first round's order measured no better reversed.
  int slot = local;
  if (D == 128 && KSPLIT == 1) {
    const int C = a.cus_per_xcd;
    const int here = full + (xcd < rem ? 1 : 0);      // this die's work-groups
    if (here <= 2 * C + a.num_seqs && local >= C && local < 2 * C)
      slot = C + min(2 * C, here) - 1 - local;
  }
  const int idx = xcd * full + min(xcd, rem) + slot;  // a bijection of [0, total)
  prefill_tile_body<E, D, WPW, NT, KSPLIT>(a, idx % tiles, idx / tiles);
}

}  // namespace
}  // namespace pa
