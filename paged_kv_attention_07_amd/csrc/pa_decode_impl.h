// Decode attention over a paged KV cache on gfx950, with a balanced
// split-KV partition-and-reduce: device code (kernels and the split body
// that the fused launch reuses).
//
// What it computes ("vLLM 架构源码解析（一）" §3.3.3 and §4.2;
// "Inside vLLM" §3.3): for each request with one new query token, softmax
// attention of that token over its seq_len cached keys, read through the
// request's block table.  Partial results over key ranges are merged with
// the online-softmax identity (max, sum, unnormalised output), the
// "Online Softmax" the first page names in §6.4.
//
// Work decomposition.  The blocks of all decode requests are laid end to end
// (request 0's blocks, then request 1's, ...) and the list is cut into
// `num_chunks` equal ranges.  One wavefront takes one range for one KV head
// (and up to four query heads of its group), so every wavefront streams the
// same number of bytes whatever the length mix; a range that covers a whole
// request finishes it in place, a request cut by range boundaries leaves one
// partial per range, and a small merge kernel combines them.  Partials of
// (request r, range c) go to workspace slot r + c, which is unique because
// both indices only grow along the list.
//
// Inside a wavefront (64 lanes).  Lane = (token group tg = lane / 8, column
// ds = lane % 8).  For each 16-token block the lane loads tokens tg and tg+8;
// the 8 lanes of a group read 128 contiguous bytes of a token's head row per
// instruction (16 bytes each), so every load instruction touches 8 full
// 128-byte lines.  Scores are 8-lane DPP sums of per-lane dot products
// (bf16/f16: v_dot2 pairs, no conversion); each token group keeps its own
// running max / sum / accumulator (no cross-group traffic in the loop), with
// the accumulator rescaled only when the max grows by more than 2^8.  P*V
// pairs the group's two tokens in one v_dot2 per output element.  At the end
// of a range the 8 groups are merged and reduce-scattered so each lane owns
// a few contiguous output elements.
#pragma once

#include <math.h>

#include "pa_common.h"
#include "pa_kernels.h"

namespace pa {
namespace {

template <typename E, int D, int HPW>
struct Shape {
  static constexpr int ESZ = E::bytes;
  static constexpr int EPV = 16 / ESZ;    // elements per 16-byte vector
  static constexpr int ROWB = D * ESZ;    // bytes of one token's row for one kv head
  static constexpr int NCH = ROWB / 128;  // 16-byte vectors per lane per token
  static constexpr int DPL = NCH * EPV;   // head dims owned by a lane
  static constexpr int NV = HPW * DPL;    // accumulator floats per lane
  static constexpr int NOUT = NV / 8;     // outputs per lane after the group merge
  static constexpr int RUN = NOUT < EPV ? NOUT : EPV;  // contiguous dims per store
  static_assert(NCH >= 1 && NOUT >= 1, "unsupported decode shape");
};

// head dim of lane-local element e for column ds
template <class S>
__device__ __forceinline__ int dim_of(int e, int ds) {
  return (e / S::EPV) * (8 * S::EPV) + ds * S::EPV + (e % S::EPV);
}

struct ReqInfo {
  int nb;   // blocks this request contributes to the decode list (0 = not a decode row)
  int row;  // query/output row
  int len;  // keys
};

__device__ __forceinline__ ReqInfo req_info(const DecodeArgs& a, int r) {
  ReqInfo ri{0, 0, 0};
  if (r < a.num_seqs) {
    const int L = a.seq_lens[r];
    bool active = L > 0;
    int row = r;
    if (a.qsl) {
      const int q0 = a.qsl[r], q1 = a.qsl[r + 1];
      active = active && (q1 - q0 == 1);
      row = q0;
    }
    // blocks past a shared prefix (attended by the prefix pass)
    ri.nb = active ? max(0, (L + kBlockSize - 1) / kBlockSize - a.skip_blocks) : 0;
    ri.row = row;
    ri.len = L;
  }
  return ri;
}

__device__ __forceinline__ int total_blocks(const DecodeArgs& a) {
  int W = 0;
  for (int base = 0; base < a.num_seqs; base += kWave)
    W += uniform(wave_sum(req_info(a, base + lane_id()).nb));
  return W;
}

__device__ __forceinline__ int64_t chunk_begin(int c, int W, int N) {
  return (int64_t)c * W / N;
}

// the range holding flat block x (ranges may be empty when W < N)
__device__ __forceinline__ int chunk_of(int64_t x, int W, int N) {
  return (int)(((x + 1) * N + W - 1) / W) - 1;
}

template <typename E>
__device__ __forceinline__ float to_f(uint32_t w, int half);

template <>
__device__ __forceinline__ float to_f<BF16>(uint32_t w, int half) {
  return half ? bf16_hi(w) : bf16_lo(w);
}
template <>
__device__ __forceinline__ float to_f<F16>(uint32_t w, int half) {
  return half ? f16_hi(w) : f16_lo(w);
}

// Store RUN consecutive values (times `mul`) as element type E.
template <typename E, int RUN>
__device__ __forceinline__ void store_run(void* dst, const float* v, float mul) {
  if constexpr (E::kind == F32::kind) {
    float* p = static_cast<float*>(dst);
    if constexpr (RUN % 4 == 0) {
#pragma unroll
      for (int i = 0; i < RUN; i += 4) {
        f32x4_t x = {v[i] * mul, v[i + 1] * mul, v[i + 2] * mul, v[i + 3] * mul};
        *reinterpret_cast<f32x4_t*>(p + i) = x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RUN; ++i) p[i] = v[i] * mul;
    }
  } else {
    if constexpr (RUN % 2 == 0) {
      uint32_t w[RUN / 2];
#pragma unroll
      for (int i = 0; i < RUN / 2; ++i) {
        w[i] = (E::kind == BF16::kind) ? pack_bf16(v[2 * i] * mul, v[2 * i + 1] * mul)
                                       : pack_f16(v[2 * i] * mul, v[2 * i + 1] * mul);
      }
      uint32_t* p = static_cast<uint32_t*>(dst);
      if constexpr (RUN == 8) {
        u32x4_t x = {w[0], w[1], w[2], w[3]};
        store16(p, x);
      } else {
#pragma unroll
        for (int i = 0; i < RUN / 2; ++i) p[i] = w[i];
      }
    } else {
      const uint32_t w = (E::kind == BF16::kind) ? pack_bf16(v[0] * mul, 0.f)
                                                 : pack_f16(v[0] * mul, 0.f);
      *static_cast<uint16_t*>(dst) = (uint16_t)(w & 0xffffu);
    }
  }
}

template <int RUN>
__device__ __forceinline__ void store_f32_run(float* p, const float* v) {
  if constexpr (RUN % 4 == 0) {
#pragma unroll
    for (int i = 0; i < RUN; i += 4) {
      f32x4_t x = {v[i], v[i + 1], v[i + 2], v[i + 3]};
      *reinterpret_cast<f32x4_t*>(p + i) = x;
    }
  } else {
#pragma unroll
    for (int i = 0; i < RUN; ++i) p[i] = v[i];
  }
}

template <typename E, int D, int HPW>
struct BlockRegs {
  using S = Shape<E, D, HPW>;
  u32x4_t k0[S::NCH], k1[S::NCH], v0[S::NCH], v1[S::NCH];
};

// Load the lane's K and V pieces of tokens tg and tg + 8 from four row
// addresses (K of token tg, K of token tg + 8, V of tg, V of tg + 8).
template <typename E, int D, int HPW>
__device__ __forceinline__ void load_rows(BlockRegs<E, D, HPW>& b, const uint8_t* k0,
                                          const uint8_t* k1, const uint8_t* v0,
                                          const uint8_t* v1) {
  using S = Shape<E, D, HPW>;
#pragma unroll
  for (int c = 0; c < S::NCH; ++c) {
    b.k0[c] = load16_stream(k0 + c * 128);
    b.k1[c] = load16_stream(k1 + c * 128);
  }
#pragma unroll
  for (int c = 0; c < S::NCH; ++c) {
    b.v0[c] = load16_stream(v0 + c * 128);
    b.v1[c] = load16_stream(v1 + c * 128);
  }
}

template <typename E, int D, int HPW>
__device__ __forceinline__ void load_block(BlockRegs<E, D, HPW>& b, const uint8_t* p,
                                           int64_t tok8, int64_t half) {
  load_rows<E, D, HPW>(b, p, p + tok8, p + half, p + half + tok8);
}

// One 16-token block of one request: scores of tokens tg and tg+8 of the
// block for the wave's query heads, running-max update, and P*V.
template <typename E, int D, int HPW>
__device__ __forceinline__ void attend_block(BlockRegs<E, D, HPW>& b, int j, int nb, int L,
                                             int tg, float scale_log2,
                                             const u32x4_t (&qv)[HPW][Shape<E, D, HPW>::NCH],
                                             float (&m)[HPW], float (&l)[HPW],
                                             float (&acc)[HPW][Shape<E, D, HPW>::DPL]) {
  using S = Shape<E, D, HPW>;
  // ---- scores of tokens tg and tg+8 for each head (log2 units)
  float s0[HPW], s1[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int c = 0; c < S::NCH; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (E::kind == F32::kind) {
          const float qf = __uint_as_float(qv[hh][c][w]);
          a0 = fmaf(__uint_as_float(b.k0[c][w]), qf, a0);
          a1 = fmaf(__uint_as_float(b.k1[c][w]), qf, a1);
        } else if constexpr (E::kind == BF16::kind) {
          a0 = dot2_bf16(b.k0[c][w], qv[hh][c][w], a0);
          a1 = dot2_bf16(b.k1[c][w], qv[hh][c][w], a1);
        } else {
          a0 = dot2_f16(b.k0[c][w], qv[hh][c][w], a0);
          a1 = dot2_f16(b.k1[c][w], qv[hh][c][w], a1);
        }
      }
    s0[hh] = sum8(a0) * scale_log2;
    s1[hh] = sum8(a1) * scale_log2;
  }
  // ---- partial last block: drop scores and values past the sequence end
  if (j == nb - 1 && (L & (kBlockSize - 1))) {
    const int nvalid = L - j * kBlockSize;
    const bool ok0 = tg < nvalid, ok1 = tg + 8 < nvalid;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      s0[hh] = ok0 ? s0[hh] : -INFINITY;
      s1[hh] = ok1 ? s1[hh] : -INFINITY;
    }
#pragma unroll
    for (int c = 0; c < S::NCH; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        b.v0[c][w] = ok0 ? b.v0[c][w] : 0u;
        b.v1[c][w] = ok1 ? b.v1[c][w] : 0u;
      }
  }
  // ---- running max; rescale only when it grows by more than 8 (log2 units)
  bool grow = false;
  float mn[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    mn[hh] = fmaxf(m[hh], fmaxf(s0[hh], s1[hh]));
    grow |= mn[hh] > m[hh] + 8.f;
  }
  if (__any(grow)) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float mu = (mn[hh] > m[hh] + 8.f) ? mn[hh] : m[hh];
      const float alpha = (mu == m[hh]) ? 1.f : __builtin_amdgcn_exp2f(m[hh] - mu);
      l[hh] *= alpha;
#pragma unroll
      for (int e = 0; e < S::DPL; ++e) acc[hh][e] *= alpha;
      m[hh] = mu;
    }
  }
  float p0[HPW], p1[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const float ms = (m[hh] == -INFINITY) ? 0.f : m[hh];
    p0[hh] = __builtin_amdgcn_exp2f(s0[hh] - ms);
    p1[hh] = __builtin_amdgcn_exp2f(s1[hh] - ms);
    l[hh] += p0[hh] + p1[hh];
  }
  // ---- P * V
  if constexpr (E::kind == F32::kind) {
#pragma unroll
    for (int c = 0; c < S::NCH; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float x0 = __uint_as_float(b.v0[c][w]);
        const float x1 = __uint_as_float(b.v1[c][w]);
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh)
          acc[hh][c * 4 + w] = fmaf(p1[hh], x1, fmaf(p0[hh], x0, acc[hh][c * 4 + w]));
      }
  } else {
    uint32_t pp[HPW];
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
      pp[hh] = (E::kind == BF16::kind) ? pack_bf16(p0[hh], p1[hh]) : pack_f16(p0[hh], p1[hh]);
#pragma unroll
    for (int c = 0; c < S::NCH; ++c)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = pair_lo(b.v0[c][w], b.v1[c][w]);
        const uint32_t hi = pair_hi(b.v0[c][w], b.v1[c][w]);
        const int e = c * S::EPV + 2 * w;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          if constexpr (E::kind == BF16::kind) {
            acc[hh][e] = dot2_bf16(lo, pp[hh], acc[hh][e]);
            acc[hh][e + 1] = dot2_bf16(hi, pp[hh], acc[hh][e + 1]);
          } else {
            acc[hh][e] = dot2_f16(lo, pp[hh], acc[hh][e]);
            acc[hh][e + 1] = dot2_f16(hi, pp[hh], acc[hh][e + 1]);
          }
        }
      }
  }
}

// Attention of one query row over keys [16*j0, min(16*j1, L)) of request r.
// `writer`: this wave stores the request's new token into the cache when the
// launch carries new tokens and the range holds the request's last block.
template <typename E, int D, int HPW>
__device__ __forceinline__ void process_range(const DecodeArgs& a, int r, int row, int L, int j0,
                                              int j1, int h, int hq0, bool whole, int slot,
                                              bool writer) {
  using S = Shape<E, D, HPW>;
  const int lane = lane_id();
  const int tg = lane >> 3;
  const int ds = lane & 7;

  // ids of the range's first two blocks, fetched before the queries (scalar
  // loads, beside the vector loads of the queries)
  const int sk = a.skip_blocks;
  const int32_t* bt = uniform_ptr(a.block_table + (int64_t)r * a.bt_stride + sk);
  const int id_first = load_scalar(bt + uniform(j0));
  const int id_first_next = load_scalar(bt + uniform(min(j0 + 1, j1 - 1)));

  // this lane's slice of the HPW query vectors
  u32x4_t qv[HPW][S::NCH];
  {
    const uint8_t* qb = static_cast<const uint8_t*>(a.q) +
                        ((int64_t)row * a.num_q_heads + hq0) * S::ROWB + ds * 16;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int c = 0; c < S::NCH; ++c) qv[hh][c] = load16(qb + hh * S::ROWB + c * 128);
  }

  const int64_t tok_stride = (int64_t)a.num_kv_heads * S::ROWB;
  const int64_t half_stride = kBlockSize * tok_stride;
  const int64_t blk_stride = 2 * half_stride;
  const int64_t tok8 = 8 * tok_stride;
  const uint8_t* kvh = static_cast<const uint8_t*>(a.kv) + (int64_t)h * S::ROWB +
                       tg * tok_stride + ds * 16;
  // j runs over the blocks after a shared prefix of sk blocks; attend_block
  // takes full-table indices (for the partial last block)
  const int nb = (L + kBlockSize - 1) / kBlockSize;

  float m[HPW], l[HPW], acc[HPW][S::DPL];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < S::DPL; ++e) acc[hh][e] = 0.f;
  }

  // The step's new token (position L - 1) lives in the request's last block:
  // when this range holds that block and the launch carries new tokens, the
  // token's rows are read from the new-token input (its cache row is being
  // written in this launch) and one wave per KV head stores them.
  const bool fresh = a.fresh.k != nullptr && j1 + sk == nb;
  const int jlast = fresh ? nb - 1 - sk : -1;  // range-local index of the last block
  const int off = (L - 1) & (kBlockSize - 1);  // the new token's row in that block
  const int64_t nrow = (int64_t)row * tok_stride + (int64_t)h * S::ROWB;
  if (fresh && writer) {
    constexpr int NL = S::ROWB / 16;           // 16-byte pieces per row
    const int64_t id = load_scalar(bt + jlast);
    if (lane < 2 * NL) {
      const int hv = lane / NL;
      const int64_t piece = nrow + (lane % NL) * 16;
      const uint8_t* src = static_cast<const uint8_t*>(hv ? a.fresh.v : a.fresh.k) + piece;
      uint8_t* dst = static_cast<uint8_t*>(a.fresh.kv) + id * blk_stride + hv * half_stride +
                     (int64_t)off * tok_stride + (int64_t)h * S::ROWB + (lane % NL) * 16;
      store16(dst, load16(src));
    }
    if (h == 0 && lane == 0 && a.fresh.slot_out) a.fresh.slot_out[row] = id * kBlockSize + off;
  }

  // two register buffers: block j+1 is in flight while block j is processed
  // (a third buffer, two blocks in flight, measured no faster and costs 32
  // VGPRs); block ids are read one step before their loads are issued
  BlockRegs<E, D, HPW> b0, b1;
  auto load_at = [&](BlockRegs<E, D, HPW>& b, int jj, int id) {
    const uint8_t* p = kvh + (int64_t)id * blk_stride;
    if (jj != jlast) {
      load_block<E, D, HPW>(b, p, tok8, half_stride);
    } else {
      // the lane whose token is the new one reads it from the input rows;
      // that address differs from the lane's cache address by the same
      // (wave-uniform) amount in every such lane: dk for K, dv for V
      const int64_t cache_row = (int64_t)reinterpret_cast<uintptr_t>(a.kv) +
                                (int64_t)id * blk_stride + (int64_t)off * tok_stride;
      const int64_t dk =
          (int64_t)reinterpret_cast<uintptr_t>(a.fresh.k) + (int64_t)row * tok_stride - cache_row;
      const int64_t dv = (int64_t)reinterpret_cast<uintptr_t>(a.fresh.v) +
                         (int64_t)row * tok_stride - cache_row - half_stride;
      const bool s0 = tg == off, s1 = tg + 8 == off;
      load_rows<E, D, HPW>(b, p + (s0 ? dk : 0), p + tok8 + (s1 ? dk : 0),
                           p + half_stride + (s0 ? dv : 0), p + half_stride + tok8 + (s1 ? dv : 0));
    }
  };
  // Every issue loads a block, also past the range (then block j1 - 1 again,
  // which this wave has just read and L2 still holds): with the same loads in
  // flight on every path the compiler keeps the next block's loads
  // outstanding while the current one is processed.  Issued only when a next
  // block exists, its wait counts were merged with the path that issued
  // nothing, and each block ended up waiting for the next block's loads.
  int id_next = id_first_next;                 // id of block min(j + 1, j1 - 1)
  load_at(b0, j0, id_first);
  int j = j0;
  auto issue = [&](BlockRegs<E, D, HPW>& b) {
    // fetch the id after block j + 1 (a scalar load: the index is marked
    // wave-uniform), then load block j + 1 (clamped) into b
    const int id = id_next;
    id_next = load_scalar(bt + uniform(min(j + 2, j1 - 1)));
    load_at(b, min(j + 1, j1 - 1), id);
  };
  while (true) {
    issue(b1);
    attend_block<E, D, HPW>(b0, j + sk, nb, L, tg, a.scale_log2, qv, m, l, acc);
    if (++j >= j1) break;
    issue(b0);
    attend_block<E, D, HPW>(b1, j + sk, nb, L, tg, a.scale_log2, qv, m, l, acc);
    if (++j >= j1) break;
  }

  // ---- merge the 8 token groups: common max, rescaled sums and accumulators
  float Mh[HPW], Lh[HPW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    float M = m[hh];
    M = fmaxf(M, xor8(M));
    M = max_over_rows(M);
    const float sc = (m[hh] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[hh] - M);
    float lt = l[hh] * sc;
    lt += xor8(lt);
    lt = sum_over_rows(lt);
#pragma unroll
    for (int e = 0; e < S::DPL; ++e) acc[hh][e] *= sc;
    Mh[hh] = M;
    Lh[hh] = lt;
  }
  // reduce-scatter over the groups: lane keeps NOUT consecutive values of
  // the flattened [HPW][DPL] accumulator, starting at `base`.  Step st pairs
  // token group tg with tg ^ (1 << st) (lanes l and l ^ (8 << st)): the one
  // whose bit st is 0 keeps the low half, its partner the high half, and each
  // adds the other's copy of the half it keeps.  Steps 1 and 2 pair whole
  // rows / half-waves, which the row-swap moves exchange in one instruction
  // per pair of halves.
  float* v = &acc[0][0];
  int base = 0;
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const int n = S::NV >> st;
    const int bit = (tg >> st) & 1;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float lo = v[i], hi = v[i + n / 2];
      if (st == 0) {
        const float send = bit ? lo : hi;
        const float keep = bit ? hi : lo;
        v[i] = keep + xor8(send);
      } else {
        const F2 r = st == 1 ? swap16(lo, hi) : swap32(lo, hi);
        v[i] = r.a + r.b;
      }
    }
    base += bit * (n / 2);
  }
  const int hsel = base / S::DPL;
  const int e0 = base % S::DPL;
  float lsel = Lh[0], msel = Mh[0];
#pragma unroll
  for (int hh = 1; hh < HPW; ++hh) {
    lsel = (hsel == hh) ? Lh[hh] : lsel;
    msel = (hsel == hh) ? Mh[hh] : msel;
  }
  const int hq = hq0 + hsel;
  if (whole) {
    uint8_t* ob = static_cast<uint8_t*>(a.out) + ((int64_t)row * a.num_q_heads + hq) * S::ROWB;
    const float inv = 1.f / lsel;
#pragma unroll
    for (int r0 = 0; r0 < S::NOUT; r0 += S::RUN)
      store_run<E, S::RUN>(ob + (int64_t)dim_of<S>(e0 + r0, ds) * S::ESZ, v + r0, inv);
  } else {
    const int64_t ps = (int64_t)slot * a.num_q_heads + hq;
    float* ob = a.ws_o + ps * D;
#pragma unroll
    for (int r0 = 0; r0 < S::NOUT; r0 += S::RUN)
      store_f32_run<S::RUN>(ob + dim_of<S>(e0 + r0, ds), v + r0);
    // one lane per head writes (max, sum): the lane whose run starts the head
    if (e0 == 0 && ds == 0) {
      f32x2_t ml = {msel, lsel};
      *reinterpret_cast<f32x2_t*>(a.ws_ml + ps * 2) = ml;
    }
  }
}

// One work-group (4 wavefronts) of the split: work-group index wg.
template <typename E, int D, int HPW>
__device__ __forceinline__ void decode_split_body(const DecodeArgs& a, int wg) {
  const int lane = lane_id();
  const int item = uniform(wg * 4 + (int)(threadIdx.x >> 6));
  const int per_chunk = a.num_kv_heads * a.head_groups;
  if (item >= a.num_chunks * per_chunk) return;
  const int c = item / per_chunk;
  const int rem = item - c * per_chunk;
  const int h = rem / a.head_groups;
  const int hs = rem - h * a.head_groups;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int hq0 = h * group + hs * HPW;

  const int W = total_blocks(a);
  if (W == 0) return;
  const int64_t b0 = chunk_begin(c, W, a.num_chunks);
  const int64_t b1 = chunk_begin(c + 1, W, a.num_chunks);
  if (b0 >= b1) return;

  int running = 0;
  for (int base = 0; base < a.num_seqs && running < b1; base += kWave) {
    const ReqInfo ri = req_info(a, base + lane);
    const int incl = wave_incl_scan(ri.nb) + running;
    const int excl = incl - ri.nb;
    uint64_t mask = __ballot(ri.nb > 0 && excl < b1 && incl > b0);
    while (mask) {
      const int src = __builtin_ctzll(mask);
      mask &= mask - 1;
      const int s = readlane(excl, src), e = readlane(incl, src);
      const int L = readlane(ri.len, src), row = readlane(ri.row, src);
      const int j0 = (int)((b0 > s ? b0 : s) - s);
      const int j1 = (int)((b1 < e ? b1 : e) - s);
      // with a shared prefix every piece is a partial (merged with the prefix's)
      const bool whole = (j0 == 0) && (j1 == e - s) && a.prefix_slot0 < 0;
      if (j0 == 0 && h == 0 && hs == 0 && lane == 0) {
        // the range holding the request's first block records how it was cut
        const int cl = whole ? -1 : chunk_of(e - 1, W, a.num_chunks);
        int4 meta = {whole ? -1 : c, cl, W, 0};
        *reinterpret_cast<int4*>(a.ws_meta + 4 * (int64_t)(base + src)) = meta;
      }
      process_range<E, D, HPW>(a, base + src, row, L, j0, j1, h, hq0, whole, base + src + c,
                               hs == 0);
    }
    running = readlane(incl, kWave - 1);
  }
}

template <typename E, int D, int HPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void decode_split_kernel(DecodeArgs a) {
  decode_split_body<E, D, HPW>(a, blockIdx.x);
}

// Merge the partials of requests cut by range boundaries.  One wavefront per
// (request, query head); lane owns D/64 consecutive dims.  The split kernel
// recorded, for each decode request, its first and last range and W.  The
// (max, sum) pairs of all ranges are read at once, one range per lane, and the
// partial outputs in batches of 8 ranges, so the merge costs a few memory
// round trips whatever the number of ranges.
template <typename E, int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs a) {
  const int lane = lane_id();
  const int r = blockIdx.x / a.num_q_heads;
  const int hq = blockIdx.x - r * a.num_q_heads;
  // the request's cut record is loaded beside its length (one round trip);
  // it is used only where the split wrote it
  const int4 meta = *reinterpret_cast<const int4*>(a.ws_meta + 4 * (int64_t)r);
  bool active = a.seq_lens[r] > 0;
  int row = r;
  if (a.qsl) {
    const int q0 = a.qsl[r], q1 = a.qsl[r + 1];
    active = active && (q1 - q0 == 1);
    row = q0;
  }
  if (!active) return;
  const bool prefix = a.prefix_slot0 >= 0;
  // a request whose keys all lie in the shared prefix has no range partials
  // (and no metadata): its prefix partial is the whole result
  const bool ranges = !prefix || (a.seq_lens[r] + kBlockSize - 1) / kBlockSize > a.skip_blocks;
  int cf = 0, cl = -1, W = 1;
  if (ranges) {
    if (meta.x < 0) return;  // finished in place by its range
    cf = uniform(meta.x);
    cl = uniform(meta.y);
    W = uniform(meta.z);
  }
  const int N = a.num_chunks;
  const int64_t base = (int64_t)r * a.num_q_heads + hq;  // slot (r + c) -> + c * Hq
  const int64_t pslot = ((int64_t)a.prefix_slot0 + r) * a.num_q_heads + hq;

  // pass 1: global max and weighted sum over ranges, lanes in parallel
  float M = -INFINITY;
  for (int c0 = cf; c0 <= cl; c0 += kWave) {
    const int c = c0 + lane;
    float mc = -INFINITY;
    if (c <= cl && chunk_begin(c, W, N) < chunk_begin(c + 1, W, N))
      mc = a.ws_ml[(base + (int64_t)c * a.num_q_heads) * 2];
    M = fmaxf(M, mc);
  }
  M = wave_max(M);
  f32x2_t pml = {-INFINITY, 0.f};
  if (prefix) {
    pml = *reinterpret_cast<const f32x2_t*>(a.ws_ml + pslot * 2);
    M = fmaxf(M, pml[0]);
  }

  constexpr int DPT = D / kWave;
  float lsum = 0.f, acc[DPT];
#pragma unroll
  for (int i = 0; i < DPT; ++i) acc[i] = 0.f;
  if (prefix) {
    // the prefix partial's share: one term, on lane 0's sum only
    const float w = __builtin_amdgcn_exp2f(pml[0] - M);
    const float* po = a.ws_o + pslot * D + lane * DPT;
#pragma unroll
    for (int i = 0; i < DPT; ++i) acc[i] = w * po[i];
    lsum = lane == 0 ? w * pml[1] : 0.f;
  }
  for (int c0 = cf; c0 <= cl; c0 += kWave) {
    const int c = c0 + lane;
    float w = 0.f;
    if (c <= cl && chunk_begin(c, W, N) < chunk_begin(c + 1, W, N)) {
      const f32x2_t ml = *reinterpret_cast<const f32x2_t*>(
          a.ws_ml + (base + (int64_t)c * a.num_q_heads) * 2);
      w = __builtin_amdgcn_exp2f(ml[0] - M);
      lsum += w * ml[1];
    }
    // pass 2: this group of up to 64 ranges, 8 loads in flight at a time
    const int n = min(kWave, cl - c0 + 1);
    for (int k0 = 0; k0 < n; k0 += 8) {
      float v[8][DPT], wk[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        wk[k] = k0 + k < n ? __int_as_float(readlane(__float_as_int(w), k0 + k)) : 0.f;
#pragma unroll
        for (int i = 0; i < DPT; ++i) v[k][i] = 0.f;
        if (wk[k] != 0.f) {
          const float* po = a.ws_o + (base + (int64_t)(c0 + k0 + k) * a.num_q_heads) * D +
                            lane * DPT;
#pragma unroll
          for (int i = 0; i < DPT; ++i) v[k][i] = po[i];
        }
      }
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int i = 0; i < DPT; ++i) acc[i] = fmaf(wk[k], v[k][i], acc[i]);
    }
  }
  lsum = wave_sum(lsum);
  uint8_t* ob = static_cast<uint8_t*>(a.out) +
                (((int64_t)row * a.num_q_heads + hq) * D + lane * DPT) * E::bytes;
  store_run<E, DPT>(ob, acc, 1.f / lsum);
}

}  // namespace
}  // namespace pa
