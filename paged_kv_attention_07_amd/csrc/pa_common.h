// Shared device helpers for the gfx950 paged-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;       // CDNA wavefront width

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Element formats.  `kind` matches pa_dtype.
struct F32 {
  using storage = float;
  static constexpr int bytes = 4;
  static constexpr int kind = 0;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  static constexpr int kind = 1;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int bytes = 2;
  static constexpr int kind = 2;
};

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
// A 16-byte load marked non-temporal (the load's nt bit): for data a launch
// reads once, such as decode's stream of K/V blocks, so it is not kept in the
// caches at the expense of data that is reused.
__device__ __forceinline__ u32x4_t load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// ---- 16-bit float helpers --------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (hardware round-to-nearest-even on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  f16x2_t r = __builtin_convertvector(v, f16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2_t, w)[1];
}

// acc + a.lo*b.lo + a.hi*b.hi for packed 16-bit pairs, fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a),
                                __builtin_bit_cast(f16x2_t, b), acc, false);
}

// (lo16(a), lo16(b)) and (hi16(a), hi16(b)) as packed pairs.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// ---- cross-lane ------------------------------------------------------------

// DPP controls (GFX9 encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowRor8 = 0x128;      // rotate right by 8 within 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 consecutive lanes of an aligned group; every lane gets it.
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  return x;
}


// gfx950's row-swap moves.  swap32(a, b) exchanges the upper 32 lanes of `a`
// with the lower 32 lanes of `b`; swap16(a, b) exchanges rows 1 and 3 of `a`
// with rows 0 and 2 of `b` (a row is 16 lanes).  Both are plain VALU moves,
// with no LDS round trip.  Returned as {new a, new b}.
struct F2 {
  float a, b;
};
__device__ __forceinline__ F2 swap32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ F2 swap16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Max / sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the same position in the
// four rows); every lane gets the result.  swap32(x, x) leaves lane l with
// x[l mod 32] in one register and x[l mod 32 + 32] in the other, and swap16
// does the same for pairs of rows.  Needs the whole wavefront active.
__device__ __forceinline__ float max_over_rows(float x) {
  const F2 h = swap32(x, x);
  x = fmaxf(h.a, h.b);
  const F2 r = swap16(x, x);
  return fmaxf(r.a, r.b);
}
__device__ __forceinline__ float sum_over_rows(float x) {
  const F2 h = swap32(x, x);
  x = h.a + h.b;
  const F2 r = swap16(x, x);
  return r.a + r.b;
}
// The value of lane l ^ 8 (rotating a 16-lane row by 8 swaps its halves).
__device__ __forceinline__ float xor8(float x) { return dpp<kDppRowRor8>(x); }
// Max / sum over the 16 lanes of a row, in registers; every lane of the row
// gets the same bits.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<kDppQuadXor1>(x));
  x = fmaxf(x, dpp<kDppQuadXor2>(x));
  x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
  return fmaxf(x, xor8(x));
}
__device__ __forceinline__ float row_sum16(float x) {
  x = sum8(x);
  return x + xor8(x);
}
// The same over the whole wavefront.  Needs the whole wavefront active.
__device__ __forceinline__ float wave_max(float x) { return max_over_rows(row_max16(x)); }
__device__ __forceinline__ float wave_sum(float x) { return sum_over_rows(row_sum16(x)); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Mark a value the whole wavefront agrees on as uniform, so that the compiler
// keeps it (and loop counters / addresses derived from it) in scalar
// registers and uses scalar loads for addresses built from it.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Load through the constant address space: for a wave-uniform address this
// becomes a scalar (SMEM) load, which does not share the in-order vector
// memory counter with the bulk K/V loads.  Only for memory no kernel of the
// launch writes (block tables, lengths).
template <typename T>
__device__ __forceinline__ T load_scalar(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// A pointer the whole wavefront agrees on, in scalar registers (so loads
// through it can be scalar loads).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Uniform value of `x` in lane `l` (l uniform).
__device__ __forceinline__ int readlane(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// Inclusive prefix sum over the wavefront.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

}  // namespace pa
