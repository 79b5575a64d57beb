// Shared device helpers for the gfx950 kernels: vector types, MFMA wrappers,
// the 32x32 accumulator layout, bf16 packing and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mapflow.h"

namespace mf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxNB = 1024;        // key blocks per sequence
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsPad = 16;         // bytes appended to every LDS row

// ---------------------------------------------------------------------------
// MFMA 32x32 tiles.
//
// Accumulator layout of every 32x32 MFMA on CDNA: lane l, register r holds
//   C[m = 8 * (r / 4) + 4 * (l / 32) + (r % 4)][n = l % 32].
// Operand layout: A lane l holds row m = l % 32, B lane l holds column
// n = l % 32; the lanes of one half (l / 32) share their k-values.  Which
// logical k each (half, element) carries is free as long as A and B agree,
// so loaders below pick contiguous memory runs per lane.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8 a, const bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16: A lane l holds row l % 16, B lane l column l % 16, the four
// lane groups (l / 16) share k-values; accumulator lane l, register r holds
//   C[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8 a, const bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// bf16 helpers (bit patterns in uint32 pairs)
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions over the 32 lanes of each wave half (lanes l and l ^ 32 are not mixed).
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Index of the calling wave in its work-group, as a value the compiler knows to
// be wave-uniform (held in a scalar register): buffer descriptors and scalar
// offsets built from it then need no per-lane waterfall loop.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Lanes l and l ^ 32 combined with one VALU swap (no LDS): v_permlane32_swap
// of v with itself gives every lane v[l % 32] in the first result and
// v[l % 32 + 32] in the second, so both halves get bitwise the same value.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide stream compaction: the mask of lanes with `pred` set, and this
// lane's rank among them (number of set lanes below it).
__device__ __forceinline__ uint64_t wave_ballot(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred);
}
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// ---------------------------------------------------------------------------
// Block-row table, built once per call from the device sequence offsets.
// Global block-row gr -> (sequence, block index in the sequence), and a
// schedule listing block-rows by block index descending (longest rows first).
// ---------------------------------------------------------------------------
struct RowInfo {
  int32_t seq;
  int32_t blk;      // I
  int32_t start;    // first token of the sequence
  int32_t len;      // sequence length
};

// Workspace carving with 256-byte alignment.
struct Carve {
  size_t off = 0;
  template <typename T>
  size_t take(size_t count) {
    size_t o = (off + 255) & ~size_t(255);
    off = o + count * sizeof(T);
    return o;
  }
};

// Inclusive prefix sum of one value per thread over a 1024-thread block: a
// shuffle scan inside each wave, then the wave totals.  `wsum` holds 16
// entries of LDS; every thread must call it.
__device__ __forceinline__ int64_t block_scan_incl(int64_t v, int64_t *wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int64_t u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += wsum[w];
  __syncthreads();  // wsum free for the next scan
  return v + before;
}

}  // namespace mf
