// Q K^T tiles on MFMA, shared by the compressor passes and dense attention.
//
// One wave owns 32 query rows of a query block and computes the transposed
// score tile S^T[j][i] = k_j . q_i for all B keys of a key block:
//   A operand = K rows (m = key j), B operand = Q rows (n = query i),
// so lane l ends up holding query row i = l % 32 and 16 keys per 32-key group
// (see acc_row).  Row-wise softmax statistics then reduce mostly inside one
// lane, with one exchange between lane l and l ^ 32.
//
// k-assignment: lane half hl carries the columns [hl * d/2, (hl + 1) * d/2) of
// both operands, so every lane reads one contiguous half-row of Q and K.
#pragma once

#include "mf_common.hpp"

namespace mf {

constexpr int kQkXcds = 8;  // XCDs; consecutive work-group ids go to them in turn

// Work-group id -> (schedule position, query head) for kernels with one
// work-group per (query block, query head) that read the K (and V) of head
// h / grp.  With those key/value heads splitting evenly over the XCDs
// (kv_major), each XCD takes its key/value heads one at a time: every position
// of one head group (the query heads sharing that K) before the next group,
// the group's query heads next to each other, so the work-groups in flight on
// one XCD read one head's K and share it in the XCD's L2.  Otherwise
// position-major.
__device__ __forceinline__ void kv_major_slot(int b, int Hq, int grp, int NBR, int kv_major,
                                              int &pos, int &h) {
  if (kv_major) {
    const int x = b % kQkXcds, k = b / kQkXcds;
    const int r = k % grp, k2 = k / grp;
    pos = k2 % NBR;
    h = (x + kQkXcds * (k2 / NBR)) * grp + r;
  } else {
    pos = b / Hq;
    h = b % Hq;
  }
}

template <int B, int D, bool F32>
struct QKCfg {
  static constexpr int NW = B / 32;                 // waves per work-group
  static constexpr int NT = B * 2;                  // threads per work-group
  static constexpr int ESZ = F32 ? 4 : 2;           // bytes per Q/K element
  static constexpr int ROWB = D * ESZ;              // bytes per K row
  static constexpr int PITCH = ROWB + kLdsPad;      // LDS row pitch
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int NCH = B * CPR / NT;          // chunks per thread per tile
  static constexpr int KBYTES = B * PITCH;          // LDS bytes of one K tile
  static_assert(NCH * NT == B * CPR, "tile chunks must divide evenly");
};

// Q operand of one lane: half of its query row, kept in registers.
template <int D, bool F32>
struct QOp;
template <int D>
struct QOp<D, false> {
  u32x4 v[D / 16];
};
template <int D>
struct QOp<D, true> {
  float v[D / 2];
};

// Loads the lane's half-row; `row` points at the row's first element or is null
// (row outside the sequence -> zeros).
template <int D>
__device__ __forceinline__ void load_q(QOp<D, false> &qo, const uint16_t *row, int hl) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (row)
      qo.v[c] = *reinterpret_cast<const u32x4 *>(row + hl * (D / 2) + c * 8);
    else
      qo.v[c] = u32x4{0u, 0u, 0u, 0u};
  }
}
template <int D>
__device__ __forceinline__ void load_q(QOp<D, true> &qo, const float *row, int hl) {
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    float4 x = row ? *reinterpret_cast<const float4 *>(row + hl * (D / 2) + c * 4)
                   : float4{0.f, 0.f, 0.f, 0.f};
    qo.v[4 * c + 0] = x.x;
    qo.v[4 * c + 1] = x.y;
    qo.v[4 * c + 2] = x.z;
    qo.v[4 * c + 3] = x.w;
  }
}

// Global -> registers: one K tile (rows [row0, row0 + nvalid) of a head, zeros
// past nvalid).  `kbase` is the byte address of token 0 of the head.
template <int B, int D, bool F32>
__device__ __forceinline__ void gload_tile(u32x4 *stg, const char *kbase,
                                           int64_t row0, int nvalid, int tid) {
  using C = QKCfg<B, D, F32>;
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    const int idx = tid + c * C::NT;
    const int r = idx / C::CPR, col = idx % C::CPR;
    if (r < nvalid)
      stg[c] = *reinterpret_cast<const u32x4 *>(kbase + (row0 + r) * C::ROWB + col * 16);
    else
      stg[c] = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int B, int D, bool F32>
__device__ __forceinline__ void lstore_tile(char *lds, const u32x4 *stg,
                                            int tid) {
  using C = QKCfg<B, D, F32>;
#pragma unroll
  for (int c = 0; c < C::NCH; ++c) {
    const int idx = tid + c * C::NT;
    const int r = idx / C::CPR, col = idx % C::CPR;
    *reinterpret_cast<u32x4 *>(lds + r * C::PITCH + col * 16) = stg[c];
  }
}

// S^T tile for the wave's 32 query rows against the B keys staged in `klds`.
template <int B, int D>
__device__ __forceinline__ void st_tile(f32x16 (&acc)[B / 32], const char *klds,
                                        const QOp<D, false> &qo, int lane) {
  using C = QKCfg<B, D, false>;
  const int m = lane & 31, hl = lane >> 5;
  const char *rowp = klds + m * C::PITCH + hl * D;  // D/2 bf16 = D bytes
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb) acc[mb] = zero16();
  // k-step outer, key groups inner: B/32 independent accumulation chains
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int mb = 0; mb < B / 32; ++mb) {
      u32x4 a = *reinterpret_cast<const u32x4 *>(rowp + mb * 32 * C::PITCH + ks * 16);
      acc[mb] = mfma_bf16(as_bf16x8(a), as_bf16x8(qo.v[ks]), acc[mb]);
    }
}

template <int B, int D>
__device__ __forceinline__ void st_tile(f32x16 (&acc)[B / 32], const char *klds,
                                        const QOp<D, true> &qo, int lane) {
  using C = QKCfg<B, D, true>;
  const int m = lane & 31, hl = lane >> 5;
  const char *rowp = klds + m * C::PITCH + hl * (D / 2) * 4;
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb) acc[mb] = zero16();
#pragma unroll
  for (int c = 0; c < D / 8; ++c)
#pragma unroll
    for (int mb = 0; mb < B / 32; ++mb) {
      float4 a = *reinterpret_cast<const float4 *>(rowp + mb * 32 * C::PITCH + c * 16);
      acc[mb] = mfma_f32(a.x, qo.v[4 * c + 0], acc[mb]);
      acc[mb] = mfma_f32(a.y, qo.v[4 * c + 1], acc[mb]);
      acc[mb] = mfma_f32(a.z, qo.v[4 * c + 2], acc[mb]);
      acc[mb] = mfma_f32(a.w, qo.v[4 * c + 3], acc[mb]);
    }
}

// Scaled logits (log2 units) with causal mask and offsets, in place.
// `plain` (uniform): the tile is strictly below the diagonal and touches
// neither sink columns nor the local window, so only the scale applies.
// Returns the lane's maximum over its 16 * B/32 values (-inf if none valid).
template <int B>
__device__ __forceinline__ float logits_inplace(f32x16 (&acc)[B / 32], bool plain, bool rvalid,
                                                int i_pos, int jbase, float scale2, int sink_n,
                                                float sink2, int local_w, float local2,
                                                int lane) {
  float mx = -INFINITY;
  if (plain) {
#pragma unroll
    for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        acc[mb][r] *= scale2;
        mx = fmaxf(mx, acc[mb][r]);
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j_pos = jbase + mb * 32 + acc_row(r, lane);
        const int diff = i_pos - j_pos;
        float x = acc[mb][r] * scale2;
        x += (j_pos < sink_n) ? sink2 : 0.f;
        x += (diff >= 0 && diff < local_w) ? local2 : 0.f;
        x = (diff < 0) ? -INFINITY : x;
        acc[mb][r] = x;
        mx = fmaxf(mx, x);
      }
  }
  return rvalid ? mx : -INFINITY;
}

// Tile class of key block J for query block I (uniform over a work-group).
// `plain`: strictly below the diagonal, no sink column, no local-window element.
__device__ __forceinline__ bool plain_tile(int I, int J, int B, int sink_n, float sink2,
                                           int local_w, float local2) {
  if (J >= I) return false;
  if (sink2 != 0.f && J * B < sink_n) return false;
  if (local2 != 0.f && I * B - (J * B + B - 1) < local_w) return false;
  return true;
}

// `uniform`: strictly below the diagonal, no sink column, and the local window
// covers either all of the tile or none of it, so every element gets the same
// offset `off` (log2 units).  Rows i of block I and keys j of block J < I differ
// by (I - J) * B - (B - 1) .. (I - J) * B + (B - 1).
__device__ __forceinline__ bool uniform_tile(int I, int J, int B, int sink_n, float sink2,
                                             int local_w, float local2, float &off) {
  off = 0.f;
  if (J >= I) return false;
  if (sink2 != 0.f && J * B < sink_n) return false;
  if (local2 != 0.f) {
    const int dmin = (I - J) * B - (B - 1), dmax = (I - J) * B + (B - 1);
    if (dmax < local_w)
      off = local2;
    else if (dmin < local_w)
      return false;
  }
  return true;
}

// Lane maximum of the raw scores (before scaling), three at a time.
template <int B>
__device__ __forceinline__ float lane_rawmax(const f32x16 (&acc)[B / 32]) {
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = max3(mx, acc[mb][r], acc[mb][r + 1]);
  return mx;
}

// Sum of exp2(acc * scale2 + c) over the lane's values, pairwise within each
// 16-group.
template <int B>
__device__ __forceinline__ float lane_expsum_fma(const f32x16 (&acc)[B / 32], float scale2, float c) {
  float tot = 0.f;
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = fast_exp2(fmaf(acc[mb][r], scale2, c));
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) e[r] += e[r + w];
    tot += e[0];
  }
  return tot;
}

// Sum of exp2(x - mx) over the lane's values, pairwise within each 16-group.
template <int B>
__device__ __forceinline__ float lane_expsum(const f32x16 (&acc)[B / 32], float mx) {
  float tot = 0.f;
#pragma unroll
  for (int mb = 0; mb < B / 32; ++mb) {
    float e[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) e[r] = fast_exp2(acc[mb][r] - mx);
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
      for (int r = 0; r < w; ++r) e[r] += e[r + w];
    tot += e[0];
  }
  return tot;
}

}  // namespace mf
