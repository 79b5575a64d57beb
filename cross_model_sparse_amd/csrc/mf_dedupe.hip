// Shared-prefix block-rows (MapFlow, "Accelerating Cross-Model LLM Inference via
// Attention Map Reuse", §5.3: the Block Manager indexes compressed blocks by
// prefix hashes; §2.3: prefix caching).
//
// A full block-row (s, I) ((I + 1) B <= L_s) depends only on q and k of tokens
// 0 .. (I + 1) B - 1 of its sequence (causal rows, offsets measured from the
// sequence start).  Two such block-rows with equal prefixes compress to the
// same kept blocks, tiles and kept masses, so only the first one is computed.
//
// Equality of prefixes is decided by hashes:
//   k_blockhash  per full block-row: a 128-bit sum over the 16-byte chunks of
//                its q and k rows (every head) of two independent 64-bit mixes of
//                (chunk value, chunk position) -- integer sums, so the result
//                does not depend on the order threads add them in;
//   k_chain      per sequence: the block hashes chained from block 0, so equal
//                chain values mean equal whole prefixes;
//   k_alias      per block-row: the first earlier sequence whose same block-row
//                is full and has the same chain value (a candidate);
//   k_verify     the hash is only a filter: consecutive block-rows of a sequence
//                whose candidates are consecutive block-rows of one earlier
//                sequence form a run, and the last row of each run compares its
//                whole prefix (every head, q and k) with the candidate's byte
//                for byte, which covers every row of the run;
//   k_alias_fix  a run with any differing byte keeps its own rows.
#include "mf_host.hpp"

namespace mf {

struct Hash128 {
  uint64_t a, b;
};

// splitmix64 finaliser
__device__ __forceinline__ uint64_t mix_a(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
// MurmurHash3 64-bit finaliser
__device__ __forceinline__ uint64_t mix_b(uint64_t z) {
  z ^= z >> 33;
  z *= 0xff51afd7ed558ccdull;
  z ^= z >> 33;
  z *= 0xc4ceb9fe1a85ec53ull;
  return z ^ (z >> 33);
}

constexpr uint64_t kGolden = 0x9e3779b97f4a7c15ull;
constexpr uint64_t kOdd2 = 0xd6e8feb86659fd93ull;

// ---------------------------------------------------------------------------
// k_blockhash: one work-group per global block-row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_blockhash(const char *__restrict__ q,
                                                   const char *__restrict__ k, int64_t T,
                                                   int32_t Hs, int32_t rowbytes, int32_t B,
                                                   const RowInfo *__restrict__ rows,
                                                   Hash128 *__restrict__ hash,
                                                   int32_t *__restrict__ full,
                                                   int32_t *__restrict__ mism) {
  __shared__ uint64_t sa[256], sb[256];
  const int gr = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) mism[gr] = 0;  // byte mismatch flag of the verify pass
  const RowInfo ri = rows[gr];
  const bool is_full = (int64_t)(ri.blk + 1) * B <= ri.len;
  if (!is_full) {
    if (tid == 0) {
      full[gr] = 0;
      hash[gr] = Hash128{0ull, 0ull};
    }
    return;
  }
  const int cpr = rowbytes / 16;                     // chunks per row
  const int64_t per_t = (int64_t)Hs * B * cpr;       // chunks per tensor
  const int64_t tok = (int64_t)ri.start + (int64_t)ri.blk * B;
  uint64_t ha = 0ull, hb = 0ull;
  for (int64_t c = tid; c < 2 * per_t; c += 256) {
    const int tsel = c >= per_t;
    const int64_t cc = c - tsel * per_t;
    const int64_t h = cc / ((int64_t)B * cpr);
    const int64_t rem = cc % ((int64_t)B * cpr);
    const int64_t r = rem / cpr, col = rem % cpr;
    const char *base = tsel ? k : q;
    const u32x4 w =
        *reinterpret_cast<const u32x4 *>(base + ((h * T + tok + r) * rowbytes) + col * 16);
    const uint64_t x0 = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
    const uint64_t x1 = (uint64_t)w[2] | ((uint64_t)w[3] << 32);
    const uint64_t pos = (uint64_t)c;
    ha += mix_a(x0 ^ (2 * pos + 1) * kGolden) + mix_a(x1 ^ (2 * pos + 2) * kGolden);
    hb += mix_b(x0 + (2 * pos + 1) * kOdd2) + mix_b(x1 + (2 * pos + 2) * kOdd2);
  }
  sa[tid] = ha;
  sb[tid] = hb;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) {
      sa[tid] += sa[tid + w];
      sb[tid] += sb[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    full[gr] = 1;
    hash[gr] = Hash128{sa[0], sb[0]};
  }
}

// ---------------------------------------------------------------------------
// k_chain: one thread per sequence; chain[gr] for full block-rows
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_chain(const int32_t *__restrict__ nbcum, int32_t nseq,
                                               const Hash128 *__restrict__ hash,
                                               const int32_t *__restrict__ full,
                                               Hash128 *__restrict__ chain) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= nseq) return;
  uint64_t ca = 0x243f6a8885a308d3ull, cb = 0x13198a2e03707344ull;
  for (int gr = nbcum[s]; gr < nbcum[s + 1]; ++gr) {
    if (!full[gr]) {
      chain[gr] = Hash128{0ull, 0ull};
      continue;
    }
    ca = mix_a(ca ^ hash[gr].a) + kGolden;
    cb = mix_b(cb + hash[gr].b) ^ kOdd2;
    chain[gr] = Hash128{ca, cb};
  }
}

// ---------------------------------------------------------------------------
// k_alias: one thread per global block-row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_alias(const RowInfo *__restrict__ rows,
                                               const int32_t *__restrict__ nbcum,
                                               const int32_t *__restrict__ cu, int32_t NBR,
                                               int32_t B, const Hash128 *__restrict__ chain,
                                               const int32_t *__restrict__ full,
                                               int32_t *__restrict__ alias) {
  const int gr = blockIdx.x * blockDim.x + threadIdx.x;
  if (gr >= NBR) return;
  int32_t out = gr;
  if (full[gr]) {
    const RowInfo ri = rows[gr];
    const Hash128 c = chain[gr];
    for (int s = 0; s < ri.seq; ++s) {
      const int64_t L = (int64_t)cu[s + 1] - cu[s];
      if ((int64_t)(ri.blk + 1) * B > L) continue;  // block-row I of s is not full
      const int g2 = nbcum[s] + ri.blk;
      const Hash128 c2 = chain[g2];
      if (c2.a == c.a && c2.b == c.b) {
        out = g2;
        break;
      }
    }
  }
  alias[gr] = out;
}

// ---------------------------------------------------------------------------
// k_verify: grid (NBR, kVerifySplit); work-group (gr, part) takes a share of the
// comparison if gr ends a run of candidates
// ---------------------------------------------------------------------------
constexpr int kVerifySplit = 64;

__device__ __forceinline__ bool run_continues(const RowInfo *__restrict__ rows,
                                              const int32_t *__restrict__ cand, int NBR, int gr) {
  // row gr + 1 continues gr's run: same sequence, and its candidate is the next
  // block-row of the same earlier sequence
  return gr + 1 < NBR && cand[gr + 1] != gr + 1 && rows[gr + 1].seq == rows[gr].seq &&
         cand[gr + 1] == cand[gr] + 1;
}

__global__ __launch_bounds__(256) void k_verify(const char *__restrict__ q,
                                                const char *__restrict__ k, int64_t T,
                                                int32_t Hs, int32_t rowbytes, int32_t B,
                                                int32_t NBR, const RowInfo *__restrict__ rows,
                                                const int32_t *__restrict__ cand,
                                                int32_t *__restrict__ mism) {
  const int gr = blockIdx.x, part = blockIdx.y, tid = threadIdx.x;
  const int c = cand[gr];
  if (c == gr || run_continues(rows, cand, NBR, gr)) return;
  const RowInfo ri = rows[gr], rc = rows[c];
  // tokens 0 .. (I + 1) B - 1 of both sequences, every head, q and k, 16-byte chunks
  const int cpr = rowbytes / 16;
  const int64_t ntok = (int64_t)(ri.blk + 1) * B;
  const int64_t per_t = (int64_t)Hs * ntok * cpr;
  bool diff = false;
  for (int64_t x = (int64_t)part * 256 + tid; x < 2 * per_t; x += (int64_t)kVerifySplit * 256) {
    const int tsel = x >= per_t;
    const int64_t xx = x - tsel * per_t;
    const int64_t h = xx / (ntok * cpr), rem = xx % (ntok * cpr);
    const int64_t r = rem / cpr, col = rem % cpr;
    const char *base = tsel ? k : q;
    const u32x4 a = *reinterpret_cast<const u32x4 *>(base + (h * T + ri.start + r) * rowbytes + col * 16);
    const u32x4 b = *reinterpret_cast<const u32x4 *>(base + (h * T + rc.start + r) * rowbytes + col * 16);
    diff |= (a[0] != b[0]) | (a[1] != b[1]) | (a[2] != b[2]) | (a[3] != b[3]);
  }
  if (__any(diff) && (tid & 63) == 0) atomicOr(&mism[gr], 1);
}

// ---------------------------------------------------------------------------
// k_alias_fix: one thread per global block-row; a candidate stands if its run
// compared equal
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_alias_fix(const RowInfo *__restrict__ rows,
                                                   const int32_t *__restrict__ cand,
                                                   const int32_t *__restrict__ mism, int32_t NBR,
                                                   int32_t *__restrict__ alias) {
  const int gr = blockIdx.x * blockDim.x + threadIdx.x;
  if (gr >= NBR) return;
  const int c = cand[gr];
  int out = gr;
  if (c != gr) {
    int e = gr;
    while (run_continues(rows, cand, NBR, e)) ++e;
    if (!mism[e]) out = c;
  }
  alias[gr] = out;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct DedupeWs {
  RowTable rt;
  size_t hash, chain, full, cand, mism;
  size_t total;
};

inline DedupeWs dedupe_ws(const SeqGeom &g) {
  Carve c;
  DedupeWs w;
  w.rt = carve_rows(c, g);
  const size_t n = g.NBR > 0 ? g.NBR : 1;
  w.hash = c.take<Hash128>(n);
  w.chain = c.take<Hash128>(n);
  w.full = c.take<int32_t>(n);
  w.cand = c.take<int32_t>(n);
  w.mism = c.take<int32_t>(n);
  w.total = c.off + 256;
  return w;
}

}  // namespace mf

using namespace mf;

extern "C" size_t mf_prefix_dedupe_workspace_bytes(const int32_t *cu, int32_t nseq, int32_t B) {
  SeqGeom g;
  if (seq_geom(cu, nseq, B, &g) != MF_OK) return 0;
  return dedupe_ws(g).total;
}

extern "C" mf_status mf_prefix_dedupe(void *stream, const void *q, const void *k,
                                      mf_dtype qk_dtype, const int32_t *cu_host,
                                      const int32_t *cu_dev, int32_t nseq, int32_t Hs, int32_t d,
                                      int32_t B, int32_t *row_alias, void *ws, size_t ws_bytes) {
  if (!cu_host || !cu_dev || Hs <= 0) return MF_ERR_INVALID_ARG;
  if (qk_dtype != MF_BF16 && qk_dtype != MF_FP32) return MF_ERR_UNSUPPORTED;
  if (!valid_dim(d)) return MF_ERR_UNSUPPORTED;
  SeqGeom g;
  mf_status st = seq_geom(cu_host, nseq, B, &g);
  if (st != MF_OK) return st;
  if (g.T > 0 && (!q || !k || !row_alias)) return MF_ERR_INVALID_ARG;
  const DedupeWs w = dedupe_ws(g);
  if (!ws || ws_bytes < w.total) return MF_ERR_WORKSPACE;
  if (g.NBR == 0) return MF_OK;
  void *wsa = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = launch_rowtable(s, cu_dev, g, B, wsa, w.rt)) != MF_OK) return st;
  const int32_t rowbytes = d * (qk_dtype == MF_FP32 ? 4 : 2);
  hipLaunchKernelGGL(k_blockhash, dim3(g.NBR), dim3(256), 0, s, static_cast<const char *>(q),
                     static_cast<const char *>(k), g.T, Hs, rowbytes, B,
                     at<RowInfo>(wsa, w.rt.rows), at<Hash128>(wsa, w.hash),
                     at<int32_t>(wsa, w.full), at<int32_t>(wsa, w.mism));
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  hipLaunchKernelGGL(k_chain, dim3((nseq + 255) / 256), dim3(256), 0, s,
                     at<int32_t>(wsa, w.rt.nbcum), nseq, at<Hash128>(wsa, w.hash),
                     at<int32_t>(wsa, w.full), at<Hash128>(wsa, w.chain));
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  int32_t *cand = at<int32_t>(wsa, w.cand);
  hipLaunchKernelGGL(k_alias, dim3((g.NBR + 255) / 256), dim3(256), 0, s,
                     at<RowInfo>(wsa, w.rt.rows), at<int32_t>(wsa, w.rt.nbcum), cu_dev, g.NBR, B,
                     at<Hash128>(wsa, w.chain), at<int32_t>(wsa, w.full), cand);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  hipLaunchKernelGGL(k_verify, dim3(g.NBR, kVerifySplit), dim3(256), 0, s,
                     static_cast<const char *>(q), static_cast<const char *>(k), g.T, Hs, rowbytes,
                     B, g.NBR, at<RowInfo>(wsa, w.rt.rows), cand, at<int32_t>(wsa, w.mism));
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  hipLaunchKernelGGL(k_alias_fix, dim3((g.NBR + 255) / 256), dim3(256), 0, s,
                     at<RowInfo>(wsa, w.rt.rows), cand, at<int32_t>(wsa, w.mism), g.NBR, row_alias);
  return hip_status();
}
