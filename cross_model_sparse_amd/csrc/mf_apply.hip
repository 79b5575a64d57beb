// Receiver-side fused retrieval with linear head translation (MapFlow,
// "Accelerating Cross-Model LLM Inference via Attention Map Reuse", §3.3 linear
// head mapping, §5.4 attention retrieval with a fused kernel):
//
//   O_t[i,:] = sum_h W[t,h] sum_{J kept by h} sum_{j in J} (A_h[i,j] / kmass_h[i]) V_g(t)[j,:]
//
// Per (target head, query block) and key block J in the union of the sources'
// kept sets, each lane rebuilds its row of the translated tile
// A~_t[i, J] = sum_h c_h[i] A_h[i, J] in fp32 registers straight from the bf16
// tiles (c_h[i] = W[t,h] / kmass_h[i]), rounds it to bf16 and feeds it as the A
// operand of 16x16x32 MFMAs against V_g(t)[J] staged in LDS.  The translated
// map never leaves registers; nothing of size L x L is written.  k_apply4 takes
// targets with at most four sources, k_apply_mix the others.
//
// V is first copied into a transposed, block-padded layout Vt[g][d][NBR * B]
// (k_vtranspose) so that the MFMA B operand (8 consecutive keys of one value
// column) is one 16-byte read.  Padding columns are zero.
//
// Work-group order: the hardware hands consecutive work-groups to the 8 XCDs in
// turn; the id is decoded so that all targets of one query block run on one XCD
// and reuse its L2 copy of the source tiles, while the 8 XCDs work on 8 query
// blocks at once and share V through the memory-side cache.
#include "mf_host.hpp"
#include <mutex>

namespace mf {

constexpr int kXcds = 8;
constexpr int kBufferFlags = 0x00020000;  // buffer descriptor word 3 for raw dword loads

// A wave-uniform value the compiler cannot prove uniform (it was loaded from
// memory, or computed from such a load), moved to a scalar register so buffer
// descriptors built from it need no per-lane loop.
__device__ __forceinline__ int uni32(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------------------
// V -> Vs [Hkv][NBR * B / 16][D][16]: each sequence block-padded to whole key
// blocks, cut into 16-key chunks, and each chunk stored head dimension major
// (column d holds its 16 keys as 32 contiguous bytes).  One chunk of one head
// is then D * 32 contiguous bytes, and 8 consecutive keys of one value column
// (an MFMA B operand) are one 16-byte piece.  Keys past a sequence end are zero.
//
// V is either contiguous [Hkv][T][D] or paged: token j of sequence s lives in
// page block_table[s][j / P] of a pool [pages][Hkv][P][D] at slot j % P (page
// indices outside the pool read as zeros).  With query windows (chunked prefill)
// only key blocks below the window's end are staged: no other block is read.
// ---------------------------------------------------------------------------
struct VSrc {
  const uint16_t *v;          // contiguous V, or null
  const uint16_t *pages;      // paged pool, or null
  const int32_t *table;       // [nseq][max_pages]
  int32_t page_size, max_pages, num_pages, Hkv;
  const int32_t *window;      // [nseq][2] query tokens [begin, end), or null
};

// element offset of (head g, global padded key column col, value column d) in Vs
__device__ __forceinline__ int64_t vs_index(int64_t NBR, int B, int D, int g, int64_t col, int d) {
  return (((int64_t)g * NBR * B + (col & ~int64_t(15))) * D) + (int64_t)d * 16 + (col & 15);
}

template <int B, int D>
__global__ __launch_bounds__(256) void k_vstage(VSrc vs, int64_t T,
                                                const RowInfo *__restrict__ rows, int32_t NBR,
                                                uint16_t *__restrict__ vt,
                                                const int32_t *__restrict__ need) {
  if (need && *need == 0) return;  // no kernel of this call reads the staged V
  constexpr int P = B + 8;  // LDS row pitch in elements
  __shared__ __attribute__((aligned(16))) uint16_t t[D * P];
  const int gr = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const RowInfo ri = rows[gr];
  if (vs.window && ri.blk * B >= vs.window[2 * ri.seq + 1]) return;  // not a key of the window
  const int nval = min(B, ri.len - ri.blk * B);
  const int64_t tok0 = (int64_t)ri.start + (int64_t)ri.blk * B;
  for (int idx = tid; idx < B * D / 8; idx += 256) {
    const int j = idx / (D / 8), c = idx % (D / 8);
    u32x4 x = u32x4{0u, 0u, 0u, 0u};
    if (j < nval) {
      const uint16_t *row = nullptr;
      if (vs.pages) {
        const int js = ri.blk * B + j;  // token index inside the sequence
        const int pg = vs.table[(int64_t)ri.seq * vs.max_pages + js / vs.page_size];
        if (pg >= 0 && pg < vs.num_pages)
          row = vs.pages + (((int64_t)pg * vs.Hkv + g) * vs.page_size + js % vs.page_size) * D;
      } else {
        row = vs.v + ((int64_t)g * T + tok0 + j) * D;
      }
      if (row) x = *reinterpret_cast<const u32x4 *>(row + c * 8);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      t[(c * 8 + 2 * e) * P + j] = (uint16_t)(x[e] & 0xffffu);
      t[(c * 8 + 2 * e + 1) * P + j] = (uint16_t)(x[e] >> 16);
    }
  }
  __syncthreads();
  // the block's B / 16 chunks are B * D contiguous elements; 16-byte piece
  // (chunk, d, half) at ((chunk * D + d) * 2 + half) * 8
  uint16_t *dst = vt + vs_index(NBR, B, D, g, (int64_t)gr * B, 0);
  for (int idx = tid; idx < B * D / 8; idx += 256) {
    const int half = idx & 1, d = (idx >> 1) % D, ch = (idx >> 1) / D;
    *reinterpret_cast<u32x4 *>(dst + (int64_t)idx * 8) =
        *reinterpret_cast<const u32x4 *>(&t[d * P + ch * 16 + half * 8]);
  }
}

// Schedule of the block-rows inside the query windows, in the longest-first
// order of the full schedule (stable compaction, one work-group).
__global__ __launch_bounds__(1024) void k_window_sched(const RowInfo *__restrict__ rows,
                                                       const int32_t *__restrict__ sched,
                                                       int32_t NBR, int32_t B,
                                                       const int32_t *__restrict__ window,
                                                       int32_t *__restrict__ wsched) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int p0 = 0; p0 < NBR; p0 += 1024) {
    const int p = p0 + tid;
    int gr = -1;
    bool keep = false;
    if (p < NBR) {
      gr = sched[p];
      const RowInfo ri = rows[gr];
      const int a = ri.blk * B;
      keep = a >= window[2 * ri.seq] && a < window[2 * ri.seq + 1];
    }
    const uint64_t mask = wave_ballot(keep);
    if (lane == 0) wsum[wave] = __popcll(mask);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (keep) wsched[off + lanes_below(mask)] = gr;
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wsum[w];
      base += tot;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// per (target, query block) set-up shared by both apply kernels
// ---------------------------------------------------------------------------
// Dynamic LDS (byte offsets; the V buffers are static): rbase[Hs] int64,
// src[Hs], wt[Hs] (every source with a nonzero weight), then for the at most
// kSrc4 sources k_apply4 mixes: bm[kSrc4][nbw], pc[kSrc4][nbw], uni[nbw],
// coef[kSrc4][B] (fp32), nsrc.  k_apply4 appends the union's key-block list:
// blist[nbw * 32] int32 and tix[nbw * 32][4] int32 (tile index of each of up
// to four sources, -1 if none).  Sized for four sources, the tables leave room
// for two work-groups per CU beside the two V tiles.
constexpr int kSrc4 = 4;
inline size_t apply_smem(int B, int Hs, int nbw) {
  size_t s = (size_t)Hs * (8 + 4 + 4);
  s += (size_t)kSrc4 * nbw * 8 + (size_t)nbw * 4;
  s += (size_t)kSrc4 * B * 4;
  s += 64;
  s += (size_t)nbw * 32 * 5 * 4;
  return s;
}

// LDS views of one (target, query block)'s source maps
struct RowMaps {
  int64_t *rbase;   // first tile of each source's block-row
  int32_t *src;     // source heads with a nonzero weight
  float *wt;        // their weights
  uint32_t *bm;     // kept bitmaps [source][nbw]
  int32_t *pc;      // exclusive popcount prefix of bm (tile rank of each word)
  uint32_t *uni;    // union of the kept bitmaps
  float *coef;      // [source][B] row coefficients W[t,h] / kmass_h[i]
  int32_t *nsrc;
  int32_t *tix;     // [k][4] tile index of source u at the k-th union block, -1 if none
  int32_t *blist;   // [k] the k-th key block of the union, ascending
  int nbw;
};

// byte offsets, kept relative to smem so every access stays an LDS access
__device__ __forceinline__ RowMaps row_maps(char *smem, int Hs, int nbw, int B) {
  const int o_rbase = 0;
  const int o_src = o_rbase + Hs * 8;
  const int o_wt = o_src + Hs * 4;
  const int o_bm = o_wt + Hs * 4;
  const int o_pc = o_bm + kSrc4 * nbw * 4;
  const int o_uni = o_pc + kSrc4 * nbw * 4;
  const int o_coef = o_uni + nbw * 4;
  const int o_ns = o_coef + kSrc4 * B * 4;
  const int o_tix = (o_ns + 4 + 15) & ~15;
  const int o_blist = o_tix + nbw * 32 * 16;
  RowMaps m;
  m.rbase = reinterpret_cast<int64_t *>(smem + o_rbase);
  m.src = reinterpret_cast<int32_t *>(smem + o_src);
  m.wt = reinterpret_cast<float *>(smem + o_wt);
  m.bm = reinterpret_cast<uint32_t *>(smem + o_bm);
  m.pc = reinterpret_cast<int32_t *>(smem + o_pc);
  m.uni = reinterpret_cast<uint32_t *>(smem + o_uni);
  m.coef = reinterpret_cast<float *>(smem + o_coef);
  m.nsrc = reinterpret_cast<int32_t *>(smem + o_ns);
  m.tix = reinterpret_cast<int32_t *>(smem + o_tix);
  m.blist = reinterpret_cast<int32_t *>(smem + o_blist);
  m.nbw = nbw;
  return m;
}

// Sources of target t (nonzero weights, ascending head order) and the start of
// their tile runs at block-row gr; clears the bitmaps.  Returns the source count
// (uniform).
template <int NT>
__device__ int row_sources(const RowMaps &m, const float *__restrict__ W, int t, int Hs,
                           const int64_t *__restrict__ row_ptr, int NBR, int gr, int tid) {
  if (tid < 64) {
    // wave 0 scans the weight row 64 heads at a time, compacting by ballot
    int ns = 0;
    for (int h0 = 0; h0 < Hs; h0 += 64) {
      const int h = h0 + tid;
      const float w = h < Hs ? W[(int64_t)t * Hs + h] : 0.f;
      const uint64_t mask = wave_ballot(w != 0.f);
      if (w != 0.f) {
        const int q = ns + lanes_below(mask);
        m.src[q] = h;
        m.wt[q] = w;
        m.rbase[q] = row_ptr[(int64_t)h * NBR + gr];
      }
      ns += __popcll(mask);
    }
    if (tid == 0) *m.nsrc = ns;
  }
  for (int i = tid; i < kSrc4 * m.nbw; i += NT) m.bm[i] = 0u;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*m.nsrc);
}

// Kept bitmaps of the ns sources at block-row gr, their tile ranks, the union
// bitmap and the per-row coefficients (fp32): W[t,h] / kmass_h[i] when
// renormalising (0 where the kept mass is 0), else W[t,h]; rows past the
// sequence end get 0.
template <int B, int NT>
__device__ void row_maps_fill(const RowMaps &m, int ns, const int64_t *__restrict__ row_ptr,
                              const int32_t *__restrict__ col_idx, int64_t capacity,
                              const float *__restrict__ kept_mass, int64_t T, int NBR, int gr,
                              int64_t tok0, int I, int L, int nw_row, int renorm, int tid) {
  for (int q = 0; q < ns; ++q) {
    // entries past the capacity of an overflowed map are treated as missing
    const int64_t b = m.rbase[q], e = min(row_ptr[(int64_t)m.src[q] * NBR + gr + 1], capacity);
    for (int64_t idx = b + tid; idx < e; idx += NT) {
      const int J = col_idx[idx];
      atomicOr(&m.bm[q * m.nbw + (J >> 5)], 1u << (J & 31));
    }
  }
  for (int idx = tid; idx < ns * B; idx += NT) {
    const int q = idx / B, il = idx % B;
    const int ip = I * B + il;
    float c = 0.f;
    if (ip < L) {
      if (renorm) {
        const float km = kept_mass[(int64_t)m.src[q] * T + tok0 + ip];
        c = km > 0.f ? m.wt[q] / km : 0.f;
      } else {
        c = m.wt[q];
      }
    }
    m.coef[q * B + il] = c;
  }
  __syncthreads();
  for (int q = tid; q < ns; q += NT) {
    int run = 0;
    for (int w = 0; w < nw_row; ++w) {
      m.pc[q * m.nbw + w] = run;
      run += __popc(m.bm[q * m.nbw + w]);
    }
  }
  if (tid < nw_row) {
    uint32_t u = 0u;
    for (int q = 0; q < ns; ++q) u |= m.bm[q * m.nbw + tid];
    m.uni[tid] = u;
  }
  __syncthreads();
}

// next key block of the union at or after `from` (uniform), -1 if none
__device__ __forceinline__ int union_next(const RowMaps &m, int n, int from) {
  if (from < 0 || from >= n) return -1;
  const int nw_row = (n + 31) / 32;
  for (int w = from >> 5; w < nw_row; ++w) {
    uint32_t bits = __builtin_amdgcn_readfirstlane(m.uni[w]);
    if (w == (from >> 5)) bits &= ~((1u << (from & 31)) - 1u);
    if (bits) return w * 32 + __ffs(bits) - 1;
  }
  return -1;
}

// tile index of source q at key block J, or -1 (uniform)
__device__ __forceinline__ int64_t tile_index(const RowMaps &m, int q, int J, int64_t capacity) {
  const uint32_t word = __builtin_amdgcn_readfirstlane(m.bm[q * m.nbw + (J >> 5)]);
  if (!((word >> (J & 31)) & 1u)) return -1;
  const int rank = __builtin_amdgcn_readfirstlane(m.pc[q * m.nbw + (J >> 5)]) +
                   __popc(word & ((1u << (J & 31)) - 1u));
  const int64_t rb = m.rbase[q];
  const int64_t ti = (int64_t)__builtin_amdgcn_readfirstlane((int)(rb & 0xffffffff)) +
                     ((int64_t)__builtin_amdgcn_readfirstlane((int)(rb >> 32)) << 32) + rank;
  return ti < capacity ? ti : -1;
}

// The union's key blocks in ascending order with the tile index of each of the
// (at most four) sources at each block; returns the number of blocks (uniform).
template <int NT>
__device__ int build_block_list(const RowMaps &m, int ns, int n, int64_t capacity, int tid) {
  const int nw_row = (n + 31) / 32;
  for (int J = tid; J < n; J += NT) {
    const uint32_t w = m.uni[J >> 5];
    if (!((w >> (J & 31)) & 1u)) continue;
    int k = __popc(w & ((1u << (J & 31)) - 1u));
    for (int i = 0; i < (J >> 5); ++i) k += __popc(m.uni[i]);
    m.blist[k] = J;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int32_t ti = -1;
      if (u < ns) {
        const uint32_t word = m.bm[u * m.nbw + (J >> 5)];
        if ((word >> (J & 31)) & 1u) {
          const int64_t x = m.rbase[u] + m.pc[u * m.nbw + (J >> 5)] +
                            __popc(word & ((1u << (J & 31)) - 1u));
          if (x < capacity) ti = (int32_t)x;
        }
      }
      m.tix[k * 4 + u] = ti;
    }
  }
  int total = 0;
  for (int i = 0; i < nw_row; ++i) total += __popc(m.uni[i]);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(total);
}

// work-group id -> (schedule position, target): consecutive ids land on XCDs in
// turn; XCD x takes every eighth query block of the longest-first order, all
// targets of one block before the next, zig-zagging between rounds so the XCDs
// stay in step and share V through the memory-side cache.
__device__ __forceinline__ void xcd_map(int Ht, int &pos, int &t) {
  const int x = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
  const int round = kx / Ht;
  t = kx % Ht;
  pos = round * kXcds + ((round & 1) ? (kXcds - 1 - x) : x);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glob_void;
// global-memory views for loads from a wave-uniform base (selects the
// base-in-SGPRs form of the global load)
typedef __attribute__((address_space(1))) const unsigned char gchar;
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2_t gu32x2;

// One 16-byte piece per lane, memory -> LDS: the wave's 64 pieces land at
// lds + 16 * lane.
template <int AUX>
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, char *lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, AUX);
}

// V tile of key block J -> LDS buffer with direct buffer->LDS loads (the same
// load class as the tile reads, so the compiler's wait counts stay exact); the
// wave moves VINST 1 KB blocks.  In LDS, row d of the tile (B keys) holds its
// 16-byte pieces c (keys 8c .. 8c + 7) at position c ^ (d % CPR), so the MFMA
// B-operand reads below are conflict-free.  In the staged V (k_vstage) the tile
// is B * D contiguous elements, piece (d, c) at ((c / 2) * D + d) * 16 + (c % 2) * 8.
template <int B, int D, int VINST>
__device__ __forceinline__ void dma_v_tile(char *dstbuf, const uint16_t *vtg, int64_t col0,
                                           int wave, int lane) {
  constexpr int CPR = B * 2 / 16;   // 16-byte pieces per row
  constexpr int RPB = 64 / CPR;     // rows per 1 KB block
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vtg + col0 * D), 0, B * D * 2, kBufferFlags);
  const int dl = lane / CPR, pp = lane % CPR;
#pragma unroll
  for (int i = 0; i < VINST; ++i) {
    const int blk = wave * VINST + i;        // 1 KB block of the tile
    const int d0 = blk * RPB;                // its first row
    const int c = pp ^ ((d0 + dl) % CPR);    // swizzled piece position
    const int voff = (((c >> 1) * D + dl) * 16 + (c & 1) * 8) * 2;
    const int soff = d0 * 32;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(dstbuf + blk * 1024), 16, voff, soff, 0, 0);
  }
}

// s_waitcnt immediate that waits until at most n vector-memory loads are
// outstanding (expcnt and lgkmcnt left unconstrained)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

template <int B>
__device__ __forceinline__ u32x4 v_frag(const char *vl, int d, int c) {
  constexpr int CPR = B * 2 / 16;
  return *reinterpret_cast<const u32x4 *>(vl + d * (B * 2) + ((c ^ (d % CPR)) << 4));
}

// ---------------------------------------------------------------------------
// k_apply4: targets with at most four sources (the translated map of a
// head-mapping row).  One work-group per (target, query block), one wave per
// RG 16-row MFMA groups.  The union's key blocks and each source's tile index
// there are listed once in LDS, so stepping to the next block is one broadcast
// read.
//
// Tile chunks (32 keys x 16 rows, 1 KB, fragment order) stream through a
// register ring of NR chunk slots, NR - 1 chunks ahead of the one being mixed,
// across key-block boundaries; V tiles go straight to a double LDS buffer one
// key block ahead.  Loads of sources without a tile at a key block (and past
// the last block) use zero-length descriptors: they return zeros without
// touching memory and keep the number of loads in flight static.
// ---------------------------------------------------------------------------
constexpr int cgcd(int a, int b) { return b == 0 ? a : cgcd(b, a % b); }

template <int B, int D, int FMT>
struct Apply4Cfg {
  static constexpr int RG = 1;                       // 16-row MFMA groups per wave
  static constexpr int NW = B / (16 * RG);           // waves
  static constexpr int NT = NW * 64;
  static constexpr int KC = B / 32;                  // 32-key chunks per key block
  // a ring unit is one load per source: a 32-key chunk of bf16 (16 bytes per
  // lane), or NP chunks of E4M3 codes (8 NP bytes per lane)
  static constexpr int NP = (FMT == MF_TILE_MXFP8 && B >= 64) ? 2 : 1;
  static constexpr int KU = KC / NP;                 // units per key block
  static constexpr int64_t TBYTES = tile_bytes(B, FMT);
  static constexpr int VBYTES = D * B * 2;
  static constexpr int VINST = VBYTES / 1024 / NW;   // 1 KB direct loads per wave per V tile
  // Ring slots (chunks).  Two, i.e. one chunk ahead.  About eight work-groups
  // of one query block read every source tile, and they hit in the XCD's L2
  // only while its recent tiles still fit there; deeper prefetch lowers that
  // hit rate (measured at L = 32K: 54% with two slots, 12% with four, and
  // twice the fabric traffic); 32-row waves with more slots lose the same way.
  static constexpr int NR = 2;
  // loads per unit: row groups x 4 sources, plus 4 scale loads with a block's first unit
  static constexpr int LPC = 4 * RG + (FMT == MF_TILE_MXFP8 ? 4 : 0);
  // key blocks per unrolled trip: ring slots and V buffers both return to their start
  static constexpr int TB = (NR * 2 * KU / cgcd(NR, 2 * KU)) / KU;
  // descriptor queue depth: blocks from the current one to the farthest prefetched
  static constexpr int DQ = (KU - 1 + NR - 1) / KU + 1;
  static_assert(VINST * 1024 * NW == VBYTES, "V tile must split into 1 KB wave loads");
  static_assert(TB % 2 == 0 && (TB * KU) % NR == 0, "trip must close the ring and V buffers");
  static_assert((NR - 1) * LPC + VINST <= 63, "vmcnt range");
  static_assert(FMT == MF_TILE_BF16 || RG == 1, "fp8 tiles take one row group per wave");
};


template <int B, int D, int FMT>
__global__ __launch_bounds__(B * 4) __attribute__((amdgpu_waves_per_eu(4))) void k_apply4(
    const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const char *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs,
    int32_t NBR, int64_t T, const float *__restrict__ W, int32_t Ht, int32_t grp,
    const uint16_t *__restrict__ vt, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, int32_t nrows, int32_t nbw, int64_t capacity,
    int32_t renorm, float *__restrict__ o, const int32_t *__restrict__ row_alias) {
  using C = Apply4Cfg<B, D, FMT>;
  constexpr int KU = C::KU, NP = C::NP, NR = C::NR, TB = C::TB, DQ = C::DQ;
  constexpr bool FP8 = FMT == MF_TILE_MXFP8;
  // separate arrays, so the compiler can tell that direct loads into one never
  // alias reads of the other
  __shared__ __attribute__((aligned(16))) char vA[C::VBYTES];
  __shared__ __attribute__((aligned(16))) char vB[C::VBYTES];
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const RowMaps mp = row_maps(smem, Hs, nbw, B);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kg = lane >> 4;
  int pos, t;
  xcd_map(Ht, pos, t);
  if (pos >= nrows) return;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int g = t / grp;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t tpad = (int64_t)NBR * B;

  // BSR row of this block-row: its own, or that of the earlier block-row it
  // shares (tiles and kept masses are equal; V and O stay this row's own)
  const int ga = row_alias ? row_alias[gr] : gr;
  const int grm = (ga >= 0 && ga < NBR) ? ga : gr;
  const int ns = row_sources<C::NT>(mp, W, t, Hs, row_ptr, NBR, grm, tid);
  if (ns > 4) return;  // handled by k_apply_mix
  row_maps_fill<B, C::NT>(mp, ns, row_ptr, col_idx, capacity, kept_mass, T, NBR, grm, tok0, I, L,
                          (n + 31) / 32, renorm, tid);

  constexpr int RG = C::RG;
  static_assert(RG == 1, "one row group per wave: the coefficients below are the lane's row's");

  const int nblk = build_block_list<C::NT>(mp, ns, n, capacity, tid);

  // k-th block of the union (uniform), -1 past the end
  auto blk_J = [&](int k) -> int {
    return k < nblk ? __builtin_amdgcn_readfirstlane(mp.blist[k]) : -1;
  };
  // tile descriptors of the k-th union block; zero-length for a source without
  // a tile there and past the last block
  struct Src4 {
    __amdgpu_buffer_rsrc_t r[4];
  };
  auto src4 = [&](Src4 &S, int k) {
    u32x4 ti4 = u32x4{~0u, ~0u, ~0u, ~0u};
    if (k < nblk) ti4 = *reinterpret_cast<const u32x4 *>(mp.tix + k * 4);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int ti = __builtin_amdgcn_readfirstlane((int)ti4[u]);
      S.r[u] = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(tiles + (int64_t)(ti >= 0 ? ti : 0) * C::TBYTES), 0,
          ti >= 0 ? (int)C::TBYTES : 0, kBufferFlags);
    }
  };
  // unit ku of the wave's row groups: bf16, the 1 KB fragment block (row group,
  // chunk ku), lane l's 16 bytes at l * 16; fp8, the (row group, piece ku)
  // block of 512 NP bytes, lane l's 8 NP bytes at l * 8 NP
  const int voff = FP8 ? (wave * KU * 64 + lane) * 8 * NP : (RG * wave * KU * 64 + lane) * 16;
  auto load_chunk = [&](u32x4 (&dst)[RG][4], const Src4 &S, int ku) {
#pragma unroll
    for (int h = 0; h < RG; ++h)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (!FP8) {
          dst[h][u] = __builtin_amdgcn_raw_buffer_load_b128(S.r[u], voff, (h * KU + ku) * 1024, 0);
        } else if constexpr (NP == 2) {
          dst[h][u] = __builtin_amdgcn_raw_buffer_load_b128(S.r[u], voff, ku * 1024, 0);
        } else {
          const auto d2 = __builtin_amdgcn_raw_buffer_load_b64(S.r[u], voff, ku * 512, 0);
          dst[h][u] = u32x4{d2[0], d2[1], 0u, 0u};
        }
      }
  };
  // scale bytes of the lane's row (B/32 of them, one per chunk), fp8 only
  const int soff_lane = (wave * 16 + m16) * (B / 32);
  auto load_scales = [&](uint32_t (&sc)[4], const Src4 &S) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (B == 128)
        sc[u] = __builtin_amdgcn_raw_buffer_load_b32(S.r[u], soff_lane, B * B, 0);
      else if constexpr (B == 64)
        sc[u] = __builtin_amdgcn_raw_buffer_load_b16(S.r[u], soff_lane, B * B, 0);
      else
        sc[u] = __builtin_amdgcn_raw_buffer_load_b8(S.r[u], soff_lane, B * B, 0);
    }
  };

  const uint16_t *vtg = vt + (int64_t)g * D * tpad;
  auto dma_v = [&](char *dstbuf, int J) {
    dma_v_tile<B, D, C::VINST>(dstbuf, vtg, (int64_t)(gr - I + J) * B, wave, lane);
  };

  f32x4 acc[RG][D / 16];
#pragma unroll
  for (int h = 0; h < RG; ++h)
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) acc[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // coefficients of the lane's row in fp32 (zero for missing sources); fp8
  // tiles scale them per chunk by the tile's block scale
  float cf[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) cf[u] = u < ns ? mp.coef[u * B + wave * 16 * RG + m16] : 0.f;

  if (nblk > 0) {
    // queue of tile descriptors: S[k] for the (cur + k)-th union block
    Src4 S[DQ];
#pragma unroll
    for (int k = 0; k < DQ; ++k) src4(S[k], k);
    u32x4 ring[NR][RG][4];
    uint32_t sc[2][4];  // fp8 scale words of blocks with even / odd trip position
    // prologue: the first V tile and units 0 .. NR-2
    dma_v(vA, blk_J(0));
#pragma unroll
    for (int p = 0; p < NR - 1; ++p) {
      load_chunk(ring[p], S[p / KU], p % KU);
      if constexpr (FP8)
        if (p % KU == 0) load_scales(sc[(p / KU) & 1], S[p / KU]);
    }
    int cur = 0;  // list position of the block being multiplied
    bool done = false;
    while (!done) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (done) break;
        const char *vcur = (tb & 1) ? vB : vA;
        char *vnxt = (tb & 1) ? vA : vB;
        const int Jc = blk_J(cur), Jn = blk_J(cur + 1);
        // block start: this wave's part of V(Jc) has landed and its LDS reads of
        // the previous block are done; then the work-group barrier.  The wait
        // is a full drain: direct-to-LDS loads are not ordered with loads into
        // registers, so no partial count proves that V has landed.  Besides V
        // only this block's first chunk is in flight, and it is needed next.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        dma_v(vnxt, Jn >= 0 ? Jn : Jc);  // unconditional: static wait counts
#pragma unroll
        for (int ku = 0; ku < KU; ++ku) {
          const int pc = tb * KU + ku;          // unit position in the trip
          const int pf = ku + NR - 1;           // prefetched unit, relative to this block
          load_chunk(ring[(pc + NR - 1) % NR], S[pf / KU], pf % KU);
          if constexpr (FP8)
            if (pf % KU == 0) load_scales(sc[(tb + pf / KU) & 1], S[pf / KU]);
          // keep the prefetch ahead of this unit's work (the scheduler would
          // otherwise sink it next to its first use)
          __builtin_amdgcn_sched_barrier(0);
          const u32x4(&cr)[RG][4] = ring[pc % NR];
#pragma unroll
          for (int sub = 0; sub < NP; ++sub) {
            const int kc = ku * NP + sub;       // 32-key chunk of the block
            u32x4 a[RG];
#pragma unroll
            for (int h = 0; h < RG; ++h) {
              float mx[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) mx[e] = 0.f;
              if constexpr (!FP8) {
                // bf16 values widened exactly, fp32 FMAs
#pragma unroll
                for (int u = 0; u < 4; ++u)
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    mx[2 * e] = fmaf(cf[u], __uint_as_float(cr[h][u][e] << 16), mx[2 * e]);
                    mx[2 * e + 1] = fmaf(cf[u], __uint_as_float(cr[h][u][e] & 0xffff0000u), mx[2 * e + 1]);
                  }
              } else {
                // code_value * 2^(scale byte - 127), the scale folded into c
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                  const int sb = (int)((sc[tb & 1][u] >> (8 * kc)) & 0xffu);
                  const float c = __builtin_amdgcn_ldexpf(cf[u], sb - 127);
#pragma unroll
                  for (int w = 0; w < 2; ++w) {
                    const uint32_t codes = cr[h][u][2 * sub + w];
                    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(codes, false);
                    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(codes, true);
                    mx[4 * w + 0] = fmaf(c, lo[0], mx[4 * w + 0]);
                    mx[4 * w + 1] = fmaf(c, lo[1], mx[4 * w + 1]);
                    mx[4 * w + 2] = fmaf(c, hi[0], mx[4 * w + 2]);
                    mx[4 * w + 3] = fmaf(c, hi[1], mx[4 * w + 3]);
                  }
                }
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) a[h][e] = pack_bf16x2(mx[2 * e], mx[2 * e + 1]);
            }
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
              const u32x4 bv = v_frag<B>(vcur, nb * 16 + m16, kc * 4 + kg);
#pragma unroll
              for (int h = 0; h < RG; ++h)
                acc[h][nb] = mfma16_bf16(as_bf16x8(a[h]), as_bf16x8(bv), acc[h][nb]);
            }
          }
        }
        // advance the queue
#pragma unroll
        for (int k = 0; k + 1 < DQ; ++k) S[k] = S[k + 1];
        src4(S[DQ - 1], cur + DQ);
        ++cur;
        done = cur >= nblk;
      }
    }
    // drain the prefetches of blocks that do not exist before the wave ends
    __builtin_amdgcn_s_waitcnt(0);
  }

  float *ot = o + (int64_t)t * T * D;
#pragma unroll
  for (int h = 0; h < RG; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ip = I * B + wave * 16 * RG + 16 * h + 4 * kg + r;
      if (ip < L) {
        float *dst = ot + (tok0 + ip) * D + m16;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) __builtin_nontemporal_store(acc[h][nb][r], dst + nb * 16);
      }
    }
}

// ---------------------------------------------------------------------------
// k_apply_mix: targets with more than four sources (dense head mixing).
//
// One work-group per (query block, group of G consecutive targets); one wave
// per 16 query rows, for all G targets.  Every source tile chunk (16 rows x 32
// keys, one 1 KB fragment block) is loaded once per work-group and mixed into
// the G translated rows.  Each stored value is widened to fp32 exactly, once
// for the G targets, and every target adds it times its fp32 coefficient
// c = W[t,h] / kmass_h[i] with one FMA, so that the translated tile is rounded
// once, to bf16, as the MFMA operand.  (Mixed-sign weights cancel: a bf16
// coefficient's rounding would grow relative to the mixed value.)
//
// Per key block of the union, the block's V tiles (one per distinct V head of
// the group) load into LDS while the first 32-key chunk is mixed; a wait for
// those loads and a barrier; then each chunk's bf16 mix is multiplied with V
// on MFMA right after it is built; a barrier frees the V buffer for the next
// block.  The source chunks stream through a three-batch register ring, two
// batches ahead of the one being mixed.
// ---------------------------------------------------------------------------
template <int B, int D, int FMT>
struct ApplyMixCfg {
  static constexpr int G = (4 * D * B * 2 <= 64 * 1024) ? 4 : 2;  // targets per work-group
  static constexpr int NW = B / 16;                 // waves, 16 rows each
  static constexpr int NT = NW * 64;
  static constexpr int KC = B / 32;                 // 32-key chunks per key block
  static constexpr int VBYTES = D * B * 2;
  static constexpr int VINST = VBYTES / 1024 / NW;  // 1 KB direct loads per wave per V tile
  static constexpr int SB = 4;                      // sources per load batch (two pairs)
  static constexpr int NP = (FMT == MF_TILE_MXFP8 && B >= 64) ? 2 : 1;  // fp8 chunks per piece
  static constexpr int64_t TBYTES = tile_bytes(B, FMT);
  static_assert(VINST * 1024 * NW == VBYTES, "V tile must split into 1 KB wave loads");
  static_assert(G * VBYTES <= 64 * 1024, "V buffers must stay in the first 64 KB of LDS");
};
// Dynamic LDS of k_apply_mix (byte offsets): the V tiles [nvh][B * D] bf16
// (nvh = most distinct V heads in one target group), then src[Hs] int32,
// rbase[Hs] int64, wtab[Hs4][4] fp32 (weight of each source for each target of
// the group), bm[Hs][nbw], pc[Hs][nbw], uni[nbw], rtab[Hs4][B] fp32 (1 / kept
// mass of each row, 0 where none), ctab[Hs4][B][4] fp32 if used (bf16 maps: each
// source's coefficient W[t,h] / kmass_h[i] per row and target, formed once
// instead of in every chunk), blist[nbw * 32], counters.  The weight and
// coefficient tables run to Hs4 = Hs rounded up to a whole source batch, zero
// past the sources, so the mixing loop reads them without bounds tests.
inline size_t mix_smem(int B, int D, int Hs, int nbw, int nvh, bool ctab) {
  const size_t Hs4 = (size_t)(Hs + 3) / 4 * 4;
  size_t s = (size_t)nvh * B * D * 2;
  s += (size_t)Hs * (4 + 8) + Hs4 * 16;
  s += (size_t)Hs * nbw * 8 + (size_t)nbw * 4;
  s += Hs4 * B * 4;
  if (ctab) s += Hs4 * B * 16;
  s += (size_t)nbw * 32 * 4;
  s += 64 + 64;
  return s;
}

template <int B, int D, int FMT, bool CT>
__global__ __launch_bounds__(B * 4) __attribute__((amdgpu_waves_per_eu(2))) void k_apply_mix(
    const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
    const char *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs,
    int32_t NBR, int64_t T, const float *__restrict__ W, int32_t Ht, int32_t grp,
    const uint16_t *__restrict__ vt, const RowInfo *__restrict__ rows,
    const int32_t *__restrict__ sched, int32_t nrows, int32_t nbw, int64_t capacity,
    int32_t renorm, float *__restrict__ o, const int32_t *__restrict__ row_alias, int32_t nvmax,
    const char *__restrict__ zbuf, const int32_t *__restrict__ mix_flag) {
  using C = ApplyMixCfg<B, D, FMT>;
  constexpr int G = C::G, KC = C::KC, SB = C::SB, NP = C::NP;
  constexpr bool FP8 = FMT == MF_TILE_MXFP8;
  constexpr int LPB = FP8 ? 2 * SB : SB;  // vector-memory loads per source batch
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char *vbuf = smem;  // first in LDS
  const int o_src = nvmax * C::VBYTES;
  const int o_rbase = (o_src + Hs * 4 + 7) & ~7;
  const int Hs4 = (Hs + 3) / 4 * 4;
  static_assert(C::SB == 4, "tables are padded to whole batches of four sources");
  const int o_wt = o_rbase + Hs * 8;
  const int o_bm = o_wt + Hs4 * 16;
  const int o_pc = o_bm + Hs * nbw * 4;
  const int o_uni = o_pc + Hs * nbw * 4;
  const int o_rt = o_uni + nbw * 4;
  const int o_ct = o_rt + Hs4 * B * 4;
  const int o_bl = o_ct + (CT ? Hs4 * B * 16 : 0);
  const int o_misc = o_bl + nbw * 32 * 4;
  int32_t *src = reinterpret_cast<int32_t *>(smem + o_src);
  int64_t *rbase = reinterpret_cast<int64_t *>(smem + o_rbase);
  float *wtab = reinterpret_cast<float *>(smem + o_wt);
  uint32_t *bm = reinterpret_cast<uint32_t *>(smem + o_bm);
  int32_t *pc = reinterpret_cast<int32_t *>(smem + o_pc);
  uint32_t *uni = reinterpret_cast<uint32_t *>(smem + o_uni);
  float *rtab = reinterpret_cast<float *>(smem + o_rt);
  f32x4 *ctab = reinterpret_cast<f32x4 *>(smem + o_ct);
  int32_t *blist = reinterpret_cast<int32_t *>(smem + o_bl);
  int32_t *misc = reinterpret_cast<int32_t *>(smem + o_misc);  // [0] ns, [1..G] active

  // no target with more than four sources (the pairing pass found none): done
  if (mix_flag && *mix_flag == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m16 = lane & 15, kg = lane >> 4;
  const int ngrp = (Ht + G - 1) / G;
  // work-group id -> (schedule position, target group), XCD-aware as in k_apply4
  const int x = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
  const int round = kx / ngrp, tg = kx % ngrp;
  const int pos = round * kXcds + ((round & 1) ? (kXcds - 1 - x) : x);
  if (pos >= nrows) return;
  const int gr = sched[pos];
  const RowInfo ri = rows[gr];
  const int I = ri.blk, L = ri.len;
  const int n = I + 1;
  const int64_t tok0 = (int64_t)ri.start;
  const int64_t tpad = (int64_t)NBR * B;
  const int ga = row_alias ? row_alias[gr] : gr;
  const int grm = (ga >= 0 && ga < NBR) ? ga : gr;  // BSR row (shared block-rows)
  const int t0 = tg * G;

  // ---- set-up: active targets, source union, weights, kept bitmaps ---------
  if (tid < 64) {
    // wave 0, 64 heads at a time: source counts of the G targets (those with at
    // most four sources are k_apply4's), then the union of the active targets'
    // sources compacted by ballot in ascending head order
    bool act[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      int cnt = 0;
      if (t0 + g < Ht)
        for (int h0 = 0; h0 < Hs; h0 += 64) {
          const int h = h0 + tid;
          cnt += __popcll(wave_ballot(h < Hs && W[(int64_t)(t0 + g) * Hs + h] != 0.f));
        }
      act[g] = cnt > 4;
    }
    int ns = 0;
    for (int h0 = 0; h0 < Hs; h0 += 64) {
      const int h = h0 + tid;
      float w[G];
      bool any = false;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        w[g] = (act[g] && h < Hs) ? W[(int64_t)(t0 + g) * Hs + h] : 0.f;
        any |= w[g] != 0.f;
      }
      const uint64_t mask = wave_ballot(any);
      if (any) {
        const int q = ns + lanes_below(mask);
        src[q] = h;
        rbase[q] = row_ptr[(int64_t)h * NBR + grm];
#pragma unroll
        for (int g = 0; g < G; ++g) wtab[q * 4 + g] = w[g];
#pragma unroll
        for (int g = G; g < 4; ++g) wtab[q * 4 + g] = 0.f;
      }
      ns += __popcll(mask);
    }
    if (tid == 0) {
      misc[0] = ns;
#pragma unroll
      for (int g = 0; g < G; ++g) misc[1 + g] = act[g];
    }
  }
  for (int i = tid; i < Hs * nbw; i += C::NT) bm[i] = 0u;
  __syncthreads();
  const int ns = __builtin_amdgcn_readfirstlane(misc[0]);
  if (ns == 0) return;
  const int ns4 = (ns + SB - 1) / SB * SB;  // whole batches; tables zero past ns
  for (int i = ns * 4 + tid; i < ns4 * 4; i += C::NT) wtab[i] = 0.f;
  for (int q = 0; q < ns; ++q) {
    // entries past the capacity of an overflowed map are treated as missing
    const int64_t b0 = rbase[q], e0 = min(row_ptr[(int64_t)src[q] * NBR + grm + 1], capacity);
    for (int64_t idx = b0 + tid; idx < e0; idx += C::NT) {
      const int J = col_idx[idx];
      atomicOr(&bm[q * nbw + (J >> 5)], 1u << (J & 31));
    }
  }
  for (int idx = tid; idx < ns4 * B; idx += C::NT) {
    const int q = idx / B, il = idx % B;
    const int ip = I * B + il;
    float r = 0.f;
    if (q < ns && ip < L) {
      if (renorm) {
        const float km = kept_mass[(int64_t)src[q] * T + tok0 + ip];
        r = km > 0.f ? 1.f / km : 0.f;
      } else {
        r = 1.f;
      }
    }
    rtab[q * B + il] = r;
  }
  __syncthreads();
  if constexpr (CT) {
    // fp32 coefficients of every source, row and target (0 past the sources)
    for (int idx = tid; idx < ns4 * B; idx += C::NT) {
      const int u = idx / B, il = idx % B;
      const float r = rtab[u * B + il];
      f32x4 cq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < G; ++g) cq[g] = wtab[u * 4 + g] * r;
      ctab[u * B + il] = cq;
    }
    __syncthreads();
  }
  const int nw_row = (n + 31) / 32;
  for (int q = tid; q < ns; q += C::NT) {
    int run = 0;
    for (int w = 0; w < nw_row; ++w) {
      pc[q * nbw + w] = run;
      run += __popc(bm[q * nbw + w]);
    }
  }
  if (tid < nw_row) {
    uint32_t u = 0u;
    for (int q = 0; q < ns; ++q) u |= bm[q * nbw + tid];
    uni[tid] = u;
  }
  __syncthreads();
  // union block list
  for (int J = tid; J < n; J += C::NT) {
    const uint32_t w = uni[J >> 5];
    if (!((w >> (J & 31)) & 1u)) continue;
    int k = __popc(w & ((1u << (J & 31)) - 1u));
    for (int i = 0; i < (J >> 5); ++i) k += __popc(uni[i]);
    blist[k] = J;
  }
  int nblk = 0;
  for (int i = 0; i < nw_row; ++i) nblk += __popc(uni[i]);
  __syncthreads();
  nblk = __builtin_amdgcn_readfirstlane(nblk);

  bool act[G];
#pragma unroll
  for (int g = 0; g < G; ++g) act[g] = misc[1 + g] != 0;
  const int gv0 = t0 / grp;                       // V head of the group's first target
  int nvh = 0;                                    // distinct V heads of the group
#pragma unroll
  for (int g = 0; g < G; ++g)
    if (t0 + g < Ht) nvh = (t0 + g) / grp - gv0 + 1;

  int vho[G];  // LDS offset of each target's V tile (a target past Ht: any)
#pragma unroll
  for (int g = 0; g < G; ++g) vho[g] = min((t0 + g) / grp - gv0, nvh - 1) * C::VBYTES;
  const int r0 = wave * 16 + m16;                 // lane row inside the block
  // lane's bytes of chunk kc: bf16 16 bytes at loff + kc * 1024; fp8 8 bytes at
  // loff + (kc / NP) * 512 NP + (kc % NP) * 8, and its row's scale byte
  const int loff = FP8 ? (wave * (KC / NP) * 64 + lane) * 8 * NP : (wave * KC * 64 + lane) * 16;
  const int soff = B * B + r0 * (B / 32);
  f32x4 acc[G][D / 16];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) acc[g][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nst = KC * ((ns + SB - 1) / SB);  // source batches per key block
  for (int kb = 0; kb < nblk; ++kb) {
    const int J = __builtin_amdgcn_readfirstlane(blist[kb]);
    // tile index of every source at J, lane u holding sources u and u + 64
    // as the tile's address (two 32-bit halves); a source without a tile at J,
    // or past the union, points at the zero block
    uint32_t tlo[2], thi[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int u = lane + 64 * hh;
      const char *a = zbuf;
      if (u < ns) {
        const uint32_t word = bm[u * nbw + (J >> 5)];
        if ((word >> (J & 31)) & 1u) {
          const int64_t tix = rbase[u] + pc[u * nbw + (J >> 5)] + __popc(word & ((1u << (J & 31)) - 1u));
          if (tix < capacity) a = tiles + tix * C::TBYTES;
        }
      }
      tlo[hh] = (uint32_t)reinterpret_cast<uintptr_t>(a);
      thi[hh] = (uint32_t)(reinterpret_cast<uintptr_t>(a) >> 32);
    }
    const uint32_t zlo = (uint32_t)reinterpret_cast<uintptr_t>(zbuf);
    const uint32_t zhi = (uint32_t)(reinterpret_cast<uintptr_t>(zbuf) >> 32);
    // V tiles of this block for every distinct V head of the group
    const int64_t col0 = (int64_t)(gr - I + J) * B;
    for (int vh = 0; vh < nvh; ++vh)
      dma_v_tile<B, D, C::VINST>(vbuf + vh * C::VBYTES, vt + (int64_t)(gv0 + vh) * D * tpad, col0,
                                 wave, lane);
    asm volatile("" ::: "memory");  // the V loads issue before this block's tile loads

    // Loads from a wave-uniform 64-bit base (the tile, or the zero block for a
    // missing tile, a source past the union or a batch past the block: `zero`)
    // plus a 32-bit lane offset, so a missing tile costs no branch and no
    // per-lane address arithmetic.
    // A batch never straddles source 64 (batches start at multiples of SB), so
    // its address pair is chosen once per batch, then read lane by lane.
    auto load_batch = [&](u32x4 (&d)[SB], uint32_t (&sb)[SB], int kc, int u0, bool zero) {
      const uint32_t blo = zero ? zlo : (u0 < 64 ? tlo[0] : tlo[1]);
      const uint32_t bhi = zero ? zhi : (u0 < 64 ? thi[0] : thi[1]);
#pragma unroll
      for (int e = 0; e < SB; ++e) {
        const int l = (u0 + e) & 63;
        const u32x2_t a2 = {(uint32_t)__builtin_amdgcn_readlane(blo, l), (uint32_t)__builtin_amdgcn_readlane(bhi, l)};
        const gchar *tb = reinterpret_cast<const gchar *>(__builtin_bit_cast(uint64_t, a2));
        if constexpr (!FP8) {
          d[e] = *reinterpret_cast<const gu32x4 *>(tb + (uint32_t)(loff + kc * 1024));
          sb[e] = 0u;
        } else {
          const auto c2 =
              *reinterpret_cast<const gu32x2 *>(tb + (uint32_t)(loff + (kc / NP) * 512 * NP + (kc % NP) * 8));
          d[e] = u32x4{c2[0], c2[1], 0u, 0u};
          sb[e] = *(tb + (uint32_t)(soff + kc));
        }
      }
    };
    // mix one batch of SB sources (u0 ..) into mx in fp32: each stored tile
    // value widened exactly (bf16 by a shift or mask, E4M3 by v_cvt_pk_f32_fp8)
    // and multiplied with its fp32 coefficient W[t,h] / kmass_h[i], so the only
    // rounding of the translated tile is the one to bf16 below
    auto mix_batch = [&](float (&mx)[G][8], const u32x4 (&cur)[SB], const uint32_t (&scur)[SB], int u0) {
#pragma unroll
      for (int b = 0; b < SB; ++b) {
        const int u = u0 + b;
        float cf[G];
        if constexpr (CT) {
          // the source's coefficients from the table (zero past the sources)
          const f32x4 cq = ctab[u * B + r0];
#pragma unroll
          for (int g = 0; g < G; ++g) cf[g] = cq[g];
        } else {
          float r = rtab[u * B + r0];
          if constexpr (FP8) {
            // the block scale 2^(byte - 127) folded into the coefficients
            r = __builtin_amdgcn_ldexpf(r, (int)scur[b] - 127);
          }
#pragma unroll
          for (int g = 0; g < G; ++g) cf[g] = wtab[u * 4 + g] * r;
        }
        float x[8];
        if constexpr (!FP8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(cur[b][e] << 16);
            x[2 * e + 1] = __uint_as_float(cur[b][e] & 0xffff0000u);
          }
        } else {
          // code byte k of word w is element 4 w + k
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)cur[b][w], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)cur[b][w], true);
            x[4 * w + 0] = lo[0];
            x[4 * w + 1] = lo[1];
            x[4 * w + 2] = hi[0];
            x[4 * w + 3] = hi[1];
          }
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int e = 0; e < 8; ++e) mx[g][e] = fmaf(cf[g], x[e], mx[g][e]);
      }
    };
    // chunk kc mixed: round to bf16 and multiply with V on MFMA
    auto finish_chunk = [&](float (&mx)[G][8], int kc) {
      u32x4 amix[G];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) amix[g][e] = pack_bf16x2(mx[g][2 * e], mx[g][2 * e + 1]);
      if (kc == 0) {
        // V tiles landed in every wave.  Vector-memory loads retire in issue
        // order and the V loads went out before any tile load of this block, so
        // allowing the two batches loaded after this one (LPB loads each) to
        // stay in flight still covers them.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPB));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
      // each 16-column slice: the G V fragments read together, then the MFMAs
      // (fp8 maps, whose mixing holds more registers: one fragment at a time)
#pragma unroll
      for (int nb = 0; nb < D / 16; ++nb) {
        if constexpr (!FP8) {
          u32x4 bq[G];
#pragma unroll
          for (int g = 0; g < G; ++g) bq[g] = v_frag<B>(vbuf + vho[g], nb * 16 + m16, kc * 4 + kg);
#pragma unroll
          for (int g = 0; g < G; ++g)
            acc[g][nb] = mfma16_bf16(as_bf16x8(amix[g]), as_bf16x8(bq[g]), acc[g][nb]);
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const u32x4 bv = v_frag<B>(vbuf + vho[g], nb * 16 + m16, kc * 4 + kg);
            acc[g][nb] = mfma16_bf16(as_bf16x8(amix[g]), as_bf16x8(bv), acc[g][nb]);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[g][e] = 0.f;
    };

    // The key block's KC * nsb source batches run as one stream through a ring
    // of three register buffers: the batch two steps ahead loads while the
    // current one is mixed, across the chunk boundary too.  The ring position
    // is static (the loop is unrolled by three), so nothing is copied.  Every
    // step issues its loads, past the last batch through zero-length
    // descriptors, so the number of loads between a batch's issue and its use
    // is fixed and the wait before the use is exact (a conditional load would
    // make it a full drain).
    float mx[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx[g][e] = 0.f;
    u32x4 ring[3][SB];
    uint32_t sring[3][SB];
    int lkc = 0, lu0 = 0;  // next batch to load
    auto next_load = [&](u32x4 (&d)[SB], uint32_t (&sb)[SB]) {
      load_batch(d, sb, lkc < KC ? lkc : 0, lu0, lkc >= KC);
      lu0 += SB;
      if (lu0 >= ns) { lu0 = 0; ++lkc; }
    };
    next_load(ring[0], sring[0]);
    next_load(ring[1], sring[1]);
    int ckc = 0, cu0 = 0;  // batch being mixed
    for (int s0 = 0; s0 < nst; s0 += 3) {
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        if (s0 + r >= nst) break;
        next_load(ring[(r + 2) % 3], sring[(r + 2) % 3]);
        mix_batch(mx, ring[r], sring[r], cu0);
        cu0 += SB;
        if (cu0 >= ns) {
          finish_chunk(mx, ckc);
          cu0 = 0;
          ++ckc;
        }
      }
    }
    // every wave's reads of V done before the next block's loads overwrite it
    __syncthreads();
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (!act[g]) continue;
    float *ot = o + (int64_t)(t0 + g) * T * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ip = I * B + wave * 16 + 4 * kg + r;
      if (ip < L) {
        float *dst = ot + (tok0 + ip) * D + m16;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) __builtin_nontemporal_store(acc[g][nb][r], dst + nb * 16);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Target pairs for k_apply_pair.
//
// Targets with at most four sources are paired so that one work-group loads
// each source tile of both once and mixes it into whichever of the two uses
// it.  Greedy and deterministic: the lowest-numbered target not yet placed
// takes the unplaced target whose sources add the fewest new ones (lowest
// number on ties).  Any two such targets fit (at most 8 sources).  Targets with
// more than four sources are left to k_apply_mix.
//
// gtab[0] = number of groups; group q holds targets gtab[1 + 2q], gtab[2 + 2q]
// (-1 for an empty slot); gtab[kMixFlag] = 1 if some target has more than four
// sources (k_apply_mix has work), else 0.  With pair == 0 every such target
// forms a group of its own.  One wave; Ht <= kMaxTargets, Hs <= kMixMaxSources.
// ---------------------------------------------------------------------------
constexpr int kPairT = 2;          // targets per work-group of the translated retrieval
constexpr int kMaxTargets = 1024;
constexpr int kMixMaxSources = 128;
constexpr int kMixFlag = 1 + 2 * kMaxTargets;

__global__ __launch_bounds__(64) void k_pairs(const float *__restrict__ W, int32_t Ht, int32_t Hs,
                                              int32_t pair, int32_t *__restrict__ gtab) {
  __shared__ uint32_t msk[kMaxTargets][4];
  __shared__ uint8_t state[kMaxTargets];  // 0 free, 1 placed, 2 not handled here
  const int lane = threadIdx.x;
  for (int t = lane; t < Ht; t += 64) {
    uint32_t m[4] = {0u, 0u, 0u, 0u};
    for (int h = 0; h < Hs; ++h)
      if (W[(int64_t)t * Hs + h] != 0.f) m[h >> 5] |= 1u << (h & 31);
#pragma unroll
    for (int w = 0; w < 4; ++w) msk[t][w] = m[w];
    const int cnt = __popc(m[0]) + __popc(m[1]) + __popc(m[2]) + __popc(m[3]);
    state[t] = cnt <= 4 ? 0 : 2;
  }
  __syncthreads();
  {
    bool mix = false;
    for (int t = lane; t < Ht; t += 64) mix |= state[t] == 2;
    const uint64_t any = wave_ballot(mix);
    if (lane == 0) gtab[kMixFlag] = any != 0ull ? 1 : 0;
  }
  auto wave_min = [](int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
    return v;
  };
  int np = 0;
  for (;;) {
    int first = INT32_MAX;
    for (int t = lane; t < Ht; t += 64)
      if (state[t] == 0) first = min(first, t);
    first = wave_min(first);
    if (first == INT32_MAX) break;
    __syncthreads();
    if (lane == 0) state[first] = 1;
    __syncthreads();
    int best = INT32_MAX;
    for (int t = lane; pair && t < Ht; t += 64) {
      if (state[t] != 0) continue;
      int nu = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) nu += __popc(msk[first][w] | msk[t][w]);
      best = min(best, nu * kMaxTargets + t);
    }
    best = wave_min(best);
    const int second = best == INT32_MAX ? -1 : best % kMaxTargets;
    __syncthreads();
    if (lane == 0 && second >= 0) state[second] = 1;
    if (lane == 0) {
      gtab[1 + 2 * np] = first;
      gtab[2 + 2 * np] = second;
    }
    __syncthreads();
    ++np;
  }
  if (lane == 0) gtab[0] = np;
}

// ---------------------------------------------------------------------------
// Query-block pairs: block-rows I and I - 1 of one sequence, counted from the
// last block-row of the sequence (or of its query window) down, so a sequence
// with an odd number of block-rows ends in a single one.  Listed lead block
// (the longer) descending, from the longest-first schedule; psched[2p] is the
// lead's global block-row, psched[2p + 1] the partner's or -1.  One work-group.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_pair_sched(const RowInfo *__restrict__ rows,
                                                     const int32_t *__restrict__ sched,
                                                     int32_t NBR, int32_t B,
                                                     const int32_t *__restrict__ window,
                                                     int32_t *__restrict__ psched,
                                                     u32x4 *__restrict__ vzero) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t base;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // the zero block: the V row the retrieval reads past a sequence's end, and
  // the tile a source without one at some key block reads (kZeroBytes)
  for (int i = tid; i < kZeroBytes / 16; i += 1024) vzero[i] = u32x4{0u, 0u, 0u, 0u};
  if (tid == 0) base = 0;
  __syncthreads();
  for (int p0 = 0; p0 < NBR; p0 += 1024) {
    const int p = p0 + tid;
    int gr = -1, partner = -1;
    bool lead = false;
    if (p < NBR) {
      gr = sched[p];
      const RowInfo ri = rows[gr];
      int lo = 0, hi = (ri.len + B - 1) / B - 1;  // block-rows of the sequence (or window)
      if (window) {
        const int a = window[2 * ri.seq], e = window[2 * ri.seq + 1];
        lo = a / B;
        hi = (e + B - 1) / B - 1;
      }
      if (ri.blk >= lo && ri.blk <= hi) {
        lead = ((hi - ri.blk) & 1) == 0;
        partner = ri.blk - 1 >= lo ? gr - 1 : -1;
      }
    }
    const uint64_t mask = wave_ballot(lead);
    if (lane == 0) wsum[wave] = __popcll(mask);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (lead) {
      const int q = off + lanes_below(mask);
      psched[2 * q] = gr;
      psched[2 * q + 1] = partner;
    }
    __syncthreads();
    if (tid == 0) {
      int tot = 0;
      for (int w = 0; w < 16; ++w) tot += wsum[w];
      base += tot;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// k_apply_pair: targets with at most four sources, one work-group per (query
// block pair, target pair).
//
// The work-group covers 2B rows (two adjacent query blocks of one sequence)
// for two targets.  Per 16-key step of each key block in the union of the
// kept sets (both query blocks, every source of either target), it stages in
// LDS, once: each source's slice of both query blocks' tiles (2B rows x 16
// keys) and each target's V slice (16 keys x D, one V for both query blocks:
// they are of one sequence).  Wave (a, part) rebuilds 64 rows of target a's
// translated tile from its (at most four) sources,
//   A~_a[i, j] = sum_b c_ab[i] A_src(a,b)[i, j],   c_ab[i] = W[t_a, h] / kmass_h[i],
// in fp32 (bf16 values widened exactly, fp32 coefficients, fp32 fused
// multiply-adds), rounds it to bf16 once and multiplies it with V on 32x32x16
// MFMAs into fp32 accumulators; each V operand read serves two 32-row blocks.
// The translated map never leaves registers.
//
// Loads go straight from memory to LDS (buffer loads with an LDS target), two
// stages: step q + 1 moves into one while step q is computed from the other;
// one barrier per step.  A wave loads, for U / (waves per query block) of the
// source slots, all rows of one query block, so per key block it builds only
// that many tile descriptors (zero-length where a source kept no tile) plus
// one per V piece; steps inside the block move the scalar offset only.
//
// Order: consecutive work-group ids go to the XCDs in turn.  One XCD runs all
// target pairs of one query-block pair at a time (32 work-groups for 64
// targets), so they start together and read each shared source tile from that
// XCD's L2.  The key blocks are walked upwards or downwards by the lead block's
// index (I / 16 odd: downwards), so the query blocks in flight on all XCDs,
// which start in rounds of 16 longest-first, stay close in J and share V
// through the memory-side cache.
// ---------------------------------------------------------------------------
constexpr int kPairVPolicy = 0;    // cache policy of the V loads

template <int B, int D, int TP>
struct PairCfg {
  static constexpr int U = 4 * TP;                      // source slots (their union)
  static constexpr int ROWS = 2 * B;                    // rows of a work-group
  static constexpr int WPT = ROWS >= 128 ? ROWS / 64 : 1;   // waves per target
  static constexpr int NW = TP * WPT;
  static constexpr int NT = NW * 64;
  static constexpr int RB = ROWS / (32 * WPT);          // 32-row blocks per wave
  static constexpr int NB = D / 32;                     // 32-column blocks
  static constexpr int KS = B / 16;                     // 16-key steps per key block
  static constexpr int SRC_BYTES = ROWS * 32;           // a source's slice of one step
  static constexpr int V_BYTES = D * 32;                // a target's V slice of one step
  static constexpr int V_OFF = U * SRC_BYTES;
  static constexpr int STAGE = V_OFF + TP * V_BYTES;
  static constexpr int WQ = NW / 2;                     // waves per query block
  static constexpr int NBQ = B / 32;                    // 1 KB blocks of a query block's slice
  static constexpr int SPW = U / WQ;                    // slots whose pieces a wave loads
  static constexpr int SP = SPW * NBQ;                  // source pieces per lane
  static constexpr int VPIECES = TP * V_BYTES / 16;
  static constexpr int VP = (VPIECES + NT - 1) / NT;                    // V pieces per lane
  static_assert(NW % 2 == 0 && U % WQ == 0 && SP == 8, "every wave loads 8 source blocks per step");
  static_assert(RB == 2 && (2 * D) % 64 == 0 && KS % 2 == 0, "layout assumptions");
};

// LDS tables after the two stages (byte offsets)
struct PairTables {
  int rbase, rend, usrc, smap, sw, sns, stgt, umask, misc, bm, pc, uni, upre, blist, total;
};
template <int B, int D, int TP>
__host__ __device__ inline PairTables pair_tables(int nbw) {
  using C = PairCfg<B, D, TP>;
  PairTables t;
  int o = 2 * C::STAGE;
  t.rbase = o; o += 2 * C::U * 8;
  t.rend = o; o += 2 * C::U * 8;
  t.usrc = o; o += C::U * 4;
  t.smap = o; o += 8 * 4;
  t.sw = o; o += 8 * 4;
  t.sns = o; o += 4 * 4;
  t.stgt = o; o += 4 * 4;
  t.umask = o; o += 4 * 4;
  t.misc = o; o += 4 * 4;
  t.bm = o; o += 2 * C::U * nbw * 4;
  t.pc = o; o += 2 * C::U * nbw * 4;
  t.uni = o; o += nbw * 4;
  t.upre = o; o += nbw * 4;
  t.blist = o; o += nbw * 32 * 4;
  t.total = o;
  return t;
}

template <int B, int D, int TP>
__global__ __launch_bounds__((PairCfg<B, D, TP>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
void k_apply_pair(const int64_t *__restrict__ row_ptr, const int32_t *__restrict__ col_idx,
                  const char *__restrict__ tiles, const float *__restrict__ kept_mass, int32_t Hs,
                  int32_t NBR, int64_t T, const float *__restrict__ W, int32_t grp, VSrc vs,
                  const char *__restrict__ vzero, const RowInfo *__restrict__ rows,
                  const int32_t *__restrict__ psched, int32_t npairs, int32_t nbw,
                  int64_t capacity, int32_t renorm, float *__restrict__ o,
                  const int32_t *__restrict__ row_alias, const int32_t *__restrict__ gtab,
                  int32_t ngmax) {
  using C = PairCfg<B, D, TP>;
  constexpr int RB = C::RB, NB = C::NB, KS = C::KS, VP = C::VP, U_MAX = C::U;
  constexpr int SPW = C::SPW, NBQ = C::NBQ;
  constexpr int64_t TBYTES = (int64_t)B * B * 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const PairTables tb = pair_tables<B, D, TP>(nbw);
  int64_t *rbase = reinterpret_cast<int64_t *>(smem + tb.rbase);  // [2][U] first tile of the row
  int64_t *rend = reinterpret_cast<int64_t *>(smem + tb.rend);    // [2][U] end (capped)
  int32_t *usrc = reinterpret_cast<int32_t *>(smem + tb.usrc);    // [U] source head
  int32_t *smap = reinterpret_cast<int32_t *>(smem + tb.smap);    // [TP][4] slot of source b of target a
  float *sw = reinterpret_cast<float *>(smem + tb.sw);            // [TP][4] weight
  int32_t *sns = reinterpret_cast<int32_t *>(smem + tb.sns);      // [TP] source count
  int32_t *stgt = reinterpret_cast<int32_t *>(smem + tb.stgt);    // [TP] target or -1
  uint32_t *umask = reinterpret_cast<uint32_t *>(smem + tb.umask);
  int32_t *misc = reinterpret_cast<int32_t *>(smem + tb.misc);    // [0] union blocks
  uint32_t *bm = reinterpret_cast<uint32_t *>(smem + tb.bm);      // [2][U][nbw] kept bitmaps
  int32_t *pc = reinterpret_cast<int32_t *>(smem + tb.pc);        // [2][U][nbw] popcount prefix
  uint32_t *uni = reinterpret_cast<uint32_t *>(smem + tb.uni);
  int32_t *upre = reinterpret_cast<int32_t *>(smem + tb.upre);
  int32_t *blist = reinterpret_cast<int32_t *>(smem + tb.blist);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // work-group -> (query-block pair, target group)
  const int x = blockIdx.x % kXcds, kx = blockIdx.x / kXcds;
  const int round = kx / ngmax, gi = kx % ngmax;
  const int pidx = round * kXcds + ((round & 1) ? (kXcds - 1 - x) : x);
  if (pidx >= npairs) return;
  if (gi >= gtab[0]) return;
  int grq[2], Iq[2], grmq[2];
  grq[0] = uni32(psched[2 * pidx]);
  grq[1] = uni32(psched[2 * pidx + 1]);
  const RowInfo r0 = rows[grq[0]];
  const int L = uni32(r0.len);
  const int seq = uni32(r0.seq);
  const int64_t tok0 = (int64_t)uni32(r0.start);
  Iq[0] = uni32(r0.blk);
  Iq[1] = Iq[0] - 1;                                   // partner (if any) is the block below
  const bool has1 = grq[1] >= 0;
  const int grow0 = grq[0] - Iq[0];                    // the sequence's first global block-row
  const int n = Iq[0] + 1;                             // key blocks J <= I of the lead
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int g = b == 0 ? grq[0] : (has1 ? grq[1] : grq[0]);
    const int ga = row_alias ? uni32(row_alias[g]) : g;
    grmq[b] = (ga >= 0 && ga < NBR) ? ga : g;
  }
  const bool desc = ((Iq[0] >> 4) & 1) != 0;

  // ---- set-up: targets, their sources, the source union -------------------
  if (tid < 4) umask[tid] = 0u;
  if (tid < TP) stgt[tid] = gtab[1 + 2 * gi + tid];
  for (int i = tid; i < 2 * U_MAX * nbw; i += C::NT) bm[i] = 0u;
  __syncthreads();
  if (wave < TP) {
    const int t = stgt[wave];
    int ns = 0;
    if (t >= 0)
      for (int h0 = 0; h0 < Hs; h0 += 64) {
        const int h = h0 + lane;
        const float w = h < Hs ? W[(int64_t)t * Hs + h] : 0.f;
        const uint64_t mask = wave_ballot(w != 0.f);
        if (w != 0.f) {
          const int q = ns + lanes_below(mask);
          if (q < 4) {
            smap[wave * 4 + q] = h;   // head for now, slot below
            sw[wave * 4 + q] = w;
          }
          atomicOr(&umask[h >> 5], 1u << (h & 31));
        }
        ns += __popcll(mask);
      }
    if (lane == 0) sns[wave] = min(ns, 4);
  }
  __syncthreads();
  const uint32_t um0 = umask[0], um1 = umask[1], um2 = umask[2], um3 = umask[3];
  auto slot_of = [&](int h) {  // rank of head h in the union
    const uint32_t below = (h & 31) ? ((1u << (h & 31)) - 1u) : 0u;
    const int w = h >> 5;
    int r = __popc((w == 0 ? um0 : w == 1 ? um1 : w == 2 ? um2 : um3) & below);
    if (w > 0) r += __popc(um0);
    if (w > 1) r += __popc(um1);
    if (w > 2) r += __popc(um2);
    return r;
  };
  const int U = __popc(um0) + __popc(um1) + __popc(um2) + __popc(um3);  // <= U_MAX
  for (int h = tid; h < kMixMaxSources; h += C::NT) {
    if ((umask[h >> 5] >> (h & 31)) & 1u) {
      const int u = slot_of(h);
      usrc[u] = h;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bool on = b == 0 || has1;
        rbase[b * U_MAX + u] = on ? row_ptr[(int64_t)h * NBR + grmq[b]] : 0;
        rend[b * U_MAX + u] = on ? min(row_ptr[(int64_t)h * NBR + grmq[b] + 1], capacity) : 0;
      }
    }
  }
  __syncthreads();
  if (tid < 4 * TP) {
    const int a = tid >> 2, b = tid & 3;
    smap[tid] = b < sns[a] ? slot_of(smap[tid]) : 0;
  }
  // kept bitmaps of the union's sources, both query blocks
  for (int bu = 0; bu < 2 * U; ++bu) {
    const int b = bu / U, u = bu % U;
    const int64_t e = rend[b * U_MAX + u];
    for (int64_t idx = rbase[b * U_MAX + u] + tid; idx < e; idx += C::NT) {
      const int J = col_idx[idx];
      atomicOr(&bm[(b * U_MAX + u) * nbw + (J >> 5)], 1u << (J & 31));
    }
  }
  __syncthreads();
  const int nw_row = (n + 31) / 32;
  for (int i = tid; i < 2 * U_MAX * nw_row; i += C::NT) {
    // popcount prefix of each bitmap (its tile rank before word w)
    const int bu = i / nw_row, w = i % nw_row;
    int run = 0;
    for (int v = 0; v < w; ++v) run += __popc(bm[bu * nbw + v]);
    pc[bu * nbw + w] = run;
  }

  for (int w = tid; w < nw_row; w += C::NT) {
    uint32_t v = 0u;
    for (int bu = 0; bu < 2 * U_MAX; ++bu) v |= bm[bu * nbw + w];
    uni[w] = v;
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nw_row; ++w) {
      upre[w] = run;
      run += __popc(uni[w]);
    }
    misc[0] = run;
  }
  __syncthreads();
  const int nblk = uni32(misc[0]);
  for (int J = tid; J < n; J += C::NT) {
    const uint32_t w = uni[J >> 5];
    if ((w >> (J & 31)) & 1u) blist[upre[J >> 5] + __popc(w & ((1u << (J & 31)) - 1u))] = J;
  }
  __syncthreads();

  // ---- per-wave constants ---------------------------------------------------
  const int a = wave % TP, part = wave / TP;           // target slot, 64-row part
  const int ta = uni32(stgt[a]);
  const int nsa = uni32(sns[a]);
  const int r32 = lane & 31;
  // coefficients c[rb][b] of the lane's rows (zero past the sequence end, for
  // absent sources and where the kept mass is 0)
  float cf[RB][4];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = 64 * part + 32 * rb + r32;           // row of the work-group
    const int q = row / B;                               // its query block
    const int ip = Iq[q] * B + row % B;                  // row inside the sequence
    const bool live = q == 0 || has1;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float c = 0.f;
      if (ta >= 0 && live && b < nsa && ip < L) {
        const int h = usrc[smap[a * 4 + b]];
        const float w = sw[a * 4 + b];
        if (renorm) {
          const float km = kept_mass[(int64_t)h * T + tok0 + ip];
          c = km > 0.f ? w / km : 0.f;
        } else {
          c = w;
        }
      }
      cf[rb][b] = c;
    }
  }
  int soff_b[4];  // LDS offset of the slot of each source of target a (uniform)
#pragma unroll
  for (int b = 0; b < 4; ++b) soff_b[b] = uni32(smap[a * 4 + b]) * C::SRC_BYTES;
  // LDS layouts are lane-linear, so every read and write of a wave covers
  // contiguous bytes (no bank conflicts): a source slice is ROWS/32 blocks of
  // 1 KB, block k holding (key half h, row r of the block) at (32 h + r) * 16,
  // the A operand of a 32x32x16 MFMA for lane 32 h + r; a V slice is D/32
  // blocks of 1 KB, block nb holding (key half h, column d of the block) at
  // (32 h + d) * 16, the B operand for lane 32 h + d.
  int aoff[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) aoff[rb] = (2 * part + rb) * 1024 + lane * 16;
  const int boff = C::V_OFF + a * C::V_BYTES + (lane >> 5) * 8 * (D * 2) + r32 * NB * 2;

  // load pieces, moved straight from memory to LDS (each load instruction of a
  // wave fills 64 consecutive 16-byte LDS positions).  A wave loads, for SPW
  // slots, every 32-row block of one query block qw: piece (slot wq * SPW + i,
  // block kb) lands at block qw * NBQ + kb of the slot.  V piece j: target
  // slot v_slot[j] (uniform), position r of its slice.
  const int qw = wave / C::WQ, wq = wave % C::WQ;
  // within a tile, a step's 16 keys of rows 16 g .. 16 g + 15 are 512 bytes at
  // g * (B / 32) * 1024 + s * 512, key half h of row r at (16 h + r % 16) * 16
  const int p_goff = ((r32 >> 4) * (B / 32) * 1024) + ((lane >> 5) * 16 + (r32 & 15)) * 16;
  constexpr int KB_STRIDE = 2 * (B / 32) * 1024;      // between 32-row blocks of a tile
  // V: each target's 16-key slice of a step sits in LDS token-major (16 rows of
  // D bf16), read straight from V (contiguous or through the page table).  A
  // 1 KB piece is TPP tokens; piece p of the step (p = wave + NW j) belongs to
  // target slot p / PPT, tokens TPP (p % PPT) ...; lane l takes 16 bytes of
  // token l / CPT of the piece.
  constexpr int CPT = D * 2 / 16;                      // 16-byte chunks of a token row
  constexpr int TPP = 64 / CPT;                        // tokens of a 1 KB piece
  constexpr int PPT = C::V_BYTES / 1024;               // pieces of a target's slice
  int v_slot[VP], v_lds[VP], v_tok0[VP], v_head[VP];
#pragma unroll
  for (int j = 0; j < VP; ++j) {
    const int p = wave + C::NW * j;
    v_slot[j] = p / PPT;                               // >= TP: no piece
    v_tok0[j] = TPP * (p % PPT);
    v_lds[j] = C::V_OFF + v_slot[j] * C::V_BYTES + (p % PPT) * 1024;
    const int t = v_slot[j] < TP ? uni32(stgt[v_slot[j]]) : -1;
    v_head[j] = t >= 0 ? t / grp : -1;
  }
  const int v_chunk = (lane % CPT) * 16;
  // contiguous V: one buffer descriptor per piece over the sequence's rows of
  // its head (zero length for an absent target), so rows past the sequence end
  // read as zeros; the lane's offset is fixed, the step moves the scalar offset
  __amdgpu_buffer_rsrc_t vdesc[VP];
  int v_voff[VP];
#pragma unroll
  for (int j = 0; j < VP; ++j) {
    const bool on = !vs.pages && v_slot[j] < TP && v_head[j] >= 0;
    vdesc[j] = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(vs.v + uni64(on ? ((int64_t)v_head[j] * T + tok0) * D : 0)), 0,
        uni32(on ? L * D * 2 : 0), kBufferFlags);
    v_voff[j] = (v_tok0[j] + lane / CPT) * (D * 2) + v_chunk;
  }
  int vJ = 0;  // key block of the walk step being loaded (past the sequence: reads zeros)
  // paged V: per key block, lane c < VP KS TPP holds the byte address of token row
  // (piece j, step s, token tl), c = (j KS + s) TPP + tl: the row of V, or a
  // zero row past the sequence end, for an absent target, a page outside the
  // pool or a walk step past the last block
  uint32_t va_lo = 0u, va_hi = 0u;
  auto make_vaddr = [&](int k) {
    const bool valid = k < nblk;
    const int J = uni32(blist[valid ? (desc ? nblk - 1 - k : k) : 0]);
    vJ = valid ? J : (L + B - 1) / B;
    if (!vs.pages) return;
    const char *row = vzero;
    if (lane < VP * KS * TPP) {
      const int jp = lane / (KS * TPP), st = (lane / TPP) % KS, tl = lane % TPP;
      int g = -1, t0 = 0;
#pragma unroll
      for (int j = 0; j < VP; ++j)
        if (j == jp) {
          g = v_head[j];
          t0 = v_tok0[j];
        }
      const int js = J * B + 16 * st + t0 + tl;        // token index inside the sequence
      if (valid && g >= 0 && js < L) {
        if (vs.pages) {
          const int pg = vs.table[(int64_t)seq * vs.max_pages + js / vs.page_size];
          if (pg >= 0 && pg < vs.num_pages)
            row = reinterpret_cast<const char *>(
                vs.pages + (((int64_t)pg * vs.Hkv + g) * vs.page_size + js % vs.page_size) * D);
        } else {
          row = reinterpret_cast<const char *>(vs.v + ((int64_t)g * T + tok0 + js) * D);
        }
      }
    }
    const uint64_t a = reinterpret_cast<uint64_t>(row);
    va_lo = (uint32_t)a;
    va_hi = (uint32_t)(a >> 32);
  };
  const int nsteps = nblk * KS;

  // per key block: descriptors of the tiles of the wave's source pieces (one
  // per slot, query block qw) and of the V block of its V pieces
  struct Desc {
    __amdgpu_buffer_rsrc_t t[SPW];
  };
  auto make_desc = [&](Desc &dd, int k) {
    const bool valid = k < nblk;
    const int kk = valid ? (desc ? nblk - 1 - k : k) : 0;
    const int J = uni32(blist[kk]);
    // lane u < U: tile index of slot u of query block qw at J, or -1
    int ti = -1;
    if (valid && lane < U && (qw == 0 || has1)) {
      const int bu = qw * U_MAX + lane;
      const uint32_t wd = bm[bu * nbw + (J >> 5)];
      if ((wd >> (J & 31)) & 1u) {
        const int64_t x = rbase[bu] + pc[bu * nbw + (J >> 5)] + __popc(wd & ((1u << (J & 31)) - 1u));
        if (x < rend[bu]) ti = (int)x;
      }
    }
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
      const int tix = __builtin_amdgcn_readlane(ti, wq * SPW + i);
      dd.t[i] = __builtin_amdgcn_make_buffer_rsrc(
          (void *)(tiles + uni64((int64_t)(tix >= 0 ? tix : 0) * TBYTES)), 0,
          tix >= 0 ? (int)TBYTES : 0, kBufferFlags);
    }
  };
  // step s of a block: every piece of the wave, memory -> LDS stage
  auto dma = [&](char *stage, const Desc &dd, int s) {
#pragma unroll
    for (int i = 0; i < SPW; ++i)
#pragma unroll
      for (int kb = 0; kb < NBQ; ++kb)
        lds_load16<0>(dd.t[i], stage + (wq * SPW + i) * C::SRC_BYTES + (qw * NBQ + kb) * 1024,
                      p_goff, s * 512 + kb * KB_STRIDE);
#pragma unroll
    for (int j = 0; j < VP; ++j)
      if (v_slot[j] < TP) {
        if (vs.pages) {
          const int c = ((j * KS + s) * TPP + lane / CPT) * 4;
          const uint64_t a = ((uint64_t)(uint32_t)__builtin_amdgcn_ds_bpermute(c, (int)va_hi) << 32) |
                             (uint32_t)__builtin_amdgcn_ds_bpermute(c, (int)va_lo);
          __builtin_amdgcn_global_load_lds((glob_void *)(a + v_chunk),
                                           (lds_void *)(stage + v_lds[j]), 16, 0, 0);
        } else {
          lds_load16<0>(vdesc[j], stage + v_lds[j], v_voff[j], (vJ * B + 16 * s) * (D * 2));
        }
      }
  };
  f32x16 acc[RB][NB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = zero16();

  // one step from an LDS stage: mix, round, multiply with V (the MFMAs of the
  // first row block interleave with the mix of the second)
  auto compute = [&](const char *stage) {
    if (ta < 0) return;
    // B operands from the token-major V slice: lane (h, m) reads, for its 8 keys
    // 8 h .. 8 h + 7, the NB consecutive columns NB m .. NB m + NB - 1 (one 8- or
    // 4-byte read per key; a half-wave reads one whole row), and v_perm_b32
    // pairs consecutive keys of one column: operand e feeds the MFMA whose
    // column n stands for value column NB n + e
    uint32_t qd[8][NB / 2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const char *src = stage + boff + i * (D * 2);
      if constexpr (NB == 4) {
        const uint64_t x = *reinterpret_cast<const uint64_t *>(src);
        qd[i][0] = (uint32_t)x;
        qd[i][1] = (uint32_t)(x >> 32);
      } else {
        qd[i][0] = *reinterpret_cast<const uint32_t *>(src);
      }
    }
    u32x4 bv[NB];
#pragma unroll
    for (int e = 0; e < NB; ++e)
#pragma unroll
      for (int pk = 0; pk < 4; ++pk)
        bv[e][pk] = __builtin_amdgcn_perm(qd[2 * pk + 1][e >> 1], qd[2 * pk][e >> 1],
                                          (e & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      u32x4 v[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        // a missing source (b >= its count) has coefficient 0 and reads slot 0
        v[b] = *reinterpret_cast<const u32x4 *>(stage + soff_b[b] + aoff[rb]);
      float mx[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) mx[e] = 0.f;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx[2 * e] = fmaf(cf[rb][b], __uint_as_float(v[b][e] << 16), mx[2 * e]);
          mx[2 * e + 1] = fmaf(cf[rb][b], __uint_as_float(v[b][e] & 0xffff0000u), mx[2 * e + 1]);
        }
      u32x4 am;
#pragma unroll
      for (int e = 0; e < 4; ++e) am[e] = pack_bf16x2(mx[2 * e], mx[2 * e + 1]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = mfma_bf16(as_bf16x8(am), as_bf16x8(bv[nb]), acc[rb][nb]);
    }
  };
  // end of a step: this wave's loads into the next stage have landed (a full
  // drain: direct-to-LDS loads complete with no finer count to wait on), then
  // the work-group barrier
  auto step_end = [] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  if (nsteps > 0) {
    char *st0 = smem, *st1 = smem + C::STAGE;
    Desc dc;
    make_desc(dc, 0);
    make_vaddr(0);
    dma(st0, dc, 0);
    step_end();
    for (int k = 0; k < nblk; ++k) {
      // step s of block k: the next step (the next block's first after the
      // last) moves into the other stage while step s is computed
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        char *cur = (s & 1) ? st1 : st0, *nxt = (s & 1) ? st0 : st1;
        if (s + 1 == KS) {
          make_desc(dc, k + 1);
          make_vaddr(k + 1);
        }
        dma(nxt, dc, (s + 1) % KS);
        compute(cur);
        step_end();
      }
    }
  }

  if (ta < 0) return;
  float *ot = o + (int64_t)ta * T * D;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row0 = 64 * part + 32 * rb;
    const int q = row0 / B;
    if (q == 1 && !has1) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ip = Iq[q] * B + (row0 % B) + acc_row(r, lane);
      if (ip < L) {
        // value columns NB r32 .. NB r32 + NB - 1
        float *dst = ot + (tok0 + ip) * D + NB * r32;
        if constexpr (NB == 4) {
          __builtin_nontemporal_store(f32x4{acc[rb][0][r], acc[rb][1][r], acc[rb][2][r], acc[rb][3][r]},
                                      reinterpret_cast<f32x4 *>(dst));
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) __builtin_nontemporal_store(acc[rb][nb][r], dst + nb);
        }
      }
    }
  }
}

// The apply kernels for one tile format, over `nrows` block-rows of `sched`.
// bf16 maps: targets with at most four sources in pairs (k_pairs, then
// k_apply_pair over the query-block pairs of `psched`); fp8 maps: one target
// per work-group (k_apply4).  Targets with
// more sources: k_apply_mix.  A work-group with nothing of its class returns
// right after reading the weights.
template <int B, int D, int FMT>
static mf_status launch_apply_fmt(hipStream_t s, const mf_bsr_map *map, const float *W, int32_t Ht,
                                  const VSrc &vs, const SeqGeom &g, int32_t renorm, float *o,
                                  void *ws, const VtWs &w, const int32_t *sched, int32_t nrows,
                                  const int32_t *psched, int32_t npairs, int nbw, size_t smem,
                                  size_t vbufs) {
  using CM = ApplyMixCfg<B, D, FMT>;
  const int32_t Hkv = vs.Hkv;
  // distinct V heads of a target group (the V tiles it holds in LDS)
  int nvmax = 1;
  for (int t0 = 0; t0 < Ht; t0 += CM::G) {
    const int t1 = std::min(t0 + CM::G, (int)Ht) - 1;
    nvmax = std::max(nvmax, t1 / (Ht / Hkv) - t0 / (Ht / Hkv) + 1);
  }
  // the coefficient table when it costs no occupancy (two work-groups per CU
  // still fit, or not even one fits without it), else coefficients inline
  const size_t mix_lo = mix_smem(B, D, map->num_heads, nbw, nvmax, false);
  const size_t mix_hi = mix_smem(B, D, map->num_heads, nbw, nvmax, true);
  const bool use_ct = FMT == MF_TILE_BF16 && mix_hi <= 160 * 1024 &&
                      (mix_hi <= 80 * 1024 || mix_lo > 80 * 1024);
  const size_t smem_mix = use_ct ? mix_hi : mix_lo;
  const void *kmix = use_ct ? reinterpret_cast<const void *>(&k_apply_mix<B, D, FMT, FMT == MF_TILE_BF16>)
                            : reinterpret_cast<const void *>(&k_apply_mix<B, D, FMT, false>);
  if (smem_mix > 64 * 1024 &&
      hipFuncSetAttribute(kmix, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_mix) != hipSuccess)
    return MF_ERR_HIP;
  const char *tiles = static_cast<const char *>(map->tiles);
  const int64_t npos = ((int64_t)nrows + kXcds - 1) / kXcds * kXcds;
  if constexpr (FMT == MF_TILE_BF16) {
    using CP = PairCfg<B, D, kPairT>;
    const size_t smem_pair = (size_t)pair_tables<B, D, kPairT>(nbw).total;
    if (smem_pair > 160 * 1024) return MF_ERR_UNSUPPORTED;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(&k_apply_pair<B, D, kPairT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem_pair) != hipSuccess)
      return MF_ERR_HIP;
    const int32_t *gtab = at<int32_t>(ws, w.gtab);
    // any two targets with at most four sources fit one work-group
    const int32_t ngmax = (Ht + kPairT - 1) / kPairT;
    const int64_t nppos = ((int64_t)npairs + kXcds - 1) / kXcds * kXcds;
    if (npairs > 0)
      hipLaunchKernelGGL((k_apply_pair<B, D, kPairT>), dim3((unsigned)(nppos * ngmax)),
                         dim3(CP::NT), smem_pair, s, map->row_ptr, map->col_idx, tiles,
                         map->kept_mass, map->num_heads, g.NBR, g.T, W, Ht / Hkv, vs,
                         at<char>(ws, w.vzero), at<RowInfo>(ws, w.rt.rows), psched, npairs, nbw,
                         map->capacity_tiles, renorm, o, map->row_alias, gtab, ngmax);
  } else {
    if (smem + vbufs > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(&k_apply4<B, D, FMT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem) != hipSuccess)
      return MF_ERR_HIP;
    hipLaunchKernelGGL((k_apply4<B, D, FMT>), dim3((unsigned)(npos * Ht)),
                       dim3(Apply4Cfg<B, D, FMT>::NT), smem, s, map->row_ptr, map->col_idx, tiles,
                       map->kept_mass, map->num_heads, g.NBR, g.T, W, Ht, Ht / Hkv,
                       at<uint16_t>(ws, w.vt), at<RowInfo>(ws, w.rt.rows), sched, nrows, nbw,
                       map->capacity_tiles, renorm, o, map->row_alias);
  }
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  const int64_t ngrp = (Ht + CM::G - 1) / CM::G;
  auto launch_mix = [&](auto ct) {
    constexpr bool CTB = decltype(ct)::value;
    hipLaunchKernelGGL((k_apply_mix<B, D, FMT, CTB>), dim3((unsigned)(npos * ngrp)), dim3(CM::NT),
                       smem_mix, s, map->row_ptr, map->col_idx, tiles, map->kept_mass,
                       map->num_heads, g.NBR, g.T, W, Ht, Ht / Hkv, at<uint16_t>(ws, w.vt),
                       at<RowInfo>(ws, w.rt.rows), sched, nrows, nbw, map->capacity_tiles, renorm,
                       o, map->row_alias, nvmax, at<char>(ws, w.vzero),
                       FMT == MF_TILE_BF16 ? at<int32_t>(ws, w.gtab) + kMixFlag : nullptr);
  };
  if (use_ct)
    launch_mix(std::integral_constant<bool, FMT == MF_TILE_BF16>{});
  else
    launch_mix(std::false_type{});
  return hip_status();
}

// V staging, the window schedule (if any), then both apply kernels.
template <int B, int D>
static mf_status launch_apply(hipStream_t s, const mf_bsr_map *map, const float *W, int32_t Ht,
                              const VSrc &vs, const SeqGeom &g, int32_t nrows, int32_t npairs,
                              int32_t renorm, float *o, void *ws, const VtWs &w) {
  const int nbw = (g.maxnb + 31) / 32 > 0 ? (g.maxnb + 31) / 32 : 1;
  const size_t smem = apply_smem(B, map->num_heads, nbw);
  // tile indices are held in int32; V rows are addressed with 32-bit byte
  // offsets d * NBR * B * 2
  if (map->capacity_tiles > INT32_MAX) return MF_ERR_UNSUPPORTED;
  if ((int64_t)D * g.NBR * B * 2 >= ((int64_t)1 << 31)) return MF_ERR_UNSUPPORTED;
  if (map->num_heads > kMixMaxSources || Ht > kMaxTargets) return MF_ERR_UNSUPPORTED;
  const size_t vbufs = 2 * (size_t)B * D * 2;  // the two static V tile buffers of k_apply4
  if (smem + vbufs > 160 * 1024 ||
      mix_smem(B, D, map->num_heads, nbw, ApplyMixCfg<B, D, MF_TILE_BF16>::G, false) > 160 * 1024)
    return MF_ERR_UNSUPPORTED;
  const int32_t *sched = at<int32_t>(ws, w.rt.sched);
  if (nrows == 0) return MF_OK;
  int32_t *psched = at<int32_t>(ws, w.psched);
  hipLaunchKernelGGL(k_pair_sched, dim3(1), dim3(1024), 0, s, at<RowInfo>(ws, w.rt.rows), sched,
                     g.NBR, B, vs.window, psched, at<u32x4>(ws, w.vzero));
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  if (vs.window) {
    hipLaunchKernelGGL(k_window_sched, dim3(1), dim3(1024), 0, s, at<RowInfo>(ws, w.rt.rows),
                       sched, g.NBR, B, vs.window, at<int32_t>(ws, w.wsched));
    if (hip_status() != MF_OK) return MF_ERR_HIP;
    sched = at<int32_t>(ws, w.wsched);
  }
  // bf16 maps: the target pairs, and whether any target is left to the
  // dense-mixing kernel; only that kernel and the fp8 one read the staged V
  int32_t *gtab = at<int32_t>(ws, w.gtab);
  const bool bf16 = map->tile_format != MF_TILE_MXFP8;
  if (bf16) {
    hipLaunchKernelGGL(k_pairs, dim3(1), dim3(64), 0, s, W, Ht, map->num_heads,
                       (int32_t)(kPairT == 2), gtab);
    if (hip_status() != MF_OK) return MF_ERR_HIP;
  }
  hipLaunchKernelGGL((k_vstage<B, D>), dim3(g.NBR, vs.Hkv), dim3(256), 0, s, vs, g.T,
                     at<RowInfo>(ws, w.rt.rows), g.NBR, at<uint16_t>(ws, w.vt),
                     bf16 ? gtab + kMixFlag : nullptr);
  if (hip_status() != MF_OK) return MF_ERR_HIP;
  if (map->tile_format == MF_TILE_MXFP8)
    return launch_apply_fmt<B, D, MF_TILE_MXFP8>(s, map, W, Ht, vs, g, renorm, o, ws, w, sched,
                                                 nrows, psched, npairs, nbw, smem, vbufs);
  return launch_apply_fmt<B, D, MF_TILE_BF16>(s, map, W, Ht, vs, g, renorm, o, ws, w, sched,
                                              nrows, psched, npairs, nbw, smem, vbufs);
}

}  // namespace mf

// Fixed device scratch of mf_apply_translated_noalloc.  Each GPU the library
// runs on holds its own copy until the process ends.  Host code never passes
// `scratch` itself (its host-side name is not a device address): it uses the
// per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[MF_APPLY_NOALLOC_SCRATCH_BYTES];

namespace mf {

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_dev[kMaxDevices];

// Device address of the current device's scratch, looked up once per device
// (with that device current); nullptr if the lookup fails.
static void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_dev[dev] = ptr;
  }
  return g_scratch_dev[dev];
}


// Shared argument checks and dispatch of the apply entry points.  With
// use_scratch the workspace is the fixed device scratch instead of ws.
static mf_status apply_common(void *stream, const mf_bsr_map *map, const float *W, int32_t Ht,
                              VSrc vs, int32_t d, const int32_t *cu_host, const int32_t *cu_dev,
                              int32_t nseq, const int32_t *window_host, int32_t renorm, float *o,
                              void *ws, size_t ws_bytes, bool use_scratch = false) {
  const int32_t Hkv = vs.Hkv;
  if (!map || !cu_host || !cu_dev || Ht <= 0 || Hkv <= 0 || Ht % Hkv != 0)
    return MF_ERR_INVALID_ARG;
  if (!valid_block(map->block)) return MF_ERR_INVALID_ARG;
  if (!valid_dim(d)) return MF_ERR_UNSUPPORTED;
  if (map->num_heads <= 0 || !W || !valid_tile_format(map->tile_format)) return MF_ERR_INVALID_ARG;
  SeqGeom g;
  mf_status st = seq_geom(cu_host, nseq, map->block, &g);
  if (st != MF_OK) return st;
  if (g.NBR != map->num_block_rows || g.T != map->total_tokens) return MF_ERR_INVALID_ARG;
  if ((int64_t)g.NBR * Ht > INT32_MAX / 2) return MF_ERR_UNSUPPORTED;
  if (g.T > 0 && (!(vs.v || vs.pages) || !o || !map->row_ptr || !map->col_idx || !map->tiles ||
                  !map->kept_mass))
    return MF_ERR_INVALID_ARG;
  const int B = map->block;
  int64_t nrows = g.NBR, npairs = 0;  // block-rows, and query-block pairs of the fused retrieval
  for (int32_t q = 0; q < nseq; ++q) npairs += ((cu_host[q + 1] - cu_host[q] + B - 1) / B + 1) / 2;
  if (vs.pages) {
    if (vs.page_size <= 0 || vs.num_pages <= 0 || vs.max_pages <= 0 || !vs.table)
      return MF_ERR_INVALID_ARG;
    for (int32_t s = 0; s < nseq; ++s)
      if ((int64_t)cu_host[s + 1] - cu_host[s] > (int64_t)vs.max_pages * vs.page_size)
        return MF_ERR_INVALID_ARG;  // the table cannot cover the sequence
  }
  if (vs.window) {
    if (!window_host) return MF_ERR_INVALID_ARG;
    nrows = 0;
    npairs = 0;
    for (int32_t s = 0; s < nseq; ++s) {
      const int32_t L = cu_host[s + 1] - cu_host[s];
      const int32_t a = window_host[2 * s], b = window_host[2 * s + 1];
      if (a < 0 || b < a || b > L) return MF_ERR_INVALID_ARG;
      if (a == b) continue;  // nothing of this sequence in the chunk
      if (a % B != 0 || (b % B != 0 && b != L)) return MF_ERR_INVALID_ARG;
      nrows += ((int64_t)b + B - 1) / B - a / B;
      npairs += (((int64_t)b + B - 1) / B - a / B + 1) / 2;
    }
  }
  const VtWs w = vt_ws(g, Hkv, B, d);
  if (use_scratch) {
    if (w.total > MF_APPLY_NOALLOC_SCRATCH_BYTES) return MF_ERR_WORKSPACE;
    if (g.NBR == 0) return MF_OK;
    ws = scratch_address();
    ws_bytes = MF_APPLY_NOALLOC_SCRATCH_BYTES;
    if (!ws) return MF_ERR_HIP;
  }
  if (!ws || ws_bytes < w.total) return MF_ERR_WORKSPACE;
  if (g.NBR == 0) return MF_OK;
  void *wsa = reinterpret_cast<void *>((reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((st = launch_rowtable(s, cu_dev, g, B, wsa, w.rt)) != MF_OK) return st;
  const int32_t nr = (int32_t)nrows, np = (int32_t)npairs;
  if (B == 32)
    return d == 64 ? launch_apply<32, 64>(s, map, W, Ht, vs, g, nr, np, renorm, o, wsa, w)
                   : launch_apply<32, 128>(s, map, W, Ht, vs, g, nr, np, renorm, o, wsa, w);
  if (B == 64)
    return d == 64 ? launch_apply<64, 64>(s, map, W, Ht, vs, g, nr, np, renorm, o, wsa, w)
                   : launch_apply<64, 128>(s, map, W, Ht, vs, g, nr, np, renorm, o, wsa, w);
  return d == 64 ? launch_apply<128, 64>(s, map, W, Ht, vs, g, nr, np, renorm, o, wsa, w)
                 : launch_apply<128, 128>(s, map, W, Ht, vs, g, nr, np, renorm, o, wsa, w);
}

}  // namespace mf

using namespace mf;

extern "C" size_t mf_apply_workspace_bytes(int32_t Hkv, const int32_t *cu, int32_t nseq, int32_t B,
                                           int32_t d) {
  SeqGeom g;
  if (Hkv <= 0 || !valid_dim(d) || seq_geom(cu, nseq, B, &g) != MF_OK) return 0;
  return vt_ws(g, Hkv, B, d).total;
}

extern "C" mf_status mf_apply_translated(void *stream, const mf_bsr_map *map, const float *W,
                                         int32_t Ht, const void *v, int32_t Hkv, int32_t d,
                                         const int32_t *cu_host, const int32_t *cu_dev,
                                         int32_t nseq, int32_t renorm, float *o, void *ws,
                                         size_t ws_bytes) {
  VSrc vs{static_cast<const uint16_t *>(v), nullptr, nullptr, 0, 0, 0, Hkv, nullptr};
  return apply_common(stream, map, W, Ht, vs, d, cu_host, cu_dev, nseq, nullptr, renorm, o, ws,
                      ws_bytes);
}

extern "C" mf_status mf_apply_translated_noalloc(void *stream, const mf_bsr_map *map,
                                                 const float *W, int32_t Ht, const void *v,
                                                 int32_t Hkv, int32_t d,
                                                 const int32_t *cu_host, const int32_t *cu_dev,
                                                 int32_t nseq, int32_t renorm, float *o) {
  VSrc vs{static_cast<const uint16_t *>(v), nullptr, nullptr, 0, 0, 0, Hkv, nullptr};
  return apply_common(stream, map, W, Ht, vs, d, cu_host, cu_dev, nseq, nullptr, renorm, o,
                      nullptr, 0, true);
}

extern "C" mf_status mf_apply_translated_paged(void *stream, const mf_bsr_map *map,
                                               const float *W, int32_t Ht, const mf_paged_v *pv,
                                               int32_t Hkv, int32_t d, const int32_t *cu_host,
                                               const int32_t *cu_dev, int32_t nseq,
                                               const int32_t *window_host,
                                               const int32_t *window_dev, int32_t renorm,
                                               float *o, void *ws, size_t ws_bytes) {
  if (!pv || !pv->pages) return MF_ERR_INVALID_ARG;
  if ((window_host == nullptr) != (window_dev == nullptr)) return MF_ERR_INVALID_ARG;
  VSrc vs{nullptr, static_cast<const uint16_t *>(pv->pages), pv->block_table, pv->page_size,
          pv->max_pages_per_seq, pv->num_pages, Hkv, window_dev};
  return apply_common(stream, map, W, Ht, vs, d, cu_host, cu_dev, nseq, window_host, renorm, o,
                      ws, ws_bytes);
}
