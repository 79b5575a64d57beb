/*
 * mapflow.h — C ABI of the attention-map reuse library for MI355X (gfx950).
 *
 * Two halves of one data path, plus dense attention for recomputed heads:
 *
 *   mf_compress_topp        sender side: attention map of every source head,
 *                           block-level top-p selection, kept blocks written as
 *                           bf16 (or block-scaled fp8) probability tiles in Block
 *                           Sparse Row (BSR) form with per-row kept mass.
 *                           MapFlow ("Accelerating Cross-Model LLM Inference via
 *                           Attention Map Reuse"), §4 (top-p compression into
 *                           BSR) and §5.2 (Attention State Compressor).
 *   mf_apply_translated     receiver side: O_t = sum_h W[t,h] renorm(A_hat_h) V_g(t)
 *                           for every target head, without a dense L x L map in
 *                           device memory.  MapFlow §3.3 (linear head mapping),
 *                           §5.4 (fused retrieval kernel).
 *   mf_apply_translated_paged
 *                           the same retrieval with V in a paged pool behind a
 *                           page table, optionally over one query window per
 *                           sequence (chunked prefill).  MapFlow §6 (paged
 *                           memory and varlen batches in the serving stack).
 *   mf_prefix_dedupe        block-rows whose query/key prefix repeats an earlier
 *                           sequence's, so compression computes them once and
 *                           both sides read the first copy.  MapFlow §5.3 (Block
 *                           Manager: blocks indexed by prefix hashes), §2.3
 *                           (prefix caching).
 *   mf_tv_distance          per-row total-variation distance between the
 *                           translated map and a receiver's own map, to choose
 *                           the receiver layers to recompute (MapFlow §3.3).
 *   mf_dense_ref_attention  softmax(Q K^T / sqrt(d) + bias) V, causal, for the
 *                           receiver layers that are recomputed (MapFlow §4) and
 *                           the exact path a cache miss falls back to (AttnCache
 *                           guide, "AttnCache Guide: Reusing Attention Maps in
 *                           LLM Prefill", threshold-gated fallback).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are device pointers unless marked "host".  The caller owns all
 *   memory; the library never allocates, frees or keeps a pointer after a call
 *   returns.  Sizes of the caller-provided buffers come from the *_bytes /
 *   *_max_tiles queries below.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *   enqueued asynchronously on it; no entry point synchronises except
 *   mf_read_status.
 * - Sequences are packed back to back along the token axis (variable-length
 *   packing, MapFlow §6): sequence s occupies tokens [cu_seqlens[s],
 *   cu_seqlens[s+1]).  Every call takes the same offsets twice: a host copy
 *   (used to validate and size the launch) and a device copy (read by kernels);
 *   they must hold the same values.
 * - Tensors are head-major, head dimension innermost: Q, K [H][T][d], V
 *   [Hkv][T][d], O [H][T][d] (fp32).  Key-block and query-block grids restart
 *   at every sequence start.
 * - Causal masking is per sequence: token i attends to keys j <= i of its own
 *   sequence.  Logit offsets (mf_logit_bias) are added after the 1/sqrt(d)
 *   scaling.
 * - Argument errors are found on the host before anything is enqueued and
 *   return MF_ERR_INVALID_ARG / MF_ERR_UNSUPPORTED / MF_ERR_WORKSPACE.  A
 *   failed kernel launch returns MF_ERR_HIP.  A map that does not fit its
 *   capacity is reported asynchronously through the map's device status word
 *   (read with mf_read_status).
 * - Results are deterministic: the same inputs give bitwise-identical maps and
 *   outputs from run to run (fixed-order reductions, no floating-point atomics).
 * - Supported: block B in {32, 64, 128}; head dim d in {64, 128}; at most 1024
 *   key blocks per sequence; 0 < p <= 1; Ht % Hkv == 0 (and Hq % Hkv == 0).
 * - Calls are thread-safe and keep no state between calls.
 */
#ifndef MAPFLOW_H
#define MAPFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mf_status {
  MF_OK = 0,
  MF_ERR_INVALID_ARG = 1,  /* bad pointer, size, offsets or threshold           */
  MF_ERR_UNSUPPORTED = 2,  /* valid but not built: block, head dim, dtype, size */
  MF_ERR_CAPACITY = 3,     /* (device status) more kept tiles than capacity     */
  MF_ERR_HIP = 4,          /* a HIP launch or runtime call failed               */
  MF_ERR_WORKSPACE = 5     /* workspace pointer NULL or smaller than required   */
} mf_status;

typedef enum mf_dtype { MF_BF16 = 0, MF_FP32 = 1 } mf_dtype;

/* How a compressed map stores its probability tiles (see mf_bsr_map).
 * MF_TILE_MXFP8 is the quantised sparse map MapFlow §9 points to: E4M3 codes
 * with one power-of-two scale per 32 keys of a row, half the bytes of bf16. */
typedef enum mf_tile_format { MF_TILE_BF16 = 0, MF_TILE_MXFP8 = 1 } mf_tile_format;

/* Logit offsets added after scaling: +sink_bias on key positions [0, sink_n) of
 * each sequence, +local_bias where 0 <= i - j < local_w.  Both may apply.  A
 * NULL pointer means no offsets. */
typedef struct mf_logit_bias {
  int32_t sink_n;
  float sink_bias;
  int32_t local_w;
  float local_bias;
} mf_logit_bias;

/* Compressed map of Hs source heads in BSR form (MapFlow §4, §5.2).
 *
 * Row r = h * num_block_rows + global block-row, where global block-rows run
 * over the sequences in order and, within a sequence, over its query blocks
 * I = 0 .. ceil(L_s / B) - 1.  Row r holds the kept key blocks J <= I of that
 * query block in ascending J: col_idx[row_ptr[r] .. row_ptr[r+1]).  Tile n is a
 * full B x B block of bf16 probabilities (round-to-nearest-even of the fp32 value
 * exp(s_ij - lse_i), i.e. normalised over the whole causal row, not
 * renormalised), zero above the diagonal and outside the sequence.
 *
 * Element order inside a tile ("fragment order", the operand order of the
 * receiver's 16x16x32 matrix instructions, so each 1 KB piece is one
 * contiguous load): the tile is cut into (B/16) x (B/32) pieces of 16 rows x 32
 * keys; piece (g, k) is the (g * B/32 + k)-th 1 KB block; inside it, 16-byte
 * chunk f holds row 16 g + (f % 16), keys 32 k + 8 (f / 16) .. + 7.  Element
 * (i, j) of the tile is therefore at
 *   ((i/16 * B/32 + j/32) * 64 + (j%32)/8 * 16 + i%16) * 8 + j%8.
 * kept_mass[h][token] is the sum, over the kept blocks of the token's row, of
 * its unrounded probabilities.
 *
 * MF_TILE_MXFP8 tiles (mf_tile_bytes(B, MF_TILE_MXFP8) = B*B + B*B/32 bytes):
 * every row of a tile is cut into B/32 blocks of 32 consecutive keys.  Block g
 * of row i has the scale exponent e = max(floor(log2 a) - 7, -126), a being the
 * block's largest fp32 probability (e = -126 for an all-zero block), stored as
 * the byte e + 127; each element is the OCP E4M3 code (bias 7, no infinities)
 * of p * 2^-e rounded to nearest even, so the block maximum scales into
 * [128, 256) and nothing saturates.  A reader decodes code_value * 2^e; the
 * error is at most max(2^-4 p, 2^(e-10)).  The first B*B bytes hold the codes:
 * with NP = 2 for B >= 64 (1 for B = 32), the tile is cut into pieces of 16
 * rows x 32*NP keys, piece (i/16, j/(32 NP)) being the
 * ((i/16) * B/(32 NP) + j/(32 NP))-th block of 512*NP bytes; inside it, lane
 * f = ((j%32)/8)*16 + i%16 holds 8*NP bytes: keys 8 of each 32-key chunk of
 * the piece, chunk by chunk.  Element (i, j) is at
 *   ((i/16 * B/(32 NP) + j/(32 NP)) * 64 + (j%32)/8 * 16 + i%16) * 8 NP
 *     + ((j % (32 NP)) / 32) * 8 + j%8.
 * The last B*B/32 bytes hold the scale bytes row by row: row i, block g at
 * B*B + i * B/32 + g.
 *
 * The caller allocates every array and sets the pointers and capacity_tiles;
 * mf_compress_topp fills the four size fields and the arrays.  Apply only reads
 * the map, so one map can serve any number of apply calls (MapFlow §5.2: one
 * compressed map serves many receivers).
 *
 * row_alias (optional, NULL for none): [NBR] global block-row -> the block-row
 * whose rows it shares, as written by mf_prefix_dedupe (itself when unique).
 * With it, mf_compress_topp computes only block-rows with row_alias[gr] == gr;
 * the others get no tiles of their own (empty BSR rows) and a copy of their
 * first copy's kept mass, and mf_apply_translated reads their tiles through the
 * alias.  Set it before mf_compress_topp and keep it with the map. */
typedef struct mf_bsr_map {
  int32_t num_heads;       /* Hs                                        (out) */
  int32_t block;           /* B                                         (out) */
  int32_t num_block_rows;  /* NBR = sum_s ceil(L_s / B)                 (out) */
  int32_t total_tokens;    /* T = cu_seqlens[nseq]                      (out) */
  int64_t capacity_tiles;  /* tiles/col_idx entries allocated            (in) */
  int64_t *row_ptr;        /* [Hs * NBR + 1]                                  */
  int32_t *col_idx;        /* [capacity_tiles]                                */
  void *tiles;             /* [capacity_tiles] tiles of mf_tile_bytes(B, tile_format) bytes */
  float *kept_mass;        /* [Hs][T]                                         */
  int64_t *nnz;            /* device scalar: number of kept tiles             */
  int32_t *status;         /* device scalar: MF_OK or MF_ERR_CAPACITY         */
  const int32_t *row_alias; /* [NBR] or NULL: shared block-rows (see above)     */
  int32_t tile_format;     /* mf_tile_format of the tiles                 (in) */
} mf_bsr_map;

/* Number of global block-rows sum_s ceil(L_s / B); -1 if the offsets are invalid.
 * cu_seqlens_host: host, nseq + 1 entries. */
int32_t mf_num_block_rows(const int32_t *cu_seqlens_host, int32_t nseq, int32_t B);

/* Bytes of one stored tile: B*B*2 for MF_TILE_BF16, B*B + B*B/32 for
 * MF_TILE_MXFP8; 0 if B or the format is not supported. */
int64_t mf_tile_bytes(int32_t B, int32_t tile_format);

/* Worst-case kept tiles (every causal block): Hs * sum_s nb_s (nb_s + 1) / 2.
 * -1 if the arguments are invalid.  A smaller capacity is allowed; overflow is
 * reported through the map's status word and no tile beyond it is written. */
int64_t mf_compress_max_tiles(int32_t Hs, const int32_t *cu_seqlens_host, int32_t nseq,
                              int32_t B);

/* Device workspace bytes mf_compress_topp needs (0 if the arguments are invalid).
 * Holds per-(row, key block) log-sum-exp partials (4 bytes per causal query/key
 * block pair and row), row normalisers, kept bitmaps and counts. */
size_t mf_compress_workspace_bytes(int32_t Hs, const int32_t *cu_seqlens_host, int32_t nseq,
                                   int32_t B, int32_t d);

/* Sender-side compression (MapFlow §4, §5.2).
 *
 * q, k        [Hs][T][d], dtype qk_dtype (bf16 bit patterns or fp32).
 * p           top-p threshold in (0, 1].  Each query-block row keeps the
 *             shortest prefix of its causal key blocks, ordered by block mass
 *             (sum of the block's probabilities) descending and lower block
 *             index first on equal mass, whose cumulative mass reaches p times
 *             the row's total.  p == 1 keeps every causal block.
 * bias        host, may be NULL.
 * map         host struct: pointers and capacity set by the caller; size fields
 *             written here.
 * workspace   device, at least mf_compress_workspace_bytes(...) bytes, 256-byte
 *             aligned; contents are scratch and may be reused after the stream
 *             has passed this call.
 * Errors: MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_WORKSPACE, MF_ERR_HIP. */
mf_status mf_compress_topp(void *stream, const void *q, const void *k, mf_dtype qk_dtype,
                           const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                           int32_t nseq, int32_t Hs, int32_t d, int32_t B, double p,
                           const mf_logit_bias *bias, mf_bsr_map *map, void *workspace,
                           size_t workspace_bytes);

/* Device workspace bytes mf_prefix_dedupe needs (0 if the arguments are invalid). */
size_t mf_prefix_dedupe_workspace_bytes(const int32_t *cu_seqlens_host, int32_t nseq, int32_t B);

/* Shared-prefix block-rows (MapFlow §5.3: the Block Manager indexes compressed
 * blocks by prefix hashes; §2.3: prefix caching skips recomputation of shared
 * prefixes).
 *
 * Block-row (s, I) is *full* when (I + 1) * B <= L_s.  A full block-row whose
 * tokens 0 .. (I + 1) B - 1 carry the same q and k values (every head, bit for
 * bit) as those of an earlier sequence s' < s whose block-row I is also full
 * has the same causal logits, offsets and probabilities, hence the same kept
 * blocks, tiles and kept masses.  row_alias[gr] is the global block-row of the
 * first such (s', I), or gr itself.
 *
 * Prefix equality is decided by a 128-bit chained hash of each block's q and k
 * content (per block: a sum of independently mixed 16-byte chunks; per
 * sequence: chained from block 0), computed on the device.
 *
 * q, k        [Hs][T][d] in qk_dtype, as passed to mf_compress_topp.
 * row_alias   [NBR] int32, written.
 * workspace   device, at least mf_prefix_dedupe_workspace_bytes(...) bytes.
 * Errors: MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_WORKSPACE, MF_ERR_HIP. */
mf_status mf_prefix_dedupe(void *stream, const void *q, const void *k, mf_dtype qk_dtype,
                           const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                           int32_t nseq, int32_t Hs, int32_t d, int32_t B, int32_t *row_alias,
                           void *workspace, size_t workspace_bytes);

/* Device workspace bytes mf_apply_translated and mf_apply_translated_paged need:
 * room for a block-padded copy of V staged in 16-key chunks
 * ([Hkv][NBR * B / 16][d][16] bf16; written only when some target has more
 * than four sources or the map holds fp8 tiles, otherwise V is read in
 * place), a 32 KB block the calls clear and read as zeros, the block-row table
 * and the query-block schedules.  0 if invalid. */
size_t mf_apply_workspace_bytes(int32_t Hkv, const int32_t *cu_seqlens_host, int32_t nseq,
                                int32_t B, int32_t d);

/* Receiver-side translated retrieval (MapFlow §3.3, §5.4):
 *   O_t[i,:] = sum_h W[t,h] sum_{J kept by h in i's row} sum_{j in J}
 *              (A_hat_h[i,j] / kept_mass_h[i]) V_g(t)[j,:],   g(t) = t / (Ht / Hkv)
 * With renorm == 0 the division by kept mass is dropped.  A row whose kept
 * mass is 0 contributes nothing.  W = identity gives per-head reuse of the
 * cached map: O_h = renorm(A_hat_h) V_h (AttnCache guide, architecture
 * figure, cache-hit path).
 *
 * Precision: each translated tile is mixed in fp32 (the stored tile values
 * widened exactly, fp32 coefficients W[t,h] / kept_mass_h[i]), rounded once to
 * bf16, and multiplied with V on bf16 MFMA with fp32 accumulation.
 *
 * map         host struct filled by mf_compress_topp; read only.
 * W           [Ht][map->num_heads] fp32, any sign; zero entries are skipped.
 * v           [Hkv][T][d] bf16 bit patterns, T = map->total_tokens.
 * cu_seqlens  the offsets the map was built with.
 * o           [Ht][T][d] fp32, fully overwritten.
 * workspace   device, at least mf_apply_workspace_bytes(...) bytes.
 * The map's status must be MF_OK (check with mf_read_status); a map that
 * overflowed its capacity gives undefined output rows for the missing tiles.
 * Errors: MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_WORKSPACE, MF_ERR_HIP. */
mf_status mf_apply_translated(void *stream, const mf_bsr_map *map, const float *W, int32_t Ht,
                              const void *v, int32_t Hkv, int32_t d,
                              const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                              int32_t nseq, int32_t renorm, float *o, void *workspace,
                              size_t workspace_bytes);

/* Bytes of the fixed device scratch that mf_apply_translated_noalloc uses in
 * place of a workspace (per GPU, held until the process ends). */
#define MF_APPLY_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* mf_apply_translated without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same computation,
 * kernels and output as mf_apply_translated.
 *
 * The workspace lives in a static device array of
 * MF_APPLY_NOALLOC_SCRATCH_BYTES bytes; a call whose
 * mf_apply_workspace_bytes(Hkv, cu_seqlens, nseq, map->block, d) exceeds it
 * returns MF_ERR_WORKSPACE (Hkv = 8, d = 128, B = 128 fits up to 65408 tokens).
 * Nothing in the scratch has to start at zero, and each call rewrites what it
 * reads.  The array is looked up on the first call on each device (the device
 * current at the call, which must be the stream's).  All calls on one GPU
 * share that array: calls that overlap in time on one GPU (different streams,
 * or host threads without ordering) race on it and give undefined output.
 * Errors: MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_WORKSPACE, MF_ERR_HIP. */
mf_status mf_apply_translated_noalloc(void *stream, const mf_bsr_map *map, const float *W,
                                      int32_t Ht, const void *v, int32_t Hkv, int32_t d,
                                      const int32_t *cu_seqlens_host,
                                      const int32_t *cu_seqlens_dev, int32_t nseq,
                                      int32_t renorm, float *o);

/* V held in a paged cache (PagedAttention-style): token j of sequence s is at
 * slot j % page_size of page block_table[s * max_pages_per_seq + j / page_size]
 * in the pool.  Page indices outside [0, num_pages) read as zeros. */
typedef struct mf_paged_v {
  const void *pages;           /* [num_pages][Hkv][page_size][d] bf16, device    */
  int32_t page_size;           /* tokens per page, >= 1                          */
  int32_t num_pages;           /* pages in the pool                              */
  const int32_t *block_table;  /* [nseq][max_pages_per_seq] int32, device        */
  int32_t max_pages_per_seq;   /* must cover every sequence: L_s <= max * size   */
} mf_paged_v;

/* Translated retrieval with paged V and, optionally, chunked prefill (MapFlow §6:
 * the fused kernel supports PagedAttention, chunked prefill and packed
 * variable-length sequences).  Same computation as mf_apply_translated, with:
 *
 * pv          V through a page table (see mf_paged_v); host struct.
 * window      NULL for whole sequences, or [nseq][2] int32 query-token windows
 *             [begin, end) per sequence (a prefill chunk), given twice (host
 *             copy for validation and sizing, device copy for the kernels).
 *             begin must be a multiple of map->block; end a multiple of it or
 *             the sequence length; an empty window (begin == end, anywhere in
 *             [0, L]) skips the sequence.  Only output
 *             rows inside the windows are written (o's other rows are left as
 *             they are), and only V of keys before each window's end is read:
 *             a chunk attends, through the map's rows of its own query blocks,
 *             to every earlier chunk's keys and to its own.
 * workspace   at least mf_apply_workspace_bytes(...) bytes.
 * Errors: MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_WORKSPACE, MF_ERR_HIP. */
mf_status mf_apply_translated_paged(void *stream, const mf_bsr_map *map, const float *W,
                                    int32_t Ht, const mf_paged_v *pv, int32_t Hkv, int32_t d,
                                    const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                                    int32_t nseq, const int32_t *window_host,
                                    const int32_t *window_dev, int32_t renorm, float *o,
                                    void *workspace, size_t workspace_bytes);

/* Device workspace bytes mf_dense_ref_attention needs (transposed V, padded per
 * sequence to 256-token blocks).  0 if invalid. */
size_t mf_dense_workspace_bytes(int32_t Hkv, const int32_t *cu_seqlens_host, int32_t nseq,
                                int32_t d);

/* Dense causal attention for recomputed heads (MapFlow §4; AttnCache guide,
 * "The Quadratic Self-Attention Cost"):
 *   O_h = softmax(Q_h K_g^T / sqrt(d) + bias) V_g,   g = h / (Hq / Hkv).
 * q [Hq][T][d] and k [Hkv][T][d] in qk_dtype; v [Hkv][T][d] bf16; o [Hq][T][d]
 * fp32.  No map is read or written.
 * Precision: products on bf16 MFMA with fp32 accumulation; P is rounded to
 * bf16 for the P V product.  With bf16 q, q times log2(e)/sqrt(d) is rounded
 * to bf16 once before the product (fp32 q keeps the scale in fp32).
 * Errors: MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_WORKSPACE, MF_ERR_HIP. */
mf_status mf_dense_ref_attention(void *stream, const void *q, const void *k, const void *v,
                                 mf_dtype qk_dtype, int32_t Hq, int32_t Hkv, int32_t d,
                                 const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                                 int32_t nseq, const mf_logit_bias *bias, float *o,
                                 void *workspace, size_t workspace_bytes);

/* Device workspace bytes mf_tv_distance needs (0 if the arguments are invalid). */
size_t mf_tv_distance_workspace_bytes(const int32_t *cu_seqlens_host, int32_t nseq, int32_t B);

/* Total-variation distance between the translated map and a receiver's own map,
 * per query row, for choosing which receiver layers to recompute (MapFlow §3.3:
 * layer-wise TV distance profiled offline).
 *
 *   tv[t][i] = 1/2 sum_j | A~_t[i,j] - A_t[i,j] |
 *
 * A~_t is the translated map exactly as mf_apply_translated uses it
 * (sum_h W[t,h] A_hat_h[i,j] / kmass_h[i] with `renorm`, W[t,h] A_hat_h[i,j]
 * without; zero outside the kept blocks); A_t is the receiver's causal
 * softmax(q_t k_g(t)^T / sqrt(d) + bias), g(t) = floor(t * Hkr / Ht).  Neither
 * map is materialised.  A layer's score is the mean of tv over rows and heads.
 *
 * map         compressed sender map (either tile format); read only.
 * W           [Ht][Hs] fp32, device.
 * q, k        receiver queries [Ht][T][d] and keys [Hkr][T][d], dtype qk_dtype.
 * bias        host, may be NULL: the receiver's logit offsets.
 * tv          [Ht][T] fp32, device, written for every token.
 * workspace   device, at least mf_tv_distance_workspace_bytes(...) bytes.
 * Errors: MF_ERR_INVALID_ARG, MF_ERR_UNSUPPORTED, MF_ERR_WORKSPACE, MF_ERR_HIP. */
mf_status mf_tv_distance(void *stream, const mf_bsr_map *map, const float *W, int32_t Ht,
                         const void *q, const void *k, mf_dtype qk_dtype, int32_t Hkr, int32_t d,
                         const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                         int32_t nseq, const mf_logit_bias *bias, int32_t renorm, float *tv,
                         void *workspace, size_t workspace_bytes);

/* Waits for `stream`, then returns the map's device status (MF_OK or
 * MF_ERR_CAPACITY) and, if nnz_out is not NULL, stores the kept-tile count
 * there (host).  The only call that synchronises.  MF_ERR_HIP if a HIP call
 * failed. */
mf_status mf_read_status(void *stream, const mf_bsr_map *map, int64_t *nnz_out);

/* Static text for a status code. */
const char *mf_status_string(mf_status status);

#ifdef __cplusplus
}
#endif

#endif /* MAPFLOW_H */
