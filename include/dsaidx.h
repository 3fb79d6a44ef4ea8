/*
 * dsaidx.h -- C ABI of the MI355X (gfx950) lightning-indexer library.
 *
 * The DeepSeek Sparse Attention lightning indexer scores, for every query
 * token t and every history token s, the relevance
 *
 *     I[t,s] = sum_{i<H} w[t,i] * ReLU( q[t,i] . k[s] / sqrt(D) )
 *
 * with H index heads on the query side and ONE D-wide key per token shared by
 * all heads, and keeps the top-k positions s of each query (the "token
 * selector").  Formula: "From principle to code -- DeepSeek-V3.2 lightning
 * indexer", section 2.1 (core formula) and "Lightning Indexer explained",
 * section 4 (scoring formula; multi-head on the query side only).  Selection:
 * "Lightning Indexer explained", section 1 (top-k of k = 2048 positions) and
 * section 2.3 (at most min(k, #history) positions come back).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer owned by the caller, row-major
 *   and contiguous unless a stride is given.  The library allocates nothing
 *   and keeps no state between calls beyond one-time, per-device set-up
 *   (kernel attributes, an occupancy query, the address of the no-alloc
 *   entry point's scratch), made thread-safely on first use; scratch memory
 *   is the caller's `workspace` (size from the matching *_workspace_bytes
 *   query; it may be NULL when that size is 0), except for
 *   indexer_prefill_noalloc below.
 * - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *   enqueue work and return; results are valid after the caller synchronises
 *   the stream.
 * - Scores are fp32.  A selected position's score is the fp32 score of that
 *   position.  Padding slots hold index -1 and score -inf.
 * - Tie rule: among equal scores the lower position wins (-0.0 equals +0.0).
 *   The order of the selected positions inside a row is unspecified; the
 *   valid entries of a row come first, then the padding.
 * - Errors: every argument check runs on the host before any launch; a
 *   non-OK status means nothing was enqueued and no output was written.
 *   DSAIDX_ERR_HIP means a launch failed (text in dsaidx_last_error()).
 *   The library never aborts, exits or prints.
 * - Undefined behaviour (not checked): NaN inputs, device arrays shorter than
 *   stated, block-table entries outside [0, num_pages), context lengths
 *   outside [0, max_pages_per_seq * page_size], negative fp8 scales.
 *
 * Input formats (dsaidx_dtype)
 * ----------------------------
 *   DSAIDX_F32      IEEE binary32.
 *   DSAIDX_BF16     bfloat16 bit patterns (uint16).
 *   DSAIDX_FP8_E4M3 OCP FP8 E4M3FN codes (uint8: bias 7, max 448, no Inf,
 *                   S.1111.111 = NaN).  Each row carries an fp32 scale: the
 *                   value of a code is decode(code) * scale.  The pages keep
 *                   the indexer keys in FP8 ("Lightning Indexer explained",
 *                   section 5; "Study MLA Indexer", data-flow diagram); the
 *                   per-row scale is this library's storage convention.
 */
#ifndef DSAIDX_H
#define DSAIDX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSAIDX_OK = 0,
    DSAIDX_ERR_NULL = 1,        /* a required pointer is NULL                     */
    DSAIDX_ERR_SHAPE = 2,       /* a size is non-positive or inconsistent         */
    DSAIDX_ERR_DTYPE = 3,       /* unknown dtype code                             */
    DSAIDX_ERR_UNSUPPORTED = 4, /* valid request outside the supported ranges     */
    DSAIDX_ERR_WORKSPACE = 5,   /* workspace smaller than the query returned      */
    DSAIDX_ERR_HIP = 6          /* a HIP launch failed                            */
} dsaidx_status;

typedef enum {
    DSAIDX_F32 = 0,
    DSAIDX_BF16 = 1,
    DSAIDX_FP8_E4M3 = 2
} dsaidx_dtype;

/*
 * indexer_prefill -- score every causal pair of B sequences of L tokens and
 * select the top-k history positions of every token.
 *
 * Passage: the core formula ("From principle to code", section 2.1) evaluated
 * for all query tokens at once, with the causal mask of that page's listing
 * (section 3: the lower-triangular mask keeps s <= t; masked scores are -inf)
 * and its top-k over the masked rows.  Row t therefore has t+1 valid
 * positions; rows with t+1 <= topk return all of them, then -1 padding.
 *
 *   q         [B][L][H][D] in qk_dtype
 *   q_scale   [B][L][H] fp32 when qk_dtype is FP8 (one scale per query-head
 *             row), else must be NULL
 *   k         [B][L][D] in qk_dtype (one key per token, shared by all heads)
 *   k_scale   [B][L] fp32 when qk_dtype is FP8, else must be NULL
 *   w         [B][L][H] fp32 head weights (any finite values)
 *   topk_idx  out [B][L][topk] int32
 *   topk_score out [B][L][topk] fp32, or NULL
 *   scores    out [B][L][L] fp32 full score matrix (-inf above the diagonal),
 *             or NULL.  Large L costs B*L*L*4 bytes of HBM writes; the fused
 *             path never writes it unless asked.
 *
 * Supported: 1 <= B, 1 <= L <= 131072, H a multiple of 4 in [4, 64],
 * D in {32, 64, 128}, 1 <= topk <= 2048.  bf16/fp8 with D = 128 and H a
 * multiple of 16 take the fused MFMA path, which stages the keys through LDS
 * and needs a workspace per key (64-padded): fp8 5 bytes, 256-byte rounded
 * (a per-key operand scale and the key scale adjusted to it); bf16 260 bytes
 * (the adjusted scale and the key scaled into [-1, 1]).
 * Other shapes score into a B*L*L fp32 matrix (the `scores` output if
 * given, else workspace) and select from it.  The workspace is caller-owned
 * device memory, 16-byte aligned, at least indexer_prefill_workspace_bytes()
 * long (else DSAIDX_ERR_WORKSPACE); its contents are scratch.
 */
dsaidx_status indexer_prefill(const void* q, const float* q_scale,
                              const void* k, const float* k_scale,
                              int qk_dtype, const float* w,
                              int B, int L, int H, int D, int topk,
                              int32_t* topk_idx, float* topk_score, float* scores,
                              void* workspace, size_t workspace_bytes, void* stream);

size_t indexer_prefill_workspace_bytes(int B, int L, int H, int D, int topk, int qk_dtype,
                                       int want_scores);

/*
 * indexer_prefill_noalloc -- indexer_prefill for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments, outputs and results
 * as indexer_prefill, without a workspace argument.  Its scratch is a device
 * array inside the library, one per GPU, of
 * indexer_prefill_noalloc_scratch_bytes() bytes (32 MiB), held from the
 * library's first use on that GPU until the process ends.  A call whose
 * indexer_prefill_workspace_bytes() exceeds it returns
 * DSAIDX_ERR_UNSUPPORTED before any launch: fp8 inputs up to about 6.7M keys
 * (B times the 64-padded L), bf16 up to about 129k keys, the other shapes
 * up to B*L*L*4 bytes unless `scores` is given.  The call makes no hipMalloc,
 * hipFree or other allocating call.  Every call on one GPU uses the same
 * scratch: calls that overlap on one GPU (on different streams, or from
 * different threads) race and give undefined results; calls ordered on one
 * stream are safe, since each call rewrites what it reads before reading it.
 */
dsaidx_status indexer_prefill_noalloc(const void* q, const float* q_scale,
                                      const void* k, const float* k_scale,
                                      int qk_dtype, const float* w,
                                      int B, int L, int H, int D, int topk,
                                      int32_t* topk_idx, float* topk_score, float* scores,
                                      void* stream);

size_t indexer_prefill_noalloc_scratch_bytes(void);

/*
 * indexer_decode_paged -- one decode step for B queries, each scoring its
 * whole cached context.
 *
 * Passage: "Lightning Indexer explained", section 2 (decode walkthrough): the
 * current query is dotted against every row of the indexer key cache, giving
 * one score per history position, then top-k; section 2.3: at most
 * min(k, context) positions.  Query b sits at position context_lens[b]-1 and
 * sees the positions s in [0, context_lens[b]).  Logical position s of query
 * b lives in page block_table[b][s / page_size], slot s % page_size of the
 * shared page pool (paging is this library's layout of that cache).
 *
 *   q            [B][H][D] bf16 (q_dtype must be DSAIDX_BF16).  The scan
 *                multiplies the query as a bf16 MFMA operand; an fp32 query
 *                would have to be rounded to bf16 first, which changes its
 *                scores, so DSAIDX_F32 returns DSAIDX_ERR_UNSUPPORTED rather
 *                than rounding silently (a caller who wants that rounding
 *                converts explicitly, and gets the rounded query's scores)
 *   w            [B][H] fp32
 *   k_cache      [num_pages][page_size][D] FP8 E4M3 codes
 *   k_scale      [num_pages][page_size] fp32, one scale per cached token
 *   block_table  [B][max_pages_per_seq] int32 page ids
 *   context_lens [B] int32, each in [0, max_context_len]
 *   max_context_len  host-side upper bound of context_lens (sizes the launch
 *                and the workspace); <= max_pages_per_seq * page_size
 *   topk_idx     out [B][topk] int32;  topk_score out [B][topk] fp32 or NULL
 *   workspace    indexer_decode_paged_workspace_bytes(B, max_context_len, H,
 *                D, topk) bytes of caller-owned device memory, 16-byte
 *                aligned: candidate scores and positions (8 bytes per
 *                position of max_context_len, 64-padded, per query), then 256
 *                bytes of counters per query, then B + 1 page offsets.  Its
 *                contents on entry do not matter: the call clears its
 *                counters before using them, so a workspace may hold anything
 *                and may be reused by any later call.  Two calls in flight
 *                on one workspace at once race.
 *
 * Supported: H a multiple of 16 in [16, 64], D = 128, page_size = 64,
 * 1 <= topk <= 2048, max_context_len <= 131072 (larger needs no change but
 * is untested).
 */
dsaidx_status indexer_decode_paged(const void* q, int q_dtype, const float* w,
                                   const uint8_t* k_cache, const float* k_scale,
                                   const int32_t* block_table, int max_pages_per_seq,
                                   const int32_t* context_lens, int max_context_len,
                                   int B, int H, int D, int page_size, int num_pages, int topk,
                                   int32_t* topk_idx, float* topk_score,
                                   void* workspace, size_t workspace_bytes, void* stream);

size_t indexer_decode_paged_workspace_bytes(int B, int max_context_len, int H, int D, int topk);

/*
 * indexer_prefill_chunk_paged -- chunked prefill of a serving batch: for each
 * of B sequences, a chunk of new query tokens at its own positions, scored
 * against that sequence's paged FP8 key cache, which already holds every key
 * up to the chunk's last position (the chunk's own keys included), with the
 * top-k of every query.
 *
 * Passage: the core formula and causal top-k of indexer_prefill, evaluated
 * for a run of rows of each sequence; the keys come from the indexer cache,
 * which each token's key enters before that token is scored ("Lightning
 * Indexer explained", sections 2.1 and 2.4 of the decode walkthrough; "Study
 * MLA Indexer", the notes on its two caches).  Query row cu_seqlens_q[b] + i
 * is position p = q_start[b] + i of sequence b and sees the p + 1 positions
 * 0 .. p: its result equals indexer_prefill's row p over the whole sequence.
 *
 *   q            [T][H][D], the sequences' chunks packed one after another:
 *                FP8 E4M3 codes with q_scale [T][H] fp32 (q_dtype
 *                DSAIDX_FP8_E4M3), or bf16 with q_scale NULL (q_dtype
 *                DSAIDX_BF16; scored against the cache's fp8 keys widened
 *                exactly to bf16);  w [T][H] fp32
 *   cu_seqlens_q [B+1] int32 (device): sequence b's rows are
 *                cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; cu_seqlens_q[0] = 0,
 *                nondecreasing, cu_seqlens_q[B] = T (a sequence may have none)
 *   q_start      [B] int32 (device): position of sequence b's first row
 *   k_cache      [num_pages][page_size][D] E4M3FN codes, k_scale
 *                [num_pages][page_size] fp32 (as indexer_kcache_append writes)
 *   block_table  [B][max_pages_per_seq] int32 page ids; position s of
 *                sequence b is page block_table[b][s / page_size], slot
 *                s % page_size
 *   T            number of query rows (host value, = cu_seqlens_q[B])
 *   max_kv_len   host-side bound: q_start[b] + (its row count) <= max_kv_len
 *                for every b, and max_kv_len <= max_pages_per_seq * page_size
 *                (a sequence beyond it sees only its first max_kv_len keys)
 *   topk_idx     out [T][topk] int32 (absolute positions, -1 padded);
 *   topk_score   out [T][topk] fp32 or NULL
 *   workspace    indexer_prefill_chunk_paged_workspace_bytes(B, T,
 *                max_kv_len, q_dtype) bytes of caller-owned device memory,
 *                16-byte aligned: per key up to max_kv_len (64-padded) per
 *                sequence 5 bytes for fp8 queries (256-byte rounded) or 260
 *                bytes for bf16 queries (the keys widened to bf16), then 8
 *                bytes per 8-row block (the launch plan)
 *
 * Supported: H a multiple of 16 in [16, 64], D = 128, page_size = 64,
 * 1 <= topk <= 2048, max_kv_len <= 131072.
 */
dsaidx_status indexer_prefill_chunk_paged(const void* q, const float* q_scale, int q_dtype, const float* w,
                                          const int32_t* cu_seqlens_q, const int32_t* q_start,
                                          const uint8_t* k_cache, const float* k_scale,
                                          const int32_t* block_table, int max_pages_per_seq, int num_pages,
                                          int B, int T, int max_kv_len, int H, int D, int page_size, int topk,
                                          int32_t* topk_idx, float* topk_score,
                                          void* workspace, size_t workspace_bytes, void* stream);

size_t indexer_prefill_chunk_paged_workspace_bytes(int B, int T, int max_kv_len, int q_dtype);

/*
 * indexer_kcache_append -- quantise T new keys to FP8 and write them into the
 * paged indexer key cache that indexer_decode_paged reads.
 *
 * Passage: "Lightning Indexer explained", sections 2.1 and 2.4 of the decode
 * walkthrough (each token's key is appended to the indexer cache once, when
 * that token is processed; later steps only read it) and section 5
 * (Indexer-Cache); "Study MLA Indexer", the data-flow diagram (the key path
 * ends in an FP8 quantisation) and the notes on its two caches (the cache is
 * updated before the scoring decision).  The pages fix neither the FP8
 * flavour nor the scaling; this library stores E4M3FN codes with one fp32
 * scale per token:
 *   scale  = max_d |k_d| / 448 (binary32 division; 1 for an all-zero key)
 *   code_d = the E4M3FN value nearest to k_d / scale (binary32 quotient),
 *            ties to the even code, magnitudes above 448 saturated, sign kept
 * so decode(code_d) * scale is within half a code step of k_d.
 *
 *   k            [T][D] new keys in k_dtype (DSAIDX_BF16 or DSAIDX_F32),
 *                16-byte aligned
 *   seq_ids      [T] int32 sequence (row of block_table) of each key; a key
 *                whose id lies outside [0, B) is skipped (-1 marks padding)
 *   positions    [T] int32 position of each key in its sequence; a key whose
 *                position lies outside [0, max_pages_per_seq * page_size) is
 *                skipped
 *   block_table  [B][max_pages_per_seq] int32 page ids (the decode layout:
 *                position p lives in page block_table[b][p / page_size],
 *                slot p % page_size)
 *   k_cache      [num_pages][page_size][D] E4M3FN codes, updated in place
 *   k_scale      [num_pages][page_size] fp32, updated in place
 * Slots no key addresses are not touched.  Two keys with the same (sequence,
 * position) in one call leave one of them, unspecified which.  T = 0 is a
 * no-op.  No workspace.
 *
 * Supported: D = 128, page_size = 64, k_dtype BF16 or F32, 0 <= T.
 */
dsaidx_status indexer_kcache_append(const void* k, int k_dtype, const int32_t* seq_ids,
                                    const int32_t* positions, const int32_t* block_table, int B,
                                    int max_pages_per_seq, uint8_t* k_cache, float* k_scale, int num_pages,
                                    int T, int D, int page_size, void* stream);

/*
 * indexer_topk_gather -- the selection's consumer: the rows of a paged latent
 * cache at each query's selected positions, gathered contiguously.
 *
 * Passage: "Study MLA Indexer", the data-flow diagram's last step (the sparse
 * attention gathers the latent c^KV at the top-k positions) and the first of
 * its "three whys" (a decode step then moves k * d_c elements, not the whole
 * context).  The latent cache is taken to share the indexer cache's paging:
 * position s of query b lives in page block_table[b][s / page_size], slot
 * s % page_size.  Rows are opaque bytes.
 *
 *   latent_cache  [num_pages][page_size][row_bytes], 16-byte aligned
 *   block_table   [B][max_pages_per_seq] int32 page ids
 *   topk_idx      [B][topk] int32 positions, e.g. indexer_decode_paged's
 *                 output; -1, or a position outside
 *                 [0, max_pages_per_seq * page_size), gives a zero row
 *   out           out [B][topk][row_bytes], 16-byte aligned
 * No workspace.
 *
 * Supported: page_size = 64, row_bytes a multiple of 16 in [16, 65536].
 */
dsaidx_status indexer_topk_gather(const void* latent_cache, int row_bytes, const int32_t* block_table,
                                  int max_pages_per_seq, int num_pages, int page_size,
                                  const int32_t* topk_idx, int B, int topk, void* out, void* stream);

/*
 * indexer_topk_gather_layers -- Index Share: one selection, gathered from
 * the latent caches of several layers in one launch.
 *
 * Passage: "Lightning Indexer explained", section 1, question 4 of the Q&A
 * (Index Share: the top-k is computed at F layers and reused by S layers,
 * which skip their own indexer) and section 3 (the selection I is reused
 * across layers).  The reusing layers read their own latent caches at the
 * shared positions; every layer's cache shares the block table and row
 * size.  Layer l's output equals indexer_topk_gather of latent_caches[l]
 * with the same table and indices; the indices and page ids are read once
 * for all layers.
 *
 *   latent_caches  HOST array [n_layers] of device pointers, each
 *                  [num_pages][page_size][row_bytes], 16-byte aligned
 *   outs           HOST array [n_layers] of device pointers, each out
 *                  [B][topk][row_bytes], 16-byte aligned
 *   block_table, topk_idx, B, topk, row_bytes: as indexer_topk_gather
 * The pointer arrays are read during the call only.  No workspace.
 *
 * Supported: 1 <= n_layers <= 64, page_size = 64, row_bytes a multiple of
 * 16 in [16, 65536].
 */
dsaidx_status indexer_topk_gather_layers(const void* const* latent_caches, void* const* outs, int n_layers,
                                         int row_bytes, const int32_t* block_table, int max_pages_per_seq,
                                         int num_pages, int page_size, const int32_t* topk_idx, int B, int topk,
                                         void* stream);

/*
 * topk_select -- the token selector on its own: top-k of each row of a score
 * matrix.
 *
 * Passage: the top-k step of "From principle to code", section 3 (top-k over
 * the masked score rows) with the tie and short-row rules above.  Row r's
 * valid entries are its first row_len[r] columns (all `cols` if row_len is
 * NULL); entries past that are never read.
 *
 *   scores   [rows] rows of `cols` fp32 values, row r starting at
 *            scores + r * row_stride (row_stride >= cols, in elements)
 *   row_len  [rows] int32 in [0, cols], or NULL
 *   idx_out  out [rows][topk] int32;  val_out out [rows][topk] fp32 or NULL
 *
 * Supported: 1 <= rows, 1 <= cols <= 4194304, 1 <= topk <= 2048.
 */
dsaidx_status topk_select(const float* scores, int rows, int cols, int64_t row_stride,
                          const int32_t* row_len, int topk,
                          int32_t* idx_out, float* val_out,
                          void* workspace, size_t workspace_bytes, void* stream);

size_t topk_select_workspace_bytes(int rows, int cols, int topk);

/*
 * dsaidx_probe_mfma, dsaidx_probe_page_read -- measurement probes.  They
 * compute nothing of the method: they measure what this GPU delivers for
 * the two resources the indexer's kernels are bound by, so a kernel can be
 * reported against a measured peak beside the published one.
 *
 * dsaidx_probe_mfma: `blocks` workgroups of 256 threads; each wave runs
 * `iters` rounds of 8 independent MFMAs of one shape:
 *   kind 0  v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3 (65536 flop each)
 *   kind 1  v_mfma_f32_16x16x32_bf16 (16384 flop each)
 *   kind 2  v_mfma_f32_16x16x32_f16 (16384 flop each)
 * so one call performs blocks * 4 * iters * 8 MFMAs.
 *
 * dsaidx_probe_page_read: reads pages page_ids[0..n) of a paged fp8 key
 * cache laid out as indexer_decode_paged reads it (page = 64 rows of 128
 * code bytes, 8192 B, plus its 64 fp32 scales, 256 B) with the decode
 * scan's load layout, `blocks` workgroups of 256 threads: 8448 * n bytes
 * per call.
 *
 *   out  [blocks * 256] fp32 device array (values carry no meaning)
 * Supported: 1 <= blocks <= 65536, 1 <= iters <= 1 << 20, 1 <= n.
 */
dsaidx_status dsaidx_probe_mfma(int kind, int blocks, int iters, float* out, void* stream);
dsaidx_status dsaidx_probe_page_read(const uint8_t* k_cache, const float* k_scale, const int32_t* page_ids, int n,
                                     int blocks, float* out, void* stream);

/* Static text for a status code. */
const char* dsaidx_status_string(int status);

/* Detail of the last non-OK status returned on the calling thread
 * (which argument, which limit, or the HIP error string).  Thread-local,
 * valid until the next call on the same thread. */
const char* dsaidx_last_error(void);

/* Library version as an integer: major * 10000 + minor * 100 + patch. */
int dsaidx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSAIDX_H */
