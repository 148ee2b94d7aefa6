/*
 * hcs.h -- C ABI of the hybrid compressed sparse attention hot path for MI355X (gfx950).
 *
 * One step of a DeepSeek-V4-style compressed attention layer, as described on the pages
 * "DeepSeek V4 Attention: Code Reading Map" (sections "How Does Compression Actually Work?",
 * "Phase 2" and "Phase 3: forward_mqa()") and the "DeepSeek V4.1 attention" API page:
 *
 *   hcs_compress_kv           the KV compressor: every block of m raw tokens becomes one
 *                             compressed entry (per-channel softmax of the gate logits over
 *                             the block, weighted sum of the raw KV rows), stored in the
 *                             compressed cache in its format;
 *   hcs_compress_kv_full      the same with the CSA overlapping window, RMSNorm and RoPE;
 *   hcs_index_topk            the Lightning Indexer of CSA layers: scores of every visible
 *                             compressed entry, I = sum_h w_h * ReLU(q_h . k), and the top-k;
 *   hcs_index_topk_chunk      the same for a chunk of consecutive queries of one sequence;
 *   hcs_index_topk_cand       the same with two-level candidate filtering (publish or follow
 *                             the top blocks of compressed positions);
 *   hcs_index_topk_compress   hcs_index_topk and hcs_compress_kv of one decode step in one
 *                             launch (they touch disjoint data);
 *   hcs_index_scores_compress the indexer's scores without the top-k (and the compressor);
 *   hcs_sparse_mla_decode     single-KV-head attention of every query head over the query's
 *                             sliding window plus its selected (CSA) or all visible (HCA)
 *                             compressed entries, K = V = the shared row;
 *   hcs_sparse_mla_decode_select  the same for CSA with the top-k of the indexer scores taken
 *                             inside the attention launch;
 *   hcs_sparse_mla_prefill_chunk  the same for a chunk of consecutive queries of one sequence;
 *   hcs_qnorm_rope_kv_insert  readies the new tokens' query heads (optional per-head RMSNorm,
 *                             RoPE) and writes their rotated KV rows into the sliding-window
 *                             cache;
 *   hcs_indexer_q_prep        the indexer queries of new tokens (RoPE, quantization to the key
 *                             cache's format) and their head weights;
 *   hcs_indexer_k_store       the indexer keys of new compressed entries (RMSNorm, RoPE,
 *                             quantization), stored in the indexer key cache.
 *
 * Conventions shared by every call
 *   - Pointers are device pointers unless marked "host". The caller owns every buffer; the
 *     library allocates nothing and keeps no state between calls except the thread-local
 *     error text and the per-device error word (hcs_device_errors).
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream). Arguments are validated on the host before any launch; a non-OK
 *     status means nothing was launched, and hcs_last_error() describes why.
 *   - Device-side faults, if any, surface at the caller's next synchronisation.
 *   - Positions are absolute token positions (int32). Compressed entry i of a sequence covers
 *     positions m*i .. m*i+m-1 and is visible to a query at position p when m*i+m-1 <= p, so
 *     n_visible(p) = (p + 1) / m. The sliding window of a query at p is positions
 *     max(0, p-window+1) .. p (its own token included).
 *
 * Paged caches (hcs_paged)
 *   A cache is a pool of pages of HCS_PAGE_ROWS = 64 rows. Logical row r of sequence s lives
 *   in page page_table[s * pt_stride + r / 64] at slot r % 64. Logical rows are absolute
 *   positions for the sliding-window cache and entry indices for the compressed and indexer
 *   caches. A negative page id (e.g. -1) means "not resident": reads of such a row are skipped
 *   (the row does not take part), writes are dropped. A page id >= num_pages is an error in
 *   the caller's data: the row is handled as not resident and HCS_DEVERR_PAGE_RANGE is set in
 *   the device error word (hcs_device_errors).
 *   Inside a page, each field of the 64 rows is stored contiguously (structure of arrays):
 *     HCS_FMT_BF16  dim D : [64][D] bf16                                  (2*D B per row)
 *     HCS_FMT_FP8DS dim 512: [64][448] e4m3 | [64][64] bf16 | [64][8] B    (584 B per row)
 *                   latent dim c (< 448) = e4m3(code) * 2^(scale[c/64] - 127); bytes 0..6 of
 *                   the 8-byte field are the UE8M0 scales, byte 7 is padding (written 0);
 *                   dims 448..511 are the bf16 rotary dims.
 *     HCS_FMT_MXFP4 dim D  : [64][D/2] packed e2m1 | [64][D/32] UE8M0     (68 B per row, D=128)
 *                   element 2j is the low nibble of byte j, 2j+1 the high nibble; element c
 *                   is scaled by 2^(scale[c/32] - 127).
 *     HCS_FMT_FP8IX dim 128: [64][128] e4m3 | [64] float32 scale          (132 B per row)
 *                   element c = e4m3(code c) * scale (an indexer key format).
 *     HCS_FMT_MXFP8 dim 512: [64][512] e4m3 | [64][16] UE8M0                (528 B per row)
 *                   element c = e4m3(code c) * 2^(scale[c/32] - 127) (the V4.1 KV record).
 *     HCS_FMT_NVFP4 dim 512: [64][256] packed e2m1 | [64][32] e4m3 scales   (288 B per row)
 *                   element 2j in the low nibble of byte j; element c = e2m1(c) *
 *                   e4m3(scale[c/16]) (the V4.1 compressed record).
 *   e4m3 is OCP FP8 E4M3 (max 448, no infinities), e2m1 is OCP MX FP4, UE8M0 is 2^(b-127).
 */
#ifndef HCS_H
#define HCS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HCS_ABI_VERSION 1
#define HCS_PAGE_ROWS 64

typedef enum {
  HCS_OK = 0,
  HCS_ERR_INVALID_ARG = 1,        /* a null pointer, a negative size, a bad enum value       */
  HCS_ERR_UNSUPPORTED = 2,        /* a valid combination this library does not implement     */
  HCS_ERR_WORKSPACE_TOO_SMALL = 3,
  HCS_ERR_HIP = 4                 /* a HIP launch error (text in hcs_last_error())            */
} hcs_status;

typedef enum {
  HCS_FMT_BF16 = 0,
  HCS_FMT_FP8DS = 1,
  HCS_FMT_MXFP4 = 2,
  HCS_FMT_FP8IX = 3,
  HCS_FMT_MXFP8 = 4,
  HCS_FMT_NVFP4 = 5
} hcs_fmt;
typedef enum { HCS_IN_BF16 = 0, HCS_IN_F32 = 1 } hcs_in_dtype;

typedef struct {
  void* base;                 /* pool of num_pages pages in the layout of `fmt`           */
  const int32_t* page_table;  /* [num_seqs * pt_stride] int32 page ids                    */
  int32_t pt_stride;          /* page-table entries per sequence (> 0)                    */
  int32_t num_pages;          /* pages in the pool                                        */
  int32_t fmt;                /* hcs_fmt                                                  */
  int32_t dim;                /* row dimension (512 for HCS_FMT_FP8DS)                    */
} hcs_paged;

/* Thread-local text of the last non-OK status returned on this thread ("" if none). */
const char* hcs_last_error(void);

/* Device error word. Invalid data found on the device by a kernel (where the host cannot see
 * it before the launch) sets bits in a per-device word that stays set until read and cleared
 * here; the kernel goes on as stated for the case and the call's status is unaffected.
 *   HCS_DEVERR_PAGE_RANGE  a page-table entry >= num_pages was met (a corrupt page table): the
 *                          row is treated as not resident (reads skipped, writes dropped).
 *   HCS_DEVERR_PAIR_WAIT   the prefill attention's two waves of a head pair did not exchange
 *                          their block maxima within the bounded wait: some outputs of that
 *                          call are wrong.
 * hcs_device_errors waits for all work on the current device (hipDeviceSynchronize), ORs the
 * device's bits into *bits (host pointer) and, if clear != 0, resets them to zero. Returns
 * HCS_ERR_INVALID_ARG for a null bits, HCS_ERR_HIP if a HIP call fails. */
#define HCS_DEVERR_PAGE_RANGE 0x1u
#define HCS_DEVERR_PAIR_WAIT 0x2u
hcs_status hcs_device_errors(uint32_t* bits, int clear);
/* HCS_ABI_VERSION of the loaded library. */
int hcs_abi_version(void);

/* ------------------------------------------------------------------------------------ */
/* KV compressor.                                                                        */
/* "Code Reading Map", "How Does Compression Actually Work?": for every completed block i */
/* of m tokens, z[j,c] = score[m*i+j, c] + ape[j, c], alpha[., c] = softmax_j z[., c] (per */
/* channel), entry[i, c] = sum_j alpha[j, c] * kv[m*i+j, c]. The float32 state of a      */
/* sequence's trailing partial block carries from one call to the next, so any split of a */
/* token stream into calls gives the same entries.                                       */
/*                                                                                        */
/* kv, score  [T_total, row_stride] rows of in_dtype (HCS_IN_BF16 or HCS_IN_F32); the     */
/*            first d columns are used. Sequence b's new tokens are rows                  */
/*            cu_new[b] .. cu_new[b+1]-1, at positions start_pos[b], start_pos[b]+1, ...  */
/* cu_new     [B+1] int32, non-decreasing, cu_new[0] = 0.                                 */
/* start_pos  [B] int32 >= 0.                                                             */
/* max_new    host: an upper bound of cu_new[b+1]-cu_new[b] (sizes the launch; any value  */
/*            >= 1 is correct, a tight one is fastest).                                   */
/* ape        [m, d] float32 positional encoding added to the gate logits, or NULL (0).   */
/* state      [B, 3*d] float32, in/out: per channel (running max, running sum of          */
/*            exp(z - max), running sum of exp(z - max) * kv) of the block containing     */
/*            position start_pos[b]-1. It is read only when start_pos[b] % m != 0 and is  */
/*            left describing the block of the last new token (reset if that block        */
/*            completed). Sequences with no new tokens are untouched.                     */
/* comp       compressed cache (HCS_FMT_BF16 with dim d, or HCS_FMT_FP8DS, HCS_FMT_MXFP8  */
/*            or HCS_FMT_NVFP4 with d = 512): every entry completed by this call is        */
/*            written at its entry index.                                                  */
/*            fp8_ds: per 64-dim latent block the scale is the smallest power of two 2^e  */
/*            with amax <= 448 * 2^e, codes are round-to-nearest-even of value / 2^e.     */
/*            MXFP8: the same rule per 32 dims over all 512. NVFP4: per 16 dims the scale */
/*            is the e4m3 value nearest amax / 6 (the quotient in float32), codes the      */
/*            nearest-even e2m1 of value / scale saturated to +-6 (0 if the scale is 0).   */
/* dbg        optional [B, dbg_seq_stride] float32 copy of the completed entries before    */
/*            rounding to the cache format: entry i of sequence b at                       */
/*            dbg[b*dbg_seq_stride + (i - start_pos[b]/m) * d]. NULL to skip.             */
/* Constraints: 1 <= d <= 1024, d % 8 == 0, 1 <= m <= 1024, B >= 0.                       */
hcs_status hcs_compress_kv(const void* kv, const void* score, int in_dtype, int64_t row_stride,
                           const int32_t* cu_new, const int32_t* start_pos, int B, int max_new,
                           int d, int m, const float* ape, float* state, hcs_paged comp,
                           float* dbg, int64_t dbg_seq_stride, void* stream);

/* ------------------------------------------------------------------------------------ */
/* The full compressor: "Code Reading Map", "How Does Compression Actually Work?", steps  */
/* 1-7 and "Key design choices". As hcs_compress_kv, plus:                                */
/*   coff = 2 (CSA overlap): kv and score rows are 2d wide; entry i's softmax runs, per   */
/*     channel c, over 2m logits: block i's tokens in columns c (primary series) and      */
/*     block i-1's tokens in columns d + c (overlapping series; entry 0 has only its m),  */
/*     weighting the matching kv values, so a block's tokens feed two entries. ape, when  */
/*     given, is [m, coff * d] and adds by the token's place in its block.                */
/*   norm_weight [d] float32 (or NULL: none): the entry becomes                          */
/*     x / sqrt(mean(x^2) + norm_eps) * norm_weight.                                      */
/*   rope_cos, rope_sin [rope_rows, d_rope / 2] float32 (or both NULL: none): the last    */
/*     d_rope dims are rotated in GPT-J pairs (2j, 2j+1) at the entry's position m * i:   */
/*     (a, b) -> (a cos - b sin, a sin + b cos) with row m * i of the tables. Every        */
/*     emitted entry's position must be below rope_rows (a larger one reads the last row).*/
/* Then the store in comp's format, and dbg holds the values after the epilogue.          */
/* state    [B, 3 * coff * d] float32: zeros for a fresh sequence, else what the previous  */
/*          call left (with coff = 2 a call starting at a block boundary reads the carried */
/*          overlap from it).                                                             */
/* Constraints: as hcs_compress_kv, coff in {1, 2}, row_stride >= coff * d, d <= 1024,     */
/* d_rope even and <= d. Errors as hcs_compress_kv.                                        */
hcs_status hcs_compress_kv_full(const void* kv, const void* score, int in_dtype, int64_t row_stride,
                                const int32_t* cu_new, const int32_t* start_pos, int B, int max_new,
                                int d, int m, int coff, const float* ape, float* state,
                                const float* norm_weight, float norm_eps, const float* rope_cos,
                                const float* rope_sin, int d_rope, int rope_rows, hcs_paged comp,
                                float* dbg, int64_t dbg_seq_stride, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Lightning-Indexer scores and top-k selection (CSA layers).                             */
/* "Code Reading Map", "Aux stream 0 (CSA only)": scores between indexer queries and the  */
/* compressed indexer keys select the top-k compressed entries. Score of entry i for      */
/* query t: I[t,i] = sum_h w[t,h] * max(0, q[t,h,:] . k[i,:]) over i < n_visible(p_t)     */
/* (scale factors are folded into w by the caller). The k largest are selected, ties to   */
/* the smaller index. When n_visible(p_t) <= k every visible entry is selected ("DeepSeek */
/* V4.1 attention" page, short-context rule) and the row is padded with -1.               */
/*                                                                                        */
/* q        keys.fmt == HCS_FMT_BF16 : [N, H_I, d_I] bf16, q_scale = NULL.                */
/*          keys.fmt == HCS_FMT_MXFP4: [N, H_I, d_I/2] packed e2m1 (low nibble first) and */
/*                                     q_scale [N, H_I, d_I/32] UE8M0 bytes.              */
/*          keys.fmt == HCS_FMT_FP8IX: [N, H_I, 128] e4m3 codes and q_scale [N, H_I]      */
/*                                     float32 (passed through the uint8_t pointer).       */
/* w        [N, H_I] float32.                                                             */
/* keys     indexer key cache, dim d_I, by entry index.                                   */
/* q_seq    [N] int32 sequence of each query (page-table row); q_pos [N] int32 position.  */
/* max_pos  host: an upper bound of q_pos (positions above it are read as max_pos).       */
/* out_idx  [N, topk] int32: the selected entry ids, in no particular order, -1 at the    */
/*          tail when fewer than topk entries are visible.                                */
/* out_score [N, topk] float32 scores of out_idx (unspecified where out_idx is -1), or NULL.*/
/* ws       workspace of at least hcs_index_topk_workspace_size(N, max_pos, m, topk) bytes, */
/*          256-byte aligned (score scratch; no initial contents needed). Calls that overlap */
/*          in time must not share it.                                                     */
/* Constraints: H_I in 1..64, d_I in {32, 64, 128} (bf16) or d_I == 128 (mxfp4, fp8ix),   */
/* 1 <= topk <= 4096, (max_pos + 1) / m <= 4194304 visible entries (HCS_ERR_UNSUPPORTED). */
size_t hcs_index_topk_workspace_size(int N, int max_pos, int m, int topk);
hcs_status hcs_index_topk(const void* q, const uint8_t* q_scale, const float* w, hcs_paged keys,
                          const int32_t* q_seq, const int32_t* q_pos, int N, int H_I, int d_I,
                          int m, int topk, int max_pos, int32_t* out_idx, float* out_score,
                          void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Two-level candidate filtering ("DeepSeek V4.1 attention", `DeepseekV4Indexer`: besides  */
/* its own top-k, the indexer of the source layer lists its best blocks of consecutive      */
/* compressed positions, and a consumer layer restricts its top-k to entries inside the     */
/* listed blocks). Arguments and scores as hcs_index_topk, plus cand_block (entries per     */
/* block: block j = entries j*cand_block .. j*cand_block+cand_block-1) and n_cand. Exactly  */
/* one of:                                                                                  */
/*   cand_out [N, n_cand] int32 (source): after the top-k, the n_cand blocks with the       */
/*            largest block score (the max of the block's visible entries' scores), ties to */
/*            the smaller block id, in no particular order, -1 at the tail when the query   */
/*            sees fewer blocks. At most 32768 blocks may be visible to a query.             */
/*   cand_in  [N, n_cand] int32 (consumer): only the visible entries of the listed blocks   */
/*            take part in the top-k (ties to the smaller id); when no more than topk of     */
/*            them exist, all are selected and out_idx is padded with -1. Ids < 0 are        */
/*            skipped; a block must not be listed twice for one query.                       */
/* ws       hcs_index_topk_cand_workspace_size(N, max_pos, m, topk, cand_block, n_cand)     */
/*          bytes, 256-byte aligned.                                                        */
/* Constraints: as hcs_index_topk, cand_block >= 1, 1 <= n_cand <= 4096.                    */
size_t hcs_index_topk_cand_workspace_size(int N, int max_pos, int m, int topk, int cand_block, int n_cand);
hcs_status hcs_index_topk_cand(const void* q, const uint8_t* q_scale, const float* w, hcs_paged keys,
                               const int32_t* q_seq, const int32_t* q_pos, int N, int H_I, int d_I, int m,
                               int topk, int max_pos, int cand_block, int n_cand, const int32_t* cand_in,
                               int32_t* cand_out, int32_t* out_idx, float* out_score, void* ws,
                               size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Lightning-Indexer for a prefill chunk: hcs_index_topk for the Q consecutive queries    */
/* P0 .. P0+Q-1 of sequence `seq` (the chunked prefill of "DeepSeek-V4 Inference on       */
/* Ascend"; the same score and selection, each query with its own n_visible(p)). All      */
/* queries read the same keys, so large chunks (Q >= 256, bf16 keys with d_I == 128,      */
/* H_I % 4 == 0, and at most 32768 visible entries) are scored as one matrix product over */
/* blocks of queries; the results are those of hcs_index_topk with q_seq[t] = seq and     */
/* q_pos[t] = P0 + t, bit for bit.                                                        */
/* q [Q, H_I, ...] and w [Q, H_I] as above; out_idx / out_score [Q, topk] as above.        */
/* ws: hcs_index_topk_workspace_size(Q, P0 + Q - 1, m, topk) bytes, 256-byte aligned.      */
/* Errors: as hcs_index_topk; P0, seq and Q must be >= 0 and P0 + Q - 1 must fit int32.   */
hcs_status hcs_index_topk_chunk(const void* q, const uint8_t* q_scale, const float* w,
                                hcs_paged keys, int seq, int P0, int Q, int H_I, int d_I, int m,
                                int topk, int32_t* out_idx, float* out_score, void* ws,
                                size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ */
/* The indexer and the KV compressor of one decode step in one launch. On the pages the   */
/* compressor and the indexer run side by side ("Code Reading Map", the multi-stream      */
/* overlap of the compressor with the indexer's aux stream): the indexer reads the        */
/* indexer key cache, the compressor writes the KV compressed cache and its state, and    */
/* neither reads what the other writes. This call is hcs_index_topk(q .. out_score, ws)   */
/* followed by hcs_compress_kv(kv .. comp) with dbg = NULL, with the same arguments,      */
/* checks and results; bf16 keys with at most 32768 visible entries, and MXFP4 keys, score */
/* and compress in one grid, other cases launch the two as separate kernels. m_ix is the  */
/* indexer's m                                                                            */
/* (the keys' compression ratio), m the compressor's. `comp` must not be `keys`.          */
/* Errors: those of either call; nothing is launched if either set of arguments fails.    */
hcs_status hcs_index_topk_compress(const void* q, const uint8_t* q_scale, const float* w,
                                   hcs_paged keys, const int32_t* q_seq, const int32_t* q_pos, int N,
                                   int H_I, int d_I, int m_ix, int topk, int max_pos,
                                   int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                                   const void* kv, const void* score, int in_dtype,
                                   int64_t row_stride, const int32_t* cu_new,
                                   const int32_t* start_pos, int B, int max_new, int d, int m,
                                   const float* ape, float* state, hcs_paged comp, void* stream);

/* ------------------------------------------------------------------------------------ */
/* The indexer's scores without the selection ("Code Reading Map", "Aux stream 0 (CSA     */
/* only)": the per-entry scores the top-k is taken over), optionally with the KV          */
/* compressor of the same decode step in the same launch, as in hcs_index_topk_compress.  */
/* For query t: scores[t, i] = sum_h w[t,h] * ReLU(q[t,h] . k_i) for i < n_visible(q_pos[t])*/
/* with the arithmetic of hcs_index_topk (entries from n_visible on are not written).     */
/* With B > 0 it is also hcs_compress_kv(kv .. comp) with dbg = NULL; B = 0 only scores,  */
/* N = 0 only compresses. hcs_sparse_mla_decode_select consumes the scores.               */
/* scores   [N, score_stride] float32, score_stride >= (max_pos + 1) / m_ix.              */
/* Errors: those of hcs_index_topk (without topk, out_idx and ws) and of hcs_compress_kv; */
/* nothing is launched if either set of arguments fails.                                  */
hcs_status hcs_index_scores_compress(const void* q, const uint8_t* q_scale, const float* w,
                                     hcs_paged keys, const int32_t* q_seq, const int32_t* q_pos, int N,
                                     int H_I, int d_I, int m_ix, int max_pos, float* scores,
                                     int64_t score_stride, const void* kv, const void* score,
                                     int in_dtype, int64_t row_stride, const int32_t* cu_new,
                                     const int32_t* start_pos, int B, int max_new, int d, int m,
                                     const float* ape, float* state, hcs_paged comp, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Sparse MLA decode (single shared KV head, MQA).                                        */
/* "Code Reading Map", "Phase 3: forward_mqa()" and "Concrete Trace": each query head     */
/* attends over the query's sliding-window rows plus its selected compressed entries      */
/* (CSA: topk_idx) or all visible ones (HCA: topk_idx == NULL); both sets are attended    */
/* together, without removing raw rows a compressed entry also covers. For head h:        */
/*   l_r = scale * q_h . row_r,  o_h = sum_r e^{l_r} row_r / (sum_r e^{l_r} + e^{sink_h}),  */
/*   lse_h = log(sum_r e^{l_r} + e^{sink_h}); the value of a row is the row itself.        */
/* Selected ids outside [0, n_visible(p)) and -1 are skipped. A query with no row and no  */
/* sink gets o = 0, lse = -inf.                                                           */
/*                                                                                        */
/* q        [N, H, d] bf16 (normalised and rotated upstream).                             */
/* swa      raw KV rows by absolute position (dim d).                                      */
/* comp     compressed entries by index. Format pairs (swa / comp): bf16 / bf16; with      */
/*          d = 512 also fp8_ds / fp8_ds, MXFP8 / MXFP8 and MXFP8 / NVFP4 (the V4.1 records). */
/* topk_idx [N, topk] int32 or NULL (HCA).                                                */
/* q_seq, q_pos  [N] int32.     sink  [H] float32 or NULL (no sink).                      */
/* max_pos  host: an upper bound of q_pos.     scale: softmax scale (d^-1/2 on the pages). */
/* out      [N, H, d] bf16.     lse  [N, H] float32 (natural log) or NULL.                */
/* ws       workspace of hcs_sparse_mla_workspace_size(N, H, d, window, m, topk, max_pos)  */
/*          bytes (topk = 0 for HCA; 0 bytes means none is needed): partial results of the */
/*          split row ranges. Calls that overlap in time must not share it.               */
/* Constraints: d in {128, 512}, 1 <= H <= 128, window >= 0, m >= 1.                      */
size_t hcs_sparse_mla_workspace_size(int N, int H, int d, int window, int m, int topk, int max_pos);
hcs_status hcs_sparse_mla_decode(const void* q, hcs_paged swa, hcs_paged comp,
                                 const int32_t* topk_idx, int topk, const int32_t* q_seq,
                                 const int32_t* q_pos, const float* sink, int N, int H, int d,
                                 int window, int m, int max_pos, float scale, void* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ */
/* hcs_sparse_mla_decode for callers that cannot allocate device memory (code under HIP    */
/* graph capture, serving loops, harnesses that forbid allocation): the same computation,  */
/* arguments and results as hcs_sparse_mla_decode, with no workspace argument. The split   */
/* partials go to a static device array of HCS_NOALLOC_SCRATCH_BYTES inside the library  */
/* (one per device it runs on, held until the process ends); the call allocates nothing   */
/* and calls no allocating routine. A call whose split plan needs more scratch than that   */
/* (hcs_sparse_mla_workspace_size) returns HCS_ERR_WORKSPACE_TOO_SMALL before any launch. */
/* All calls on one device share its scratch: calls that overlap in time on one device    */
/* (several streams) race and give wrong results; calls in order on one stream are safe.  */
#define HCS_NOALLOC_SCRATCH_BYTES (32u << 20)
hcs_status hcs_sparse_mla_decode_noalloc(const void* q, hcs_paged swa, hcs_paged comp,
                                         const int32_t* topk_idx, int topk, const int32_t* q_seq,
                                         const int32_t* q_pos, const float* sink, int N, int H, int d,
                                         int window, int m, int max_pos, float scale, void* out,
                                         float* lse, void* stream);

/* ------------------------------------------------------------------------------------ */
/* hcs_sparse_mla_decode for CSA with the selection inside the attention launch: query    */
/* t's compressed rows are the top-k of its indexer scores scores[t, i], i < n_visible,   */
/* chosen exactly as hcs_index_topk chooses them ("Code Reading Map", "Aux stream 0": the */
/* top-k of the per-entry scores; ties at the k-th score to the smaller ids, every       */
/* visible entry when there are at most topk), so the attended set is that of            */
/* hcs_index_topk followed by hcs_sparse_mla_decode. Each workgroup of a query selects     */
/* the same set and attends its share of it in id order; the result equals the two-call  */
/* path up to the order of the floating-point sums.                                       */
/* scores   [N, score_stride] float32 (hcs_index_scores_compress), score_stride >=        */
/*          n_visible(max_pos).                                                           */
/* sel_idx  [N, topk] int32 or NULL: the selected ids in ascending order, -1 padded.      */
/* Other arguments as for hcs_sparse_mla_decode; ws: hcs_sparse_mla_workspace_size(N, H,  */
/* d, window, m, topk, max_pos) bytes.                                                    */
/* Constraints: d = 512, bf16 swa and comp, 1 <= topk <= 4096 and n_visible(max_pos) <=   */
/* 8192, else HCS_ERR_UNSUPPORTED (use hcs_index_topk and hcs_sparse_mla_decode).         */
hcs_status hcs_sparse_mla_decode_select(const void* q, hcs_paged swa, hcs_paged comp,
                                        const float* scores, int64_t score_stride, int topk,
                                        const int32_t* q_seq, const int32_t* q_pos, const float* sink,
                                        int N, int H, int d, int window, int m, int max_pos,
                                        float scale, void* out, float* lse, int32_t* sel_idx,
                                        void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Sparse MLA for a prefill chunk: hcs_sparse_mla_decode for the Q consecutive queries    */
/* P0 .. P0+Q-1 of sequence `seq` ("DeepSeek-V4 Inference on Ascend", prefill path; the   */
/* chunk bounds the gathered KV). Each query has its own causal n_visible(p) and window;  */
/* the window reaches into the chunk itself, whose raw rows must already be in `swa`, and */
/* the chunk's own completed entries must already be in `comp` (hcs_compress_kv first).   */
/* q [Q, H, d] bf16, topk_idx [Q, topk] or NULL, out [Q, H, d] bf16, lse [Q, H] or NULL.   */
/* ws: hcs_sparse_mla_prefill_workspace_size(...) bytes (0 is valid).                      */
size_t hcs_sparse_mla_prefill_workspace_size(int Q, int H, int d, int window, int m, int topk,
                                             int P0);
hcs_status hcs_sparse_mla_prefill_chunk(const void* q, hcs_paged swa, hcs_paged comp,
                                        const int32_t* topk_idx, int topk, int seq, int P0, int Q,
                                        const float* sink, int H, int d, int window, int m,
                                        float scale, void* out, float* lse, void* ws,
                                        size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Query preparation and sliding-window insert of new tokens: "Code Reading Map", "Default */
/* stream" (the fused q-norm / RoPE / KV insert) and the "DeepSeek V4.1 attention" page's  */
/* `_fused_qnorm_rope_kv_insert`. For token t at position p = tok_pos[t]:                  */
/*   every query head h: when q_norm, q[t,h,:] /= sqrt(mean(q[t,h,:]^2) + eps) (no weight), */
/*     then its last d_rope dims are rotated in GPT-J pairs (2j, 2j+1) at position p:      */
/*     (a, b) -> (a cos - b sin, a sin + b cos) with row p of the tables; written back in   */
/*     place as bf16;                                                                     */
/*   the KV row kv[t, 0..d-1] is rotated the same way (not normalised) and stored as       */
/*     logical row p of sequence tok_seq[t] in `swa`, in its format (bf16; fp8_ds or     */
/*     MXFP8 with the compressor's scale and rounding rules; in fp8_ds the rotary dims are */
/*     the record's bf16 part when d_rope <= 64). kv itself is not modified.               */
/* Values are computed in float32 from the bf16 inputs and rounded once.                  */
/*                                                                                        */
/* q        [N, H, d] bf16, in/out; may be NULL when H == 0 (insert only).                */
/* kv       [N, kv_stride] bf16 rows (kv_stride >= d, a multiple of 8), or NULL: no        */
/*          insert (query preparation only).                                               */
/* tok_seq  [N] int32 page-table row of each token (needed with kv).                       */
/* tok_pos  [N] int32 position of each token; a negative position skips the token.         */
/* rope_cos, rope_sin [rope_rows, d_rope / 2] float32, or both NULL: no rotation. A        */
/*          position at or past rope_rows reads the last row.                              */
/* swa      sliding-window cache (dim d; HCS_FMT_BF16, or HCS_FMT_FP8DS / HCS_FMT_MXFP8    */
/*          with d = 512).                                                                 */
/*          A row whose page is not resident (or past the page table) is not written.      */
/* Tokens must have distinct (tok_seq, tok_pos) pairs: two writes of one row race.         */
/* Constraints: d in {128, 512}, 0 <= H <= 128, eps >= 0, d_rope even in 2..d, q and kv    */
/* 16-byte aligned. Errors: HCS_ERR_INVALID_ARG / HCS_ERR_UNSUPPORTED as stated, before any */
/* launch.                                                                                */
hcs_status hcs_qnorm_rope_kv_insert(void* q, int H, const void* kv, int64_t kv_stride,
                                    const int32_t* tok_seq, const int32_t* tok_pos, int N, int d,
                                    int q_norm, float eps, const float* rope_cos,
                                    const float* rope_sin, int d_rope, int rope_rows, hcs_paged swa,
                                    void* stream);

/* ------------------------------------------------------------------------------------ */
/* Indexer queries of new tokens: "DeepSeek V4.1 attention", `DeepseekV4Indexer.forward_q` */
/* (after the wq_b projection: RoPE and quantization of the query, and the head weights    */
/* times softmax_scale * n_head^-1/2). For token t at position p = tok_pos[t] and head h:   */
/*   the last d_rope dims of q[t,h,:] are rotated in GPT-J pairs at position p, as in       */
/*   hcs_qnorm_rope_kv_insert (no norm), then written in out_fmt:                           */
/*     HCS_FMT_BF16 : q_out [N, H_I, d_I] bf16 (q_out == q rewrites in place), q_scale_out  */
/*                    NULL;                                                                 */
/*     HCS_FMT_MXFP4: q_out [N, H_I, d_I/2] packed e2m1 (element 2j in the low nibble),     */
/*                    q_scale_out [N, H_I, d_I/32] UE8M0 bytes: per 32 values the smallest  */
/*                    2^e with amax <= 6 * 2^e, codes round-to-nearest-even of value / 2^e; */
/*     HCS_FMT_FP8IX: q_out [N, H_I, d_I] e4m3 codes, q_scale_out [N, H_I] float32: per row */
/*                    the smallest power of two s with amax <= 448 * s, codes RNE(value/s); */
/*   w_out[t,h] = w[t,h] * w_scale (w_scale = softmax_scale * H_I^-1/2 on the pages).        */
/* Values are computed in float32 from the bf16 input and rounded once.                   */
/* q [N, H_I, d_I] bf16, w [N, H_I] float32, tok_pos [N] int32 (a negative position skips   */
/* the token: nothing of it is written). rope_cos / rope_sin as hcs_qnorm_rope_kv_insert.   */
/* Constraints: d_I == 128, 1 <= H_I <= 64, q and q_out 16-byte aligned.                   */
hcs_status hcs_indexer_q_prep(const void* q, const float* w, const int32_t* tok_pos, int N, int H_I,
                              int d_I, float w_scale, const float* rope_cos, const float* rope_sin,
                              int d_rope, int rope_rows, int out_fmt, void* q_out,
                              void* q_scale_out, float* w_out, void* stream);

/* ------------------------------------------------------------------------------------ */
/* Indexer keys of new compressed entries: "DeepSeek V4.1 attention",                    */
/* `DeepseekV4Indexer._produce_k` (after the wk projection of the compressor's latent: the  */
/* k_norm RMSNorm, RoPE at the group position, quantization into the paged key cache). For  */
/* row r (entry i = ent_idx[r] of sequence ent_seq[r]):                                    */
/*   k = k_pre[r,:] / sqrt(mean(k_pre[r,:]^2) + eps) * norm_weight, then its last d_rope    */
/*   dims rotated in GPT-J pairs at position m * i, then stored as logical row i of        */
/*   `keys` in its format (bf16; MXFP4 and FP8IX with hcs_indexer_q_prep's rules). A row   */
/*   whose page is not resident (or past the page table), or with i < 0, is not written.    */
/* k_pre [n, k_stride] bf16 (first d_I columns; k_stride >= d_I, a multiple of 8),          */
/* ent_seq, ent_idx [n] int32, norm_weight [d_I] float32.                                   */
/* Constraints: d_I == 128, m >= 1, eps >= 0; rows must name distinct entries.             */
hcs_status hcs_indexer_k_store(const void* k_pre, int64_t k_stride, const int32_t* ent_seq,
                               const int32_t* ent_idx, int n, int d_I, int m,
                               const float* norm_weight, float eps, const float* rope_cos,
                               const float* rope_sin, int d_rope, int rope_rows, hcs_paged keys,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HCS_H */
