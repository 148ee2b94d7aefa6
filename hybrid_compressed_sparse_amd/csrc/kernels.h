// Kernel argument blocks and host-side launchers (implemented in the *.hip files).
#pragma once

#include "common.h"

namespace hcs {

// Host readers of each source file's device error word (HCS_DEVICE_ERROR_WORD): OR the bits
// into *bits and clear them when asked; the caller synchronises the device first.
hipError_t dev_errors_attention(uint32_t* bits, bool clear);
hipError_t dev_errors_compress(uint32_t* bits, bool clear);
hipError_t dev_errors_indexer(uint32_t* bits, bool clear);
hipError_t dev_errors_indexer_prep(uint32_t* bits, bool clear);
hipError_t dev_errors_insert(uint32_t* bits, bool clear);

// ---------------------------------------------------------------- attention
struct AttnArgs {
  const uint16_t* q;          // [N, H, D] bf16
  Paged swa, comp;
  const int32_t* topk_idx;    // [N, topk] or nullptr (all visible entries)
  int topk;
  const int32_t* q_seq;       // [N] or nullptr: then every query is of sequence seq_const
  const int32_t* q_pos;       // [N] or nullptr: then query t is at position p0 + t
  int seq_const, p0;
  const float* sink;          // [H] or nullptr
  int N, H, window, m, nv_cap, pos_cap;
  int nsplit, n_hg, n_h16, rows_per_split;   // n_hg: head groups of a kernel block
  float scale_log2;           // softmax scale * log2(e)
  uint16_t* out;              // [N, H, D] bf16
  float* lse;                 // [N, H] or nullptr
  uint16_t* ws_o;             // [N, n_h16, nsplit, 16, D] bf16 partial outputs: each split's
                              // unnormalised sums relative to its max (nsplit > 1)
  float* ws_ml;               // [N, n_h16, nsplit, 16, 2] partial (max, sum), log2 units
  // rows selected by the kernel itself (topk_idx == nullptr): the top-k of each query's indexer
  // scores [N, score_stride] over its visible entries; the selected ids in ascending order go
  // to sel_out [N, topk] (-1 padded) when it is set
  const float* scores;
  int64_t score_stride;
  int32_t* sel_out;
};

// Most visible entries a query may have when the attention kernel selects its own rows.
constexpr int kSelMax = 8192;

struct AttnPlan {
  int nsplit, n_hg, n_h16, rows_per_split;
  size_t ws_o_bytes, ws_ml_bytes, ws_bytes;
};
AttnPlan attn_plan(int N, int H, int d, int window, int m, int topk, int max_pos);
bool attn_formats_supported(int d, int swa_fmt, int comp_fmt);
hipError_t launch_sparse_mla(const AttnArgs& a, int d, int swa_fmt, int comp_fmt, hipStream_t stream);

// ---------------------------------------------------------------- compressor
struct CompressArgs {
  const void* kv;
  const void* score;
  int in_bf16;
  int64_t row_stride;
  const int32_t* cu_new;
  const int32_t* start_pos;
  int B, d, m, fmt;
  const float* ape;
  float* state;
  uint8_t* comp_base;
  const int32_t* comp_pt;
  int comp_pt_stride, comp_num_pages;
  float* dbg;
  int64_t dbg_stride;
  // the full compressor (launch_compress_full): overlapping window, RMSNorm, RoPE
  int coff;                   // 1, or 2: overlapping window (kv / score rows are 2d wide)
  const float* norm_w;        // [d] or nullptr: no RMSNorm
  float norm_eps;
  const float* rope_cos;      // [rope_rows, d_rope / 2] or nullptr: no RoPE
  const float* rope_sin;
  int d_rope, rope_rows;
};
hipError_t launch_compress(const CompressArgs& a, int max_new, hipStream_t stream);
hipError_t launch_compress_full(const CompressArgs& a, int max_new, hipStream_t stream);

// ---------------------------------------------------------------- query preparation + SWA insert
struct InsertArgs {
  uint16_t* q;                // [N, H, d] bf16, rewritten in place (H may be 0)
  const uint16_t* kv;         // [N, kv_stride] bf16 (first d columns), or nullptr: no insert
  int64_t kv_stride;
  const int32_t* tok_seq;     // [N] page-table row of each token
  const int32_t* tok_pos;     // [N] position of each token (< 0: the token is skipped)
  int N, H, d;
  int q_norm;                 // unit RMS per query head before the rotation
  float eps;
  const float* rope_cos;      // [rope_rows, d_rope / 2] or nullptr: no rotation
  const float* rope_sin;
  int d_rope, rope_rows;
  uint8_t* swa_base;
  const int32_t* swa_pt;
  int swa_pt_stride, swa_num_pages, fmt;
};
hipError_t launch_qrope_insert(const InsertArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- indexer query / key production
struct IxQArgs {
  const uint16_t* q;          // [N, H, 128] bf16
  const float* w;             // [N, H]
  const int32_t* tok_pos;     // [N]
  int N, H, fmt;              // fmt: output format (HCS_FMT_BF16 / MXFP4 / FP8IX)
  float w_scale;
  const float* rope_cos;      // [rope_rows, d_rope / 2] or nullptr
  const float* rope_sin;
  int d_rope, rope_rows;
  uint16_t* q_out16;          // bf16 output
  uint8_t* q_out8;            // MXFP4 / FP8 codes
  uint8_t* q_scale8;          // MXFP4 scale bytes [N, H, 4]
  float* q_scalef;            // FP8 row scales [N, H]
  float* w_out;               // [N, H]
};
hipError_t launch_indexer_q(const IxQArgs& a, hipStream_t stream);

struct IxKArgs {
  const uint16_t* k;          // [n, k_stride] bf16
  int64_t k_stride;
  const int32_t* ent_seq;
  const int32_t* ent_idx;
  int n, m, fmt;
  const float* norm_w;        // [128]
  float eps;
  const float* rope_cos;
  const float* rope_sin;
  int d_rope, rope_rows;
  Paged keys;
};
hipError_t launch_indexer_k(const IxKArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- indexer + top-k
struct IndexArgs {
  const uint8_t* q;           // bf16 [N, H_I, d_I] or packed e2m1 [N, H_I, d_I/2]
  const uint8_t* q_scale;     // [N, H_I, d_I/32] (mxfp4)
  const float* w;             // [N, H_I]
  Paged keys;
  const int32_t* q_seq;
  const int32_t* q_pos;
  int N, H_I, d_I, m, nv_cap, pos_cap;
  float* scores;              // [N, score_stride]
  int64_t score_stride;
  // large selections: per scoring block, the kb-th largest score key of a full block
  // (kb = ceil(topk / full blocks of the query)); nullptr when not needed
  uint32_t* blk_thr;          // [N, thr_stride]
  unsigned* cand_count;       // [N] candidate counters of the listed-block gather, zeroed by the
                              // scoring launch (nullptr: none)
  int thr_stride, topk;
  // a chunk of consecutive queries of one sequence (q_seq == nullptr): query t is at position
  // p0 + t of sequence seq_const
  int seq_const, p0;
  // > 0: a query's count is of blocks of nv_div entries (ceil), for selections over block scores
  int nv_div;
};

// the most visible entries per query of an indexer selection (the filter's 512 chunks of 8192)
constexpr int64_t kMaxTopkVisible = 4194304;
struct TopkPlan {
  int large;                  // n_visible may exceed kSingleMax: threshold + filter + select
  int thr_stride;             // block thresholds per query (scoring blocks of >= 256 entries)
  int cnt_stride;             // filter chunks (of 8192 entries) per query: candidate counts
  size_t score_bytes, thr_off, cand_off, cnt_off, ws_bytes;
};
TopkPlan topk_plan(int N, int max_pos, int m, int topk);
hipError_t launch_index_scores(const IndexArgs& a, int fmt, hipStream_t stream);
// the per-query scoring blocks (bf16 keys with at most 32768 visible entries, or MXFP4 keys) and
// the compressor's blocks in one launch (neither reads what the other writes)
hipError_t launch_index_scores_compress(const IndexArgs& a, const CompressArgs& c, int max_new, int fmt,
                                        hipStream_t stream);
hipError_t launch_topk(const IndexArgs& a, const TopkPlan& plan, int topk, int32_t* out_idx,
                       float* out_score, uint8_t* ws, int blk_entries, hipStream_t stream);

// Two-level candidate filtering. Workspace past the plain plan's: candidate keys and ids
// [N, cstride] and counters [N] (consumer), or block scores [N, bstride] (source).
struct CandPlan {
  int64_t cstride, bstride;
  size_t ckey_off, cid_off, cnt_off, bmax_off, ws_bytes;
};
CandPlan cand_plan(const TopkPlan& base, int N, int nv_cap, int cand_block, int n_cand);
// consumer: after the scores (launched with a.cand_count = the plan's counters, a.blk_thr null),
// gather the entries of the listed blocks and select the top-k among them
hipError_t launch_topk_in_blocks(const IndexArgs& a, const CandPlan& cp, uint8_t* ws, const int32_t* cand_in,
                                 int n_cand, int cand_block, int topk, int32_t* out_idx, float* out_score,
                                 hipStream_t stream);
// source: after its own top-k, the n_cand blocks with the largest block max
hipError_t launch_candidate_blocks(const IndexArgs& a, const CandPlan& cp, uint8_t* ws, int cand_block,
                                   int n_cand, int32_t* cand_out, hipStream_t stream);

}  // namespace hcs
