// C ABI entry points: host-side validation, workspace planning and kernel launches.
// Every check runs before any HIP call, so invalid arguments never touch the device.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

hcs_status fail(hcs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

hcs_status ok() {
  g_err[0] = 0;
  return HCS_OK;
}

hcs_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(HCS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

hcs_status check_paged(const hcs_paged& p, const char* name, int want_dim, bool allow_fp8,
                       bool allow_mx) {
  if (!p.base || !p.page_table) return fail(HCS_ERR_INVALID_ARG, "%s: null base or page_table", name);
  if (p.pt_stride <= 0 || p.num_pages <= 0)
    return fail(HCS_ERR_INVALID_ARG, "%s: pt_stride and num_pages must be positive", name);
  if (p.fmt < HCS_FMT_BF16 || p.fmt > HCS_FMT_NVFP4)
    return fail(HCS_ERR_INVALID_ARG, "%s: unknown format %d", name, p.fmt);
  if (p.dim != want_dim) return fail(HCS_ERR_INVALID_ARG, "%s: dim %d, expected %d", name, p.dim, want_dim);
  if ((p.fmt == HCS_FMT_FP8DS || p.fmt == HCS_FMT_MXFP8 || p.fmt == HCS_FMT_NVFP4) && (!allow_fp8 || p.dim != 512))
    return fail(HCS_ERR_UNSUPPORTED, "%s: fp8_ds / MXFP8 / NVFP4 rows need dim 512 and a KV cache", name);
  if ((p.fmt == HCS_FMT_MXFP4 || p.fmt == HCS_FMT_FP8IX) && !allow_mx)
    return fail(HCS_ERR_UNSUPPORTED, "%s: MXFP4 and FP8IX are indexer-key formats", name);
  if (p.fmt == HCS_FMT_FP8IX && p.dim != 128)
    return fail(HCS_ERR_UNSUPPORTED, "%s: FP8IX rows have 128 dims", name);
  if (!aligned(p.base, 16)) return fail(HCS_ERR_INVALID_ARG, "%s: base must be 16-byte aligned", name);
  return HCS_OK;
}

}  // namespace

extern "C" {

const char* hcs_last_error(void) { return g_err; }
int hcs_abi_version(void) { return HCS_ABI_VERSION; }

hcs_status hcs_device_errors(uint32_t* bits, int clear) {
  if (!bits) return fail(HCS_ERR_INVALID_ARG, "null bits");
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_status(e, "device_errors (synchronize)");
  uint32_t v = 0;
  hipError_t (*const readers[])(uint32_t*, bool) = {hcs::dev_errors_attention, hcs::dev_errors_compress,
                                                    hcs::dev_errors_indexer, hcs::dev_errors_indexer_prep,
                                                    hcs::dev_errors_insert};
  for (auto r : readers) {
    e = r(&v, clear != 0);
    if (e != hipSuccess) return hip_status(e, "device_errors (read)");
  }
  *bits |= v;
  return ok();
}

// ------------------------------------------------------------------------------ compressor
// Checks of hcs_compress_kv; fills `a` (nothing is launched). B == 0 returns HCS_OK with a.B 0.
static hcs_status prep_compress(const void* kv, const void* score, int in_dtype, int64_t row_stride,
                                const int32_t* cu_new, const int32_t* start_pos, int B, int max_new,
                                int d, int m, const float* ape, float* state, hcs_paged comp,
                                float* dbg, int64_t dbg_seq_stride, hcs::CompressArgs& a) {
  a = hcs::CompressArgs{};
  if (B < 0) return fail(HCS_ERR_INVALID_ARG, "B must be >= 0");
  if (d < 1 || d > 1024 || d % 8) return fail(HCS_ERR_UNSUPPORTED, "d must be in 1..1024 and a multiple of 8");
  if (m < 1 || m > 1024) return fail(HCS_ERR_UNSUPPORTED, "m must be in 1..1024");
  if (in_dtype != HCS_IN_BF16 && in_dtype != HCS_IN_F32) return fail(HCS_ERR_INVALID_ARG, "unknown in_dtype %d", in_dtype);
  if (B == 0) return HCS_OK;
  if (!kv || !score || !cu_new || !start_pos || !state)
    return fail(HCS_ERR_INVALID_ARG, "null kv, score, cu_new, start_pos or state");
  if (row_stride < d) return fail(HCS_ERR_INVALID_ARG, "row_stride %lld < d %d", (long long)row_stride, d);
  if (max_new < 1) return fail(HCS_ERR_INVALID_ARG, "max_new must be >= 1");
  hcs_status s = check_paged(comp, "comp", d, true, false);
  if (s != HCS_OK) return s;
  if (dbg && dbg_seq_stride < 0) return fail(HCS_ERR_INVALID_ARG, "negative dbg_seq_stride");
  a.kv = kv;
  a.score = score;
  a.in_bf16 = in_dtype == HCS_IN_BF16;
  a.row_stride = row_stride;
  a.cu_new = cu_new;
  a.start_pos = start_pos;
  a.B = B;
  a.d = d;
  a.m = m;
  a.fmt = comp.fmt;
  a.ape = ape;
  a.state = state;
  a.comp_base = static_cast<uint8_t*>(comp.base);
  a.comp_pt = comp.page_table;
  a.comp_pt_stride = comp.pt_stride;
  a.comp_num_pages = comp.num_pages;
  a.dbg = dbg;
  a.dbg_stride = dbg_seq_stride;
  return HCS_OK;
}

hcs_status hcs_compress_kv(const void* kv, const void* score, int in_dtype, int64_t row_stride,
                           const int32_t* cu_new, const int32_t* start_pos, int B, int max_new,
                           int d, int m, const float* ape, float* state, hcs_paged comp,
                           float* dbg, int64_t dbg_seq_stride, void* stream) {
  hcs::CompressArgs a;
  const hcs_status s = prep_compress(kv, score, in_dtype, row_stride, cu_new, start_pos, B, max_new, d, m,
                                     ape, state, comp, dbg, dbg_seq_stride, a);
  if (s != HCS_OK || B == 0) return s == HCS_OK ? ok() : s;
  return hip_status(hcs::launch_compress(a, max_new, static_cast<hipStream_t>(stream)), "compress_kv");
}

hcs_status hcs_compress_kv_full(const void* kv, const void* score, int in_dtype, int64_t row_stride,
                                const int32_t* cu_new, const int32_t* start_pos, int B, int max_new,
                                int d, int m, int coff, const float* ape, float* state,
                                const float* norm_weight, float norm_eps, const float* rope_cos,
                                const float* rope_sin, int d_rope, int rope_rows, hcs_paged comp,
                                float* dbg, int64_t dbg_seq_stride, void* stream) {
  if (coff != 1 && coff != 2) return fail(HCS_ERR_UNSUPPORTED, "coff must be 1 or 2");
  hcs::CompressArgs a;
  hcs_status s = prep_compress(kv, score, in_dtype, row_stride, cu_new, start_pos, B, max_new, d, m,
                               ape, state, comp, dbg, dbg_seq_stride, a);
  if (s != HCS_OK) return s;
  if (B > 0 && row_stride < (int64_t)coff * d)
    return fail(HCS_ERR_INVALID_ARG, "row_stride %lld < coff * d = %d", (long long)row_stride, coff * d);
  if (norm_weight && !(norm_eps >= 0.f)) return fail(HCS_ERR_INVALID_ARG, "norm_eps must be >= 0");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(HCS_ERR_INVALID_ARG, "rope_cos and rope_sin are given together or not at all");
  if (rope_cos && (d_rope < 2 || d_rope > d || d_rope % 2 || rope_rows < 1))
    return fail(HCS_ERR_INVALID_ARG, "RoPE needs an even d_rope in 2..d and rope_rows >= 1");
  if (B == 0) return ok();
  a.coff = coff;
  a.norm_w = norm_weight;
  a.norm_eps = norm_eps;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.d_rope = rope_cos ? d_rope : 0;
  a.rope_rows = rope_rows;
  return hip_status(hcs::launch_compress_full(a, max_new, static_cast<hipStream_t>(stream)),
                    "compress_kv_full");
}

// ------------------------------------------------------------------------------ query prep + SWA insert
hcs_status hcs_qnorm_rope_kv_insert(void* q, int H, const void* kv, int64_t kv_stride,
                                    const int32_t* tok_seq, const int32_t* tok_pos, int N, int d,
                                    int q_norm, float eps, const float* rope_cos,
                                    const float* rope_sin, int d_rope, int rope_rows, hcs_paged swa,
                                    void* stream) {
  if (N < 0) return fail(HCS_ERR_INVALID_ARG, "N must be >= 0");
  if (H < 0 || H > 128) return fail(HCS_ERR_UNSUPPORTED, "H must be in 0..128");
  if (d != 128 && d != 512) return fail(HCS_ERR_UNSUPPORTED, "d must be 128 or 512");
  if (q_norm && !(eps >= 0.f)) return fail(HCS_ERR_INVALID_ARG, "eps must be >= 0");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(HCS_ERR_INVALID_ARG, "rope_cos and rope_sin are given together or not at all");
  if (rope_cos && (d_rope < 2 || d_rope > d || d_rope % 2 || rope_rows < 1))
    return fail(HCS_ERR_INVALID_ARG, "RoPE needs an even d_rope in 2..d and rope_rows >= 1");
  if (N == 0 || (H == 0 && !kv)) return ok();
  if (!tok_pos) return fail(HCS_ERR_INVALID_ARG, "null tok_pos");
  if (H > 0 && (!q || !aligned(q, 16))) return fail(HCS_ERR_INVALID_ARG, "q must be non-null and 16-byte aligned");
  hcs::InsertArgs a{};
  if (kv) {
    if (!tok_seq) return fail(HCS_ERR_INVALID_ARG, "null tok_seq");
    if (!aligned(kv, 16) || kv_stride < d || kv_stride % 8)
      return fail(HCS_ERR_INVALID_ARG, "kv must be 16-byte aligned with kv_stride >= d and a multiple of 8");
    hcs_status s = check_paged(swa, "swa", d, true, false);
    if (s != HCS_OK) return s;
    if (swa.fmt == HCS_FMT_NVFP4)
      return fail(HCS_ERR_UNSUPPORTED, "swa: window rows are stored as bf16, fp8_ds or MXFP8");
    a.swa_base = static_cast<uint8_t*>(swa.base);
    a.swa_pt = swa.page_table;
    a.swa_pt_stride = swa.pt_stride;
    a.swa_num_pages = swa.num_pages;
    a.fmt = swa.fmt;
  }
  a.q = static_cast<uint16_t*>(q);
  a.kv = static_cast<const uint16_t*>(kv);
  a.kv_stride = kv_stride;
  a.tok_seq = tok_seq;
  a.tok_pos = tok_pos;
  a.N = N;
  a.H = H;
  a.d = d;
  a.q_norm = q_norm ? 1 : 0;
  a.eps = eps;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.d_rope = rope_cos ? d_rope : 0;
  a.rope_rows = rope_rows;
  return hip_status(hcs::launch_qrope_insert(a, static_cast<hipStream_t>(stream)), "qnorm_rope_kv_insert");
}

// ------------------------------------------------------------------------------ indexer Q / K production
static hcs_status check_rope(const float* rope_cos, const float* rope_sin, int d_rope, int rope_rows, int d) {
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(HCS_ERR_INVALID_ARG, "rope_cos and rope_sin are given together or not at all");
  if (rope_cos && (d_rope < 2 || d_rope > d || d_rope % 2 || rope_rows < 1))
    return fail(HCS_ERR_INVALID_ARG, "RoPE needs an even d_rope in 2..d and rope_rows >= 1");
  return HCS_OK;
}

hcs_status hcs_indexer_q_prep(const void* q, const float* w, const int32_t* tok_pos, int N, int H_I,
                              int d_I, float w_scale, const float* rope_cos, const float* rope_sin,
                              int d_rope, int rope_rows, int out_fmt, void* q_out,
                              void* q_scale_out, float* w_out, void* stream) {
  if (N < 0) return fail(HCS_ERR_INVALID_ARG, "N must be >= 0");
  if (H_I < 1 || H_I > 64) return fail(HCS_ERR_UNSUPPORTED, "H_I must be in 1..64");
  if (d_I != 128) return fail(HCS_ERR_UNSUPPORTED, "d_I must be 128");
  if (out_fmt != HCS_FMT_BF16 && out_fmt != HCS_FMT_MXFP4 && out_fmt != HCS_FMT_FP8IX)
    return fail(HCS_ERR_INVALID_ARG, "out_fmt must be HCS_FMT_BF16, HCS_FMT_MXFP4 or HCS_FMT_FP8IX");
  hcs_status s = check_rope(rope_cos, rope_sin, d_rope, rope_rows, d_I);
  if (s != HCS_OK) return s;
  if (N == 0) return ok();
  if (!q || !w || !tok_pos || !q_out || !w_out) return fail(HCS_ERR_INVALID_ARG, "null q, w, tok_pos, q_out or w_out");
  if (out_fmt != HCS_FMT_BF16 && !q_scale_out) return fail(HCS_ERR_INVALID_ARG, "null q_scale_out");
  if (!aligned(q, 16) || !aligned(q_out, 16)) return fail(HCS_ERR_INVALID_ARG, "q and q_out must be 16-byte aligned");
  if (out_fmt == HCS_FMT_FP8IX && !aligned(q_scale_out, 4))
    return fail(HCS_ERR_INVALID_ARG, "q_scale_out must be 4-byte aligned");
  hcs::IxQArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.w = w;
  a.tok_pos = tok_pos;
  a.N = N;
  a.H = H_I;
  a.fmt = out_fmt;
  a.w_scale = w_scale;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.d_rope = rope_cos ? d_rope : 0;
  a.rope_rows = rope_rows;
  a.q_out16 = static_cast<uint16_t*>(q_out);
  a.q_out8 = static_cast<uint8_t*>(q_out);
  a.q_scale8 = static_cast<uint8_t*>(q_scale_out);
  a.q_scalef = static_cast<float*>(q_scale_out);
  a.w_out = w_out;
  return hip_status(hcs::launch_indexer_q(a, static_cast<hipStream_t>(stream)), "indexer_q_prep");
}

hcs_status hcs_indexer_k_store(const void* k_pre, int64_t k_stride, const int32_t* ent_seq,
                               const int32_t* ent_idx, int n, int d_I, int m,
                               const float* norm_weight, float eps, const float* rope_cos,
                               const float* rope_sin, int d_rope, int rope_rows, hcs_paged keys,
                               void* stream) {
  if (n < 0) return fail(HCS_ERR_INVALID_ARG, "n must be >= 0");
  if (d_I != 128) return fail(HCS_ERR_UNSUPPORTED, "d_I must be 128");
  if (m < 1) return fail(HCS_ERR_INVALID_ARG, "m must be >= 1");
  if (!(eps >= 0.f)) return fail(HCS_ERR_INVALID_ARG, "eps must be >= 0");
  hcs_status s = check_rope(rope_cos, rope_sin, d_rope, rope_rows, d_I);
  if (s != HCS_OK) return s;
  if (n == 0) return ok();
  if (!k_pre || !ent_seq || !ent_idx || !norm_weight)
    return fail(HCS_ERR_INVALID_ARG, "null k_pre, ent_seq, ent_idx or norm_weight");
  if (!aligned(k_pre, 16) || k_stride < d_I || k_stride % 8)
    return fail(HCS_ERR_INVALID_ARG, "k_pre must be 16-byte aligned with k_stride >= d_I and a multiple of 8");
  s = check_paged(keys, "keys", d_I, false, true);
  if (s != HCS_OK) return s;
  hcs::IxKArgs a{};
  a.k = static_cast<const uint16_t*>(k_pre);
  a.k_stride = k_stride;
  a.ent_seq = ent_seq;
  a.ent_idx = ent_idx;
  a.n = n;
  a.m = m;
  a.fmt = keys.fmt;
  a.norm_w = norm_weight;
  a.eps = eps;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.d_rope = rope_cos ? d_rope : 0;
  a.rope_rows = rope_rows;
  a.keys = hcs::to_paged(keys);
  return hip_status(hcs::launch_indexer_k(a, static_cast<hipStream_t>(stream)), "indexer_k_store");
}

// ------------------------------------------------------------------------------ indexer
size_t hcs_index_topk_workspace_size(int N, int max_pos, int m, int topk) {
  if (N <= 0 || max_pos < 0 || m < 1 || topk < 1) return 0;
  return hcs::topk_plan(N, max_pos, m, topk).ws_bytes;
}

// Checks shared by the indexer entry points that do not depend on the selection; fills `a`
// except its scores and selection fields. q_seq == NULL means a chunk of queries of sequence
// `seq` at positions P0 .. P0+N-1.
static hcs_status prep_index_args(const void* q, const uint8_t* q_scale, const float* w, hcs_paged keys,
                                  const int32_t* q_seq, const int32_t* q_pos, int seq, int P0, int N,
                                  int H_I, int d_I, int m, int max_pos, hcs::IndexArgs& a) {
  a = hcs::IndexArgs{};
  if (N < 0) return fail(HCS_ERR_INVALID_ARG, "N must be >= 0");
  if (H_I < 1 || H_I > 64) return fail(HCS_ERR_UNSUPPORTED, "H_I must be in 1..64");
  if (m < 1) return fail(HCS_ERR_INVALID_ARG, "m must be >= 1");
  if (max_pos < 0) return fail(HCS_ERR_INVALID_ARG, "max_pos must be >= 0");
  if (N == 0) return HCS_OK;
  if (!q || !w) return fail(HCS_ERR_INVALID_ARG, "null q or w");
  hcs_status s = check_paged(keys, "keys", d_I, false, true);
  if (s != HCS_OK) return s;
  if (keys.fmt == HCS_FMT_BF16 && d_I != 32 && d_I != 64 && d_I != 128)
    return fail(HCS_ERR_UNSUPPORTED, "bf16 indexer keys need d_I in {32, 64, 128}");
  if (keys.fmt == HCS_FMT_FP8IX && (d_I != 128 || !q_scale || !aligned(q_scale, 4)))
    return fail(HCS_ERR_UNSUPPORTED, "FP8IX indexer keys need d_I == 128 and a 4-byte aligned float32 q_scale");
  if (keys.fmt == HCS_FMT_MXFP4 && (d_I != 128 || !q_scale))
    return fail(HCS_ERR_UNSUPPORTED, "MXFP4 indexer keys need d_I == 128 and q_scale");
  if (!aligned(q, 16)) return fail(HCS_ERR_INVALID_ARG, "q must be 16-byte aligned");
  if ((int64_t)keys.pt_stride * HCS_PAGE_ROWS < (int64_t)(max_pos + 1) / m)
    return fail(HCS_ERR_INVALID_ARG, "keys: pt_stride %d does not cover %d entries", keys.pt_stride,
                (max_pos + 1) / m);
  a.q = static_cast<const uint8_t*>(q);
  a.q_scale = q_scale;
  a.w = w;
  a.keys = hcs::to_paged(keys);
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.seq_const = seq;
  a.p0 = P0;
  a.N = N;
  a.H_I = H_I;
  a.d_I = d_I;
  a.m = m;
  a.pos_cap = max_pos;
  a.nv_cap = (max_pos + 1) / m;
  return HCS_OK;
}

// Checks shared by the indexer entry points with a selection; fills `a` and `plan` (nothing is
// launched; N == 0 returns HCS_OK with a.N 0).
static hcs_status prep_index(const void* q, const uint8_t* q_scale, const float* w, hcs_paged keys,
                             const int32_t* q_seq, const int32_t* q_pos, int seq, int P0, int N,
                             int H_I, int d_I, int m, int topk, int max_pos, int32_t* out_idx,
                             void* ws, size_t ws_bytes, hcs::IndexArgs& a, hcs::TopkPlan& plan) {
  if (topk < 1 || topk > 4096) return fail(HCS_ERR_UNSUPPORTED, "topk must be in 1..4096");
  hcs_status s = prep_index_args(q, q_scale, w, keys, q_seq, q_pos, seq, P0, N, H_I, d_I, m, max_pos, a);
  if (s != HCS_OK || N == 0) return s;
  if (!out_idx) return fail(HCS_ERR_INVALID_ARG, "null out_idx");
  if ((int64_t)(max_pos + 1) / m > hcs::kMaxTopkVisible)
    return fail(HCS_ERR_UNSUPPORTED, "(max_pos + 1) / m = %lld visible entries exceed %lld",
                (long long)((int64_t)(max_pos + 1) / m), (long long)hcs::kMaxTopkVisible);
  plan = hcs::topk_plan(N, max_pos, m, topk);
  if (!ws || ws_bytes < plan.ws_bytes)
    return fail(HCS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", plan.ws_bytes, ws_bytes);
  if (!aligned(ws, 256)) return fail(HCS_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  a.scores = static_cast<float*>(ws);
  a.score_stride = (int64_t)(plan.score_bytes / sizeof(float) / N);
  a.topk = topk;
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  if (plan.large) {
    a.blk_thr = reinterpret_cast<uint32_t*>(w8 + plan.thr_off);
    a.thr_stride = plan.thr_stride;
  }
  return HCS_OK;
}

// The selection launch after the scores (entries per threshold block: 512 FP8; 256 bf16 and
// MXFP4, whose scoring waves each bound their own 256 entries).
static hcs_status run_topk(const hcs::IndexArgs& a, const hcs::TopkPlan& plan, int fmt, int topk,
                           int32_t* out_idx, float* out_score, void* ws, void* stream) {
  const int blk_entries = fmt == HCS_FMT_FP8IX ? 512 : 256;     // MXFP4: a threshold per wave
  return hip_status(hcs::launch_topk(a, plan, topk, out_idx, out_score, static_cast<uint8_t*>(ws),
                                     blk_entries, static_cast<hipStream_t>(stream)),
                    "index_topk select");
}

static hcs_status run_index(const void* q, const uint8_t* q_scale, const float* w, hcs_paged keys,
                            const int32_t* q_seq, const int32_t* q_pos, int seq, int P0, int N,
                            int H_I, int d_I, int m, int topk, int max_pos, int32_t* out_idx,
                            float* out_score, void* ws, size_t ws_bytes, void* stream) {
  hcs::IndexArgs a;
  hcs::TopkPlan plan;
  const hcs_status s = prep_index(q, q_scale, w, keys, q_seq, q_pos, seq, P0, N, H_I, d_I, m, topk,
                                  max_pos, out_idx, ws, ws_bytes, a, plan);
  if (s != HCS_OK || N == 0) return s == HCS_OK ? ok() : s;
  const hipError_t e = hcs::launch_index_scores(a, keys.fmt, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_status(e, "index_topk scores");
  return run_topk(a, plan, keys.fmt, topk, out_idx, out_score, ws, stream);
}

hcs_status hcs_index_topk(const void* q, const uint8_t* q_scale, const float* w, hcs_paged keys,
                          const int32_t* q_seq, const int32_t* q_pos, int N, int H_I, int d_I,
                          int m, int topk, int max_pos, int32_t* out_idx, float* out_score,
                          void* ws, size_t ws_bytes, void* stream) {
  if (N > 0 && (!q_seq || !q_pos)) return fail(HCS_ERR_INVALID_ARG, "null q_seq or q_pos");
  return run_index(q, q_scale, w, keys, q_seq, q_pos, 0, 0, N, H_I, d_I, m, topk, max_pos,
                   out_idx, out_score, ws, ws_bytes, stream);
}

size_t hcs_index_topk_cand_workspace_size(int N, int max_pos, int m, int topk, int cand_block, int n_cand) {
  if (N <= 0 || max_pos < 0 || m < 1 || topk < 1 || cand_block < 1 || n_cand < 1) return 0;
  const hcs::TopkPlan plan = hcs::topk_plan(N, max_pos, m, topk);
  return hcs::cand_plan(plan, N, (max_pos + 1) / m, cand_block, n_cand).ws_bytes;
}

hcs_status hcs_index_topk_cand(const void* q, const uint8_t* q_scale, const float* w, hcs_paged keys,
                               const int32_t* q_seq, const int32_t* q_pos, int N, int H_I, int d_I, int m,
                               int topk, int max_pos, int cand_block, int n_cand, const int32_t* cand_in,
                               int32_t* cand_out, int32_t* out_idx, float* out_score, void* ws,
                               size_t ws_bytes, void* stream) {
  if ((cand_in == nullptr) == (cand_out == nullptr))
    return fail(HCS_ERR_INVALID_ARG, "exactly one of cand_in (consumer) and cand_out (source) is given");
  if (cand_block < 1) return fail(HCS_ERR_INVALID_ARG, "cand_block must be >= 1");
  if (n_cand < 1 || n_cand > 4096) return fail(HCS_ERR_UNSUPPORTED, "n_cand must be in 1..4096");
  if (m >= 1 && max_pos >= 0 && cand_out && ((int64_t)(max_pos + 1) / m + cand_block - 1) / cand_block > 32768)
    return fail(HCS_ERR_UNSUPPORTED, "a query may see more than 32768 blocks of cand_block entries");
  if ((int64_t)n_cand * cand_block > INT32_MAX) return fail(HCS_ERR_INVALID_ARG, "n_cand * cand_block overflows");
  if (N > 0 && (!q_seq || !q_pos)) return fail(HCS_ERR_INVALID_ARG, "null q_seq or q_pos");
  hcs::IndexArgs a;
  hcs::TopkPlan plan;
  hcs_status s = prep_index(q, q_scale, w, keys, q_seq, q_pos, 0, 0, N, H_I, d_I, m, topk, max_pos, out_idx,
                            ws, ws_bytes, a, plan);
  if (s != HCS_OK || N == 0) return s == HCS_OK ? ok() : s;
  const hcs::CandPlan cp = hcs::cand_plan(plan, N, a.nv_cap, cand_block, n_cand);
  if (ws_bytes < cp.ws_bytes)
    return fail(HCS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", cp.ws_bytes, ws_bytes);
  uint8_t* w8 = static_cast<uint8_t*>(ws);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (cand_in) {                                     // consumer: no block thresholds, own counters
    a.blk_thr = nullptr;
    a.cand_count = reinterpret_cast<unsigned*>(w8 + cp.cnt_off);
    hipError_t e = hcs::launch_index_scores(a, keys.fmt, st);
    if (e == hipSuccess)
      e = hcs::launch_topk_in_blocks(a, cp, w8, cand_in, n_cand, cand_block, topk, out_idx, out_score, st);
    return hip_status(e, "index_topk_cand (consumer)");
  }
  hipError_t e = hcs::launch_index_scores(a, keys.fmt, st);
  if (e != hipSuccess) return hip_status(e, "index_topk_cand scores");
  s = run_topk(a, plan, keys.fmt, topk, out_idx, out_score, ws, stream);
  if (s != HCS_OK) return s;
  return hip_status(hcs::launch_candidate_blocks(a, cp, w8, cand_block, n_cand, cand_out, st),
                    "index_topk_cand (source)");
}

hcs_status hcs_index_topk_chunk(const void* q, const uint8_t* q_scale, const float* w,
                                hcs_paged keys, int seq, int P0, int Q, int H_I, int d_I, int m,
                                int topk, int32_t* out_idx, float* out_score, void* ws,
                                size_t ws_bytes, void* stream) {
  if (P0 < 0 || seq < 0) return fail(HCS_ERR_INVALID_ARG, "P0 and seq must be >= 0");
  if (Q < 0) return fail(HCS_ERR_INVALID_ARG, "Q must be >= 0");
  if ((int64_t)P0 + Q > INT32_MAX) return fail(HCS_ERR_INVALID_ARG, "P0 + Q overflows int32");
  if (Q == 0) return ok();
  return run_index(q, q_scale, w, keys, nullptr, nullptr, seq, P0, Q, H_I, d_I, m, topk,
                   P0 + Q - 1, out_idx, out_score, ws, ws_bytes, stream);
}

hcs_status hcs_index_topk_compress(const void* q, const uint8_t* q_scale, const float* w,
                                   hcs_paged keys, const int32_t* q_seq, const int32_t* q_pos, int N,
                                   int H_I, int d_I, int m_ix, int topk, int max_pos,
                                   int32_t* out_idx, float* out_score, void* ws, size_t ws_bytes,
                                   const void* kv, const void* score, int in_dtype,
                                   int64_t row_stride, const int32_t* cu_new,
                                   const int32_t* start_pos, int B, int max_new, int d, int m,
                                   const float* ape, float* state, hcs_paged comp, void* stream) {
  if (N > 0 && (!q_seq || !q_pos)) return fail(HCS_ERR_INVALID_ARG, "null q_seq or q_pos");
  hcs::IndexArgs a;
  hcs::TopkPlan plan;
  hcs_status s = prep_index(q, q_scale, w, keys, q_seq, q_pos, 0, 0, N, H_I, d_I, m_ix, topk, max_pos,
                            out_idx, ws, ws_bytes, a, plan);
  if (s != HCS_OK) return s;
  hcs::CompressArgs c;
  s = prep_compress(kv, score, in_dtype, row_stride, cu_new, start_pos, B, max_new, d, m, ape, state,
                    comp, nullptr, 0, c);
  if (s != HCS_OK) return s;
  if (comp.base == keys.base) return fail(HCS_ERR_INVALID_ARG, "comp and keys must be different caches");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (N == 0) {
    if (B == 0) return ok();
    return hip_status(hcs::launch_compress(c, max_new, st), "compress_kv");
  }
  hipError_t e;
  if ((keys.fmt == HCS_FMT_BF16 && !plan.large) || keys.fmt == HCS_FMT_MXFP4)
    e = hcs::launch_index_scores_compress(a, c, max_new, keys.fmt, st);
  else {
    e = B > 0 ? hcs::launch_compress(c, max_new, st) : hipSuccess;
    if (e == hipSuccess) e = hcs::launch_index_scores(a, keys.fmt, st);
  }
  if (e != hipSuccess) return hip_status(e, "index_topk_compress scores");
  return run_topk(a, plan, keys.fmt, topk, out_idx, out_score, ws, stream);
}

hcs_status hcs_index_scores_compress(const void* q, const uint8_t* q_scale, const float* w,
                                     hcs_paged keys, const int32_t* q_seq, const int32_t* q_pos, int N,
                                     int H_I, int d_I, int m_ix, int max_pos, float* scores,
                                     int64_t score_stride, const void* kv, const void* score,
                                     int in_dtype, int64_t row_stride, const int32_t* cu_new,
                                     const int32_t* start_pos, int B, int max_new, int d, int m,
                                     const float* ape, float* state, hcs_paged comp, void* stream) {
  if (N > 0 && (!q_seq || !q_pos)) return fail(HCS_ERR_INVALID_ARG, "null q_seq or q_pos");
  hcs::IndexArgs a;
  hcs_status s = prep_index_args(q, q_scale, w, keys, q_seq, q_pos, 0, 0, N, H_I, d_I, m_ix, max_pos, a);
  if (s != HCS_OK) return s;
  if (N > 0) {
    if (!scores || !aligned(scores, 4)) return fail(HCS_ERR_INVALID_ARG, "scores must be a non-null float32 buffer");
    if (score_stride < a.nv_cap)
      return fail(HCS_ERR_INVALID_ARG, "score_stride %lld < %d visible entries", (long long)score_stride, a.nv_cap);
    a.scores = scores;
    a.score_stride = score_stride;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hcs::CompressArgs c;
  if (B > 0) {
    s = prep_compress(kv, score, in_dtype, row_stride, cu_new, start_pos, B, max_new, d, m, ape, state,
                      comp, nullptr, 0, c);
    if (s != HCS_OK) return s;
    if (N > 0 && comp.base == keys.base) return fail(HCS_ERR_INVALID_ARG, "comp and keys must be different caches");
  } else if (B < 0) {
    return fail(HCS_ERR_INVALID_ARG, "B must be >= 0");
  }
  if (N == 0) return B > 0 ? hip_status(hcs::launch_compress(c, max_new, st), "compress_kv") : ok();
  hipError_t e;
  if (B > 0 && ((keys.fmt == HCS_FMT_BF16 && a.nv_cap <= 32768) || keys.fmt == HCS_FMT_MXFP4))
    e = hcs::launch_index_scores_compress(a, c, max_new, keys.fmt, st);
  else {
    e = B > 0 ? hcs::launch_compress(c, max_new, st) : hipSuccess;
    if (e == hipSuccess) e = hcs::launch_index_scores(a, keys.fmt, st);
  }
  return hip_status(e, "index_scores_compress");
}

// ------------------------------------------------------------------------------ attention
static hcs_status check_attn(const void* q, const hcs_paged& swa, const hcs_paged& comp,
                             const int32_t* topk_idx, int topk, int N, int H, int d, int window,
                             int m, const void* out) {
  if (N < 0) return fail(HCS_ERR_INVALID_ARG, "N must be >= 0");
  if (d != 128 && d != 512) return fail(HCS_ERR_UNSUPPORTED, "d must be 128 or 512");
  if (H < 1 || H > 128) return fail(HCS_ERR_UNSUPPORTED, "H must be in 1..128");
  if (window < 0) return fail(HCS_ERR_INVALID_ARG, "window must be >= 0");
  if (m < 1) return fail(HCS_ERR_INVALID_ARG, "m must be >= 1");
  if (topk_idx && topk < 1) return fail(HCS_ERR_INVALID_ARG, "topk must be >= 1 with topk_idx");
  if (N == 0) return HCS_OK;
  if (!q || !out) return fail(HCS_ERR_INVALID_ARG, "null q or out");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(HCS_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  hcs_status s = check_paged(swa, "swa", d, true, false);
  if (s != HCS_OK) return s;
  s = check_paged(comp, "comp", d, true, false);
  if (s != HCS_OK) return s;
  if (!hcs::attn_formats_supported(d, swa.fmt, comp.fmt))
    return fail(HCS_ERR_UNSUPPORTED, "swa / comp formats %d / %d: supported are bf16 / bf16, fp8_ds / fp8_ds, "
                "MXFP8 / MXFP8 and MXFP8 / NVFP4", swa.fmt, comp.fmt);
  return HCS_OK;
}

size_t hcs_sparse_mla_workspace_size(int N, int H, int d, int window, int m, int topk, int max_pos) {
  if (N <= 0 || H <= 0 || m < 1 || max_pos < 0 || window < 0) return 0;
  // (the same plan for every cache format)
  return hcs::attn_plan(N, H, d, window, m, topk, max_pos).ws_bytes;
}

static hcs_status run_attn(hcs::AttnArgs& a, int d, int fmt, int comp_fmt, int window, int m, int topk,
                           int max_pos, void* ws, size_t ws_bytes, void* stream) {
  if (window > 0 && (int64_t)a.swa.pt_stride * HCS_PAGE_ROWS <= (int64_t)max_pos)
    return fail(HCS_ERR_INVALID_ARG, "swa: pt_stride %d does not cover position %d", a.swa.pt_stride,
                max_pos);
  if ((int64_t)a.comp.pt_stride * HCS_PAGE_ROWS < (int64_t)(max_pos + 1) / m)
    return fail(HCS_ERR_INVALID_ARG, "comp: pt_stride %d does not cover %d entries", a.comp.pt_stride,
                (max_pos + 1) / m);
  const hcs::AttnPlan plan = hcs::attn_plan(a.N, a.H, d, window, m, topk, max_pos);
  if (plan.ws_bytes && (!ws || ws_bytes < plan.ws_bytes))
    return fail(HCS_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", plan.ws_bytes, ws_bytes);
  if (plan.ws_bytes && !aligned(ws, 256)) return fail(HCS_ERR_INVALID_ARG, "ws must be 256-byte aligned");
  a.nsplit = plan.nsplit;
  a.n_hg = plan.n_hg;
  a.n_h16 = plan.n_h16;
  a.rows_per_split = plan.rows_per_split;
  if (plan.nsplit > 1) {
    uint8_t* w = static_cast<uint8_t*>(ws);
    a.ws_o = reinterpret_cast<uint16_t*>(w);
    a.ws_ml = reinterpret_cast<float*>(w + plan.ws_o_bytes);
  }
  return hip_status(hcs::launch_sparse_mla(a, d, fmt, comp_fmt, static_cast<hipStream_t>(stream)), "sparse_mla");
}

hcs_status hcs_sparse_mla_decode(const void* q, hcs_paged swa, hcs_paged comp,
                                 const int32_t* topk_idx, int topk, const int32_t* q_seq,
                                 const int32_t* q_pos, const float* sink, int N, int H, int d,
                                 int window, int m, int max_pos, float scale, void* out,
                                 float* lse, void* ws, size_t ws_bytes, void* stream) {
  hcs_status s = check_attn(q, swa, comp, topk_idx, topk, N, H, d, window, m, out);
  if (s != HCS_OK) return s;
  if (max_pos < 0) return fail(HCS_ERR_INVALID_ARG, "max_pos must be >= 0");
  if (N == 0) return ok();
  if (!q_seq || !q_pos) return fail(HCS_ERR_INVALID_ARG, "null q_seq or q_pos");
  hcs::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.swa = hcs::to_paged(swa);
  a.comp = hcs::to_paged(comp);
  a.topk_idx = topk_idx;
  a.topk = topk_idx ? topk : 0;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.sink = sink;
  a.N = N;
  a.H = H;
  a.window = window;
  a.m = m;
  a.pos_cap = max_pos;
  a.nv_cap = (max_pos + 1) / m;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return run_attn(a, d, swa.fmt, comp.fmt, window, m, a.topk, max_pos, ws, ws_bytes, stream);
}

hcs_status hcs_sparse_mla_decode_select(const void* q, hcs_paged swa, hcs_paged comp,
                                        const float* scores, int64_t score_stride, int topk,
                                        const int32_t* q_seq, const int32_t* q_pos, const float* sink,
                                        int N, int H, int d, int window, int m, int max_pos,
                                        float scale, void* out, float* lse, int32_t* sel_idx,
                                        void* ws, size_t ws_bytes, void* stream) {
  if (topk < 1 || topk > 4096) return fail(HCS_ERR_UNSUPPORTED, "topk must be in 1..4096");
  hcs_status s = check_attn(q, swa, comp, nullptr, topk, N, H, d, window, m, out);
  if (s != HCS_OK) return s;
  if (max_pos < 0) return fail(HCS_ERR_INVALID_ARG, "max_pos must be >= 0");
  if (N == 0) return ok();
  if (d != 512 || swa.fmt != HCS_FMT_BF16 || comp.fmt != HCS_FMT_BF16)
    return fail(HCS_ERR_UNSUPPORTED, "selection inside the attention needs d = 512 and bf16 caches");
  const int nv_cap = (max_pos + 1) / m;
  if (nv_cap > hcs::kSelMax)
    return fail(HCS_ERR_UNSUPPORTED, "selection inside the attention takes at most %d visible entries, got %d",
                hcs::kSelMax, nv_cap);
  if (!q_seq || !q_pos) return fail(HCS_ERR_INVALID_ARG, "null q_seq or q_pos");
  if (!scores || !aligned(scores, 4)) return fail(HCS_ERR_INVALID_ARG, "scores must be a non-null float32 buffer");
  if (score_stride < nv_cap)
    return fail(HCS_ERR_INVALID_ARG, "score_stride %lld < %d visible entries", (long long)score_stride, nv_cap);
  hcs::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.swa = hcs::to_paged(swa);
  a.comp = hcs::to_paged(comp);
  a.topk_idx = nullptr;
  a.topk = topk;
  a.scores = scores;
  a.score_stride = score_stride;
  a.sel_out = sel_idx;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.sink = sink;
  a.N = N;
  a.H = H;
  a.window = window;
  a.m = m;
  a.pos_cap = max_pos;
  a.nv_cap = nv_cap;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return run_attn(a, d, swa.fmt, comp.fmt, window, m, topk, max_pos, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------------------ decode without allocation
// The split partials of hcs_sparse_mla_decode_noalloc live in this file-scope device array (each
// device the library runs on holds its own copy until the process ends). Host code never uses
// the array's name as an address: the address is taken once per device with
// hipGetSymbolAddress and kept in g_scratch_dev.
static __device__ __align__(256) uint8_t scratch[HCS_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

hcs_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "sparse_mla_decode_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= kMaxDevices) return fail(HCS_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                 "sparse_mla_decode_noalloc (hipGetSymbolAddress)");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return HCS_OK;
}
}  // namespace

hcs_status hcs_sparse_mla_decode_noalloc(const void* q, hcs_paged swa, hcs_paged comp,
                                         const int32_t* topk_idx, int topk, const int32_t* q_seq,
                                         const int32_t* q_pos, const float* sink, int N, int H, int d,
                                         int window, int m, int max_pos, float scale, void* out,
                                         float* lse, void* stream) {
  hcs_status s = check_attn(q, swa, comp, topk_idx, topk, N, H, d, window, m, out);
  if (s != HCS_OK) return s;
  if (max_pos < 0) return fail(HCS_ERR_INVALID_ARG, "max_pos must be >= 0");
  if (N == 0) return ok();
  const size_t need = hcs::attn_plan(N, H, d, window, m, topk_idx ? topk : 0, max_pos).ws_bytes;
  if (need > (size_t)HCS_NOALLOC_SCRATCH_BYTES)
    return fail(HCS_ERR_WORKSPACE_TOO_SMALL, "sparse_mla_decode_noalloc: the call needs %zu bytes of scratch, "
                "the library's static scratch holds %zu (use hcs_sparse_mla_decode with a workspace)",
                need, (size_t)HCS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need) {
    s = scratch_of_current_device(&ws);
    if (s != HCS_OK) return s;
  }
  return hcs_sparse_mla_decode(q, swa, comp, topk_idx, topk, q_seq, q_pos, sink, N, H, d, window, m, max_pos,
                               scale, out, lse, ws, need ? (size_t)HCS_NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t hcs_sparse_mla_prefill_workspace_size(int Q, int H, int d, int window, int m, int topk, int P0) {
  if (Q <= 0 || P0 < 0) return 0;
  return hcs_sparse_mla_workspace_size(Q, H, d, window, m, topk, P0 + Q - 1);
}

hcs_status hcs_sparse_mla_prefill_chunk(const void* q, hcs_paged swa, hcs_paged comp,
                                        const int32_t* topk_idx, int topk, int seq, int P0, int Q,
                                        const float* sink, int H, int d, int window, int m,
                                        float scale, void* out, float* lse, void* ws,
                                        size_t ws_bytes, void* stream) {
  hcs_status s = check_attn(q, swa, comp, topk_idx, topk, Q, H, d, window, m, out);
  if (s != HCS_OK) return s;
  if (P0 < 0 || seq < 0) return fail(HCS_ERR_INVALID_ARG, "P0 and seq must be >= 0");
  if ((int64_t)P0 + Q > INT32_MAX) return fail(HCS_ERR_INVALID_ARG, "P0 + Q overflows int32");
  if (Q == 0) return ok();
  hcs::AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.swa = hcs::to_paged(swa);
  a.comp = hcs::to_paged(comp);
  a.topk_idx = topk_idx;
  a.topk = topk_idx ? topk : 0;
  a.q_seq = nullptr;
  a.q_pos = nullptr;
  a.seq_const = seq;
  a.p0 = P0;
  a.sink = sink;
  a.N = Q;
  a.H = H;
  a.window = window;
  a.m = m;
  a.pos_cap = P0 + Q - 1;
  a.nv_cap = (P0 + Q) / m;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  return run_attn(a, d, swa.fmt, comp.fmt, window, m, a.topk, P0 + Q - 1, ws, ws_bytes, stream);
}

}  // extern "C"
