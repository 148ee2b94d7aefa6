// Lightning-Indexer scores and exact top-k selection for gfx950.
//
// What it computes: "DeepSeek V4 Attention: Code Reading Map", section "Aux stream 0 (CSA
// only)": scores between the indexer queries and the compressed indexer keys, then the top-k
// compressed entries; score I[t,i] = sum_h w[t,h] * ReLU(q[t,h] . k[i]). When a query sees no
// more entries than k, all of them are selected ("DeepSeek V4.1 attention" API page,
// short-context rule).
//
// Scores: one workgroup scores 256 (bf16) or 512 (MXFP4) consecutive entries of one query.
// The query's heads are the MFMA M dimension and stay in registers; each lane streams 16-byte
// pieces of key rows straight from the paged cache (no LDS: every key byte is used once).
//   bf16 : v_mfma_f32_16x16x32_bf16, K = d_I in steps of 32;
//   MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands e2m1 and the UE8M0 block
//          scales as the instruction's scale operands; the documented cache layout (32
//          consecutive values per 16 bytes, low nibble first, one scale byte per 32) is exactly
//          the instruction's per-lane operand, so keys go from HBM to the matrix core untouched.
// The C layout puts 4 heads x 1 entry in each lane: ReLU, the head weights and the sum over
// heads are done in registers plus two cross-lane shuffles.
//
// Top-k: exact radix select on order-preserving 32-bit keys of the fp32 scores, 8 bits per
// pass from the top, with LDS histograms in one 1024-thread workgroup per query; ties at the
// threshold are broken towards smaller entry ids by a second radix select on the ids. Queries
// with more than 32768 visible entries go through two stages: every 16384-entry chunk keeps
// its own exact top-k, then the chunk winners are selected again (exact: an entry of the
// global top-k is always in its chunk's top-k).
#include "kernels.h"

namespace hcs {

namespace {

constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kChunk = 16384;           // stage-1 chunk of the two-stage select
constexpr int kSingleMax = 32768;       // largest n_visible selected in one stage
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ void query_of(const IndexArgs& a, int t, int& seq, int& nv) {
  seq = __ldg(a.q_seq + t);
  const int pos = min(__ldg(a.q_pos + t), a.pos_cap);
  nv = min((pos + 1) / a.m, a.nv_cap);
}

// ---------------------------------------------------------------- bf16 scores
template <int DI, int MT>
__global__ __launch_bounds__(kScoreThreads) void index_score_bf16_kernel(IndexArgs a) {
  constexpr int KS = DI / 32;
  constexpr int NT = 4;                  // 4 x 16 entries per wave
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  int seq, nv;
  query_of(a, t, seq, nv);
  const int e_base = blockIdx.y * (kScoreThreads / 64) * NT * 16 + wave * NT * 16;
  if (e_base >= nv) return;

  bf16x8 qreg[MT][KS];
  float wreg[MT][4];
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4 v = h < a.H_I ? *(const i32x4*)(q + ((int64_t)t * a.H_I + h) * DI + 32 * ks + 8 * g)
                          : i32x4{0, 0, 0, 0};
      qreg[mt][ks] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = mt * 16 + 4 * g + i;
      wreg[mt][i] = hw < a.H_I ? a.w[(int64_t)t * a.H_I + hw] : 0.f;
    }
  }

  bf16x8 kreg[NT][KS];
  bool kval[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = e_base + nt * 16 + l16;
    const int pg = e < nv ? page_of(a.keys, seq, e) : -1;
    kval[nt] = pg >= 0;
    const uint8_t* row = a.keys.base + (int64_t)(pg < 0 ? 0 : pg) * (kPageRows * DI * 2) + (e & 63) * (DI * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4 v = pg >= 0 ? *(const i32x4*)(row + (32 * ks + 8 * g) * 2) : i32x4{0, 0, 0, 0};
      kreg[nt][ks] = __builtin_bit_cast(bf16x8, v);
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qreg[mt][ks], kreg[nt][ks], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wreg[mt][i] * fmaxf(acc[i], 0.f);
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    const int e = e_base + nt * 16 + l16;
    if (g == 0 && e < nv) a.scores[(int64_t)t * a.score_stride + e] = kval[nt] ? part : kNegInf;
  }
}

// ---------------------------------------------------------------- MXFP4 scores (d_I = 128)
template <int MT>
__global__ __launch_bounds__(kScoreThreads) void index_score_mxfp4_kernel(IndexArgs a) {
  constexpr int DI = 128;
  constexpr int NT = 8;                  // 8 x 16 entries per wave
  constexpr int PAGE = kPageRows * (DI / 2 + DI / kMxBlock);     // 4352
  constexpr int SCALES = kPageRows * (DI / 2);                   // scale region offset
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  int seq, nv;
  query_of(a, t, seq, nv);
  const int e_base = blockIdx.y * (kScoreThreads / 64) * NT * 16 + wave * NT * 16;
  if (e_base >= nv) return;

  i32x8 qa[MT];
  int qs[MT];
  float wreg[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + l16;
    i32x4 v = {0, 0, 0, 0};
    int sc = 127;
    if (h < a.H_I) {
      v = *(const i32x4*)(a.q + ((int64_t)t * a.H_I + h) * (DI / 2) + 16 * g);
      sc = a.q_scale[((int64_t)t * a.H_I + h) * (DI / kMxBlock) + g];
    }
    qa[mt] = i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
    qs[mt] = sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = mt * 16 + 4 * g + i;
      wreg[mt][i] = hw < a.H_I ? a.w[(int64_t)t * a.H_I + hw] : 0.f;
    }
  }

  i32x4 kc[NT];
  int ksc[NT];
  bool kval[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = e_base + nt * 16 + l16;
    const int pg = e < nv ? page_of(a.keys, seq, e) : -1;
    kval[nt] = pg >= 0;
    kc[nt] = i32x4{0, 0, 0, 0};
    ksc[nt] = 127;
    if (pg >= 0) {
      const uint8_t* pb = a.keys.base + (int64_t)pg * PAGE;
      kc[nt] = *(const i32x4*)(pb + (e & 63) * (DI / 2) + 16 * g);
      ksc[nt] = pb[SCALES + (e & 63) * (DI / kMxBlock) + g];
    }
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const i32x8 kb = {kc[nt].x, kc[nt].y, kc[nt].z, kc[nt].w, 0, 0, 0, 0};
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kb, acc, 4, 4, 0, qs[mt], 0,
                                                              ksc[nt]);
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wreg[mt][i] * fmaxf(acc[i], 0.f);
    }
    part += __shfl_xor(part, 16, 64);
    part += __shfl_xor(part, 32, 64);
    const int e = e_base + nt * 16 + l16;
    if (g == 0 && e < nv) a.scores[(int64_t)t * a.score_stride + e] = kval[nt] ? part : kNegInf;
  }
}

// ---------------------------------------------------------------- radix select
struct SelShared {
  unsigned hist[256];
  unsigned bin, above, cnt_bin;
  unsigned out_count;
};

// Finds the k-th largest key among participating elements (k >= 1, at least k participate).
// Returns the key; *need = how many elements equal to it belong to the top-k; *n_eq = how
// many participate with that key.
template <class KeyOf>
__device__ uint32_t radix_kth(SelShared& sh, int n, unsigned k, KeyOf key_of, unsigned* need,
                              unsigned* n_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  unsigned remaining = k;
  unsigned cnt_bin = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kTopkThreads) {
      uint32_t key;
      if (key_of(i, key) && (key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending)
      unsigned c[4], tot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = sh.hist[255 - 4 * tid - j];
        tot += c[j];
      }
      unsigned incl = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned v = __shfl_up(incl, o, 64);
        if (tid >= o) incl += v;
      }
      unsigned run = incl - tot;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run < remaining && run + c[j] >= remaining) {
          sh.bin = 255 - 4 * tid - j;
          sh.above = run;
          sh.cnt_bin = c[j];
        }
        run += c[j];
      }
    }
    __syncthreads();
    prefix |= sh.bin << shift;
    mask |= 255u << shift;
    remaining -= sh.above;
    cnt_bin = sh.cnt_bin;
    __syncthreads();
  }
  *need = remaining;
  *n_eq = cnt_bin;
  return prefix;
}

// Select the top-k of n elements (n > k) given key_of(i, key) and id_of(i); writes k ids (and
// scores) in arbitrary order.
template <class KeyOf, class IdOf, class Emit>
__device__ void block_topk(SelShared& sh, int n, int k, KeyOf key_of, IdOf id_of, Emit emit) {
  unsigned need, n_eq;
  const uint32_t T = radix_kth(sh, n, (unsigned)k, key_of, &need, &n_eq);
  uint32_t T2 = 0;          // ties: take ids whose ~id >= T2 (the `need` smallest ids)
  const bool tie_break = n_eq > need;
  if (tie_break) {
    unsigned need2, neq2;
    T2 = radix_kth(
        sh, n, need,
        [&](int i, uint32_t& key) {
          uint32_t kk;
          if (!key_of(i, kk) || kk != T) return false;
          key = ~(uint32_t)id_of(i);
          return true;
        },
        &need2, &neq2);
  }
  if (threadIdx.x == 0) sh.out_count = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kTopkThreads) {
    uint32_t key;
    if (!key_of(i, key)) continue;
    bool take = key > T;
    if (key == T) take = !tie_break || (~(uint32_t)id_of(i) >= T2);
    if (take) {
      const unsigned slot = atomicAdd(&sh.out_count, 1u);
      emit(slot, id_of(i), key);
    }
  }
  __syncthreads();
}

// One query per workgroup: short-context fill or one-stage select over its scores.
__global__ __launch_bounds__(kTopkThreads) void topk_single_kernel(IndexArgs a, int k,
                                                                   int32_t* out_idx,
                                                                   float* out_score) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  int seq, nv;
  query_of(a, t, seq, nv);
  const float* sc = a.scores + (int64_t)t * a.score_stride;
  int32_t* oi = out_idx + (int64_t)t * k;
  float* os = out_score ? out_score + (int64_t)t * k : nullptr;
  if (nv <= k) {
    for (int j = threadIdx.x; j < k; j += kTopkThreads) {
      oi[j] = j < nv ? j : -1;
      if (os) os[j] = j < nv ? sc[j] : 0.f;
    }
    return;
  }
  block_topk(
      sh, nv, k, [&](int i, uint32_t& key) { key = f32_order_key(sc[i]); return true; },
      [&](int i) { return i; },
      [&](unsigned slot, int id, uint32_t key) {
        if (slot < (unsigned)k) {
          oi[slot] = id;
          if (os) os[slot] = order_key_f32(key);
        }
      });
}

// Stage 1: the top-k of each 16384-entry chunk -> candidates (key, id); id -1 pads.
__global__ __launch_bounds__(kTopkThreads) void topk_stage1_kernel(IndexArgs a, int k, int nchunks,
                                                                   uint32_t* ckey, int32_t* cid) {
  __shared__ SelShared sh;
  const int t = blockIdx.x, c = blockIdx.y;
  int seq, nv;
  query_of(a, t, seq, nv);
  const int lo = c * kChunk;
  const int n = max(0, min(nv, lo + kChunk) - lo);
  uint32_t* ok = ckey + ((int64_t)t * nchunks + c) * k;
  int32_t* oi = cid + ((int64_t)t * nchunks + c) * k;
  const float* sc = a.scores + (int64_t)t * a.score_stride + lo;
  if (nv <= k) return;                   // stage 2 fills short-context queries directly
  if (n <= k) {
    for (int j = threadIdx.x; j < k; j += kTopkThreads) {
      oi[j] = j < n ? lo + j : -1;
      ok[j] = j < n ? f32_order_key(sc[j]) : 0u;
    }
    return;
  }
  block_topk(
      sh, n, k, [&](int i, uint32_t& key) { key = f32_order_key(sc[i]); return true; },
      [&](int i) { return lo + i; },
      [&](unsigned slot, int id, uint32_t key) {
        if (slot < (unsigned)k) {
          oi[slot] = id;
          ok[slot] = key;
        }
      });
}

// Stage 2: the top-k of a query's chunk winners.
__global__ __launch_bounds__(kTopkThreads) void topk_stage2_kernel(IndexArgs a, int k, int nchunks,
                                                                   const uint32_t* ckey,
                                                                   const int32_t* cid,
                                                                   int32_t* out_idx,
                                                                   float* out_score) {
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  int seq, nv;
  query_of(a, t, seq, nv);
  int32_t* oi = out_idx + (int64_t)t * k;
  float* os = out_score ? out_score + (int64_t)t * k : nullptr;
  if (nv <= k) {
    const float* sc = a.scores + (int64_t)t * a.score_stride;
    for (int j = threadIdx.x; j < k; j += kTopkThreads) {
      oi[j] = j < nv ? j : -1;
      if (os) os[j] = j < nv ? sc[j] : 0.f;
    }
    return;
  }
  const uint32_t* ck = ckey + (int64_t)t * nchunks * k;
  const int32_t* ci = cid + (int64_t)t * nchunks * k;
  block_topk(
      sh, nchunks * k,
      k, [&](int i, uint32_t& key) { key = ck[i]; return ci[i] >= 0; }, [&](int i) { return ci[i]; },
      [&](unsigned slot, int id, uint32_t key) {
        if (slot < (unsigned)k) {
          oi[slot] = id;
          if (os) os[slot] = order_key_f32(key);
        }
      });
}

}  // namespace

TopkPlan topk_plan(int N, int max_pos, int m, int topk) {
  TopkPlan p{};
  const int64_t nv = (int64_t)(max_pos + 1) / m;
  const int64_t stride = std::max<int64_t>(64, (nv + 63) / 64 * 64);
  p.score_bytes = (size_t)N * stride * sizeof(float);
  p.two_stage = nv > kSingleMax;
  p.nchunks = p.two_stage ? (int)((nv + kChunk - 1) / kChunk) : 0;
  p.cand_bytes = p.two_stage ? (size_t)N * p.nchunks * topk * (sizeof(uint32_t) + sizeof(int32_t)) : 0;
  p.ws_bytes = p.score_bytes + p.cand_bytes + 256;
  return p;
}

hipError_t launch_index_scores(const IndexArgs& a, int fmt, hipStream_t stream) {
  if (a.N == 0 || a.nv_cap == 0) return hipSuccess;
  const int MT = (a.H_I + 15) / 16;
  if (fmt == HCS_FMT_MXFP4) {
    const int per_wg = (kScoreThreads / 64) * 8 * 16;
    dim3 grid(a.N, (a.nv_cap + per_wg - 1) / per_wg);
    switch (MT) {
      case 1: hipLaunchKernelGGL((index_score_mxfp4_kernel<1>), grid, dim3(kScoreThreads), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((index_score_mxfp4_kernel<2>), grid, dim3(kScoreThreads), 0, stream, a); break;
      case 3: hipLaunchKernelGGL((index_score_mxfp4_kernel<3>), grid, dim3(kScoreThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL((index_score_mxfp4_kernel<4>), grid, dim3(kScoreThreads), 0, stream, a); break;
    }
    return hipGetLastError();
  }
  const int per_wg = (kScoreThreads / 64) * 4 * 16;
  dim3 grid(a.N, (a.nv_cap + per_wg - 1) / per_wg);
#define HCS_SCORE_CASE(DI_, MT_)                                                                    \
  if (a.d_I == DI_ && MT == MT_) {                                                                  \
    hipLaunchKernelGGL((index_score_bf16_kernel<DI_, MT_>), grid, dim3(kScoreThreads), 0, stream, a); \
    return hipGetLastError();                                                                       \
  }
  HCS_SCORE_CASE(32, 1) HCS_SCORE_CASE(32, 2) HCS_SCORE_CASE(32, 3) HCS_SCORE_CASE(32, 4)
  HCS_SCORE_CASE(64, 1) HCS_SCORE_CASE(64, 2) HCS_SCORE_CASE(64, 3) HCS_SCORE_CASE(64, 4)
  HCS_SCORE_CASE(128, 1) HCS_SCORE_CASE(128, 2) HCS_SCORE_CASE(128, 3) HCS_SCORE_CASE(128, 4)
#undef HCS_SCORE_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const IndexArgs& a, const TopkPlan& plan, int topk, int32_t* out_idx,
                       float* out_score, void* cand, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  if (!plan.two_stage) {
    hipLaunchKernelGGL(topk_single_kernel, dim3(a.N), dim3(kTopkThreads), 0, stream, a, topk,
                       out_idx, out_score);
    return hipGetLastError();
  }
  uint32_t* ckey = static_cast<uint32_t*>(cand);
  int32_t* cid = reinterpret_cast<int32_t*>(ckey + (size_t)a.N * plan.nchunks * topk);
  hipLaunchKernelGGL(topk_stage1_kernel, dim3(a.N, plan.nchunks), dim3(kTopkThreads), 0, stream, a,
                     topk, plan.nchunks, ckey, cid);
  hipLaunchKernelGGL(topk_stage2_kernel, dim3(a.N), dim3(kTopkThreads), 0, stream, a, topk,
                     plan.nchunks, ckey, cid, out_idx, out_score);
  return hipGetLastError();
}

}  // namespace hcs
