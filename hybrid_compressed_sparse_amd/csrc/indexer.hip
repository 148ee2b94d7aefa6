// Lightning-Indexer scores and exact top-k selection for gfx950.
//
// What it computes: "DeepSeek V4 Attention: Code Reading Map", section "Aux stream 0 (CSA
// only)": scores between the indexer queries and the compressed indexer keys, then the top-k
// compressed entries; score I[t,i] = sum_h w[t,h] * ReLU(q[t,h] . k[i]). When a query sees no
// more entries than k, all of them are selected ("DeepSeek V4.1 attention" API page,
// short-context rule).
//
// Scores: one workgroup scores 256 (bf16), 512 (FP8) or 1024 (MXFP4) consecutive entries of one
// query.
// The query's heads are the MFMA M dimension. bf16: a wave's 64 entries are one page of the
// cache, copied whole into LDS with async loads (as is the query), then read in MFMA operand
// order. MXFP4: the same, two pages per wave, and the cache's 32-value blocks are the MFMA
// operands as stored.
//   bf16 : v_mfma_f32_16x16x32_bf16, K = d_I in steps of 32;
//   MXFP4: v_mfma_scale_f32_16x16x128_f8f6f4 with both operands e2m1 and the UE8M0 block
//          scales as the instruction's scale operands; the documented cache layout (32
//          consecutive values per 16 bytes, low nibble first, one scale byte per 32) is exactly
//          the instruction's per-lane operand, so keys go from HBM to the matrix core untouched.
// The C layout puts 4 heads x 1 entry in each lane: ReLU, the head weights and the sum over
// heads are done in registers plus two cross-lane shuffles.
//
// Top-k: exact radix select on order-preserving 32-bit keys of the fp32 scores, 11 bits per
// pass below the keys' common leading bits, with LDS histograms in one 1024-thread workgroup
// per query (usually one pass: it stops when the k-th key's bin holds exactly the keys still
// needed); ties at the
// threshold are broken towards smaller entry ids by a second radix select on the ids. Queries
// that may see more than 32768 entries are filtered first: every full scoring block also
// records the kb-th largest of its scores; a bound taken from these (below) is at most the
// query's k-th largest score, so keeping only the scores at or above it loses nothing (a filter
// launch appends them as candidates), and the select then runs over the few candidates left.
#include "compress_impl.h"
#include "select.h"

namespace hcs {

HCS_DEVICE_ERROR_WORD(indexer)

namespace {

constexpr int kScoreThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kSingleMax = 32768;       // largest n_visible selected in one stage
constexpr float kNegInf = -__builtin_huge_valf();

// max(x, 0) as one integer max on the bits (a negative float is a negative int32; -0 gives
// +0). fmaxf costs two instructions here (it first quiets a possible NaN).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// v summed over lanes l, l ^ 16, l ^ 32, l ^ 48, in every lane, without LDS: after
// v_permlane16_swap of v with itself its two results hold v and the value of lane l ^ 16 (in
// one order or the other), and likewise v_permlane32_swap for lane l ^ 32. Each sum is the
// same float as v + (value of the partner lane).
__device__ __forceinline__ float sum_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ void query_of(const IndexArgs& a, int t, int& seq, int& nv) {
  int pos;
  if (a.q_seq) {
    seq = __ldg(a.q_seq + t);
    pos = min(__ldg(a.q_pos + t), a.pos_cap);
  } else {
    seq = a.seq_const;
    pos = a.p0 + t;
  }
  nv = min((pos + 1) / a.m, a.nv_cap);
  if (a.nv_div > 0) nv = (nv + a.nv_div - 1) / a.nv_div;
}

// ---------------------------------------------------------------- block thresholds
// A lower bound of a query's k-th largest score from per-block statistics: each of the F full
// blocks (E entries each) records b = its kb-th largest key. Take any T such that at least
// J = ceil(k / kb) of the blocks have b >= T: each of those holds kb keys >= b >= T, so the query
// has J * kb >= k keys >= T, its k-th largest key is >= T, and selecting among the keys >= T is
// exact. With kb = ceil(k / F), J <= F and T = min b works; with kb half as large again, J is
// about 2F/3 and T can sit near the upper third of the b's, a much tighter bound (about 3.5k
// instead of 9k candidates out of 262144 entries for k = 2048).
constexpr int kMaxKb = 32;                      // larger kb: no bound (T = 0, every key kept)

// kb of the block bounds for top-k over F full blocks (> kMaxKb: none recorded)
__device__ __forceinline__ int bound_kb(int topk, int full) {
  const int kb0 = (topk + full - 1) / full;
  const int kb = kb0 + (kb0 + 1) / 2;
  return kb <= kMaxKb ? kb : kb0;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v);

// One block's kb-th largest key (kb <= kMaxKb) over its waves' keys: lane L of wave w holds
// keys[0..NS) (0 for none; every entry held by exactly one lane). Returns the result in every
// thread. `wbest` is LDS of NW * kMaxKb words. Contains one barrier; call from all threads.
template <int NS, int NW>
__device__ __forceinline__ uint32_t block_kth_key(uint32_t (&keys)[NS], int kb, uint32_t* wbest,
                                                  uint32_t* result) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int it = 0; it < kb; ++it) {
    uint32_t lm = 0;
    int li = -1;
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (keys[j] > lm) {
        lm = keys[j];
        li = j;
      }
    const uint32_t wm = wave_max_u32(lm);
    const uint64_t who = __ballot(li >= 0 && lm == wm);
    const bool mine = who != 0 && lane == (int)__builtin_ctzll(who);
#pragma unroll
    for (int j = 0; j < NS; ++j) keys[j] = mine && j == li ? 0u : keys[j];
    if (lane == 0) wbest[wave * kMaxKb + it] = wm;
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int PER = (NW * kMaxKb + 63) / 64;
    uint32_t v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = lane + 64 * j, w = i / kMaxKb, it = i % kMaxKb;
      v[j] = w < NW && it < kb ? wbest[i] : 0u;
    }
    uint32_t kth = 0;
    for (int it = 0; it < kb; ++it) {
      uint32_t lm = 0;
      int li = -1;
#pragma unroll
      for (int j = 0; j < PER; ++j)
        if (v[j] > lm) {
          lm = v[j];
          li = j;
        }
      kth = wave_max_u32(lm);
      const uint64_t who = __ballot(li >= 0 && lm == kth);
      const bool mine = who != 0 && lane == (int)__builtin_ctzll(who);
#pragma unroll
      for (int j = 0; j < PER; ++j) v[j] = mine && j == li ? 0u : v[j];
    }
    if (lane == 0) *result = kth;
  }
  __syncthreads();
  return *result;
}

// One wave's kb-th largest key (kb <= kMaxKb) over its lanes' keys[0..NS) (0 for none; every
// entry held by exactly one lane), in every lane; 0 when the wave holds fewer than kb keys.
template <int NS>
__device__ __forceinline__ uint32_t wave_kth_key(uint32_t (&keys)[NS], int kb) {
  const int lane = threadIdx.x & 63;
  uint32_t wm = 0u;
  for (int it = 0; it < kb; ++it) {
    uint32_t lm = 0;
    int li = -1;
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (keys[j] > lm) {
        lm = keys[j];
        li = j;
      }
    wm = wave_max_u32(lm);
    const uint64_t who = __ballot(li >= 0 && lm == wm);
    const bool mine = who != 0 && lane == (int)__builtin_ctzll(who);
#pragma unroll
    for (int j = 0; j < NS; ++j) keys[j] = mine && j == li ? 0u : keys[j];
  }
  return wm;
}

// Scoring blocks call this after writing their scores when a.blk_thr is set: E entries per
// block, `keys` as for block_kth_key. Writes the block's threshold when the block is full.
template <int NS, int NW, int E>
__device__ __forceinline__ void write_block_threshold(const IndexArgs& a, int nv, uint32_t (&keys)[NS],
                                                      uint32_t* wbest, uint32_t* result) {
  const int full = nv / E;                             // full blocks of this query
  if (full == 0 || (int)blockIdx.y >= full) return;    // uniform over the block
  const int kb = bound_kb(a.topk, full);
  if (kb > kMaxKb) return;                             // the filter keeps every key then
  const uint32_t kth = block_kth_key<NS, NW>(keys, kb, wbest, result);
  if (threadIdx.x == 0) a.blk_thr[(int64_t)blockIdx.x * a.thr_stride + blockIdx.y] = kth;
}

// ---------------------------------------------------------------- bf16 scores
// A zero row for the query heads a launch pads to a multiple of 16.
__device__ __attribute__((aligned(64))) uint8_t g_ix_zero[1024];
// A zero page of MXFP4 keys (64 rows of 64 code bytes and 4 scale bytes) for absent pages.
__device__ __attribute__((aligned(64))) uint8_t g_ix_zero_page[64 * 68];

// Block = 256 entries of one query (4 waves x one 64-entry page each). The page of a wave's
// entries is one contiguous region of the paged cache, so it is copied into LDS with 1 KiB
// async loads, as is the query (64 heads x d_I, shared by the waves); both are stored with the
// 16-byte chunks of row r at chunk ^ (r mod CPR), which makes the MFMA operand reads below free
// of bank conflicts.
template <int DI>
struct Bf16ScoreLds {
  static constexpr int RB = DI * 2;                   // bytes per key / query row
  static constexpr int PAGE = kPageRows * RB;
  static constexpr int BYTES = 64 * RB + 4 * PAGE;    // q rows, then one key page per wave
};

// Scores of query t, 256-entry chunk yb into a.scores. Every thread of the block must call it
// (it has one barrier); `smem` holds Bf16ScoreLds<DI>::BYTES.
template <int DI, int MT>
__device__ __forceinline__ void score_block_bf16(const IndexArgs& a, uint8_t* smem, uint32_t (&tkeys)[4],
                                                 int t, int yb) {
  constexpr int KS = DI / 32;
  constexpr int NT = 4;                  // 4 x 16 entries per wave
  constexpr int RB = Bf16ScoreLds<DI>::RB;
  constexpr int CPR = RB / 16;           // 16-byte chunks per row
  constexpr int RPI = 1024 / RB;         // rows per 1 KiB async load
  constexpr int PAGE = Bf16ScoreLds<DI>::PAGE;
  uint8_t* qs = smem;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  // query rows: wave w copies heads 16w .. 16w+15 (heads >= H_I read zeros)
  const uint8_t* q = reinterpret_cast<const uint8_t*>(a.q);
#pragma unroll
  for (int i = 0; i < 16 / RPI; ++i) {
    const int h = 16 * wave + i * RPI + lane / CPR, c = lane % CPR;
    const uint8_t* src = h < a.H_I ? q + ((int64_t)t * a.H_I + h) * RB + ((c ^ (h & (CPR - 1))) << 4)
                                   : g_ix_zero + lane * 16;
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)(qs + (16 * wave + i * RPI) * RB),
                                     16, 0, 0);
  }
  float wreg[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = mt * 16 + 4 * g + i;
      wreg[mt][i] = hw < a.H_I ? a.w[(int64_t)t * a.H_I + hw] : 0.f;
    }
  int seq, nv;
  query_of(a, t, seq, nv);
  const int e_base = yb * 256 + wave * 64;                  // first entry of this wave's page
  const bool active = e_base < nv;
  const int pg = active ? page_of(a.keys, seq, e_base) : -1;
  uint8_t* kl = smem + 64 * RB + wave * PAGE;
  if (pg >= 0) {
    const uint8_t* page = a.keys.base + (int64_t)pg * PAGE;
#pragma unroll
    for (int i = 0; i < kPageRows / RPI; ++i) {
      const int r = i * RPI + lane / CPR, c = lane % CPR;
      __builtin_amdgcn_global_load_lds((const void*)(page + r * RB + ((c ^ (r & (CPR - 1))) << 4)),
                                       (__attribute__((address_space(3))) void*)(kl + i * 1024), 16, 0, 0);
    }
  }
  __syncthreads();                                    // every wave's copies have landed
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) tkeys[nt] = 0u;
  if (!active) return;
  bf16x8 qreg[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + l16;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qreg[mt][kk] = *(const bf16x8*)(qs + h * RB + (((4 * kk + g) ^ (h & (CPR - 1))) << 4));
  }
  bf16x8 kreg[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int r = nt * 16 + l16;
      kreg[nt][kk] = *(const bf16x8*)(kl + r * RB + (((4 * kk + g) ^ (r & (CPR - 1))) << 4));
    }
  // Software-pipelined over the wave's entry tiles: tile nt's MFMAs are issued among tile nt-1's
  // ReLU, weighting and cross-lane sum (groups of one MFMA and two VALU instructions). Every
  // accumulator and partial sum keeps its order, so the bits do not depend on the interleave.
  f32x4 acc[2][MT];
  auto mfma_tile = [&](int nt, f32x4 (&ac)[MT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ac[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        ac[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qreg[mt][kk], kreg[nt][kk], ac[mt], 0, 0, 0);
  };
  auto finish_tile = [&](int nt, const f32x4 (&ac)[MT]) {
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part += wreg[mt][i] * relu(ac[mt][i]);
    part = sum_xor16_32(part);
    const int e = e_base + nt * 16 + l16;
    const float sv = pg >= 0 ? part : kNegInf;
    if (g == 0 && e < nv) a.scores[(int64_t)t * a.score_stride + e] = sv;
    tkeys[nt] = g == 0 && e < nv ? f32_order_key(sv) : 0u;
  };
  mfma_tile(0, acc[0]);
#pragma unroll
  for (int nt = 1; nt < NT; ++nt) {
    __builtin_amdgcn_sched_barrier(0);
    mfma_tile(nt, acc[nt & 1]);
    finish_tile(nt - 1, acc[(nt - 1) & 1]);
#pragma unroll
    for (int i = 0; i < MT * KS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  finish_tile(NT - 1, acc[(NT - 1) & 1]);
}

template <int DI, int MT>
__global__ __launch_bounds__(kScoreThreads) void index_score_bf16_kernel(IndexArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Bf16ScoreLds<DI>::BYTES];
  __shared__ uint32_t wbest[4 * kMaxKb + 1];
  uint32_t tkeys[4];
  if (a.cand_count && blockIdx.y == 0 && threadIdx.x == 0) a.cand_count[blockIdx.x] = 0u;
  score_block_bf16<DI, MT>(a, smem, tkeys, blockIdx.x, blockIdx.y);
  if (a.blk_thr) {
    int seq, nv;
    query_of(a, blockIdx.x, seq, nv);
    write_block_threshold<4, 4, 256>(a, nv, tkeys, wbest, wbest + 4 * kMaxKb);
  }
}

// Scoring blocks and compressor blocks in one launch (a decode step): the two touch disjoint
// data (the indexer keys and scores; the KV compressor's state and compressed cache), so the
// step saves one dependent launch. Blocks [0, nc) compress (they are short and start first),
// the rest score: block nc + i is query i / chunks, chunk i % chunks.
template <int DI, int MT>
__global__ __launch_bounds__(kScoreThreads) void index_score_compress_kernel(IndexArgs a, CompressArgs c,
                                                                              int chunks, int cy, int cz) {
  static_assert(kScoreThreads == kCompressThreads, "one block size for both roles");
  __shared__ __attribute__((aligned(16))) uint8_t smem[Bf16ScoreLds<DI>::BYTES];
  const int nc = c.B * cy * cz;
  const int bid = blockIdx.x;
  if (bid < nc) {                                   // uniform over the block
    const int z = bid % cz, y = (bid / cz) % cy, b = bid / (cz * cy);
    compress_block(c, b, y, z, cy);
    return;
  }
  const int i = bid - nc;
  uint32_t tkeys[4];
  score_block_bf16<DI, MT>(a, smem, tkeys, i / chunks, i % chunks);
}

// ---------------------------------------------------------------- bf16 scores, query chunks
// The queries of a chunk (consecutive positions of one sequence, as in prefill) score the same
// keys, so their scores are one matrix product, [queries x heads, d_I] x [d_I, entries],
// followed by ReLU and the weighted sum over heads. A block holds 512 consecutive entries in
// registers (8 waves x one 64-entry page, the B operand of v_mfma_f32_16x16x32_bf16, loaded
// once) and walks up to 64 queries: the q rows (64 x 128 bf16) and head weights of query t+1
// are copied into the other half of a double-buffered LDS slot while query t is scored, so keys
// are read once per 64 queries instead of once per query. Per query a wave does 64 MFMAs
// (4 entry tiles x 4 head tiles x 4 k-steps) with q read from LDS in operand order (16-byte
// chunk c of head h stored at c ^ (h mod 16): conflict-free). The arithmetic per score is that
// of index_score_bf16_kernel, in the same order, so both give the same bits.
// The scores of query t are stored one iteration later, after the wait for the copy of query
// t+1: on gfx9 one counter covers loads and stores, and stores issued a whole query earlier
// have completed by then, so that wait does not stall on them.
#ifndef HCS_CHUNK_WAVES
#define HCS_CHUNK_WAVES 4
#endif
#ifndef HCS_CHUNK_TILES
#define HCS_CHUNK_TILES 4
#endif
constexpr int kChunkWaves = HCS_CHUNK_WAVES;
constexpr int kChunkThreads = 64 * kChunkWaves;
constexpr int kChunkTiles = HCS_CHUNK_TILES;     // 16-entry tiles per wave
constexpr int kChunkEntries = kChunkWaves * 16 * kChunkTiles;   // entries per block
constexpr int kChunkQueries = 64;                // queries per block
constexpr int kChunkMinQueries = 256;            // smaller chunks use the per-query kernel
#ifndef HCS_CHUNK_PER_STEP
#define HCS_CHUNK_PER_STEP 2
#endif
constexpr int kChunkPerStep = HCS_CHUNK_PER_STEP; // queries per barrier

template <int MT>
__global__ __launch_bounds__(kChunkThreads, 512 / kChunkThreads) void index_score_chunk_kernel(IndexArgs a) {
  constexpr int DI = 128, KS = DI / 32, RB = DI * 2, CPR = RB / 16;
  constexpr int PAGE = kPageRows * RB;
  constexpr int QP = kChunkPerStep;               // queries per LDS slot (one barrier each)
  __shared__ __attribute__((aligned(16))) uint8_t qbuf[2][QP][64 * RB];
  __shared__ __attribute__((aligned(16))) float wbuf[2][QP][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int eb = blockIdx.x * kChunkEntries;                      // first entry of the block
  constexpr int NTW = kChunkTiles, HPW = 64 / kChunkWaves;        // heads each wave copies
  static_assert(NTW == 4, "a wave's entries are one 64-entry page (score rows are whole pages)");
  const int e0 = eb + wave * 16 * NTW;                            // this wave's entries
  // queries t0 .. t1-1; the first that sees any entry of the block is the first with
  // (p0 + t + 1) / m > eb, i.e. p0 + t + 1 >= (eb + 1) m
  const int t1 = min((int)(blockIdx.y + 1) * kChunkQueries, a.N);
  const int64_t t_vis = (int64_t)(eb + 1) * a.m - a.p0 - 1;
  const int t0 = (int)max<int64_t>((int64_t)blockIdx.y * kChunkQueries, t_vis);
  if (t0 >= t1 || eb >= a.nv_cap) return;                        // uniform over the block

  // q rows and head weights of queries t .. t+QP-1 (those below t1) into slot `buf`: wave w
  // copies heads HPW w .. +HPW-1, each lane at a constant offset from the query's q (a head of
  // H_I or more reads the last real head; its weight is 0); lanes below H_I / 4 of wave 0 copy
  // the weights (H_I % 4 == 0) into a slot whose other words stay zero
  if (threadIdx.x < 2 * QP * 64) (&wbuf[0][0][0])[threadIdx.x] = 0.f;
  uint32_t q_off[HPW / 4];
#pragma unroll
  for (int i = 0; i < HPW / 4; ++i) {
    const int h = HPW * wave + 4 * i + lane / CPR, c = lane % CPR;
    q_off[i] = (uint32_t)(min(h, a.H_I - 1) * RB + ((c ^ (h & 15)) << 4));
  }
  auto copy_q = [&](int t, int buf) {
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      if (t + u >= t1) break;
      const uint8_t* qt = a.q + (int64_t)(t + u) * a.H_I * RB;
#pragma unroll
      for (int i = 0; i < HPW / 4; ++i) dma16(qt, q_off[i], lds_addr(qbuf[buf][u]) + (HPW * wave + 4 * i) * RB);
      if (wave == 0 && lane < a.H_I / 4)
        dma16(reinterpret_cast<const uint8_t*>(a.w + (int64_t)(t + u) * a.H_I), (uint32_t)lane * 16,
              lds_addr(wbuf[buf][u]));
    }
  };
  __syncthreads();                               // zeroed weight slots before any copy
  copy_q(t0, 0);

  // keys: kreg[nt][ks] = elements 32 ks + 8 g .. +7 of entry e0 + 16 nt + l16 (B operand)
  bf16x8 kreg[NTW][KS];
#pragma unroll
  for (int p = 0; p < NTW / 4; ++p) {                             // one 64-entry page each
    const int ep = e0 + 64 * p;
    const int pg = ep < a.nv_cap ? page_of(a.keys, a.seq_const, ep) : -1;
    const uint8_t* page = pg >= 0 ? a.keys.base + (int64_t)pg * PAGE : nullptr;
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const i32x4 v = page ? *(const i32x4*)(page + (16 * n4 + l16) * RB + 64 * ks + 16 * g)
                             : i32x4{0, 0, 0, 0};
        kreg[4 * p + n4][ks] = __builtin_bit_cast(bf16x8, v);
      }
  }

  // scores of the previous step, not yet stored. A query's row is written for every entry of
  // this wave's page, also those it does not see (the selection reads only visible ones); the
  // row stride covers every page below nv_cap.
  float sc[QP][NTW];
  int t_prev = -1;
  const bool wave_has_entries = e0 < a.nv_cap;
  auto store_prev = [&]() {
    if (t_prev < 0 || !wave_has_entries || g != 0) return;
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int t = t_prev + u;
      if (t >= t1) break;
      float* row = a.scores + (int64_t)t * a.score_stride + e0 + l16;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) row[16 * nt] = sc[u][nt];
    }
  };
  for (int t = t0, it = 0; t < t1; t += QP, ++it) {
    const int buf = it & 1;
    wait_vm_zero();                              // this wave's copies of this step (and keys)
    lds_barrier();                               // every wave's copies of this step
    store_prev();
    if (t + QP < t1) copy_q(t + QP, buf ^ 1);
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      bf16x8 qa[MT][KS];
      float wreg[MT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int h = mt * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qa[mt][ks] = *(const bf16x8*)(qbuf[buf][u] + h * RB + (((4 * ks + g) ^ (h & (CPR - 1))) << 4));
        const f32x4 w4 = *(const f32x4*)(wbuf[buf][u] + mt * 16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) wreg[mt][i] = w4[i];
      }
      // Software-pipelined over the wave's four entry tiles: tile nt's 16 MFMAs are issued among
      // tile nt-1's ReLU, weight and cross-lane reduction (scheduling groups of one MFMA and two
      // VALU instructions), so the VALU work runs in the MFMAs' shadow instead of after them.
      // Each accumulator still sums its k-steps in order: the same bits as before.
      f32x4 acc[2][MT];
      auto mfma_tile = [&](int nt, f32x4 (&ac)[MT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ac[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            ac[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kreg[nt][ks], ac[mt], 0, 0, 0);
      };
      auto reduce_tile = [&](const f32x4 (&ac)[MT]) {
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) part += wreg[mt][i] * relu(ac[mt][i]);
        return sum_xor16_32(part);
      };
      mfma_tile(0, acc[0]);
#pragma unroll
      for (int nt = 1; nt < NTW; ++nt) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_tile(nt, acc[nt & 1]);
        sc[u][nt - 1] = reduce_tile(acc[(nt - 1) & 1]);
#pragma unroll
        for (int i = 0; i < MT * KS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      sc[u][NTW - 1] = reduce_tile(acc[(NTW - 1) & 1]);
    }
    t_prev = t;
  }
  store_prev();
}

// ---------------------------------------------------------------- MXFP4 scores (d_I = 128)
// Block = 1024 entries of one query: 4 waves x four 64-entry pages. Heads are the M dimension of
// v_mfma_scale_f32_16x16x128_f8f6f4, entries the N dimension; a lane's operand is the 16 bytes
// (32 e2m1 values) of one 32-value block and its scale byte. In the cache's layout (a page is
// 64 x 64 B codes, then 64 x 4 UE8M0 bytes) the operand of lane (g, l16) for entry r is bytes
// 16 g .. 16 g + 15 of row r, so the 16 rows of an MFMA are 1 KiB of consecutive bytes: keys go
// from HBM straight into registers with coalesced loads, no LDS, and a wave has all four of
// its pages in flight at once (the query's codes likewise, from its contiguous rows).
constexpr int kMx4BlockEntries = 1024;

// One scoring block of query t: entries y * kMx4BlockEntries .. + kMx4BlockEntries - 1.
template <int MT>
__device__ __forceinline__ void score_block_mxfp4(const IndexArgs& a, int t, int y) {
  constexpr int DI = 128;
  constexpr int CB = DI / 2;                                     // code bytes per row
  constexpr int SB = DI / kMxBlock;                              // scale bytes per row
  constexpr int PAGE = kPageRows * (CB + SB);                    // 4352
  constexpr int SCALES = kPageRows * CB;                         // scale region offset
  constexpr int PPW = kMx4BlockEntries / 4 / kPageRows;          // pages per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  if (a.cand_count && y == 0 && threadIdx.x == 0) a.cand_count[t] = 0u;
  int seq, nv;
  query_of(a, t, seq, nv);
  const int e_base = y * kMx4BlockEntries + wave * (PPW * 64);   // first entry of the wave
  // the wave's page ids: lane p < PPW reads page p's table entry
  int my_pg = -1;
  if (lane < PPW && e_base + 64 * lane < nv) {
    const int pg = __ldg(a.keys.pt + (int64_t)seq * a.keys.pt_stride + (e_base >> 6) + lane);
    if (pg >= a.keys.num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
    my_pg = pg >= 0 && pg < a.keys.num_pages ? pg : -1;
  }
  // query codes (head mt*16 + l16, block g) and scales, head weights
  i32x8 qa[MT];
  int qs[MT];
  float wreg[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int h = mt * 16 + l16;
    const i32x4 v = h < a.H_I ? *(const i32x4*)(a.q + ((int64_t)t * a.H_I + h) * CB + 16 * g)
                              : i32x4{0, 0, 0, 0};
    qa[mt] = i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
    qs[mt] = h < a.H_I ? a.q_scale[((int64_t)t * a.H_I + h) * SB + g] : 127;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = mt * 16 + 4 * g + i;
      wreg[mt][i] = hw < a.H_I ? a.w[(int64_t)t * a.H_I + hw] : 0.f;
    }
  }
  // every key operand of the wave's pages (a page that is not there reads the zero page)
  int pgs[PPW];
  i32x4 kc[PPW][4];
  int ksc[PPW][4];
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    pgs[p] = __builtin_amdgcn_readlane(my_pg, p);
    const uint8_t* page = pgs[p] >= 0 ? a.keys.base + (int64_t)pgs[p] * PAGE : g_ix_zero_page;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int r = nt * 16 + l16;
      kc[p][nt] = *(const i32x4*)(page + r * CB + 16 * g);
      ksc[p][nt] = page[SCALES + r * SB + g];
    }
  }
  // after the sum over heads every lane of a 16-lane group holds the score of entry row r = 16 nt
  // + l16; lane (g, l16) keeps group nt == g's, so the 64 lanes hold the 64 entries of each page
  // once (entry e_base + 64 p + lane)
  float sc[PPW];
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const i32x8 kbv = {kc[p][nt].x, kc[p][nt].y, kc[p][nt].z, kc[p][nt].w, 0, 0, 0, 0};
      float part = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kbv, acc, 4, 4, 0, qs[mt], 0, ksc[p][nt]);
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wreg[mt][i] * relu(acc[i]);
      }
      part = sum_xor16_32(part);
      if (nt == 0 || g == nt) sc[p] = part;
    }
  }
  uint32_t lmax = 0u;                                 // this lane's largest key (0: none)
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    const int e = e_base + 64 * p + lane;
    const float sv = pgs[p] >= 0 ? sc[p] : kNegInf;
    if (e < nv) {
      a.scores[(int64_t)t * a.score_stride + e] = sv;
      lmax = max(lmax, f32_order_key(sv));
    }
  }
  if (a.blk_thr) {
    // a threshold per wave (its 256 entries are a block of the bound): the kb-th largest of the
    // 64 lanes' largest keys. At least kb lanes, so at least kb distinct entries, have a key at
    // or above it, which is all the bound needs; no barrier
    const int full = nv / (PPW * 64), wb = y * 4 + wave;
    const int kb = full > 0 ? bound_kb(a.topk, full) : kMaxKb + 1;
    if (wb < full && kb <= kMaxKb) {
      uint32_t kth = 0u, v = lmax;
      for (int it = 0; it < kb; ++it) {
        kth = wave_max_u32(v);
        const uint64_t who = __ballot(v == kth);
        if (lane == (int)__builtin_ctzll(who)) v = 0u;   // who != 0: the maximum is some lane's
      }
      if (lane == 0) a.blk_thr[(int64_t)t * a.thr_stride + wb] = kth;
    }
  }
}

// (at least four waves per SIMD: 126 VGPRs, no spills; five would spill)
template <int MT>
__global__ __launch_bounds__(kScoreThreads, 4) void index_score_mxfp4_kernel(IndexArgs a) {
  score_block_mxfp4<MT>(a, blockIdx.x, blockIdx.y);
}

// The MXFP4 scoring blocks and the compressor's blocks of one decode step in one grid (as
// index_score_compress_kernel for bf16 keys): the compressor's blocks first, then query t's
// scoring block y at t * chunks + y.
template <int MT>
__global__ __launch_bounds__(kScoreThreads, 4) void index_score_mxfp4_compress_kernel(IndexArgs a, CompressArgs c,
                                                                                   int chunks, int cy, int cz) {
  static_assert(kScoreThreads == kCompressThreads, "one block size for both roles");
  const int nc = c.B * cy * cz;
  const int bid = blockIdx.x;
  if (bid < nc) {                                   // uniform over the block
    const int z = bid % cz, y = (bid / cz) % cy, b = bid / (cz * cy);
    compress_block(c, b, y, z, cy);
    return;
  }
  const int i = bid - nc;
  score_block_mxfp4<MT>(a, i / chunks, i % chunks);
}

// ---------------------------------------------------------------- FP8 scores (d_I = 128)
// The MXFP4 kernel's structure for the 132-byte FP8 rows (128 e4m3 codes, one float32 scale):
// 512 entries of one query per block, 4 waves x two pages. A page is [64 x 128 B codes][64 x
// float32 scales]; a row's 16-byte chunk c is stored in LDS at c ^ ((r >> 1) & 7), so the 16
// rows of an operand read fall on distinct banks. The codes go to
// v_mfma_scale_f32_16x16x128_f8f6f4 as e4m3 with unit block scales (a lane's operand is 32
// consecutive codes of one row); the float scales are applied after the product: the query's
// per head with its weight (ReLU commutes with a positive factor), the key's per entry after the
// sum over heads.
template <int MT>
__global__ __launch_bounds__(kScoreThreads) void index_score_fp8_kernel(IndexArgs a) {
  constexpr int DI = 128;
  constexpr int PAGE = kPageRows * (DI + 4);                     // 8448
  constexpr int SCALES = kPageRows * DI;                         // scale region offset
  constexpr int PPW = 2;                                         // pages per wave
  __shared__ __attribute__((aligned(16))) uint8_t qc[64 * DI];
  __shared__ __attribute__((aligned(16))) uint8_t kb[4][PPW][PAGE];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  if (a.cand_count && blockIdx.y == 0 && threadIdx.x == 0) a.cand_count[t] = 0u;
  // query codes: wave w copies heads 16w .. 16w+15, 2 loads of 8 heads (heads >= H_I read zeros)
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int h = 16 * wave + 8 * i + lane / 8, c = lane % 8;
    const uint8_t* src = h < a.H_I ? a.q + ((int64_t)t * a.H_I + h) * DI + ((c ^ ((h >> 1) & 7)) << 4)
                                   : g_ix_zero + lane * 16;
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)(qc + (16 * wave + 8 * i) * DI), 16, 0, 0);
  }
  const float* q_scalef = reinterpret_cast<const float*>(a.q_scale);
  float wq[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hw = mt * 16 + 4 * g + i;
      wq[mt][i] = hw < a.H_I ? a.w[(int64_t)t * a.H_I + hw] * q_scalef[(int64_t)t * a.H_I + hw] : 0.f;
    }
  }
  int seq, nv;
  query_of(a, t, seq, nv);
  const int e_base = blockIdx.y * (4 * PPW * 64) + wave * (PPW * 64);
  int my_pg = -1;
  if (lane < PPW && e_base + 64 * lane < nv) {
    const int pg = __ldg(a.keys.pt + (int64_t)seq * a.keys.pt_stride + (e_base >> 6) + lane);
    if (pg >= a.keys.num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
    my_pg = pg >= 0 && pg < a.keys.num_pages ? pg : -1;
  }
  int pgs[PPW];
#pragma unroll
  for (int p = 0; p < PPW; ++p) {
    pgs[p] = __builtin_amdgcn_readlane(my_pg, p);
    if (pgs[p] < 0) continue;
    const uint8_t* page = a.keys.base + (int64_t)pgs[p] * PAGE;
    uint8_t* dst = kb[wave][p];
#pragma unroll
    for (int i = 0; i < 8; ++i) {                                 // codes: 8 entries per load
      const int r = 8 * i + lane / 8, c = lane % 8;
      __builtin_amdgcn_global_load_lds((const void*)(page + r * DI + ((c ^ ((r >> 1) & 7)) << 4)),
                                       (__attribute__((address_space(3))) void*)(dst + i * 1024), 16, 0, 0);
    }
    if (lane < 16)                                                // scales: 256 bytes
      __builtin_amdgcn_global_load_lds((const void*)(page + SCALES + lane * 16),
                                       (__attribute__((address_space(3))) void*)(dst + SCALES), 16, 0, 0);
  }
  __syncthreads();                                                // every copy has landed
  uint32_t tkeys[PPW * 4];
#pragma unroll
  for (int j = 0; j < PPW * 4; ++j) tkeys[j] = 0u;
  if (e_base < nv) {
    // a lane's operand: codes 32g .. 32g+31 of its row = chunks 2g and 2g+1
    auto operand = [&](const uint8_t* base, int r) __attribute__((always_inline)) {
      const int f = (r >> 1) & 7;
      const i32x4 lo = *(const i32x4*)(base + r * DI + (((2 * g) ^ f) << 4));
      const i32x4 hi = *(const i32x4*)(base + r * DI + (((2 * g + 1) ^ f) << 4));
      return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    };
    i32x8 qa[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) qa[mt] = operand(qc, mt * 16 + l16);
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const uint8_t* kp = kb[wave][p];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int r = nt * 16 + l16;
        const i32x8 kbv = operand(kp, r);
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[mt], kbv, acc, 0, 0, 0, 127, 0, 127);
#pragma unroll
          for (int i = 0; i < 4; ++i) part += wq[mt][i] * relu(acc[i]);
        }
        part = sum_xor16_32(part) * reinterpret_cast<const float*>(kp + SCALES)[r];
        const int e = e_base + 64 * p + r;
        const float sv = pgs[p] >= 0 ? part : kNegInf;
        if (g == 0 && e < nv) a.scores[(int64_t)t * a.score_stride + e] = sv;
        tkeys[p * 4 + nt] = g == 0 && e < nv ? f32_order_key(sv) : 0u;
      }
    }
  }
  if (a.blk_thr) {
    __shared__ uint32_t wbest[4 * kMaxKb + 1];
    write_block_threshold<PPW * 4, 4, 4 * PPW * 64>(a, nv, tkeys, wbest, wbest + 4 * kMaxKb);
  }
}

// dst[i] = f(src[i]) for i < n (global to LDS), NT threads: eight loads per thread are issued
// before their stores, at clamped indices (a conditional load would be a branch, and the
// compiler waits for each such load alone at its merge).
template <int NT, class T, class F>
__device__ __forceinline__ void lds_fill(uint32_t* dst, const T* src, int n, F f) {
  if (n <= 0) return;
  for (int i0 = 0; i0 < n; i0 += 8 * NT) {
    T v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[min(i0 + u * NT + (int)threadIdx.x, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * NT + (int)threadIdx.x;
      if (i < n) dst[i] = f(v[u]);
    }
  }
}

// One query's select over its scores with IPT keys per thread (ids tid * IPT ..), in registers.
template <int NT, int IPT>
__device__ __forceinline__ void topk_single_regs(SelShared& sh, const float* sc, int nv, int k, int32_t* oi,
                                                 float* os) {
  const int i0 = threadIdx.x * IPT;
  float v[IPT];
  // loads at clamped indices (a conditional load would be a branch and a wait of its own)
#pragma unroll
  for (int j = 0; j < IPT; ++j) v[j] = sc[min(i0 + j, nv - 1)];
  uint32_t key[IPT], vmask = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    key[j] = f32_order_key(v[j]);
    vmask |= (i0 + j < nv ? 1u : 0u) << j;
  }
  sel_reset<NT>(sh);
  __syncthreads();
  reg_topk<NT, IPT>(sh, key, vmask, (unsigned)k, true, [&](int j) { return i0 + j; },
                    [&](unsigned pos, int j, uint32_t kk) {
                      if (pos < (unsigned)k) {
                        oi[pos] = i0 + j;
                        if (os) os[pos] = order_key_f32(kk);
                      }
                    });
}

// The same with the ids strided over the threads (slot j of thread tid: id j NT + tid), so that
// every load instruction reads consecutive scores and every thread holds keys; the output order
// is thread, then slot (fixed, not ascending), ties to the smaller ids by a second select.
template <int NT, int IPT>
__device__ __forceinline__ void topk_single_strided(SelShared& sh, const float* sc, int nv, int k, int32_t* oi,
                                                    float* os) {
  const int tid = threadIdx.x;
  float v[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) v[j] = sc[min(j * NT + tid, nv - 1)];
  uint32_t key[IPT], vmask = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    key[j] = f32_order_key(v[j]);
    vmask |= (j * NT + tid < nv ? 1u : 0u) << j;
  }
  sel_reset<NT>(sh);
  __syncthreads();
  reg_topk<NT, IPT>(sh, key, vmask, (unsigned)k, false, [&](int j) { return j * NT + tid; },
                    [&](unsigned pos, int j, uint32_t kk) {
                      if (pos < (unsigned)k) {
                        oi[pos] = j * NT + tid;
                        if (os) os[pos] = order_key_f32(kk);
                      }
                    });
}

// One query per workgroup: short-context fill or one-stage select over its scores, the keys in
// registers. Up to 8 NT visible entries (decode) the ids come out in ascending order; more
// (prefill chunks) in a fixed order of their own. NT threads, at most KL visible entries.
template <int NT, int KL>
__global__ __launch_bounds__(NT) void topk_single_kernel(IndexArgs a, int k, int32_t* out_idx,
                                                         float* out_score) {
  static_assert(KL <= 32 * NT, "at most 32 keys per thread");
  __shared__ SelShared sh;
  const int t = blockIdx.x;
  int seq, nv;
  query_of(a, t, seq, nv);
  const float* sc = a.scores + (int64_t)t * a.score_stride;
  int32_t* oi = out_idx + (int64_t)t * k;
  float* os = out_score ? out_score + (int64_t)t * k : nullptr;
  if (nv <= k) {
    for (int j = threadIdx.x; j < k; j += NT) {
      oi[j] = j < nv ? j : -1;
      if (os) os[j] = j < nv ? sc[j] : 0.f;
    }
    return;
  }
  if (nv <= 4 * NT) {
    topk_single_regs<NT, 4>(sh, sc, nv, k, oi, os);
    return;
  }
  if (nv <= 8 * NT) {
    topk_single_regs<NT, 8>(sh, sc, nv, k, oi, os);
    return;
  }
  if (nv <= 16 * NT) {
    topk_single_strided<NT, 16>(sh, sc, nv, k, oi, os);
    return;
  }
  // 32 keys per thread spill registers: instantiated only where KL needs it
  if constexpr (KL <= 24 * NT) {
    topk_single_strided<NT, 24>(sh, sc, nv, k, oi, os);
  } else {
    if (nv <= 24 * NT) topk_single_strided<NT, 24>(sh, sc, nv, k, oi, os);
    else topk_single_strided<NT, 32>(sh, sc, nv, k, oi, os);
  }
}

// The one-stage select launch for at most nv_cap visible entries per query.
hipError_t launch_topk_single(const IndexArgs& a, int nv_cap, int k, int32_t* out_idx, float* out_score,
                              hipStream_t stream) {
  if (nv_cap <= 24 * kTopkThreads)
    hipLaunchKernelGGL((topk_single_kernel<kTopkThreads, 24 * kTopkThreads>), dim3(a.N), dim3(kTopkThreads), 0,
                       stream, a, k, out_idx, out_score);
  else
    hipLaunchKernelGGL((topk_single_kernel<kTopkThreads, kSingleMax>), dim3(a.N), dim3(kTopkThreads), 0, stream,
                       a, k, out_idx, out_score);
  return hipGetLastError();
}

// Large selections, step 2: keep every key >= the query's threshold T (the minimum of its full
// scoring blocks' thresholds, or 0 when there is no bound) as a candidate (key, id). Block =
// (query, chunk of 8192 entries); the chunk's candidates go to the start of its own 8192 slots
// and their number to its count (plain stores: no counter shared between blocks).
constexpr int kFilterChunk = 8192;
constexpr int kMaxFilterChunks = (int)(kMaxTopkVisible / kFilterChunk);
__global__ __launch_bounds__(kScoreThreads) void topk_filter_kernel(IndexArgs a, int blk_entries,
                                                                    uint32_t* ckey, int32_t* cid,
                                                                    unsigned* ccount, int ccs,
                                                                    int64_t cstride) {
  __shared__ uint32_t wmin[kScoreThreads / 64];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lo = blockIdx.y * kFilterChunk;          // < nv_cap: the grid covers nv_cap
  // The block bounds and the chunk's scores are requested before the query's position is known
  // (indices clamped to the plan's capacity, entries past the query's visible ones masked
  // later), so that the position's load and theirs overlap. The output pointers are formed here
  // too, so that their kernel arguments are read at the start, not after the barriers where
  // they are first used (a scalar load there would cost a memory latency of its own).
  constexpr int kThrRegs = 8;                        // block bounds held per thread
  constexpr int kPer = kFilterChunk / kScoreThreads;
  const uint32_t* thr = a.blk_thr + (int64_t)t * a.thr_stride;
  uint32_t v[kThrRegs];
#pragma unroll
  for (int u = 0; u < kThrRegs; ++u) v[u] = thr[min(u * kScoreThreads + (int)threadIdx.x, a.thr_stride - 1)];
  const float* sc = a.scores + (int64_t)t * a.score_stride;
  const int cap = min(lo + kFilterChunk, a.nv_cap) - 1;
  // (loads at clamped indices, results selected after: a conditional load would be a branch,
  // and every branch merge a wait for that load alone)
  uint32_t key[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) key[j] = __float_as_uint(sc[min(lo + j * kScoreThreads + (int)threadIdx.x, cap)]);
  uint32_t* ck0 = ckey + (int64_t)t * cstride + lo;   // slots < hi - lo: inside the query's range
  int32_t* ci0 = cid + (int64_t)t * cstride + lo;
  unsigned* cnt0 = ccount + (int64_t)t * ccs + blockIdx.y;
  asm volatile("" : "+s"(ck0), "+s"(ci0), "+s"(cnt0));
  // global pointers again (through the asm the compiler no longer knows the address space, and
  // a generic store is a flat store, whose waits also cover LDS operations)
  auto* ck = (__attribute__((address_space(1))) uint32_t*)ck0;
  auto* ci = (__attribute__((address_space(1))) int32_t*)ci0;
  auto* cnt_out = (__attribute__((address_space(1))) unsigned*)cnt0;
  int seq, nv;
  query_of(a, t, seq, nv);
  if (nv <= a.topk || lo >= nv) return;              // short context: the select fills it directly
  const int full = nv / blk_entries;
  const int kb = full > 0 ? bound_kb(a.topk, full) : kMaxKb + 1;
  const bool few_bounds = kb <= kMaxKb && full <= kThrRegs * kScoreThreads;
  const int hi = min(nv, lo + kFilterChunk);
  uint32_t T = 0u;
  if (few_bounds) {
    // T = the lower edge of the highest of 256 equal bins over [min b, max b] whose suffix
    // holds at least J = ceil(k / kb) bounds: at least J bounds are >= T (valid), and T is
    // within one bin of the J-th largest bound
    __shared__ uint32_t wmax[kScoreThreads / 64], hist[256], tsel;
    const uint32_t J = (uint32_t)((a.topk + kb - 1) / kb);
    uint32_t blo = ~0u, bhi = 0u;
#pragma unroll
    for (int u = 0; u < kThrRegs; ++u)
      if (u * kScoreThreads + (int)threadIdx.x < full) {
        blo = min(blo, v[u]);
        bhi = max(bhi, v[u]);
      }
    blo = ~wave_max_u32(~blo);
    bhi = wave_max_u32(bhi);
    if (lane == 0) {
      wmin[wave] = blo;
      wmax[wave] = bhi;
    }
    static_assert(kScoreThreads == 256, "one histogram bin per thread");
    hist[threadIdx.x] = 0u;
    __syncthreads();
    blo = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
    bhi = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    const uint32_t width = (bhi - blo) / 256u + 1u;
#pragma unroll
    for (int u = 0; u < kThrRegs; ++u)
      if (u * kScoreThreads + (int)threadIdx.x < full) atomicAdd(&hist[(v[u] - blo) / width], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane holds bins 4 lane .. 4 lane + 3; incl = bounds in bins >= 4 lane (suffix sum)
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t tot = c0 + c1 + c2 + c3;
      uint32_t incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += o;
      }
      const uint32_t above = incl - tot;               // bounds in bins above this lane's
      if (above < J && J <= incl) {                    // exactly one lane: incl(0) = full >= J
        uint32_t sfx = above + c3;
        int b = 4 * lane + 3;
        if (sfx < J) {
          sfx += c2;
          b = 4 * lane + 2;
          if (sfx < J) {
            sfx += c1;
            b = sfx < J ? 4 * lane : 4 * lane + 1;
          }
        }
        tsel = blo + (uint32_t)b * width;
      }
    }
    __syncthreads();
    T = tsel;
  } else if (kb <= kMaxKb) {
    // many bounds: their minimum (valid for any kb >= ceil(k / full))
    uint32_t m = ~0u;
    for (int i0 = 0; i0 < full; i0 += 8 * kScoreThreads) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = thr[min(i0 + u * kScoreThreads + (int)threadIdx.x, full - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * kScoreThreads + (int)threadIdx.x < full) m = min(m, v[u]);
    }
    m = ~wave_max_u32(~m);
    if (lane == 0) wmin[wave] = m;
    __syncthreads();
    T = min(min(wmin[0], wmin[1]), min(wmin[2], wmin[3]));
  }
#pragma unroll
  for (int j = 0; j < kPer; ++j) key[j] = f32_order_key(__uint_as_float(key[j]));
  // keep flags of the block's entries (entry lo + 256 j + tid for j < kPer) as one bit mask per
  // thread; slots in thread order, then j: the thread's prefix within its wave (DPP scan) plus
  // the earlier waves' counts from LDS
  __shared__ unsigned wcnt[kScoreThreads / 64];
  uint32_t keep = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    keep |= (lo + j * kScoreThreads + (int)threadIdx.x < hi && key[j] >= T ? 1u : 0u) << j;
  const unsigned mine = (unsigned)__popc(keep);
  const unsigned incl = wave_incl_scan_u32(mine);
  if (lane == 63) wcnt[wave] = incl;                 // the wave's kept entries
  __syncthreads();
  unsigned slot = incl - mine;
#pragma unroll
  for (int w = 0; w < kScoreThreads / 64; ++w) slot += w < wave ? wcnt[w] : 0u;
  if (threadIdx.x == 0) *cnt_out = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if ((keep >> j) & 1u) {
      ck[slot] = key[j];
      ci[slot] = lo + j * kScoreThreads + threadIdx.x;
      ++slot;
    }
  }
}

// Large selections, step 3: the top-k of a query's candidates, in one of two layouts:
//  * filter (cand_mode 0): chunk c of the query's 8192-entry chunks has ccount[t * ccs + c]
//    candidates at slots c * 8192 + 0, 1, ...; at most 32 chunks of at most 256 candidates each
//    (the usual case) are loaded with their counts in one go, slot u of a thread holding slot
//    (u % 4) * 64 + lane of chunk 2 wave + u / 4, and selected in registers; otherwise the
//    chunks' offsets are summed in LDS and candidate i is found by a search over them;
//  * listed blocks (cand_mode 1): ccount[t] candidates at slots 0, 1, ... .
// With more candidates than fit the register or LDS selections, keys (and ids) are read from
// memory where each pass needs them.
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(IndexArgs a, int k,
                                                                   const uint32_t* ckey,
                                                                   const int32_t* cid,
                                                                   const unsigned* ccount, int ccs,
                                                                   int64_t cstride,
                                                                   int32_t* out_idx,
                                                                   float* out_score,
                                                                   int cand_mode) {
  __shared__ SelShared sh;
  __shared__ uint32_t kl[kSingleMax];
  __shared__ unsigned coff[kMaxFilterChunks + 1];
  __shared__ unsigned wfit[kTopkThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* ck = ckey + (int64_t)t * cstride;
  const int32_t* ci = cid + (int64_t)t * cstride;
  // filter layout: the first 256 slots of chunks 2 wave and 2 wave + 1 and the two counts are
  // requested before the query's position is known (indices clamped to the plan's capacity;
  // chunks past the query's are dropped once it is)
  constexpr int kSpecPT = 8, kSpecChunk = 256;
  static_assert(kSpecPT * kTopkThreads == 32 * kSpecChunk, "two chunks per wave");
  uint32_t sk[kSpecPT], sid[kSpecPT];
  unsigned n0 = 0u, n1 = 0u;
  const unsigned* cc = ccount + (int64_t)t * ccs;
  if (!cand_mode) {
#pragma unroll
    for (int u = 0; u < kSpecPT; ++u) {
      const int64_t i = min((int64_t)(2 * wave + u / 4) * kFilterChunk + (u % 4) * 64 + lane, cstride - 1);
      sk[u] = ck[i];
      sid[u] = (uint32_t)ci[i];
    }
    n0 = cc[min(2 * wave, ccs - 1)];
    n1 = cc[min(2 * wave + 1, ccs - 1)];
  }
  int seq, nv;
  query_of(a, t, seq, nv);
  int32_t* oi = out_idx + (int64_t)t * k;
  float* os = out_score ? out_score + (int64_t)t * k : nullptr;
  auto emit = [&](unsigned slot, int id, uint32_t key) {
    if (slot < (unsigned)k) {
      oi[slot] = id;
      if (os) os[slot] = order_key_f32(key);
    }
  };
  int n;                                             // candidates
  int nch = 0;                                       // filter: chunks (offsets in coff)
  if (cand_mode) {                                   // the listed blocks' entries are the candidates
    n = (int)ccount[t];
    if (n <= k) {
      for (int j = tid; j < k; j += kTopkThreads) {
        oi[j] = j < n ? ci[j] : -1;
        if (os) os[j] = j < n ? order_key_f32(ck[j]) : 0.f;
      }
      return;
    }
  } else {
    if (nv <= k) {
      const float* sc = a.scores + (int64_t)t * a.score_stride;
      for (int j = tid; j < k; j += kTopkThreads) {
        oi[j] = j < nv ? j : -1;
        if (os) os[j] = j < nv ? sc[j] : 0.f;
      }
      return;
    }
    nch = (nv + kFilterChunk - 1) / kFilterChunk;
    n0 = 2 * wave < nch ? n0 : 0u;
    n1 = 2 * wave + 1 < nch ? n1 : 0u;
    if (lane == 0) wfit[wave] = n0 <= kSpecChunk && n1 <= kSpecChunk ? 1u : 0u;
    sel_reset<kTopkThreads>(sh);
    __syncthreads();
    bool fits = nch <= 32;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) fits = fits && wfit[w] != 0u;
    if (fits) {
      uint32_t vmask = 0u;
#pragma unroll
      for (int u = 0; u < kSpecPT; ++u) vmask |= ((u % 4) * 64 + lane < (int)(u < 4 ? n0 : n1) ? 1u : 0u) << u;
      const unsigned n_sel = reg_topk<kTopkThreads, kSpecPT>(
          sh, sk, vmask, (unsigned)k, false, [&](int u) { return (int)sid[u]; },
          [&](unsigned pos, int u, uint32_t key) { emit(pos, (int)sid[u], key); });
      for (int j = (int)n_sel + tid; j < k; j += kTopkThreads) oi[j] = -1;   // (fewer than k: not expected)
      return;
    }
    // chunk offsets: exclusive prefix sum of the counts (nch <= kMaxFilterChunks <= threads)
    static_assert(kMaxFilterChunks <= kTopkThreads, "one chunk count per thread");
    const unsigned c = tid < nch ? cc[tid] : 0u;
    const unsigned incl = wave_incl_scan_u32(c);
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    unsigned before = incl - c, all = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / 64; ++w) {
      before += w < wave ? sh.wsum[w] : 0u;
      all += sh.wsum[w];
    }
    if (tid < nch) coff[tid] = before;
    if (tid == 0) coff[nch] = all;
    n = (int)all;
    __syncthreads();
    if (n <= k) {                                    // (not expected: T is at most the k-th key)
      for (int j = tid; j < k; j += kTopkThreads) {
        int id = -1;
        uint32_t key = 0u;
        if (j < n) {
          int lo = 0, hi = nch;
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (coff[mid] <= (unsigned)j) lo = mid;
            else hi = mid;
          }
          const int64_t sl = (int64_t)lo * kFilterChunk + (j - (int)coff[lo]);
          id = ci[sl];
          key = ck[sl];
        }
        oi[j] = id;
        if (os) os[j] = j < n ? order_key_f32(key) : 0.f;
      }
      return;
    }
  }
  // slot of candidate i: i itself (listed blocks) or its place in its chunk (filter)
  auto slot_of = [&](int i) -> int64_t {
    if (cand_mode) return i;
    int lo = 0, hi = nch;                            // coff[lo] <= i < coff[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (coff[mid] <= (unsigned)i) lo = mid;
      else hi = mid;
    }
    return (int64_t)lo * kFilterChunk + (i - (int)coff[lo]);
  };
  if (n <= kSingleMax / 2) {
    // keys and ids in LDS
    uint32_t* kid = kl + kSingleMax / 2;
    for (int i = tid; i < n; i += kTopkThreads) {
      const int64_t sl = slot_of(i);
      kl[i] = ck[sl];
      kid[i] = (uint32_t)ci[sl];
    }
    sel_reset<kTopkThreads>(sh);
    __syncthreads();
    block_topk<kTopkThreads>(
        sh, n, k, [&](int i, uint32_t& key) { key = kl[i]; return true; }, [&](int i) { return (int)kid[i]; },
        emit);
    return;
  }
  if (n <= kSingleMax) {
    for (int i = tid; i < n; i += kTopkThreads) kl[i] = ck[slot_of(i)];
    sel_reset<kTopkThreads>(sh);
    __syncthreads();
    block_topk<kTopkThreads>(
        sh, n, k, [&](int i, uint32_t& key) { key = kl[i]; return true; }, [&](int i) { return ci[slot_of(i)]; },
        emit);
    return;
  }
  sel_reset<kTopkThreads>(sh);
  __syncthreads();
  block_topk<kTopkThreads>(
      sh, n, k, [&](int i, uint32_t& key) { key = ck[slot_of(i)]; return true; },
      [&](int i) { return ci[slot_of(i)]; }, emit);
}

// ---------------------------------------------------------------- two-level candidate filtering
// Consumer: the entries of a query's listed blocks (block j = entries j*cb .. j*cb+cb-1, the
// visible ones) become its selection candidates (key, id), appended through the per-query
// counter that the scoring launch zeroed. Block = (query, listed block).
__global__ __launch_bounds__(kScoreThreads) void cand_gather_kernel(IndexArgs a, const int32_t* cand, int n_cand,
                                                                    int cb, uint32_t* ckey, int32_t* cid,
                                                                    unsigned* ccount, int64_t cstride) {
  __shared__ unsigned wcnt[kScoreThreads / 64], wbase[kScoreThreads / 64];
  const int t = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int seq, nv;
  query_of(a, t, seq, nv);
  const int blk = cand[(int64_t)t * n_cand + blockIdx.y];
  if (blk < 0 || (int64_t)blk * cb >= nv) return;
  const int lo = blk * cb, hi = (int)min((int64_t)nv, (int64_t)lo + cb);
  const float* sc = a.scores + (int64_t)t * a.score_stride;
  for (int c0 = lo; c0 < hi; c0 += kScoreThreads) {
    const int i = c0 + threadIdx.x;
    const bool in = i < hi;
    const uint64_t bm = __ballot(in);
    if (lane == 0) wcnt[wave] = (unsigned)__popcll(bm);
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned tot = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
      unsigned run = atomicAdd(ccount + t, tot);
      for (int w = 0; w < kScoreThreads / 64; ++w) {
        wbase[w] = run;
        run += wcnt[w];
      }
    }
    __syncthreads();
    if (in) {
      const unsigned sl = wbase[wave] + (unsigned)__popcll(bm & ((1ull << lane) - 1));
      ckey[(int64_t)t * cstride + sl] = f32_order_key(sc[i]);
      cid[(int64_t)t * cstride + sl] = i;
    }
    __syncthreads();                                 // wcnt / wbase are reused
  }
}

// Source: block b's score is the max of its visible entries' scores. Thread = (query, block).
__global__ __launch_bounds__(kScoreThreads) void block_max_kernel(IndexArgs a, int cb, float* bmax,
                                                                  int64_t bstride) {
  const int t = blockIdx.x;
  int seq, nv;
  query_of(a, t, seq, nv);
  const int b = blockIdx.y * kScoreThreads + threadIdx.x;
  if ((int64_t)b * cb >= nv) return;
  const float* sc = a.scores + (int64_t)t * a.score_stride + (int64_t)b * cb;
  const int n = (int)min((int64_t)cb, (int64_t)nv - (int64_t)b * cb);
  float m = kNegInf;
  for (int i = 0; i < n; ++i) m = fmaxf(m, sc[i]);
  bmax[(int64_t)t * bstride + b] = m;
}

}  // namespace

TopkPlan topk_plan(int N, int max_pos, int m, int topk) {
  TopkPlan p{};
  const int64_t nv = (int64_t)(max_pos + 1) / m;
  const int64_t stride = std::max<int64_t>(64, (nv + 63) / 64 * 64);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  p.score_bytes = (size_t)N * stride * sizeof(float);
  p.large = nv > kSingleMax;
  size_t off = up(p.score_bytes);
  if (p.large) {
    p.thr_stride = (int)((nv + 255) / 256);          // the smallest scoring block is 256 entries
    p.thr_off = off;
    off += up((size_t)N * p.thr_stride * sizeof(uint32_t));
    p.cand_off = off;                                // keys [N, stride] then ids [N, stride]
    off += up((size_t)N * stride * sizeof(uint32_t)) + up((size_t)N * stride * sizeof(int32_t));
    p.cnt_stride = (int)((nv + kFilterChunk - 1) / kFilterChunk);   // per-chunk candidate counts
    p.cnt_off = off;
    off += up((size_t)N * p.cnt_stride * sizeof(unsigned));
  }
  p.ws_bytes = off;
  return p;
}

hipError_t launch_index_scores(const IndexArgs& a, int fmt, hipStream_t stream) {
  if (a.N == 0 || a.nv_cap == 0) return hipSuccess;
  const int MT = (a.H_I + 15) / 16;
  if (fmt == HCS_FMT_FP8IX) {
    dim3 grid(a.N, (a.nv_cap + 511) / 512);
    switch (MT) {
      case 1: hipLaunchKernelGGL((index_score_fp8_kernel<1>), grid, dim3(kScoreThreads), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((index_score_fp8_kernel<2>), grid, dim3(kScoreThreads), 0, stream, a); break;
      case 3: hipLaunchKernelGGL((index_score_fp8_kernel<3>), grid, dim3(kScoreThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL((index_score_fp8_kernel<4>), grid, dim3(kScoreThreads), 0, stream, a); break;
    }
    return hipGetLastError();
  }
  if (fmt == HCS_FMT_MXFP4) {
    const int per_wg = kMx4BlockEntries;
    dim3 grid(a.N, (a.nv_cap + per_wg - 1) / per_wg);
    switch (MT) {
      case 1: hipLaunchKernelGGL((index_score_mxfp4_kernel<1>), grid, dim3(kScoreThreads), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((index_score_mxfp4_kernel<2>), grid, dim3(kScoreThreads), 0, stream, a); break;
      case 3: hipLaunchKernelGGL((index_score_mxfp4_kernel<3>), grid, dim3(kScoreThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL((index_score_mxfp4_kernel<4>), grid, dim3(kScoreThreads), 0, stream, a); break;
    }
    return hipGetLastError();
  }
  if (!a.q_seq && !a.blk_thr && a.d_I == 128 && a.H_I % 4 == 0 && a.N >= kChunkMinQueries) {
    dim3 grid((a.nv_cap + kChunkEntries - 1) / kChunkEntries, (a.N + kChunkQueries - 1) / kChunkQueries);
    switch (MT) {
      case 1: hipLaunchKernelGGL((index_score_chunk_kernel<1>), grid, dim3(kChunkThreads), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((index_score_chunk_kernel<2>), grid, dim3(kChunkThreads), 0, stream, a); break;
      case 3: hipLaunchKernelGGL((index_score_chunk_kernel<3>), grid, dim3(kChunkThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL((index_score_chunk_kernel<4>), grid, dim3(kChunkThreads), 0, stream, a); break;
    }
    return hipGetLastError();
  }
  const int per_wg = 256;
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

hipError_t launch_index_scores_compress(const IndexArgs& a, const CompressArgs& c, int max_new, int fmt,
                                        hipStream_t stream) {
  const int MT = (a.H_I + 15) / 16;
  if (a.N == 0 || a.nv_cap == 0) return launch_compress(c, max_new, stream);
  if (c.B == 0) return launch_index_scores(a, fmt, stream);
  if (fmt == HCS_FMT_MXFP4) {
    const dim3 cg = compress_grid(c, max_new);
    const int chunks = (a.nv_cap + kMx4BlockEntries - 1) / kMx4BlockEntries;
    const int64_t blocks = (int64_t)cg.x * cg.y * cg.z + (int64_t)a.N * chunks;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (MT) {
      case 1: hipLaunchKernelGGL((index_score_mxfp4_compress_kernel<1>), grid, dim3(kScoreThreads), 0, stream, a, c, chunks, (int)cg.y, (int)cg.z); break;
      case 2: hipLaunchKernelGGL((index_score_mxfp4_compress_kernel<2>), grid, dim3(kScoreThreads), 0, stream, a, c, chunks, (int)cg.y, (int)cg.z); break;
      case 3: hipLaunchKernelGGL((index_score_mxfp4_compress_kernel<3>), grid, dim3(kScoreThreads), 0, stream, a, c, chunks, (int)cg.y, (int)cg.z); break;
      default: hipLaunchKernelGGL((index_score_mxfp4_compress_kernel<4>), grid, dim3(kScoreThreads), 0, stream, a, c, chunks, (int)cg.y, (int)cg.z); break;
    }
    return hipGetLastError();
  }
  const dim3 cg = compress_grid(c, max_new);
  const int chunks = (a.nv_cap + 255) / 256;
  const int64_t blocks = (int64_t)cg.x * cg.y * cg.z + (int64_t)a.N * chunks;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
#define HCS_SC_CASE(DI_, MT_)                                                                       \
  if (a.d_I == DI_ && MT == MT_) {                                                                  \
    hipLaunchKernelGGL((index_score_compress_kernel<DI_, MT_>), grid, dim3(kScoreThreads), 0, stream, a, c, \
                       chunks, (int)cg.y, (int)cg.z);                                                 \
    return hipGetLastError();                                                                       \
  }
  HCS_SC_CASE(32, 1) HCS_SC_CASE(32, 2) HCS_SC_CASE(32, 3) HCS_SC_CASE(32, 4)
  HCS_SC_CASE(64, 1) HCS_SC_CASE(64, 2) HCS_SC_CASE(64, 3) HCS_SC_CASE(64, 4)
  HCS_SC_CASE(128, 1) HCS_SC_CASE(128, 2) HCS_SC_CASE(128, 3) HCS_SC_CASE(128, 4)
#undef HCS_SC_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const IndexArgs& a, const TopkPlan& plan, int topk, int32_t* out_idx,
                       float* out_score, uint8_t* ws, int blk_entries, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  if (!plan.large) {
    return launch_topk_single(a, a.nv_cap, topk, out_idx, out_score, stream);
  }
  const int64_t cstride = a.score_stride;
  uint32_t* ckey = reinterpret_cast<uint32_t*>(ws + plan.cand_off);
  int32_t* cid = reinterpret_cast<int32_t*>(ws + plan.cand_off + ((size_t)a.N * cstride * 4 + 255) / 256 * 256);
  unsigned* cnt = reinterpret_cast<unsigned*>(ws + plan.cnt_off);
  if (plan.cnt_stride > kMaxFilterChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_filter_kernel, dim3(a.N, (a.nv_cap + kFilterChunk - 1) / kFilterChunk),
                     dim3(kScoreThreads), 0, stream, a, blk_entries, ckey, cid, cnt, plan.cnt_stride, cstride);
  hipLaunchKernelGGL(topk_select_kernel, dim3(a.N), dim3(kTopkThreads), 0, stream, a, topk, ckey, cid,
                     cnt, plan.cnt_stride, cstride, out_idx, out_score, 0);
  return hipGetLastError();
}

CandPlan cand_plan(const TopkPlan& base, int N, int nv_cap, int cand_block, int n_cand) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  CandPlan c{};
  c.cstride = ((int64_t)n_cand * cand_block + 63) / 64 * 64;
  c.bstride = std::max<int64_t>(64, ((int64_t)nv_cap / cand_block + 1 + 63) / 64 * 64);
  size_t off = base.ws_bytes;
  c.ckey_off = off;
  off += up((size_t)N * c.cstride * sizeof(uint32_t));
  c.cid_off = off;
  off += up((size_t)N * c.cstride * sizeof(int32_t));
  c.cnt_off = off;
  off += up((size_t)N * sizeof(unsigned));
  c.bmax_off = off;
  off += up((size_t)N * c.bstride * sizeof(float));
  c.ws_bytes = off;
  return c;
}

hipError_t launch_topk_in_blocks(const IndexArgs& a, const CandPlan& cp, uint8_t* ws, const int32_t* cand_in,
                                 int n_cand, int cand_block, int topk, int32_t* out_idx, float* out_score,
                                 hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  uint32_t* ckey = reinterpret_cast<uint32_t*>(ws + cp.ckey_off);
  int32_t* cid = reinterpret_cast<int32_t*>(ws + cp.cid_off);
  unsigned* cnt = reinterpret_cast<unsigned*>(ws + cp.cnt_off);
  hipLaunchKernelGGL(cand_gather_kernel, dim3(a.N, n_cand), dim3(kScoreThreads), 0, stream, a, cand_in, n_cand,
                     cand_block, ckey, cid, cnt, cp.cstride);
  hipLaunchKernelGGL(topk_select_kernel, dim3(a.N), dim3(kTopkThreads), 0, stream, a, topk, ckey, cid, cnt, 1,
                     cp.cstride, out_idx, out_score, 1);
  return hipGetLastError();
}

hipError_t launch_candidate_blocks(const IndexArgs& a, const CandPlan& cp, uint8_t* ws, int cand_block,
                                   int n_cand, int32_t* cand_out, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  float* bmax = reinterpret_cast<float*>(ws + cp.bmax_off);
  const int nb_cap = (a.nv_cap + cand_block - 1) / cand_block;
  hipLaunchKernelGGL(block_max_kernel, dim3(a.N, (nb_cap + kScoreThreads - 1) / kScoreThreads), dim3(kScoreThreads),
                     0, stream, a, cand_block, bmax, cp.bstride);
  IndexArgs b = a;                                   // the selection over block scores
  b.scores = bmax;
  b.score_stride = cp.bstride;
  b.nv_div = cand_block;
  b.blk_thr = nullptr;
  b.cand_count = nullptr;
  return launch_topk_single(b, nb_cap, n_cand, cand_out, static_cast<float*>(nullptr), stream);
}

}  // namespace hcs
