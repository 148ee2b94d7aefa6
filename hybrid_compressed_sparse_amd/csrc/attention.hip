// Sparse MLA (single shared KV head) attention for gfx950.
//
// What it computes: "DeepSeek V4 Attention: Code Reading Map", section "Phase 3: forward_mqa()":
// every query head attends over the query's sliding-window rows plus its selected (CSA) or all
// visible (HCA) compressed entries; K and V are the same shared row.
//
// Building blocks shared by both kernels:
//   * a workgroup first resolves the physical row of every logical row it will read (window
//     position or compressed id -> page table -> page, slot) into an LDS table, with all
//     loads issued together and no branches, so each later row load is a single independent
//     16-byte gather; rows that do not take part read a zero row;
//   * the math on a 32-row tile for 16 heads, per wave: S^T = K Q^T with
//     v_mfma_f32_16x16x32_bf16 (rows on M, heads on N, q in registers as the B operand), whose
//     accumulator layout is already the B-operand layout of P^T, then O^T += V^T P^T with V^T
//     read from the same LDS rows by ds_read_b64_tr_b16 (16-bit transpose across each 16-lane
//     group); online softmax in base 2 with one head per lane (lane % 16);
//   * fp8_ds rows are dequantised on their way into LDS (e4m3 * 2^(scale-127) is exact in bf16).
//
// Decode kernel (few queries): a workgroup is (query, split of its rows, 16 heads). Each of
// its 4 waves walks its own 32-row sub-tiles (wave w takes sub-tiles w, w+4, ...) with a
// private LDS buffer and a one-sub-tile register prefetch, so waves never wait for each other
// inside the loop and a CU keeps 4 x 32 KiB of gathers in flight. The waves' softmax states
// merge through LDS at the end. The 4 head groups of a query run on the same XCD (blocks are
// dispatched round-robin over the 8 XCDs, and the block index is mapped so that all blocks of
// a query share one), so a row fetched from HBM by one of them is an L2 hit for the others,
// and split partials are merged by the last block to finish, through that XCD's L2.
//
// Prefill kernel (many queries): a workgroup is one query and 64 heads; wave w owns heads
// 16w..16w+15 and all 4 waves share each 32-row tile, staged cooperatively into a
// double-buffered LDS ring, so each gathered row is read from L2/HBM once for all heads.
#include "kernels.h"

namespace hcs {

// A zero row: rows that take part in nothing load from here, so loads never branch.
__device__ __attribute__((aligned(64))) uint8_t g_zero_row[1024];

namespace {

constexpr int kTile = 32;
constexpr int kThreads = 256;
constexpr int kMaxRowsWG = 2304;            // rows in one workgroup's address table
constexpr uint32_t kNoRow = 0xFFFFFFFFu;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 __attribute__((address_space(3)))*)(p));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, float sc) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return (__float_as_uint(f.x * sc) >> 16) | (__float_as_uint(f.y * sc) & 0xffff0000u);
}

// The rows a query attends: window positions lo..lo+n_swa-1, then n_comp compressed slots.
struct QueryRows {
  int seq, pos, lo, n_swa, nv, n_comp, R;
};

__device__ __forceinline__ QueryRows query_rows(const AttnArgs& a, int t) {
  QueryRows q;
  if (a.q_seq) {
    q.seq = __ldg(a.q_seq + t);
    q.pos = min(__ldg(a.q_pos + t), a.pos_cap);
  } else {
    q.seq = a.seq_const;
    q.pos = a.p0 + t;
  }
  q.lo = max(0, q.pos - a.window + 1);
  q.n_swa = a.window > 0 ? q.pos - q.lo + 1 : 0;
  q.nv = min((q.pos + 1) / a.m, a.nv_cap);
  q.n_comp = a.topk_idx ? a.topk : q.nv;
  q.R = q.n_swa + q.n_comp;
  return q;
}

// Fill rowtab[0 .. n) with the entries of logical rows r0 .. r0+n-1 (all threads of the block),
// and rowtab[n .. n rounded up to `pad`) with kNoRow.
// Every thread resolves up to kRowsPerThread rows; all id loads are issued, then all page-table
// loads, so the table costs two memory latencies whatever its length.
constexpr int kRowsPerThread = (kMaxRowsWG + kThreads - 1) / kThreads;

__device__ __forceinline__ void fill_rowtab(const AttnArgs& a, int t, const QueryRows& q, int r0,
                                            int n, uint32_t* rowtab, int pad = kTile) {
  int id[kRowsPerThread];
  const int last = max(q.R - 1, 0);
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int gr = min(r0 + (int)threadIdx.x + i * kThreads, last);
    const int j = min(max(gr - q.n_swa, 0), max(q.n_comp - 1, 0));
    id[i] = a.topk_idx ? __ldg(a.topk_idx + (int64_t)t * a.topk + j) : j;
  }
  int pg[kRowsPerThread], row[kRowsPerThread];
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int gr = min(r0 + (int)threadIdx.x + i * kThreads, last);
    const bool is_swa = gr < q.n_swa;
    const bool ok_id = is_swa || (id[i] >= 0 && id[i] < q.nv);
    row[i] = ok_id ? (is_swa ? q.lo + gr : id[i]) : -1;
    const int rc = max(row[i], 0);
    const int32_t* pt = is_swa ? a.swa.pt : a.comp.pt;
    const int stride = is_swa ? a.swa.pt_stride : a.comp.pt_stride;
    pg[i] = __ldg(pt + (int64_t)q.seq * stride + (rc >> 6));
  }
  const int n32 = min((n + pad - 1) / pad * pad, kMaxRowsWG);   // padded with kNoRow to whole tiles
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int li = (int)threadIdx.x + i * kThreads;
    const int gr = r0 + li;
    if (li < n32) {
      const bool is_swa = gr < q.n_swa;
      const int npages = is_swa ? a.swa.num_pages : a.comp.num_pages;
      const bool ok = li < n && gr < q.R && row[i] >= 0 && pg[i] >= 0 && pg[i] < npages;
      rowtab[li] = ok ? ((is_swa ? 0u : 0x80000000u) | (uint32_t)(pg[i] * 64 + (row[i] & 63))) : kNoRow;
    }
  }
}

// ---------------------------------------------------------------- row staging
// LDS tiles hold rows of D bf16 without padding; the 16-byte chunk c of row r sits at chunk
// c ^ swz(r), a 4-bit XOR that depends on r mod 16. gfx950's LDS serves a 128-bit read for 16
// lanes (256 bytes) per cycle, so a reader is free of bank conflicts when the 16-byte chunks its
// 16 lanes touch fall on 16 distinct chunk positions mod 16 (and on 8 distinct positions mod 8
// for a 32-bank view). Each kernel reads its tile in its own pattern, hence two swizzles:
//   decode: K reads rows 16w + l (l = 0..15, one chunk); V^T reads rows 8g + j (+4), chunks
//           2c, 2c+1 for two groups g at a time. swz_dec gives distinct positions in both views.
//   prefill: K reads rows l = 0..15; V^T reads rows 4g + j (+16) for g pairs (0,1)/(2,3).
__device__ __forceinline__ int swz_dec(int r) {
  return ((r & 3) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 3);
}
__device__ __forceinline__ int swz_pre(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// Each variant loads one 32-row tile's worth of 16-byte pieces per lane into registers and
// later writes them (dequantised to bf16 for fp8_ds) into the LDS tile.
template <int D, int FMT>
struct Stage {
  static constexpr int RS = D * 2;                           // LDS row stride
  static constexpr int PB = FMT == HCS_FMT_FP8DS ? kFp8PageBytes : kPageRows * D * 2;
  // rows per load instruction over a wave: bf16 D=512 and fp8ds: 1; bf16 D=128: 4
  static constexpr int RPL = (FMT == HCS_FMT_BF16 && D == 128) ? 4 : 1;
  static constexpr int NLD_TILE = kTile / RPL;               // loads for a whole 32-row tile

  // Row within the load and 16-byte chunk index of this lane.
  __device__ static __forceinline__ int lane_row(int lane) { return RPL == 1 ? 0 : lane >> 4; }
  __device__ static __forceinline__ int lane_chunk(int lane) { return RPL == 1 ? lane : lane & 15; }

  // Issue the load of this lane's piece of the row with table entry `e` (wave-uniform when
  // RPL == 1, so the row address is computed once in scalar registers).
  __device__ static __forceinline__ void load(const AttnArgs& a, uint32_t e, int lane, i32x4& v,
                                              float& sc) {
    sc = 1.f;
    if constexpr (FMT == HCS_FMT_FP8DS) {
      e = (uint32_t)__builtin_amdgcn_readfirstlane((int)e);
      const bool ok = e != kNoRow;
      const uint32_t ridx = e & 0x7fffffffu;
      const uint8_t* page = ok ? ((e >> 31) ? a.comp.base : a.swa.base) + (size_t)(ridx >> 6) * PB
                               : g_zero_row;
      const int slot = ok ? (int)(ridx & 63) : 0;
      // lanes 0..27: 16 latent codes, lanes 28..35: 8 rope values, others: nothing useful
      const int off = lane < 28 ? kFp8PageCodes + slot * kFp8Latent + lane * 16
                                : (lane < 36 ? kFp8PageRope + slot * (kFp8Rope * 2) + (lane - 28) * 16
                                             : kFp8PageCodes + slot * kFp8Latent);
      v = ok ? *(const i32x4*)(page + off) : *(const i32x4*)(g_zero_row + (lane & 31) * 16);
      const int se = ok ? page[kFp8PageScales + slot * 8 + (min(lane, 27) >> 2)] : 0;
      sc = ok && lane < 28 ? __builtin_ldexpf(1.f, se - 127) : 1.f;
    } else if constexpr (RPL == 1) {
      e = (uint32_t)__builtin_amdgcn_readfirstlane((int)e);
      const uint8_t* rb = e != kNoRow
                              ? ((e >> 31) ? a.comp.base : a.swa.base) + (size_t)(e & 0x7fffffffu) * (D * 2)
                              : g_zero_row;
      v = *(const i32x4*)(rb + lane * 16);
    } else {
      const int chunk = lane_chunk(lane);
      const bool ok = e != kNoRow;
      const uint8_t* base = (e >> 31) ? a.comp.base : a.swa.base;
      const uint8_t* p = ok ? base + (size_t)(e & 0x7fffffffu) * (D * 2) + chunk * 16 : g_zero_row + chunk * 16;
      v = *(const i32x4*)p;
    }
  }

  // Write this lane's piece of row `r` (tile-local) into the LDS tile.
  __device__ static __forceinline__ void store(uint8_t* tile, int r, int sw, int lane,
                                               const i32x4& v, float sc) {
    const int chunk = lane_chunk(lane);
    uint8_t* row = tile + r * RS;
    if constexpr (FMT == HCS_FMT_FP8DS) {
      if (chunk < 28) {
        i32x4 lo4, hi4;
        lo4.x = e4m3x2_to_bf16x2<false>(v.x, sc);
        lo4.y = e4m3x2_to_bf16x2<true>(v.x, sc);
        lo4.z = e4m3x2_to_bf16x2<false>(v.y, sc);
        lo4.w = e4m3x2_to_bf16x2<true>(v.y, sc);
        hi4.x = e4m3x2_to_bf16x2<false>(v.z, sc);
        hi4.y = e4m3x2_to_bf16x2<true>(v.z, sc);
        hi4.z = e4m3x2_to_bf16x2<false>(v.w, sc);
        hi4.w = e4m3x2_to_bf16x2<true>(v.w, sc);
        *(i32x4*)(row + ((2 * chunk) ^ sw) * 16) = lo4;
        *(i32x4*)(row + ((2 * chunk + 1) ^ sw) * 16) = hi4;
      } else if (chunk < 36) {
        *(i32x4*)(row + ((56 + chunk - 28) ^ sw) * 16) = v;
      }
    } else {
      *(i32x4*)(row + (chunk ^ sw) * 16) = v;
    }
  }
};

// ---------------------------------------------------------------- per-wave tile math
// One wave, 16 heads (q in registers), one LDS tile of 32 rows; `valid` bit r = row r takes
// part. Keeps a reference max m_ref (base 2) per head: probabilities are exp2(x - m_ref), and
// the accumulators are rescaled only when a tile's max exceeds m_ref by more than kLazy, so
// the rescale (a multiply of all 128 accumulators) is rare; probabilities stay below 2^kLazy.
constexpr float kLazy = 8.f;
// In the decode kernel the reference max may lag further behind (probabilities up to 2^32,
// still exact enough in bf16 and far from float32 overflow), so that a new shared reference
// is agreed on only when some wave sees scores 2^32 above it.
constexpr float kLazyBlock = 32.f;

// Q is either in registers (qreg, 4 VGPRs per k-step) or, with QLDS, in an LDS copy qL of the
// 16 heads' rows laid out like a tile (swizzled chunks).
template <int D, bool QLDS>
__device__ __forceinline__ void tile_math(const uint8_t* L, uint32_t valid, const bf16x8* qreg,
                                          const uint8_t* qL, float scale_log2, float& m_ref,
                                          float& l_run, f32x4* oacc) {
  constexpr int KS = D / 32, CT = D / 16, RS = D * 2;
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  // K operand: row mt*16 + l16, chunk (4ks + g) ^ s = 4 (ks ^ (s >> 2)) + ((g ^ s) & 3)
  const int sk = swz_pre(l16);
  const int koff = l16 * RS + ((g ^ sk) & 3) * 16;
  int ko4[4];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) ko4[k4] = koff + 64 * (k4 ^ (sk >> 2));
  f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int ko = ko4[ks & 3] + (ks >> 2) * 256;
    bf16x8 qb;
    if constexpr (QLDS) qb = *(const bf16x8*)(qL + ko);
    else qb = qreg[ks];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bf16x8 av = *(const bf16x8*)(L + ko + mt * 16 * RS);
      sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qb, sacc[mt], 0, 0, 0);
    }
  }
  float x[8];
  float tmax = kNegInf;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt * 16 + 4 * g + i;
      const float v = ((valid >> row) & 1u) ? sacc[mt][i] * scale_log2 : kNegInf;
      x[mt * 4 + i] = v;
      tmax = fmaxf(tmax, v);
    }
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const bool grow = tmax > m_ref + kLazy;
  if (__any(grow)) {
    const float mnew = grow ? tmax : m_ref;
    const float alpha = __builtin_amdgcn_exp2f(m_ref - mnew);   // 0 when m_ref = -inf
    l_run *= alpha;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) oacc[ct] *= alpha;
    m_ref = mnew;
  }
  const float mr = m_ref == kNegInf ? 0.f : m_ref;
  float p[8];
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = __builtin_amdgcn_exp2f(x[j] - mr);
    psum += p[j];
  }
  l_run += psum;
  bf16x8 pb;
#pragma unroll
  for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[j];
  // V^T: group g reads rows ra = 4g + (l16 >> 2) and ra + 16, 8 bytes at column 16 ct + 4 (l16 & 3)
  //   byte 32 ct + 8 q -> chunk (2 ct + (q >> 1)) ^ s = 2 (ct ^ (s >> 1)) + (((q >> 1) ^ s) & 1)
  const int ra = 4 * g + (l16 >> 2), q4 = l16 & 3;
  const int sv = swz_pre(ra);                      // rows ra and ra + 16 share it
  const uint8_t* vb = L + ra * RS + ((((q4 >> 1) ^ sv) & 1) * 16) + (q4 & 1) * 8;
  const uint8_t* vo[8];
#pragma unroll
  for (int c8 = 0; c8 < 8; ++c8) vo[c8] = vb + 32 * (c8 ^ (sv >> 1));
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const uint8_t* va = vo[ct & 7] + (ct >> 3) * 256;
    const i16x4 v0 = lds_read_tr16(va);
    const i16x4 v1 = lds_read_tr16(va + 16 * RS);
    const i16x8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pb, oacc[ct], 0,
                                                       0, 0);
  }
}

template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int t, int head, bf16x8* qreg) {
  constexpr int KS = D / 32;
  const int g = (threadIdx.x & 63) >> 4;
  const bool hv = head < a.H;
  const uint16_t* qrow = a.q + ((int64_t)t * a.H + (hv ? head : 0)) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    i32x4 v = hv ? *(const i32x4*)(qrow + 32 * ks + 8 * g) : i32x4{0, 0, 0, 0};
    qreg[ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// Final (m, l) of one head with the optional sink; returns the factor to apply to O.
__device__ __forceinline__ float finish_head(const AttnArgs& a, int head, float& m, float& l) {
  if (!a.sink) return 1.f;
  const float s2 = a.sink[head] * kLog2e;
  const float mm = fmaxf(m, s2);
  if (mm == kNegInf) return 1.f;
  const float f = __builtin_amdgcn_exp2f(m - mm);
  l = l * f + __builtin_amdgcn_exp2f(s2 - mm);
  m = mm;
  return f;
}

__device__ __forceinline__ float lse_of(float m, float l) {
  return l > 0.f ? (m + __builtin_log2f(l)) * 0.6931471805599453f : kNegInf;
}

// ================================================================ decode kernel
// A block is (query, split of its rows, 16 heads); it walks its rows in 64-row blocks held in a
// double-buffered LDS ring. Wave w gathers rows 16w..16w+15 of the next block while the
// current one is processed: bf16 rows go straight from the paged cache into LDS with
// global_load_lds (no registers; the chunk swizzle is applied to the source addresses), fp8_ds
// rows go through registers to be dequantised. Wave w computes S^T for its 16 rows, the waves
// agree on the block's max per head through LDS, each writes its rows' probabilities (bf16) to
// LDS, and each accumulates O^T for its own quarter of the output columns over all 64 rows:
// 32 accumulator registers per lane, no cross-wave merge of O.
__device__ __forceinline__ void wait_vm_zero() {
  // s_waitcnt vmcnt(0): vmcnt 0, expcnt 7, lgkmcnt 15 (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// Workgroup barrier for LDS data written with ds_write only: waits for this wave's LDS
// operations, not for its outstanding global loads (a __syncthreads() fence would also wait for
// the asynchronous row loads into the other buffer, which must stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0); vmcnt 63, expcnt 7 (no wait)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, int FMT>
__global__ __launch_bounds__(kThreads, 1) void mla_decode_kernel(AttnArgs a) {
  using S = Stage<D, FMT>;
  constexpr int RS = D * 2, KS = D / 32;
  constexpr int CTW = D / 16 / 4;                 // 16-column output tiles per wave
  constexpr int BT = 64;                          // rows per block
  constexpr int WR = BT / 4;                      // rows per wave
  constexpr int PR = BT + 8;                      // P row stride (elements), padded
  constexpr bool ASYNC = FMT == HCS_FMT_BF16;     // rows straight to LDS
  // bf16: rows per 1 KiB load instruction; fp8ds: one row per register load
  constexpr int RPI = ASYNC ? 1024 / RS : 1;
  constexpr int NLD = WR / RPI;
  __shared__ __attribute__((aligned(16))) uint8_t tile0[BT * RS];
  __shared__ __attribute__((aligned(16))) uint8_t tile1[BT * RS];
  // ASYNC: byte address of every row (the zero row where a row does not take part);
  // otherwise the packed (cache, page, slot) entries
  __shared__ __attribute__((aligned(16))) uint32_t rowtab[ASYNC ? 2 * kMaxRowsWG : kMaxRowsWG];
  __shared__ __attribute__((aligned(16))) __bf16 p_lds0[16 * PR];
  __shared__ __attribute__((aligned(16))) __bf16 p_lds1[16 * PR];
  __shared__ float mx[4][16];
  __shared__ float lsum[4][16];
  __shared__ int flag0[4], flag1[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  // block -> (query, split, head group) with all blocks of a query on one XCD
  const int G = a.nsplit * a.n_hg;
  const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int t = (r / G) * 8 + xcd;
  if (t >= a.N) return;
  const int j = r - (r / G) * G;
  const int s = j / a.n_hg, hg = j - (j / a.n_hg) * a.n_hg;

  const QueryRows q = query_rows(a, t);
  const int r0 = s * a.rows_per_split;
  const int n_rows = max(0, min(q.R, r0 + a.rows_per_split) - r0);
  fill_rowtab(a, t, q, r0, n_rows, rowtab, BT);
  if constexpr (ASYNC) {
    // entries -> addresses, in place from the top so no entry is overwritten before it is read
    __syncthreads();
    const int n64 = (n_rows + BT - 1) / BT * BT;
    uint32_t ent[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int li = (int)threadIdx.x + i * kThreads;
      ent[i] = li < n64 ? rowtab[li] : kNoRow;
    }
    __syncthreads();
    uint64_t* addr = reinterpret_cast<uint64_t*>(rowtab);
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
      const int li = (int)threadIdx.x + i * kThreads;
      const uint32_t e = ent[i];
      const uint8_t* p = e != kNoRow
                             ? ((e >> 31) ? a.comp.base : a.swa.base) + (size_t)(e & 0x7fffffffu) * RS
                             : g_zero_row;
      if (li < n64) addr[li] = reinterpret_cast<uint64_t>(p);
    }
  }
  // q of the 16 heads as the B operand (same for the 4 waves)
  bf16x8 qreg[KS];
  load_q<D>(a, t, hg * 16 + l16, qreg);

  f32x4 oacc[CTW];
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_part = 0.f;
  const int nblk = (n_rows + BT - 1) / BT;

  i32x4 pre[ASYNC ? 1 : NLD];
  float psc[ASYNC ? 1 : NLD];
  __syncthreads();

  // gather this wave's rows of block b into buffer tbuf
  // per-lane source offsets of the async row loads (the swizzle is applied on the source side:
  // LDS chunk slot `lane` of row r receives source chunk lane ^ swz(r))
  int soff[ASYNC ? NLD : 1];
  if constexpr (ASYNC) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int rw = i * RPI + lane / (64 / RPI);
      soff[i] = ((lane % (64 / RPI)) ^ swz_dec(rw)) * 16;         // rows 16w + rw share swz_dec(rw)
    }
  }
  auto issue = [&](int b, uint8_t* tbuf) {
    if constexpr (ASYNC) {
      const uint64_t* at = reinterpret_cast<const uint64_t*>(rowtab) + b * BT + wave * WR;
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int rw = i * RPI + lane / (64 / RPI);             // row of this lane within the wave's rows
        uint64_t src;
        if constexpr (RPI == 1) {
          // both halves zero-extended (readfirstlane returns a signed int)
          const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)at[i]);
          const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(at[i] >> 32));
          src = (uint64_t)lo | ((uint64_t)hi << 32);
        } else {
          src = at[rw];
        }
        uint8_t* dst = tbuf + (wave * WR + i * RPI) * RS;       // 1 KiB of consecutive rows
        __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const uint8_t*>(src) + soff[i]),
                                         (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
      }
    } else {
      const uint32_t* rt = rowtab + b * BT + wave * WR;
#pragma unroll
      for (int i = 0; i < NLD; ++i) S::load(a, rt[i], lane, pre[i], psc[i]);
    }
  };
  if (nblk > 0) issue(0, tile0);

  // lane-constant LDS offsets
  // K row 16w + l16, chunk (4ks + g) ^ s = 4 (ks ^ (s >> 2)) + ((g ^ s) & 3), s = swz_dec(l16)
  const int sk = swz_dec(l16);
  const int koff = (wave * WR + l16) * RS + ((g ^ sk) & 3) * 16;
  int ko4[4];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) ko4[k4] = koff + 64 * (k4 ^ (sk >> 2));
  // V^T rows 8g + jv and 8g + 4 + jv of a 32-row step: swz_dec = 2 jv + 8 (g & 1) (+1), so
  // chunk (2 ctg + h) lands at 2 (ctg ^ (jv + 4 (g & 1))) + (h, resp. h ^ 1)
  const int jv = l16 >> 2, q4 = l16 & 3, h2 = q4 >> 1;
  const int vx = jv + 4 * (g & 1);
  const int vrow = (8 * g + jv) * RS + (q4 & 1) * 8;
  int vo0[8], vo1[8];
#pragma unroll
  for (int c8 = 0; c8 < 8; ++c8) {
    vo0[c8] = vrow + 32 * (c8 ^ vx) + 16 * h2;
    vo1[c8] = vrow + 4 * RS + 32 * (c8 ^ vx) + 16 * (h2 ^ 1);
  }
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

  // One block; T holds it, TN receives the next one, P/F are this block's probability buffer
  // and flags. The loop below is unrolled by two so that the two LDS buffers are distinct
  // objects: the async loads into TN are then known not to alias reads of T (no wait).
  // Shared reference max: every wave uses the same m_ref for the whole block, so each can
  // write its rows' probabilities for the column-split PV. A wave whose scores exceed
  // m_ref + kLazyBlock raises a flag; only then do the waves exchange maxima and rescale.
  auto block = [&](int b, uint8_t* T, uint8_t* TN, __bf16* P, int* F) {
    if constexpr (!ASYNC) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) S::store(T, wave * WR + i, swz_dec(i), lane, pre[i], psc[i]);
    } else {
      wait_vm_zero();                                    // this wave's rows of block b landed
    }
    lds_barrier();                                       // block b is in LDS
    if (b + 1 < nblk) issue(b + 1, TN);
    bool vr;
    if constexpr (ASYNC)
      vr = reinterpret_cast<const uint64_t*>(rowtab)[b * BT + wave * WR + (lane & 15)] !=
           reinterpret_cast<uint64_t>(g_zero_row);
    else
      vr = rowtab[b * BT + wave * WR + (lane & 15)] != kNoRow;
    const uint32_t valid = (uint32_t)__ballot(vr && lane < 16);
    // ---- S^T for this wave's 16 rows (two accumulators halve the dependent chain)
    f32x4 sacc2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ko = ko4[ks & 3] + (ks >> 2) * 256;
      const bf16x8 av = *(const bf16x8*)(T + ko);
      sacc2[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[ks], sacc2[ks & 1], 0, 0, 0);
    }
    const f32x4 sacc = sacc2[0] + sacc2[1];
    float x[4];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * g + i;
      x[i] = ((valid >> row) & 1u) ? sacc[i] * a.scale_log2 : kNegInf;
      tmax = fmaxf(tmax, x[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const bool over = tmax > m_ref + kLazyBlock;
    const bool any_over = __any(over);
    float mr = m_ref == kNegInf ? 0.f : m_ref;
    bf16x4 p4;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pv = __builtin_amdgcn_exp2f(x[i] - mr);
      psum += pv;
      p4[i] = (__bf16)pv;
    }
    if (g == 0) mx[wave][l16] = tmax;
    if (lane == 0) F[wave] = any_over ? 1 : 0;
    if (!any_over) *(bf16x4*)(P + l16 * PR + wave * WR + 4 * g) = p4;
    lds_barrier();                                       // probabilities (or flags) of the block
    if (F[0] | F[1] | F[2] | F[3]) {
      // rare: a new reference max for the heads whose block max is above m_ref + kLazy
      const float bmax = fmaxf(fmaxf(mx[0][l16], mx[1][l16]), fmaxf(mx[2][l16], mx[3][l16]));
      const bool grow = bmax > m_ref + kLazy;
      const float mnew = grow ? bmax : m_ref;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - mnew);
      l_part *= alpha;
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) oacc[ct] *= alpha;
      m_ref = mnew;
      mr = m_ref == kNegInf ? 0.f : m_ref;
      psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(x[i] - mr);
        psum += pv;
        p4[i] = (__bf16)pv;
      }
      *(bf16x4*)(P + l16 * PR + wave * WR + 4 * g) = p4;
      lds_barrier();
    }
    l_part += psum;
    // ---- O^T (this wave's columns) += V^T P^T over the block's 64 rows
#pragma unroll
    for (int kk = 0; kk < BT / 32; ++kk) {
      const bf16x8 pb = *(const bf16x8*)(P + l16 * PR + kk * 32 + 8 * g);
      const uint8_t* vb = T + kk * 32 * RS;
#pragma unroll
      for (int ct = 0; ct < CTW; ++ct) {
        const int ctg = wave * CTW + ct;
        const int hi = (ctg >> 3) * 256;
        const i16x4 v0 = lds_read_tr16(vb + vo0[ctg & 7] + hi);
        const i16x4 v1 = lds_read_tr16(vb + vo1[ctg & 7] + hi);
        const i16x8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pb, oacc[ct],
                                                           0, 0, 0);
      }
    }
  };
  for (int b = 0; b < nblk; b += 2) {
    block(b, tile0, tile1, p_lds0, flag0);
    if (b + 1 < nblk) block(b + 1, tile1, tile0, p_lds1, flag1);
  }

  // ---- sums over the waves' rows (all waves share m_ref)
  float lw = l_part + __shfl_xor(l_part, 16, 64);
  lw += __shfl_xor(lw, 32, 64);
  if (g == 0) lsum[wave][l16] = lw;
  __syncthreads();
  float L = lsum[0][l16] + lsum[1][l16] + lsum[2][l16] + lsum[3][l16];
  float M = m_ref;
  const int hh = hg * 16 + l16;
  const bool hv = hh < a.H;
  // lane holds O^T[c = 16 ctg + 4g + i][head l16] for ctg = wave * CTW + ct
  if (a.nsplit == 1) {
    if (!hv) return;
    const float f = finish_head(a, hh, M, L);
    const float inv = L > 0.f ? f / L : 0.f;
    uint16_t* orow = a.out + ((int64_t)t * a.H + hh) * D;
#pragma unroll
    for (int ct = 0; ct < CTW; ++ct) {
      const f32x4 o = oacc[ct] * inv;
      uint2 pk;
      pk.x = pack_bf16x2(o[0], o[1]);
      pk.y = pack_bf16x2(o[2], o[3]);
      *(uint2*)(orow + 16 * (wave * CTW + ct) + 4 * g) = pk;
    }
    if (a.lse && g == 0 && wave == 0) a.lse[(int64_t)t * a.H + hh] = lse_of(M, L);
    return;
  }

  // ---- split: write this split's partial (unnormalised O, reference max, sum); a second
  // kernel merges the splits (a kernel boundary orders the writes before the reads on every
  // XCD, which in-kernel device-scope fences would do at a far higher cost)
  const int64_t prow = ((int64_t)(t * a.n_hg + hg) * a.nsplit + s) * 16 + l16;
  float* po = a.ws_o + prow * D;
#pragma unroll
  for (int ct = 0; ct < CTW; ++ct) *(f32x4*)(po + 16 * (wave * CTW + ct) + 4 * g) = oacc[ct];
  if (g == 0 && wave == 0) {
    a.ws_ml[prow * 2 + 0] = M;
    a.ws_ml[prow * 2 + 1] = L;
  }
}

// Merge the split partials of one (query, 16-head group): thread -> head tid / 16, D/16 columns.
template <int D>
__global__ __launch_bounds__(kThreads) void mla_combine_kernel(AttnArgs a) {
  constexpr int PER = D / 16;
  const int t = blockIdx.x, hg = blockIdx.y, tid = threadIdx.x;
  const int h = tid >> 4, c0 = (tid & 15) * PER;
  const int hq = hg * 16 + h;
  const int64_t pbase = ((int64_t)(t * a.n_hg + hg) * a.nsplit) * 16 + h;   // row of split 0
  float Ms = kNegInf;
  for (int ss = 0; ss < a.nsplit; ++ss) Ms = fmaxf(Ms, a.ws_ml[(pbase + (int64_t)ss * 16) * 2]);
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;
  float Ls = 0.f;
  if (Ms != kNegInf) {
    for (int ss = 0; ss < a.nsplit; ++ss) {
      const int64_t pr = pbase + (int64_t)ss * 16;
      const float ms = a.ws_ml[pr * 2], ls = a.ws_ml[pr * 2 + 1];
      if (!(ls > 0.f)) continue;
      const float f = __builtin_amdgcn_exp2f(ms - Ms);
      Ls += ls * f;
      const float* src = a.ws_o + pr * D + c0;
#pragma unroll
      for (int c = 0; c < PER; c += 4) {
        const f32x4 v = *(const f32x4*)(src + c);
        acc[c] += f * v[0];
        acc[c + 1] += f * v[1];
        acc[c + 2] += f * v[2];
        acc[c + 3] += f * v[3];
      }
    }
  }
  if (hq >= a.H) return;
  const float f = finish_head(a, hq, Ms, Ls);
  const float inv = Ls > 0.f ? f / Ls : 0.f;
  uint16_t* orow = a.out + ((int64_t)t * a.H + hq) * D + c0;
#pragma unroll
  for (int c = 0; c < PER; c += 2) *(uint32_t*)(orow + c) = pack_bf16x2(acc[c] * inv, acc[c + 1] * inv);
  if (a.lse && (tid & 15) == 0) a.lse[(int64_t)t * a.H + hq] = lse_of(Ms, Ls);
}

// ================================================================ prefill kernel
template <int D, int FMT>
__global__ __launch_bounds__(kThreads, 1) void mla_prefill_kernel(AttnArgs a) {
  using S = Stage<D, FMT>;
  constexpr int CT = D / 16, KS = D / 32;
  // each wave stages 8 rows of every 32-row tile (RPL rows per load)
  constexpr int NLDW = (kTile / 4) / S::RPL > 0 ? (kTile / 4) / S::RPL : 1;
  constexpr int WROWS = NLDW * S::RPL;               // rows staged per wave per tile
  __shared__ __attribute__((aligned(16))) uint8_t lds_tile[2][kTile * S::RS];
  __shared__ uint32_t rowtab[kMaxRowsWG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int t = blockIdx.x;
  const int hbase = blockIdx.y * 64 + wave * 16;
  const int head = hbase + l16;
  const bool wave_active = hbase < a.H;

  const QueryRows q = query_rows(a, t);
  const int n_rows = min(q.R, kMaxRowsWG);
  fill_rowtab(a, t, q, 0, n_rows, rowtab);
  bf16x8 qreg[KS];
  load_q<D>(a, t, head, qreg);
  __syncthreads();

  f32x4 oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const int ntiles = (n_rows + kTile - 1) / kTile;

  i32x4 pre[NLDW];
  float psc[NLDW];
  auto issue = [&](int tt) {
#pragma unroll
    for (int i = 0; i < NLDW; ++i) {
      const int rr = tt * kTile + wave * WROWS + i * S::RPL + S::lane_row(lane);
      const uint32_t e = rr < n_rows ? rowtab[rr] : kNoRow;
      S::load(a, e, lane, pre[i], psc[i]);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NLDW; ++i)
      S::store(lds_tile[buf], wave * WROWS + i * S::RPL + S::lane_row(lane),
               swz_pre(wave * WROWS + i * S::RPL + S::lane_row(lane)), lane, pre[i], psc[i]);
  };
  if (ntiles > 0) {
    issue(0);
    store(0);
  }
  __syncthreads();
  for (int tt = 0; tt < ntiles; ++tt) {
    const int buf = tt & 1;
    const bool more = tt + 1 < ntiles;
    if (more) issue(tt + 1);
    const bool vr = rowtab[tt * kTile + (lane & 31)] != kNoRow;
    const uint32_t valid = (uint32_t)__ballot(vr && lane < 32);
    if (wave_active)
      tile_math<D, false>(lds_tile[buf], valid, qreg, nullptr, a.scale_log2, m_run, l_run, oacc);
    if (more) store(buf ^ 1);
    __syncthreads();
  }
  if (!wave_active) return;
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (head >= a.H) return;
  float mfin = m_run;
  const float f = finish_head(a, head, mfin, l_tot);
  const float inv = l_tot > 0.f ? f / l_tot : 0.f;
  uint16_t* orow = a.out + ((int64_t)t * a.H + head) * D;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const f32x4 o = oacc[ct] * inv;
    uint2 pk;
    pk.x = pack_bf16x2(o[0], o[1]);
    pk.y = pack_bf16x2(o[2], o[3]);
    *(uint2*)(orow + 16 * ct + 4 * g) = pk;
  }
  if (a.lse && g == 0) a.lse[(int64_t)t * a.H + head] = lse_of(mfin, l_tot);
}

template <int D, int FMT>
hipError_t launch_impl(const AttnArgs& a, hipStream_t stream) {
  if (a.kind == 1) {
    dim3 grid((unsigned)a.N, (unsigned)((a.H + 63) / 64));
    hipLaunchKernelGGL((mla_prefill_kernel<D, FMT>), grid, dim3(kThreads), 0, stream, a);
  } else {
    const int n8 = (a.N + 7) / 8;
    dim3 grid((unsigned)(n8 * 8 * a.nsplit * a.n_hg));
    hipLaunchKernelGGL((mla_decode_kernel<D, FMT>), grid, dim3(kThreads), 0, stream, a);
    if (a.nsplit > 1)
      hipLaunchKernelGGL((mla_combine_kernel<D>), dim3(a.N, a.n_hg), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int N, int H, int d, int window, int m, int topk, int max_pos) {
  AttnPlan p{};
  const int64_t nv = (int64_t)(max_pos + 1) / m;
  const int64_t rows = (int64_t)std::min(window, max_pos + 1) + (topk > 0 ? topk : nv);
  const int64_t tiles = std::max<int64_t>(1, (rows + kTile - 1) / kTile);
  const int64_t fits = tiles * kTile <= kMaxRowsWG;
  // many queries and every row list fits one block: one block per query and 64 heads
  if (fits && (int64_t)N * ((H + 63) / 64) >= 256) {
    p.kind = 1;
    p.nsplit = 1;
    p.n_hg = (H + 63) / 64;
    p.rows_per_split = (int)(tiles * kTile);
    return p;
  }
  p.kind = 0;
  p.n_hg = (H + 15) / 16;
  constexpr int64_t kBlock = 64;                       // decode blocks walk 64 rows at a time
  const int64_t blocks = (rows + kBlock - 1) / kBlock;
  const int64_t max_bps = kMaxRowsWG / kBlock;
  const int64_t per_split = (int64_t)((N + 7) / 8) * 8 * p.n_hg;
  int64_t nsplit = std::max<int64_t>(1, (256 + per_split - 1) / per_split);
  nsplit = std::min(nsplit, blocks);
  nsplit = std::max<int64_t>(nsplit, (blocks + max_bps - 1) / max_bps);
  const int64_t bps = (blocks + nsplit - 1) / nsplit;
  nsplit = (blocks + bps - 1) / bps;
  p.nsplit = (int)nsplit;
  p.rows_per_split = (int)(bps * kBlock);
  if (nsplit > 1) {
    const size_t parts = (size_t)N * p.n_hg * nsplit * 16;
    p.ws_o_bytes = parts * d * sizeof(float);
    p.ws_ml_bytes = parts * 2 * sizeof(float);
    p.ws_bytes = p.ws_o_bytes + p.ws_ml_bytes;
  }
  return p;
}

hipError_t launch_sparse_mla(const AttnArgs& a, int d, int fmt, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  if (d == 512 && fmt == HCS_FMT_BF16) return launch_impl<512, HCS_FMT_BF16>(a, stream);
  if (d == 512 && fmt == HCS_FMT_FP8DS) return launch_impl<512, HCS_FMT_FP8DS>(a, stream);
  if (d == 128 && fmt == HCS_FMT_BF16) return launch_impl<128, HCS_FMT_BF16>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace hcs
