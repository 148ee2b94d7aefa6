// Sparse MLA (single shared KV head) attention for gfx950.
//
// What it computes: "DeepSeek V4 Attention: Code Reading Map", section "Phase 3: forward_mqa()":
// every query head attends over the query's sliding-window rows plus its selected (CSA) or all
// visible (HCA) compressed entries; K and V are the same shared row.
//
// Design:
//   * a workgroup is (query, split of its rows, 64 heads), so each gathered row is read once for
//     all heads of the query; it first resolves the physical row of every logical row it will
//     read (window position or compressed id -> page table -> page, slot) into an LDS table,
//     with all loads issued together and no branches, so each later row load is a single
//     independent gather; rows that do not take part read a zero row;
//   * rows are walked in 32-row blocks through a ring of four LDS tiles, their 16-byte chunks
//     swizzled so that both readers below are free of bank conflicts. bf16 rows go straight
//     from the paged cache into LDS with global_load_lds; quantized rows (fp8_ds, MXFP8, NVFP4)
//     come through registers one block ahead and are written dequantised to bf16 (every
//     format's values are exact in bf16);
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (rows on M, 16 heads on N, q in registers as
//     the B operand), whose accumulator layout is the one P^T is written in, then
//     O^T += V^T P^T with V^T read from the same LDS rows by ds_read_b64_tr_b16 (16-bit
//     transpose across each 16-lane group); online softmax in base 2, one head per lane % 16;
//   * a query's rows may be split over several workgroups; their partial (O, max, sum) are
//     merged by a second kernel.
#include "kernels.h"
#include "select.h"

namespace hcs {

HCS_DEVICE_ERROR_WORD(attention)

// A zero row: rows that take part in nothing load from here, so loads never branch.
__device__ __attribute__((aligned(64))) uint8_t g_zero_row[1024];
// A page of zeros in every quantised row format (the fp8_ds page is the largest): absent rows
// are read from it, so the loads of a row never depend on whether the row exists.
__device__ __attribute__((aligned(64))) uint8_t g_zero_page[kFp8PageBytes];
static_assert(kFp8PageBytes >= kMx8PageBytes && kFp8PageBytes >= kNv4PageBytes, "zero page size");

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRowsWG = 2304;            // rows in one workgroup's address table
constexpr uint32_t kNoRow = 0xFFFFFFFFu;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 __attribute__((address_space(3)))*)(p));
}

// max of v over lanes l, l ^ 16, l ^ 32, l ^ 48, in every lane, with two VALU lane swaps
// (v_permlane16_swap / v_permlane32_swap of v with itself give v and the partner lane's value).
__device__ __forceinline__ float max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// the same for a sum: (v_l + v_{l^16}) + (v_{l^32} + v_{l^48})
__device__ __forceinline__ float sum_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// two floats -> packed bf16 (round to nearest even), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// two e4m3 values (bytes 0-1, or 2-3 with HI) times the power of two sc, as bf16 (exact: the
// product has at most four significant bits), by one scaled hardware conversion
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, float sc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, sc, HI);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
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
  q.n_comp = a.topk_idx || a.scores ? a.topk : q.nv;
  q.R = q.n_swa + q.n_comp;
  return q;
}

// Entries of a sequence's compressed page table that the all-heads kernel keeps in LDS.
constexpr int kPtCache = 2048;

// fill_rowtab for the all-heads kernel (NT threads), with one memory latency fewer: the page-table
// row of the sequence's compressed cache (its first kPtCache entries) is read into LDS (ptl)
// together with the selected ids and the window rows' page entries, so that a selected row's
// page is then an LDS lookup. A sequence with more pages than that reads them from memory.
// rowtab[0 .. n rounded up to `pad`) is written; ends with a barrier.
template <int NT, int PTC = kPtCache>
__device__ __forceinline__ void fill_rows(const AttnArgs& a, int t, const QueryRows& q, int r0, int n,
                                          uint32_t* rowtab, int* ptl, int pad) {
  constexpr int RPT = (kMaxRowsWG + NT - 1) / NT;
  constexpr int PPT = PTC / NT;
  const int tid = threadIdx.x;
  const int npg = (q.nv + 63) >> 6;
  const bool cached = npg <= PTC;
  const int32_t* cpt = a.comp.pt + (int64_t)q.seq * a.comp.pt_stride;
  const int32_t* spt = a.swa.pt + (int64_t)q.seq * a.swa.pt_stride;
  int pv[PPT];
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int idx = tid + k * NT;
    pv[k] = cached && idx < npg ? __ldg(cpt + idx) : 0;
  }
  const int last = max(q.R - 1, 0);
  int id[RPT], spg[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int gr = min(r0 + tid + i * NT, last);
    const int j = min(max(gr - q.n_swa, 0), max(q.n_comp - 1, 0));
    id[i] = a.topk_idx ? __ldg(a.topk_idx + (int64_t)t * a.topk + j) : j;
    spg[i] = gr < q.n_swa ? __ldg(spt + ((q.lo + gr) >> 6)) : 0;
  }
#pragma unroll
  for (int k = 0; k < PPT; ++k) {
    const int idx = tid + k * NT;
    if (idx < npg && cached) ptl[idx] = pv[k];
  }
  __syncthreads();
  const int np = min((n + pad - 1) / pad * pad, kMaxRowsWG);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int li = tid + i * NT;
    const int gr = r0 + li;
    const bool is_swa = gr < q.n_swa;
    const bool ok_id = is_swa || (id[i] >= 0 && id[i] < q.nv);
    const int row = ok_id ? (is_swa ? q.lo + gr : id[i]) : 0;
    int pg = spg[i];
    if (!is_swa && li < np) pg = cached ? ptl[row >> 6] : __ldg(cpt + (row >> 6));
    const int npages = is_swa ? a.swa.num_pages : a.comp.num_pages;
    const bool used = li < n && gr < q.R && ok_id;
    if (used && pg >= npages) dev_error(HCS_DEVERR_PAGE_RANGE);
    const bool ok = used && pg >= 0 && pg < npages;
    if (li < np) rowtab[li] = ok ? ((is_swa ? 0u : 0x80000000u) | (uint32_t)(pg * 64 + (row & 63))) : kNoRow;
  }
  wait_vm_zero();     // LDS copies the caller started before (dma16) have landed as well
  __syncthreads();
}

// fill_rows for a block that selects its query's compressed rows itself from the indexer scores
// (a.scores): the top-k of the visible entries' scores, exact, ties at the k-th score going to the
// smaller ids (the rule of the indexer's selection kernels), or every visible entry when there
// are at most k. Each thread holds the keys of a contiguous run of ids in registers, and reg_topk
// places the selected ids in id order, so that every split of the query computes the same row
// order and takes its own range of it. `scratch` is LDS of kSelScratch bytes that
// nothing else uses until the caller's next barrier; rowtab[0 .. n rounded up to `pad`) is
// written; ends with a barrier. Split 0 writes the ids to a.sel_out.
constexpr int kSelScratch = (int)sizeof(SelShared);

// IPT: the scores a thread holds (ids tid * IPT ..), the least of 4, 8, 16 with NT * IPT >= nv
template <int NT, int IPT>
__device__ __forceinline__ void fill_rows_sel(const AttnArgs& a, int t, int s, const QueryRows& q, int r0,
                                              int n, uint32_t* rowtab, int* ptl, int pad, uint8_t* scratch) {
  static_assert(NT * 16 >= kSelMax && IPT <= 16, "selection size");
  constexpr int RPT = (kMaxRowsWG + NT - 1) / NT;
  constexpr int PPT = kPtCache / NT;
  SelShared& sh = *reinterpret_cast<SelShared*>(scratch);
  const int tid = threadIdx.x;
  const int nv = q.nv, k = a.topk;
  const int npg = (nv + 63) >> 6;
  const bool cached = npg <= kPtCache;
  const int32_t* cpt = a.comp.pt + (int64_t)q.seq * a.comp.pt_stride;
  const int32_t* spt = a.swa.pt + (int64_t)q.seq * a.swa.pt_stride;
  const float* sc = a.scores + (int64_t)t * a.score_stride;
  // ---- every load at once: compressed page table, window rows' pages, the scores of this
  // thread's ids i0 .. i0 + c - 1
  int pv[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int idx = tid + j * NT;
    pv[j] = cached && idx < npg ? __ldg(cpt + idx) : 0;
  }
  int spg[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int gr = r0 + tid + i * NT;
    spg[i] = gr < q.n_swa ? __ldg(spt + ((q.lo + gr) >> 6)) : 0;
  }
  const int i0 = tid * IPT;
  float sv[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) sv[j] = i0 + j < nv ? __ldg(sc + i0 + j) : 0.f;
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int idx = tid + j * NT;
    if (idx < npg && cached) ptl[idx] = pv[j];
  }
  uint32_t key[IPT], vmask = 0u;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    key[j] = f32_order_key(sv[j]);
    vmask |= (i0 + j < nv ? 1u : 0u) << j;
  }
  const int np = min((n + pad - 1) / pad * pad, kMaxRowsWG);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int li = tid + i * NT;
    if (li < np) rowtab[li] = kNoRow;
  }
  sel_reset<NT>(sh);
  __syncthreads();
  // ---- the top-k (every visible entry when nv <= k), in id order: rowtab entries of this
  // split's range, and split 0 writes the ids to a.sel_out
  int32_t* out = a.sel_out && s == 0 ? a.sel_out + (int64_t)t * k : nullptr;
  const unsigned n_sel = reg_topk<NT, IPT>(
      sh, key, vmask, (unsigned)k, true, [&](int j) { return i0 + j; },
      [&](unsigned pos, int j, uint32_t) {
        const int li = q.n_swa + (int)pos - r0;
        if (li >= 0 && li < n) rowtab[li] = (uint32_t)(i0 + j);
        if (out && pos < (unsigned)k) out[pos] = i0 + j;
      });
  if (out)
    for (int j = (int)n_sel + tid; j < k; j += NT) out[j] = -1;
  // ---- ids -> row entries (each thread converts the entries it owns)
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int li = tid + i * NT;
    if (li >= np) continue;
    const int gr = r0 + li;
    uint32_t e = kNoRow;
    if (li < n && gr < q.R) {
      if (gr < q.n_swa) {
        const int pg = spg[i];
        const int row = q.lo + gr;
        if (pg >= a.swa.num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
        if (pg >= 0 && pg < a.swa.num_pages) e = (uint32_t)(pg * 64 + (row & 63));
      } else {
        const uint32_t id = rowtab[li];
        if (id != kNoRow) {
          // (nv <= kSelMax: the page-table row is always in LDS; no flat load)
          static_assert(kSelMax / 64 <= kPtCache, "the selection's page-table row fits in LDS");
          const int pg = ptl[id >> 6];
          if (pg >= a.comp.num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
          if (pg >= 0 && pg < a.comp.num_pages) e = 0x80000000u | (uint32_t)(pg * 64 + (id & 63));
        }
      }
    }
    rowtab[li] = e;
  }
  wait_vm_zero();     // LDS copies the caller started before (dma16) have landed as well
  __syncthreads();
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

// Quantized 512-dim rows, one row per wave-wide register load, written dequantised to bf16 into
// the LDS tile (every format's value is exact in bf16). For each format: `load` takes this
// lane's 16-byte piece of row `slot` of `page` (nullptr: the row does not take part; it then
// reads the zero row, so a wave's loads never branch and all stay in flight together) and the
// scale bits the piece needs; `store` writes the piece's bf16 values into the tile row, its
// 16-byte chunks swizzled by `sw` (the bf16 row is 1 KiB = 64 chunks).
template <int FMT>
struct RowFmt;

// fp8_ds: 448 e4m3 latent + 64 bf16 rope + a UE8M0 scale per 64 latent dims. Lanes 0..27 take
// 16 latent codes, lanes 28..35 8 rope values, the others nothing.
template <>
struct RowFmt<HCS_FMT_FP8DS> {
  static constexpr int PB = kFp8PageBytes;
  // byte offsets in the page of the lane's 16-byte load and of its scale byte
  __device__ static __forceinline__ int voff(int slot, int lane) {
    const bool rope = lane >= 28 && lane < 36;
    const int base = rope ? kFp8PageRope + (lane - 28) * 16 : kFp8PageCodes + (lane < 28 ? lane * 16 : 0);
    return base + slot * (rope ? kFp8Rope * 2 : kFp8Latent);
  }
  __device__ static __forceinline__ int soff(int slot, int lane) {
    return kFp8PageScales + slot * 8 + (min(lane, 27) >> 2);
  }
  __device__ static __forceinline__ void store(uint8_t* row, int sw, int lane, const i32x4& v, int se) {
    const float sc = __builtin_ldexpf(1.f, se - 127);
    if (lane < 28) {
      i32x4 lo4, hi4;
      lo4.x = e4m3x2_to_bf16x2<false>(v.x, sc);
      lo4.y = e4m3x2_to_bf16x2<true>(v.x, sc);
      lo4.z = e4m3x2_to_bf16x2<false>(v.y, sc);
      lo4.w = e4m3x2_to_bf16x2<true>(v.y, sc);
      hi4.x = e4m3x2_to_bf16x2<false>(v.z, sc);
      hi4.y = e4m3x2_to_bf16x2<true>(v.z, sc);
      hi4.z = e4m3x2_to_bf16x2<false>(v.w, sc);
      hi4.w = e4m3x2_to_bf16x2<true>(v.w, sc);
      *(i32x4*)(row + ((2 * lane) ^ sw) * 16) = lo4;
      *(i32x4*)(row + ((2 * lane + 1) ^ sw) * 16) = hi4;
    } else if (lane < 36) {
      *(i32x4*)(row + ((56 + lane - 28) ^ sw) * 16) = v;
    }
  }
};

// MXFP8: 512 e4m3 + a UE8M0 scale per 32 dims. Lanes 0..31 take 16 codes (half a scale block).
template <>
struct RowFmt<HCS_FMT_MXFP8> {
  static constexpr int PB = kMx8PageBytes;
  __device__ static __forceinline__ int voff(int slot, int lane) { return slot * 512 + (lane & 31) * 16; }
  __device__ static __forceinline__ int soff(int slot, int lane) {
    return kMx8Scales + slot * 16 + ((lane & 31) >> 1);
  }
  __device__ static __forceinline__ void store(uint8_t* row, int sw, int lane, const i32x4& v, int se) {
    if (lane >= 32) return;
    const float sc = __builtin_ldexpf(1.f, se - 127);
    i32x4 lo4, hi4;
    lo4.x = e4m3x2_to_bf16x2<false>(v.x, sc);
    lo4.y = e4m3x2_to_bf16x2<true>(v.x, sc);
    lo4.z = e4m3x2_to_bf16x2<false>(v.y, sc);
    lo4.w = e4m3x2_to_bf16x2<true>(v.y, sc);
    hi4.x = e4m3x2_to_bf16x2<false>(v.z, sc);
    hi4.y = e4m3x2_to_bf16x2<true>(v.z, sc);
    hi4.z = e4m3x2_to_bf16x2<false>(v.w, sc);
    hi4.w = e4m3x2_to_bf16x2<true>(v.w, sc);
    *(i32x4*)(row + ((2 * lane) ^ sw) * 16) = lo4;
    *(i32x4*)(row + ((2 * lane + 1) ^ sw) * 16) = hi4;
  }
};

// NVFP4: 512 e2m1 (two per byte, element 2j low) + an e4m3 scale per 16 dims. Every lane takes
// 8 values (4 code bytes, one 16-byte bf16 chunk) and the scale byte of its half block; the
// 4 code bytes come in the aligned 16-byte load shared by lanes 4j .. 4j+3 (the same load
// shape as the other formats, so a row's loads never depend on its format).
template <>
struct RowFmt<HCS_FMT_NVFP4> {
  static constexpr int PB = kNv4PageBytes;
  __device__ static __forceinline__ int voff(int slot, int lane) { return slot * 256 + (lane >> 2) * 16; }
  __device__ static __forceinline__ int soff(int slot, int lane) { return kNv4Scales + slot * 32 + (lane >> 1); }
  // byte k of the codes -> its two values (low nibble first) as bf16 by the hardware conversion
  // (unit scale), then times the e4m3 block scale; the product has at most 6 significant bits,
  // so it is exact in bf16 and the float32 result's upper half is the bf16
  template <int K>
  __device__ static __forceinline__ uint32_t pair(uint32_t w, float s) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, K);
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    const float lo = __uint_as_float(u << 16) * s, hi = __uint_as_float(u & 0xffff0000u) * s;
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
  }
  __device__ static __forceinline__ void store(uint8_t* row, int sw, int lane, const i32x4& v, int se) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 sc = __builtin_amdgcn_cvt_pk_f32_fp8(se, false);
    const uint32_t w = (uint32_t)((lane & 2) ? ((lane & 1) ? v.w : v.z) : ((lane & 1) ? v.y : v.x));
    *(i32x4*)(row + (lane ^ sw) * 16) = i32x4{(int)pair<0>(w, sc.x), (int)pair<1>(w, sc.x),
                                              (int)pair<2>(w, sc.x), (int)pair<3>(w, sc.x)};
  }
};

// The rows of one attention call: window rows in format SF, compressed rows in format CF. The
// row table entry's top bit says which cache a row comes from (wave-uniform); `load` returns it
// for the store. Every format loads 16 bytes and a scale byte per lane, so the source only picks
// the addresses: no branch, and no wait on one row's loads before the next row's are issued.
template <int SF, int CF>
struct QuantStage {
  static constexpr int D = 512, RS = D * 2;
  __device__ static __forceinline__ bool load(const uint8_t* swa_base, const uint8_t* comp_base,
                                              uint32_t e, int lane, i32x4& v, int& se) {
    e = (uint32_t)__builtin_amdgcn_readfirstlane((int)e);
    const bool ok = e != kNoRow;
    const bool comp = (e >> 31) != 0;
    const uint32_t ridx = e & 0x7fffffffu;
    const int slot = (int)(ridx & 63);
    const size_t pg = ridx >> 6;
    // an absent row reads the zero page (slot 63 of it lies inside the page in every format)
    const uint8_t* page = !ok ? g_zero_page
                        : comp ? comp_base + pg * RowFmt<CF>::PB : swa_base + pg * RowFmt<SF>::PB;
    const bool cf = ok && comp;
    const int vo = cf ? RowFmt<CF>::voff(slot, lane) : RowFmt<SF>::voff(slot, lane);
    const int so = cf ? RowFmt<CF>::soff(slot, lane) : RowFmt<SF>::soff(slot, lane);
    v = *(const i32x4*)(page + vo);
    se = page[so];
    return cf;
  }
  __device__ static __forceinline__ void store(uint8_t* tile, int r, int sw, int lane, const i32x4& v, int se,
                                               bool cf) {
    uint8_t* row = tile + r * RS;
    if constexpr (SF == CF) {
      RowFmt<SF>::store(row, sw, lane, v, se);
    } else {
      // the row's source is wave-uniform (a scalar branch)
      if (cf) RowFmt<CF>::store(row, sw, lane, v, se);
      else RowFmt<SF>::store(row, sw, lane, v, se);
    }
  }
};

// ---------------------------------------------------------------- online softmax
// Each head keeps a reference max m_ref (base 2): probabilities are exp2(x - m_ref), and the
// accumulators are rescaled only when a block's max exceeds m_ref by more than kLazyBlock; the
// new reference is then the block max if it is more than kLazy above the old one. Probabilities
// stay below 2^kLazyBlock, exact enough in bf16 and far from float32 overflow, and the rescale
// (a multiply of every accumulator) is rare.
constexpr float kLazy = 8.f;
constexpr float kLazyBlock = 32.f;

// A merge's sink logit of head h in log2 units (-inf without sinks), from a load issued
// whether or not there are sinks (a zero word without), so that it goes out with the partials'
// loads instead of behind a branch and a wait of its own.
__device__ __forceinline__ float merge_sink2(const AttnArgs& a, int h) {
  const float v = *(a.sink ? a.sink + h : reinterpret_cast<const float*>(g_zero_row));
  return a.sink ? v * kLog2e : kNegInf;
}

// Final (m, l) of one head with the optional sink, its logit s2 already loaded (in log2 units;
// -inf when there is none); returns the factor to apply to O.
__device__ __forceinline__ float finish_head_s2(float s2, float& m, float& l) {
  const float mm = fmaxf(m, s2);
  if (mm == kNegInf || s2 == kNegInf) return 1.f;
  const float f = __builtin_amdgcn_exp2f(m - mm);
  l = l * f + __builtin_amdgcn_exp2f(s2 - mm);
  m = mm;
  return f;
}

__device__ __forceinline__ float lse_of(float m, float l) {
  return l > 0.f ? (m + __builtin_log2f(l)) * 0.6931471805599453f : kNegInf;
}

// Merge the split partials of one query head: a block is (query, head); its four waves take
// every fourth split (wave w: splits w, w + 4, ...), each lane D/64 columns, and the waves' merged
// parts are combined through LDS. A partial row holds that split's sums of p * v with p relative
// to its own reference max, unnormalised (bf16), and ws_ml its (max, sum of p) in log2 units; the
// merge weights split s by 2^(max_s - max) and its sum likewise. A wave takes U of its splits at a time (U >= nsplit / 4 when nsplit
// <= 4 U), every load of a batch issued at a clamped split index before any is used (a load
// under a condition would be a branch, and each branch a wait for that load alone), merged
// online: one memory latency per batch.
template <int D, int U>
__global__ __launch_bounds__(kThreads) void mla_combine_kernel(AttnArgs a) {
  constexpr int PER = D / 64;                       // 8 (one 16-byte load) or 2 (4 bytes)
  constexpr int NW = kThreads / 64;
  __shared__ float wpart[NW][D];
  __shared__ float wml[NW][2];
  const int t = blockIdx.x, h = blockIdx.y, wave = threadIdx.x >> 6;
  const float sink2 = merge_sink2(a, h);
  const int c0 = (threadIdx.x & 63) * PER;
  const int64_t pbase = ((int64_t)(t * a.n_h16 + h / 16) * a.nsplit) * 16 + (h & 15);  // split 0
  const int ns = a.nsplit, mine = (ns - wave + NW - 1) / NW;   // splits wave, wave + NW, ...
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;
  float Ms = kNegInf, Ls = 0.f;
  for (int j0 = 0; j0 < mine; j0 += U) {
    float ms[U], ls[U];
    uint32_t v[U][PER / 2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(wave + NW * (j0 + u), ns - 1);
      const int64_t pr = pbase + (int64_t)sp * 16;
      ms[u] = a.ws_ml[pr * 2];
      ls[u] = a.ws_ml[pr * 2 + 1];
      const uint16_t* src = a.ws_o + pr * D + c0;
      if constexpr (PER == 8) {
        const i32x4 w = *(const i32x4*)src;
        v[u][0] = w.x; v[u][1] = w.y; v[u][2] = w.z; v[u][3] = w.w;
      } else {
        v[u][0] = *(const uint32_t*)src;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) ls[u] = j0 + u < mine ? ls[u] : 0.f;   // past this wave's last split
    float mb = Ms;
#pragma unroll
    for (int u = 0; u < U; ++u) mb = ls[u] > 0.f ? fmaxf(mb, ms[u]) : mb;
    // (no early exit when mb = -inf: everything below then multiplies by 0, and a branch here let
    // the compiler move the row loads behind the wait for the (max, sum) loads)
    const float r = Ms == kNegInf || mb == kNegInf ? 0.f : __builtin_amdgcn_exp2f(Ms - mb);
    Ls *= r;
#pragma unroll
    for (int c = 0; c < PER; ++c) acc[c] *= r;
    Ms = mb;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a split's partial rows are its sums relative to its own max (unnormalised)
      const float f = ls[u] > 0.f ? __builtin_amdgcn_exp2f(ms[u] - Ms) : 0.f;
      Ls += f * ls[u];
#pragma unroll
      for (int c = 0; c < PER / 2; ++c) {
        acc[2 * c] += f * __uint_as_float(v[u][c] << 16);
        acc[2 * c + 1] += f * __uint_as_float(v[u][c] & 0xffff0000u);
      }
    }
  }
  // the waves' parts: (max, sum) and the unnormalised sums relative to their own max
#pragma unroll
  for (int c = 0; c < PER; ++c) wpart[wave][c0 + c] = acc[c];
  if ((threadIdx.x & 63) == 0) {
    wml[wave][0] = Ms;
    wml[wave][1] = Ls;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) M = wml[w][1] > 0.f ? fmaxf(M, wml[w][0]) : M;
  float L = 0.f, o[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) o[c] = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float f = wml[w][1] > 0.f ? __builtin_amdgcn_exp2f(wml[w][0] - M) : 0.f;
    L += f * wml[w][1];
#pragma unroll
    for (int c = 0; c < PER; ++c) o[c] += f * wpart[w][c0 + c];
  }
  const float f = finish_head_s2(sink2, M, L);
  const float inv = L > 0.f ? f / L : 0.f;
  uint16_t* orow = a.out + ((int64_t)t * a.H + h) * D + c0;
#pragma unroll
  for (int c = 0; c < PER; c += 2) *(uint32_t*)(orow + c) = pack_bf16x2(o[c] * inv, o[c + 1] * inv);
  if (a.lse && (threadIdx.x & 63) == 0) a.lse[(int64_t)t * a.H + h] = lse_of(M, L);
}

// The split merge with one wave per (query, head), for at most four splits: the wave loads every
// split of its head at once (all loads issued before any is used), merges them and writes the
// head's output; four heads per workgroup, no LDS and no barrier. (Measured at HCA decode, four
// splits: merge 0.6 us faster than mla_combine_kernel; at five splits and more the four-wave
// merge is faster.)
template <int D, int U>
__global__ __launch_bounds__(256) void mla_combine_wave_kernel(AttnArgs a) {
  constexpr int PER = D / 64;
  const int t = blockIdx.x, h = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (h >= a.H) return;
  const float sink2 = merge_sink2(a, h);
  const int c0 = (threadIdx.x & 63) * PER;
  const int64_t pbase = ((int64_t)(t * a.n_h16 + h / 16) * a.nsplit) * 16 + (h & 15);  // split 0
  const int ns = a.nsplit;
  float acc[PER];
#pragma unroll
  for (int c = 0; c < PER; ++c) acc[c] = 0.f;
  float Ms = kNegInf, Ls = 0.f;
  for (int j0 = 0; j0 < ns; j0 += U) {
    float ms[U], ls[U];
    uint32_t v[U][PER / 2];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(j0 + u, ns - 1);
      const int64_t pr = pbase + (int64_t)sp * 16;
      ms[u] = a.ws_ml[pr * 2];
      ls[u] = a.ws_ml[pr * 2 + 1];
      const uint16_t* src = a.ws_o + pr * D + c0;
      if constexpr (PER == 8) {
        const i32x4 w = *(const i32x4*)src;
        v[u][0] = w.x; v[u][1] = w.y; v[u][2] = w.z; v[u][3] = w.w;
      } else {
        v[u][0] = *(const uint32_t*)src;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) ls[u] = j0 + u < ns ? ls[u] : 0.f;
    float mb = Ms;
#pragma unroll
    for (int u = 0; u < U; ++u) mb = ls[u] > 0.f ? fmaxf(mb, ms[u]) : mb;
    // (no early exit when mb = -inf, as in mla_combine_kernel)
    const float r = Ms == kNegInf || mb == kNegInf ? 0.f : __builtin_amdgcn_exp2f(Ms - mb);
    Ls *= r;
#pragma unroll
    for (int c = 0; c < PER; ++c) acc[c] *= r;
    Ms = mb;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // a split's partial rows are its sums relative to its own max (unnormalised)
      const float f = ls[u] > 0.f ? __builtin_amdgcn_exp2f(ms[u] - Ms) : 0.f;
      Ls += f * ls[u];
#pragma unroll
      for (int c = 0; c < PER / 2; ++c) {
        acc[2 * c] += f * __uint_as_float(v[u][c] << 16);
        acc[2 * c + 1] += f * __uint_as_float(v[u][c] & 0xffff0000u);
      }
    }
  }
  const float f = finish_head_s2(sink2, Ms, Ls);
  const float inv = Ls > 0.f ? f / Ls : 0.f;
  uint16_t* orow = a.out + ((int64_t)t * a.H + h) * D + c0;
#pragma unroll
  for (int c = 0; c < PER; c += 2) *(uint32_t*)(orow + c) = pack_bf16x2(acc[c] * inv, acc[c + 1] * inv);
  if (a.lse && (threadIdx.x & 63) == 0) a.lse[(int64_t)t * a.H + h] = lse_of(Ms, Ls);
}

// ================================================================ all-heads kernel (bf16)
// A block is (query, split of its rows, 64 heads), so every gathered row is read once for all
// heads of the query. Rows go from the paged cache straight into a ring of four 32-row LDS
// tiles with global_load_lds (no registers; the chunk swizzle is applied to the source
// addresses), from a table of row byte addresses built once per block.
// The eight waves have two roles, one of each per SIMD, and work on consecutive row blocks at
// the same time, so that one role's MFMAs cover the other's LDS waits:
//   S waves (0..3), in head pairs: wave w holds q of heads 32 (w >> 1) .. +31 in registers and
//     computes S^T for rows 16 (w & 1) .. +15 of block i (each K fragment read from LDS feeds two
//     MFMAs), agrees on the block's per-head maxima with its partner, runs the online softmax
//     and writes P^T (bf16) and any rescale factors to LDS;
//   O waves (4..7): wave 4+c accumulates O^T for output columns D/4 * c .. +D/4 of all 64
//     heads over block i-1, from that block's tile and P^T, and issues the row copies.
// While block i is scored and block i-1 accumulated, the rows of blocks i+1 and i+2 are in
// flight into the other two tiles. Each role runs its own loop (so q and the O accumulators are
// never live in the same wave) and both pass one barrier per block.
constexpr int kHeadsThreads = 512;

// s_waitcnt vmcnt(n) (gfx9 encoding, n < 16): expcnt and lgkmcnt not waited for
#define HCS_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

template <int D, bool SEL, int SF = HCS_FMT_BF16, int CF = HCS_FMT_BF16>
__global__ __launch_bounds__(kHeadsThreads, 1) void mla_heads_kernel(AttnArgs a) {
  constexpr bool QR = SF != HCS_FMT_BF16;         // quantized rows, dequantised through registers
  static_assert(!QR || (D == 512 && !SEL), "quantized rows are 512 wide, bf16 selection only");
  constexpr int RS = D * 2, KS = D / 32;
  constexpr int BT = 32;                          // rows per block
  constexpr int TB = BT * RS;                     // bytes per tile
  constexpr int CTO = D / 16 / 4;                 // 16-column output tiles per O wave
  constexpr int PR = BT + 8;                      // P row stride (elements), padded
  constexpr int RPI = 1024 / RS;                  // rows per 1 KiB async load
  constexpr int LPR = 64 / RPI;                   // lanes per row in an async load
  constexpr int WRL = BT / 8;                     // quantized rows each wave stages per block
  constexpr int WRO = BT / 4;                     // rows each O wave copies per block
  constexpr int NLO = WRO / RPI;                  // async loads per O wave per block
  constexpr int PD = 4;                           // K-fragment steps read ahead in S^T
  static_assert(CTO >= 1 && NLO >= 1 && NLO < 16 && KS % PD == 0, "unsupported head dim");
  static_assert(!SEL || 2 * TB >= kSelScratch, "the row selection's scratch lives in tiles 0-1");
  // Tiles in the ring: bf16 rows are copied two blocks ahead (four tiles: S on block i, O on
  // block i-1, copies of i+1 and i+2 in flight); quantized rows are staged one block ahead in
  // registers and stored at the top of their step (three tiles), and the LDS this frees holds a
  // longer page-table row (4096 pages: a 1M-token sequence's compressed cache).
  constexpr int NTL = QR ? 3 : 4;
  constexpr int PTC = QR ? 2 * kPtCache : kPtCache;
  // tiles 2 and 3 first hold q of the 64 heads (64 rows of RS bytes)
  __shared__ __attribute__((aligned(16))) uint8_t tiles[NTL * TB];
  __shared__ __attribute__((aligned(16))) uint32_t rowtab[kMaxRowsWG];
  __shared__ int ptl[PTC];
  __shared__ __attribute__((aligned(16))) __bf16 p_lds[2][64 * PR];
  __shared__ float alpha_lds[2][64];
  __shared__ __attribute__((aligned(16))) int flags[2][4];
  __shared__ float hm[64], hl[2][64];
  __shared__ float pmax[4][32];                   // S waves' block maxima, per head pair
  __shared__ int pseq[4];                         // S waves' step counters

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, l16 = lane & 15;
  const int G = a.nsplit * a.n_hg;
  const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3;
  const int t = (r / G) * 8 + xcd;
  if (t >= a.N) return;
  const int j = r - (r / G) * G;
  const int s = j / a.n_hg, hg = j - (j / a.n_hg) * a.n_hg;
  const int hbase = hg * 64;

  const QueryRows q = query_rows(a, t);
  const int r0 = s * a.rows_per_split;
  const int n_rows = max(0, min(q.R, r0 + a.rows_per_split) - r0);
  uint8_t* const qstage = tiles + (NTL - 2) * TB;  // the last two tiles (rows reach them after the
                                                  // S waves have read q, at the first barrier)
  // q of the block's 64 heads: one contiguous row per head, copied into tiles 2-3 by async
  // loads (wave w: heads 8w..8w+7, chunk c of head h stored at c ^ (h mod 16)); the S waves read
  // it into registers before the first barrier of the block loop, and tile 2 receives rows only
  // after that barrier.
  {
    constexpr int QLPR = RS / 16;                  // lanes per head row in one load
    constexpr int QHPI = 64 / QLPR;                // heads per load
#pragma unroll
    for (int i = 0; i < 8 / QHPI; ++i) {
      const int hl_ = 8 * wave + i * QHPI + lane / QLPR;
      const int hh = hbase + hl_;
      const uint8_t* src = hh < a.H ? reinterpret_cast<const uint8_t*>(a.q + ((int64_t)t * a.H + hh) * D)
                                    : g_zero_row;
      const int ch = (lane % QLPR) ^ (hl_ & 15);
      dma16v(src + ch * 16, lds_addr(qstage) + (8 * wave + i * QHPI) * RS);
    }
  }
  if (tid < 4) pseq[tid] = 0;                     // ordered by the row table's barriers
  if constexpr (SEL) {
    if (q.nv <= 4 * kHeadsThreads) fill_rows_sel<kHeadsThreads, 4>(a, t, s, q, r0, n_rows, rowtab, ptl, BT, tiles);
    else if (q.nv <= 8 * kHeadsThreads) fill_rows_sel<kHeadsThreads, 8>(a, t, s, q, r0, n_rows, rowtab, ptl, BT, tiles);
    else fill_rows_sel<kHeadsThreads, 16>(a, t, s, q, r0, n_rows, rowtab, ptl, BT, tiles);
  }
  else fill_rows<kHeadsThreads, PTC>(a, t, q, r0, n_rows, rowtab, ptl, BT);
  const int nblk = (n_rows + BT - 1) / BT;

  // async loads: O wave 4 + ow fills rows WRO ow .. +WRO-1 of a block; LDS chunk slot c of row r
  // receives source chunk c ^ swz_dec(r mod 16)
  auto row_ptr = [&](uint32_t e) {
    return e != kNoRow ? ((e >> 31) ? a.comp.base : a.swa.base) + (size_t)(e & 0x7fffffffu) * RS
                       : g_zero_row;
  };
  // A block's copies in two halves: the source addresses come from the row table (fixed after
  // the prologue), so they are read before a step's waits; the copies themselves are issued
  // after its barrier, once their tile is free. RPI == 1: one row per copy, the address
  // wave-uniform; otherwise each lane has its own row's address. The O waves issue them all: they
  // finish each step early and wait at its barrier, while the S waves' chain (S^T, maxima, pair
  // wait, probabilities) sets the step time (prefill attention 1336 -> 1295 us against copies on
  // all eight waves).
  struct RowSrcO { const uint8_t* p[NLO]; };
  auto prep_o = [&](int b) {
    RowSrcO r;
    const int ow = wave - 4;
    const uint32_t* at = rowtab + b * BT + WRO * ow;
    if constexpr (RPI == 1) {
      const uint32_t my = at[lane & (WRO - 1)];
#pragma unroll
      for (int i = 0; i < NLO; ++i) r.p[i] = row_ptr((uint32_t)__builtin_amdgcn_readlane((int)my, i));
    } else {
#pragma unroll
      for (int i = 0; i < NLO; ++i) {
        const int rl = i * RPI + lane / LPR;
        const int sw = swz_dec((WRO * ow + rl) & 15);
        r.p[i] = row_ptr(at[rl]) + (((lane % LPR) ^ sw) * 16);
      }
    }
    return r;
  };
  auto fire_o = [&](int b, const RowSrcO& r) {
    const int ow = wave - 4;
    uint8_t* tb = tiles + (b & 3) * TB;
#pragma unroll
    for (int i = 0; i < NLO; ++i) {
      if constexpr (RPI == 1) {
        const int sw = swz_dec((WRO * ow + i) & 15);
        dma16(r.p[i], (uint32_t)((lane ^ sw) * 16), lds_addr(tb) + (WRO * ow + i) * RS);
      } else {
        dma16v(r.p[i], lds_addr(tb) + (WRO * ow + i * RPI) * RS);
      }
    }
  };
  // Quantized rows: wave w loads rows WRL w .. +WRL-1 of block i+1 into registers (16 bytes and a
  // scale byte per lane, the same load shape for every format) during step i, and writes them
  // dequantised to bf16 into the block's tile, chunk-swizzled as the copies above, at the top of
  // step i+1; tile i mod 4 was last read by the O waves three steps before.
  using QS = QuantStage<QR ? SF : HCS_FMT_FP8DS, QR ? CF : HCS_FMT_FP8DS>;
  i32x4 qv[QR ? WRL : 1];
  int qsc[QR ? WRL : 1];
  uint32_t qcf = 0;
  auto qload = [&](int b) {
    if constexpr (QR) {
      const uint32_t my = rowtab[b * BT + WRL * wave + (lane & (WRL - 1))];
      qcf = 0;
#pragma unroll
      for (int i = 0; i < WRL; ++i)
        qcf |= (QS::load(a.swa.base, a.comp.base, (uint32_t)__builtin_amdgcn_readlane((int)my, i), lane, qv[i],
                         qsc[i]) ? 1u : 0u) << i;
    }
  };
  auto qstore = [&](int b) {
    if constexpr (QR) {
      uint8_t* tb = tiles + (b % NTL) * TB;
#pragma unroll
      for (int i = 0; i < WRL; ++i) {
        const int r = WRL * wave + i;
        QS::store(tb, r, swz_dec(r & 15), lane, qv[i], qsc[i], (qcf >> i) & 1u);
      }
    }
  };
  if constexpr (QR) {
    if (nblk > 0) qload(0);
  } else {
    if (wave >= 4) {
      if (nblk > 0) fire_o(0, prep_o(0));
      if (nblk > 1) fire_o(1, prep_o(1));
    }
  }
  // top of block step i: the O waves' copies of block i have landed (those of block i+1 may
  // still be in flight), then the barrier makes them and the previous step's LDS writes
  // visible, and block i+2's copies go into the tile that block i-2 left
  auto step_sync = [&](int i) {
    if constexpr (QR) {
      if (i < nblk) {
        qstore(i);
        if (i + 1 < nblk) qload(i + 1);
      }
      lds_barrier();
    } else {
      if (wave >= 4) {
        RowSrcO r{};
        if (i + 2 < nblk) r = prep_o(i + 2);
        if (i + 1 < nblk) HCS_WAIT_VMCNT(NLO);
        else wait_vm_zero();
        lds_barrier();
        if (i + 2 < nblk) fire_o(i + 2, r);
      } else {
        lds_barrier();
      }
    }
  };

  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const bool split = a.nsplit > 1;
  if (wave < 4) {
    {
      // ================= S waves: wave w takes heads hbase + 32 (w >> 1) + 16 nt + l16 (nt = 0, 1)
      // over rows 16 (w & 1) .. +15 of each block, so each K fragment read from LDS feeds two
      // MFMAs. The two waves of a head pair agree on each block's max per head before either
      // writes its probabilities: each publishes its maxima and a step counter in LDS and waits
      // for its partner's (a bounded wait; both waves are resident in this workgroup).
      const int hp = wave >> 1, rh = wave & 1, partner = wave ^ 1;
      bf16x8 qreg[2][KS];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qreg[nt][ks] = *(const bf16x8*)(qstage + (32 * hp + 16 * nt + l16) * RS + (((4 * ks + g) ^ l16) << 4));
      // K row 16 rh + l16, chunk (4ks + g) ^ s = 4 (ks ^ (s >> 2)) + ((g ^ s) & 3), s = swz_dec(l16)
      const int sk = swz_dec(l16);
      int ko4[4];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) ko4[k4] = (16 * rh + l16) * RS + ((g ^ sk) & 3) * 16 + 64 * (k4 ^ (sk >> 2));
      float m_ref[2] = {kNegInf, kNegInf}, l_part[2] = {0.f, 0.f};
      for (int i = 0; i <= nblk; ++i) {
        step_sync(i);
        if (i == nblk) break;
        const uint8_t* T = tiles + (i % NTL) * TB;
        const int pb = i & 1;
        const uint32_t valid = (uint32_t)__ballot(rowtab[i * BT + 16 * rh + (lane & 15)] != kNoRow) & 0xFFFFu;
        // ---- S^T[16 rows][32 heads], K fragments read PD k-steps ahead of their MFMAs
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        bf16x8 kf[PD];
        auto kload = [&](int ks) { return *(const bf16x8*)(T + ko4[ks & 3] + (ks >> 2) * 256); };
#pragma unroll
        for (int ks = 0; ks < PD; ++ks) kf[ks] = kload(ks);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
            sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks % PD], qreg[nt][ks], sacc[nt], 0, 0, 0);
          if (ks + PD < KS) kf[ks % PD] = kload(ks + PD);
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- online softmax: lane (g, l16) holds rows 4g .. 4g+3 of this wave's 16 for head
        // 32 hp + 16 nt + l16
        float x[2][4], tmax[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          tmax[nt] = kNegInf;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[nt][e] = ((valid >> (4 * g + e)) & 1u) ? sacc[nt][e] * a.scale_log2 : kNegInf;
            tmax[nt] = fmaxf(tmax[nt], x[nt][e]);
          }
          tmax[nt] = max_xor16_32(tmax[nt]);
        }
        // the partner wave's maxima of block i (LDS operations of one wave complete in order, so
        // a partner step count of i + 1 means its maxima of block i are in place)
        if (g == 0) {
          pmax[wave][l16] = tmax[0];
          pmax[wave][16 + l16] = tmax[1];
        }
        if (lane == 0) pseq[wave] = i + 1;
        // (a tight spin: an s_sleep between the reads made the wake-up later by up to its 64
        // clocks, 3% of a prefill chunk's attention; the partner is a block phase away at most)
        // (LDS atomic loads: a volatile access through a generic pointer would be a flat load,
        // whose wait also covers every copy in flight)
        bool met = false;
        for (int spin = 0; spin < (1 << 16) && !met; ++spin)
          met = __builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(&pseq[partner], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) > i;
        // a wait that ran out goes on with this wave's own maxima (a wrong result, reported)
        if (!met && lane == 0) dev_error(HCS_DEVERR_PAIR_WAIT);
        tmax[0] = fmaxf(tmax[0], __hip_atomic_load(&pmax[partner][l16], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        tmax[1] = fmaxf(tmax[1], __hip_atomic_load(&pmax[partner][16 + l16], __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          // the same decision in both waves of the pair (same maxima, same history)
          const bool any_over = __any(tmax[nt] > m_ref[nt] + kLazyBlock);
          if (any_over) {
            // rare: new reference maxima for these heads
            const float mnew = tmax[nt] > m_ref[nt] + kLazy ? tmax[nt] : m_ref[nt];
            // 0 when m_ref = -inf; 1 for a head with no row yet (-inf - -inf would be NaN)
            const float alpha = mnew == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_ref[nt] - mnew);
            l_part[nt] *= alpha;
            m_ref[nt] = mnew;
            if (rh == 0 && g == 0) alpha_lds[pb][32 * hp + 16 * nt + l16] = alpha;
          }
          if (rh == 0 && lane == 0) flags[pb][2 * hp + nt] = any_over ? 1 : 0;
          const float mr = m_ref[nt] == kNegInf ? 0.f : m_ref[nt];
          bf16x4 p4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pv = __builtin_amdgcn_exp2f(x[nt][e] - mr);
            l_part[nt] += pv;
            p4[e] = (__bf16)pv;
          }
          *(bf16x4*)(p_lds[pb] + (32 * hp + 16 * nt + l16) * PR + 16 * rh + 4 * g) = p4;
        }
      }
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float lt = sum_xor16_32(l_part[nt]);
        if (g == 0) {
          hl[rh][32 * hp + 16 * nt + l16] = lt;
          if (rh == 0) hm[32 * hp + 16 * nt + l16] = m_ref[nt];
        }
      }
    }
    lds_barrier();                                  // (E1) per-head (max, sum) published
    lds_barrier();                                  // (E2) O waves have staged the output
  } else {
    // ================= O waves: output columns D/4 * ow .. +D/4 of all 64 heads
    const int ow = wave - 4;
    f32x4 oacc[CTO][4];
#pragma unroll
    for (int ct = 0; ct < CTO; ++ct)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) oacc[ct][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // V^T rows 8g + jv and 8g + 4 + jv: swz_dec = 2 jv + 8 (g & 1) (+1), so chunk (2 ctg + h)
    // lands at 2 (ctg ^ (jv + 4 (g & 1))) + (h, resp. h ^ 1)
    const int jv = l16 >> 2, q4 = l16 & 3, h2 = q4 >> 1;
    const int vx = jv + 4 * (g & 1);
    const int vrow = (8 * g + jv) * RS + (q4 & 1) * 8;
    for (int i = 0; i <= nblk; ++i) {
      step_sync(i);
      if (i == 0) continue;
      const int b = i - 1;
      const uint8_t* T = tiles + (b % NTL) * TB;
      const int pb = b & 1;
      // the S waves' rescale flags of block b (one read), issued with the operand reads below
      const i32x4 fl = *reinterpret_cast<const i32x4*>(&flags[pb][0]);
      auto vload = [&](int ct) {
        const int ctg = ow * CTO + ct;
        const uint8_t* vb = T + vrow + 32 * ((ctg & 7) ^ vx) + (ctg >> 3) * 256;
        const i16x4 v0 = lds_read_tr16(vb + 16 * h2);
        const i16x4 v1 = lds_read_tr16(vb + 4 * RS + 16 * (h2 ^ 1));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 pbf[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) pbf[nt] = *(const bf16x8*)(p_lds[pb] + (16 * nt + l16) * PR + 8 * g);
      constexpr int VD = CTO < 2 ? CTO : 2;         // V^T fragments read ahead
      bf16x8 vf[VD];
#pragma unroll
      for (int ct = 0; ct < VD; ++ct) vf[ct] = vload(ct);
      // rescale the heads whose reference max moved in block b (rare)
      if (fl.x | fl.y | fl.z | fl.w) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (fl[nt]) {
            const float al = alpha_lds[pb][16 * nt + l16];
#pragma unroll
            for (int ct = 0; ct < CTO; ++ct) oacc[ct][nt] *= al;
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < CTO; ++ct) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 v = vf[ct % VD];
        if (ct + VD < CTO) vf[ct % VD] = vload(ct + VD);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          oacc[ct][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v, pbf[nt], oacc[ct][nt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // sink logits (log2 units) of the heads this lane finishes, hbase + 16 nt + l16, loaded before
    // any store is issued (a load wait also waits for earlier stores)
    float sink2[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int hh = hbase + 16 * nt + l16;
      sink2[nt] = a.sink && hh < a.H && !split ? a.sink[hh] * kLog2e : kNegInf;
    }
    lds_barrier();                                  // (E1)
    // The result goes through LDS so that each global store writes whole rows: lane holds
    // O^T[c = 16 (ow * CTO + ct) + 4g + e][head 16 nt + l16]; in LDS (tiles 0-1, free now), row h
    // holds head h with its 16-byte chunks XOR-swizzled by h mod 16 (conflict-free for both the
    // scattered writes here and the row reads below). Whole rows then go to `out` (normalised,
    // with the sink) or, when the rows are split, to this split's partial rows: its unnormalised
    // sums relative to its reference max, with that (max, sum) in ws_ml for the merge, so the
    // staging of a split's rows waits for neither the per-head sums nor a division.
    auto stage = [&](int nt, float inv, bool scale) {
      uint8_t* hrow = tiles + (16 * nt + l16) * RS;
#pragma unroll
      for (int ct = 0; ct < CTO; ++ct) {
        const f32x4 o = scale ? oacc[ct][nt] * inv : oacc[ct][nt];
        uint2 pk;
        pk.x = pack_bf16x2(o[0], o[1]);
        pk.y = pack_bf16x2(o[2], o[3]);
        const int cb = (16 * (ow * CTO + ct) + 4 * g) * 2;           // byte in the row
        *(uint2*)(hrow + ((((cb >> 4) ^ l16) << 4) | (cb & 15))) = pk;
      }
    };
    if (split) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) stage(nt, 1.f, false);
      if (ow == 0 && g == 0) {                      // lanes 0-15 of the first O wave
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int hh = hbase + 16 * nt + l16;
          if (hh < a.H) {
            const int64_t prow16 = ((int64_t)(t * a.n_h16 + hh / 16) * a.nsplit + s) * 16 + (hh & 15);
            a.ws_ml[prow16 * 2 + 0] = hm[16 * nt + l16];
            a.ws_ml[prow16 * 2 + 1] = hl[0][16 * nt + l16] + hl[1][16 * nt + l16];
          }
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int hh = hbase + 16 * nt + l16;
        float M = hm[16 * nt + l16], L = hl[0][16 * nt + l16] + hl[1][16 * nt + l16];
        const float f = finish_head_s2(sink2[nt], M, L);
        const float inv = L > 0.f ? f / L : 0.f;
        if (a.lse && g == 0 && ow == 0 && hh < a.H) a.lse[(int64_t)t * a.H + hh] = lse_of(M, L);
        stage(nt, inv, true);
      }
    }
    lds_barrier();                                  // (E2): LDS only, the partials' (max, sum)
                                                    // stores need no wait inside this kernel
  }
  constexpr int LPH = RS / 16;                       // lanes per head row
  constexpr int HPI = 64 / LPH;                      // heads per wave instruction
  i32x4 v[8 / HPI];
#pragma unroll
  for (int k = 0; k < 8 / HPI; ++k) {
    const int hl_ = wave * 8 + k * HPI + lane / LPH, ch = lane % LPH;
    v[k] = *(const i32x4*)(tiles + hl_ * RS + ((ch ^ (hl_ & 15)) << 4));
  }
#pragma unroll
  for (int k = 0; k < 8 / HPI; ++k) {
    const int hl_ = wave * 8 + k * HPI + lane / LPH, ch = lane % LPH;
    const int hh = hbase + hl_;
    if (hh >= a.H) continue;
    uint16_t* dst = split ? a.ws_o + (((int64_t)(t * a.n_h16 + hh / 16) * a.nsplit + s) * 16 + (hh & 15)) * D
                          : a.out + ((int64_t)t * a.H + hh) * D;
    // streaming stores: the rows are read next by another launch (the merge) or not at all, so
    // they need not stay in this XCD's L2 (CSA decode step 0.3 us faster than plain stores)
    __builtin_nontemporal_store(v[k], (i32x4*)(reinterpret_cast<uint8_t*>(dst) + ch * 16));
  }
}

template <int D, int SF, int CF>
hipError_t launch_impl(const AttnArgs& a, hipStream_t stream) {
  const int n8 = (a.N + 7) / 8;
  dim3 grid((unsigned)(n8 * 8 * a.nsplit * a.n_hg));
  // (The S waves work in head pairs at decode too: once they issued no row copies and their wait
  // became a plain LDS read, half the K reads from LDS paid for the per-block exchange of
  // maxima there as well: HCA step 34.8 -> 33.5 us.)
  if constexpr (SF == HCS_FMT_BF16) {
    if (!a.scores) {
      hipLaunchKernelGGL((mla_heads_kernel<D, false>), grid, dim3(kHeadsThreads), 0, stream, a);
    } else if constexpr (D == 512) {
      hipLaunchKernelGGL((mla_heads_kernel<D, true>), grid, dim3(kHeadsThreads), 0, stream, a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    static_assert(D == QuantStage<SF, CF>::D, "quantized rows are 512 wide");
    hipLaunchKernelGGL((mla_heads_kernel<D, false, SF, CF>), grid, dim3(kHeadsThreads), 0, stream, a);
  }
  if (a.nsplit > 1) {
    const dim3 cg(a.N, a.H);
    if (a.nsplit <= 4)
      hipLaunchKernelGGL((mla_combine_wave_kernel<D, 4>), dim3(a.N, (a.H + 3) / 4), dim3(256), 0, stream, a);
    else if (a.nsplit <= 8) hipLaunchKernelGGL((mla_combine_kernel<D, 2>), cg, dim3(kThreads), 0, stream, a);
    else if (a.nsplit <= 16) hipLaunchKernelGGL((mla_combine_kernel<D, 4>), cg, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((mla_combine_kernel<D, 8>), cg, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int N, int H, int d, int window, int m, int topk, int max_pos) {
  AttnPlan p{};
  const int64_t nv = (int64_t)(max_pos + 1) / m;
  const int64_t rows = (int64_t)std::min(window, max_pos + 1) + (topk > 0 ? topk : nv);
  // 64 heads per kernel block (the all-heads kernel, every row format), 32 rows per row block;
  // splits are whole row blocks
  p.n_hg = (H + 63) / 64;
  p.n_h16 = (H + 15) / 16;
  const int64_t kBlock = 32;
  const int64_t blocks = std::max<int64_t>(1, (rows + kBlock - 1) / kBlock);
  const int64_t max_bps = kMaxRowsWG / kBlock;
  const int64_t per_split = (int64_t)((N + 7) / 8) * 8 * p.n_hg;
  // enough splits to give every CU a block, but at least two blocks each: a split adds 64 KiB of
  // partial stores and merge reads per query (measured at the decode configurations: CSA seven
  // splits of three blocks against five of four, 0.4 us faster; at 1M 23 splits of three against
  // 17 of four, 1.4 us faster)
  const int64_t min_bps = 2;
  int64_t nsplit = std::max<int64_t>(1, (256 + per_split - 1) / per_split);
  nsplit = std::min(nsplit, std::max<int64_t>(1, blocks / min_bps));
  nsplit = std::max<int64_t>(nsplit, (blocks + max_bps - 1) / max_bps);
  const int64_t bps = (blocks + nsplit - 1) / nsplit;
  nsplit = (blocks + bps - 1) / bps;
  p.nsplit = (int)nsplit;
  p.rows_per_split = (int)(bps * kBlock);
  if (nsplit > 1) {
    const size_t parts = (size_t)N * p.n_h16 * nsplit * 16;
    p.ws_o_bytes = parts * d * sizeof(uint16_t);
    p.ws_ml_bytes = parts * 2 * sizeof(float);
    p.ws_bytes = p.ws_o_bytes + p.ws_ml_bytes;
  }
  return p;
}

bool attn_formats_supported(int d, int swa_fmt, int comp_fmt) {
  if (swa_fmt == HCS_FMT_BF16) return comp_fmt == HCS_FMT_BF16 && (d == 512 || d == 128);
  if (d != 512) return false;
  return (swa_fmt == HCS_FMT_FP8DS && comp_fmt == HCS_FMT_FP8DS) ||
         (swa_fmt == HCS_FMT_MXFP8 && (comp_fmt == HCS_FMT_MXFP8 || comp_fmt == HCS_FMT_NVFP4));
}

hipError_t launch_sparse_mla(const AttnArgs& a, int d, int swa_fmt, int comp_fmt, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  if (d == 512 && swa_fmt == HCS_FMT_BF16) return launch_impl<512, HCS_FMT_BF16, HCS_FMT_BF16>(a, stream);
  if (d == 128 && swa_fmt == HCS_FMT_BF16) return launch_impl<128, HCS_FMT_BF16, HCS_FMT_BF16>(a, stream);
  if (d == 512 && swa_fmt == HCS_FMT_FP8DS && comp_fmt == HCS_FMT_FP8DS)
    return launch_impl<512, HCS_FMT_FP8DS, HCS_FMT_FP8DS>(a, stream);
  if (d == 512 && swa_fmt == HCS_FMT_MXFP8 && comp_fmt == HCS_FMT_MXFP8)
    return launch_impl<512, HCS_FMT_MXFP8, HCS_FMT_MXFP8>(a, stream);
  if (d == 512 && swa_fmt == HCS_FMT_MXFP8 && comp_fmt == HCS_FMT_NVFP4)
    return launch_impl<512, HCS_FMT_MXFP8, HCS_FMT_NVFP4>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace hcs
