// Exact top-k selection helpers shared by the indexer's selection kernels and the attention
// kernel that selects its own rows from indexer scores: radix select of the k-th largest
// order key with LDS histograms, and the emission of the selected ids (ties at the k-th key go
// to the smaller ids). Included by one translation unit each (internal linkage).
#pragma once

#include "common.h"

namespace hcs {
namespace {
// ---------------------------------------------------------------- radix select
constexpr int kDigitBits = 11;                 // radix digit: 2048 bins
constexpr int kBins = 1 << kDigitBits;

constexpr int kCandMax = 64;            // a k-th key bin this small is resolved by ranking

struct SelShared {
  unsigned hist[2][kBins];               // pass p counts into hist[p & 1]; the other is cleared
  unsigned wsum[16];                     // per-wave bin totals of a pass
  unsigned wmax[16], wmin[16], wcnt[16]; // per-wave key range and count (register-key select)
  unsigned bin, above, cnt_bin;
  unsigned kmax, kmin, count;            // range and number of the participating keys
  unsigned out_count;
  uint32_t cand_key[kCandMax];           // the keys of the k-th key's bin, and their ids
  int cand_id[kCandMax];
  unsigned cand_count;
};

// Wave-wide reductions through DPP row operations (no LDS round trips); every lane gets the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return ~wave_max_u32(~v);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Inclusive prefix sum over the 64 lanes of a wave, by DPP: within each row of 16 lanes the sums
// of the 1, 2, 3 lanes before (row_shr), then of 4 and 8 lanes before (on the banks those reach),
// then the last lane of row 0 into row 1 and of row 2 into row 3 (row_bcast:15), then the last
// lane of row 1 into rows 2-3 (row_bcast:31). Disabled and out-of-row lanes contribute 0.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  uint32_t x = v;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x113, 0xF, 0xF, true);   // row_shr:3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xE, false);  // row_shr:4, lanes 4-15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xC, false);  // row_shr:8, lanes 8-15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1, 3
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2, 3
  return x;
}

// Clears what radix_kth expects cleared; the caller puts a barrier between this and the call.
// NT is the block's thread count (a multiple of 64, 256..1024) in all the selection helpers.
template <int NT>
__device__ __forceinline__ void sel_reset(SelShared& sh) {
  for (int j = threadIdx.x; j < kBins; j += NT) sh.hist[0][j] = 0;
  if (threadIdx.x == 0) {
    sh.kmax = 0u;
    sh.kmin = ~0u;
    sh.count = 0u;
  }
}

struct KthResult {
  uint32_t prefix, mask;                 // keys with (key & mask) > prefix are above the k-th
  unsigned need, n_eq;                   // of the n_eq keys with (key & mask) == prefix, need belong
};

// Radix select of the k-th largest key among the participating elements (1 <= k <= their
// number). Keys first agree on a common leading part (the range min ^ max), so the digits start
// below it: 11 bits per pass, stopping once the bin holding the k-th key holds exactly the keys
// still needed (then every key of that bin is taken, no further digit is needed; with 2048 bins
// this is usually the first pass). One barrier for the range, three per pass. Expects
// sel_reset() state; leaves it reset (ordered by the caller's next barrier).
template <int NT, class KeyOf>
__device__ KthResult radix_kth(SelShared& sh, int n, unsigned k, KeyOf key_of, unsigned small_bin = 0) {
  static_assert(NT % 64 == 0 && NT >= 256 && NT <= 1024 && kBins % NT == 0, "block size");
  constexpr int BPT = kBins / NT;        // bins per thread in the scan
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ---- range and count of the participating keys
  uint32_t lmax = 0u, lmin = ~0u;
  unsigned lcnt = 0;
  for (int i = tid; i < n; i += NT) {
    uint32_t key;
    if (key_of(i, key)) {
      lmax = max(lmax, key);
      lmin = min(lmin, key);
      ++lcnt;
    }
  }
  lmax = wave_max_u32(lmax);
  lmin = wave_min_u32(lmin);
  lcnt = wave_sum_u32(lcnt);
  if (lane == 0) {
    atomicMax(&sh.kmax, lmax);
    atomicMin(&sh.kmin, lmin);
    atomicAdd(&sh.count, lcnt);
  }
  __syncthreads();
  const uint32_t kmax = sh.kmax, diff = kmax ^ sh.kmin;
  const unsigned total = sh.count;
  KthResult r;
  if (diff == 0u) {                      // all participating keys are equal
    __syncthreads();                     // every thread has read the range
    if (tid == 0) {
      sh.kmax = 0u;
      sh.kmin = ~0u;
      sh.count = 0u;
    }
    r.prefix = kmax;
    r.mask = ~0u;
    r.need = k;
    r.n_eq = total;
    return r;
  }
  int top = 31 - __builtin_clz(diff);    // highest bit where the keys differ
  uint32_t mask = top == 31 ? 0u : ~((2u << top) - 1u);
  uint32_t prefix = kmax & mask;
  unsigned remaining = k, cnt_bin = total;
  for (int pass = 0; top >= 0; ++pass) {
    const int width = min(kDigitBits, top + 1);
    const int shift = top - width + 1;
    unsigned* hist = sh.hist[pass & 1];
    for (int i = tid; i < n; i += NT) {
      uint32_t key;
      if (key_of(i, key) && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & (kBins - 1)], 1u);
    }
    __syncthreads();
    // thread i owns bins kBins-1-BPT*i .. kBins-BPT*i (descending); exclusive prefix of the
    // threads' totals = the wave's prefix (from ballots of the totals' bits) + earlier waves'
    unsigned c[BPT], tot = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = hist[kBins - 1 - BPT * tid - j];
      tot += c[j];
    }
    const uint64_t below = (1ull << lane) - 1;
    unsigned run = 0;
    // every thread's total is at most `total`, so its bits above nbits are zero (a fixed bit
    // count would truncate totals of large selections)
    const int nbits = 32 - __builtin_clz(total | 1u);
    for (int b = 0; b < nbits; ++b) run += (unsigned)__popcll(__ballot((tot >> b) & 1u) & below) << b;
    if (lane == 63) sh.wsum[wave] = run + tot;
    for (int j = tid; j < kBins; j += NT) sh.hist[(pass & 1) ^ 1][j] = 0;   // the next pass's
    __syncthreads();
    {
      const unsigned ws = lane < wave ? sh.wsum[lane] : 0u;   // lower waves' totals
      run += wave_sum_u32(ws);
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (run < remaining && run + c[j] >= remaining) {
        sh.bin = kBins - 1 - BPT * tid - j;
        sh.above = run;
        sh.cnt_bin = c[j];
      }
      run += c[j];
    }
    __syncthreads();
    prefix |= sh.bin << shift;
    mask |= ((1u << width) - 1u) << shift;
    remaining -= sh.above;
    cnt_bin = sh.cnt_bin;
    top = shift - 1;
    // hist[pass & 1] was counted into; clear it for a later pass or call (ordered by the
    // barriers that follow before any reuse)
    for (int j = tid; j < kBins; j += NT) hist[j] = 0;
    if (cnt_bin == remaining || cnt_bin <= small_bin) break;
  }
  if (tid == 0) {                        // range state for a later call
    sh.kmax = 0u;
    sh.kmin = ~0u;
    sh.count = 0u;
  }
  r.prefix = prefix;
  r.mask = mask;
  r.need = remaining;
  r.n_eq = cnt_bin;
  return r;
}

// The bin of the k-th largest key as a key range: keys k with k - lo <= span (k >= lo) are in
// it, keys above lo + span are above the k-th; `need` of its n_eq keys belong to the top k.
struct KthRange {
  uint32_t lo, span;
  unsigned need, n_eq;
  __device__ bool in_bin(uint32_t key) const { return key >= lo && key - lo <= span; }
  __device__ bool above(uint32_t key) const { return key >= lo && key - lo > span; }
};

// Radix select of the k-th largest key when every thread holds its keys in registers (up to IPT,
// key_at(j) the key of slot j, present when bit j of vmask is set) in a block of 512 or 1024
// threads: the key range and count come from wave reductions; the digits are taken from the
// offset key - min (so that the first pass spreads the keys over its 2048 bins by value even
// when they straddle a power of two, where a digit below the common leading bits would put
// nearly all of them in a few bins and serialise the histogram's atomics), 11 bits per pass.
// Each pass is one histogram (LDS atomics issued back to back), a wave prefix sum over the 4
// or 2 bins of each thread and the bin search, with three LDS-only barriers. The passes stop
// once the bin of the k-th key holds exactly the keys still needed, or every bit is resolved
// (then that bin holds equal keys). All present keys are taken when there are at most k of
// them (the "bin" is every key). Expects hist[0] cleared and a barrier after; leaves both
// histograms cleared (ordered by the caller's next barrier).
template <int NT, int IPT, class KeyAt>
__device__ KthRange reg_kth(SelShared& sh, KeyAt key_at, uint32_t vmask, unsigned k) {
  static_assert((NT == 512 || NT == 1024) && IPT <= 32, "512 or 1024 threads");
  constexpr int NW = NT / 64, BPT = kBins / NT;   // bins per thread in the scan: 4 or 2
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t lmax = 0u, lmin = ~0u;
  unsigned lcnt = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if ((vmask >> j) & 1u) {
      lmax = max(lmax, key_at(j));
      lmin = min(lmin, key_at(j));
      ++lcnt;
    }
  }
  lmax = wave_max_u32(lmax);
  lmin = wave_min_u32(lmin);
  lcnt = wave_sum_u32(lcnt);
  if (lane == 0) {
    sh.wmax[wave] = lmax;
    sh.wmin[wave] = lmin;
    sh.wcnt[wave] = lcnt;
  }
  lds_barrier();
  uint32_t kmax = 0u, kmin = ~0u;
  unsigned total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    kmax = max(kmax, sh.wmax[v]);
    kmin = min(kmin, sh.wmin[v]);
    total += sh.wcnt[v];
  }
  KthRange r;
  if (total <= k) {
    r.lo = 0u;
    r.span = ~0u;
    r.need = r.n_eq = total;
    return r;
  }
  if (kmax == kmin) {                    // all present keys are equal
    r.lo = kmax;
    r.span = 0u;
    r.need = k;
    r.n_eq = total;
    return r;
  }
  // the bin so far: keys lo .. lo + 2^w - 1 (w <= 32: kmax - kmin < 2^w)
  uint32_t lo = kmin;
  int w = 32 - __builtin_clz(kmax - kmin);
  unsigned remaining = k, cnt_bin = total;
  for (int pass = 0; w > 0; ++pass) {
    const int width = min(kDigitBits, w);
    const int shift = w - width;
    const uint32_t wspan = w >= 32 ? ~0u : (1u << w) - 1u;
    unsigned* hist = sh.hist[pass & 1];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const uint32_t off = key_at(j) - lo;
      if (((vmask >> j) & 1u) && key_at(j) >= lo && off <= wspan) atomicAdd(&hist[off >> shift], 1u);
    }
    lds_barrier();
    // thread t owns bins kBins-1-BPT t down to kBins-BPT-BPT t, one 16- or 8-byte read
    unsigned cc[BPT], tot = 0;
    if constexpr (BPT == 4) {
      const uint4 c4 = *reinterpret_cast<const uint4*>(hist + kBins - 4 - 4 * tid);
      cc[0] = c4.w;
      cc[1] = c4.z;
      cc[2] = c4.y;
      cc[3] = c4.x;
    } else {
      const uint2 c2 = *reinterpret_cast<const uint2*>(hist + kBins - 2 - 2 * tid);
      cc[0] = c2.y;
      cc[1] = c2.x;
    }
#pragma unroll
    for (int j = 0; j < BPT; ++j) tot += cc[j];
    const unsigned incl = wave_incl_scan_u32(tot);
    if (lane == 63) sh.wsum[wave] = incl;
    for (int j = tid; j < kBins; j += NT) sh.hist[(pass & 1) ^ 1][j] = 0;   // the next pass's
    lds_barrier();
    unsigned run = incl - tot;
#pragma unroll
    for (int v = 0; v < NW; ++v) run += v < wave ? sh.wsum[v] : 0u;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      if (run < remaining && run + cc[j] >= remaining) {
        sh.bin = kBins - 1 - BPT * tid - j;
        sh.above = run;
        sh.cnt_bin = cc[j];
      }
      run += cc[j];
    }
    lds_barrier();
    lo += sh.bin << shift;
    remaining -= sh.above;
    cnt_bin = sh.cnt_bin;
    w = shift;
    for (int j = tid; j < kBins; j += NT) hist[j] = 0;
    if (cnt_bin == remaining) break;
  }
  r.lo = lo;
  r.span = w >= 32 ? ~0u : (1u << w) - 1u;
  r.need = remaining;
  r.n_eq = cnt_bin;
  return r;
}

// Top-k over keys held in registers (as reg_kth; element order is thread, then slot), ties at the
// k-th key going to the smaller ids: with ids_ascending (ids rise with element order) the first
// ones in element order, otherwise a second select on ~id among the keys equal to the k-th.
// emit(pos, slot, key) for every selected element, pos = 0, 1, ... in element order; returns
// their number (min(k, present keys)). Expects hist[0] cleared (sel_reset) and a barrier after;
// leaves both histograms cleared. Ends with an LDS-only barrier after the emits.
template <int NT, int IPT, class IdOf, class Emit>
__device__ unsigned reg_topk(SelShared& sh, const uint32_t (&key)[IPT], uint32_t vmask, unsigned k,
                             bool ids_ascending, IdOf id_of, Emit emit) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const KthRange r = reg_kth<NT, IPT>(sh, [&](int j) { return key[j]; }, vmask, k);
  // the keys equal to the k-th that are taken: all of them unless r.need < r.n_eq
  uint32_t tmask = 0u;                              // slots of keys in the k-th key's bin
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    tmask |= (((vmask >> j) & 1u) && r.in_bin(key[j]) ? 1u : 0u) << j;
  const bool by_id = r.need < r.n_eq && !ids_ascending;
  uint32_t take_tie = tmask;                        // by_id: those of the r.need smallest ids
  if (by_id) {
    // keys ~id, recomputed where used rather than held in registers
    const auto nid = [&](int j) { return ~(uint32_t)id_of(j); };
    lds_barrier();                                  // the histograms' clears are done
    const KthRange r2 = reg_kth<NT, IPT>(sh, nid, tmask, r.need);
    take_tie = 0u;
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      take_tie |= (((tmask >> j) & 1u) && nid(j) >= r2.lo ? 1u : 0u) << j;
  }
  // counts of this thread: keys above the bin, keys in it (ties)
  unsigned na = 0, ne = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if ((vmask >> j) & 1u) {
      na += r.above(key[j]) ? 1u : 0u;
      ne += (take_tie >> j) & 1u;
    }
  }
  const unsigned packed = (na << 16) | ne;          // both sums stay below 2^16 (<= 32768 keys)
  const unsigned incl = wave_incl_scan_u32(packed);
  if (lane == 63) sh.wsum[wave] = incl;
  lds_barrier();
  unsigned before = incl - packed, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const unsigned ws = sh.wsum[w];
    before += w < wave ? ws : 0u;
    all += ws;
  }
  // in element order the ties taken are the first r.need of the bin (ids_ascending) or the
  // marked ones (by id); both counts below are exact for this thread's position
  unsigned eq_seen = before & 0xFFFFu;
  const unsigned need = by_id ? ~0u : r.need;
  unsigned pos = (before >> 16) + min(eq_seen, need);
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    if ((vmask >> j) & 1u) {
      bool take = r.above(key[j]);
      if ((take_tie >> j) & 1u) take = eq_seen++ < need;
      if (take) emit(pos++, j, key[j]);
    }
  }
  lds_barrier();
  return (all >> 16) + min(all & 0xFFFFu, need);
}

// Select the top-k of n elements (n > k) given key_of(i, key) and id_of(i); writes k ids (and
// scores). Ties at the k-th key go to the smaller ids.
// The radix passes stop as soon as the bin holding the k-th key has at most kCandMax keys;
// those candidates are gathered and ranked by one wave (larger key first, then smaller id), and
// the r.need best are taken with every key above the bin. Only a larger bin of keys that are
// all equal to the k-th falls back to a second select on ~id.
// Slots: with ORDERED the taken elements get slots 0, 1, ... in ascending element order i and
// the ranked candidates follow in rank order, so the output is the same on every run (each wave
// walks a contiguous range of elements twice: once to count, once to emit); without it, slots
// go to waves in completion order (one counter update per wave and 64 elements, no second pass),
// for callers that only mark the selected ids.
template <int NT, bool ORDERED = true, class KeyOf, class IdOf, class Emit>
__device__ void block_topk(SelShared& sh, int n, int k, KeyOf key_of, IdOf id_of, Emit emit) {
  const KthResult r = radix_kth<NT>(sh, n, (unsigned)k, key_of, kCandMax);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NW = NT / 64;
  const uint64_t below = (1ull << lane) - 1;
  const bool partial = r.n_eq > r.need;            // only part of the k-th key's bin is taken
  const bool ranked = partial && r.n_eq <= (unsigned)kCandMax;
  // ties of more than kCandMax equal keys (every bit resolved): the r.need smallest ids, i.e.
  // the largest ~id
  KthResult r2{};
  if (partial && !ranked) {
    __syncthreads();
    r2 = radix_kth<NT>(
        sh, n, r.need,
        [&](int i, uint32_t& key) {
          uint32_t kk;
          if (!key_of(i, kk) || (kk & r.mask) != r.prefix) return false;
          key = ~(uint32_t)id_of(i);
          return true;
        });
  }
  if (threadIdx.x == 0) {
    sh.out_count = 0;
    sh.cand_count = 0;
  }
  __syncthreads();
  // element i is taken when its key is above the bin (or in the bin, unless only part of it is
  // taken); the bin's keys go to the candidate slots when they are ranked
  auto classify = [&](int i, uint32_t& key, bool& take, bool& cand) {
    key = 0;
    take = cand = false;
    if (i < n && key_of(i, key)) {
      const uint32_t km = key & r.mask;
      take = km > r.prefix;
      if (km == r.prefix) {
        if (!partial) take = true;
        else if (ranked) cand = true;
        else take = ((~(uint32_t)id_of(i)) & r2.mask) >= r2.prefix;     // ids are distinct
      }
    }
  };
  auto add_cand = [&](bool cand, uint32_t key, int i) {
    const uint64_t cm = __ballot(cand);
    if (cm != 0) {
      unsigned base = 0;
      if (lane == __builtin_ctzll(cm)) base = atomicAdd(&sh.cand_count, (unsigned)__popcll(cm));
      base = __shfl(base, __builtin_ctzll(cm), 64);
      if (cand) {
        const unsigned slot = base + (unsigned)__popcll(cm & below);
        sh.cand_key[slot] = key;
        sh.cand_id[slot] = id_of(i);
      }
    }
  };
  if constexpr (ORDERED) {
    // wave w walks chunks [c0, c1) of 64 elements
    const int nch = (n + 63) >> 6, per = (nch + NW - 1) / NW;
    const int c0 = min(wave * per, nch), c1 = min(c0 + per, nch);
    unsigned cnt = 0;
    for (int c = c0; c < c1; ++c) {
      uint32_t key;
      bool take, cand;
      classify(c * 64 + lane, key, take, cand);
      cnt += (unsigned)__popcll(__ballot(take));
      if (ranked) add_cand(cand, key, c * 64 + lane);
    }
    if (lane == 0) sh.wsum[wave] = cnt;
    __syncthreads();
    unsigned slot = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const unsigned ws = sh.wsum[w];
      slot += w < wave ? ws : 0u;
      total += ws;
    }
    for (int c = c0; c < c1; ++c) {
      uint32_t key;
      bool take, cand;
      classify(c * 64 + lane, key, take, cand);
      const uint64_t tm = __ballot(take);
      if (take) emit(slot + (unsigned)__popcll(tm & below), id_of(c * 64 + lane), key);
      slot += (unsigned)__popcll(tm);
    }
    if (lane == 0 && wave == 0) sh.out_count = total;
  } else {
    for (int i0 = threadIdx.x & ~63; i0 < n; i0 += NT) {
      const int i = i0 + lane;
      uint32_t key;
      bool take, cand;
      classify(i, key, take, cand);
      const uint64_t tm = __ballot(take);
      if (tm != 0) {
        unsigned base = 0;
        if (lane == __builtin_ctzll(tm)) base = atomicAdd(&sh.out_count, (unsigned)__popcll(tm));
        base = __shfl(base, __builtin_ctzll(tm), 64);
        if (take) emit(base + (unsigned)__popcll(tm & below), id_of(i), key);
      }
      if (ranked) add_cand(cand, key, i);
    }
  }
  __syncthreads();
  if (ranked && wave == 0) {
    // rank of candidate `lane` among the n_eq (all in LDS now): larger key first, then smaller
    // id; the r.need best follow every other taken key, in rank order
    const int nc = (int)r.n_eq;
    const uint32_t mk = lane < nc ? sh.cand_key[lane] : 0u;
    const int mi = lane < nc ? sh.cand_id[lane] : 0;
    unsigned rank = 0;
    for (int j = 0; j < nc; ++j) {
      const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)mk, j);
      const int ij = __builtin_amdgcn_readlane(mi, j);
      rank += (kj > mk || (kj == mk && ij < mi)) ? 1u : 0u;
    }
    const unsigned base = sh.out_count;           // every other key is counted by now
    if (lane < nc && rank < r.need) emit(base + rank, mi, mk);
  }
  __syncthreads();
}

}  // namespace
}  // namespace hcs
