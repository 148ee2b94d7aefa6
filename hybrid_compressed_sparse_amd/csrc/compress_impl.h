// Compressor device code, shared by its own launch (compress.hip, which says what it computes
// and how) and the indexer launch that runs compressor blocks beside its scoring blocks.
#pragma once

#include <algorithm>

#include "kernels.h"

namespace hcs {

constexpr int kCompressThreads = 256;

// element idx of a compressor input (bf16 or float32); the type is a template argument so that
// loads of several tokens or channels are not split by a branch on it
template <bool BF16>
__device__ __forceinline__ float compress_load_in(const void* p, int64_t idx) {
  if constexpr (BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[idx]);
  else return static_cast<const float*>(p)[idx];
}

// Stores channel c (of a completed entry kb of sequence b) of value C: the optional float32
// copy, and the cache row: bf16; fp8_ds (per 64-dim latent block a power-of-two scale from
// the wave's amax, e4m3 codes by the hardware's round-to-nearest-even conversion; the 64
// rotary dims as bf16); MXFP8 (the same per 32 dims, all 512 in e4m3); NVFP4 (per 16 dims an
// e4m3 scale nearest amax / 6, e2m1 codes). `page` is the entry's page (nullptr: not resident).
// Called by every lane of a wave, a wave holding 64 consecutive channels.
__device__ __forceinline__ void compress_store(const CompressArgs& a, int b, int kb, int kb_first,
                                               const uint8_t* page, int c, bool act, float C) {
  const int d = a.d, slot = kb & 63;
  if (act && a.dbg) a.dbg[(int64_t)b * a.dbg_stride + (int64_t)(kb - kb_first) * d + c] = C;
  if (a.fmt == HCS_FMT_FP8DS) {
    if (c < kFp8Latent) {
      const int e = fp8ds_scale_exp(warp_max(fabsf(C)));
      const float y = __builtin_ldexpf(C, -e);
      const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0, false);
      if (page) {
        uint8_t* pw = const_cast<uint8_t*>(page);
        pw[kFp8PageCodes + slot * kFp8Latent + c] = (uint8_t)(packed & 0xff);
        if ((c & 63) == 0) pw[kFp8PageScales + slot * 8 + (c >> 6)] = (uint8_t)(e + 127);
        if (c == 0) pw[kFp8PageScales + slot * 8 + 7] = 0;
      }
    } else if (act && page) {
      uint16_t* rope = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(page) + kFp8PageRope +
                                                   slot * kFp8Rope * 2);
      rope[c - kFp8Latent] = (uint16_t)f32_to_bf16_bits(C);
    }
  } else if (a.fmt == HCS_FMT_MXFP8) {            // 512 e4m3, one power-of-two scale per 32
    float amax = fabsf(C);
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const int e = fp8ds_scale_exp(amax);
    const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(C, -e), 0.f, 0, false);
    if (page) {
      uint8_t* pw = const_cast<uint8_t*>(page);
      pw[slot * 512 + c] = (uint8_t)(packed & 0xff);
      if ((c & 31) == 0) pw[kMx8Scales + slot * 16 + (c >> 5)] = (uint8_t)(e + 127);
    }
  } else if (a.fmt == HCS_FMT_NVFP4) {            // 512 e2m1, one e4m3 scale per 16
    float amax = fabsf(C);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    // scale: e4m3 nearest amax / 6 (the quotient in float32); codes: nearest-even e2m1 of
    // C / scale, saturated to 6; a zero scale stores zero codes
    const int sc = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(amax / 6.f, 448.f), 0.f, 0, false) & 0xff;
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    const f32x2 sv2 = __builtin_amdgcn_cvt_pk_f32_fp8(sc, false);
    const float sv = sv2.x;
    const float y = sv > 0.f ? fminf(fmaxf(C / sv, -6.f), 6.f) : 0.f;
    const uint32_t code = e2m1_code(y);
    const uint32_t pair = code | (__shfl_xor(code, 1, 64) << 4);   // element 2j low, 2j+1 high
    if (page) {
      uint8_t* pw = const_cast<uint8_t*>(page);
      if ((c & 1) == 0) pw[slot * 256 + (c >> 1)] = (uint8_t)pair;
      if ((c & 15) == 0) pw[kNv4Scales + slot * 32 + (c >> 4)] = (uint8_t)sc;
    }
  } else if (act && page) {
    uint16_t* row = reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(page)) + (int64_t)slot * d;
    row[c] = (uint16_t)f32_to_bf16_bits(C);
  }
}

// Page of completed entry kb of sequence b in the compressed cache, or nullptr.
__device__ __forceinline__ const uint8_t* compress_entry_page(const CompressArgs& a, int b, int kb) {
  const int pg = (kb >> 6) < a.comp_pt_stride ? __ldg(a.comp_pt + (int64_t)b * a.comp_pt_stride + (kb >> 6)) : -1;
  if (pg >= a.comp_num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
  if (pg < 0 || pg >= a.comp_num_pages) return nullptr;
  const int64_t pb = a.fmt == HCS_FMT_BF16 ? (int64_t)kPageRows * a.d * 2 : kv_page_bytes(a.fmt);
  return a.comp_base + (int64_t)pg * pb;
}

// The work of compressor block (b, y, z) of a grid with ny blocks along y (see compress_grid):
// sequence b, block slot y, channel group z. Every thread of the block calls it.
template <bool BF16>
__device__ __forceinline__ void compress_block_t(const CompressArgs& a, int b, int y, int z, int ny) {
  const int row0 = a.cu_new[b];
  const int n = a.cu_new[b + 1] - row0;
  const int start = a.start_pos[b];
  if (n <= 0 || start < 0) return;               // (testing start too loads it beside n)
  const int m = a.m, d = a.d;
  const int kb_first = start / m;
  const int kb_last = (start + n - 1) / m;
  const int dpad = (d + 63) & ~63;
  const float kNegInf = -__builtin_huge_valf();
  float* st = a.state + (int64_t)b * 3 * d;
  // this workgroup's channels (group z of kCompressThreads channels, whole 64-channel waves)
  const int c0 = z * kCompressThreads, c1 = min(dpad, c0 + kCompressThreads);

  // The first block (which may resume from the carried state) and the last block (which
  // leaves the state for the next call) are walked by the same workgroup, first then last, so
  // the state is read before it is overwritten. Middle blocks are spread over the others.
  auto do_block = [&](int kb) {
    const int blk_lo = kb * m;
    const int tok_lo = max(start, blk_lo);
    const int tok_hi = min(start + n, blk_lo + m);
    const bool complete = blk_lo + m <= start + n;
    const bool resume = blk_lo < start;       // the block began in an earlier call
    const uint8_t* page = complete ? compress_entry_page(a, b, kb) : nullptr;   // its destination
    for (int c = c0 + threadIdx.x; c < c1; c += kCompressThreads) {
      const bool act = c < d;
      float M = kNegInf, Z = 0.f, A = 0.f;
      if (act) {
        if (resume) {
          M = st[c];
          Z = st[d + c];
          A = st[2 * d + c];
        }
        for (int tok = tok_lo; tok < tok_hi; ++tok) {
          const int64_t r = (int64_t)(row0 + tok - start) * a.row_stride + c;
          float z = compress_load_in<BF16>(a.score, r);
          if (a.ape) z += a.ape[(int64_t)(tok - blk_lo) * d + c];
          const float x = compress_load_in<BF16>(a.kv, r);
          const float Mn = fmaxf(M, z);
          const float f_old = __expf(M - Mn);      // 0 when M = -inf
          const float f_new = __expf(z - Mn);
          Z = Z * f_old + f_new;
          A = A * f_old + x * f_new;
          M = Mn;
        }
      }
      if (complete) compress_store(a, b, kb, kb_first, page, c, act, act ? A / Z : 0.f);
      if (act && kb == kb_last) {
        if (complete) {
          st[c] = kNegInf;
          st[d + c] = 0.f;
          st[2 * d + c] = 0.f;
        } else {
          st[c] = M;
          st[d + c] = Z;
          st[2 * d + c] = A;
        }
      }
    }
  };

  if (y == 0) {
    do_block(kb_first);
    if (kb_last != kb_first) do_block(kb_last);
  }
  const int workers = ny > 1 ? ny - 1 : 1;
  if (ny == 1 || y > 0) {
    const int w0 = ny > 1 ? y - 1 : 0;
    for (int kb = kb_first + 1 + w0; kb < kb_last; kb += workers) do_block(kb);
  }
}

__device__ __forceinline__ void compress_block(const CompressArgs& a, int b, int y, int z, int ny) {
  if (a.in_bf16) compress_block_t<true>(a, b, y, z, ny);
  else compress_block_t<false>(a, b, y, z, ny);
}

// Grid of a compressor launch: (sequences, block slots, channel groups): one workgroup for the
// first and last block of each sequence, one per middle block, each split over channel groups
// of kCompressThreads (one channel per thread: a thread's state and token loads are one memory
// round trip).
inline dim3 compress_grid(const CompressArgs& a, int max_new) {
  const int slots = std::min(65535, std::max(1, (max_new + a.m - 1) / a.m));
  const int groups = ((a.d + 63) / 64 * 64 + kCompressThreads - 1) / kCompressThreads;
  return dim3(a.B, slots, groups);
}

}  // namespace hcs
