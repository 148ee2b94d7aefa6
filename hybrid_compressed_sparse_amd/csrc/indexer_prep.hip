// Indexer query and key production for gfx950.
//
// What it computes: the "DeepSeek V4.1 attention" page, `DeepseekV4Indexer`: `forward_q` rotates
// the projected indexer query (GPT-J pairs on its last d_rope dims, at the token's position),
// quantizes it to the key cache's format and scales the head weights by softmax_scale and
// n_head^-1/2; `_produce_k` normalises the projected latent of each new compressed entry with
// the k_norm RMSNorm, rotates it at the entry's position and stores it, quantized, in the paged
// indexer key cache (`_indexer_k_cache_head_dim`: 68-byte MXFP4 rows, 132-byte FP8 rows).
//
// Design: d_I = 128, so a lane holds the two dims (2l, 2l+1) of a row: exactly one GPT-J pair
// and one MXFP4 byte. A query wave takes G heads of one token and loads all G rows before using
// any. MXFP4 blocks of 32 values are 16 lanes (amax by four xor shuffles), an FP8 row's scale
// is the whole wave's amax. e2m1 codes come from threshold counting (exact round-to-nearest-
// even), e4m3 codes from the hardware's round-to-nearest-even conversion.
#include "kernels.h"

namespace hcs {

HCS_DEVICE_ERROR_WORD(indexer_prep)

namespace {

constexpr int kIxThreads = 256;
constexpr int kIxWaves = kIxThreads / 64;
constexpr int kIxDim = 128;
constexpr int kIxHeadsPerWave = 8;

struct Pair {
  float u, v;
};

__device__ __forceinline__ Pair load_pair(const uint16_t* row, int lane) {
  const uint32_t w = reinterpret_cast<const uint32_t*>(row)[lane];
  return {bf16_bits_to_f32(w & 0xffffu), bf16_bits_to_f32(w >> 16)};
}

// cos / sin of this lane's pair at position pos (identity below the rotated dims)
__device__ __forceinline__ void pair_angle(const float* rc, const float* rsn, int d_rope, int rope_rows,
                                           int pos, int lane, float& c, float& s) {
  c = 1.f;
  s = 0.f;
  if (!rc) return;
  const int j = lane - (kIxDim - d_rope) / 2;
  const int64_t ri = (int64_t)min(pos, rope_rows - 1) * (d_rope / 2) + max(j, 0);
  const float cc = rc[ri], ss = rsn[ri];
  if (j >= 0) {
    c = cc;
    s = ss;
  }
}

__device__ __forceinline__ Pair rotate(Pair p, float c, float s) {
  return {p.u * c - p.v * s, p.u * s + p.v * c};
}

// One row (two values per lane) in `fmt`: bf16 to dst16, MXFP4 codes to codes (64 B) and its four
// scale bytes to scale8, FP8 codes to codes (128 B) and the row scale to scalef.
__device__ __forceinline__ void store_row(int fmt, Pair p, int lane, uint16_t* dst16, uint8_t* codes,
                                          uint8_t* scale8, float* scalef) {
  if (fmt == HCS_FMT_BF16) {
    reinterpret_cast<uint32_t*>(dst16)[lane] = f32_to_bf16_bits(p.u) | (f32_to_bf16_bits(p.v) << 16);
    return;
  }
  float amax = fmaxf(fabsf(p.u), fabsf(p.v));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 8, 64));
  if (fmt == HCS_FMT_MXFP4) {                    // 16 lanes = one 32-value block
    const int e = mxfp4_scale_exp(amax);
    const uint32_t lo = e2m1_code(__builtin_ldexpf(p.u, -e)), hi = e2m1_code(__builtin_ldexpf(p.v, -e));
    codes[lane] = (uint8_t)(lo | (hi << 4));
    if ((lane & 15) == 0) scale8[lane >> 4] = (uint8_t)(e + 127);
    return;
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));  // FP8: one scale for the row
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  const int e = fp8ds_scale_exp(amax);
  const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(p.u, -e), __builtin_ldexpf(p.v, -e), 0, false);
  reinterpret_cast<uint16_t*>(codes)[lane] = (uint16_t)(pk & 0xffff);
  if (lane == 0) *scalef = __builtin_ldexpf(1.f, e);
}

__global__ __launch_bounds__(kIxThreads) void indexer_q_kernel(IxQArgs a) {
  constexpr int G = kIxHeadsPerWave;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kIxWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int per = (a.H + G - 1) / G;
  const int64_t t64 = gw / per;
  if (t64 >= a.N) return;
  const int t = (int)t64, h0 = (int)(gw - t64 * per) * G;
  const int pos = a.tok_pos[t];
  if (pos < 0) return;
  Pair x[G];
#pragma unroll
  for (int g = 0; g < G; ++g) x[g] = load_pair(a.q + ((int64_t)t * a.H + min(h0 + g, a.H - 1)) * kIxDim, lane);
  float c, s;
  pair_angle(a.rope_cos, a.rope_sin, a.d_rope, a.rope_rows, pos, lane, c, s);
  if (h0 == 0 && lane < a.H) a.w_out[(int64_t)t * a.H + lane] = a.w[(int64_t)t * a.H + lane] * a.w_scale;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int h = h0 + g;
    if (h >= a.H) break;
    const int64_t row = (int64_t)t * a.H + h;
    store_row(a.fmt, rotate(x[g], c, s), lane, a.q_out16 + row * kIxDim,
              a.q_out8 + row * (a.fmt == HCS_FMT_MXFP4 ? kIxDim / 2 : kIxDim),
              a.q_scale8 + row * (kIxDim / kMxBlock), a.q_scalef + row);
  }
}

__global__ __launch_bounds__(kIxThreads) void indexer_k_kernel(IxKArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t r64 = (int64_t)blockIdx.x * kIxWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r64 >= a.n) return;
  const int r = (int)r64;
  const int seq = a.ent_seq[r], ent = a.ent_idx[r];
  if (ent < 0) return;
  Pair x = load_pair(a.k + r64 * a.k_stride, lane);
  const float w0 = a.norm_w[2 * lane], w1 = a.norm_w[2 * lane + 1];
  float c, s;
  const int64_t pos = (int64_t)a.m * ent;
  pair_angle(a.rope_cos, a.rope_sin, a.d_rope, a.rope_rows, (int)min(pos, (int64_t)INT32_MAX), lane, c, s);
  if ((ent >> 6) >= a.keys.pt_stride) return;
  const int pg = a.keys.pt[(int64_t)seq * a.keys.pt_stride + (ent >> 6)];
  if (pg >= a.keys.num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
  if (pg < 0 || pg >= a.keys.num_pages) return;   // not resident: the write is dropped
  const float ss = warp_sum(x.u * x.u + x.v * x.v);
  const float rn = 1.f / __builtin_sqrtf(ss / (float)kIxDim + a.eps);
  x = rotate({x.u * rn * w0, x.v * rn * w1}, c, s);
  const int slot = ent & 63;
  uint8_t* page = const_cast<uint8_t*>(a.keys.base);
  if (a.fmt == HCS_FMT_BF16) {
    page += (int64_t)pg * kPageRows * kIxDim * 2;
    store_row(a.fmt, x, lane, reinterpret_cast<uint16_t*>(page) + slot * kIxDim, nullptr, nullptr, nullptr);
  } else if (a.fmt == HCS_FMT_MXFP4) {
    constexpr int CB = kIxDim / 2, SB = kIxDim / kMxBlock;
    page += (int64_t)pg * kPageRows * (CB + SB);
    store_row(a.fmt, x, lane, nullptr, page + slot * CB, page + kPageRows * CB + slot * SB, nullptr);
  } else {
    page += (int64_t)pg * kPageRows * (kIxDim + 4);
    store_row(a.fmt, x, lane, nullptr, page + slot * kIxDim,
              nullptr, reinterpret_cast<float*>(page + kPageRows * kIxDim) + slot);
  }
}

}  // namespace

hipError_t launch_indexer_q(const IxQArgs& a, hipStream_t stream) {
  const int64_t waves = (int64_t)a.N * ((a.H + kIxHeadsPerWave - 1) / kIxHeadsPerWave);
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_q_kernel, dim3((unsigned)((waves + kIxWaves - 1) / kIxWaves)), dim3(kIxThreads),
                     0, stream, a);
  return hipGetLastError();
}

hipError_t launch_indexer_k(const IxKArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  hipLaunchKernelGGL(indexer_k_kernel, dim3((unsigned)((a.n + kIxWaves - 1) / kIxWaves)), dim3(kIxThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace hcs
