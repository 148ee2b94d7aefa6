// Query preparation and sliding-window KV insert for gfx950.
//
// What it computes: "DeepSeek V4 Attention: Code Reading Map", section "Default stream" (the
// fused q-norm / RoPE / KV insert), and the "DeepSeek V4.1 attention" page's
// `_fused_qnorm_rope_kv_insert`: for every new token, each query head is optionally brought to
// unit RMS over its d dims (no weight) and its last d_rope dims are rotated in GPT-J pairs at
// the token's position; the token's KV row is rotated the same way and written to the
// sliding-window cache at logical row = the token's position, as a bf16 row, an fp8_ds record or
// an MXFP8 record. The query is rewritten in place; the KV input is not modified.
//
// Design: one wave per (token, group of G query heads) and one per (token, KV row), four waves
// to a workgroup. A lane holds E = d / 64 consecutive dims of a row (16 B at d = 512), so a row
// is one coalesced load and store, and a GPT-J pair (2j, 2j+1) never leaves its lane. A wave
// loads all G of its rows before using any (the kernel streams q through HBM once; the bytes a
// wave keeps in flight set the rate). The norm is a wave sum per head. The RoPE row is loaded
// with the data (clamped indices, no branch), so a wave makes one memory round trip before its
// stores. For the fp8_ds store eight lanes hold one 64-dim
// latent block, so the block amax is three xor shuffles; lanes 56..63 hold the 64 rotary dims,
// stored as bf16.
#include "kernels.h"

namespace hcs {

HCS_DEVICE_ERROR_WORD(insert)

namespace {

constexpr int kInsertThreads = 256;
constexpr int kInsertWaves = kInsertThreads / 64;

template <int E>
__device__ __forceinline__ void load_bf16_row(const uint16_t* p, float (&x)[E]) {
  uint32_t w[E / 2];
  if constexpr (E == 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
  } else {
    static_assert(E == 2, "rows of 128 or 512 dims");
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

template <int E>
__device__ __forceinline__ void store_bf16_row(uint16_t* p, const float (&x)[E]) {
  uint32_t w[E / 2];
#pragma unroll
  for (int i = 0; i < E / 2; ++i) w[i] = f32_to_bf16_bits(x[2 * i]) | (f32_to_bf16_bits(x[2 * i + 1]) << 16);
  if constexpr (E == 8) *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  else *reinterpret_cast<uint32_t*>(p) = w[0];
}

// this lane's RoPE pairs (dims E*lane + 2i, +1) at position pos; rows clamped so that the loads
// need no branch (pairs below r0 get the identity when applied)
template <int E>
__device__ __forceinline__ void rope_row(const InsertArgs& a, int pos, int lane, float (&rc)[E / 2],
                                         float (&rs)[E / 2]) {
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    rc[i] = 1.f;
    rs[i] = 0.f;
  }
  if (!a.rope_cos) return;
  const int r0 = E * 64 - a.d_rope;
  const int64_t row = (int64_t)min(pos, a.rope_rows - 1) * (a.d_rope / 2);
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    const int64_t ri = row + (max(E * lane + 2 * i - r0, 0) >> 1);
    rc[i] = a.rope_cos[ri];
    rs[i] = a.rope_sin[ri];
  }
}

template <int E>
__device__ __forceinline__ void apply_rope(const InsertArgs& a, int lane, float (&x)[E],
                                           const float (&rc)[E / 2], const float (&rs)[E / 2]) {
  if (!a.rope_cos) return;
  const int r0 = E * 64 - a.d_rope;
#pragma unroll
  for (int i = 0; i < E / 2; ++i) {
    if (E * lane + 2 * i < r0) continue;
    const float u = x[2 * i], v = x[2 * i + 1];
    x[2 * i] = u * rc[i] - v * rs[i];
    x[2 * i + 1] = u * rs[i] + v * rc[i];
  }
}

// G query heads of token t, starting at head h0: all G rows are loaded before any is used, so
// a wave keeps G x 1 KiB in flight (at d = 512)
template <int E, int G>
__device__ __forceinline__ void prep_q_heads(const InsertArgs& a, int t, int h0, int pos, int lane) {
  constexpr int d = E * 64;
  float x[G][E];
  uint16_t* base = a.q + ((int64_t)t * a.H) * d + lane * E;
#pragma unroll
  for (int g = 0; g < G; ++g) load_bf16_row<E>(base + (int64_t)min(h0 + g, a.H - 1) * d, x[g]);
  float rc[E / 2], rs[E / 2];
  rope_row<E>(a, pos, lane, rc, rs);
  if (a.q_norm) {                                // unit RMS over each head's d dims
    float ss[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      ss[g] = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) ss[g] += x[g][i] * x[g][i];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) ss[g] += __shfl_xor(ss[g], o, 64);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float r = 1.f / __builtin_sqrtf(ss[g] / (float)d + a.eps);
#pragma unroll
      for (int i = 0; i < E; ++i) x[g][i] *= r;
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    apply_rope<E>(a, lane, x[g], rc, rs);
    if (h0 + g < a.H) store_bf16_row<E>(base + (int64_t)(h0 + g) * d, x[g]);
  }
}

// the KV row of token t: rotated, stored as logical row pos of sequence seq
template <int E>
__device__ __forceinline__ void insert_kv_row(const InsertArgs& a, int t, int seq, int pos, int lane) {
  constexpr int d = E * 64;
  float x[E];
  load_bf16_row<E>(a.kv + (int64_t)t * a.kv_stride + lane * E, x);
  float rc[E / 2], rs[E / 2];
  rope_row<E>(a, pos, lane, rc, rs);
  if ((pos >> 6) >= a.swa_pt_stride) return;
  const int pg = a.swa_pt[(int64_t)seq * a.swa_pt_stride + (pos >> 6)];
  if (pg >= a.swa_num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
  if (pg < 0 || pg >= a.swa_num_pages) return;   // not resident: the write is dropped
  apply_rope<E>(a, lane, x, rc, rs);
  const int slot = pos & 63;
  if (a.fmt == HCS_FMT_BF16) {
    uint16_t* page = reinterpret_cast<uint16_t*>(a.swa_base + (int64_t)pg * kPageRows * d * 2);
    store_bf16_row<E>(page + (int64_t)slot * d + lane * E, x);
    return;
  }
  if constexpr (E == 8) {
    if (a.fmt == HCS_FMT_MXFP8) {                // MXFP8 record: 4 lanes = one 32-value block
      uint8_t* page = a.swa_base + (int64_t)pg * kMx8PageBytes;
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(x[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
      const int e = fp8ds_scale_exp(amax);
      float y[E];
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] = __builtin_ldexpf(x[i], -e);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
      *reinterpret_cast<uint2*>(page + slot * 512 + lane * E) = make_uint2((uint32_t)lo, (uint32_t)hi);
      if ((lane & 3) == 0) page[kMx8Scales + slot * 16 + (lane >> 2)] = (uint8_t)(e + 127);
      return;
    }
    // fp8_ds record (d = 512)
    uint8_t* page = a.swa_base + (int64_t)pg * kFp8PageBytes;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(x[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    constexpr int kLatentLanes = kFp8Latent / E;   // 56
    if (lane < kLatentLanes) {
      const int e = fp8ds_scale_exp(amax);
      float y[E];
#pragma unroll
      for (int i = 0; i < E; ++i) y[i] = __builtin_ldexpf(x[i], -e);
      int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
      int hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
      *reinterpret_cast<uint2*>(page + kFp8PageCodes + slot * kFp8Latent + lane * E) =
          make_uint2((uint32_t)lo, (uint32_t)hi);
      if ((lane & 7) == 0) page[kFp8PageScales + slot * 8 + (lane >> 3)] = (uint8_t)(e + 127);
    } else {
      store_bf16_row<E>(reinterpret_cast<uint16_t*>(page + kFp8PageRope + slot * kFp8Rope * 2) +
                            (lane - kLatentLanes) * E, x);
      if (lane == kLatentLanes) page[kFp8PageScales + slot * 8 + 7] = 0;
    }
  }
}

// wave w of token t: w < ceil(H / G) prepares G query heads, the last one (when kv is given)
// inserts the KV row
template <int E, int G>
__global__ __launch_bounds__(kInsertThreads) void qrope_insert_kernel(InsertArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * kInsertWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qw = (a.H + G - 1) / G;
  const int per = qw + (a.kv ? 1 : 0);
  const int64_t t64 = gw / per;
  if (t64 >= a.N) return;
  const int t = (int)t64, w = (int)(gw - t64 * per);
  const int pos = a.tok_pos[t];
  const int seq = w < qw ? 0 : a.tok_seq[t];
  if (pos < 0) return;
  if (w < qw) prep_q_heads<E, G>(a, t, w * G, pos, lane);
  else insert_kv_row<E>(a, t, seq, pos, lane);
}

}  // namespace

hipError_t launch_qrope_insert(const InsertArgs& a, hipStream_t stream) {
  // heads per wave: 4 rows of 512 dims (4 KiB in flight per wave), 8 of 128 dims
  constexpr int G512 = 4, G128 = 8;
  const int G = a.d == 512 ? G512 : G128;
  const int64_t waves = (int64_t)a.N * ((a.H + G - 1) / G + (a.kv ? 1 : 0));
  if (waves == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((waves + kInsertWaves - 1) / kInsertWaves);
  if (a.d == 512)
    hipLaunchKernelGGL((qrope_insert_kernel<8, G512>), dim3(blocks), dim3(kInsertThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((qrope_insert_kernel<2, G128>), dim3(blocks), dim3(kInsertThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hcs
