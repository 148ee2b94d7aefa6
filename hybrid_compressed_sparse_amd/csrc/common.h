// Shared device helpers for the gfx950 kernels of the hybrid compressed sparse attention path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hcs.h"

namespace hcs {

constexpr int kPageRows = HCS_PAGE_ROWS;
constexpr int kFp8Latent = 448;      // e4m3 latent dims of an fp8_ds row
constexpr int kFp8Rope = 64;         // bf16 rotary dims of an fp8_ds row
constexpr int kFp8Block = 64;        // latent dims per UE8M0 scale
constexpr int kFp8PageCodes = 0;                              // [64][448] u8
constexpr int kFp8PageRope = kPageRows * kFp8Latent;          // [64][64] bf16 at 28672
constexpr int kFp8PageScales = kFp8PageRope + kPageRows * kFp8Rope * 2;   // [64][8] u8 at 36864
constexpr int kFp8PageBytes = kFp8PageScales + kPageRows * 8;             // 37376 = 64 * 584
constexpr int kMxBlock = 32;
// MXFP8 rows (512 e4m3 + one UE8M0 per 32): [64][512] codes | [64][16] scales
constexpr int kMx8Scales = kPageRows * 512;                   // 32768
constexpr int kMx8PageBytes = kMx8Scales + kPageRows * 16;     // 33792 = 64 * 528
// NVFP4 rows (512 e2m1 + one e4m3 per 16): [64][256] packed codes | [64][32] scales
constexpr int kNv4Scales = kPageRows * 256;                   // 16384
constexpr int kNv4PageBytes = kNv4Scales + kPageRows * 32;     // 18432 = 64 * 288

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// A paged cache as the kernels see it.
struct Paged {
  const uint8_t* base;
  const int32_t* pt;
  int32_t pt_stride;
  int32_t num_pages;
};

inline Paged to_paged(const hcs_paged& p) {
  return Paged{static_cast<const uint8_t*>(p.base), p.page_table, p.pt_stride, p.num_pages};
}

// ---------------------------------------------------------------- device error word
// Kernels OR the HCS_DEVERR_* bits of hcs.h into a word that stays set until the host reads and
// clears it (hcs_device_errors). Each .hip file is its own device code object, so each defines
// its own word, its dev_error() and a host reader dev_errors_<file>() with
// HCS_DEVICE_ERROR_WORD(<file>) at namespace hcs scope.
namespace {
__device__ void dev_error(unsigned bits);
}
#define HCS_DEVICE_ERROR_WORD(NAME)                                                                   \
  __device__ unsigned g_dev_err_##NAME;                                                               \
  namespace {                                                                                         \
  __device__ void dev_error(unsigned bits) { atomicOr(&g_dev_err_##NAME, bits); }                     \
  }                                                                                                   \
  hipError_t dev_errors_##NAME(uint32_t* bits, bool clear) {                                          \
    uint32_t v = 0;                                                                                   \
    hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_dev_err_##NAME), sizeof(v), 0,                \
                                       hipMemcpyDeviceToHost);                                        \
    if (e == hipSuccess && clear && v) {                                                              \
      const uint32_t zero = 0;                                                                        \
      e = hipMemcpyToSymbol(HIP_SYMBOL(g_dev_err_##NAME), &zero, sizeof(zero), 0,                     \
                            hipMemcpyHostToDevice);                                                   \
    }                                                                                                 \
    *bits |= v;                                                                                       \
    return e;                                                                                         \
  }

// Page id of logical row `row` of sequence `seq`, or -1 if not resident (a negative entry); an
// entry past the pool (>= num_pages) is also treated as not resident and flagged in the error
// word.
__device__ __forceinline__ int page_of(const Paged& c, int seq, int row) {
  int pg = __ldg(c.pt + (int64_t)seq * c.pt_stride + (row >> 6));
  if (pg >= c.num_pages) dev_error(HCS_DEVERR_PAGE_RANGE);
  return (pg >= 0 && pg < c.num_pages) ? pg : -1;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round-to-nearest-even float32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float warp_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float warp_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// UE8M0 exponent of a block scaled into a format whose largest value is qf * 2^qe (qf in
// [0.5, 1)): the smallest e with amax <= qf * 2^(qe + e), 0 for an all-zero block, clamped to
// [-127, 127].
__device__ __forceinline__ int ue8m0_scale_exp(float amax, float qf, int qe) {
  int E;
  const float f = __builtin_frexpf(amax, &E);
  const int e = amax > 0.f ? E - qe + (f > qf ? 1 : 0) : 0;
  return max(-127, min(127, e));
}
// e4m3: 448 = 0.875 * 2^9 (the fp8_ds latent blocks and the FP8 indexer rows)
__device__ __forceinline__ int fp8ds_scale_exp(float amax) { return ue8m0_scale_exp(amax, 0.875f, 9); }
// e2m1: 6 = 0.75 * 2^3 (MXFP4 blocks)
__device__ __forceinline__ int mxfp4_scale_exp(float amax) { return ue8m0_scale_exp(amax, 0.75f, 3); }

// Bytes of a 64-row page of a 512-dim KV cache in `fmt` (bf16 pages are 64 x 1 KiB).
__host__ __device__ inline int64_t kv_page_bytes(int fmt) {
  return fmt == HCS_FMT_FP8DS ? kFp8PageBytes
         : fmt == HCS_FMT_MXFP8 ? kMx8PageBytes
         : fmt == HCS_FMT_NVFP4 ? kNv4PageBytes
                                : (int64_t)kPageRows * 512 * 2;
}

// e2m1 nibble (sign in bit 3) -> float
__device__ __forceinline__ float e2m1_value(uint32_t n) {
  const uint32_t mag = n & 7u;
  const float f = mag < 2u ? 0.5f * (float)mag
                           : __uint_as_float(((126u + (mag >> 1)) << 23) | ((mag & 1u) << 22));
  return (n & 8u) ? -f : f;
}

// Nearest e2m1 code of y (|y| <= 6), ties to the even code: the magnitude code counts the
// thresholds |y| passes (halfway points; those that round up to an even code are inclusive).
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
                     (a >= 3.5f) + (a > 5.f);
  return c | (y < 0.f ? 8u : 0u);
}

// Order-preserving map of float32 to uint32: a < b  <=>  key(a) < key(b) (for non-NaN).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// s_waitcnt vmcnt(0): this wave's global loads (including those into LDS) have completed.
__device__ __forceinline__ void wait_vm_zero() {
  // s_waitcnt vmcnt(0): vmcnt 0, expcnt 7, lgkmcnt 15 (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// LDS byte address of a __shared__ location.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// global_load_lds_dwordx4 as inline assembly: lane i copies the 16 bytes at base + voff to LDS
// address lds + 16 i (lds wave-uniform). The compiler does not see this LDS write, so it adds
// no vmcnt waits of its own before later LDS reads (it cannot tell a read of the other tile of
// a double buffer from a read of this one); the caller waits (s_waitcnt vmcnt) before the
// destination is read. Every LDS DMA of a kernel goes through here, so no M0 value of the
// compiler's own is live across it.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane((int)lds)) : "memory", "m0");
}

// The same with a per-lane source address.
__device__ __forceinline__ void dma16v(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(__builtin_amdgcn_readfirstlane((int)lds)) : "memory", "m0");
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

}  // namespace hcs
