// KV compressor for gfx950.
//
// What it computes: "DeepSeek V4 Attention: Code Reading Map", section "How Does Compression
// Actually Work?": for every block of m consecutive tokens, the gate logits (plus the
// positional encoding of each token's place in the block) go through a softmax over the m
// tokens, and the entry is the weighted sum of the block's raw KV rows. The softmax runs per
// channel: the gate-score half of the compressor input has the KV half's width.
//
// Design: instead of keeping the block's raw tokens (the pages' float32 state cache holds the
// partial block's KV and scores), each channel keeps the online-softmax triple
// (running max M, running sum Z of e^(z-M), running sum A of e^(z-M) * kv) in float32: the
// same entry A/Z, O(d) state per sequence whatever m is, and no re-gather of the block when it
// completes. One workgroup walks one block of one sequence for 256 channels; each thread owns
// one channel and streams the block's tokens through the recurrence (rows are read coalesced
// across channels). A completed entry is written straight into the paged compressed cache, either as
// a bf16 row or as an fp8_ds record (per 64-dim latent block: power-of-two scale, e4m3 codes by
// the hardware's round-to-nearest-even conversion; the 64 rotary dims as bf16). The block's
// amax is a wave reduction, because one wave covers exactly one 64-channel block.
#include "compress_impl.h"

namespace hcs {

namespace {

__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressArgs a) {
  compress_block(a, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.y);
}

// ---------------------------------------------------------------- full compressor
// "How Does Compression Actually Work?", steps 1-7: with the overlapping window (coff = 2) an
// entry's softmax runs over 2m logits per channel, block i's tokens in the primary series
// (columns 0..d-1) and block i-1's tokens in the overlapping series (columns d..2d-1), so the
// tokens of a block feed two entries; then the entry is RMS-normalised over its d dims and its
// last d_rope dims are rotated (GPT-J pairs) at position m * i before the store.
// Online form, per channel, two (max, sum, acc) triples: `cur` accumulates the entry of the
// block being filled (its primary tokens plus the previous block's overlapping tokens), `nxt`
// the overlapping tokens of that block, which start the next entry. At a block's end `cur` is
// emitted and `nxt` becomes the next `cur`. The state [3 coff d] keeps both between calls.
// A workgroup covers all d channels of an entry (the norm needs them all): up to four per
// thread. Workgroup y = 0 walks the call's first block, the one after it and its last block (in
// that order, so the carried state is read before it is overwritten); the others walk the
// middle blocks, each re-reading the previous block's overlapping tokens.
constexpr int kFullCPT = 4;                       // channels per thread (d <= 1024)

struct Online {
  float M, Z, A;
  __device__ __forceinline__ void empty() { M = -__builtin_huge_valf(); Z = 0.f; A = 0.f; }
  __device__ __forceinline__ void add(float z, float x) {
    const float Mn = fmaxf(M, z);
    const float f_old = __expf(M - Mn);         // 0 when M = -inf
    const float f_new = __expf(z - Mn);
    Z = Z * f_old + f_new;
    A = A * f_old + x * f_new;
    M = Mn;
  }
};

__global__ __launch_bounds__(kCompressThreads) void compress_full_kernel(CompressArgs a) {
  const int b = blockIdx.x, y = blockIdx.y, ny = gridDim.y;
  const int row0 = a.cu_new[b];
  const int n = a.cu_new[b + 1] - row0;
  if (n <= 0) return;
  const int start = a.start_pos[b];
  const int m = a.m, d = a.d, coff = a.coff, w = coff * d;
  const int kb_first = start / m, kb_last = (start + n - 1) / m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* st = a.state + (int64_t)b * 3 * w;       // cur (M, Z, A) at 0, d, 2d; nxt at 3d, 4d, 5d
  __shared__ float red[kCompressThreads / 64];

  // this call's tokens [lo, hi) of one series (col 0: primary, d: overlapping) at channel c
  auto scan = [&](Online& o, int c, int col, int lo, int hi) __attribute__((always_inline)) {
    for (int tok = lo; tok < hi; ++tok) {
      const int64_t r = (int64_t)(row0 + tok - start) * a.row_stride + col + c;
      float z = compress_load_in(a.score, a.in_bf16, r);
      if (a.ape) z += a.ape[(int64_t)(tok % m) * w + col + c];
      o.add(z, compress_load_in(a.kv, a.in_bf16, r));
    }
  };
  // a stored triple with no weight (Z = 0: zeros of a fresh sequence, or a reset) is empty
  auto load_triple = [&](Online& o, int c, int off) __attribute__((always_inline)) {
    o.M = st[off + c];
    o.Z = st[off + d + c];
    o.A = st[off + 2 * d + c];
    if (o.Z == 0.f) o.empty();
  };
  auto save_triple = [&](const Online& o, int c, int off) __attribute__((always_inline)) {
    st[off + c] = o.M;
    st[off + d + c] = o.Z;
    st[off + 2 * d + c] = o.A;
  };

  auto do_block = [&](int kb) {
    const int blk_lo = kb * m;
    const int tok_lo = max(start, blk_lo), tok_hi = min(start + n, blk_lo + m);
    const bool complete = blk_lo + m <= start + n;
    const uint8_t* page = complete ? compress_entry_page(a, b, kb) : nullptr;
    float C[kFullCPT];
    Online cur[kFullCPT], nxt[kFullCPT];
#pragma unroll
    for (int k = 0; k < kFullCPT; ++k) {
      const int c = threadIdx.x + k * kCompressThreads;
      cur[k].empty();
      nxt[k].empty();
      C[k] = 0.f;
      if (c >= d) continue;
      if (kb == kb_first) {                      // resume from the state (empty when fresh)
        load_triple(cur[k], c, 0);
        if (coff == 2) load_triple(nxt[k], c, 3 * d);
      } else if (coff == 2) {                    // the previous block's overlapping tokens
        if (kb - 1 == kb_first) load_triple(cur[k], c, 3 * d);
        scan(cur[k], c, d, max(start, blk_lo - m), blk_lo);
      }
      scan(cur[k], c, 0, tok_lo, tok_hi);
      if (coff == 2 && kb == kb_last) scan(nxt[k], c, d, tok_lo, tok_hi);
      if (complete) C[k] = cur[k].A / cur[k].Z;
    }
    if (complete) {
      if (a.norm_w) {                            // RMSNorm over the d channels
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < kFullCPT; ++k) ss += C[k] * C[k];
        ss = warp_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < kCompressThreads / 64; ++i) tot += red[i];
        __syncthreads();                         // red is reused by the next block
        const float r = 1.f / __builtin_sqrtf(tot / (float)d + a.norm_eps);
#pragma unroll
        for (int k = 0; k < kFullCPT; ++k) {
          const int c = threadIdx.x + k * kCompressThreads;
          if (c < d) C[k] = C[k] * r * a.norm_w[c];
        }
      }
      if (a.rope_cos) {                          // GPT-J pairs (c, c ^ 1) of the last d_rope dims
        const int pos = min(m * kb, a.rope_rows - 1);
        const int half = a.d_rope / 2, r0 = d - a.d_rope;
#pragma unroll
        for (int k = 0; k < kFullCPT; ++k) {
          const int c = threadIdx.x + k * kCompressThreads;
          const float p = __shfl_xor(C[k], 1, 64);   // the pair's other member (lane ^ 1)
          if (c >= r0 && c < d) {
            const int j = (c - r0) >> 1;
            const float cs = a.rope_cos[(int64_t)pos * half + j], sn = a.rope_sin[(int64_t)pos * half + j];
            C[k] = (c & 1) ? p * sn + C[k] * cs : C[k] * cs - p * sn;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kFullCPT; ++k) {
        const int c = threadIdx.x + k * kCompressThreads;
        if (c < ((d + 63) & ~63)) compress_store(a, b, kb, kb_first, page, c, c < d, C[k]);
      }
    }
    if (kb == kb_last) {
#pragma unroll
      for (int k = 0; k < kFullCPT; ++k) {
        const int c = threadIdx.x + k * kCompressThreads;
        if (c >= d) continue;
        if (complete) {                          // the next entry starts with this block's overlap
          Online e;
          e.empty();
          save_triple(coff == 2 ? nxt[k] : e, c, 0);
          if (coff == 2) save_triple(e, c, 3 * d);
        } else {
          save_triple(cur[k], c, 0);
          if (coff == 2) save_triple(nxt[k], c, 3 * d);
        }
      }
    }
  };

  if (y == 0) {
    do_block(kb_first);
    if (kb_first + 1 < kb_last) do_block(kb_first + 1);
    if (kb_last != kb_first) do_block(kb_last);
  }
  const int workers = ny > 1 ? ny - 1 : 1;
  if (ny == 1 || y > 0) {
    const int w0 = ny > 1 ? y - 1 : 0;
    for (int kb = kb_first + 2 + w0; kb < kb_last; kb += workers) do_block(kb);
  }
}

}  // namespace

hipError_t launch_compress_full(const CompressArgs& a, int max_new, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  const int slots = std::min(65535, std::max(1, (max_new + a.m - 1) / a.m));
  hipLaunchKernelGGL(compress_full_kernel, dim3(a.B, slots), dim3(kCompressThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, int max_new, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_kernel, compress_grid(a, max_new), dim3(kCompressThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hcs
