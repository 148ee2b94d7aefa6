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

HCS_DEVICE_ERROR_WORD(compress)

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
// A workgroup covers all d channels of an entry (the norm needs them all): CPT per thread, the
// loads of all of a thread's channels issued together (one memory round trip for the carried
// state, the RMSNorm weights and the RoPE row, one per token). Workgroup y = 0 walks the call's
// first block, the one after it and its last block (in that order, so the carried state is
// read before it is overwritten); the others walk the middle blocks, each re-reading the
// previous block's overlapping tokens.
struct Online {
  float M, Z, A;
  __device__ __forceinline__ void empty() { M = -__builtin_huge_valf(); Z = 0.f; A = 0.f; }
  // a triple with no weight (Z = 0: the zeros of a fresh sequence, or a reset) is empty
  __device__ __forceinline__ void add(float z, float x) {
    const float Mo = Z == 0.f ? -__builtin_huge_valf() : M;
    const float Mn = fmaxf(Mo, z);
    const float f_old = __expf(Mo - Mn);        // 0 when empty
    const float f_new = __expf(z - Mn);
    Z = Z * f_old + f_new;
    A = A * f_old + x * f_new;
    M = Mn;
  }
};

template <int CPT, bool BF16>
__global__ __launch_bounds__(kCompressThreads) void compress_full_kernel(CompressArgs a) {
  const int b = blockIdx.x, y = blockIdx.y, ny = gridDim.y;
  const int row0 = a.cu_new[b];
  const int n = a.cu_new[b + 1] - row0;
  const int start = a.start_pos[b];
  if (n <= 0 || start < 0) return;               // (testing start too loads it beside n)
  const int m = a.m, d = a.d, coff = a.coff, w = coff * d;
  const int kb_first = start / m, kb_last = (start + n - 1) / m;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* st = a.state + (int64_t)b * 3 * w;       // cur (M, Z, A) at 0, d, 2d; nxt at 3d, 4d, 5d
  __shared__ float red[kCompressThreads / 64];
  // a thread's channels; loads use the clamped index so that they need no branch
  int cc[CPT];
  bool act[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = threadIdx.x + k * kCompressThreads;
    act[k] = c < d;
    cc[k] = min(c, d - 1);
  }

  // this call's tokens [lo, hi) of one series (col 0: primary, d: overlapping) into o[]
  auto scan = [&](Online* o, int col, int lo, int hi) __attribute__((always_inline)) {
    for (int tok = lo; tok < hi; ++tok) {
      const int64_t r = (int64_t)(row0 + tok - start) * a.row_stride + col;
      const float* ape = a.ape ? a.ape + (int64_t)(tok % m) * w + col : nullptr;
      float z[CPT], x[CPT], pe[CPT];
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        z[k] = compress_load_in<BF16>(a.score, r + cc[k]);
        x[k] = compress_load_in<BF16>(a.kv, r + cc[k]);
        pe[k] = 0.f;
      }
      if (ape) {
#pragma unroll
        for (int k = 0; k < CPT; ++k) pe[k] = ape[cc[k]];
      }
#pragma unroll
      for (int k = 0; k < CPT; ++k) o[k].add(z[k] + pe[k], x[k]);
    }
  };
  auto load_triples = [&](Online* o, int off) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      o[k].M = st[off + cc[k]];
      o[k].Z = st[off + d + cc[k]];
      o[k].A = st[off + 2 * d + cc[k]];
    }
  };
  auto save_triples = [&](const Online* o, int off) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      if (!act[k]) continue;
      st[off + cc[k]] = o[k].M;
      st[off + d + cc[k]] = o[k].Z;
      st[off + 2 * d + cc[k]] = o[k].A;
    }
  };

  auto do_block = [&](int kb) {
    const int blk_lo = kb * m;
    const int tok_lo = max(start, blk_lo), tok_hi = min(start + n, blk_lo + m);
    const bool complete = blk_lo + m <= start + n;
    const uint8_t* page = complete ? compress_entry_page(a, b, kb) : nullptr;
    Online cur[CPT], nxt[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      cur[k].empty();
      nxt[k].empty();
    }
    if (kb == kb_first) {                        // resume from the state (empty when fresh)
      load_triples(cur, 0);
      if (coff == 2) load_triples(nxt, 3 * d);
    } else if (coff == 2 && kb - 1 == kb_first) {
      load_triples(cur, 3 * d);
    }
    // epilogue operands (independent of the accumulation; clamped rows, used where they apply)
    float nw[CPT], rc[CPT], rs[CPT];
    const int r0 = d - a.d_rope, half = a.d_rope / 2;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
      nw[k] = 1.f;
      rc[k] = 1.f;
      rs[k] = 0.f;
    }
    if (complete && a.norm_w) {
#pragma unroll
      for (int k = 0; k < CPT; ++k) nw[k] = a.norm_w[cc[k]];
    }
    if (complete && a.rope_cos) {
      const int64_t row = (int64_t)min(m * kb, a.rope_rows - 1) * half;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int64_t ri = row + (max(cc[k] - r0, 0) >> 1);
        rc[k] = a.rope_cos[ri];
        rs[k] = a.rope_sin[ri];
      }
    }
    if (kb != kb_first && coff == 2) scan(cur, d, max(start, blk_lo - m), blk_lo);   // previous block's overlap
    scan(cur, 0, tok_lo, tok_hi);
    if (coff == 2 && kb == kb_last) scan(nxt, d, tok_lo, tok_hi);
    if (complete) {
      float C[CPT];
#pragma unroll
      for (int k = 0; k < CPT; ++k) C[k] = act[k] ? cur[k].A / cur[k].Z : 0.f;
      if (a.norm_w) {                            // RMSNorm over the d channels
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < CPT; ++k) ss += C[k] * C[k];
        ss = warp_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < kCompressThreads / 64; ++i) tot += red[i];
        __syncthreads();                         // red is reused by the next block
        const float r = 1.f / __builtin_sqrtf(tot / (float)d + a.norm_eps);
#pragma unroll
        for (int k = 0; k < CPT; ++k) C[k] = C[k] * r * nw[k];
      }
      if (a.rope_cos) {                          // GPT-J pairs (c, c ^ 1) of the last d_rope dims
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          const float p = __shfl_xor(C[k], 1, 64);   // the pair's other member (lane ^ 1)
          if (act[k] && cc[k] >= r0) C[k] = (cc[k] & 1) ? p * rs[k] + C[k] * rc[k] : C[k] * rc[k] - p * rs[k];
        }
      }
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int c = threadIdx.x + k * kCompressThreads;
        if (c < ((d + 63) & ~63)) compress_store(a, b, kb, kb_first, page, c, act[k], C[k]);
      }
    }
    if (kb == kb_last) {
      if (complete) {                            // the next entry starts with this block's overlap
        Online e[CPT];
#pragma unroll
        for (int k = 0; k < CPT; ++k) e[k].empty();
        save_triples(coff == 2 ? nxt : e, 0);
        if (coff == 2) save_triples(e, 3 * d);
      } else {
        save_triples(cur, 0);
        if (coff == 2) save_triples(nxt, 3 * d);
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
  const dim3 grid(a.B, slots), block(kCompressThreads);
  const int cpt = a.d <= kCompressThreads ? 1 : a.d <= 2 * kCompressThreads ? 2 : 4;
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, stream, a); };
  if (a.in_bf16) {
    if (cpt == 1) go(compress_full_kernel<1, true>);
    else if (cpt == 2) go(compress_full_kernel<2, true>);
    else go(compress_full_kernel<4, true>);
  } else {
    if (cpt == 1) go(compress_full_kernel<1, false>);
    else if (cpt == 2) go(compress_full_kernel<2, false>);
    else go(compress_full_kernel<4, false>);
  }
  return hipGetLastError();
}

hipError_t launch_compress(const CompressArgs& a, int max_new, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_kernel, compress_grid(a, max_new), dim3(kCompressThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hcs
