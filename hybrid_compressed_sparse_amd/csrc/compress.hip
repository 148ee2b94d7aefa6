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

}  // namespace

hipError_t launch_compress(const CompressArgs& a, int max_new, hipStream_t stream) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(compress_kernel, compress_grid(a, max_new), dim3(kCompressThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace hcs
