// Sparse MLA (single shared KV head) attention for gfx950.
//
// What it computes: "DeepSeek V4 Attention: Code Reading Map", section "Phase 3: forward_mqa()":
// every query head attends over the query's sliding-window rows plus its selected (CSA) or all
// visible (HCA) compressed entries; K and V are the same shared row.
//
// Design (one workgroup = one query x one split of its row list x up to 64 heads, 4 waves):
//   * the row list (window positions, then compressed ids) is walked in tiles of 32 rows; each
//     tile is gathered through the page tables with 16-byte loads (one wave reads a whole
//     1 KiB row for d = 512, so every row is one coalesced burst), prefetched into registers
//     one tile ahead and written to a double-buffered LDS tile; fp8_ds rows are dequantised to
//     bf16 on the way into LDS (e4m3 * 2^(scale-127) is exact in bf16);
//   * wave w owns heads 16w..16w+15 and keeps their q in registers (the B operand);
//     S^T = K Q^T is computed with v_mfma_f32_16x16x32_bf16 (rows on M, heads on N), so the
//     result already sits in the B-operand layout of P^T for O^T = V^T P^T: the probabilities
//     never leave registers;
//   * V^T is read from the same LDS tile with ds_read_b64_tr_b16, which transposes 16-bit
//     elements across each 16-lane group, so the tile is stored once and read both ways;
//   * online softmax in base 2 per head: each lane owns one head (lane % 16), the running max
//     is reduced over the 4 lane groups with two shuffles, O^T stays in 128 accumulator
//     registers per lane;
//   * when there are too few queries to fill the chip the row list is split; partial
//     (unnormalised O, max, sum) go to the workspace and a combine kernel merges them.
#include "kernels.h"

namespace hcs {

namespace {

constexpr int kTile = 32;
constexpr int kThreads = 256;
constexpr float kNegInf = -__builtin_huge_valf();

template <int D, int FMT>
struct RowLayout {
  static constexpr int kPageBytes = FMT == HCS_FMT_FP8DS ? kFp8PageBytes : kPageRows * D * 2;
  static constexpr int kLdsRow = D * 2 + 16;      // padded bf16 row in LDS
};

__device__ __forceinline__ i16x4 lds_read_tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 __attribute__((address_space(3)))*)(p));
}

// Resolve row `gr` of query's row list: returns the page base (or nullptr if the row does not
// take part) and its slot.
struct RowRef {
  const uint8_t* page;
  int slot;
};

template <int PAGE_BYTES>
__device__ __forceinline__ RowRef resolve_row(const AttnArgs& a, int t, int seq, int lo, int n_swa,
                                              int nv, int R, int gr) {
  RowRef r{nullptr, 0};
  if (gr < n_swa) {
    const int p = lo + gr;
    const int pg = page_of(a.swa, seq, p);
    if (pg >= 0) r = RowRef{a.swa.base + (int64_t)pg * PAGE_BYTES, p & 63};
  } else if (gr < R) {
    const int j = gr - n_swa;
    const int id = a.topk_idx ? __ldg(a.topk_idx + (int64_t)t * a.topk + j) : j;
    if (id >= 0 && id < nv) {
      const int pg = page_of(a.comp, seq, id);
      if (pg >= 0) r = RowRef{a.comp.base + (int64_t)pg * PAGE_BYTES, id & 63};
    }
  }
  return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Two e4m3 codes (bytes 0,1 or 2,3 of `w`) scaled by `sc` -> packed bf16x2 (exact).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, float sc) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  return (__float_as_uint(f.x * sc) >> 16) | (__float_as_uint(f.y * sc) & 0xffff0000u);
}

template <int D, int FMT>
__global__ __launch_bounds__(kThreads, 1) void sparse_mla_kernel(AttnArgs a) {
  using RL = RowLayout<D, FMT>;
  constexpr int KS = D / 32;          // k-steps of S^T = K Q^T
  constexpr int CT = D / 16;          // column tiles of O^T
  constexpr int LR = RL::kLdsRow;
  constexpr int PB = RL::kPageBytes;
  // bf16 staging: CH 16-byte chunks per row, RPP rows per pass of the 256 threads
  constexpr int CH = D * 2 / 16;
  constexpr int RPP = FMT == HCS_FMT_FP8DS ? 4 : kThreads / CH;
  constexpr int PASSES = kTile / RPP;

  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kTile * LR];
  __shared__ int lds_valid[2][kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int t = blockIdx.x / a.nsplit, s = blockIdx.x - (blockIdx.x / a.nsplit) * a.nsplit;
  const int hbase = blockIdx.y * 64 + wave * 16;
  const int head = hbase + l16;
  const bool wave_active = hbase < a.H;

  int seq, pos;
  if (a.q_seq) {
    seq = __ldg(a.q_seq + t);
    pos = min(__ldg(a.q_pos + t), a.pos_cap);
  } else {
    seq = a.seq_const;
    pos = a.p0 + t;
  }
  const int lo = max(0, pos - a.window + 1);
  const int n_swa = a.window > 0 ? pos - lo + 1 : 0;
  const int nv = min((pos + 1) / a.m, a.nv_cap);
  const int n_comp = a.topk_idx ? a.topk : nv;
  const int R = n_swa + n_comp;
  const int ntiles = (R + kTile - 1) / kTile;
  const int tile0 = s * a.tiles_per_split;
  const int tile1 = min(ntiles, tile0 + a.tiles_per_split);

  // ---- q of this wave's 16 heads as the B operand: lane -> head l16, dims 32ks + 8g .. +7
  bf16x8 qreg[KS];
  {
    const bool hv = head < a.H;
    const uint16_t* qrow = a.q + ((int64_t)t * a.H + (hv ? head : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4 v = hv ? *(const i32x4*)(qrow + 32 * ks + 8 * g) : i32x4{0, 0, 0, 0};
      qreg[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 oacc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) oacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // ---- staging registers
  i32x4 pre[PASSES];
  float psc[PASSES];
  bool pval[PASSES];
  const int chunk = FMT == HCS_FMT_FP8DS ? lane : (tid % CH);
  const int rsub = FMT == HCS_FMT_FP8DS ? wave : (tid / CH);

  auto load_tile = [&](int tt) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = p * RPP + rsub;
      const RowRef ref = resolve_row<PB>(a, t, seq, lo, n_swa, nv, R, tt * kTile + r);
      pval[p] = ref.page != nullptr;
      pre[p] = i32x4{0, 0, 0, 0};
      psc[p] = 1.f;
      if constexpr (FMT == HCS_FMT_FP8DS) {
        if (ref.page) {
          if (chunk < 28) {
            pre[p] = *(const i32x4*)(ref.page + kFp8PageCodes + ref.slot * kFp8Latent + chunk * 16);
            const int e = ref.page[kFp8PageScales + ref.slot * 8 + (chunk >> 2)];
            psc[p] = __builtin_ldexpf(1.f, e - 127);
          } else if (chunk < 36) {
            pre[p] = *(const i32x4*)(ref.page + kFp8PageRope + ref.slot * (kFp8Rope * 2) +
                                     (chunk - 28) * 16);
          }
        }
      } else {
        if (ref.page) pre[p] = *(const i32x4*)(ref.page + ref.slot * (D * 2) + chunk * 16);
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = p * RPP + rsub;
      uint8_t* row = lds[buf] + r * LR;
      if constexpr (FMT == HCS_FMT_FP8DS) {
        if (chunk < 28) {
          const float sc = psc[p];
          i32x4 lo4, hi4;
          lo4.x = e4m3x2_to_bf16x2<false>(pre[p].x, sc);
          lo4.y = e4m3x2_to_bf16x2<true>(pre[p].x, sc);
          lo4.z = e4m3x2_to_bf16x2<false>(pre[p].y, sc);
          lo4.w = e4m3x2_to_bf16x2<true>(pre[p].y, sc);
          hi4.x = e4m3x2_to_bf16x2<false>(pre[p].z, sc);
          hi4.y = e4m3x2_to_bf16x2<true>(pre[p].z, sc);
          hi4.z = e4m3x2_to_bf16x2<false>(pre[p].w, sc);
          hi4.w = e4m3x2_to_bf16x2<true>(pre[p].w, sc);
          *(i32x4*)(row + chunk * 32) = lo4;
          *(i32x4*)(row + chunk * 32 + 16) = hi4;
        } else if (chunk < 36) {
          *(i32x4*)(row + kFp8Latent * 2 + (chunk - 28) * 16) = pre[p];
        }
      } else {
        *(i32x4*)(row + chunk * 16) = pre[p];
      }
      if (chunk == 0) lds_valid[buf][r] = pval[p] ? 1 : 0;
    }
  };

  if (tile0 < tile1) {
    load_tile(tile0);
    store_tile(0);
  }
  __syncthreads();

  // lane-constant parts of the transposed V^T reads: group g reads rows 4g + (l16>>2)
  // (and +16), 8 bytes at column 4*(l16&3) of each 16-column tile
  const int tr_row = 4 * g + (l16 >> 2);
  const int tr_col = 4 * (l16 & 3);

  for (int tt = tile0; tt < tile1; ++tt) {
    const int buf = (tt - tile0) & 1;
    const bool more = tt + 1 < tile1;
    if (more) load_tile(tt + 1);

    if (wave_active) {
      const uint8_t* L = lds[buf];
      // ---- S^T = K Q^T : rows mt*16 + l16 are the A operand
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x8 av = *(const bf16x8*)(L + (mt * 16 + l16) * LR + (32 * ks + 8 * g) * 2);
          sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[ks], sacc[mt], 0, 0, 0);
        }
      }
      // ---- online softmax (base 2). lane holds rows mt*16 + 4g + i of head l16
      float x[8];
      float tmax = kNegInf;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mt * 16 + 4 * g + i;
          const float v = lds_valid[buf][row] ? sacc[mt][i] * a.scale_log2 : kNegInf;
          x[mt * 4 + i] = v;
          tmax = fmaxf(tmax, v);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(m_run, tmax);
      float alpha = 1.f;
      float p[8];
      if (mnew == kNegInf) {
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = 0.f;
      } else {
        alpha = __builtin_amdgcn_exp2f(m_run - mnew);
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(x[j] - mnew);
      }
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) psum += p[j];
      l_run = l_run * alpha + psum;
      m_run = mnew;
      i32x4 pk;
      pk.x = pack_bf16x2(p[0], p[1]);
      pk.y = pack_bf16x2(p[2], p[3]);
      pk.z = pack_bf16x2(p[4], p[5]);
      pk.w = pack_bf16x2(p[6], p[7]);
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk);
      // ---- O^T += V^T P^T
      const uint8_t* tra = L + tr_row * LR + tr_col * 2;
      const uint8_t* trb = tra + 16 * LR;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const i16x4 v0 = lds_read_tr16(tra + ct * 32);
        const i16x4 v1 = lds_read_tr16(trb + ct * 32);
        typedef short i16x8 __attribute__((ext_vector_type(8)));
        const i16x8 v = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        f32x4 acc = oacc[ct] * alpha;
        oacc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v), pb, acc,
                                                           0, 0, 0);
      }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (!wave_active) return;

  // ---- epilogue. lane holds O^T[c = 16ct + 4g + i][head l16]
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const bool hv = head < a.H;
  if (a.nsplit == 1) {
    float mfin = m_run;
    if (a.sink && hv) {
      const float s2 = a.sink[head] * 1.4426950408889634f;
      const float mm = fmaxf(m_run, s2);
      if (mm != kNegInf) {
        const float f = __builtin_amdgcn_exp2f(m_run - mm);
        l_tot = l_tot * f + __builtin_amdgcn_exp2f(s2 - mm);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) oacc[ct] = oacc[ct] * f;
        mfin = mm;
      }
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (hv) {
      uint16_t* orow = a.out + ((int64_t)t * a.H + head) * D;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const f32x4 o = oacc[ct] * inv;
        uint2 pk;
        pk.x = pack_bf16x2(o[0], o[1]);
        pk.y = pack_bf16x2(o[2], o[3]);
        *(uint2*)(orow + 16 * ct + 4 * g) = pk;
      }
      if (a.lse && g == 0)
        a.lse[(int64_t)t * a.H + head] =
            l_tot > 0.f ? (mfin + __builtin_log2f(l_tot)) * 0.6931471805599453f : kNegInf;
    }
  } else if (hv) {
    const int64_t part = ((int64_t)t * a.nsplit + s) * a.H + head;
    float* orow = a.ws_o + part * D;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) *(f32x4*)(orow + 16 * ct + 4 * g) = oacc[ct];
    if (g == 0) {
      a.ws_ml[part * 2 + 0] = m_run;
      a.ws_ml[part * 2 + 1] = l_tot;
    }
  }
}

// Merge the split partials of one (query, head): 64 threads, D/64 columns each.
template <int D>
__global__ __launch_bounds__(64) void sparse_mla_combine_kernel(AttnArgs a) {
  constexpr int PER = D / 64;
  const int t = blockIdx.x, head = blockIdx.y, tid = threadIdx.x;
  const int64_t base = (int64_t)t * a.nsplit * a.H + head;
  float M = kNegInf;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.ws_ml[(base + (int64_t)s * a.H) * 2]);
  const float s2 = a.sink ? a.sink[head] * 1.4426950408889634f : kNegInf;
  M = fmaxf(M, s2);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float L = 0.f;
  if (M != kNegInf) {
    L = __builtin_amdgcn_exp2f(s2 - M);
    for (int s = 0; s < a.nsplit; ++s) {
      const int64_t part = base + (int64_t)s * a.H;
      const float ms = a.ws_ml[part * 2], ls = a.ws_ml[part * 2 + 1];
      if (ls <= 0.f) continue;
      const float f = __builtin_amdgcn_exp2f(ms - M);
      L += ls * f;
      const float* o = a.ws_o + part * D + tid * PER;
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += f * o[j];
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* orow = a.out + ((int64_t)t * a.H + head) * D + tid * PER;
#pragma unroll
  for (int j = 0; j < PER; ++j) orow[j] = (uint16_t)f32_to_bf16_bits(acc[j] * inv);
  if (a.lse && tid == 0)
    a.lse[(int64_t)t * a.H + head] = L > 0.f ? (M + __builtin_log2f(L)) * 0.6931471805599453f : kNegInf;
}

template <int D, int FMT>
hipError_t launch_impl(const AttnArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)(a.N * a.nsplit), (unsigned)((a.H + 63) / 64));
  hipLaunchKernelGGL((sparse_mla_kernel<D, FMT>), grid, dim3(kThreads), 0, stream, a);
  if (a.nsplit > 1) {
    hipLaunchKernelGGL((sparse_mla_combine_kernel<D>), dim3(a.N, a.H), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

AttnPlan attn_plan(int N, int H, int d, int window, int m, int topk, int max_pos) {
  AttnPlan p{1, 1, 0};
  const int64_t nv = (int64_t)(max_pos + 1) / m;
  const int64_t rows = (int64_t)std::min(window, max_pos + 1) + (topk > 0 ? topk : nv);
  const int tiles = (int)std::max<int64_t>(1, (rows + kTile - 1) / kTile);
  const int64_t wgs = (int64_t)N * ((H + 63) / 64);
  const int64_t target = 512;
  int nsplit = 1;
  if (wgs > 0 && wgs < target) nsplit = (int)std::min<int64_t>(tiles, (target + wgs - 1) / wgs);
  const int tps = (tiles + nsplit - 1) / nsplit;
  nsplit = (tiles + tps - 1) / tps;
  p.nsplit = nsplit;
  p.tiles_per_split = tps;
  if (nsplit > 1) p.ws_bytes = (size_t)N * nsplit * H * (size_t)(d + 2) * sizeof(float);
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
