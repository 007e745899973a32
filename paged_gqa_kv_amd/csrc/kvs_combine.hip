// Split combine and block-mass reduction shared by every decode kernel
// (fp16, FP8 E4M3 and KIVI caches):
//   combine_splits    merges the splits of each (sequence, layer, head) into the
//                     fp16 output and the per-split normalising weights.
//   block_mass        sums the mass partials of every (layer, query head) into
//                     one fp32 number per (sequence, block), in a fixed order.
//
// Sources: "KV-Cache Offloading for LLM Inference -- Visual Reference"
// Sec. 2 (attention); "GQA Per-Head Scoring Streams" (head grouping, stream
// aggregation into one score per block).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvs.h"
#include "kvs_device.h"
#include "kvs_internal.h"

namespace kvs {
// ---------------------------------------------------------------------------
// combine_splits: one wave per (s, layer, head).  Lane handles d = 2 lane, +1.
//   M = max_k m_k, Lambda = sum_k l_k 2^(m_k - M), w_k = 2^(m_k - M) / Lambda,
//   out = sum_k w_k o_k (fp16), and w_k is kept for the mass reduction.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void combine_row(const CombineArgs& a, uint32_t w, int lane) {
  const int h = (int)(w % kQHeads);
  w /= kQHeads;
  const int lr = (int)(w % (uint32_t)a.n_layers);
  const int s = (int)(w / (uint32_t)a.n_layers);
  const int layer = a.layer_begin + lr;
  uint32_t* outp = reinterpret_cast<uint32_t*>(
      a.out + ((((size_t)s * a.num_layers + layer) * kQHeads + h) * kHeadDim));
  const size_t base = (((size_t)s * a.n_layers + lr) * kQHeads + h) * a.n_splits;
  const float2* orow = reinterpret_cast<const float2*>(a.opart + base * kHeadDim) + lane;

  // Loads whose addresses do not depend on the sequence's length are issued
  // before it is read: the lane's own split statistics (lane k holds split k)
  // and the first kPre splits' statistics and partial rows.  The workspace
  // holds n_splits of each per row, so every such load is in bounds; entries
  // past the sequence's own splits are stale and never used.
  constexpr int kPre = 8;
  const float2 mine = lane < a.n_splits ? a.ml[base + lane] : make_float2(-INFINITY, 0.f);
  float2 pv[kPre], pov[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int k = min(u, a.n_splits - 1);
    pv[u] = a.ml[base + k];
    pov[u] = orow[(size_t)k * (kHeadDim / 2)];
  }

  int r0 = 0;
  const int nb = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                            false, &r0);
  if (nb <= 0) {
    outp[lane] = 0u;
    return;
  }
  const int nsp = (nb + a.split_blocks - 1) / a.split_blocks;

  float M = -INFINITY;
  if (lane < nsp) M = fmaxf(M, mine.x);
  for (int k = lane + 64; k < nsp; k += 64) M = fmaxf(M, a.ml[base + k].x);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, xor_f(M, m));
  double L = 0.0;
  if (M != -INFINITY) {
    if (lane < nsp) L += (double)mine.y * (double)__builtin_amdgcn_exp2f(mine.x - M);
    for (int k = lane + 64; k < nsp; k += 64) {
      const float2 v = a.ml[base + k];
      L += (double)v.y * (double)__builtin_amdgcn_exp2f(v.x - M);
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) L += __shfl_xor(L, m, 64);
  const bool dead = !(L > 0.0);
  const double invL = dead ? 0.0 : 1.0 / L;

  if (lane < nsp)
    a.wsplit[base + lane] = dead ? 0.f : (float)((double)__builtin_amdgcn_exp2f(mine.x - M) * invL);
  for (int k = lane + 64; k < nsp; k += 64) {
    const float2 v = a.ml[base + k];
    a.wsplit[base + k] = dead ? 0.f : (float)((double)__builtin_amdgcn_exp2f(v.x - M) * invL);
  }
  // Weighted sum of the partial outputs in split order: the prefetched splits
  // first, then rounds of eight whose statistics and partial rows are all
  // loaded before the first is used (eight 512-byte rows in flight per wave).
  float o0 = 0.f, o1 = 0.f;
  auto add_split = [&](float2 v, float2 ov) {
    const float wk = dead ? 0.f : (float)((double)__builtin_amdgcn_exp2f(v.x - M) * invL);
    o0 = fmaf(wk, ov.x, o0);
    o1 = fmaf(wk, ov.y, o1);
  };
#pragma unroll
  for (int u = 0; u < kPre; ++u)
    if (u < nsp) add_split(pv[u], pov[u]);
  int k = kPre;
  for (; k + 8 <= nsp; k += 8) {
    float2 v[8], ov[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u] = a.ml[base + k + u];
      ov[u] = orow[(size_t)(k + u) * (kHeadDim / 2)];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) add_split(v[u], ov[u]);
  }
  for (; k < nsp; ++k) add_split(a.ml[base + k], orow[(size_t)k * (kHeadDim / 2)]);
  const _Float16 h0 = (_Float16)o0, h1 = (_Float16)o1;
  outp[lane] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
}

__global__ void __launch_bounds__(64) combine_splits(CombineArgs a) {
  combine_row(a, blockIdx.x, threadIdx.x);
}

// ---------------------------------------------------------------------------
// block_mass: mass[s, b] = sum over (layer, query head) of pi * w_split, fp64
// accumulation in a fixed order, so the result depends only on logical
// indices.  A work-group takes 32 blocks; its 32 row streams (two per wave:
// lanes 0..31 and 32..63, each reading 128 contiguous bytes of a row) take rows
// q, q + 32, q + 64, ... in order, and the 32 stream sums are added in stream
// order.  32 blocks per work-group (not 64) gives a 128K-token sequence 256
// work-groups, one per compute unit: with 128, half the chip's load slots sat
// idle and the kernel read at half the rate.
// ---------------------------------------------------------------------------
// Mass of the 32 blocks of column group cg of sequence s, with the weight of
// (row, split) at wt[row * wstride + split].
__device__ __forceinline__ void mass_columns(const MassArgs& a, int s, int cg, int nb, int r0,
                                             const float* wt, int wstride,
                                             double (*red)[kMassCols]) {
  constexpr int kStreams = kMassThreads / kMassCols;
  const int col = threadIdx.x % kMassCols;
  const int q = threadIdx.x / kMassCols;     // row stream; a wave holds two
  const int b = cg * kMassCols + col;
  const bool act = b < nb;
  const int r = r0 + (act ? b : 0);
  const int split = (act ? b : 0) / a.split_blocks;
  const int rows = a.n_layers * kQHeads;
  double acc = 0.0;
  if (act) {
    const float* pcol = a.pi + r;
    const float* wcol = wt + split;
    // Rounds of 16 rows: all 32 loads of a round are issued before the first
    // product (rows past the end re-read the last row, unconditionally, so no
    // load sits behind a branch); the sum runs in row order and skips them.
    constexpr int kRound = 16;
    for (int row0 = q; row0 < rows; row0 += kStreams * kRound) {
      float pv[kRound], wv[kRound];
#pragma unroll
      for (int u = 0; u < kRound; ++u) {
        const int row = min(row0 + u * kStreams, rows - 1);
        pv[u] = pcol[(size_t)row * a.total_blocks];
        wv[u] = wcol[(size_t)row * wstride];
      }
#pragma unroll
      for (int u = 0; u < kRound; ++u)
        if (row0 + u * kStreams < rows) acc += (double)pv[u] * (double)wv[u];
    }
  }
  red[q][col] = acc;
  __syncthreads();
  if (q == 0 && act) {
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < kStreams; ++k) t += red[k][col];
    if (a.accumulate) t += (double)a.mass[r];
    a.mass[r] = (float)t;
  }
}

__global__ void __launch_bounds__(kMassThreads) block_mass(MassArgs a) {
  __shared__ double red[kMassThreads / kMassCols][kMassCols];
  const int s = blockIdx.y;
  int r0 = 0;
  const int nb = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                            false, &r0);
  if (nb <= 0 || (int)blockIdx.x * kMassCols >= nb) return;
  const float* wt = a.wsplit + (size_t)s * a.n_layers * kQHeads * a.n_splits;
  mass_columns(a, s, blockIdx.x, nb, r0, wt, a.n_splits, red);
}

// ---------------------------------------------------------------------------
// combine_mass: both steps above in one launch, for small problems, where the
// launch and the wait between the two kernels are a visible part of the step
// (8 sequences x 8K tokens x 4 layers: 5.5 + 4.7 us of kernels in a 0.2 ms
// step).  The first work-groups combine 16 (sequence, layer, head) rows each,
// one per wave.  The others reduce the mass of 32 blocks, computing the split
// weights they need themselves from the split statistics: per (layer, head)
// row, M = max_k m_k, Lambda = sum_k l_k 2^(m_k - M) in split order, w_k =
// 2^(m_k - M) / Lambda, into LDS.  That costs every mass work-group a read of
// all its sequence's statistics, which is why it is kept for small problems.
// ---------------------------------------------------------------------------
constexpr int kFusedMaxWeights = 4096;   // (layer, head) rows x splits in LDS
constexpr int kFusedRegSplits = 16;      // rows of up to this many splits load them at once

__global__ void __launch_bounds__(kMassThreads) combine_mass(CombineArgs c, MassArgs a,
                                                             uint32_t comb_wgs,
                                                             uint32_t col_groups) {
  constexpr uint32_t kRowsPerWg = kMassThreads / 64;
  if (blockIdx.x < comb_wgs) {
    const uint32_t row = blockIdx.x * kRowsPerWg + (threadIdx.x >> 6);
    const uint32_t total_rows = (gridDim.x - comb_wgs) / col_groups * (uint32_t)c.n_layers * kQHeads;
    if (row < total_rows) combine_row(c, row, threadIdx.x & 63);
    return;
  }
  __shared__ double red[kMassThreads / kMassCols][kMassCols];
  __shared__ float wl[kFusedMaxWeights];
  const uint32_t mw = blockIdx.x - comb_wgs;
  const int s = (int)(mw / col_groups);
  const int cg = (int)(mw % col_groups);
  const int rows = a.n_layers * kQHeads;
  // With one row per thread and every row's splits fitting the registers, the
  // statistics are loaded before the sequence's length is read (in bounds:
  // the workspace holds n_splits per row; those past the sequence's own
  // splits are stale and skipped below).
  const bool early = a.n_splits <= kFusedRegSplits && rows <= kMassThreads;
  float2 pre[kFusedRegSplits];
  {
    // threads past the last row re-read it (unused)
    const float2* st = c.ml + ((size_t)s * rows + min((int)threadIdx.x, rows - 1)) * a.n_splits;
#pragma unroll
    for (int k = 0; k < kFusedRegSplits; ++k)
      pre[k] = early ? st[min(k, a.n_splits - 1)] : make_float2(0.f, 0.f);
  }
  int r0 = 0;
  const int nb = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                            false, &r0);
  if (nb <= 0 || cg * kMassCols >= nb) return;
  const int nsp = (nb + a.split_blocks - 1) / a.split_blocks;
  for (int row = threadIdx.x; row < rows; row += kMassThreads) {
    const float2* st = c.ml + ((size_t)s * rows + row) * a.n_splits;
    if (nsp <= kFusedRegSplits) {
      // The row's statistics in registers, all loads issued at once (indices
      // past nsp re-read the last split and are skipped): the loops below
      // would otherwise wait for one load per split, three times over.
      float2 v[kFusedRegSplits];
      if (early) {
#pragma unroll
        for (int k = 0; k < kFusedRegSplits; ++k) v[k] = pre[k];
      } else {
#pragma unroll
        for (int k = 0; k < kFusedRegSplits; ++k) v[k] = st[min(k, nsp - 1)];
      }
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < kFusedRegSplits; ++k)
        if (k < nsp) M = fmaxf(M, v[k].x);
      double L = 0.0;
      if (M != -INFINITY) {
#pragma unroll
        for (int k = 0; k < kFusedRegSplits; ++k)
          if (k < nsp) L += (double)v[k].y * (double)__builtin_amdgcn_exp2f(v[k].x - M);
      }
      const bool dead = !(L > 0.0);
      const double invL = dead ? 0.0 : 1.0 / L;
#pragma unroll
      for (int k = 0; k < kFusedRegSplits; ++k)
        if (k < nsp)
          wl[row * nsp + k] = dead ? 0.f : (float)((double)__builtin_amdgcn_exp2f(v[k].x - M) * invL);
      continue;
    }
    float M = -INFINITY;
    for (int k = 0; k < nsp; ++k) M = fmaxf(M, st[k].x);
    double L = 0.0;
    if (M != -INFINITY)
      for (int k = 0; k < nsp; ++k) L += (double)st[k].y * (double)__builtin_amdgcn_exp2f(st[k].x - M);
    const bool dead = !(L > 0.0);
    const double invL = dead ? 0.0 : 1.0 / L;
    for (int k = 0; k < nsp; ++k)
      wl[row * nsp + k] = dead ? 0.f : (float)((double)__builtin_amdgcn_exp2f(st[k].x - M) * invL);
  }
  __syncthreads();
  mass_columns(a, s, cg, nb, r0, wl, nsp, red);
}

hipError_t launch_combine(const CombineArgs& a, int batch, hipStream_t stream) {
  const uint64_t wgs = (uint64_t)batch * a.n_layers * kQHeads;
  hipLaunchKernelGGL(combine_splits, dim3((uint32_t)wgs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine_mass(const CombineArgs& c, const MassArgs& a, int batch,
                               hipStream_t stream) {
  const uint64_t rows = (uint64_t)a.n_layers * kQHeads;
  const uint64_t col_groups = ((uint64_t)a.max_nb + kMassCols - 1) / kMassCols;
  const uint64_t weights = rows * (uint64_t)a.n_splits;
  // fused while the weights fit the LDS table and the statistics every mass
  // work-group re-reads stay under 2 MiB in total
  if (a.total_blocks > 0 && weights <= (uint64_t)kFusedMaxWeights &&
      weights * 8u * col_groups * (uint64_t)batch <= (2ull << 20)) {
    const uint64_t comb_wgs = ((uint64_t)batch * rows + kMassThreads / 64 - 1) / (kMassThreads / 64);
    const uint64_t wgs = comb_wgs + col_groups * (uint64_t)batch;
    hipLaunchKernelGGL(combine_mass, dim3((uint32_t)wgs), dim3(kMassThreads), 0, stream, c, a,
                       (uint32_t)comb_wgs, (uint32_t)col_groups);
    return hipGetLastError();
  }
  hipError_t e = launch_combine(c, batch, stream);
  if (e != hipSuccess || a.total_blocks <= 0) return e;
  return launch_mass(a, batch, stream);
}

hipError_t launch_mass(const MassArgs& a, int batch, hipStream_t stream) {
  const dim3 grid((a.max_nb + kMassCols - 1) / kMassCols, batch);
  hipLaunchKernelGGL(block_mass, grid, dim3(kMassThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvs

