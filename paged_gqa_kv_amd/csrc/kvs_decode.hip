// Paged GQA decode kernel over fp16 and FP8 E4M3 pools:
//   paged_decode_gqa  split-K decode: one wave per (sequence, layer, KV head,
//                     split of blocks); QK^T and PV on MFMA; online softmax;
//                     per-(layer, head, block) probability-mass partials.
// The split combine and block-mass reduction that follow it are in
// kvs_combine.hip.
//
// Sources: "KV-Cache Offloading for LLM Inference -- Visual Reference"
// Sec. 2 (attention), Sec. 11 (EMA), Sec. 12 (priority, cut points);
// "GQA Per-Head Scoring Streams" (head grouping, stream aggregation, the
// 64-byte record); "KV cache offload" post, "Top row" (block tables);
// "Fitting a Million Tokens", Sec. 02 (FP8 E4M3 and KIVI 2-bit KV).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvs.h"
#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_decode_tiles.h"

namespace kvs {

// ---------------------------------------------------------------------------
// paged_decode_gqa
//
// One 64-lane wave owns (s, layer, split) and F::kHeads adjacent KV heads from
// g: two for E4M3; for fp16 one, or two when the sequences fill their splits
// (the host's choice, DecodeArgs::kv_heads).  Lane l = 16 j + c.
//  QK:  S^T[token][col] = K[token][:] . q[col][:] on v_mfma_f32_16x16x32_f16,
//       A = a 16x128 key tile (lane reads 64 contiguous bytes of row c), B =
//       the queries: column c holds query head 8 g + c for c < 8 F::kHeads, the
//       rest are zero.  With two KV heads, column c belongs to head g + c / 8
//       and takes its logits from that head's MFMA chain.  Lane (j, c) gets
//       the logits of column c for tokens 4j..4j+3.
//  PV:  O^T[d][col] += V^T[d][token] P^T[token][col] on
//       v_mfma_f32_16x16x16_f16.  P^T is exactly the QK result layout (after
//       rounding to fp16).  V^T needs the value tile transposed: it is staged
//       through 4 KiB of LDS, each lane reads 4 rows x 16 bytes, and byte
//       permutes build the operand of each of the 8 output tiles.  Output tile
//       k holds d = 8 m + k, so lane (j, c) ends with the 32 contiguous values
//       d in [32 j, 32 j + 32) of column c.  With two KV heads each head's
//       value tile is multiplied by P^T with the other head's columns zeroed,
//       so every column accumulates only its own head's values.
//  Online softmax in base 2: logits are scaled by scale * log2(e); a running
//  maximum per column; the per-block mass of each column is kept in LDS
//  relative to the current maximum and rescaled whenever that maximum grows.
//  Per column the arithmetic does not depend on F::kHeads (the other head's
//  PV product adds exact zeros), as long as the stored values are finite.
// ---------------------------------------------------------------------------
// Blocks whose loads are in flight per wave: the ring slot being processed
// plus kRing - 1 ahead (32 VGPRs per slot).  Deeper rings at lower occupancy
// measured no faster on gfx950.  One wave per work-group: work-groups of 4 or
// 8 waves reading neighbouring heads measured no faster for fp16.
template <class F>
__global__ void __launch_bounds__(64, F::kWavesPerSimd) paged_decode_gqa(DecodeArgs a) {
  static_assert(F::kPer == 1, "one block per step");
  constexpr int kHeads = F::kHeads;
  constexpr int kCols = kGroup * kHeads;              // MFMA columns holding query heads
  constexpr uint32_t kWaveGroups = 8u / kHeads;       // waves per (layer, split)
  constexpr int kGroupShift = kHeads == 1 ? 3 : 2;    // log2(kWaveGroups)
  static_assert((1u << kGroupShift) == kWaveGroups, "power-of-two head groups");
  extern __shared__ __align__(16) uint8_t smem[];
  const int SB = a.split_blocks;
  // LDS layout (decode_lds_bytes): block ids, mass partials, value stage.
  const int SP = decode_pi_stride(SB, kHeads);        // row stride of the mass partials
  const int ids = kHeads == 1 ? SB : (SB + 3) & ~3;
  int32_t* tbl = reinterpret_cast<int32_t*>(smem);                          // [SB] block ids
  float* pi_lds = reinterpret_cast<float*>(smem + (size_t)4 * ids);         // [kCols][SP]
  u4_t* vstage = reinterpret_cast<u4_t*>(smem + (size_t)4 * ids + (size_t)4 * kCols * SP);

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int j = lane >> 4;

  uint32_t w = xcd_item(blockIdx.x, gridDim.x);
  const uint32_t lgg_count = (uint32_t)a.n_layers * kWaveGroups;
  const int lgg = (int)(w % lgg_count);
  w /= lgg_count;
  const int split = (int)(w % (uint32_t)a.n_splits);
  const int s = (int)(w / (uint32_t)a.n_splits);
  const int lr = lgg >> kGroupShift;
  const int g = (lgg & (int)(kWaveGroups - 1)) * kHeads;   // first KV head of the wave
  const int layer = a.layer_begin + lr;

  int r0 = 0;
  const bool report = (threadIdx.x == 0) && split == 0 && lgg == 0;
  const int nb = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                            report, &r0);
  const int b0 = split * SB;
  if (nb < 0 || b0 >= nb) return;
  const int b1 = min(nb, b0 + SB);
  const int n = a.seq_lens[s];

  // The split's block ids go to LDS once, so that no later block-id read waits
  // on the vector-memory counter behind the in-flight K/V loads.
  for (int i = threadIdx.x; i < b1 - b0; i += 64)
    tbl[i] = a.table[(size_t)s * a.max_nb + b0 + i];
  __syncthreads();

  // B operand of QK: query heads 8 g .. 8 g + kCols - 1, other columns zero.
  h8_t qb[4];
  if (c < kCols) {
    const uint16_t* qp =
        a.q + ((((size_t)s * a.num_layers + layer) * kQHeads + kGroup * g + c) * kHeadDim);
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = *reinterpret_cast<const h8_t*>(qp + qk_elem<F>(i, j));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = h8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  constexpr int64_t kLayerBytes = 16 * (int64_t)tile_bytes<F>();   // one block, one layer
  const size_t block_stride = (size_t)a.num_layers * kLayerBytes;
  const size_t tile_off = (size_t)layer * kLayerBytes + (size_t)g * tile_bytes<F>();
  float m_run = -INFINITY;
  f4_t acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};

  // Physical block of logical block bidx of this split; positions past the
  // split's end reuse its last block (a cached, in-bounds tile whose data is
  // masked), and ids outside the pool read block 0 and are masked.
  auto slot_block = [&](int bidx, bool* ok) -> const uint8_t* {
    const int clamped = min(bidx, b1 - 1);
    const int pid = tbl[clamped - b0];
    const bool in_pool = pid >= 0 && (int64_t)pid < a.pool_blocks;
    *ok = in_pool && bidx < b1;
    return a.pool + (size_t)(in_pool ? pid : 0) * block_stride + tile_off;
  };

  constexpr int kRing = F::kRing;
  StepRegs<F> ring[kRing];
  bool ring_ok[kRing];
  // the wave's heads' tiles of block bidx (adjacent: the key tiles form one
  // run, the value tiles another)
  auto load_step = [&](StepRegs<F>& r, bool& ok, int bidx) {
    const uint8_t* base = slot_block(bidx, &ok);
#pragma unroll
    for (int h = 0; h < kHeads; ++h)
      load_block(r.blk[h], base + (size_t)h * tile_bytes<F>(), lane, c, j);
  };
#pragma unroll
  for (int k = 0; k < kRing; ++k) load_step(ring[k], ring_ok[k], b0 + k);

  bool saw_bad = false;
  for (int bbase = b0; bbase < b1; bbase += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int bs = bbase + k;        // this step's block
      const bool active = bs < b1;
      saw_bad |= active && !ring_ok[k];
      const int valid = ring_ok[k] ? min(16, n - 16 * bs) : 0;

      // ---- value tiles to LDS (the slot's value registers are free after this)
#pragma unroll
      for (int h = 0; h < kHeads; ++h) stage_values<F>(ring[k].blk[h], vstage, lane, h);

      // ---- logits of 16 tokens x 16 columns per head
      f4_t sacc[kHeads];
#pragma unroll
      for (int h = 0; h < kHeads; ++h) sacc[h] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int h = 0; h < kHeads; ++h)
          sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand<F>(ring[k].blk[h], i),
                                                           qb[i], sacc[h], 0, 0, 0);

      // ---- refill this slot with the step kRing ahead
      load_step(ring[k], ring_ok[k], bs + kRing);

      // the lane's column belongs to head g + c / 8
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[0][i];
        if constexpr (kHeads == 2) x = c < kGroup ? sacc[0][i] : sacc[1][i];
        sv[i] = x * a.scale_log2;
      }
      if (valid < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * j + i >= valid) sv[i] = -INFINITY;
      }

      // ---- online softmax over the block (per column; the 4 lanes j share one)
      float bm = -INFINITY;
      bm = fmaxf(bm, fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      bm = head_max4(bm);
      const float m_new = fmaxf(m_run, bm - kProbShift);   // reference below the maximum
      const bool live = m_new != -INFINITY;
      const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = live ? __builtin_amdgcn_exp2f(sv[i] - m_new) : 0.f;
      const float bsum = head_sum4((pv[0] + pv[1]) + (pv[2] + pv[3]));

      if (__ballot(c < kCols && alpha != 1.f) != 0ull) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] *= alpha;
        if (c < kCols) {
          if constexpr (kHeads == 2) {   // four partials per LDS access (rows 16-byte aligned)
            f4_t* row = reinterpret_cast<f4_t*>(pi_lds + c * SP);
            for (int v = j; 4 * v < bs - b0; v += 4) row[v] *= alpha;
          } else {
            for (int idx = j; idx < bs - b0; idx += 4) pi_lds[c * SP + idx] *= alpha;
          }
        }
      }
      if (active && c < kCols && j == 0) pi_lds[c * SP + (bs - b0)] = bsum;
      m_run = m_new;

      // ---- PV: transposed value rows from LDS, one head at a time
      const h4_t pb = h4_t{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
#pragma unroll
      for (int h = 0; h < kHeads; ++h) {
        u4_t R[4];
        value_rows<F>(vstage, h, j, c, R);
        if (valid < 16) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * j + i >= valid) R[i] = u4_t{0u, 0u, 0u, 0u};
        }
        // columns of the other head take no part in this head's product
        const h4_t ph = (kHeads == 1 || (c >> 3) == h) ? pb : h4_t{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t lo01 = __builtin_amdgcn_perm(R[1][q], R[0][q], 0x05040100u);
          const uint32_t lo23 = __builtin_amdgcn_perm(R[3][q], R[2][q], 0x05040100u);
          const uint32_t hi01 = __builtin_amdgcn_perm(R[1][q], R[0][q], 0x07060302u);
          const uint32_t hi23 = __builtin_amdgcn_perm(R[3][q], R[2][q], 0x07060302u);
          acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(
              __builtin_bit_cast(h4_t, u2_t{lo01, lo23}), ph, acc[2 * q], 0, 0, 0);
          acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(
              __builtin_bit_cast(h4_t, u2_t{hi01, hi23}), ph, acc[2 * q + 1], 0, 0, 0);
        }
      }
    }
  }
  if (saw_bad && lane == 0) flag(a.status, KVS_DEV_BAD_BLOCK_ID);

  // ---- split epilogue: statistics, partial output, mass partials
  const size_t st = (((size_t)s * a.n_layers + lr) * kQHeads + kGroup * g + c) * a.n_splits + split;
  if (c < kCols) {
    float* op = a.opart + st * kHeadDim + 32 * j;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f4_t*>(op + 8 * i) = f4_t{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *reinterpret_cast<f4_t*>(op + 8 * i + 4) = f4_t{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
  }
  __syncthreads();
  const int cnt = b1 - b0;
  const float lt = split_norm<kCols>(pi_lds, SP, lane, cnt, cnt);
  if (c < kCols && j == 0) a.ml[st] = make_float2(m_run, lt);
  // four rows at a time, so that four LDS reads are in flight per store round
  for (int hh = 0; hh < kCols; hh += 4) {
    float* dst = a.pi + ((size_t)lr * kQHeads + kGroup * g + hh) * a.total_blocks + r0 + b0;
    for (int bb = lane; bb < cnt; bb += 64) {
      float x[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) x[t] = pi_lds[(hh + t) * SP + bb];
#pragma unroll
      for (int t = 0; t < 4; ++t) dst[(size_t)t * a.total_blocks + bb] = x[t];
    }
  }
}

static_assert(decode_lds_bytes(1024, KvE4M3::kHeads) <= kMaxDecodeLds,
              "largest E4M3 split must fit the LDS bound");
static_assert(decode_lds_bytes(1024, 2, 2 * tile_bytes<KvF16x2>()) <= kMaxDecodeLds,
              "largest two-head fp16 split must fit the LDS bound");

hipError_t launch_decode(const DecodeArgs& a, int batch, hipStream_t stream) {
  if (a.kv_format == KVS_KV_KIVI2) return launch_decode_kivi(a, batch, stream);
  if (a.pair_role) return launch_decode_pair(a, batch, stream);
  // one wave per (sequence, split, layer, group of F::kHeads KV heads)
  const uint64_t items = (uint64_t)batch * a.n_splits * a.n_layers;
  if (a.kv_format == KVS_KV_E4M3) {
    const size_t lds = decode_lds_bytes(a.split_blocks, KvE4M3::kHeads);
    if (lds > kMaxDecodeLds) return hipErrorInvalidValue;
    const uint64_t wgs = items * (8u / KvE4M3::kHeads);
    hipLaunchKernelGGL(paged_decode_gqa<KvE4M3>, dim3((uint32_t)wgs), dim3(64), lds, stream, a);
  } else if (a.kv_heads == 2) {
    const size_t lds = decode_lds_bytes(a.split_blocks, 2, 2 * tile_bytes<KvF16x2>());
    if (lds > kMaxDecodeLds) return hipErrorInvalidValue;
    hipLaunchKernelGGL(paged_decode_gqa<KvF16x2>, dim3((uint32_t)(items * 4u)), dim3(64), lds,
                       stream, a);
  } else {
    const size_t lds = decode_lds_bytes(a.split_blocks);
    if (lds > kMaxDecodeLds) return hipErrorInvalidValue;
    hipLaunchKernelGGL(paged_decode_gqa<KvF16>, dim3((uint32_t)(items * 8u)), dim3(64), lds,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace kvs
