// Paired paged decode over an fp16 pool:
//   paged_decode_pair  the decode of paged_decode_gqa, where one wave serves
//                      two sequences of the batch that share blocks (the
//                      refcounted blocks of a prefix cache): each block the two
//                      hold at the same logical position is loaded once and
//                      scored for both.
//
// Sources: "KV-Cache Offloading for LLM Inference -- Visual Reference"
// Sec. 2 (attention); "GQA Per-Head Scoring Streams" (head grouping, per-block
// mass); "KV cache offload" post, "Top row" (block tables of physical ids,
// refcounted blocks shared between sequences).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvs.h"
#include "kvs_device.h"
#include "kvs_internal.h"
#include "kvs_decode_tiles.h"

namespace kvs {

// ---------------------------------------------------------------------------
// paged_decode_pair
//
// The QK operand's 16 columns hold the 8 query heads of the group for two
// sequences: columns 0..7 for sequence A, 8..15 for sequence B (lanes with
// c >= 8, "hi", carry B).  Both sequences walk the split's logical positions
// in order.  At a position where both hold the same physical block, one step
// loads it and both column groups are live; otherwise A's block and then B's
// block get a step each, with the other group's logits masked to -inf.  A
// masked step is an exact no-op for the masked group (p = 0, rescale factor
// 1, nothing added), and every column's arithmetic is the one paged_decode_gqa
// does for its head, in the same order, so each sequence's output, statistics
// and mass partials are bit-identical to the unpaired decode.
//
// Pairs come from the caller's pair_role array: role[a] = b and role[b] =
// -2 - a link sequences a and b.  A split is decoded jointly, by the wave of
// the lower sequence a, when the link is mutual, both sequences are valid and
// both hold the split's first block as the same physical block; the wave of b
// then exits.  Both waves evaluate the same condition on the same data, so
// every (sequence, split) is decoded exactly once whatever the array holds.
// ---------------------------------------------------------------------------
namespace {

// Joint decode of split `split` by the pair (a, b)?
__device__ __forceinline__ bool joint_split(const DecodeArgs& a, int sa, int sb_, int split) {
  int ra = 0, rb = 0;
  const int nba = seq_blocks(a.seq_lens, a.meta_off, sa, a.max_nb, a.total_blocks, a.status,
                             false, &ra);
  const int nbb = seq_blocks(a.seq_lens, a.meta_off, sb_, a.max_nb, a.total_blocks, a.status,
                             false, &rb);
  const int b0 = split * a.split_blocks;
  if (nba < 0 || nbb < 0 || b0 >= nba || b0 >= nbb) return false;
  return a.table[(size_t)sa * a.max_nb + b0] == a.table[(size_t)sb_ * a.max_nb + b0];
}

// One step of the pair's walk: the block to load, which column groups are
// live (bit 0: A, bit 1: B) and the logical position.
struct PairStep {
  int pid;
  int mask;
  int b;
};

}  // namespace

// The LDS of a paired split keeps at most 2 work-groups per SIMD; the launch
// bound gives the kernel their VGPR budget (178, no spills).
__global__ void __launch_bounds__(64, 2) paged_decode_pair(DecodeArgs a) {
  using F = KvF16;
  extern __shared__ __align__(16) uint8_t smem[];
  const int SB = a.split_blocks;
  // LDS layout (decode_pair_lds_bytes): block ids of A and B, mass partials of
  // the 16 columns, value stage.
  int32_t* tbl = reinterpret_cast<int32_t*>(smem);                          // [2][SB]
  float* pi_lds = reinterpret_cast<float*>(smem + (size_t)8 * SB);          // [16][SB]
  u4_t* vstage = reinterpret_cast<u4_t*>(smem + (size_t)72 * SB);           // 4 KiB

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int j = lane >> 4;
  const bool hi = c >= kGroup;

  uint32_t w = xcd_item(blockIdx.x, gridDim.x);
  const uint32_t lgg_count = (uint32_t)a.n_layers * 8u;
  const int lgg = (int)(w % lgg_count);
  w /= lgg_count;
  const int split = (int)(w % (uint32_t)a.n_splits);
  const int s = (int)(w / (uint32_t)a.n_splits);
  const int batch = (int)(gridDim.x / (lgg_count * (uint32_t)a.n_splits));
  const int lr = lgg >> 3;
  const int g = lgg & 7;
  const int layer = a.layer_begin + lr;

  // ---- pairing
  int sB = -1;
  {
    const int role = a.pair_role[s];
    const int other = role >= 0 ? role : -2 - role;
    if (role != -1 && other != s && other >= 0 && other < batch) {
      const int back = a.pair_role[other];
      if (role >= 0 && back == -2 - s && joint_split(a, s, other, split)) sB = other;
      if (role <= -2 && back == s && joint_split(a, other, s, split)) return;  // done by `other`
    }
  }
  const bool paired = sB >= 0;

  int r0A = 0, r0B = 0;
  const bool report = (threadIdx.x == 0) && split == 0 && lgg == 0;
  const int nbA = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                             report, &r0A);
  const int b0 = split * SB;
  if (nbA < 0 || b0 >= nbA) return;   // never paired: joint_split checked both
  const int nbB = paired ? seq_blocks(a.seq_lens, a.meta_off, sB, a.max_nb, a.total_blocks,
                                      a.status, false, &r0B)
                         : 0;
  const int b1A = min(nbA, b0 + SB);
  const int b1B = paired ? min(nbB, b0 + SB) : b0;
  const int bend = max(b1A, b1B);
  const int nA = a.seq_lens[s];
  const int nB = paired ? a.seq_lens[sB] : 0;

  for (int i = threadIdx.x; i < b1A - b0; i += 64) tbl[i] = a.table[(size_t)s * a.max_nb + b0 + i];
  for (int i = threadIdx.x; i < b1B - b0; i += 64)
    tbl[SB + i] = a.table[(size_t)sB * a.max_nb + b0 + i];
  __syncthreads();

  // B operand of QK: columns 0..7 the group's queries of A, 8..15 those of B
  // (zero when unpaired).
  h8_t qb[4];
  if (!hi || paired) {
    const uint16_t* qp = a.q + ((((size_t)(hi ? sB : s) * a.num_layers + layer) * kQHeads +
                                 kGroup * g + (c & (kGroup - 1))) * kHeadDim);
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = *reinterpret_cast<const h8_t*>(qp + qk_elem<F>(i, j));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = h8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  // ---- the walk: steps over positions [b0, bend)
  auto shared_at = [&](int b) {
    return b < b1A && b < b1B && tbl[b - b0] == tbl[SB + b - b0];
  };
  int nsteps = 0;
  for (int i = lane; i < bend - b0; i += 64) {
    const int b = b0 + i;
    nsteps += shared_at(b) ? 1 : (int)(b < b1A) + (int)(b < b1B);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) nsteps += __shfl_xor(nsteps, m, 64);

  int cur_b = b0, cur_ph = 0;   // load cursor: position and, for an unshared position, A done
  auto next_step = [&]() -> PairStep {
    PairStep st;
    if (cur_b >= bend) {          // past the end: a cached block of the split, nothing live
      st.pid = tbl[b1A - 1 - b0];
      st.mask = 0;
      st.b = b0;
      return st;
    }
    const int b = cur_b;
    const bool hasA = b < b1A, hasB = b < b1B;
    st.b = b;
    if (shared_at(b)) {
      st.pid = tbl[b - b0];
      st.mask = 3;
      ++cur_b;
    } else if (cur_ph == 0 && hasA) {
      st.pid = tbl[b - b0];
      st.mask = 1;
      if (hasB) cur_ph = 1; else ++cur_b;
    } else {
      st.pid = tbl[SB + b - b0];
      st.mask = 2;
      cur_ph = 0;
      ++cur_b;
    }
    st.pid = __builtin_amdgcn_readfirstlane(st.pid);
    st.mask = __builtin_amdgcn_readfirstlane(st.mask);
    st.b = __builtin_amdgcn_readfirstlane(st.b);
    return st;
  };

  constexpr int64_t kLayerBytes = 16 * (int64_t)tile_bytes<F>();
  const size_t block_stride = (size_t)a.num_layers * kLayerBytes;
  const size_t tile_off = (size_t)layer * kLayerBytes + (size_t)g * tile_bytes<F>();
  auto step_base = [&](int pid, bool* ok) -> const uint8_t* {
    const bool in_pool = pid >= 0 && (int64_t)pid < a.pool_blocks;
    *ok = in_pool;
    return a.pool + (size_t)(in_pool ? pid : 0) * block_stride + tile_off;
  };

  float m_run = -INFINITY;
  float l_run = 0.f;
  f4_t acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int kRing = F::kRing;
  BlockRegs<F> ring[kRing];
  int ring_mask[kRing], ring_b[kRing];
  bool ring_ok[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k) {
    const PairStep st = next_step();
    ring_mask[k] = st.mask;
    ring_b[k] = st.b;
    load_block(ring[k], step_base(st.pid, &ring_ok[k]), lane, c, j);
  }

  bool saw_bad = false;
  for (int sbase = 0; sbase < nsteps; sbase += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int mask = sbase + k < nsteps ? ring_mask[k] : 0;
      const int b = ring_b[k];
      const bool ok = ring_ok[k];
      saw_bad |= mask != 0 && !ok;
      const int vA = (mask & 1) && ok ? min(16, nA - 16 * b) : 0;
      const int vB = (mask & 2) && ok ? min(16, nB - 16 * b) : 0;
      const int vown = hi ? vB : vA;
      const int vrows = max(vA, vB);

      // ---- value tile to LDS (the slot's value registers are free after this)
      stage_values<F>(ring[k], vstage, lane, 0);

      // ---- logits of 16 tokens x 16 columns
      f4_t sacc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand<F>(ring[k], i), qb[i], sacc,
                                                      0, 0, 0);

      // ---- refill this slot with the step kRing ahead
      {
        const PairStep st = next_step();
        ring_mask[k] = st.mask;
        ring_b[k] = st.b;
        load_block(ring[k], step_base(st.pid, &ring_ok[k]), lane, c, j);
      }

      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = sacc[i] * a.scale_log2;
      if (vown < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * j + i >= vown) sv[i] = -INFINITY;
      }

      // ---- online softmax (per column; the 4 lanes j share a column)
      float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      bm = head_max4(bm);
      const float m_new = fmaxf(m_run, bm);
      const bool live = m_new != -INFINITY;
      const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = live ? __builtin_amdgcn_exp2f(sv[i] - m_new) : 0.f;
      const float ps = (pv[0] + pv[1]) + (pv[2] + pv[3]);
      l_run = l_run * alpha + ps;
      const float bsum = head_sum4(ps);

      if (__ballot((!hi || paired) && alpha != 1.f) != 0ull) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] *= alpha;
        if (!hi || paired)
          for (int idx = j; idx < b - b0; idx += 4) pi_lds[c * SB + idx] *= alpha;
      }
      if (j == 0 && (hi ? (mask & 2) : (mask & 1))) pi_lds[c * SB + (b - b0)] = bsum;
      m_run = m_new;

      // ---- PV: transposed value rows from LDS
      u4_t R[4];
      value_rows<F>(vstage, 0, j, c, R);
      if (vrows < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * j + i >= vrows) R[i] = u4_t{0u, 0u, 0u, 0u};
      }
      const h4_t pb = h4_t{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo01 = __builtin_amdgcn_perm(R[1][q], R[0][q], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(R[3][q], R[2][q], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(R[1][q], R[0][q], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(R[3][q], R[2][q], 0x07060302u);
        acc[2 * q] = __builtin_amdgcn_mfma_f32_16x16x16f16(
            __builtin_bit_cast(h4_t, u2_t{lo01, lo23}), pb, acc[2 * q], 0, 0, 0);
        acc[2 * q + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(
            __builtin_bit_cast(h4_t, u2_t{hi01, hi23}), pb, acc[2 * q + 1], 0, 0, 0);
      }
    }
  }
  if (saw_bad && lane == 0) flag(a.status, KVS_DEV_BAD_BLOCK_ID);

  // ---- split epilogue: statistics and partial outputs of both sequences, mass partials
  const float lt = head_sum4(l_run);
  if (!hi || paired) {
    const int so = hi ? sB : s;
    const size_t st = (((size_t)so * a.n_layers + lr) * kQHeads + kGroup * g + (c & (kGroup - 1))) *
                          a.n_splits + split;
    if (j == 0) a.ml[st] = make_float2(m_run, lt);
    float* op = a.opart + st * kHeadDim + 32 * j;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f4_t*>(op + 8 * i) = f4_t{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *reinterpret_cast<f4_t*>(op + 8 * i + 4) = f4_t{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
  }
  __syncthreads();
  for (int hh = 0; hh < kGroup; ++hh) {
    float* dst = a.pi + ((size_t)lr * kQHeads + kGroup * g + hh) * a.total_blocks + r0A + b0;
    for (int bb = lane; bb < b1A - b0; bb += 64) dst[bb] = pi_lds[hh * SB + bb];
    if (paired) {
      float* dstB = a.pi + ((size_t)lr * kQHeads + kGroup * g + hh) * a.total_blocks + r0B + b0;
      for (int bb = lane; bb < b1B - b0; bb += 64) dstB[bb] = pi_lds[(kGroup + hh) * SB + bb];
    }
  }
}

hipError_t launch_decode_pair(const DecodeArgs& a, int batch, hipStream_t stream) {
  const uint64_t wgs = (uint64_t)batch * a.n_splits * a.n_layers * 8u;
  const size_t lds = decode_pair_lds_bytes(a.split_blocks);
  if (a.kv_format != KVS_KV_FP16 || lds > kMaxDecodeLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL(paged_decode_pair, dim3((uint32_t)wgs), dim3(64), lds, stream, a);
  return hipGetLastError();
}

}  // namespace kvs
