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

// One step of the pair's walk: the kPer blocks to load, which column groups
// are live (bit 0: A, bit 1: B) and the first logical position.
template <int kPer>
struct PairStep {
  int pid[kPer];
  int mask;
  int b;
};

}  // namespace

// The LDS of a paired split keeps at most 2 work-groups per SIMD; the launch
// bound gives the kernel their VGPR budget (fp16: 178, no spills).
template <class F>
__global__ void __launch_bounds__(64, 2) paged_decode_pair(DecodeArgs a) {
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

  // ---- the walk: steps over groups of kPer positions from b0, the grouping of
  // paged_decode_gqa.  A group is joint when no position of it holds
  // different blocks in A and B (a position only one of them reaches is
  // loaded for that one); a joint group is one step with both column groups
  // live, any other group one step for A's blocks and one for B's.
  constexpr int kPer = F::kPer;
  const int cachedA = tbl[b1A - 1 - b0];                    // an in-split block of A
  const int cachedB = paired ? tbl[SB + b1B - 1 - b0] : cachedA;
  auto joint_group = [&](int b) {
    bool joint = true;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int q = b + p;
      joint &= !(q < b1A && q < b1B && tbl[q - b0] != tbl[SB + q - b0]);
    }
    return joint;
  };
  const int ngroups = (bend - b0 + kPer - 1) / kPer;
  int nsteps = 0;
  for (int i = lane; i < ngroups; i += 64) nsteps += joint_group(b0 + kPer * i) ? 1 : 2;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) nsteps += __shfl_xor(nsteps, m, 64);

  int cur_b = b0, cur_ph = 0;   // load cursor: first position of the group; A done
  auto next_step = [&]() -> PairStep<kPer> {
    PairStep<kPer> st;
    const int b = cur_b;
    st.b = b0;
    st.mask = 0;
    if (b >= bend) {              // past the end: cached blocks of the split, nothing live
#pragma unroll
      for (int p = 0; p < kPer; ++p) st.pid[p] = cachedA;
    } else if (joint_group(b)) {
      st.b = b;
      st.mask = 3;
#pragma unroll
      for (int p = 0; p < kPer; ++p) {
        const int q = b + p;
        st.pid[p] = q < b1A ? tbl[q - b0] : q < b1B ? tbl[SB + q - b0] : cachedA;
      }
      cur_b += kPer;
    } else if (cur_ph == 0) {     // both reach the group: A's blocks, then B's
      st.b = b;
      st.mask = 1;
#pragma unroll
      for (int p = 0; p < kPer; ++p) st.pid[p] = b + p < b1A ? tbl[b + p - b0] : cachedA;
      cur_ph = 1;
    } else {
      st.b = b;
      st.mask = 2;
#pragma unroll
      for (int p = 0; p < kPer; ++p) st.pid[p] = b + p < b1B ? tbl[SB + b + p - b0] : cachedB;
      cur_ph = 0;
      cur_b += kPer;
    }
#pragma unroll
    for (int p = 0; p < kPer; ++p) st.pid[p] = __builtin_amdgcn_readfirstlane(st.pid[p]);
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
  f4_t acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int kRing = F::kRing;
  StepRegs<F> ring[kRing];
  int ring_mask[kRing], ring_b[kRing];
  bool ring_ok[kRing][kPer];
  auto load_next = [&](int k) {
    const PairStep<kPer> st = next_step();
    ring_mask[k] = st.mask;
    ring_b[k] = st.b;
#pragma unroll
    for (int p = 0; p < kPer; ++p)
      load_block(ring[k].blk[p], step_base(st.pid[p], &ring_ok[k][p]), lane, c, j);
  };
#pragma unroll
  for (int k = 0; k < kRing; ++k) load_next(k);

  bool saw_bad = false;
  for (int sbase = 0; sbase < nsteps; sbase += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int mask = sbase + k < nsteps ? ring_mask[k] : 0;
      const int b = ring_b[k];
      int vown[kPer], vrows[kPer];
      bool own_active[kPer];
#pragma unroll
      for (int p = 0; p < kPer; ++p) {
        const int q = b + p;
        const bool ok = ring_ok[k][p];
        const bool liveA = (mask & 1) && q < b1A;
        const bool liveB = (mask & 2) && q < b1B;
        saw_bad |= (liveA || liveB) && !ok;
        const int vA = liveA && ok ? min(16, nA - 16 * q) : 0;
        const int vB = liveB && ok ? min(16, nB - 16 * q) : 0;
        vown[p] = hi ? vB : vA;
        vrows[p] = max(vA, vB);
        own_active[p] = hi ? liveB : liveA;
      }

      // ---- value tiles to LDS (the slot's value registers are free after this)
#pragma unroll
      for (int p = 0; p < kPer; ++p) stage_values<F>(ring[k].blk[p], vstage, lane, p);

      // ---- logits of 16 tokens x 16 columns per block
      f4_t sacc[kPer];
#pragma unroll
      for (int p = 0; p < kPer; ++p) sacc[p] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int p = 0; p < kPer; ++p)
          sacc[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand<F>(ring[k].blk[p], i),
                                                           qb[i], sacc[p], 0, 0, 0);

      // ---- refill this slot with the step kRing ahead
      load_next(k);

      float sv[kPer][4];
#pragma unroll
      for (int p = 0; p < kPer; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[p][i] = sacc[p][i] * a.scale_log2;
        if (vown[p] < 16) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * j + i >= vown[p]) sv[p][i] = -INFINITY;
        }
      }

      // ---- online softmax over the step (per column; the 4 lanes j share a column)
      float bm = -INFINITY;
#pragma unroll
      for (int p = 0; p < kPer; ++p)
        bm = fmaxf(bm, fmaxf(fmaxf(sv[p][0], sv[p][1]), fmaxf(sv[p][2], sv[p][3])));
      bm = head_max4(bm);
      const float m_new = fmaxf(m_run, bm - kProbShift);   // reference below the maximum
      const bool live = m_new != -INFINITY;
      const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      float pv[kPer][4];
      float bsum[kPer];
#pragma unroll
      for (int p = 0; p < kPer; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[p][i] = live ? __builtin_amdgcn_exp2f(sv[p][i] - m_new) : 0.f;
        bsum[p] = head_sum4((pv[p][0] + pv[p][1]) + (pv[p][2] + pv[p][3]));
      }

      if (__ballot((!hi || paired) && alpha != 1.f) != 0ull) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] *= alpha;
        if (!hi || paired)
          for (int idx = j; idx < b - b0; idx += 4) pi_lds[c * SB + idx] *= alpha;
      }
#pragma unroll
      for (int p = 0; p < kPer; ++p)
        if (own_active[p] && j == 0) pi_lds[c * SB + (b + p - b0)] = bsum[p];
      m_run = m_new;

      // ---- PV: transposed value rows from LDS
#pragma unroll
      for (int p = 0; p < kPer; ++p) {
        u4_t R[4];
        value_rows<F>(vstage, p, j, c, R);
        if (vrows[p] < 16) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * j + i >= vrows[p]) R[i] = u4_t{0u, 0u, 0u, 0u};
        }
        const h4_t pb = h4_t{(_Float16)pv[p][0], (_Float16)pv[p][1], (_Float16)pv[p][2],
                             (_Float16)pv[p][3]};
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
  }
  if (saw_bad && lane == 0) flag(a.status, KVS_DEV_BAD_BLOCK_ID);

  // ---- split epilogue: statistics and partial outputs of both sequences, mass partials
  const size_t st = (((size_t)(hi ? sB : s) * a.n_layers + lr) * kQHeads + kGroup * g +
                     (c & (kGroup - 1))) * a.n_splits + split;
  if (!hi || paired) {
    float* op = a.opart + st * kHeadDim + 32 * j;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f4_t*>(op + 8 * i) = f4_t{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *reinterpret_cast<f4_t*>(op + 8 * i + 4) = f4_t{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
  }
  __syncthreads();
  // rows 0..7: the first sequence's heads, rows 8..15: the second's
  const float lt = split_norm<2 * kGroup>(pi_lds, SB, lane, b1A - b0, paired ? b1B - b0 : 0);
  if ((!hi || paired) && j == 0) a.ml[st] = make_float2(m_run, lt);
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
  if (lds > kMaxDecodeLds) return hipErrorInvalidValue;
  if (a.kv_format == KVS_KV_FP16)
    hipLaunchKernelGGL(paged_decode_pair<KvF16>, dim3((uint32_t)wgs), dim3(64), lds, stream, a);
  else if (a.kv_format == KVS_KV_E4M3)
    hipLaunchKernelGGL(paged_decode_pair<KvE4M3Pair>, dim3((uint32_t)wgs), dim3(64), lds, stream,
                       a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvs
