// KIVI 2-bit KV kernels: paged_decode_kivi (decode over 2-bit codes plus the
// fp16 residual window), kivi_quantize (fp16 pairs to quantised blocks) and
// the boundary advance after appends (kivi_advance_alloc / _commit).
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

namespace kvs {

// ---------------------------------------------------------------------------
// paged_decode_kivi
//
// The split-K decode above over a KIVI cache (Fitting a Million Tokens, Sec.
// 02: 2-bit codes plus fp16 scales, dequantised inside the attention kernel).
// Quantised blocks come in 32-token pairs (one key group).  A wave loads a
// pair's four 768-byte tiles of its (layer, KV head) with one coalesced
// 16-byte load per lane and tile into a register slot, stages them in LDS and
// works on the codes directly, never forming dequantised keys or values:
//  QK:  S^T[t][h] = sum_d c[t][d] (q[h][d] s[d]) + sum_d q[h][d] z[d].  The
//       pair's per-channel scales fold into the query as an fp16 pair
//       q s = hi + lo (v_pk_mul_f16, then v_pk_fma_f16 of the remainder:
//       exact up to fp16 underflow), and the key codes enter
//       v_mfma_f32_16x16x32_f16 as the fp16 integers 0..3, converted by
//       gfx950's packed FP4 (E2M1) conversion at scale 2.  The zero-point
//       term is one dot product per head and pair.
//  PV:  O[d][h] = sum_t c[t][d] (p[t][h] s[t][g(d)]) + sum_t p[t][h] z[t][g(d)].
//       Output tile k of v_mfma_f32_16x16x16_f16 covers channels
//       16 k .. 16 k + 15, inside value group k / 2, so each group's per-token
//       scales fold into the fp16 probability operand; the zero-point term is
//       accumulated per group and added at the end.  Lane (j, c) ends with
//       channels 16 k + 4 j + i of head c.
//       The two terms nearly cancel when values sit around zero (each is about
//       the group minimum times the weight sum, their difference the output),
//       so both must see the same weights: the folded operand p s enters as its
//       fp16 product plus the product's fp16 remainder (two MFMAs), not rounded
//       once.  Rounded once, weights that all round to the same fp16 value (a
//       nearly flat softmax) bias every product the same way: -1e-4 of the code
//       term, 1e-2 of an output 100 times smaller than the group minima.
//  fp16 residual blocks (from quant_lens[s] on) run one by one with the same
//  operand layouts (value tile transposed through LDS).
// ---------------------------------------------------------------------------
// 32-token pairs in flight per wave.  A pair is staged in LDS as soon as its
// loads land, so one slot already overlaps the next pair's loads with this
// pair's arithmetic; two slots measured 4 % slower (more registers, larger
// loop body) in this issue-bound kernel.
constexpr int kKiviRing = 1;
// Launch bound: 4 waves per SIMD (at most 128 VGPRs).
constexpr int kKiviWavesPerSimd = 4;

// The 8 codes of one set (code m at bits 4 m, 4 m + 1 of w, other bits 0) as
// fp16 0..3: E2M1 reads a nibble 0..3 as 0, 0.5, 1, 1.5; the scale 2 makes
// them the integers.
__device__ __forceinline__ h8_t codes_to_h8(uint32_t w) {
  const h2_t x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 0);
  const h2_t x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 1);
  const h2_t x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 2);
  const h2_t x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 2.0f, 3);
  return h8_t{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
}

// Set S of an 8-byte code entry, its codes moved to the low bits of nibbles.
__device__ __forceinline__ uint32_t code_set(u2_t entry, int S) {
  return (entry[S >> 1] >> (2 * (S & 1))) & 0x33333333u;
}

__device__ __forceinline__ float dot2(h2_t x, h2_t y, float acc) {
  return __builtin_amdgcn_fdot2(x, y, acc, false);
}

__global__ void __launch_bounds__(64, kKiviWavesPerSimd) paged_decode_kivi(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int SB = a.split_blocks;
  int32_t* tbl = reinterpret_cast<int32_t*>(smem);                          // [SB] block ids
  float* pi_lds = reinterpret_cast<float*>(smem + (size_t)4 * SB);          // [8][SB]
  uint8_t* stage = smem + (size_t)36 * SB;       // 4 KiB: a pair's four tiles or an fp16 value tile

  const int lane = threadIdx.x;
  const int c = lane & 15;
  const int j = lane >> 4;

  uint32_t w = xcd_item(blockIdx.x, gridDim.x);
  const uint32_t lgg_count = (uint32_t)a.n_layers * 8u;
  const int lgg = (int)(w % lgg_count);
  w /= lgg_count;
  const int split = (int)(w % (uint32_t)a.n_splits);
  const int s = (int)(w / (uint32_t)a.n_splits);
  const int lr = lgg >> 3;
  const int g = lgg & 7;
  const int layer = a.layer_begin + lr;

  int r0 = 0;
  const bool report = lane == 0 && split == 0 && lgg == 0;
  const int nb = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                            report, &r0);
  const int b0 = split * SB;
  if (nb < 0 || b0 >= nb) return;
  const int b1 = min(nb, b0 + SB);
  const int n = a.seq_lens[s];
  const int nq = a.quant_lens[s];
  const size_t st = (((size_t)s * a.n_layers + lr) * kQHeads + kGroup * g + c) * a.n_splits + split;
  if (nq < 0 || (nq & 31) != 0 || nq > n) {
    // unusable boundary: this split contributes nothing (empty statistics, zero
    // partial output and mass), so the sequence's output and mass are zero
    if (report) flag(a.status, KVS_DEV_BAD_SEQ_LEN);
    if (c < kGroup) {
      if (j == 0) a.ml[st] = make_float2(-INFINITY, 0.f);
      float* op = a.opart + st * kHeadDim + 32 * j;
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<f4_t*>(op + 4 * i) = f4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int hh = 0; hh < kGroup; ++hh) {
      float* dst = a.pi + ((size_t)lr * kQHeads + kGroup * g + hh) * a.total_blocks + r0 + b0;
      for (int bb = lane; bb < b1 - b0; bb += 64) dst[bb] = 0.f;
    }
    return;
  }

  for (int i = lane; i < b1 - b0; i += 64) tbl[i] = a.table[(size_t)s * a.max_nb + b0 + i];
  __syncthreads();

  // B operand of QK: queries of the group, channels 32 i + 8 j .. + 8.  Columns
  // 8..15 repeat heads 0..7.  In a quantised pair the first block's logits are
  // taken from columns 0..7 and the second block's from columns 8..15, so that
  // every lane holds a real (block, head) value through the softmax; a lane's
  // half of the wave (hi) says which block of the pair it carries.  Columns
  // 8..15 of the output accumulators collect the second blocks and are added
  // to columns 0..7 at the end of the split.
  const bool hi = c >= kGroup;
  h8_t qb[4];
  {
    const uint16_t* qp = a.q + ((((size_t)s * a.num_layers + layer) * kQHeads + kGroup * g +
                                 (c & (kGroup - 1))) * kHeadDim);
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = *reinterpret_cast<const h8_t*>(qp + 32 * i + 8 * j);
  }

  // Weights relative to a reference 2^kshift below the running maximum (see
  // kProbShift).  Here they also form the fp16 PV operand p s with the value
  // scales, so the shift is chosen per split from its first pair's largest
  // value scale s1: kshift = clamp(7 - floor(log2 s1), 0, 15) keeps
  // 2^kshift s1 below 2^8.  A product p s 2^kshift then overflows fp16 only
  // for a scale above about 128 s1 in the same split, and that split is run
  // again with kshift = 0 (weights <= 1, scales < 2^16: no overflow).  Products
  // below 2^-25 of the reference round to zero, so the code term of a split
  // loses at most 3 x tokens x 2^-(25 + kshift) against a largest weight of
  // 2^kshift: under 2^-32 s1 per token.
  float kshift = kProbShift;
  float m_run = -INFINITY;
  f4_t acc[8];
  float zacc[4];
  bool saw_bad = false;

  // Online softmax of one block's 16 x 16 logits (base 2); returns p relative
  // to the running maximum and keeps the block's probability mass in LDS.
  auto softmax_block = [&](const float (&sv)[4], int b, float (&pv)[4]) {
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = head_max4(bm);
    bm = fmaxf(bm, swap8(bm));   // both halves keep the same running maximum
    const float m_new = fmaxf(m_run, bm - kshift);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = live ? __builtin_amdgcn_exp2f(sv[i] - m_new) : 0.f;
    const float bs = head_sum4((pv[0] + pv[1]) + (pv[2] + pv[3]));
    if (__ballot(c < kGroup && alpha != 1.f) != 0ull) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) zacc[k] *= alpha;
      if (c < kGroup)
        for (int idx = j; idx < b - b0; idx += 4) pi_lds[c * SB + idx] *= alpha;
    }
    if (c < kGroup && j == 0) pi_lds[c * SB + (b - b0)] = bs;
    m_run = m_new;
  };

  // One update for the two blocks of a quantised pair (32 tokens, all logits
  // finite): lanes of the lower half hold the first block, lanes of the upper
  // half the second, for the same heads.  Returns p relative to the running
  // maximum and keeps both blocks' probability mass in LDS.
  auto softmax_pair = [&](const float (&sv)[4], int be, float (&pv)[4]) {
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = head_max4(bm);
    bm = fmaxf(bm, swap8(bm));
    const float m_new = fmaxf(m_run, bm - kshift);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_new);
    const float bs = head_sum4((pv[0] + pv[1]) + (pv[2] + pv[3]));
    if (__ballot(alpha != 1.f) != 0ull) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] *= alpha;
#pragma unroll
      for (int k = 0; k < 4; ++k) zacc[k] *= alpha;
      if (!hi)
        for (int idx = j; idx < be - b0; idx += 4) pi_lds[c * SB + idx] *= alpha;
    }
    if (j == 0) pi_lds[(c & (kGroup - 1)) * SB + (be + (hi ? 1 : 0) - b0)] = bs;
    m_run = m_new;
  };

  // ---- quantised blocks [b0, bq1), in pairs (b0 and nq / 16 are even)
  const int bq1 = min(b1, nq >> 4);
  // One pass over the split.  Called once, and a second time (inlined again,
  // not a loop, so the first pass keeps its own register allocation) only
  // when the first pass overflowed.
  auto run_split = [&](bool first) __attribute__((always_inline)) {
  m_run = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) zacc[k] = 0.f;
  if (bq1 > b0) {
    const size_t kblock = (size_t)a.num_layers * 16 * kKiviTileBytes;
    const size_t ktile = ((size_t)(layer * 2) * 8 + g) * kKiviTileBytes;
    const size_t vtile = ((size_t)(layer * 2 + 1) * 8 + g) * kKiviTileBytes;
    // A lane loads 16 bytes of each of the pair's four 768-byte tiles [K even |
    // K odd | V even | V odd] and writes them to the same place in the stage.
    // Lanes 48..63 repeat lanes 0..15: the same bytes in the same load
    // instruction (no extra memory traffic) and the same values to the same LDS
    // bytes.  Each load so has one wave-uniform base, held in scalar registers,
    // and the pair's address arithmetic stays off the VALU.
    const uint32_t voff = 16u * (uint32_t)(lane < 48 ? lane : lane - 48);
    // Loads of the pair starting at block be; pairs past the split's quantised
    // range reuse its last pair (in-bounds, unused), ids outside the pool read
    // block 0 and are masked.
    auto load_pair = [&](u4_t (&r)[4], int be, bool* ok) {
      const int cl = min(be, bq1 - 2);
      // block ids are wave-uniform: scalar registers keep the address math off the VALU
      const int pe = __builtin_amdgcn_readfirstlane(tbl[cl - b0]);
      const int po = __builtin_amdgcn_readfirstlane(tbl[cl + 1 - b0]);
      const bool in = pe >= 0 && (int64_t)pe < a.kivi_blocks && po >= 0 &&
                      (int64_t)po < a.kivi_blocks;
      *ok = in && be < bq1;
      const uint8_t* pe_p = a.kivi + (size_t)(in ? pe : 0) * kblock;
      const uint8_t* po_p = a.kivi + (size_t)(in ? po : 0) * kblock;
      r[0] = stream_load(reinterpret_cast<const u4_t*>(pe_p + ktile + voff));
      r[1] = stream_load(reinterpret_cast<const u4_t*>(po_p + ktile + voff));
      r[2] = stream_load(reinterpret_cast<const u4_t*>(pe_p + vtile + voff));
      r[3] = stream_load(reinterpret_cast<const u4_t*>(po_p + vtile + voff));
    };

    u4_t ring[kKiviRing][4];
    bool ring_ok[kKiviRing];
#pragma unroll
    for (int k = 0; k < kKiviRing; ++k) load_pair(ring[k], b0 + 2 * k, &ring_ok[k]);
    if (first) {
      // largest value scale of the split's first pair: bytes 512..639 of its two
      // value tiles, held by lanes 32..39 (scales are >= 0, so their fp16 bit
      // patterns order like their values)
      uint32_t sbits = 0u;
      if (lane >= 32 && lane < 40)
#pragma unroll
        for (int t = 2; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sbits = max(sbits, max(ring[0][t][i] & 0x7FFFu, (ring[0][t][i] >> 16) & 0x7FFFu));
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) sbits = max(sbits, (uint32_t)__shfl_xor((int)sbits, m, 64));
      const int e5 = (int)(__builtin_amdgcn_readfirstlane(sbits) >> 10);   // fp16 exponent field
      kshift = (float)min(15, max(0, 22 - e5));
    }

    for (int pb = b0; pb < bq1; pb += 2 * kKiviRing) {
#pragma unroll
      for (int k = 0; k < kKiviRing; ++k) {
        const int be = pb + 2 * k;
        const bool active = be < bq1;
        const bool ok = ring_ok[k];
        saw_bad |= active && !ok;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          *reinterpret_cast<u4_t*>(stage + kKiviTileBytes * t + voff) = ring[k][t];
        load_pair(ring[k], be + 2 * kKiviRing, &ring_ok[k]);
        if (!active) continue;
        if (!ok) {
          // a pair with an id outside the pool contributes nothing
          if (c < kGroup && j == 0) {
            pi_lds[c * SB + (be - b0)] = 0.f;
            pi_lds[c * SB + (be + 1 - b0)] = 0.f;
          }
          continue;
        }

        // key scales of the lane's channels folded into q (exact hi + lo), and the
        // zero-point term sum_d z[d] q[h][d] from MFMAs whose A rows all hold z:
        // it lands in every token row, so it starts both blocks' accumulators.
        f4_t zsacc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint8_t* km = stage + (i >> 1) * kKiviTileBytes + 640 + 2 * (32 * (i & 1) + 8 * j);
          zsacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(*reinterpret_cast<const h8_t*>(km), qb[i],
                                                         zsacc, 0, 0, 0);
        }

        // ---- logits of both blocks (two independent MFMA chains), one softmax update.
        // The scaled query of channel slice i is formed just before its MFMAs, so
        // only one slice's hi / lo operands are live at a time.
        f4_t sacc[2] = {zsacc, zsacc};
        u2_t kent[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
          kent[hb] = *reinterpret_cast<const u2_t*>(stage + hb * kKiviTileBytes + 8 * lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint8_t* km = stage + (i >> 1) * kKiviTileBytes + 512 + 2 * (32 * (i & 1) + 8 * j);
          const h8_t s8 = *reinterpret_cast<const h8_t*>(km);
          const h8_t qhi = qb[i] * s8;
          const h8_t qlo = __builtin_elementwise_fma(qb[i], s8, -qhi);
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const h8_t kc = codes_to_h8(code_set(kent[hb], i));
            sacc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc, qhi, sacc[hb], 0, 0, 0);
            sacc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc, qlo, sacc[hb], 0, 0, 0);
          }
        }
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = (hi ? sacc[1][i] : sacc[0][i]) * a.scale_log2;
        float pv[4];
        softmax_pair(sv, be, pv);

        // ---- PV.  Each lane's probabilities belong to its own block, so the value
        // zero-point term (each lane against its block's zero points) is one pass;
        // the products with the codes run per block, with the other half's
        // probabilities zeroed.
        const h4_t pb4 = h4_t{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
        {
          const uint8_t* vz = stage + (hi ? 3 : 2) * kKiviTileBytes + 640;
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const h4_t z4 = *reinterpret_cast<const h4_t*>(vz + 2 * (16 * grp + 4 * j));
            zacc[grp] = dot2(h2_t{pb4[2], pb4[3]}, h2_t{z4[2], z4[3]},
                             dot2(h2_t{pb4[0], pb4[1]}, h2_t{z4[0], z4[1]}, zacc[grp]));
          }
        }
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const h4_t pbm = (hi == (hb == 1)) ? pb4 : h4_t{0, 0, 0, 0};
          const uint8_t* vt = stage + (2 + hb) * kKiviTileBytes;
          const u2_t vent = *reinterpret_cast<const u2_t*>(vt + 8 * lane);
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const h4_t s4 = *reinterpret_cast<const h4_t*>(vt + 512 + 2 * (16 * grp + 4 * j));
            // p s as bp + br: the fp16 product and its remainder (exact in fp16
            // unless it falls below 2^-24), so that the code term weighs each
            // token by the same fp16 weight as the zero-point term
            const h4_t bp = pbm * s4;
            const h4_t br = __builtin_elementwise_fma(pbm, s4, -bp);
            const h8_t vc = codes_to_h8(code_set(vent, grp));
            const h4_t va = h4_t{vc[0], vc[1], vc[2], vc[3]};
            const h4_t vb = h4_t{vc[4], vc[5], vc[6], vc[7]};
            acc[2 * grp] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, bp, acc[2 * grp], 0, 0, 0);
            acc[2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(vb, bp, acc[2 * grp + 1], 0, 0, 0);
            acc[2 * grp] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, br, acc[2 * grp], 0, 0, 0);
            acc[2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(vb, br, acc[2 * grp + 1], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- fp16 residual blocks [max(b0, nq / 16), b1)
  {
    const size_t fblock = (size_t)a.num_layers * 16 * kTileBytes;
    const size_t ftile = ((size_t)(layer * 2) * 8 + g) * kTileBytes;
    const _Float16* vt = reinterpret_cast<const _Float16*>(stage);
    for (int b = max(b0, nq >> 4); b < b1; ++b) {
      const int pid = tbl[b - b0];
      const bool in = pid >= 0 && (int64_t)pid < a.pool_blocks;
      saw_bad |= !in;
      const uint8_t* base = a.pool + (size_t)(in ? pid : 0) * fblock + ftile;
      u4_t kr[4], vr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        kr[i] = plain_load(reinterpret_cast<const u4_t*>(base + c * 256 + j * 16 + i * 64));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[i] = stream_load(reinterpret_cast<const u4_t*>(base + 8 * kTileBytes + lane * 16 + i * 1024));
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<u4_t*>(stage + i * 1024 + lane * 16) = vr[i];
      const int valid = in ? min(16, n - 16 * b) : 0;
      f4_t sacc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, kr[i]), qb[i], sacc,
                                                      0, 0, 0);
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sv[i] = (!hi && 4 * j + i < valid) ? sacc[i] * a.scale_log2 : -INFINITY;
      float pv[4];
      softmax_block(sv, b, pv);
      const h4_t pb4 = h4_t{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        h4_t av;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          av[i] = 4 * j + i < valid ? vt[(4 * j + i) * kHeadDim + 16 * k + c] : (_Float16)0;
        acc[k] = __builtin_amdgcn_mfma_f32_16x16x16f16(av, pb4, acc[k], 0, 0, 0);
      }
    }
  }
  };
  run_split(true);
  if (kshift != 0.f) {
    bool finite = true;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) finite = finite && __builtin_isfinite(acc[k][i]);
    if (__ballot(!finite) != 0ull) {
      kshift = 0.f;   // an fp16 product overflowed: run the split again unshifted
      run_split(false);
    }
  }
  if (saw_bad && lane == 0) flag(a.status, KVS_DEV_BAD_BLOCK_ID);

  // ---- split epilogue: statistics, partial output (+ value zero-point terms), mass partials
  // The upper half's columns (second blocks of the pairs) join the lower half's.
  float zt[4];
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    zt[grp] = head_sum4(zacc[grp]);
    zt[grp] += swap8(zt[grp]);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[k][i] += swap8(acc[k][i]);
  if (c < kGroup) {
    float* op = a.opart + st * kHeadDim + 4 * j;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float zk = zt[k >> 1];
      *reinterpret_cast<f4_t*>(op + 16 * k) =
          f4_t{acc[k][0] + zk, acc[k][1] + zk, acc[k][2] + zk, acc[k][3] + zk};
    }
  }
  __syncthreads();
  const int cnt = b1 - b0;
  const float lt = split_norm<kGroup>(pi_lds, SB, lane, cnt, 0);
  if (c < kGroup && j == 0) a.ml[st] = make_float2(m_run, lt);
  for (int hh = 0; hh < kGroup; ++hh) {
    float* dst = a.pi + ((size_t)lr * kQHeads + kGroup * g + hh) * a.total_blocks + r0 + b0;
    for (int bb = lane; bb < cnt; bb += 64) dst[bb] = pi_lds[hh * SB + bb];
  }
}

// ---------------------------------------------------------------------------
// kivi_quantize: one work-group of 256 threads per (pair, layer, KV head).
// Threads 0..127 each take one key channel over the pair's 32 tokens, threads
// 128..255 one (token, 32-channel group) of the values (Fitting a Million
// Tokens, Sec. 02: keys per channel, values per token, groups of 32).  Codes
// go through LDS, then every thread packs one 32-bit word of a key tile and
// one of a value tile in the library's block format.
// ---------------------------------------------------------------------------
constexpr int kQuantThreads = 256;

// Asymmetric 2-bit code of x for a group with minimum lo and fp16 scale s
// (as fp32): clamp(rint((x - lo) / s), 0, 3), 0 when s == 0.  fp32, IEEE
// division and round-to-nearest-even, as the format defines.
__device__ __forceinline__ uint32_t kivi_code(float x, float lo, float s) {
  if (s == 0.f) return 0u;
  const float t = rintf((x - lo) / s);
  return (uint32_t)fminf(fmaxf(t, 0.f), 3.f);
}

__global__ void __launch_bounds__(kQuantThreads) kivi_quantize(KiviQuantArgs a) {
  __shared__ uint8_t kc[32][kHeadDim];   // key codes [token][channel]
  __shared__ uint8_t vc[32][kHeadDim];   // value codes [token][channel]
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const int g = blockIdx.z;
  const int tid = threadIdx.x;
  if (a.count && pair >= *a.count) return;
  const int32_t* pr = a.pairs + (size_t)pair * 4;
  const int src[2] = {pr[0], pr[1]};
  const int dst[2] = {pr[2], pr[3]};
  if (src[0] < 0 || src[0] >= a.pool_blocks || src[1] < 0 || src[1] >= a.pool_blocks ||
      dst[0] < 0 || dst[0] >= a.kivi_blocks || dst[1] < 0 || dst[1] >= a.kivi_blocks) {
    if (tid == 0 && layer == 0 && g == 0) flag(a.status, KVS_DEV_BAD_BLOCK_ID);
    return;
  }
  const size_t fp16_block = (size_t)a.num_layers * 16 * kTileBytes;
  const size_t kivi_block = (size_t)a.num_layers * 16 * kKiviTileBytes;
  // (layer, K|V, head) tiles of the two source and two destination blocks
  auto src_tile = [&](int h, int kv) {
    return reinterpret_cast<const _Float16*>(a.pool + (size_t)src[h] * fp16_block +
                                             ((size_t)(layer * 2 + kv) * 8 + g) * kTileBytes);
  };
  auto dst_tile = [&](int h, int kv) {
    return a.kivi + (size_t)dst[h] * kivi_block +
           ((size_t)(layer * 2 + kv) * 8 + g) * kKiviTileBytes;
  };

  if (tid < kHeadDim) {
    // one key channel over tokens 0..31 of the pair
    const int ch = tid;
    float x[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) x[t] = (float)src_tile(t >> 4, 0)[(t & 15) * kHeadDim + ch];
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int t = 1; t < 32; ++t) { lo = fminf(lo, x[t]); hi = fmaxf(hi, x[t]); }
    const _Float16 s16 = (_Float16)((hi - lo) / 3.0f);
    const float sc = (float)s16;
#pragma unroll
    for (int t = 0; t < 32; ++t) kc[t][ch] = (uint8_t)kivi_code(x[t], lo, sc);
    uint8_t* meta = dst_tile(ch >> 6, 0) + 512;
    reinterpret_cast<_Float16*>(meta)[ch & 63] = s16;
    reinterpret_cast<_Float16*>(meta + 128)[ch & 63] = (_Float16)lo;
  } else {
    // one token, one 32-channel group of the values
    const int u = tid - kHeadDim;
    const int t = u >> 2, grp = u & 3;
    const _Float16* row = src_tile(t >> 4, 1) + (t & 15) * kHeadDim + 32 * grp;
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = (float)row[i];
    float lo = x[0], hi = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) { lo = fminf(lo, x[i]); hi = fmaxf(hi, x[i]); }
    const _Float16 s16 = (_Float16)((hi - lo) / 3.0f);
    const float sc = (float)s16;
#pragma unroll
    for (int i = 0; i < 32; ++i) vc[t][32 * grp + i] = (uint8_t)kivi_code(x[i], lo, sc);
    uint8_t* meta = dst_tile(t >> 4, 1) + 512;
    reinterpret_cast<_Float16*>(meta)[16 * grp + (t & 15)] = s16;
    reinterpret_cast<_Float16*>(meta + 128)[16 * grp + (t & 15)] = (_Float16)lo;
  }
  __syncthreads();

  // Packing: thread -> (block h of the pair, word w of its tile's 128 code words);
  // word w is half ww of entry e = (j, c), holding sets 2 ww and 2 ww + 1.
  const int h = tid >> 7;
  const int w = tid & 127;
  const int e = w >> 1, ww = w & 1;
  const int j = e >> 4, c = e & 15;
  uint32_t kword = 0u, vword = 0u;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int S = 2 * ww + sb;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int shift = 4 * m + 2 * sb;
      kword |= (uint32_t)kc[16 * h + c][32 * S + 8 * j + m] << shift;
      const int k = 2 * S + (m >> 2);
      vword |= (uint32_t)vc[16 * h + 4 * j + (m & 3)][16 * k + c] << shift;
    }
  }
  reinterpret_cast<uint32_t*>(dst_tile(h, 0))[w] = kword;
  reinterpret_cast<uint32_t*>(dst_tile(h, 1))[w] = vword;
}

// ---------------------------------------------------------------------------
// KIVI boundary advance.  kivi_advance_alloc (one work-group) walks the batch in
// order; a sequence whose fp16 residual has reached residual + 32 tokens gets
// its next 32-token pair quantised: two quantised blocks from the top of the
// KIVI free stack (an exclusive prefix count over the sequences that advance)
// and a job {fp16 even, fp16 odd, KIVI even, KIVI odd}.  kivi_quantize then
// runs over the jobs, and kivi_advance_commit points the table entries at the
// quantised blocks, grows quant_lens by 32 and pushes the two fp16 blocks onto
// the fp16 free stack, in job order.
// ---------------------------------------------------------------------------
constexpr int kAdvanceThreads = 1024;

__global__ void __launch_bounds__(kAdvanceThreads) kivi_advance_alloc(KiviAdvanceArgs a,
                                                                      int batch) {
  __shared__ int scan[kAdvanceThreads];
  const int tid = threadIdx.x;
  int top0 = *a.kivi_free_top;
  if (top0 < 0 || top0 > a.kivi_free_capacity) {
    if (tid == 0) flag(a.status, KVS_DEV_BAD_OFFSETS);
    top0 = top0 < 0 ? 0 : a.kivi_free_capacity;
  }
  int carry = 0;
  for (int base = 0; base < batch; base += kAdvanceThreads) {
    const int s = base + tid;
    int need = 0, src_e = -1, src_o = -1;
    if (s < batch) {
      const int n = a.seq_lens[s];
      const int nq = a.quant_lens[s];
      const bool valid = n >= 0 && nq >= 0 && (nq & 31) == 0 && nq <= n && n <= 16 * a.max_nb;
      if (!valid) {
        flag(a.status, KVS_DEV_BAD_SEQ_LEN);
      } else if (kivi_quant_len(n, a.residual) > nq) {   // the next pair has left the window
        const int b = nq >> 4;
        src_e = a.table[(size_t)s * a.max_nb + b];
        src_o = a.table[(size_t)s * a.max_nb + b + 1];
        if (src_e >= 0 && src_e < a.pool_blocks && src_o >= 0 && src_o < a.pool_blocks) need = 1;
        else flag(a.status, KVS_DEV_BAD_BLOCK_ID);
      }
    }
    scan[tid] = need;
    __syncthreads();
    for (int off = 1; off < kAdvanceThreads; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int job = carry + scan[tid] - need;          // this sequence's job index
    if (need) {
      if (2 * job + 2 <= top0) {
        const int de = a.kivi_free[top0 - 1 - 2 * job];
        const int dO = a.kivi_free[top0 - 2 - 2 * job];
        const bool good = de >= 0 && de < a.kivi_blocks && dO >= 0 && dO < a.kivi_blocks;
        int32_t* j4 = a.jobs + (size_t)job * 4;
        // a job with a bad stack entry stays in place with ids -1: the
        // quantiser skips it (raising the status bit) and commit ignores it
        j4[0] = good ? src_e : -1;
        j4[1] = good ? src_o : -1;
        j4[2] = good ? de : -1;
        j4[3] = good ? dO : -1;
        a.job_seq[job] = good ? s : -1;
        if (!good) flag(a.status, KVS_DEV_BAD_BLOCK_ID);
      } else {
        flag(a.status, KVS_DEV_POOL_EXHAUSTED);   // later sequences: no job written
      }
    }
    carry += scan[kAdvanceThreads - 1];
    __syncthreads();
  }
  // Jobs are granted in batch order, so the ones that found KIVI blocks are
  // exactly jobs [0, granted); each consumed two stack entries.
  if (tid == 0) {
    const int granted = min(carry, top0 / 2);
    *a.count = granted;
    *a.kivi_free_top = top0 - 2 * granted;
  }
}

__global__ void __launch_bounds__(256) kivi_advance_commit(KiviAdvanceArgs a) {
  const int count = *a.count;
  int ftop = *a.fp16_free_top;
  const int tid = threadIdx.x;
  if (ftop < 0 || ftop > a.fp16_free_capacity) {   // a top outside the stack: clamped
    if (tid == 0) flag(a.status, KVS_DEV_BAD_OFFSETS);
    ftop = ftop < 0 ? 0 : a.fp16_free_capacity;
  }
  // exclusive count of committed jobs before each job, in job order
  __shared__ int done[256];
  int pushed = 0;
  for (int base = 0; base < count; base += 256) {
    const int job = base + tid;
    const int s = job < count ? a.job_seq[job] : -1;
    const int ok = s >= 0 ? 1 : 0;
    done[tid] = ok;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? done[tid - off] : 0;
      __syncthreads();
      done[tid] += v;
      __syncthreads();
    }
    const int before = pushed + done[tid] - ok;
    if (ok) {
      const int32_t* j4 = a.jobs + (size_t)job * 4;
      const int b = a.quant_lens[s] >> 4;
      a.table[(size_t)s * a.max_nb + b] = j4[2];
      a.table[(size_t)s * a.max_nb + b + 1] = j4[3];
      a.quant_lens[s] += 32;
      const int slot = ftop + 2 * before;
      if (slot + 2 <= a.fp16_free_capacity) {
        a.fp16_free[slot] = j4[0];
        a.fp16_free[slot + 1] = j4[1];
      } else {
        flag(a.status, KVS_DEV_POOL_EXHAUSTED);
      }
    }
    pushed += done[255];
    __syncthreads();
  }
  if (tid == 0) *a.fp16_free_top = min(ftop + 2 * pushed, a.fp16_free_capacity);
}

hipError_t launch_kivi_quantize(const KiviQuantArgs& a, hipStream_t stream) {
  if (a.num_layers > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kivi_quantize, dim3((uint32_t)a.n_pairs, (uint32_t)a.num_layers, 8),
                     dim3(kQuantThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kivi_advance(const KiviAdvanceArgs& adv, const KiviQuantArgs& q, int batch,
                               hipStream_t stream) {
  if (q.num_layers > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kivi_advance_alloc, dim3(1), dim3(kAdvanceThreads), 0, stream, adv, batch);
  hipLaunchKernelGGL(kivi_quantize, dim3((uint32_t)batch, (uint32_t)q.num_layers, 8),
                     dim3(kQuantThreads), 0, stream, q);
  hipLaunchKernelGGL(kivi_advance_commit, dim3(1), dim3(256), 0, stream, adv);
  return hipGetLastError();
}

hipError_t launch_decode_kivi(const DecodeArgs& a, int batch, hipStream_t stream) {
  const uint64_t wgs = (uint64_t)batch * a.n_splits * a.n_layers * 8u;
  const size_t lds = decode_lds_bytes(a.split_blocks);
  if (lds > kMaxDecodeLds) return hipErrorInvalidValue;
  hipLaunchKernelGGL(paged_decode_kivi, dim3((uint32_t)wgs), dim3(64), lds, stream, a);
  return hipGetLastError();
}

}  // namespace kvs
