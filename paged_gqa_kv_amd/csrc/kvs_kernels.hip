// Device kernels of the paged GQA decode + block-scoring library (gfx950 only).
//
// Kernels, in the order one decode step runs them:
//   paged_decode_gqa  split-K decode: one wave per (sequence, layer, KV head,
//                     split of blocks); QK^T and PV on MFMA; online softmax;
//                     per-(layer, head, block) probability-mass partials.
//   combine_splits    merges the splits of each (sequence, layer, head) into the
//                     fp16 output and the per-split normalising weights.
//   block_mass        sums the mass partials of every (layer, query head) into
//                     one fp32 number per (sequence, block), in a fixed order.
//   seq_chunk_max /   the scoring step: per-sequence maximum, then normalise,
//   score_update      EMA, touch, priority and tier per 64-byte record (fp64).
//   classify_records, meta_init, clear_status: the remaining entry points.
//
// Sources: "KV-Cache Offloading for LLM Inference -- Visual Reference"
// Sec. 2 (attention), Sec. 11 (EMA), Sec. 12 (priority, cut points);
// "GQA Per-Head Scoring Streams" (head grouping, stream aggregation, the
// 64-byte record); "KV cache offload" post, "Top row" (block tables).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kvs.h"
#include "kvs_internal.h"

namespace kvs {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));

constexpr int kHeadDim = 128;
constexpr int kGroup = 8;                 // query heads per KV head
constexpr int kQHeads = 64;
constexpr int kTileBytes = 16 * kHeadDim * 2;          // fp16 (layer, K|V, KV head) tile: 4 KiB
static_assert(decode_lds_bytes(1024) <= kMaxDecodeLds, "largest split must fit the LDS bound");
static_assert(decode_lds_bytes(0) == kTileBytes, "value stage holds one fp16 tile");

__device__ __forceinline__ float xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ void flag(uint32_t* status, uint32_t bit) {
  atomicOr(status, bit);
}

// Shared validity check of one sequence's device-side description.  Returns the
// number of blocks, or -1 (and sets a status bit from lane 0 of the first wave
// that sees it) when the sequence must be skipped.
__device__ __forceinline__ int seq_blocks(const int32_t* seq_lens, const int32_t* meta_off,
                                          int s, int max_nb, int64_t total_blocks,
                                          uint32_t* status, bool report, int* r0_out) {
  const int n = seq_lens[s];
  const int r0 = meta_off[s];
  const int r1 = meta_off[s + 1];
  if (n < 0 || n > 16 * max_nb) {
    if (report) flag(status, KVS_DEV_BAD_SEQ_LEN);
    return -1;
  }
  const int nb = (n + 15) >> 4;
  if (r0 < 0 || r1 - r0 < nb || (int64_t)r1 > total_blocks) {
    if (report) flag(status, KVS_DEV_BAD_OFFSETS);
    return -1;
  }
  *r0_out = r0;
  return nb;
}

// ---------------------------------------------------------------------------
// paged_decode_gqa
//
// One 64-lane wave owns (s, layer, g, split).  Lane l = 16 j + c.
//  QK:  S^T[token][head] = K[token][:] . q[head][:] on v_mfma_f32_16x16x32_f16,
//       A = the 16x128 key tile (lane reads 64 contiguous bytes of row c), B =
//       the 8 queries of the group padded to 16 columns.  The result gives
//       lane (j, c) the logits of head c for tokens 4j..4j+3.
//  PV:  O^T[d][head] += V^T[d][token] P^T[token][head] on
//       v_mfma_f32_16x16x16_f16.  P^T is exactly the QK result layout (after
//       rounding to fp16).  V^T needs the value tile transposed: it is staged
//       through 4 KiB of LDS, each lane reads 4 rows x 16 bytes, and byte
//       permutes build the operand of each of the 8 output tiles.  Output tile
//       k holds d = 8 m + k, so lane (j, c) ends with the 32 contiguous values
//       d in [32 j, 32 j + 32) of head c.
//  Online softmax in base 2: logits are scaled by scale * log2(e); a running
//  maximum per head; the per-block mass of head c is kept in LDS relative to
//  the current maximum and rescaled whenever that maximum grows.
// ---------------------------------------------------------------------------
// K/V tiles are read exactly once per step.  Value loads are non-temporal:
// each instruction reads 1 KiB contiguous, and on gfx950 that measured ~10 %
// faster than plain loads.  Key loads stay plain: an instruction covers 16 rows
// x 64 bytes, half of each 128-byte line, and non-temporal loads of partial
// lines measured slower (the line is fetched again by the second half).
__device__ __forceinline__ u4_t stream_load(const u4_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u4_t plain_load(const u4_t* p) { return *p; }

// Stored K/V element formats.  A (layer, K|V, KV head) tile is 16 rows of 128
// elements; a block holds, per layer, 8 key tiles then 8 value tiles.
struct KvF16 {
  static constexpr int kElemBytes = 2;
  static constexpr int kLoads = 4;   // 16-byte loads per lane per tile
  static constexpr int kRing = 2;    // ring slots (32 VGPRs each)
};
struct KvE4M3 {                      // FP8 E4M3 codes, no scale
  static constexpr int kElemBytes = 1;
  static constexpr int kLoads = 2;
  static constexpr int kRing = 2;    // 16 VGPRs each; 3 and 4 measured slower
};

template <class F>
struct BlockRegs {
  u4_t k[F::kLoads];
  u4_t v[F::kLoads];
};

template <class F>
constexpr int tile_bytes() { return 16 * kHeadDim * F::kElemBytes; }

// First of the 8 elements of a 128-element row that lane group j feeds to QK
// step i (key and query alike, so the 128-term dot product is covered once).
// Key load i of lane (j, c) reads bytes [64 i + 16 j, 64 i + 16 j + 16) of row
// c: each load instruction reads whole 64-byte row segments.
template <class F>
__device__ __forceinline__ int qk_elem(int i, int j) {
  if constexpr (F::kElemBytes == 2) return 32 * i + 8 * j;          // load i
  else return 64 * (i >> 1) + 16 * j + 8 * (i & 1);                 // half i & 1 of load i >> 1
}

// Issues exactly 2 * F::kLoads 16-byte loads per lane: the key tile in the QK
// operand layout above and the value tile in plain order (load i covers bytes
// [1024 i, 1024 i + 1024)).  Always issuing the same number of loads on every
// path lets the compiler wait for one ring slot precisely instead of draining
// every load in flight.
template <class F>
__device__ __forceinline__ void load_block(BlockRegs<F>& r, const uint8_t* base, int lane, int c,
                                           int j) {
  const uint8_t* kp = base + c * (kHeadDim * F::kElemBytes) + j * 16;
  const uint8_t* vp = base + 8 * tile_bytes<F>() + lane * 16;
#pragma unroll
  for (int i = 0; i < F::kLoads; ++i)
    r.k[i] = plain_load(reinterpret_cast<const u4_t*>(kp + i * 64));
#pragma unroll
  for (int i = 0; i < F::kLoads; ++i)
    r.v[i] = stream_load(reinterpret_cast<const u4_t*>(vp + i * 1024));
}

// Four E4M3 codes to four fp16 values (exact: every finite E4M3 value is an
// fp16 value), with gfx950's packed scaled conversion at scale 1.
__device__ __forceinline__ u2_t e4m3x4_to_f16(uint32_t w) {
  const h2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const h2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return u2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Value tile of one ring slot to LDS as row-major fp16 [16][128].
template <class F>
__device__ __forceinline__ void stage_values(const BlockRegs<F>& r, u4_t* vstage, int lane) {
  if constexpr (F::kElemBytes == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vstage[i * 64 + lane] = r.v[i];
  } else {
    // load i, lane l: row 8 i + l / 8, elements [16 (l % 8), 16 (l % 8) + 16)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const u2_t a = e4m3x4_to_f16(r.v[i][0]);
      const u2_t b = e4m3x4_to_f16(r.v[i][1]);
      const u2_t c2 = e4m3x4_to_f16(r.v[i][2]);
      const u2_t d = e4m3x4_to_f16(r.v[i][3]);
      const int base = (8 * i + (lane >> 3)) * 16 + 2 * (lane & 7);
      vstage[base] = u4_t{a[0], a[1], b[0], b[1]};
      vstage[base + 1] = u4_t{c2[0], c2[1], d[0], d[1]};
    }
  }
}

// QK operand i of one ring slot: 8 fp16 key elements from qk_elem(i, j) on.
template <class F>
__device__ __forceinline__ h8_t key_operand(const BlockRegs<F>& r, int i) {
  if constexpr (F::kElemBytes == 2) {
    return __builtin_bit_cast(h8_t, r.k[i]);
  } else {
    const u4_t w = r.k[i >> 1];
    const u2_t a = e4m3x4_to_f16(w[(i & 1) * 2]);
    const u2_t b = e4m3x4_to_f16(w[(i & 1) * 2 + 1]);
    return __builtin_bit_cast(h8_t, u4_t{a[0], a[1], b[0], b[1]});
  }
}

// Blocks whose loads are in flight per wave: the ring slot being processed
// plus kRing - 1 ahead (32 VGPRs per slot).  Deeper rings at lower occupancy
// measured no faster on gfx950.  One wave per work-group, one KV head each:
// work-groups of 4 or 8 waves reading neighbouring heads measured no faster.
template <class F>
__global__ void __launch_bounds__(64, kDecodeWavesPerSimd) paged_decode_gqa(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int SB = a.split_blocks;
  // LDS layout (decode_lds_bytes): block ids, mass partials, value stage.
  int32_t* tbl = reinterpret_cast<int32_t*>(smem);                          // [SB] block ids
  float* pi_lds = reinterpret_cast<float*>(smem + (size_t)4 * SB);          // [8][SB]
  u4_t* vstage = reinterpret_cast<u4_t*>(smem + (size_t)36 * SB);           // 16 x 16 chunks of 16 B

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int j = lane >> 4;

  uint32_t w = blockIdx.x;
  const uint32_t lgg_count = (uint32_t)a.n_layers * 8u;
  const int lgg = (int)(w % lgg_count);
  w /= lgg_count;
  const int split = (int)(w % (uint32_t)a.n_splits);
  const int s = (int)(w / (uint32_t)a.n_splits);
  const int lr = lgg >> 3;
  const int g = lgg & 7;
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

  // B operand of QK: queries of the group, rows 8..15 zero.
  h8_t qb[4];
  if (c < kGroup) {
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
  float l_run = 0.f;
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
  BlockRegs<F> ring[kRing];
  bool ring_ok[kRing];
#pragma unroll
  for (int k = 0; k < kRing; ++k)
    load_block(ring[k], slot_block(b0 + k, &ring_ok[k]), lane, c, j);

  bool saw_bad = false;
  for (int bbase = b0; bbase < b1; bbase += kRing) {
#pragma unroll
    for (int k = 0; k < kRing; ++k) {
      const int b = bbase + k;
      const bool active = b < b1;
      const bool cur_ok = ring_ok[k];
      saw_bad |= active && !cur_ok;
      const int valid = cur_ok ? min(16, n - 16 * b) : 0;

      // ---- value tile to LDS (the slot's value registers are free after this)
      stage_values<F>(ring[k], vstage, lane);

      // ---- logits of 16 tokens x 16 (8 real) heads
      f4_t sacc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand<F>(ring[k], i), qb[i], sacc,
                                                      0, 0, 0);

      // ---- refill this slot with the block kRing ahead
      load_block(ring[k], slot_block(b + kRing, &ring_ok[k]), lane, c, j);

      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = sacc[i] * a.scale_log2;
      if (valid < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * j + i >= valid) sv[i] = -INFINITY;
      }

      // ---- online softmax (per head = per c; the 4 lanes j share a head)
      float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      bm = fmaxf(bm, xor_f(bm, 16));
      bm = fmaxf(bm, xor_f(bm, 32));
      const float m_new = fmaxf(m_run, bm);
      const bool live = m_new != -INFINITY;
      const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[i] = live ? __builtin_amdgcn_exp2f(sv[i] - m_new) : 0.f;
      const float ps = (pv[0] + pv[1]) + (pv[2] + pv[3]);
      l_run = l_run * alpha + ps;
      float bs = ps + xor_f(ps, 16);
      bs += xor_f(bs, 32);

      if (__ballot(c < kGroup && alpha != 1.f) != 0ull) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] *= alpha;
        if (c < kGroup)
          for (int idx = j; idx < b - b0; idx += 4) pi_lds[c * SB + idx] *= alpha;
      }
      if (active && c < kGroup && j == 0) pi_lds[c * SB + (b - b0)] = bs;
      m_run = m_new;

      // ---- PV: transposed value rows from LDS
      u4_t R[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) R[i] = vstage[(4 * j + i) * 16 + c];
      if (valid < 16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * j + i >= valid) R[i] = u4_t{0u, 0u, 0u, 0u};
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

  // ---- split epilogue: statistics, partial output, mass partials
  float lt = l_run + xor_f(l_run, 16);
  lt += xor_f(lt, 32);
  const size_t st = (((size_t)s * a.n_layers + lr) * kQHeads + kGroup * g + c) * a.n_splits + split;
  if (c < kGroup) {
    if (j == 0) a.ml[st] = make_float2(m_run, lt);
    float* op = a.opart + st * kHeadDim + 32 * j;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<f4_t*>(op + 8 * i) = f4_t{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
      *reinterpret_cast<f4_t*>(op + 8 * i + 4) = f4_t{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
    }
  }
  __syncthreads();
  const int cnt = b1 - b0;
  for (int hh = 0; hh < kGroup; ++hh) {
    float* dst = a.pi + ((size_t)lr * kQHeads + kGroup * g + hh) * a.total_blocks + r0 + b0;
    for (int bb = lane; bb < cnt; bb += 64) dst[bb] = pi_lds[hh * SB + bb];
  }
}

// ---------------------------------------------------------------------------
// paged_decode_kivi
//
// The split-K decode above over a KIVI cache (Fitting a Million Tokens, Sec.
// 02: 2-bit codes plus fp16 scales, dequantised inside the attention kernel).
// Quantised blocks come in 32-token pairs (one key group).  A wave loads a
// pair's four 768-byte tiles of its (layer, KV head) with three coalesced
// 16-byte loads per lane into a register ring, stages them in LDS and works on
// the codes directly, never forming dequantised keys or values:
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
//  fp16 residual blocks (from quant_lens[s] on) run one by one with the same
//  operand layouts (value tile transposed through LDS).
// ---------------------------------------------------------------------------
constexpr int kKiviRing = 2;     // 32-token pairs in flight per wave

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

__global__ void __launch_bounds__(64, kDecodeWavesPerSimd) paged_decode_kivi(DecodeArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int SB = a.split_blocks;
  int32_t* tbl = reinterpret_cast<int32_t*>(smem);                          // [SB] block ids
  float* pi_lds = reinterpret_cast<float*>(smem + (size_t)4 * SB);          // [8][SB]
  uint8_t* stage = smem + (size_t)36 * SB;       // 4 KiB: a pair's four tiles or an fp16 value tile

  const int lane = threadIdx.x;
  const int c = lane & 15;
  const int j = lane >> 4;

  uint32_t w = blockIdx.x;
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

  // B operand of QK: queries of the group, channels 32 i + 8 j .. + 8; rows 8..15 zero.
  h8_t qb[4];
  if (c < kGroup) {
    const uint16_t* qp =
        a.q + ((((size_t)s * a.num_layers + layer) * kQHeads + kGroup * g + c) * kHeadDim);
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = *reinterpret_cast<const h8_t*>(qp + 32 * i + 8 * j);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) qb[i] = h8_t{0, 0, 0, 0, 0, 0, 0, 0};
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f4_t acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f4_t{0.f, 0.f, 0.f, 0.f};
  float zacc[4] = {0.f, 0.f, 0.f, 0.f};
  bool saw_bad = false;

  // Online softmax of one block's 16 x 16 logits (base 2); returns p relative
  // to the running maximum and keeps the block's probability mass in LDS.
  auto softmax_block = [&](const float (&sv)[4], int b, float (&pv)[4]) {
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = fmaxf(bm, xor_f(bm, 16));
    bm = fmaxf(bm, xor_f(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const bool live = m_new != -INFINITY;
    const float alpha = live ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = live ? __builtin_amdgcn_exp2f(sv[i] - m_new) : 0.f;
    const float ps = (pv[0] + pv[1]) + (pv[2] + pv[3]);
    l_run = l_run * alpha + ps;
    float bs = ps + xor_f(ps, 16);
    bs += xor_f(bs, 32);
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

  // The same for a block whose 16 logits are all finite (m_new is finite, so
  // no masked-out head needs guarding).
  auto softmax_full = [&](const float (&sv)[4], int b, float (&pv)[4]) {
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = fmaxf(bm, xor_f(bm, 16));
    bm = fmaxf(bm, xor_f(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_new);
    const float ps = (pv[0] + pv[1]) + (pv[2] + pv[3]);
    l_run = l_run * alpha + ps;
    float bs = ps + xor_f(ps, 16);
    bs += xor_f(bs, 32);
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

  // ---- quantised blocks [b0, bq1), in pairs (b0 and nq / 16 are even)
  const int bq1 = min(b1, nq >> 4);
  if (bq1 > b0) {
    const size_t kblock = (size_t)a.num_layers * 16 * kKiviTileBytes;
    const size_t ktile = ((size_t)(layer * 2) * 8 + g) * kKiviTileBytes;
    const size_t vtile = ((size_t)(layer * 2 + 1) * 8 + g) * kKiviTileBytes;
    // lane's 16-byte pieces: byte 1024 k + 16 lane of [K even | K odd | V even | V odd]
    int piece_tile[3], piece_off[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const int P = 1024 * k + 16 * lane;
      piece_tile[k] = P / kKiviTileBytes;
      piece_off[k] = P - piece_tile[k] * kKiviTileBytes;
    }
    // Loads of the pair starting at block be; pairs past the split's quantised
    // range reuse its last pair (in-bounds, unused), ids outside the pool read
    // block 0 and are masked.
    auto load_pair = [&](u4_t (&r)[3], int be, bool* ok) {
      const int cl = min(be, bq1 - 2);
      // block ids are wave-uniform: scalar registers keep the address math off the VALU
      const int pe = __builtin_amdgcn_readfirstlane(tbl[cl - b0]);
      const int po = __builtin_amdgcn_readfirstlane(tbl[cl + 1 - b0]);
      const bool in = pe >= 0 && (int64_t)pe < a.kivi_blocks && po >= 0 &&
                      (int64_t)po < a.kivi_blocks;
      *ok = in && be < bq1;
      const uint8_t* pe_p = a.kivi + (size_t)(in ? pe : 0) * kblock;
      const uint8_t* po_p = a.kivi + (size_t)(in ? po : 0) * kblock;
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int ti = piece_tile[k];
        const uint8_t* base = ((ti & 1) ? po_p : pe_p) + ((ti & 2) ? vtile : ktile);
        r[k] = stream_load(reinterpret_cast<const u4_t*>(base + piece_off[k]));
      }
    };

    u4_t ring[kKiviRing][3];
    bool ring_ok[kKiviRing];
#pragma unroll
    for (int k = 0; k < kKiviRing; ++k) load_pair(ring[k], b0 + 2 * k, &ring_ok[k]);

    for (int pb = b0; pb < bq1; pb += 2 * kKiviRing) {
#pragma unroll
      for (int k = 0; k < kKiviRing; ++k) {
        const int be = pb + 2 * k;
        const bool active = be < bq1;
        const bool ok = ring_ok[k];
        saw_bad |= active && !ok;
#pragma unroll
        for (int kk = 0; kk < 3; ++kk)
          *reinterpret_cast<u4_t*>(stage + 1024 * kk + 16 * lane) = ring[k][kk];
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
        h8_t qhi[4], qlo[4];
        f4_t zsacc = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint8_t* km = stage + (i >> 1) * kKiviTileBytes + 512 + 2 * (32 * (i & 1) + 8 * j);
          const h8_t s8 = *reinterpret_cast<const h8_t*>(km);
          const h8_t z8 = *reinterpret_cast<const h8_t*>(km + 128);
          qhi[i] = qb[i] * s8;
          qlo[i] = __builtin_elementwise_fma(qb[i], s8, -qhi[i]);
          zsacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(z8, qb[i], zsacc, 0, 0, 0);
        }

#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int b = be + hb;
          const u2_t kent = *reinterpret_cast<const u2_t*>(stage + hb * kKiviTileBytes + 8 * lane);
          f4_t sacc = zsacc;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const h8_t kc = codes_to_h8(code_set(kent, i));
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc, qhi[i], sacc, 0, 0, 0);
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc, qlo[i], sacc, 0, 0, 0);
          }
          float sv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[i] = sacc[i] * a.scale_log2;
          float pv[4];
          softmax_full(sv, b, pv);

          const uint8_t* vt = stage + (2 + hb) * kKiviTileBytes;
          const u2_t vent = *reinterpret_cast<const u2_t*>(vt + 8 * lane);
          const h4_t pb4 = h4_t{(_Float16)pv[0], (_Float16)pv[1], (_Float16)pv[2], (_Float16)pv[3]};
#pragma unroll
          for (int grp = 0; grp < 4; ++grp) {
            const h4_t s4 = *reinterpret_cast<const h4_t*>(vt + 512 + 2 * (16 * grp + 4 * j));
            const h4_t z4 = *reinterpret_cast<const h4_t*>(vt + 640 + 2 * (16 * grp + 4 * j));
            const h4_t bp = pb4 * s4;
            zacc[grp] = dot2(h2_t{pb4[2], pb4[3]}, h2_t{z4[2], z4[3]},
                             dot2(h2_t{pb4[0], pb4[1]}, h2_t{z4[0], z4[1]}, zacc[grp]));
            const h8_t vc = codes_to_h8(code_set(vent, grp));
            acc[2 * grp] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                h4_t{vc[0], vc[1], vc[2], vc[3]}, bp, acc[2 * grp], 0, 0, 0);
            acc[2 * grp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                h4_t{vc[4], vc[5], vc[6], vc[7]}, bp, acc[2 * grp + 1], 0, 0, 0);
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
      for (int i = 0; i < 4; ++i) sv[i] = 4 * j + i < valid ? sacc[i] * a.scale_log2 : -INFINITY;
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
  if (saw_bad && lane == 0) flag(a.status, KVS_DEV_BAD_BLOCK_ID);

  // ---- split epilogue: statistics, partial output (+ value zero-point terms), mass partials
  float lt = l_run + xor_f(l_run, 16);
  lt += xor_f(lt, 32);
  float zt[4];
#pragma unroll
  for (int grp = 0; grp < 4; ++grp) {
    zt[grp] = zacc[grp] + xor_f(zacc[grp], 16);
    zt[grp] += xor_f(zt[grp], 32);
  }
  if (c < kGroup) {
    if (j == 0) a.ml[st] = make_float2(m_run, lt);
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
  for (int hh = 0; hh < kGroup; ++hh) {
    float* dst = a.pi + ((size_t)lr * kQHeads + kGroup * g + hh) * a.total_blocks + r0 + b0;
    for (int bb = lane; bb < cnt; bb += 64) dst[bb] = pi_lds[hh * SB + bb];
  }
}

// ---------------------------------------------------------------------------
// combine_splits: one wave per (s, layer, head).  Lane handles d = 2 lane, +1.
//   M = max_k m_k, Lambda = sum_k l_k 2^(m_k - M), w_k = 2^(m_k - M) / Lambda,
//   out = sum_k w_k o_k (fp16), and w_k is kept for the mass reduction.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) combine_splits(CombineArgs a) {
  const int lane = threadIdx.x;
  uint32_t w = blockIdx.x;
  const int h = (int)(w % kQHeads);
  w /= kQHeads;
  const int lr = (int)(w % (uint32_t)a.n_layers);
  const int s = (int)(w / (uint32_t)a.n_layers);
  const int layer = a.layer_begin + lr;
  uint32_t* outp = reinterpret_cast<uint32_t*>(
      a.out + ((((size_t)s * a.num_layers + layer) * kQHeads + h) * kHeadDim));

  int r0 = 0;
  const int nb = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                            false, &r0);
  if (nb <= 0) {
    outp[lane] = 0u;
    return;
  }
  const int nsp = (nb + a.split_blocks - 1) / a.split_blocks;
  const size_t base = (((size_t)s * a.n_layers + lr) * kQHeads + h) * a.n_splits;

  float M = -INFINITY;
  for (int k = lane; k < nsp; k += 64) M = fmaxf(M, a.ml[base + k].x);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, xor_f(M, m));
  double L = 0.0;
  if (M != -INFINITY)
    for (int k = lane; k < nsp; k += 64) {
      const float2 v = a.ml[base + k];
      L += (double)v.y * (double)__builtin_amdgcn_exp2f(v.x - M);
    }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) L += __shfl_xor(L, m, 64);
  const bool dead = !(L > 0.0);
  const double invL = dead ? 0.0 : 1.0 / L;

  for (int k = lane; k < nsp; k += 64) {
    const float2 v = a.ml[base + k];
    a.wsplit[base + k] = dead ? 0.f : (float)((double)__builtin_amdgcn_exp2f(v.x - M) * invL);
  }
  float o0 = 0.f, o1 = 0.f;
  for (int k = 0; k < nsp; ++k) {
    const float2 v = a.ml[base + k];
    const float wk = dead ? 0.f : (float)((double)__builtin_amdgcn_exp2f(v.x - M) * invL);
    const float2 ov = reinterpret_cast<const float2*>(a.opart + (base + k) * kHeadDim)[lane];
    o0 = fmaf(wk, ov.x, o0);
    o1 = fmaf(wk, ov.y, o1);
  }
  const _Float16 h0 = (_Float16)o0, h1 = (_Float16)o1;
  outp[lane] = (uint32_t)__builtin_bit_cast(uint16_t, h0) |
               ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
}

// ---------------------------------------------------------------------------
// block_mass: mass[s, b] = sum over (layer, query head) of pi * w_split, fp64
// accumulation in a fixed order (row order within each wave, then waves in
// order), so the result depends only on logical indices.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kMassThreads) block_mass(MassArgs a) {
  __shared__ double red[kMassThreads / 64][64];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  constexpr int kWaves = kMassThreads / 64;
  const int s = blockIdx.y;
  int r0 = 0;
  const int nb = seq_blocks(a.seq_lens, a.meta_off, s, a.max_nb, a.total_blocks, a.status,
                            false, &r0);
  if (nb <= 0 || (int)blockIdx.x * 64 >= nb) return;
  const int b = blockIdx.x * 64 + lane;
  const bool act = b < nb;
  const int r = r0 + (act ? b : 0);
  const int split = (act ? b : 0) / a.split_blocks;
  const int rows = a.n_layers * kQHeads;
  double acc = 0.0;
  if (act) {
    const float* pcol = a.pi + r;
    const float* wcol = a.wsplit + (size_t)s * a.n_layers * kQHeads * a.n_splits + split;
#pragma unroll 8
    for (int row = wv; row < rows; row += kWaves)
      acc += (double)pcol[(size_t)row * a.total_blocks] * (double)wcol[(size_t)row * a.n_splits];
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && act) {
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) t += red[k][lane];
    if (a.accumulate) t += (double)a.mass[r];
    a.mass[r] = (float)t;
  }
}

// ---------------------------------------------------------------------------
// Scoring kernels.  Grid (chunk of kScoreThreads records, sequence).
// ---------------------------------------------------------------------------
// Live records of sequence s: [r0, r0 + nb).  Records [r0, r1) are the
// sequence's capacity; with seq_lens, nb = ceil(seq_lens[s] / 16) <= r1 - r0,
// otherwise every record of the capacity is live.
__device__ __forceinline__ int seq_records(const int32_t* off, const int32_t* seq_lens, int s,
                                           int max_nb, int64_t total_blocks, uint32_t* status,
                                           bool report, int* r0_out) {
  const int r0 = off[s];
  const int r1 = off[s + 1];
  if (r0 < 0 || r1 < r0 || r1 - r0 > max_nb || (int64_t)r1 > total_blocks) {
    if (report) flag(status, KVS_DEV_BAD_OFFSETS);
    return -1;
  }
  int nb = r1 - r0;
  if (seq_lens) {
    const int n = seq_lens[s];
    if (n < 0 || ((n + 15) >> 4) > nb) {
      if (report) flag(status, KVS_DEV_BAD_SEQ_LEN);
      return -1;
    }
    nb = (n + 15) >> 4;
  }
  *r0_out = r0;
  return nb;
}

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, xor_f(v, m));
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int k = 1; k < kScoreThreads / 64; ++k) r = fmaxf(r, red[k]);
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kScoreThreads) seq_chunk_max(ScoreArgs a) {
  __shared__ float red[kScoreThreads / 64];
  const int s = blockIdx.y;
  const int chunk = blockIdx.x;
  int r0 = 0;
  const int nb = seq_records(a.meta_off, a.seq_lens, s, a.max_nb, a.total_blocks, a.status,
                             threadIdx.x == 0 && chunk == 0, &r0);
  if (nb <= 0 || chunk * kScoreThreads >= nb) return;
  const int b = chunk * kScoreThreads + threadIdx.x;
  float v = b < nb ? a.mass[r0 + b] : 0.f;
  v = block_reduce_max(v, red);
  if (threadIdx.x == 0) a.chunk_max[(size_t)s * a.max_chunks + chunk] = v;
}

__device__ __forceinline__ void priority_and_tier(const ScorePolicy& p, int b, int nb, double score,
                                                  uint8_t flags, double* P, uint8_t* tier) {
  const double R = (double)(b + 1) / (double)nb;
  const double N = (flags & KVS_FLAG_ANCHOR) ? 1.0 : 0.0;
  const double pr = p.w_recency * R + p.w_ema * score + p.w_anchor * N;
  *P = pr;
  *tier = pr >= p.t_high ? 0 : (pr >= p.t_low ? 1 : 2);
}

__global__ void __launch_bounds__(kScoreThreads) score_update(ScoreArgs a) {
  __shared__ float red[kScoreThreads / 64];
  const int s = blockIdx.y;
  const int chunk = blockIdx.x;
  int r0 = 0;
  const int nb = seq_records(a.meta_off, a.seq_lens, s, a.max_nb, a.total_blocks, a.status, false, &r0);
  if (nb <= 0 || chunk * kScoreThreads >= nb) return;
  const int nch = (nb + kScoreThreads - 1) / kScoreThreads;
  float M = 0.f;
  for (int k = threadIdx.x; k < nch; k += kScoreThreads)
    M = fmaxf(M, a.chunk_max[(size_t)s * a.max_chunks + k]);
  M = block_reduce_max(M, red);

  const int b = chunk * kScoreThreads + threadIdx.x;
  bool stale = false;
  if (b < nb) {
    kvs_block_meta* rec = a.meta + r0 + b;
    const uint64_t tt = rec->t_touch;
    if (tt != KVS_NEVER_TOUCHED && tt >= a.step) {
      stale = true;
    } else {
      const double mh = M > 0.f ? (double)a.mass[r0 + b] / (double)M : 0.0;
      // Input 0 on the steps since the last touch: the stored score first
      // decays over the gap, then takes the one-step update.
      double prev = rec->score;
      if (tt != KVS_NEVER_TOUCHED && a.step - tt > 1)
        prev *= pow(1.0 - a.pol.alpha, (double)(a.step - tt - 1));
      const double e = a.pol.alpha * mh + (1.0 - a.pol.alpha) * prev;
      rec->score = e;
      rec->touch_count = rec->touch_count + 1u;
      rec->t_touch = a.step;
      if (a.classify) {
        double P;
        uint8_t tier;
        priority_and_tier(a.pol, b, nb, e, rec->flags, &P, &tier);
        rec->priority = P;
        rec->tier = tier;
      }
    }
  }
  if (__ballot(stale) != 0ull && (threadIdx.x & 63) == 0) flag(a.status, KVS_DEV_STALE_STEP);
}

// ---------------------------------------------------------------------------
// eviction candidates: per sequence, argmin over its records of the
// order-preserving key K = ln score + t_touch * (-ln(1 - alpha)) (a zero score
// gives -inf), ties to the lowest logical block.  Pass 1 reduces chunks of
// kScoreThreads records, pass 2 the chunks; both in a fixed order.
// ---------------------------------------------------------------------------
struct KeyIdx {
  double key;
  int32_t idx;   // logical block, or -1 for none
};

__device__ __forceinline__ KeyIdx better(KeyIdx x, KeyIdx y) {
  if (x.idx < 0) return y;
  if (y.idx < 0) return x;
  if (y.key < x.key || (y.key == x.key && y.idx < x.idx)) return y;
  return x;
}

__device__ __forceinline__ KeyIdx block_reduce_argmin(KeyIdx v, double* rk, int32_t* ri) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    KeyIdx o;
    o.key = __shfl_xor(v.key, m, 64);
    o.idx = __shfl_xor(v.idx, m, 64);
    v = better(v, o);
  }
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    rk[wv] = v.key;
    ri[wv] = v.idx;
  }
  __syncthreads();
  KeyIdx r{rk[0], ri[0]};
#pragma unroll
  for (int k = 1; k < kScoreThreads / 64; ++k) r = better(r, KeyIdx{rk[k], ri[k]});
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kScoreThreads) evict_chunks(EvictArgs a) {
  __shared__ double rk[kScoreThreads / 64];
  __shared__ int32_t ri[kScoreThreads / 64];
  const int s = blockIdx.y;
  const int chunk = blockIdx.x;
  int r0 = 0;
  const int nb = seq_records(a.meta_off, a.seq_lens, s, a.max_nb, a.total_blocks, a.status,
                             threadIdx.x == 0 && chunk == 0, &r0);
  if (nb <= 0 || chunk * kScoreThreads >= nb) return;
  const bool active = a.active == nullptr || a.active[s] != 0;
  const int b = chunk * kScoreThreads + threadIdx.x;
  KeyIdx v{0.0, -1};
  bool future = false;
  if (active && b < nb) {
    const kvs_block_meta* rec = a.meta + r0 + b;
    const uint64_t tt = rec->t_touch;
    const bool pinned = a.exclude_pinned && rec->tier == 0;
    future = tt != KVS_NEVER_TOUCHED && tt > a.now;
    if (!pinned && !future) {
      const double sc = rec->score;
      const double t = tt == KVS_NEVER_TOUCHED ? 0.0 : (double)tt;
      v.key = sc > 0.0 ? log(sc) + t * a.neg_log_keep : -INFINITY;
      v.idx = b;
    }
  }
  if (__ballot(future) != 0ull && (threadIdx.x & 63) == 0) flag(a.status, KVS_DEV_STALE_STEP);
  const KeyIdx r = block_reduce_argmin(v, rk, ri);
  if (threadIdx.x == 0) {
    a.part_key[(size_t)s * a.max_chunks + chunk] = r.key;
    a.part_idx[(size_t)s * a.max_chunks + chunk] = r.idx;
  }
}

__global__ void __launch_bounds__(kScoreThreads) evict_final(EvictArgs a) {
  __shared__ double rk[kScoreThreads / 64];
  __shared__ int32_t ri[kScoreThreads / 64];
  const int s = blockIdx.x;
  int r0 = 0;
  const int nb = seq_records(a.meta_off, a.seq_lens, s, a.max_nb, a.total_blocks, a.status, false, &r0);
  const bool active = a.active == nullptr || a.active[s] != 0;
  KeyIdx v{0.0, -1};
  if (nb > 0 && active) {
    const int nch = (nb + kScoreThreads - 1) / kScoreThreads;
    for (int k = threadIdx.x; k < nch; k += kScoreThreads)
      v = better(v, KeyIdx{a.part_key[(size_t)s * a.max_chunks + k],
                           a.part_idx[(size_t)s * a.max_chunks + k]});
  }
  const KeyIdx r = block_reduce_argmin(v, rk, ri);
  if (threadIdx.x == 0) {
    a.out_block[s] = r.idx;
    a.out_key[s] = r.idx < 0 ? INFINITY : r.key;
  }
}

__global__ void __launch_bounds__(kScoreThreads) classify_records(ScoreArgs a) {
  const int s = blockIdx.y;
  int r0 = 0;
  const int nb = seq_records(a.meta_off, a.seq_lens, s, a.max_nb, a.total_blocks, a.status, false, &r0);
  const int b = blockIdx.x * kScoreThreads + threadIdx.x;
  if (nb <= 0 || b >= nb) return;
  kvs_block_meta* rec = a.meta + r0 + b;
  double P;
  uint8_t tier;
  priority_and_tier(a.pol, b, nb, rec->score, rec->flags, &P, &tier);
  rec->priority = P;
  rec->tier = tier;
  if (a.tiers_out) a.tiers_out[r0 + b] = tier;
}

__global__ void __launch_bounds__(kScoreThreads) meta_init(MetaInitArgs a) {
  const int s = blockIdx.y;
  int r0 = 0;
  const int nb = seq_records(a.meta_off, a.seq_lens, s, a.max_nb, a.total_blocks, a.status, false, &r0);
  const int b = blockIdx.x * kScoreThreads + threadIdx.x;
  if (nb <= 0 || b >= nb) return;
  kvs_block_meta rec;
  rec.key[0] = a.seq_ids[s];
  rec.key[1] = (uint64_t)b;
  rec.score = 0.0;
  rec.t_touch = KVS_NEVER_TOUCHED;
  rec.touch_count = 0u;
  rec.tier = KVS_UNCLASSIFIED;
  rec.flags = b < a.anchor_blocks ? KVS_FLAG_ANCHOR : 0u;
  rec.reserved0 = 0u;
  rec.priority = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) rec.reserved1[i] = 0u;
  a.meta[r0 + b] = rec;
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
      } else if (n - nq >= a.residual + 32) {
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

// ---------------------------------------------------------------------------
// KV append.  append_alloc (one work-group) walks the batch in order, hands
// each sequence whose new token opens a block the next id from the top of the
// free stack (an exclusive prefix count over the sequences that need one),
// sets the table entry, creates the block's record and advances seq_lens.
// append_scatter writes the token's K and V rows into their slot.
// ---------------------------------------------------------------------------
constexpr int kAllocThreads = 1024;

__device__ __forceinline__ kvs_block_meta fresh_record(uint64_t seq_id, int b, int anchor_blocks) {
  kvs_block_meta rec;
  rec.key[0] = seq_id;
  rec.key[1] = (uint64_t)b;
  rec.score = 0.0;
  rec.t_touch = KVS_NEVER_TOUCHED;
  rec.touch_count = 0u;
  rec.tier = KVS_UNCLASSIFIED;
  rec.flags = b < anchor_blocks ? KVS_FLAG_ANCHOR : 0u;
  rec.reserved0 = 0u;
  rec.priority = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) rec.reserved1[i] = 0u;
  return rec;
}

__global__ void __launch_bounds__(kAllocThreads) append_alloc(AppendArgs a, int batch) {
  __shared__ int scan[kAllocThreads];
  const int tid = threadIdx.x;
  int top0 = *a.free_top;
  if (top0 < 0 || top0 > a.free_capacity) {
    if (tid == 0) flag(a.status, KVS_DEV_BAD_OFFSETS);
    top0 = top0 < 0 ? 0 : a.free_capacity;
  }
  int carry = 0;
  for (int base = 0; base < batch; base += kAllocThreads) {
    const int s = base + tid;
    int need = 0, t = 0, b = 0, slot = 0, r0 = 0, cap = 0;
    bool valid = false;
    if (s < batch) {
      t = a.seq_lens[s];
      r0 = a.meta_off[s];
      cap = a.meta_off[s + 1] - r0;
      valid = t >= 0 && r0 >= 0 && cap >= 0 && cap <= a.max_nb &&
              (int64_t)r0 + cap <= a.total_blocks && ((t + 15) >> 4) <= cap;
      b = t >> 4;
      slot = t & 15;
      need = (valid && slot == 0 && b < cap) ? 1 : 0;
    }
    scan[tid] = need;
    __syncthreads();
    for (int off = 1; off < kAllocThreads; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int prefix = carry + scan[tid] - need;
    if (s < batch) {
      int pid = -1;
      if (!valid) {
        flag(a.status, KVS_DEV_BAD_SEQ_LEN);
      } else if (slot == 0) {
        if (need && prefix < top0) {
          const int cand = a.free_stack[top0 - 1 - prefix];
          if (cand >= 0 && (int64_t)cand < a.pool_blocks) {
            pid = cand;
            a.table[(size_t)s * a.max_nb + b] = pid;
            a.meta[r0 + b] = fresh_record(a.seq_ids[s], b, a.anchor_blocks);
          } else {
            flag(a.status, KVS_DEV_BAD_BLOCK_ID);
          }
        } else {
          flag(a.status, KVS_DEV_POOL_EXHAUSTED);
        }
      } else {
        const int cur = a.table[(size_t)s * a.max_nb + b];
        if (cur >= 0 && (int64_t)cur < a.pool_blocks) pid = cur;
        else flag(a.status, KVS_DEV_BAD_BLOCK_ID);
      }
      if (pid >= 0) a.seq_lens[s] = t + 1;
      a.slot_pid[s] = pid;
      a.slot_idx[s] = slot;
    }
    carry += scan[kAllocThreads - 1];
    __syncthreads();
  }
  if (tid == 0) *a.free_top = top0 - min(carry, top0);
}

__global__ void __launch_bounds__(256) append_scatter(AppendArgs a) {
  const int s = blockIdx.x;
  const int layer = blockIdx.y;
  const int pid = a.slot_pid[s];
  if (pid < 0) return;
  const int slot = a.slot_idx[s];
  const int row_bytes = kHeadDim * a.elem_bytes;          // one token, one head
  const int row16 = row_bytes / 16;
  const size_t tile = (size_t)16 * row_bytes;
  const size_t blk = (size_t)a.num_layers * 16 * tile;    // 16 tiles (K, V x 8 heads) per layer
  uint8_t* dst_layer = a.pool + (size_t)pid * blk + (size_t)layer * 16 * tile;
  const size_t src_off = ((size_t)s * a.num_layers + layer) * 8 * row_bytes;
  for (int idx = threadIdx.x; idx < 16 * row16; idx += 256) {
    const int row = idx / row16;          // kv * 8 + head
    const int part = idx - row * row16;
    const int kv = row >> 3;
    const int g = row & 7;
    const uint8_t* src = (kv == 0 ? a.k_new : a.v_new) + src_off + (size_t)g * row_bytes + part * 16;
    uint8_t* dst = dst_layer + (size_t)row * tile + (size_t)slot * row_bytes + part * 16;
    *reinterpret_cast<u4_t*>(dst) = *reinterpret_cast<const u4_t*>(src);
  }
}

__global__ void __launch_bounds__(64) clear_words(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += 64) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// stream probe: grid-stride 16-byte loads, 8 in flight per lane.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) stream_read(const u4_t* __restrict__ src, size_t n16,
                                                  uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u4_t v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = acc;
}

__global__ void __launch_bounds__(256) stream_copy(const u4_t* __restrict__ src, size_t n16,
                                                  u4_t* __restrict__ dst) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_decode(const DecodeArgs& a, int batch, hipStream_t stream) {
  const uint64_t wgs = (uint64_t)batch * a.n_splits * a.n_layers * 8u;
  const size_t lds = decode_lds_bytes(a.split_blocks);
  if (lds > kMaxDecodeLds) return hipErrorInvalidValue;
  if (a.kv_format == KVS_KV_KIVI2)
    hipLaunchKernelGGL(paged_decode_kivi, dim3((uint32_t)wgs), dim3(64), lds, stream, a);
  else if (a.kv_format == KVS_KV_E4M3)
    hipLaunchKernelGGL(paged_decode_gqa<KvE4M3>, dim3((uint32_t)wgs), dim3(64), lds, stream, a);
  else
    hipLaunchKernelGGL(paged_decode_gqa<KvF16>, dim3((uint32_t)wgs), dim3(64), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int batch, hipStream_t stream) {
  const uint64_t wgs = (uint64_t)batch * a.n_layers * kQHeads;
  hipLaunchKernelGGL(combine_splits, dim3((uint32_t)wgs), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mass(const MassArgs& a, int batch, hipStream_t stream) {
  const dim3 grid((a.max_nb + 63) / 64, batch);
  hipLaunchKernelGGL(block_mass, grid, dim3(kMassThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs& a, int batch, hipStream_t stream) {
  const dim3 grid(a.max_chunks, batch);
  hipLaunchKernelGGL(seq_chunk_max, grid, dim3(kScoreThreads), 0, stream, a);
  hipLaunchKernelGGL(score_update, grid, dim3(kScoreThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_classify(const ScoreArgs& a, int batch, hipStream_t stream) {
  const dim3 grid(a.max_chunks, batch);
  hipLaunchKernelGGL(classify_records, grid, dim3(kScoreThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_evict(const EvictArgs& a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(evict_chunks, dim3(a.max_chunks, batch), dim3(kScoreThreads), 0, stream, a);
  hipLaunchKernelGGL(evict_final, dim3(batch), dim3(kScoreThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_meta_init(const MetaInitArgs& a, int batch, hipStream_t stream) {
  const dim3 grid(a.max_chunks, batch);
  hipLaunchKernelGGL(meta_init, grid, dim3(kScoreThreads), 0, stream, a);
  return hipGetLastError();
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

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(append_alloc, dim3(1), dim3(kAllocThreads), 0, stream, a, batch);
  hipLaunchKernelGGL(append_scatter, dim3(batch, a.num_layers), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_clear(uint32_t* p, int n, hipStream_t stream) {
  hipLaunchKernelGGL(clear_words, dim3(1), dim3(64), 0, stream, p, n);
  return hipGetLastError();
}

hipError_t launch_probe(const void* src, void* dst, size_t bytes, int mode, int grid,
                        hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (mode == 0)
    hipLaunchKernelGGL(stream_read, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u4_t*>(src), n16, static_cast<uint32_t*>(dst));
  else
    hipLaunchKernelGGL(stream_copy, dim3(grid), dim3(256), 0, stream,
                       static_cast<const u4_t*>(src), n16, static_cast<u4_t*>(dst));
  return hipGetLastError();
}

}  // namespace kvs
