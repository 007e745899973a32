// Device-side helpers shared by the library's kernel sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
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
static_assert(decode_pair_lds_bytes(kMaxPairSplit) <= kMaxDecodeLds / 1.5,
              "paired splits keep 4 work-groups per CU");

// XCD-aware order of the decode grids.  Work-group w goes to XCD w % 8 (the
// dispatcher deals work-groups round-robin over the 8 XCDs, each with its own
// L2).  In the kernels' item order the (layer, KV head) index varies fastest,
// then the split, then the sequence, so without remapping the 8 KV heads of one
// layer -- whose tiles are adjacent in every block -- would be read through 8
// different XCDs.  This permutation deals the items to the XCDs in runs of
// kXcdRun consecutive items (two layers' 8 KV heads of one sequence and split),
// dispatched back to back on one XCD.  Grid positions past the last whole
// round of runs keep their order.  A bijection on [0, grid).  Measured on
// gfx950 against the plain order: +1 to +2 % at 128K tokens x 80 layers, +2 %
// at 1M tokens x 32 layers and on 32 sequences sharing a 2K prefix, +3 to +4 %
// on 8 sequences of 8K tokens x 4 layers.
constexpr uint32_t kXcds = 8;
constexpr uint32_t kXcdRun = 16;
__device__ __forceinline__ uint32_t xcd_item(uint32_t w, uint32_t grid) {
  constexpr uint32_t span = kXcds * kXcdRun;
  if (w >= grid / span * span) return w;
  return w / span * span + (w % kXcds) * kXcdRun + (w / kXcds) % kXcdRun;
}

// Softmax weights enter the PV products as fp16.  A split takes its weights
// relative to a reference 2^kProbShift below its running maximum (base 2), so
// they lie in (0, 2^15] instead of (0, 1]: fp16 then rounds a weight w (as a
// fraction of the split's maximum) with relative error 2^-11 down to
// w = 2^-29 and absolute error at most 2^-41 below that, where weights in
// (0, 1] would lose every w < 2^-25.  Over a 16,384-token split the weight
// lost to that floor is at most 16,384 x 2^-41 < 2^-27 of the maximum.  The
// split's sum, partial output and mass partials carry the same factor 2^15,
// and so does the reference it stores with them, so the split combine
// (weights 2^(m_k - M) / Lambda) cancels it exactly.
constexpr float kProbShift = 15.f;

__device__ __forceinline__ float xor_f(float v, int m) { return __shfl_xor(v, m, 64); }

// Maximum / sum of v over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (the 4 lanes j
// that hold one head in the MFMA output layout).  gfx950's permlane16 and
// permlane32 swaps hand each lane both values of its pair (l, l ^ 16), then
// (l, l ^ 32), in VALU registers -- {v[l], v[l ^ 16]} and {v[l], v[l ^ 32]} in
// some order, as an in-bounds lane probe on the GPU showed -- so each step is
// one swap and one max or add, with no LDS round trip and no lane-index
// arithmetic.  max and + are commutative, so the order within a pair does not
// change the result: it equals v[l] op v[l ^ 16], then op the l ^ 32 partner.
// Every lane of the wave must be active.
__device__ __forceinline__ float head_max4(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Value of lane l ^ 8: the other half of the lane's 16-lane row (a DPP row
// rotation by 8 within each row).
__device__ __forceinline__ float swap8(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ float head_sum4(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Softmax normaliser of each row (head) of a split: the sum of the row's
// block-mass partials in LDS, row r holding its cnt blocks at
// pi_lds[r * SB + b] (cnt_lo for rows 0..7, cnt_hi for rows 8..15), all taken
// relative to the split's final reference.  It is summed in fp64 in a fixed
// order: a running fp32 sum would take a dominant block's weight plus
// thousands of increments near its rounding unit and drift (a 17-nat peak over
// 16,384 tokens moved an fp32 sum by 3e-5).  The 64 / kRows lanes of a row
// share its blocks; every lane returns its row's sum.
// Eight LDS reads are issued per round and added in the order of the blocks,
// so the sum is the same as one read at a time without a wait per block.
template <int kRows>
__device__ __forceinline__ float split_norm(const float* pi_lds, int SB, int lane, int cnt_lo,
                                            int cnt_hi) {
  constexpr int kParts = 64 / kRows;
  const int r = lane % kRows;
  const int cnt = r < 8 ? cnt_lo : cnt_hi;
  const float* row = pi_lds + r * SB;
  double acc = 0.0;
  int b = lane / kRows;
  for (; b + 7 * kParts < cnt; b += 8 * kParts) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = row[b + u * kParts];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += (double)x[u];
  }
  for (; b < cnt; b += kParts) acc += (double)row[b];
#pragma unroll
  for (int m = kRows; m < 64; m <<= 1) acc += __shfl_xor(acc, m, 64);
  return (float)acc;
}

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

// K/V tiles are read exactly once per step.  Value loads are non-temporal:
// each instruction reads 1 KiB contiguous, and on gfx950 that measured ~10 %
// faster than plain loads.  Key loads stay plain: an instruction covers 16 rows
// x 64 bytes, half of each 128-byte line, and non-temporal loads of partial
// lines measured slower (the line is fetched again by the second half).
__device__ __forceinline__ u4_t stream_load(const u4_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ u4_t plain_load(const u4_t* p) { return *p; }

}  // namespace kvs
