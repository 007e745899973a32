// Tile-level helpers of the paged decode kernels (fp16 and FP8 E4M3 pools):
// the stored formats, the per-lane loads of one block's key and value tiles,
// the value stage in LDS and the MFMA operands built from them.  Included by
// the decode kernel sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvs_device.h"

namespace kvs {

// Stored K/V element formats.  A (layer, K|V, KV head) tile is 16 rows of 128
// elements; a block holds, per layer, 8 key tiles then 8 value tiles.  A step
// of a decode wave loads kPer blocks of kHeads adjacent KV heads.
struct KvF16 {
  static constexpr int kElemBytes = 2;
  static constexpr int kLoads = 4;   // 16-byte loads per lane per tile
  static constexpr int kPer = 1;     // blocks per step
  static constexpr int kHeads = 1;   // KV heads per wave
  static constexpr int kRing = 2;    // ring slots (32 VGPRs each)
  static constexpr int kWavesPerSimd = kDecodeWavesPerSimd;
};
// fp16 with two adjacent KV heads per wave: 8 KiB runs of keys and of values
// per step.  The decode takes it when the sequences fill their splits.
struct KvF16x2 {
  static constexpr int kElemBytes = 2;
  static constexpr int kLoads = 4;
  static constexpr int kPer = 1;
  static constexpr int kHeads = 2;
  static constexpr int kRing = 2;    // ring slots (64 VGPRs each)
  static constexpr int kWavesPerSimd = kDecodeWavesPerSimdF16x2;
};
struct KvE4M3 {                      // FP8 E4M3 codes, no scale
  static constexpr int kElemBytes = 1;
  static constexpr int kLoads = 2;
  static constexpr int kPer = 1;
  // Two adjacent KV heads per wave: a step reads one 4 KiB run of keys and one
  // of values, as the fp16 decode does, and fills all 16 MFMA columns.
  static constexpr int kHeads = kE4M3HeadsPerWave;
  static constexpr int kRing = 2;    // ring slots (32 VGPRs each); 3 measured no faster
  static constexpr int kWavesPerSimd = kDecodeWavesPerSimdE4M3;
};
// The paired decode over E4M3 codes: one KV head and one block per step, so
// that each (sequence, head) sees the arithmetic of the E4M3 decode above.
struct KvE4M3Pair {
  static constexpr int kElemBytes = 1;
  static constexpr int kLoads = 2;
  static constexpr int kPer = 1;
  static constexpr int kHeads = 1;
  static constexpr int kRing = 2;
  static constexpr int kWavesPerSimd = kDecodeWavesPerSimd;
};

template <class F>
struct BlockRegs {
  u4_t k[F::kLoads];
  u4_t v[F::kLoads];
};

// One ring slot: the tiles of one step, tile t = kHeads * p + h for block p of
// the step and head h of the wave.
template <class F>
struct StepRegs {
  BlockRegs<F> blk[F::kPer * F::kHeads];
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

// Value tile t of a step to the LDS stage, as stored ([16][128] fp16 values or
// E4M3 codes), at byte t * tile_bytes.
template <class F>
__device__ __forceinline__ void stage_values(const BlockRegs<F>& r, u4_t* vstage, int lane,
                                             int p) {
#pragma unroll
  for (int i = 0; i < F::kLoads; ++i) vstage[p * (tile_bytes<F>() / 16) + i * 64 + lane] = r.v[i];
}

// The PV operand rows of tile p: R[i] = 8 fp16 values, elements [8 c, 8 c + 8)
// of value row 4 j + i (E4M3 codes are converted here, after the LDS read).
template <class F>
__device__ __forceinline__ void value_rows(const u4_t* vstage, int p, int j, int c, u4_t (&R)[4]) {
  if constexpr (F::kElemBytes == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) R[i] = vstage[p * 256 + (4 * j + i) * 16 + c];
  } else {
    const uint8_t* tile = reinterpret_cast<const uint8_t*>(vstage) + 2048 * p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u2_t w = *reinterpret_cast<const u2_t*>(tile + (4 * j + i) * 128 + 8 * c);
      const u2_t lo = e4m3x4_to_f16(w[0]);
      const u2_t hi = e4m3x4_to_f16(w[1]);
      R[i] = u4_t{lo[0], lo[1], hi[0], hi[1]};
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

}  // namespace kvs
