// Internal interface between the C-ABI host code and the device kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvs.h"

namespace kvs {

constexpr int kMassThreads = 1024;   // 16 waves share one 32-block column group
constexpr int kMassCols = 32;
constexpr int kScoreThreads = 256;   // records per scoring work-group
// Dynamic LDS a decode work-group may request (gfx950 allows up to 160 KiB
// per work-group).
constexpr size_t kMaxDecodeLds = 98304;
constexpr size_t kLdsPerCu = 163840;     // gfx950: 160 KiB of LDS per compute unit
constexpr int kDecodeWavesPerSimd = 3;   // decode kernel launch bound (VGPR budget)
constexpr int kDecodeWavesPerSimdE4M3 = 2;   // E4M3 decode: two KV heads per step need more VGPRs
constexpr int kDecodeWavesPerSimdF16x2 = 2;  // fp16 decode with two KV heads per wave
constexpr int kE4M3HeadsPerWave = 2;     // KV heads one E4M3 decode wave serves

// LDS of one decode work-group (one wave serving `kv_heads` KV heads): the
// split's block ids (4 B each), per-block mass partials of the 8 query heads
// of each KV head (4 B each per head) and the value stage (`stage_bytes`: one
// 4 KiB fp16 tile, two 2 KiB E4M3 tiles, or two fp16 tiles).  With two KV
// heads the id list is rounded up to 4 entries and each head's partial row to
// decode_pi_stride() floats, so rows are 16-byte aligned and fall on
// different LDS banks.
constexpr int32_t decode_pi_stride(int32_t split_blocks, int kv_heads) {
  return kv_heads == 1 ? split_blocks : ((split_blocks + 3) & ~3) + 4;
}
constexpr size_t decode_lds_bytes(int32_t split_blocks, int kv_heads = 1,
                                  size_t stage_bytes = 4096) {
  const int32_t ids = kv_heads == 1 ? split_blocks : (split_blocks + 3) & ~3;
  return (size_t)4 * (size_t)ids +
         (size_t)4 * 8 * (size_t)kv_heads * (size_t)decode_pi_stride(split_blocks, kv_heads) +
         stage_bytes;
}

// LDS of one paired decode work-group: block ids of both sequences, mass
// partials of 16 (sequence, head) columns and the 4 KiB value stage.
constexpr size_t decode_pair_lds_bytes(int32_t split_blocks) {
  return (size_t)72 * (size_t)split_blocks + 4096;
}
constexpr int32_t kMaxPairSplit = 512;   // paired splits: LDS and 4 work-groups per CU

// The KIVI window rule (Fitting a Million Tokens, Sec. 02: the newest ~128
// tokens stay fp16, quantisation works in whole 32-token key groups): tokens
// [0, quant_len) of an n-token sequence are quantised, quant_len being the
// largest multiple of 32 that leaves at least `residual` tokens in fp16 (0 when
// fewer than residual + 32 tokens).  The one implementation of the rule, used
// by kvs_kivi_quant_len on the host and by the boundary advance on the device.
__host__ __device__ constexpr int32_t kivi_quant_len(int32_t n, int32_t residual) {
  return n - residual < 32 ? 0 : (n - residual) / 32 * 32;
}
static_assert(kivi_quant_len(159, 128) == 0 && kivi_quant_len(160, 128) == 32 &&
              kivi_quant_len(191, 128) == 32 && kivi_quant_len(192, 128) == 64 &&
              kivi_quant_len(0, 128) == 0, "window rule");

// Device address of the library-owned scratch array used by
// kvs_decode_step_noalloc, for the current device (looked up once per device);
// nullptr with *err set when the lookup fails.
void* noalloc_scratch(hipError_t* err);

struct DecodeArgs {
  const uint16_t* q;        // fp16 bits [B][num_layers][64][128]
  const uint8_t* pool;      // [P][num_layers][2][8][16][128] fp16 values or E4M3 codes
  const int32_t* table;     // [B][max_nb]
  const int32_t* seq_lens;  // [B]
  const int32_t* meta_off;  // [B + 1]
  int64_t pool_blocks;
  int64_t total_blocks;
  int32_t max_nb;
  int32_t num_layers;
  int32_t layer_begin;
  int32_t n_layers;         // layers in range
  int32_t split_blocks;
  int32_t n_splits;
  float scale_log2;         // softmax scale * log2(e)
  int32_t kv_format;        // KVS_KV_FP16, KVS_KV_E4M3 or KVS_KV_KIVI2
  const uint8_t* kivi;      // KVS_KV_KIVI2: quantised pool [kivi_blocks][num_layers][2][8][768]
  int64_t kivi_blocks;
  const int32_t* quant_lens;  // KVS_KV_KIVI2: [B] quantised tokens per sequence
  const int32_t* pair_role;   // nullable: pairs of sequences decoded by one wave (fp16)
  int32_t kv_heads;           // fp16 decode: KV heads per wave (1 or 2)
  float2* ml;               // [B][n_layers][64][n_splits]: (running max, sum), base 2
  float* opart;             // [B][n_layers][64][n_splits][128]
  float* pi;                // [n_layers][64][total_blocks]
  uint32_t* status;
};

struct CombineArgs {
  const int32_t* seq_lens;
  const int32_t* meta_off;
  const float2* ml;
  const float* opart;
  float* wsplit;            // [B][n_layers][64][n_splits]
  uint16_t* out;            // fp16 bits [B][num_layers][64][128]
  int64_t total_blocks;
  int32_t max_nb;
  int32_t num_layers;
  int32_t layer_begin;
  int32_t n_layers;
  int32_t split_blocks;
  int32_t n_splits;
  uint32_t* status;
};

struct MassArgs {
  const int32_t* seq_lens;
  const int32_t* meta_off;
  const float* pi;
  const float* wsplit;
  float* mass;
  int64_t total_blocks;
  int32_t max_nb;
  int32_t n_layers;
  int32_t split_blocks;
  int32_t n_splits;
  int32_t accumulate;
  uint32_t* status;
};

struct ScorePolicy {
  double alpha, w_recency, w_ema, w_anchor, t_low, t_high;
};

struct ScoreArgs {
  kvs_block_meta* meta;
  const float* mass;
  const int32_t* meta_off;
  const int32_t* seq_lens;  // nullable: every record of the capacity is live
  float* chunk_max;         // [B][max_chunks]
  uint8_t* tiers_out;
  int64_t total_blocks;
  uint64_t step;
  ScorePolicy pol;
  int32_t max_nb;
  int32_t max_chunks;
  int32_t classify;
  uint32_t* status;
};

struct EvictArgs {
  const kvs_block_meta* meta;
  const int32_t* meta_off;
  const int32_t* seq_lens;  // nullable
  const uint8_t* active;    // nullable
  double* part_key;         // [B][max_chunks]
  int32_t* part_idx;        // [B][max_chunks]
  int32_t* out_block;       // [B]
  double* out_key;          // [B]
  int64_t total_blocks;
  uint64_t now;
  double neg_log_keep;      // -ln(1 - alpha)
  int32_t max_nb;
  int32_t max_chunks;
  int32_t exclude_pinned;
  uint32_t* status;
};

struct AppendArgs {
  const uint8_t* k_new;     // [B][num_layers][8][128] elements (pool's format)
  const uint8_t* v_new;
  uint8_t* pool;
  int64_t pool_blocks;
  int32_t* table;           // [B][max_nb]
  int32_t max_nb;
  int32_t* seq_lens;        // in / out
  const int32_t* free_stack;
  int32_t free_capacity;    // entries in free_stack
  int32_t* free_top;        // in / out
  kvs_block_meta* meta;
  const int32_t* meta_off;
  const uint64_t* seq_ids;
  int32_t anchor_blocks;
  int64_t total_blocks;
  int32_t num_layers;
  int32_t elem_bytes;       // 2: fp16, 1: E4M3
  int32_t* slot_pid;        // [B] workspace: block written, -1 none
  int32_t* slot_idx;        // [B] workspace: slot written
  uint32_t* status;
};

struct MetaInitArgs {
  kvs_block_meta* meta;
  const int32_t* meta_off;
  const int32_t* seq_lens;  // always null: initialise the whole capacity
  const uint64_t* seq_ids;
  int64_t total_blocks;
  int32_t max_nb;
  int32_t max_chunks;
  int32_t anchor_blocks;
  uint32_t* status;         // may be a scratch word; init reports nothing
};

constexpr int kKiviTileBytes = 768;     // (layer, K|V, KV head) tile of a quantised block

struct KiviQuantArgs {
  const uint8_t* pool;      // fp16 [P][num_layers][2][8][16][128]
  uint8_t* kivi;            // [kivi_blocks][num_layers][2][8][768]
  const int32_t* pairs;     // [n_pairs][4]
  int64_t pool_blocks;
  int64_t kivi_blocks;
  int32_t num_layers;
  int32_t n_pairs;          // grid size (upper bound on pairs)
  const int32_t* count;     // nullable: pairs at or past *count are skipped
  uint32_t* status;
};

// KIVI boundary advance after appends (kvs_kivi_advance).
struct KiviAdvanceArgs {
  int32_t* table;           // [B][max_nb] in / out
  int32_t max_nb;
  const int32_t* seq_lens;
  int32_t* quant_lens;      // in / out
  int32_t residual;         // fp16 residual window (tokens)
  int64_t pool_blocks;
  int64_t kivi_blocks;
  const int32_t* kivi_free;
  int32_t kivi_free_capacity;
  int32_t* kivi_free_top;   // in / out
  int32_t* fp16_free;       // released fp16 ids are pushed here
  int32_t fp16_free_capacity;
  int32_t* fp16_free_top;   // in / out
  int32_t* jobs;            // [B][4] workspace: src even, src odd, dst even, dst odd
  int32_t* job_seq;         // [B] workspace: sequence of each job
  int32_t* count;           // workspace: number of jobs
  uint32_t* status;
};

hipError_t launch_decode(const DecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_decode_kivi(const DecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_kivi_quantize(const KiviQuantArgs& a, hipStream_t stream);
hipError_t launch_kivi_advance(const KiviAdvanceArgs& adv, const KiviQuantArgs& q, int batch,
                               hipStream_t stream);
hipError_t launch_decode_pair(const DecodeArgs& a, int batch, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int batch, hipStream_t stream);
hipError_t launch_mass(const MassArgs& a, int batch, hipStream_t stream);
// combine, then mass (mass only when total_blocks > 0): one fused launch for
// small problems, the two kernels otherwise
hipError_t launch_combine_mass(const CombineArgs& c, const MassArgs& m, int batch,
                               hipStream_t stream);
hipError_t launch_score(const ScoreArgs& a, int batch, hipStream_t stream);
hipError_t launch_classify(const ScoreArgs& a, int batch, hipStream_t stream);
hipError_t launch_meta_init(const MetaInitArgs& a, int batch, hipStream_t stream);
hipError_t launch_evict(const EvictArgs& a, int batch, hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t stream);
hipError_t launch_clear(uint32_t* p, int n, hipStream_t stream);
hipError_t launch_probe(const void* src, void* dst, size_t bytes, int mode, int grid,
                        hipStream_t stream);

}  // namespace kvs
