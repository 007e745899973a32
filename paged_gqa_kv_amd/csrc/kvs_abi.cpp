// C-ABI host side: argument validation, workspace layout, launches.
// Every host-checkable error returns before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "kvs.h"
#include "kvs_internal.h"

static_assert(sizeof(kvs_block_meta) == 64, "record must be 64 bytes");
static_assert(offsetof(kvs_block_meta, key) == 0, "");
static_assert(offsetof(kvs_block_meta, score) == 16, "");
static_assert(offsetof(kvs_block_meta, t_touch) == 24, "");
static_assert(offsetof(kvs_block_meta, touch_count) == 32, "");
static_assert(offsetof(kvs_block_meta, tier) == 36, "");
static_assert(offsetof(kvs_block_meta, flags) == 37, "");
static_assert(offsetof(kvs_block_meta, reserved0) == 38, "");
static_assert(offsetof(kvs_block_meta, priority) == 40, "");
static_assert(offsetof(kvs_block_meta, reserved1) == 48, "");

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return KVS_OK;
}

constexpr size_t kHeader = 256;
constexpr size_t kAlign = 256;
// Split-K sizing.  Each decode wave keeps two blocks of its (layer, KV head)
// in flight: 16 KiB for fp16, 8 KiB for E4M3.  The chip needs about 16 MiB of
// reads in flight to stay at HBM bandwidth, and on gfx950 about 56 KiB per
// compute unit; within those, the longest splits measured fastest (fewer
// partial results, longer streams per wave, fewer resident streams).
// The E4M3 and KIVI decodes are limited by their instruction stream more than
// by bytes in flight, and measured fastest at shorter splits than fp16: E4M3
// at 512 blocks (one wave per SIMD at 1,024 leaves its conversions and
// softmax exposed: -10 %), KIVI at 128 (more, shorter waves even out the end
// of the grid: +3 % over 256 at 128K tokens; 64 slower again).
constexpr uint64_t kChipInflightBytes = 16ull << 20;
constexpr uint64_t kCuInflightBytes = 56ull << 10;
constexpr int32_t kMaxAutoSplit = 1024;
constexpr int32_t kMaxAutoSplitE4M3 = 512;
constexpr int32_t kMaxAutoSplitKivi = 128;
constexpr uint64_t kChipSimds = 1024;   // gfx950: 256 compute units x 4 SIMDs
// Automatic split of an E4M3 paired decode: at 512 blocks the paired LDS
// leaves 4 waves per CU, too few for that decode's instruction stream (14.0
// against 11.7 ms at 256 on the 32-sequence shared-prefix batch); 256 leaves 7.
constexpr int32_t kMaxAutoPairSplitE4M3 = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Layers are a grid dimension factor and a size factor of the workspace; the
// cap keeps every size computation far from 64-bit overflow.
constexpr int32_t kMaxLayers = 65535;

int check_shape(const kvs_shape* s) {
  if (!s) return fail(KVS_E_NULL, "shape is NULL");
  if (s->num_layers < 1 || s->num_layers > kMaxLayers || s->num_q_heads != 64 ||
      s->num_kv_heads != 8 || s->head_dim != 128 || s->block_tokens != 16)
    return fail(KVS_E_SHAPE,
                "unsupported shape {layers=%d, q_heads=%d, kv_heads=%d, head_dim=%d, block=%d}; "
                "kernels support 64/8/128/16 with 1 <= layers <= 65535",
                s->num_layers, s->num_q_heads, s->num_kv_heads, s->head_dim, s->block_tokens);
  return KVS_OK;
}

int check_policy(const kvs_policy* p) {
  if (!p) return fail(KVS_E_NULL, "policy is NULL");
  const double v[6] = {p->alpha, p->w_recency, p->w_ema, p->w_anchor, p->t_low, p->t_high};
  for (double x : v)
    if (!std::isfinite(x)) return fail(KVS_E_POLICY, "policy holds a non-finite value");
  if (!(p->alpha > 0.0 && p->alpha <= 1.0))
    return fail(KVS_E_POLICY, "alpha %.17g not in (0, 1]", p->alpha);
  if (p->w_recency < 0 || p->w_ema < 0 || p->w_anchor < 0)
    return fail(KVS_E_POLICY, "negative weight");
  if (!(p->t_low >= 0.0 && p->t_low <= p->t_high && p->t_high <= 1.0))
    return fail(KVS_E_POLICY, "cut points must satisfy 0 <= t_low <= t_high <= 1");
  return KVS_OK;
}

kvs::ScorePolicy to_score_policy(const kvs_policy* p) {
  return kvs::ScorePolicy{p->alpha, p->w_recency, p->w_ema, p->w_anchor, p->t_low, p->t_high};
}

// Batch is a grid dimension of the per-sequence kernels; block counts are
// scaled by 16 tokens in 32-bit device arithmetic.
constexpr int32_t kMaxBatch = 65535;
constexpr int32_t kMaxBlocksPerSeq = 1 << 26;

int check_counts(int32_t batch, int32_t max_blocks) {
  if (batch < 1 || batch > kMaxBatch) return fail(KVS_E_RANGE, "batch %d not in [1, %d]", batch, kMaxBatch);
  if (max_blocks < 1 || max_blocks > kMaxBlocksPerSeq)
    return fail(KVS_E_RANGE, "max_blocks_per_seq %d not in [1, %d]", max_blocks, kMaxBlocksPerSeq);
  return KVS_OK;
}

// The largest power-of-two split in [16, the format's cap] whose launch keeps
// enough bytes in flight on the whole chip (wave count) and per compute unit
// (waves that fit the LDS a split needs, at most the kernel's waves per SIMD).
// Reads one decode wave keeps in flight: two fp16 blocks (K and V tiles of its
// KV head) or two E4M3 blocks of its two KV heads.  For KIVI the figure is a sizing
// constant of two 32-token pairs (4 tiles of 768 bytes each): the kernel has
// one pair's loads in flight while it works on the previous pair from LDS.
uint64_t wave_inflight_bytes(int32_t kv_format) {
  switch (kv_format) {
    case KVS_KV_FP16: return 2ull * 2ull * 4096ull;
    case KVS_KV_E4M3: return 2ull * 2ull * 2ull * 2048ull;
    default: return 2ull * 4ull * (uint64_t)kvs::kKiviTileBytes;
  }
}

// KV heads per wave of the fp16 decode for these sizes.  Two adjacent heads
// per wave read 8 KiB runs per step (+3.2 % at 128K x 80 layers, +1.7 % at
// 1M x 32, +1 % on 8 x 8K x 4), but their LDS leaves 2-3 waves per CU, and
// when the sequences fill their splits only in part (the 32-sequence batch of
// mixed lengths: -3 % at its best split) one head per wave is faster.  So two
// heads when the records cover at least 3/4 of the splits' blocks.
int32_t fp16_heads_per_wave(int32_t batch, int64_t total_blocks, int32_t n_splits,
                            int32_t split_blocks) {
  const int64_t cover = (int64_t)batch * (int64_t)n_splits * (int64_t)split_blocks;
  return 4 * total_blocks >= 3 * cover ? 2 : 1;
}

// KV heads one decode wave serves, as the split choice sizes it (the fp16
// decode is sized for one head).
uint32_t heads_per_wave(int32_t kv_format) {
  return kv_format == KVS_KV_E4M3 ? (uint32_t)kvs::kE4M3HeadsPerWave : 1u;
}

uint64_t waves_per_simd(int32_t kv_format) {
  return kv_format == KVS_KV_E4M3 ? kvs::kDecodeWavesPerSimdE4M3 : kvs::kDecodeWavesPerSimd;
}

// Waves the grid must provide (1,024 SIMDs on gfx950).  The E4M3 decode needs
// one per SIMD: each wave's conversions and softmax must have loads of other
// waves to hide behind (8 sequences x 8K x 4 layers: 6.1 TB/s at split 64 with
// 1,024 waves, 5.8 TB/s at split 32 with 2,048, 5.4 TB/s at split 16).
uint64_t min_grid_waves(int32_t kv_format) {
  return kv_format == KVS_KV_E4M3 ? kChipSimds : 0u;
}

int32_t max_auto_split(int32_t kv_format) {
  switch (kv_format) {
    case KVS_KV_FP16: return kMaxAutoSplit;
    case KVS_KV_E4M3: return kMaxAutoSplitE4M3;
    default: return kMaxAutoSplitKivi;
  }
}

bool format_valid(int32_t f) { return f == KVS_KV_FP16 || f == KVS_KV_E4M3 || f == KVS_KV_KIVI2; }

int32_t choose_split(int32_t batch, int32_t max_nb, int32_t n_layers, int32_t kv_format) {
  const uint32_t heads = heads_per_wave(kv_format);
  const uint64_t streams = (uint64_t)batch * (uint64_t)n_layers * (8u / heads);
  const uint64_t wave_inflight = wave_inflight_bytes(kv_format);
  const uint64_t cu_waves = 4u * waves_per_simd(kv_format);
  for (int32_t cand = max_auto_split(kv_format); cand >= 16; cand >>= 1) {
    const uint64_t waves = streams * (uint64_t)((max_nb + cand - 1) / cand);
    uint64_t per_cu = kvs::kLdsPerCu / kvs::decode_lds_bytes(cand, (int)heads);
    if (per_cu > cu_waves) per_cu = cu_waves;
    if (waves * wave_inflight >= kChipInflightBytes && per_cu * wave_inflight >= kCuInflightBytes &&
        waves >= min_grid_waves(kv_format))
      return cand;
  }
  return 16;
}

// Upper bound keeps the decode work-group's LDS (36 B per block + 4 KiB, 68 B
// per block for the E4M3 decode's two KV heads) within the 96 KiB it may request.
bool split_valid(int32_t sb) { return sb >= 4 && sb <= 1024; }

struct DecodeLayout {
  size_t ml, wsplit, opart, pi, total;
  int32_t split_blocks, n_splits;
};

// Returns false on invalid sizes (no message).
bool decode_layout(const kvs_shape* shape, int32_t kv_format, int32_t batch, int32_t max_nb,
                   int64_t total_blocks, int32_t lb, int32_t le, int32_t split_blocks,
                   DecodeLayout* L) {
  if (!shape || !format_valid(kv_format) || batch < 1 || batch > kMaxBatch || max_nb < 1 ||
      max_nb > kMaxBlocksPerSeq || total_blocks < 0 || total_blocks > INT32_MAX || lb < 0 ||
      le <= lb || le > shape->num_layers || shape->num_layers > kMaxLayers)
    return false;
  const int32_t nl = le - lb;
  const int32_t sb =
      split_blocks == 0 ? choose_split(batch, max_nb, nl, kv_format) : split_blocks;
  if (!split_valid(sb)) return false;
  if (kv_format == KVS_KV_KIVI2 && (sb & 1)) return false;
  // batch < 2^16, layers < 2^16, splits < 2^24 and total_blocks < 2^31 keep
  // every term below 2^63: stats < 2^62 and stats * 512 would not be, so the
  // partial-output term is checked before it is formed.
  const uint64_t nsplit = (uint64_t)(max_nb + sb - 1) / sb;
  const uint64_t stats = (uint64_t)batch * nl * 64u * nsplit;
  if (stats > (1ull << 50)) return false;
  size_t off = kHeader;
  L->ml = off;
  off = align_up(off + stats * 8u);
  L->wsplit = off;
  off = align_up(off + stats * 4u);
  L->opart = off;
  off = align_up(off + stats * 128u * 4u);
  L->pi = off;
  off = align_up(off + (uint64_t)nl * 64u * (uint64_t)total_blocks * 4u);
  L->total = off;
  L->split_blocks = sb;
  L->n_splits = (int32_t)nsplit;
  return true;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KVS_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char* kvs_status_string(int code) {
  switch (code) {
    case KVS_OK: return "ok";
    case KVS_E_NULL: return "null pointer";
    case KVS_E_SHAPE: return "unsupported shape";
    case KVS_E_RANGE: return "argument out of range";
    case KVS_E_ALIGN: return "misaligned pointer";
    case KVS_E_WORKSPACE: return "workspace too small";
    case KVS_E_POLICY: return "invalid policy";
    case KVS_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* kvs_last_error(void) { return g_err; }

size_t kvs_bytes_per_token(const kvs_shape* s) {
  if (!s || s->num_layers < 1 || s->num_kv_heads < 1 || s->head_dim < 1) return 0;
  return (size_t)2 * (size_t)s->num_layers * (size_t)s->num_kv_heads * (size_t)s->head_dim * 2u;
}

size_t kvs_block_bytes(const kvs_shape* s) {
  if (!s || s->block_tokens < 1) return 0;
  return (size_t)s->block_tokens * kvs_bytes_per_token(s);
}

size_t kvs_meta_layout(size_t* offsets, int n) {
  if (offsets && n >= 9) {
    offsets[0] = offsetof(kvs_block_meta, key);
    offsets[1] = offsetof(kvs_block_meta, score);
    offsets[2] = offsetof(kvs_block_meta, t_touch);
    offsets[3] = offsetof(kvs_block_meta, touch_count);
    offsets[4] = offsetof(kvs_block_meta, tier);
    offsets[5] = offsetof(kvs_block_meta, flags);
    offsets[6] = offsetof(kvs_block_meta, reserved0);
    offsets[7] = offsetof(kvs_block_meta, priority);
    offsets[8] = offsetof(kvs_block_meta, reserved1);
  }
  return sizeof(kvs_block_meta);
}

int32_t kvs_decode_split_blocks(const kvs_shape* shape, int32_t kv_format, int32_t batch,
                                int32_t max_blocks_per_seq, int32_t layer_begin, int32_t layer_end,
                                int32_t split_blocks) {
  DecodeLayout L;
  if (!decode_layout(shape, kv_format, batch, max_blocks_per_seq, 0, layer_begin, layer_end,
                     split_blocks, &L))
    return 0;
  return L.split_blocks;
}

size_t kvs_decode_workspace_bytes(const kvs_shape* shape, int32_t kv_format, int32_t batch,
                                  int32_t max_blocks_per_seq, int64_t total_blocks,
                                  int32_t layer_begin, int32_t layer_end, int32_t split_blocks) {
  DecodeLayout L;
  if (!decode_layout(shape, kv_format, batch, max_blocks_per_seq, total_blocks, layer_begin,
                     layer_end, split_blocks, &L))
    return 0;
  return L.total;
}

size_t kvs_score_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq) {
  if (batch < 1 || max_blocks_per_seq < 1) return 0;
  const uint64_t chunks = (uint64_t)(max_blocks_per_seq + kvs::kScoreThreads - 1) / kvs::kScoreThreads;
  return align_up(kHeader + (uint64_t)batch * chunks * 4u);
}

int kvs_set_decode_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(KVS_E_NULL, "both events or neither must be given");
  g_ev_before = static_cast<hipEvent_t>(before);
  g_ev_after = static_cast<hipEvent_t>(after);
  return ok();
}

int kvs_stream_probe(const void* src, void* dst, size_t bytes, int mode, int32_t grid,
                     void* stream) {
  if (!src || !dst) return fail(KVS_E_NULL, "src and dst must be non-NULL");
  if (bytes == 0 || bytes % 16) return fail(KVS_E_RANGE, "bytes must be a non-zero multiple of 16");
  if (mode != 0 && mode != 1) return fail(KVS_E_RANGE, "mode must be 0 (read) or 1 (copy)");
  if (grid < 0 || grid > (1 << 20)) return fail(KVS_E_RANGE, "grid out of range");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(KVS_E_ALIGN, "src/dst must be 16-byte aligned");
  const int g = grid == 0 ? 256 * 8 : grid;
  hipError_t e = kvs::launch_probe(src, dst, bytes, mode, g, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "stream probe launch");
  return ok();
}

int kvs_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace) return fail(KVS_E_NULL, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(KVS_E_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < kHeader)
    return fail(KVS_E_WORKSPACE, "workspace of %zu bytes is smaller than its %zu-byte header",
                workspace_bytes, kHeader);
  hipError_t e = kvs::launch_clear(static_cast<uint32_t*>(workspace), (int)(kHeader / 4),
                                   static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "clear_words launch");
  return ok();
}

int kvs_device_status(void* workspace, void* stream, uint32_t* bits) {
  if (!workspace || !bits) return fail(KVS_E_NULL, "workspace and bits must be non-NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint32_t host = 0;
  hipError_t e = hipMemcpyAsync(&host, workspace, sizeof(host), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "reading the status word");
  e = kvs::launch_clear(static_cast<uint32_t*>(workspace), 1, st);
  if (e != hipSuccess) return hip_fail(e, "clearing the status word");
  *bits = host;
  return ok();
}

}  // extern "C"

namespace {

int decode_step(int32_t kv_format, const kvs_shape* shape, const void* q, const void* kv_pool,
                int64_t pool_blocks, const void* kivi_pool, int64_t kivi_blocks,
                const int32_t* block_table, int32_t max_blocks_per_seq,
                const int32_t* seq_lens, const int32_t* quant_lens, const int32_t* pair_role,
                const int32_t* meta_offsets, int32_t batch,
                int64_t total_blocks, int32_t layer_begin, int32_t layer_end, float scale,
                void* out, float* block_mass, int accumulate, int32_t split_blocks,
                void* workspace, size_t workspace_bytes, void* stream,
                uint32_t* status_word = nullptr) {
  // status_word != NULL: the library's own scratch (kvs_decode_step_noalloc)
  // stands in for the workspace, and the status bits go to status_word.
  const bool library_scratch = status_word != nullptr;
  if (library_scratch) workspace_bytes = KVS_NOALLOC_SCRATCH_BYTES;
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!q || !kv_pool || !block_table || !seq_lens || !meta_offsets || !out || !block_mass ||
      (!workspace && !library_scratch))
    return fail(KVS_E_NULL, "a required pointer is NULL");
  rc = check_counts(batch, max_blocks_per_seq);
  if (rc) return rc;
  if (pool_blocks < 1) return fail(KVS_E_RANGE, "pool_blocks %lld < 1", (long long)pool_blocks);
  if (pool_blocks > INT32_MAX) return fail(KVS_E_RANGE, "pool_blocks exceeds int32 block ids");
  if (total_blocks < 0 || total_blocks > INT32_MAX)
    return fail(KVS_E_RANGE, "total_blocks %lld out of range", (long long)total_blocks);
  if (layer_begin < 0 || layer_end <= layer_begin || layer_end > shape->num_layers)
    return fail(KVS_E_RANGE, "layer range [%d, %d) not inside [0, %d)", layer_begin, layer_end,
                shape->num_layers);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(KVS_E_RANGE, "scale must be finite and > 0");
  if (accumulate != 0 && accumulate != 1) return fail(KVS_E_RANGE, "accumulate must be 0 or 1");
  if (split_blocks != 0 && !split_valid(split_blocks))
    return fail(KVS_E_RANGE, "split_blocks %d not in [4, 1024]", split_blocks);
  const bool kivi = kv_format == KVS_KV_KIVI2;
  if (kivi) {
    if (!kivi_pool || !quant_lens) return fail(KVS_E_NULL, "kivi_pool and quant_lens are required");
    if (kivi_blocks < 1 || kivi_blocks > INT32_MAX)
      return fail(KVS_E_RANGE, "kivi_blocks %lld out of range", (long long)kivi_blocks);
    if (split_blocks & 1) return fail(KVS_E_RANGE, "split_blocks must be even for KIVI pairs");
    if (!aligned(kivi_pool, 16) || !aligned(quant_lens, 4))
      return fail(KVS_E_ALIGN, "kivi_pool must be 16-byte and quant_lens 4-byte aligned");
  }
  if (!aligned(q, 16) || !aligned(kv_pool, 16) || !aligned(out, 16))
    return fail(KVS_E_ALIGN, "q, kv_pool and out must be 16-byte aligned");
  if (!aligned(block_mass, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
      !aligned(meta_offsets, 4))
    return fail(KVS_E_ALIGN, "int32 / fp32 arrays must be 4-byte aligned");
  if (!library_scratch && !aligned(workspace, kAlign))
    return fail(KVS_E_ALIGN, "workspace must be 256-byte aligned");
  if (pair_role) {
    if (kv_format != KVS_KV_FP16 && kv_format != KVS_KV_E4M3)
      return fail(KVS_E_RANGE, "paired decode runs over fp16 or E4M3 pools only");
    if (!aligned(pair_role, 4)) return fail(KVS_E_ALIGN, "pair_role must be 4-byte aligned");
    if (split_blocks > kvs::kMaxPairSplit)
      return fail(KVS_E_RANGE, "split_blocks %d above %d for a paired decode", split_blocks,
                  kvs::kMaxPairSplit);
    if (split_blocks == 0) {
      const int32_t cap = kv_format == KVS_KV_E4M3 ? kMaxAutoPairSplitE4M3 : kvs::kMaxPairSplit;
      split_blocks = choose_split(batch, max_blocks_per_seq, layer_end - layer_begin, kv_format);
      if (split_blocks > cap) split_blocks = cap;
    }
  }
  DecodeLayout L;
  if (!decode_layout(shape, kv_format, batch, max_blocks_per_seq, total_blocks, layer_begin,
                     layer_end, split_blocks, &L))
    return fail(KVS_E_RANGE, "inconsistent sizes");
  if (workspace_bytes < L.total) {
    if (library_scratch)
      return fail(KVS_E_WORKSPACE,
                  "this call needs %zu bytes of scratch, above the %zu bytes "
                  "kvs_decode_step_noalloc holds: split the layer range into several calls "
                  "(accumulate = 1)",
                  L.total, workspace_bytes);
    return fail(KVS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  }
  const int32_t nl = layer_end - layer_begin;
  const uint64_t wgs = (uint64_t)batch * (uint64_t)L.n_splits * (uint64_t)nl * 8u;
  if (wgs * 64u >= (1ull << 32))
    return fail(KVS_E_RANGE, "problem too large for one launch (%llu work-groups)",
                (unsigned long long)wgs);
  if ((uint64_t)batch * nl * 64u >= (1ull << 32))
    return fail(KVS_E_RANGE, "batch x layers too large for one launch");
  if (library_scratch) {   // every host check passed: the per-device address
    hipError_t e = hipSuccess;
    workspace = kvs::noalloc_scratch(&e);
    if (!workspace) return hip_fail(e, "looking up the library's scratch array");
  }

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  // sticky status bits: the workspace header, or a caller-owned word
  uint32_t* status = status_word ? status_word : reinterpret_cast<uint32_t*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);

  kvs::DecodeArgs d{};
  d.q = static_cast<const uint16_t*>(q);
  d.pool = static_cast<const uint8_t*>(kv_pool);
  d.table = block_table;
  d.seq_lens = seq_lens;
  d.meta_off = meta_offsets;
  d.pool_blocks = pool_blocks;
  d.total_blocks = total_blocks;
  d.max_nb = max_blocks_per_seq;
  d.num_layers = shape->num_layers;
  d.layer_begin = layer_begin;
  d.n_layers = nl;
  d.split_blocks = L.split_blocks;
  d.n_splits = L.n_splits;
  d.scale_log2 = (float)((double)scale * 1.4426950408889634);
  d.kv_format = kv_format;
  d.kivi = static_cast<const uint8_t*>(kivi_pool);
  d.kivi_blocks = kivi ? kivi_blocks : 0;
  d.quant_lens = kivi ? quant_lens : nullptr;
  d.pair_role = pair_role;
  d.kv_heads = kv_format == KVS_KV_E4M3   ? kvs::kE4M3HeadsPerWave
               : kv_format == KVS_KV_FP16 ? fp16_heads_per_wave(batch, total_blocks, L.n_splits,
                                                                L.split_blocks)
                                          : 1;
  d.ml = reinterpret_cast<float2*>(ws + L.ml);
  d.opart = reinterpret_cast<float*>(ws + L.opart);
  d.pi = reinterpret_cast<float*>(ws + L.pi);
  d.status = status;

  kvs::CombineArgs c{};
  c.seq_lens = seq_lens;
  c.meta_off = meta_offsets;
  c.ml = d.ml;
  c.opart = d.opart;
  c.wsplit = reinterpret_cast<float*>(ws + L.wsplit);
  c.out = static_cast<uint16_t*>(out);
  c.total_blocks = total_blocks;
  c.max_nb = max_blocks_per_seq;
  c.num_layers = shape->num_layers;
  c.layer_begin = layer_begin;
  c.n_layers = nl;
  c.split_blocks = L.split_blocks;
  c.n_splits = L.n_splits;
  c.status = status;

  kvs::MassArgs m{};
  m.seq_lens = seq_lens;
  m.meta_off = meta_offsets;
  m.pi = d.pi;
  m.wsplit = c.wsplit;
  m.mass = block_mass;
  m.total_blocks = total_blocks;
  m.max_nb = max_blocks_per_seq;
  m.n_layers = nl;
  m.split_blocks = L.split_blocks;
  m.n_splits = L.n_splits;
  m.accumulate = accumulate;
  m.status = status;

  hipError_t e = hipSuccess;
  if (g_ev_before) {
    e = hipEventRecord(g_ev_before, st);
    if (e != hipSuccess) return hip_fail(e, "recording the before-decode event");
  }
  e = kvs::launch_decode(d, batch, st);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  if (g_ev_after) {
    e = hipEventRecord(g_ev_after, st);
    if (e != hipSuccess) return hip_fail(e, "recording the after-decode event");
  }
  e = kvs::launch_combine_mass(c, m, batch, st);
  if (e != hipSuccess) return hip_fail(e, "combine / block_mass launch");
  return ok();
}

}  // namespace

extern "C" {

int kvs_decode_step(const kvs_shape* shape, const void* q, const void* kv_pool, int64_t pool_blocks,
                    const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                    const int32_t* meta_offsets, int32_t batch, int64_t total_blocks,
                    int32_t layer_begin, int32_t layer_end, float scale, void* out,
                    float* block_mass, int accumulate, int32_t split_blocks, void* workspace,
                    size_t workspace_bytes, void* stream) {
  return decode_step(KVS_KV_FP16, shape, q, kv_pool, pool_blocks, nullptr, 0, block_table,
                     max_blocks_per_seq, seq_lens, nullptr, nullptr, meta_offsets, batch,
                     total_blocks, layer_begin, layer_end, scale, out, block_mass, accumulate,
                     split_blocks, workspace, workspace_bytes, stream);
}

int kvs_decode_step_noalloc(const kvs_shape* shape, const void* q, const void* kv_pool,
                            int64_t pool_blocks, const int32_t* block_table,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            const int32_t* meta_offsets, int32_t batch, int64_t total_blocks,
                            int32_t layer_begin, int32_t layer_end, float scale, void* out,
                            float* block_mass, int accumulate, int32_t split_blocks,
                            uint32_t* status, void* stream) {
  if (!status) return fail(KVS_E_NULL, "status is NULL");
  if (!aligned(status, 4)) return fail(KVS_E_ALIGN, "status must be 4-byte aligned");
  return decode_step(KVS_KV_FP16, shape, q, kv_pool, pool_blocks, nullptr, 0, block_table,
                     max_blocks_per_seq, seq_lens, nullptr, nullptr, meta_offsets, batch,
                     total_blocks, layer_begin, layer_end, scale, out, block_mass, accumulate,
                     split_blocks, nullptr, 0, stream, status);
}

int kvs_decode_step_e4m3(const kvs_shape* shape, const void* q, const void* kv_pool,
                         int64_t pool_blocks, const int32_t* block_table,
                         int32_t max_blocks_per_seq, const int32_t* seq_lens,
                         const int32_t* meta_offsets, int32_t batch, int64_t total_blocks,
                         int32_t layer_begin, int32_t layer_end, float scale, void* out,
                         float* block_mass, int accumulate, int32_t split_blocks, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_step(KVS_KV_E4M3, shape, q, kv_pool, pool_blocks, nullptr, 0, block_table,
                     max_blocks_per_seq, seq_lens, nullptr, nullptr, meta_offsets, batch,
                     total_blocks, layer_begin, layer_end, scale, out, block_mass, accumulate,
                     split_blocks, workspace, workspace_bytes, stream);
}

int kvs_decode_step_paired(const kvs_shape* shape, const void* q, const void* kv_pool,
                           int64_t pool_blocks, const int32_t* block_table,
                           int32_t max_blocks_per_seq, const int32_t* seq_lens,
                           const int32_t* pair_role, const int32_t* meta_offsets, int32_t batch,
                           int64_t total_blocks, int32_t layer_begin, int32_t layer_end,
                           float scale, void* out, float* block_mass, int accumulate,
                           int32_t split_blocks, void* workspace, size_t workspace_bytes,
                           void* stream) {
  if (!pair_role) return fail(KVS_E_NULL, "pair_role is NULL");
  return decode_step(KVS_KV_FP16, shape, q, kv_pool, pool_blocks, nullptr, 0, block_table,
                     max_blocks_per_seq, seq_lens, nullptr, pair_role, meta_offsets, batch,
                     total_blocks, layer_begin, layer_end, scale, out, block_mass, accumulate,
                     split_blocks, workspace, workspace_bytes, stream);
}

int kvs_decode_step_e4m3_paired(const kvs_shape* shape, const void* q, const void* kv_pool,
                                int64_t pool_blocks, const int32_t* block_table,
                                int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                const int32_t* pair_role, const int32_t* meta_offsets,
                                int32_t batch, int64_t total_blocks, int32_t layer_begin,
                                int32_t layer_end, float scale, void* out, float* block_mass,
                                int accumulate, int32_t split_blocks, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!pair_role) return fail(KVS_E_NULL, "pair_role is NULL");
  return decode_step(KVS_KV_E4M3, shape, q, kv_pool, pool_blocks, nullptr, 0, block_table,
                     max_blocks_per_seq, seq_lens, nullptr, pair_role, meta_offsets, batch,
                     total_blocks, layer_begin, layer_end, scale, out, block_mass, accumulate,
                     split_blocks, workspace, workspace_bytes, stream);
}

int kvs_decode_step_kivi(const kvs_shape* shape, const void* q, const void* kv_pool,
                         int64_t pool_blocks, const void* kivi_pool, int64_t kivi_blocks,
                         const int32_t* block_table, int32_t max_blocks_per_seq,
                         const int32_t* seq_lens, const int32_t* quant_lens,
                         const int32_t* meta_offsets, int32_t batch, int64_t total_blocks,
                         int32_t layer_begin, int32_t layer_end, float scale, void* out,
                         float* block_mass, int accumulate, int32_t split_blocks, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_step(KVS_KV_KIVI2, shape, q, kv_pool, pool_blocks, kivi_pool, kivi_blocks,
                     block_table, max_blocks_per_seq, seq_lens, quant_lens, nullptr, meta_offsets,
                     batch, total_blocks, layer_begin, layer_end, scale, out, block_mass,
                     accumulate, split_blocks, workspace, workspace_bytes, stream);
}

int32_t kvs_kivi_quant_len(int32_t seq_len, int32_t residual_tokens) {
  if (seq_len < 0 || residual_tokens < 0) return -1;
  return kvs::kivi_quant_len(seq_len, residual_tokens);
}

size_t kvs_kivi_advance_workspace_bytes(int32_t batch) {
  if (batch < 1) return 0;
  return align_up(kHeader + 16u + (size_t)batch * 20u);
}

int kvs_kivi_advance(const kvs_shape* shape, const void* kv_pool, int64_t pool_blocks,
                     void* kivi_pool, int64_t kivi_blocks, int32_t* block_table,
                     int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t* quant_lens,
                     int32_t batch, int32_t residual_tokens, const int32_t* kivi_free,
                     int32_t kivi_free_capacity, int32_t* kivi_free_top, int32_t* fp16_free,
                     int32_t fp16_free_capacity, int32_t* fp16_free_top, void* workspace,
                     size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!kv_pool || !kivi_pool || !block_table || !seq_lens || !quant_lens || !kivi_free ||
      !kivi_free_top || !fp16_free || !fp16_free_top || !workspace)
    return fail(KVS_E_NULL, "a required pointer is NULL");
  rc = check_counts(batch, max_blocks_per_seq);
  if (rc) return rc;
  if (pool_blocks < 1 || pool_blocks > INT32_MAX || kivi_blocks < 1 || kivi_blocks > INT32_MAX)
    return fail(KVS_E_RANGE, "pool sizes out of range");
  if (residual_tokens < 0 || residual_tokens > 16 * max_blocks_per_seq)
    return fail(KVS_E_RANGE, "residual_tokens %d out of range", residual_tokens);
  if (kivi_free_capacity < 0 || fp16_free_capacity < 0)
    return fail(KVS_E_RANGE, "free-stack capacities must be >= 0");
  if ((uint64_t)shape->num_layers > 65535) return fail(KVS_E_RANGE, "num_layers > 65535");
  if (!aligned(kv_pool, 16) || !aligned(kivi_pool, 16))
    return fail(KVS_E_ALIGN, "pools must be 16-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(KVS_E_ALIGN, "workspace must be 256-byte aligned");
  const size_t need = kvs_kivi_advance_workspace_bytes(batch);
  if (workspace_bytes < need)
    return fail(KVS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  kvs::KiviAdvanceArgs a{};
  a.table = block_table;
  a.max_nb = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.quant_lens = quant_lens;
  a.residual = residual_tokens;
  a.pool_blocks = pool_blocks;
  a.kivi_blocks = kivi_blocks;
  a.kivi_free = kivi_free;
  a.kivi_free_capacity = kivi_free_capacity;
  a.kivi_free_top = kivi_free_top;
  a.fp16_free = fp16_free;
  a.fp16_free_capacity = fp16_free_capacity;
  a.fp16_free_top = fp16_free_top;
  a.count = reinterpret_cast<int32_t*>(ws + kHeader);
  a.jobs = reinterpret_cast<int32_t*>(ws + kHeader + 16u);
  a.job_seq = reinterpret_cast<int32_t*>(ws + kHeader + 16u + (size_t)batch * 16u);
  a.status = reinterpret_cast<uint32_t*>(ws);
  kvs::KiviQuantArgs q{};
  q.pool = static_cast<const uint8_t*>(kv_pool);
  q.kivi = static_cast<uint8_t*>(kivi_pool);
  q.pairs = a.jobs;
  q.pool_blocks = pool_blocks;
  q.kivi_blocks = kivi_blocks;
  q.num_layers = shape->num_layers;
  q.n_pairs = batch;
  q.count = a.count;
  q.status = a.status;
  hipError_t e = kvs::launch_kivi_advance(a, q, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kivi_advance launch");
  return ok();
}

size_t kvs_kivi_block_bytes(const kvs_shape* shape) {
  if (!shape) return 0;
  return (size_t)shape->num_layers * 2u * 8u * (size_t)kvs::kKiviTileBytes;
}

int kvs_kivi_quantize(const kvs_shape* shape, const void* kv_pool, int64_t pool_blocks,
                      void* kivi_pool, int64_t kivi_blocks, const int32_t* pairs, int32_t n_pairs,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!kv_pool || !kivi_pool || !pairs || !workspace)
    return fail(KVS_E_NULL, "kv_pool, kivi_pool, pairs and workspace must be non-NULL");
  if (n_pairs < 0) return fail(KVS_E_RANGE, "n_pairs %d < 0", n_pairs);
  if (pool_blocks < 1 || pool_blocks > INT32_MAX || kivi_blocks < 1 || kivi_blocks > INT32_MAX)
    return fail(KVS_E_RANGE, "pool sizes out of range");
  if (!aligned(kv_pool, 16) || !aligned(kivi_pool, 16) || !aligned(pairs, 4))
    return fail(KVS_E_ALIGN, "pools must be 16-byte aligned, pairs 4-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(KVS_E_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < kHeader)
    return fail(KVS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, kHeader);
  if (n_pairs == 0) return ok();
  kvs::KiviQuantArgs a{};
  a.pool = static_cast<const uint8_t*>(kv_pool);
  a.kivi = static_cast<uint8_t*>(kivi_pool);
  a.pairs = pairs;
  a.pool_blocks = pool_blocks;
  a.kivi_blocks = kivi_blocks;
  a.num_layers = shape->num_layers;
  a.n_pairs = n_pairs;
  a.status = static_cast<uint32_t*>(workspace);
  hipError_t e = kvs::launch_kivi_quantize(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kivi_quantize launch");
  return ok();
}

int kvs_meta_init(kvs_block_meta* meta, const int32_t* meta_offsets, const uint64_t* seq_ids,
                  int32_t batch, int32_t max_blocks_per_seq, int64_t total_blocks,
                  int32_t anchor_blocks, void* stream) {
  if (!meta || !meta_offsets || !seq_ids) return fail(KVS_E_NULL, "a required pointer is NULL");
  int rc = check_counts(batch, max_blocks_per_seq);
  if (rc) return rc;
  if (total_blocks < 0 || total_blocks > INT32_MAX || anchor_blocks < 0)
    return fail(KVS_E_RANGE, "total_blocks or anchor_blocks out of range");
  if (!aligned(meta, 16) || !aligned(seq_ids, 8)) return fail(KVS_E_ALIGN, "meta or seq_ids misaligned");
  kvs::MetaInitArgs a{};
  a.meta = meta;
  a.meta_off = meta_offsets;
  a.seq_lens = nullptr;
  a.seq_ids = seq_ids;
  a.total_blocks = total_blocks;
  a.max_nb = max_blocks_per_seq;
  a.max_chunks = (max_blocks_per_seq + kvs::kScoreThreads - 1) / kvs::kScoreThreads;
  a.anchor_blocks = anchor_blocks;
  a.status = nullptr;
  hipError_t e = kvs::launch_meta_init(a, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "meta_init launch");
  return ok();
}

int kvs_score_update(kvs_block_meta* meta, const float* block_mass, const int32_t* meta_offsets,
                     const int32_t* seq_lens, int32_t batch, int32_t max_blocks_per_seq,
                     int64_t total_blocks, uint64_t step, const kvs_policy* policy, int classify,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!meta || !block_mass || !meta_offsets || !workspace)
    return fail(KVS_E_NULL, "a required pointer is NULL");
  int rc = check_policy(policy);
  if (rc) return rc;
  rc = check_counts(batch, max_blocks_per_seq);
  if (rc) return rc;
  if (total_blocks < 0 || total_blocks > INT32_MAX)
    return fail(KVS_E_RANGE, "total_blocks out of range");
  if (classify != 0 && classify != 1) return fail(KVS_E_RANGE, "classify must be 0 or 1");
  if (step == KVS_NEVER_TOUCHED) return fail(KVS_E_RANGE, "step UINT64_MAX is reserved");
  if (!aligned(meta, 16)) return fail(KVS_E_ALIGN, "meta must be 16-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(KVS_E_ALIGN, "workspace must be 256-byte aligned");
  const size_t need = kvs_score_workspace_bytes(batch, max_blocks_per_seq);
  if (workspace_bytes < need)
    return fail(KVS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  kvs::ScoreArgs a{};
  a.meta = meta;
  a.mass = block_mass;
  a.meta_off = meta_offsets;
  a.seq_lens = seq_lens;
  a.chunk_max = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kHeader);
  a.tiers_out = nullptr;
  a.total_blocks = total_blocks;
  a.step = step;
  a.pol = to_score_policy(policy);
  a.max_nb = max_blocks_per_seq;
  a.max_chunks = (max_blocks_per_seq + kvs::kScoreThreads - 1) / kvs::kScoreThreads;
  a.classify = classify;
  a.status = static_cast<uint32_t*>(workspace);
  if (total_blocks == 0) return ok();
  hipError_t e = kvs::launch_score(a, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "score_update launch");
  return ok();
}

size_t kvs_evict_workspace_bytes(int32_t batch, int32_t max_blocks_per_seq) {
  if (batch < 1 || batch > kMaxBatch || max_blocks_per_seq < 1 || max_blocks_per_seq > kMaxBlocksPerSeq)
    return 0;
  const uint64_t chunks = (uint64_t)(max_blocks_per_seq + kvs::kScoreThreads - 1) / kvs::kScoreThreads;
  return align_up(align_up(kHeader + (uint64_t)batch * chunks * 8u) + (uint64_t)batch * chunks * 4u);
}

int kvs_evict_candidates(const kvs_block_meta* meta, const int32_t* meta_offsets,
                         const int32_t* seq_lens, const uint8_t* active, int32_t batch,
                         int32_t max_blocks_per_seq,
                         int64_t total_blocks, uint64_t now, double alpha, int exclude_pinned,
                         int32_t* out_block, double* out_key, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!meta || !meta_offsets || !out_block || !out_key || !workspace)
    return fail(KVS_E_NULL, "a required pointer is NULL");
  int rc = check_counts(batch, max_blocks_per_seq);
  if (rc) return rc;
  if (total_blocks < 0 || total_blocks > INT32_MAX)
    return fail(KVS_E_RANGE, "total_blocks out of range");
  if (exclude_pinned != 0 && exclude_pinned != 1)
    return fail(KVS_E_RANGE, "exclude_pinned must be 0 or 1");
  if (now == KVS_NEVER_TOUCHED) return fail(KVS_E_RANGE, "now UINT64_MAX is reserved");
  if (!std::isfinite(alpha) || !(alpha > 0.0 && alpha < 1.0))
    return fail(KVS_E_POLICY, "alpha %.17g not in (0, 1)", alpha);
  if (!aligned(meta, 16) || !aligned(out_key, 8) || !aligned(out_block, 4))
    return fail(KVS_E_ALIGN, "meta, out_key or out_block misaligned");
  if (!aligned(workspace, kAlign)) return fail(KVS_E_ALIGN, "workspace must be 256-byte aligned");
  const size_t need = kvs_evict_workspace_bytes(batch, max_blocks_per_seq);
  if (workspace_bytes < need)
    return fail(KVS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  const int32_t chunks = (max_blocks_per_seq + kvs::kScoreThreads - 1) / kvs::kScoreThreads;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  kvs::EvictArgs a{};
  a.meta = meta;
  a.meta_off = meta_offsets;
  a.seq_lens = seq_lens;
  a.active = active;
  a.part_key = reinterpret_cast<double*>(ws + kHeader);
  a.part_idx = reinterpret_cast<int32_t*>(ws + align_up(kHeader + (size_t)batch * chunks * 8u));
  a.out_block = out_block;
  a.out_key = out_key;
  a.total_blocks = total_blocks;
  a.now = now;
  a.neg_log_keep = -std::log1p(-alpha);
  a.max_nb = max_blocks_per_seq;
  a.max_chunks = chunks;
  a.exclude_pinned = exclude_pinned;
  a.status = static_cast<uint32_t*>(workspace);
  hipError_t e = kvs::launch_evict(a, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "eviction-candidate launch");
  return ok();
}

size_t kvs_append_workspace_bytes(int32_t batch) {
  if (batch < 1 || batch > kMaxBatch) return 0;
  return align_up(kHeader + (uint64_t)batch * 8u);
}

int kvs_append_kv(const kvs_shape* shape, int kv_elem_bytes, const void* k_new, const void* v_new,
                  void* kv_pool, int64_t pool_blocks, int32_t* block_table,
                  int32_t max_blocks_per_seq, int32_t* seq_lens, const int32_t* free_stack,
                  int32_t free_capacity, int32_t* free_top, kvs_block_meta* meta,
                  const int32_t* meta_offsets,
                  const uint64_t* seq_ids, int32_t anchor_blocks, int32_t batch,
                  int64_t total_blocks, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_shape(shape);
  if (rc) return rc;
  if (!k_new || !v_new || !kv_pool || !block_table || !seq_lens || !free_stack || !free_top ||
      !meta || !meta_offsets || !seq_ids || !workspace)
    return fail(KVS_E_NULL, "a required pointer is NULL");
  if (kv_elem_bytes != 1 && kv_elem_bytes != 2)
    return fail(KVS_E_RANGE, "kv_elem_bytes must be 1 (E4M3) or 2 (fp16)");
  rc = check_counts(batch, max_blocks_per_seq);
  if (rc) return rc;
  if (pool_blocks < 1 || pool_blocks > INT32_MAX) return fail(KVS_E_RANGE, "pool_blocks out of range");
  if (total_blocks < 0 || total_blocks > INT32_MAX) return fail(KVS_E_RANGE, "total_blocks out of range");
  if (anchor_blocks < 0) return fail(KVS_E_RANGE, "anchor_blocks < 0");
  if (free_capacity < 0) return fail(KVS_E_RANGE, "free_capacity < 0");
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(kv_pool, 16) || !aligned(meta, 16))
    return fail(KVS_E_ALIGN, "k_new, v_new, kv_pool and meta must be 16-byte aligned");
  if (!aligned(workspace, kAlign)) return fail(KVS_E_ALIGN, "workspace must be 256-byte aligned");
  const size_t need = kvs_append_workspace_bytes(batch);
  if (workspace_bytes < need)
    return fail(KVS_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if ((uint64_t)shape->num_layers > 65535) return fail(KVS_E_RANGE, "num_layers > 65535");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  kvs::AppendArgs a{};
  a.k_new = static_cast<const uint8_t*>(k_new);
  a.v_new = static_cast<const uint8_t*>(v_new);
  a.pool = static_cast<uint8_t*>(kv_pool);
  a.pool_blocks = pool_blocks;
  a.table = block_table;
  a.max_nb = max_blocks_per_seq;
  a.seq_lens = seq_lens;
  a.free_stack = free_stack;
  a.free_capacity = free_capacity;
  a.free_top = free_top;
  a.meta = meta;
  a.meta_off = meta_offsets;
  a.seq_ids = seq_ids;
  a.anchor_blocks = anchor_blocks;
  a.total_blocks = total_blocks;
  a.num_layers = shape->num_layers;
  a.elem_bytes = kv_elem_bytes;
  a.slot_pid = reinterpret_cast<int32_t*>(ws + kHeader);
  a.slot_idx = reinterpret_cast<int32_t*>(ws + kHeader + (size_t)batch * 4u);
  a.status = reinterpret_cast<uint32_t*>(ws);
  hipError_t e = kvs::launch_append(a, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

int kvs_classify(kvs_block_meta* meta, const int32_t* meta_offsets, const int32_t* seq_lens,
                 int32_t batch, int32_t max_blocks_per_seq, int64_t total_blocks,
                 const kvs_policy* policy, uint8_t* tiers_out, void* stream) {
  if (!meta || !meta_offsets) return fail(KVS_E_NULL, "a required pointer is NULL");
  int rc = check_policy(policy);
  if (rc) return rc;
  rc = check_counts(batch, max_blocks_per_seq);
  if (rc) return rc;
  if (total_blocks < 0 || total_blocks > INT32_MAX)
    return fail(KVS_E_RANGE, "total_blocks out of range");
  if (!aligned(meta, 16)) return fail(KVS_E_ALIGN, "meta must be 16-byte aligned");
  kvs::ScoreArgs a{};
  a.meta = meta;
  a.meta_off = meta_offsets;
  a.seq_lens = seq_lens;
  a.tiers_out = tiers_out;
  a.total_blocks = total_blocks;
  a.pol = to_score_policy(policy);
  a.max_nb = max_blocks_per_seq;
  a.max_chunks = (max_blocks_per_seq + kvs::kScoreThreads - 1) / kvs::kScoreThreads;
  a.status = nullptr;
  if (total_blocks == 0) return ok();
  hipError_t e = kvs::launch_classify(a, batch, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "classify launch");
  return ok();
}

}  // extern "C"
