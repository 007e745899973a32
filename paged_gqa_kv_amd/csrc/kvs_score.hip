// Scoring kernels over the 64-byte records: seq_chunk_max / score_update
// (normalise, EMA, touch, priority, tier), classify_records, the eviction
// candidate (evict_chunks / evict_final) and meta_init.
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

// Up to this many chunks per sequence (4,096 records), score_update takes each
// sequence's maximum straight from the block mass (every work-group reads its
// sequence's whole mass: at most 16 KiB, eight loads in flight per thread) and
// seq_chunk_max is not launched: one launch fewer per step (8 x 8K tokens:
// 11 -> 7 us).  Longer sequences use the two-kernel form, which measured
// faster from 8,192 records on.  max is exact in any order, so both forms give
// the same bits.
constexpr int kDirectMaxChunks = 16;

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
  const bool direct = a.max_chunks <= kDirectMaxChunks;
  int r0 = 0;
  const int nb = seq_records(a.meta_off, a.seq_lens, s, a.max_nb, a.total_blocks, a.status,
                             direct && threadIdx.x == 0 && chunk == 0, &r0);
  if (nb <= 0 || chunk * kScoreThreads >= nb) return;
  // This thread's record and mass are loaded before the sequence maximum, so
  // that their latency overlaps it; no other thread touches the record.
  const int b = chunk * kScoreThreads + threadIdx.x;
  const bool live = b < nb;
  kvs_block_meta* rec = a.meta + r0 + (live ? b : 0);
  uint64_t tt = 0;
  double prev = 0.0;
  uint32_t count = 0;
  uint8_t flags = 0;
  float mb = 0.f;
  if (live) {
    tt = rec->t_touch;
    prev = rec->score;
    count = rec->touch_count;
    flags = rec->flags;
    mb = a.mass[r0 + b];
  }
  float M = 0.f;
  if (direct) {
    // indices past the end re-read the last record: harmless for a maximum
    for (int k0 = threadIdx.x; k0 < nb; k0 += 8 * kScoreThreads) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = a.mass[r0 + min(k0 + u * kScoreThreads, nb - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) M = fmaxf(M, v[u]);
    }
  } else {
    const int nch = (nb + kScoreThreads - 1) / kScoreThreads;
    for (int k = threadIdx.x; k < nch; k += kScoreThreads)
      M = fmaxf(M, a.chunk_max[(size_t)s * a.max_chunks + k]);
  }
  M = block_reduce_max(M, red);

  bool stale = false;
  if (live) {
    if (tt != KVS_NEVER_TOUCHED && tt >= a.step) {
      stale = true;
    } else {
      const double mh = M > 0.f ? (double)mb / (double)M : 0.0;
      // Input 0 on the steps since the last touch: the stored score first
      // decays over the gap, then takes the one-step update.
      if (tt != KVS_NEVER_TOUCHED && a.step - tt > 1)
        prev *= pow(1.0 - a.pol.alpha, (double)(a.step - tt - 1));
      const double e = a.pol.alpha * mh + (1.0 - a.pol.alpha) * prev;
      rec->score = e;
      rec->touch_count = count + 1u;
      rec->t_touch = a.step;
      if (a.classify) {
        double P;
        uint8_t tier;
        priority_and_tier(a.pol, b, nb, e, flags, &P, &tier);
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

hipError_t launch_score(const ScoreArgs& a, int batch, hipStream_t stream) {
  const dim3 grid(a.max_chunks, batch);
  if (a.max_chunks > kDirectMaxChunks)
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

}  // namespace kvs
