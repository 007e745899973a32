// KV append with block allocation: append_alloc / append_scatter.
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

hipError_t launch_append(const AppendArgs& a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(append_alloc, dim3(1), dim3(kAllocThreads), 0, stream, a, batch);
  hipLaunchKernelGGL(append_scatter, dim3(batch, a.num_layers), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace kvs
