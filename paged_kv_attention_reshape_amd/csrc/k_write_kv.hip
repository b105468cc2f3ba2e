// Cache-write kernel: scatter the step's new K/V rows into the paged pool.
//
// "AI Infra入门干货总结：大模型是如何高效推理的", section "Paged Attention":
// the slot of a token is block * block_size + offset, and the cache of a
// layer is [num_blocks, block_size, num_kv_heads, head_dim], so one token's
// K (or V) for all kv heads is one contiguous row of num_kv_heads * head_dim
// elements at row index `slot` of the pool viewed as [num_blocks*block_size,
// row].  The write is therefore a row gather-scatter: every 16-byte chunk of
// the source row goes to the same offset of the destination row.
//
// MI355X mapping: consecutive lanes move consecutive 16-byte chunks of the
// same row, so each wavefront issues fully coalesced 1 KiB loads and stores;
// K and V of a token are handled by the same workgroup (second half of the
// block), which keeps the slot value in one cache line for both.  The kernel
// is bandwidth- and latency-bound and touches each byte exactly once.
//
// The same file holds the device slot mapping and the block-copy kernel that
// executes a plan's copy-on-write copies and swap transfers.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int64_t kHostLinkGroups = 64;  // copy workgroups for host-link transfers

__global__ void __launch_bounds__(kThreads)
write_kv_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
                const int64_t* __restrict__ slots, int64_t T, int64_t num_slots,
                int32_t chunks_per_row) {
  // one block handles `tokens_per_block` tokens; threads [0, half) copy K,
  // [half, 2*half) copy V of the same tokens
  const int32_t half = kThreads / 2;
  const bool is_v = threadIdx.x >= half;
  const int32_t lt = is_v ? threadIdx.x - half : threadIdx.x;
  const int64_t total = T * (int64_t)chunks_per_row;
  const uint4* __restrict__ src = is_v ? value : key;
  uint4* __restrict__ dst = is_v ? value_cache : key_cache;
  for (int64_t idx = (int64_t)blockIdx.x * half + lt; idx < total;
       idx += (int64_t)gridDim.x * half) {
    const int64_t t = idx / chunks_per_row;
    const int64_t c = idx - t * chunks_per_row;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    dst[slot * chunks_per_row + c] = src[t * chunks_per_row + c];
  }
}

// Slot mapping on the device: one workgroup per request, threads over its
// tokens.  Position p of request r maps to block_table[r][p / B] * B + p % B.
__global__ void __launch_bounds__(kThreads)
slot_mapping_kernel(int64_t* __restrict__ slots, const int32_t* __restrict__ block_table,
                    int32_t M, const int32_t* __restrict__ qsl, const int32_t* __restrict__ num_computed,
                    int64_t T, int32_t num_blocks, int32_t B) {
  const int r = blockIdx.x;
  const int64_t t0 = qsl[r];
  int64_t q = (int64_t)qsl[r + 1] - t0;
  if (t0 < 0 || t0 > T) return;
  if (q > T - t0) q = T - t0;
  const int64_t c = num_computed[r];
  for (int64_t i = threadIdx.x; i < q; i += blockDim.x) {
    const int64_t p = c + i;
    const int64_t j = p / B;
    int64_t s = -1;
    if (p >= 0 && j < M) {
      const int32_t blk = block_table[(int64_t)r * M + j];
      if (blk >= 0 && blk < num_blocks) s = (int64_t)blk * B + p % B;
    }
    slots[t0 + i] = s;
  }
}

// Block copies between pools of the same block layout: pair i moves block
// pairs[i].src of every source pool to block pairs[i].dst of the matching
// destination pool (pool k at base + k * stride).  A unit is one (pair,
// pool) block; the grid's workgroups stride over the units (pool-fastest, so
// consecutive units of one pair touch the pools in address order); each
// thread moves 16-byte chunks, eight loads in flight before the stores.
// Serves copy-on-write (same pool) and swap between the device cache and a
// pinned host pool: the kernel reads or writes host memory over the host
// link directly, one launch for any scattered block list, and for such
// transfers the grid is a few dozen workgroups (the link, not the compute
// units, bounds the copy), so a swap running beside a step leaves the compute
// units to attention.
__global__ void __launch_bounds__(kThreads)
copy_blocks_kernel(const char* src, char* dst,
                   const int32_t* __restrict__ pairs, int64_t src_stride, int64_t dst_stride,
                   int32_t src_blocks, int32_t dst_blocks, int64_t chunks, int64_t units,
                   int32_t num_pools) {
  for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int64_t i = unit / num_pools;
    const int64_t k = unit - i * num_pools;
    const int32_t sb = pairs[2 * i];
    const int32_t db = pairs[2 * i + 1];
    if (sb < 0 || sb >= src_blocks || db < 0 || db >= dst_blocks) continue;
    // source and destination may be the same pool (distinct blocks)
    const uint4* sp = reinterpret_cast<const uint4*>(src + k * src_stride) + (int64_t)sb * chunks;
    uint4* dp = reinterpret_cast<uint4*>(dst + k * dst_stride) + (int64_t)db * chunks;
    constexpr int U = 8;
    int64_t c = threadIdx.x;
    for (; c + (U - 1) * kThreads < chunks; c += U * kThreads) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = sp[c + u * kThreads];
#pragma unroll
      for (int u = 0; u < U; ++u) dp[c + u * kThreads] = v[u];
    }
    for (; c < chunks; c += kThreads) dp[c] = sp[c];
  }
}

}  // namespace

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* block_table, int32_t M,
                               const int32_t* qsl, const int32_t* num_computed, int32_t R,
                               int64_t T, int32_t num_blocks, int32_t B, hipStream_t s) {
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(R), dim3(kThreads), 0, s, slots, block_table, M,
                     qsl, num_computed, T, num_blocks, B);
  return hipGetLastError();
}

hipError_t launch_write_kv(const void* key, const void* value, void* key_cache, void* value_cache,
                           const int64_t* slots, int64_t T, int64_t num_slots, int32_t row_bytes,
                           hipStream_t s) {
  const int32_t cpr = row_bytes / 16;
  const int64_t total = T * (int64_t)cpr;
  int64_t blocks = (total + kThreads / 2 - 1) / (kThreads / 2);
  if (blocks > 1 << 20) blocks = 1 << 20;
  hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache), slots, T,
                     num_slots, cpr);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const void* src, void* dst, const int32_t* pairs, int32_t n,
                              int32_t num_pools, int64_t src_stride, int64_t dst_stride,
                              int32_t src_blocks, int32_t dst_blocks, int64_t block_bytes,
                              bool host_link, hipStream_t s) {
  if (n == 0 || num_pools == 0) return hipSuccess;
  const int64_t units = (int64_t)n * num_pools;
  // host-link transfers: a few dozen workgroups keep about 2 MiB in flight,
  // enough for the link; device copies: up to eight workgroups per compute unit
  const int64_t cap = host_link ? kHostLinkGroups : 2048;
  const int64_t grid = units < cap ? units : cap;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s,
                     static_cast<const char*>(src), static_cast<char*>(dst), pairs, src_stride,
                     dst_stride, src_blocks, dst_blocks, block_bytes / 16, units, num_pools);
  return hipGetLastError();
}

}  // namespace pa
