// Plan kernel: turns query_start_loc / seq_lens into the step's work tables
// (row-wise split-K items, chunk items, merge records) on the device.
//
// One workgroup of 1024 threads walks the requests 1024 at a time.  Phase 1:
// each thread counts its request's records with request_counts() (the same
// function the host uses to size the tables) and a block-wide scan turns the
// counts into offsets.  Phase 2: the threads emit the records in parallel,
// record index idx going to the request whose scanned range contains idx
// (binary search in LDS), so a request with many records does not serialise
// the kernel; a record's row, q-tile, segment and partial-slot offset come
// from the closed forms of pa_internal.h (no loop over the request's rows or
// q-tiles).  Phase 3 puts the items in launch order, longest first (a
// counting sort in LDS): workgroups are dispatched in item order, and
// longest-first list scheduling keeps the last, partly filled round of
// workgroups short.  Row-wise items are sorted by their key count and keep
// their plan-order index as partial slot (rw_slot); chunk items are sorted by
// the size of their (request, key segment) group and carry their slots.  Every write is bounded by the capacities the host computed and
// unused trailing records get sentinels: device metadata that disagrees with
// the host mirrors gives wrong numbers, never an out-of-bounds access.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;

struct ReqView {
  int32_t r, q, L, c, t0;
};

// first position in the inclusive scan whose value exceeds idx
__device__ __forceinline__ int upper_bound(const int32_t* inc, int n, int32_t idx) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (inc[mid] > idx) hi = mid; else lo = mid + 1;
  }
  return lo;
}

__device__ __forceinline__ int32_t min32(int32_t a, int32_t b) { return a < b ? a : b; }

// j-th row-wise item of a request; item index k (also its partial slot)
__device__ void emit_rowwise(const ReqView& v, int32_t j, int32_t k, const PlanShape& ps,
                             int4* items_rw) {
  const int32_t i = rw_row_of_item(v.c, v.q, j, ps.S);
  const int32_t jj = (int32_t)(j - rw_items_before(v.c, i, ps.S));
  const int32_t keys = v.c + i + 1;
  const int32_t parts = cdiv(keys, ps.S);
  const int32_t kb = jj * ps.S;
  const int32_t ke = min32(kb + ps.S, keys);
  if (k < ps.n_rw) items_rw[k] = make_int4(v.r, v.t0 + i, kb, ke | (parts == 1 ? kDirect : 0));
}

// j-th merge record of a row-wise request whose first item is k_first: the
// j-th row with more than one partition
__device__ void emit_merge_rowwise(const ReqView& v, int32_t j, int32_t k_first, int32_t m,
                                   const PlanShape& ps, int4* merge) {
  if (m >= ps.n_mg) return;
  const int32_t i = rw_first_split_row(v.c, ps.S) + j;
  const int64_t item = k_first + rw_items_before(v.c, i, ps.S);
  const int32_t parts = cdiv(v.c + i + 1, ps.S);
  merge[m] = i < v.q && item + parts <= ps.n_rw ? make_int4(v.t0 + i, (int32_t)item, parts, (1 << 16) | 1)
                                                : make_int4(-1, 0, 0, 0);
}

// j-th chunk item of a chunk request whose partial slots start at pbase
// (order: chunk_item_of).  Segment-major order keeps the q-tiles that read the
// same key segment consecutive, so the XCD-aware launch keeps them on one L2.
__device__ void emit_chunk(const ReqView& v, int32_t j, int32_t k, int32_t pbase,
                           const PlanShape& ps, int4* items_ck) {
  const ChunkItem it = chunk_item_of(v.c, v.q, j, ps.TQ, ps.SEG);
  if (it.qt < 0 || k >= ps.n_ck) return;
  const int64_t pb = pbase + it.slots_before;
  const bool split = it.nseg > 1 && pb + (int64_t)it.nseg * ps.TQ <= (int64_t)ps.n_rw + ps.n_ck_parts;
  items_ck[k] = make_int4(v.r, it.qt, it.seg, split ? (int32_t)pb : -1);
}

// j-th merge record of a chunk request (chunk_merge_of)
__device__ void emit_merge_chunk(const ReqView& v, int32_t j, int32_t m, int32_t pbase,
                                 const PlanShape& ps, int4* merge) {
  if (m >= ps.n_mg) return;
  const ChunkMerge r = chunk_merge_of(v.c, v.q, j, ps.TQ, ps.SEG, ps.MT);
  int4 rec = make_int4(-1, 0, 0, 0);
  if (r.qt >= 0) {
    const int64_t pb = pbase + r.slots_before;
    if (pb + (int64_t)r.nseg * ps.TQ <= (int64_t)ps.n_rw + ps.n_ck_parts)
      rec = make_int4(v.t0 + r.qt * ps.TQ + r.tau0, (int32_t)(pb + r.tau0), r.nseg, (r.n << 16) | ps.TQ);
  }
  merge[m] = rec;
}

// Sort key of a chunk item: the 64-key tiles of its key segment for the
// request's last q-tile (0 for a sentinel).  All q-tiles of one (request,
// segment) share the key, so they stay together (they read the same keys
// and values, which the XCD's L2 then serves); the item's own size is at
// most 512 keys smaller.
__device__ int32_t chunk_item_tiles(const int4 it, const int32_t* qsl, const int32_t* seq_lens,
                                    const PlanShape& ps) {
  const int32_t r = it.x;
  if (r < 0 || r >= ps.R) return 0;
  int32_t q = qsl[r + 1] - qsl[r];
  int32_t L = seq_lens[r];
  sanitize(q, L, ps.M, ps.B);
  const int32_t k0 = it.z * ps.SEG;
  const int32_t k1 = min32(k0 + ps.SEG, L);
  return k1 > k0 ? cdiv(k1 - k0, 64) : 0;
}

// block-wide exclusive scan of one value per thread (1024 threads)
__device__ int32_t block_exclusive_scan(int32_t x, int32_t* wsum16) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t v = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t y = __shfl_up(v, o, 64);
    if (lane >= o) v += y;
  }
  if (lane == 63) wsum16[wave] = v;
  __syncthreads();
  if (tid == 0) {
    int32_t acc = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int32_t t = wsum16[w];
      wsum16[w] = acc;
      acc += t;
    }
  }
  __syncthreads();
  return v - x + wsum16[wave];
}

// Stable-enough counting sort of n staged records into out, by bucket
// key(rec) in [0, kPlanThreads) ascending; slot_out (optional) receives each
// record's staged index.  Within a bucket the order follows the atomics of
// the LDS histogram (each wave's records stay in lane order).  Uses hist as
// scratch; every thread of the block must call it.
template <typename KeyFn>
__device__ void bucket_sort(const int4* stage, int32_t n, KeyFn key, int4* out, int32_t* slot_out,
                            int32_t* hist, int32_t* wsum16) {
  const int tid = threadIdx.x;
  hist[tid] = 0;
  __syncthreads();
  for (int32_t i = tid; i < n; i += kPlanThreads) atomicAdd(&hist[key(stage[i])], 1);
  __syncthreads();
  const int32_t start = block_exclusive_scan(hist[tid], wsum16);
  __syncthreads();
  hist[tid] = start;
  __syncthreads();
  for (int32_t i = tid; i < n; i += kPlanThreads) {
    const int4 rec = stage[i];
    const int32_t pos = atomicAdd(&hist[key(rec)], 1);
    if (pos < n) {
      out[pos] = rec;
      if (slot_out != nullptr) slot_out[pos] = i;
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, PlanShape ps,
            int4* __restrict__ items_rw, int4* __restrict__ rw_stage, int32_t* __restrict__ rw_slot,
            int4* __restrict__ items_ck, int4* __restrict__ ck_stage, int4* __restrict__ merge) {
  __shared__ int32_t scan[4][kPlanThreads];   // inclusive scans of the 4 counts
  __shared__ int32_t s_q[kPlanThreads], s_L[kPlanThreads], s_t0[kPlanThreads];
  __shared__ int32_t carry[4];
  __shared__ int32_t wsum[4][kPlanThreads / 64];
  const int tid = threadIdx.x;
  if (tid < 4) carry[tid] = 0;
  __syncthreads();
  for (int32_t base = 0; base < ps.R; base += kPlanThreads) {
    const int32_t r = base + tid;
    const int n_here = min32(kPlanThreads, ps.R - base);
    int32_t q = 0, L = 0, t0 = 0;
    if (r < ps.R) {
      t0 = qsl[r];
      q = qsl[r + 1] - t0;
      L = seq_lens[r];
      sanitize(q, L, ps.M, ps.B);
      if (t0 < 0 || (int64_t)t0 + q > (int64_t)ps.T) q = 0;
    }
    s_q[tid] = q;
    s_L[tid] = L;
    s_t0[tid] = t0;
    const ReqCounts n = request_counts(q, L, ps);
    // block-wide inclusive scan of the 4 counts: wave scans with shuffles,
    // then the 16 wave totals
    int32_t v[4] = {n.rw, n.ck, n.mg, n.ck_parts};
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(v[k], o, 64);
        if (lane >= o) v[k] += y;
      }
      if (lane == 63) wsum[k][wave] = v[k];
    }
    __syncthreads();
    if (tid < 4) {
      int32_t acc = 0;
      for (int w = 0; w < kPlanThreads / 64; ++w) {
        const int32_t t = wsum[tid][w];
        wsum[tid][w] = acc;
        acc += t;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) scan[k][tid] = v[k] + wsum[k][wave];
    __syncthreads();
    auto view = [&](int rl) {
      ReqView v;
      v.r = base + rl;
      v.q = s_q[rl];
      v.L = s_L[rl];
      v.c = v.L - v.q;
      v.t0 = s_t0[rl];
      return v;
    };
    auto excl = [&](int k, int rl) { return rl > 0 ? scan[k][rl - 1] : 0; };
    // row-wise items: staged for the longest-first sort, or (one-round grid,
    // where the launch order does not matter) straight into the launch table
    // with the plan-order index as partial slot
    for (int32_t idx = tid; idx < scan[0][n_here - 1]; idx += kPlanThreads) {
      const int rl = upper_bound(scan[0], n_here, idx);
      const int32_t k = carry[0] + idx;
      emit_rowwise(view(rl), idx - excl(0, rl), k, ps, ps.sort_rw ? rw_stage : items_rw);
      if (!ps.sort_rw && k < ps.n_rw) rw_slot[k] = k;
    }
    // chunk items
    for (int32_t idx = tid; idx < scan[1][n_here - 1]; idx += kPlanThreads) {
      const int rl = upper_bound(scan[1], n_here, idx);
      const int32_t pbase = ps.n_rw + carry[3] + excl(3, rl);
      emit_chunk(view(rl), idx - excl(1, rl), carry[1] + idx, pbase, ps, ck_stage);
    }
    // merge records
    for (int32_t idx = tid; idx < scan[2][n_here - 1]; idx += kPlanThreads) {
      const int rl = upper_bound(scan[2], n_here, idx);
      const ReqView v = view(rl);
      if (goes_rowwise(v.q, ps))
        emit_merge_rowwise(v, idx - excl(2, rl), carry[0] + excl(0, rl), carry[2] + idx, ps, merge);
      else
        emit_merge_chunk(v, idx - excl(2, rl), carry[2] + idx, ps.n_rw + carry[3] + excl(3, rl), ps, merge);
    }
    __syncthreads();
    if (tid == 0) {
#pragma unroll
      for (int k = 0; k < 4; ++k) carry[k] += scan[k][n_here - 1];
    }
    __syncthreads();
  }
  // sentinels for records the device did not produce (only when the device
  // metadata disagrees with the host mirrors)
  for (int32_t i = carry[0] + tid; i < ps.n_rw; i += kPlanThreads) items_rw[i] = make_int4(-1, 0, 0, 0);
  for (int32_t i = carry[1] + tid; i < ps.n_ck; i += kPlanThreads) items_ck[i] = make_int4(-1, 0, 0, 0);
  for (int32_t i = carry[2] + tid; i < ps.n_mg; i += kPlanThreads) merge[i] = make_int4(-1, 0, 0, 0);

  // phase 3: launch order, longest first.  The staged records were written
  // by this workgroup: the barrier makes them visible to all its threads.
  __syncthreads();
  const int32_t n_rw_items = min32(carry[0], ps.n_rw);
  if (n_rw_items > 0 && ps.sort_rw) {
    auto rw_key = [&](const int4 it) {
      const int32_t keys = (it.w & 0x7FFFFFFF) - it.z;
      return kPlanThreads - 1 - min32(keys < 0 ? 0 : keys, kPlanThreads - 1);
    };
    bucket_sort(rw_stage, n_rw_items, rw_key, items_rw, rw_slot, scan[0], wsum[0]);
  }
  const int32_t n_ck_items = min32(carry[1], ps.n_ck);
  if (n_ck_items > 0) {
    auto ck_key = [&](const int4 it) {
      const int32_t t = chunk_item_tiles(it, qsl, seq_lens, ps);
      return kPlanThreads - 1 - min32(t, kPlanThreads - 1);
    };
    bucket_sort(ck_stage, n_ck_items, ck_key, items_ck, nullptr, scan[0], wsum[0]);
  }
}

}  // namespace

hipError_t launch_plan(const int32_t* qsl, const int32_t* seq_lens, const PlanShape& ps,
                       int4* items_rw, int4* rw_stage, int32_t* rw_slot, int4* items_ck,
                       int4* ck_stage, int4* merge, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, qsl, seq_lens, ps, items_rw,
                     rw_stage, rw_slot, items_ck, ck_stage, merge);
  return hipGetLastError();
}

}  // namespace pa
