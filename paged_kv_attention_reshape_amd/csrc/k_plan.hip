// Plan kernel: turns query_start_loc / seq_lens into the step's work tables
// (row-wise split-K items, chunk items, merge rows) on the device.
//
// One workgroup of 1024 threads walks the requests 1024 at a time; each
// thread counts its request's work with request_counts() (the same function
// the host uses to size the tables), a block-wide scan turns the counts into
// table offsets, and each thread writes its records.  Every write is bounded
// by the table capacities the host computed, and unused trailing records are
// filled with sentinels, so a mismatch between device metadata and the host
// mirrors can give wrong numbers but never an out-of-bounds access.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kPlanThreads = 1024;

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, PlanShape ps,
            int4* __restrict__ items_rw, int4* __restrict__ items_ck, int4* __restrict__ merge) {
  __shared__ int32_t scan[4][kPlanThreads];
  __shared__ int32_t carry[4];
  const int tid = threadIdx.x;
  if (tid < 4) carry[tid] = 0;
  __syncthreads();
  for (int32_t base = 0; base < ps.R; base += kPlanThreads) {
    const int32_t r = base + tid;
    int32_t q = 0, L = 0, t0 = 0;
    if (r < ps.R) {
      t0 = qsl[r];
      q = qsl[r + 1] - t0;
      L = seq_lens[r];
      sanitize(q, L, ps.M, ps.B);
      if (t0 < 0 || (int64_t)t0 + q > (int64_t)ps.T) q = 0;
    }
    const ReqCounts n = request_counts(q, L, ps);
    scan[0][tid] = n.rw;
    scan[1][tid] = n.ck;
    scan[2][tid] = n.mg;
    scan[3][tid] = n.ck_parts;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      int32_t v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = tid >= off ? scan[k][tid - off] : 0;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 4; ++k) scan[k][tid] += v[k];
      __syncthreads();
    }
    int32_t k_rw = carry[0] + scan[0][tid] - n.rw;
    int32_t k_ck = carry[1] + scan[1][tid] - n.ck;
    int32_t k_mg = carry[2] + scan[2][tid] - n.mg;
    int32_t pb = ps.n_rw + carry[3] + scan[3][tid] - n.ck_parts;
    const int32_t pb_end = ps.n_rw + ps.n_ck_parts;
    if (q > 0) {
      const int32_t c = L - q;
      if (goes_rowwise(q, ps)) {
        for (int32_t i = 0; i < q; ++i) {
          const int32_t keys = c + i + 1;
          const int32_t parts = cdiv(keys, ps.S);
          if (parts > 1) {
            if (k_mg < ps.n_mg) merge[k_mg] = make_int4(t0 + i, k_rw, parts, (1 << 8) | 1);
            ++k_mg;
          }
          for (int32_t p = 0; p < parts; ++p) {
            const int32_t kb = p * ps.S;
            const int32_t ke = kb + ps.S < keys ? kb + ps.S : keys;
            if (k_rw < ps.n_rw)
              items_rw[k_rw] = make_int4(r, t0 + i, kb, ke | (parts == 1 ? kDirect : 0));
            ++k_rw;
          }
        }
      } else {
        const int32_t nqt = cdiv(q, ps.TQ);
        for (int32_t qt = 0; qt < nqt; ++qt) {
          const int32_t tok_end = (qt + 1) * ps.TQ < q ? (qt + 1) * ps.TQ : q;
          const int32_t nseg = cdiv(c + tok_end, ps.SEG);
          const bool split = nseg > 1 && pb + nseg * ps.TQ <= pb_end;
          for (int32_t sg = 0; sg < nseg; ++sg) {
            if (k_ck < ps.n_ck) items_ck[k_ck] = make_int4(r, qt, sg, split ? pb : -1);
            ++k_ck;
          }
          if (nseg > 1) {
            if (k_mg < ps.n_mg)
              merge[k_mg] = split ? make_int4(t0 + qt * ps.TQ, pb, nseg,
                                              ((tok_end - qt * ps.TQ) << 8) | ps.TQ)
                                  : make_int4(-1, 0, 0, 0);
            ++k_mg;
            pb += nseg * ps.TQ;
          }
        }
      }
    }
    __syncthreads();
    if (tid == kPlanThreads - 1) {
#pragma unroll
      for (int k = 0; k < 4; ++k) carry[k] += scan[k][tid];
    }
    __syncthreads();
  }
  // sentinels for records the device did not produce (only when the device
  // metadata disagrees with the host mirrors)
  for (int32_t i = carry[0] + tid; i < ps.n_rw; i += kPlanThreads) items_rw[i] = make_int4(-1, 0, 0, 0);
  for (int32_t i = carry[1] + tid; i < ps.n_ck; i += kPlanThreads) items_ck[i] = make_int4(-1, 0, 0, 0);
  for (int32_t i = carry[2] + tid; i < ps.n_mg; i += kPlanThreads) merge[i] = make_int4(-1, 0, 0, 0);
}

}  // namespace

hipError_t launch_plan(const int32_t* qsl, const int32_t* seq_lens, const PlanShape& ps,
                       int4* items_rw, int4* items_ck, int4* merge, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, qsl, seq_lens, ps, items_rw,
                     items_ck, merge);
  return hipGetLastError();
}

}  // namespace pa
