// Internal declarations shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <functional>
#include <vector>

#include "pa.h"

namespace pa {

// ---------------------------------------------------------------------------
// Work plan.
//
// pa_attention splits the step's query rows into two kinds of work:
//   * row-wise split-K items (decode rows, and every row of a multi-token
//     request when the chunk kernel does not handle its dtype): one item is
//     one query row x one key partition [kb, ke) x one kv head (grid y);
//   * chunk items (multi-token requests in bf16, matrix-core kernel): one
//     item is one query tile of TQ tokens x one key segment x one kv head.
// A query row whose keys were split over several items gets a merge row that
// combines the partial results by log-sum-exp ("AI Infra入门干货总结…",
// section "总结": Flash-Decoding splits the KV dimension and normalises the
// partitions with log-sum-exp).
//
// The plan is computed on the device by plan_kernel from query_start_loc and
// seq_lens, so no host-to-device copy sits on the step's critical path; the
// host evaluates the same per-request counts (request_counts below, one
// definition for both sides) from its mirrors to size the launches.
// ---------------------------------------------------------------------------

// Records (int4):
//   row-wise item  {r, t, kb, ke | kDirect}   t = flattened query row; the
//                  items are launched longest first and rw_slot[i] is the
//                  partial slot of launched item i (its index in plan order)
//   chunk item     {r, qt, seg, part_base}    part_base < 0: single segment
//   merge record   {t_first, first_part, n_parts, (n_tok << 16) | stride}:
//                  tokens t_first + tau (tau < n_tok); token tau's partials
//                  are first_part + tau + p * stride, p < n_parts.  One record
//                  per split decode row (n_tok 1, stride 1) or per group of at
//                  most MT = chunk_merge_tokens(G) tokens of a split chunk tile
//                  (stride TQ), so a record is at most max(4, G) (token, head)
//                  pairs: one per wave of the merge workgroup.
// Unused trailing records hold r = -1 / t = -1.
constexpr int32_t kDirect = (int32_t)0x80000000;

// Number of query tokens per chunk-kernel tile as a function of the GQA group:
// a tile is always 128 (token, head) rows of one kv head.
constexpr int32_t kChunkRows = 128;
__host__ __device__ inline int32_t chunk_tile_tokens(int32_t G) { return kChunkRows / G; }
__host__ __device__ inline int32_t chunk_merge_tokens(int32_t G) { return G >= 4 ? 1 : 4 / G; }

struct PlanShape {
  int32_t R;
  int32_t T;             // flattened query rows
  int32_t M;             // block-table row length
  int32_t B;             // block size
  int32_t S;             // row-wise partition length (keys), multiple of 16 and of B
  int32_t rowwise_all;   // 1: multi-token requests go row-wise too
  int32_t TQ;            // chunk tile tokens
  int32_t MT;            // tokens per chunk merge record
  int32_t SEG;           // chunk key-segment length, multiple of 64
  int32_t sort_rw;       // 1: row-wise items go to the launch order longest first
                         // (0 when the split-K grid fits in one round)
  // exact totals for this step (host mirrors); capacities of the tables
  int32_t n_rw;          // row-wise items (= row-wise partial slots)
  int32_t n_ck;          // chunk items
  int32_t n_mg;          // merge rows
  int32_t n_ck_parts;    // chunk partial slots (after the n_rw row-wise ones)
};

struct ReqCounts {
  int32_t rw;
  int32_t ck;
  int32_t mg;
  int32_t ck_parts;
};

__host__ __device__ inline int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Sanitised view of one request: L clamped into the block-table row, q into
// [0, L].  On the host the same values have already been validated, so the
// clamps change nothing there; on the device they keep every access inside
// the caller's buffers even if device metadata disagrees with the mirrors.
__host__ __device__ inline void sanitize(int32_t& q, int32_t& L, int32_t M, int32_t B) {
  const int64_t cap = (int64_t)M * B;
  if (L < 0) L = 0;
  if ((int64_t)L > cap) L = (int32_t)cap;
  if (q < 0) q = 0;
  if (q > L) q = L;
}

__host__ __device__ inline bool goes_rowwise(int32_t q, const PlanShape& ps) {
  return q == 1 || (q > 1 && ps.rowwise_all);
}

// ---- per-request plan arithmetic in closed form ---------------------------
// Every count and every record index below is O(1) or O(segments) per
// request, so a long prefill chunk (hundreds of q-tiles, thousands of rows)
// costs the planner no more than a short one.

// sum_{k=1..n} cdiv(k, S) for n >= 0: with n = a S + b, S (1 + ... + a) + b (a + 1)
__host__ __device__ inline int64_t ceil_sum(int64_t n, int64_t S) {
  const int64_t a = n / S, b = n % S;
  return S * a * (a + 1) / 2 + b * (a + 1);
}

// Row-wise request (history c): row i sees keys c + i + 1, cdiv(c + i + 1, S)
// partitions.  Items of rows 0 .. i-1:
__host__ __device__ inline int64_t rw_items_before(int32_t c, int32_t i, int32_t S) {
  return ceil_sum((int64_t)c + i, S) - ceil_sum(c, S);
}
// rows with more than one partition are rows i >= rw_first_split_row
__host__ __device__ inline int32_t rw_first_split_row(int32_t c, int32_t S) {
  return S - c > 0 ? S - c : 0;
}
// row of item j (0 <= j < items of the request): the last row i < q with
// rw_items_before(i) <= j
__host__ __device__ inline int32_t rw_row_of_item(int32_t c, int32_t q, int64_t j, int32_t S) {
  int32_t lo = 0, hi = q - 1;
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (rw_items_before(c, mid, S) <= j) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Chunk request (history c, q tokens, nqt = cdiv(q, TQ) q-tiles): q-tile t
// reads keys up to c + tok_end(t) and is cut into nseg(t) = cdiv(c +
// tok_end(t), SEG) key segments; nseg is non-decreasing in t and the last
// tile has the most, max_seg = cdiv(c + q, SEG).  The first tile with more
// than s segments (s < max_seg): tiles before the last satisfy
// c + (t + 1) TQ > s SEG exactly when t >= floor((s SEG - c) / TQ), and the
// last tile always does.
__host__ __device__ inline int32_t chunk_first_tile(int32_t c, int32_t nqt, int32_t s, int32_t TQ, int32_t SEG) {
  const int64_t x = (int64_t)s * SEG - c;
  if (x < 0) return 0;
  const int64_t t = x / TQ;
  return t < nqt - 1 ? (int32_t)t : nqt - 1;
}
__host__ __device__ inline int32_t chunk_nseg(int32_t c, int32_t q, int32_t t, int32_t TQ, int32_t SEG) {
  const int32_t tok_end = (t + 1) * TQ < q ? (t + 1) * TQ : q;
  return cdiv(c + tok_end, SEG);
}
// partial slots (nseg TQ per split tile) of the split tiles before tile t
__host__ __device__ inline int64_t chunk_slots_before(int32_t c, int32_t q, int32_t t, int32_t TQ, int32_t SEG) {
  const int32_t nqt = cdiv(q, TQ), max_seg = cdiv(c + q, SEG);
  int64_t n = 0;
  int32_t lo = max_seg > 1 ? chunk_first_tile(c, nqt, 1, TQ, SEG) : nqt;  // first tile with 2+ segments
  for (int32_t k = 2; k <= max_seg && lo < t; ++k) {
    const int32_t hi = k < max_seg ? chunk_first_tile(c, nqt, k, TQ, SEG) : nqt;  // tiles [lo, hi) have k
    const int32_t e = hi < t ? hi : t;
    if (e > lo) n += (int64_t)k * TQ * (e - lo);
    lo = hi;
  }
  return n;
}

// Chunk item j of a request (0 <= j < its item count): items are ordered
// segment-major, (segment, q-tile descending); the q-tiles that have segment
// s are tiles chunk_first_tile(s) .. nqt - 1.  slots_before = partial slots of
// the request's split tiles before this one.
struct ChunkItem {
  int32_t qt, seg, nseg;
  int64_t slots_before;
};
__host__ __device__ inline ChunkItem chunk_item_of(int32_t c, int32_t q, int32_t j, int32_t TQ, int32_t SEG) {
  const int32_t nqt = cdiv(q, TQ), max_seg = cdiv(c + q, SEG);
  ChunkItem it{-1, -1, 0, 0};
  for (int32_t sg = 0; sg < max_seg; ++sg) {
    const int32_t count = nqt - chunk_first_tile(c, nqt, sg, TQ, SEG);
    if (j < count) {
      it.qt = nqt - 1 - j;
      it.seg = sg;
      it.nseg = chunk_nseg(c, q, it.qt, TQ, SEG);
      it.slots_before = chunk_slots_before(c, q, it.qt, TQ, SEG);
      return it;
    }
    j -= count;
  }
  return it;
}

// Chunk merge record j of a request: groups of MT tokens of the split tiles
// (tiles chunk_first_tile(1) .. nqt - 1), cdiv(TQ, MT) records per tile and
// cdiv(tokens of the last tile, MT) for the last one.  qt < 0: no such record.
struct ChunkMerge {
  int32_t qt, tau0, n, nseg;
  int64_t slots_before;
};
__host__ __device__ inline ChunkMerge chunk_merge_of(int32_t c, int32_t q, int32_t j, int32_t TQ, int32_t SEG,
                                                     int32_t MT) {
  const int32_t nqt = cdiv(q, TQ), max_seg = cdiv(c + q, SEG);
  ChunkMerge r{-1, 0, 0, 0, 0};
  if (max_seg <= 1 || j < 0) return r;
  const int32_t f1 = chunk_first_tile(c, nqt, 1, TQ, SEG);
  const int32_t rec_full = cdiv(TQ, MT);
  int32_t qt = f1 + j / rec_full, jj = j % rec_full;
  if (qt >= nqt - 1) {  // the last tile (possibly fewer tokens)
    jj = j - (nqt - 1 - f1) * rec_full;
    qt = nqt - 1;
  }
  const int32_t ntok = (qt + 1) * TQ < q ? TQ : q - qt * TQ;
  const int32_t tau0 = jj * MT;
  if (tau0 >= ntok) return r;
  r.qt = qt;
  r.tau0 = tau0;
  r.n = MT < ntok - tau0 ? MT : ntok - tau0;
  r.nseg = chunk_nseg(c, q, qt, TQ, SEG);
  r.slots_before = chunk_slots_before(c, q, qt, TQ, SEG);
  return r;
}

__host__ __device__ inline ReqCounts request_counts(int32_t q, int32_t L, const PlanShape& ps) {
  ReqCounts n{0, 0, 0, 0};
  if (q <= 0) return n;
  const int32_t c = L - q;
  if (goes_rowwise(q, ps)) {
    n.rw = (int32_t)rw_items_before(c, q, ps.S);
    const int32_t f = rw_first_split_row(c, ps.S);
    n.mg = q > f ? q - f : 0;
  } else {
    const int32_t TQ = ps.TQ, SEG = ps.SEG;
    const int32_t nqt = cdiv(q, TQ), max_seg = cdiv(c + q, SEG);
    const int32_t rec_full = cdiv(TQ, ps.MT), rec_last = cdiv(q - (nqt - 1) * TQ, ps.MT);
    int32_t lo = 0;
    for (int32_t k = 1; k <= max_seg; ++k) {  // tiles [lo, hi) have k segments
      const int32_t hi = k < max_seg ? chunk_first_tile(c, nqt, k, TQ, SEG) : nqt;
      const int32_t cnt = hi - lo;
      n.ck += k * cnt;
      if (k > 1 && cnt > 0) {
        n.ck_parts += k * TQ * cnt;
        n.mg += hi == nqt ? (cnt - 1) * rec_full + rec_last : cnt * rec_full;
      }
      lo = hi;
    }
  }
  return n;
}

// ---- split-K partition length: simulated launch schedule (host) ------------
// Per-item cost of a split-K work item beyond its keys, in keys: prologue,
// pipeline fill, partial write and its share of the merge (fitted to measured
// partition-length sweeps on MI355X).
constexpr int64_t kItemOverheadKeys = 128;

// Makespan (in keys) of longest-processing-time list scheduling of the split-K
// items at partition length S on P item slots: the hardware dispatches the
// workgroups in launch order, which the planner sorts longest first, onto
// whichever slot frees first.  A row of k keys makes ceil(k / S) - 1 full
// items and one remainder; the full items, the longest, are dealt first and
// spread evenly (the slots are then loaded q or q + 1 times), the remainders
// follow longest first, each onto the least-loaded slot.  rem and heap are
// scratch vectors.
inline int64_t lpt_makespan(const std::vector<int64_t>& row_keys, int64_t S, int64_t P,
                            std::vector<int64_t>* rem, std::vector<int64_t>* heap) {
  rem->clear();
  int64_t full = 0;
  for (const int64_t k : row_keys) {
    const int64_t n = (k + S - 1) / S;
    full += n - 1;
    rem->push_back(k - (n - 1) * S + kItemOverheadKeys);
  }
  std::sort(rem->begin(), rem->end(), std::greater<int64_t>());
  const int64_t cost = S + kItemOverheadKeys;
  heap->assign((size_t)P, (full / P) * cost);
  for (int64_t i = 0; i < full % P; ++i) (*heap)[(size_t)i] += cost;
  std::make_heap(heap->begin(), heap->end(), std::greater<int64_t>());
  for (const int64_t c : *rem) {
    std::pop_heap(heap->begin(), heap->end(), std::greater<int64_t>());
    heap->back() += c;
    std::push_heap(heap->begin(), heap->end(), std::greater<int64_t>());
  }
  return *std::max_element(heap->begin(), heap->end());
}

struct WorkspaceLayout {
  size_t off_rw, off_rws, off_rwslot, off_ck, off_cks, off_mg, off_ml, off_o, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout for table sizes n_rw, n_ck, n_mg and n_ck_parts.
inline WorkspaceLayout workspace_layout_counts(int64_t n_rw, int64_t n_ck, int64_t n_mg, int64_t n_ck_parts,
                                               int32_t Hq, int32_t D) {
  WorkspaceLayout w;
  size_t o = 0;
  w.off_rw = o; o = align256(o + sizeof(int4) * (size_t)n_rw);
  w.off_rws = o; o = align256(o + sizeof(int4) * (size_t)n_rw);      // items in plan order
  w.off_rwslot = o; o = align256(o + sizeof(int32_t) * (size_t)n_rw);
  w.off_ck = o; o = align256(o + sizeof(int4) * (size_t)n_ck);
  w.off_cks = o; o = align256(o + sizeof(int4) * (size_t)n_ck);   // chunk items before sorting
  w.off_mg = o; o = align256(o + sizeof(int4) * (size_t)n_mg);
  const size_t parts = (size_t)n_rw + (size_t)n_ck_parts;
  w.off_ml = o; o = align256(o + sizeof(float) * 2 * parts * Hq);
  w.off_o = o;  o = align256(o + sizeof(float) * parts * Hq * D);
  w.total = o;
  return w;
}

inline WorkspaceLayout workspace_layout(const PlanShape& ps, int32_t Hq, int32_t D) {
  return workspace_layout_counts(ps.n_rw, ps.n_ck, ps.n_mg, ps.n_ck_parts, Hq, D);
}

// ---------------------------------------------------------------------------
// Overrides of the library's own choices, set through pa_set_tuning (tests and
// measurements).  Every knob is 0 by default, which is the product behaviour;
// the values are process-wide.
// ---------------------------------------------------------------------------
int32_t tuning(int32_t knob);

// ---------------------------------------------------------------------------
// launchers (each returns the launch's hipError_t)
// ---------------------------------------------------------------------------
hipError_t launch_write_kv(const void* key, const void* value, void* key_cache, void* value_cache,
                           const int64_t* slots, int64_t T, int64_t num_slots, int32_t row_bytes,
                           hipStream_t s);

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* block_table, int32_t M,
                               const int32_t* qsl, const int32_t* num_computed, int32_t R,
                               int64_t T, int32_t num_blocks, int32_t B, hipStream_t s);

hipError_t launch_plan(const int32_t* qsl, const int32_t* seq_lens, const PlanShape& ps,
                       int4* items_rw, int4* rw_stage, int32_t* rw_slot, int4* items_ck,
                       int4* ck_stage, int4* merge, hipStream_t s);

struct AttnArgs {
  void* out;
  const void* query;
  const void* kcache;
  const void* vcache;
  const int32_t* block_table;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* num_computed;
  int32_t M, R, Hq, Hkv, D, B, num_blocks;
  float scale_log2;   // scale * log2(e): softmax runs in base 2
  bool bf16;
  PlanShape ps;
  int4* items_rw;
  const int32_t* rw_slot;
  int4* items_ck;
  int4* merge;
  float* ml_part;     // [parts, Hq, 2] (running max in log2 units, sum)
  float* o_part;      // [parts, Hq, D] unnormalised
};

hipError_t launch_copy_blocks(const void* src, void* dst, const int32_t* pairs, int32_t n,
                              int32_t num_pools, int64_t src_stride, int64_t dst_stride,
                              int32_t src_blocks, int32_t dst_blocks, int64_t block_bytes,
                              bool host_link, hipStream_t s);

// Fused rotary embedding + cache write (one workgroup per token).
struct RopeArgs {
  void* query;                 // [T, Hq, D], rotated in place
  const void* key;             // [T, Hkv, D]
  const void* value;           // [T, Hkv, D]
  void* key_cache;             // [num_slots, Hkv, D]
  void* value_cache;
  const int64_t* slots;        // [T]
  const int64_t* positions;    // [T]
  const float* cos_sin;        // [max_position, rotary_dim]
  int64_t T;
  int64_t num_slots;
  int64_t max_position;
  int32_t rotary_dim;
  int32_t Hq, Hkv;
};
hipError_t launch_rope_write_kv(const RopeArgs& a, bool bf16, int32_t D, bool neox, hipStream_t s);

// ---- whole-block staging shared by the split-K kernels ----------------------
// A 16-token sub-tile of a partition is one contiguous slab of the cache: 16
// slots x Hkv kv heads x head row (block sizes are multiples of 16 and
// sub-tiles start at multiples of 16, so the slab never crosses a block).  One
// workgroup of Hkv waves stages it in LDS with 1-KB global -> LDS DMA
// instructions (lane l of an instruction lands at LDS base + 16 l), and wave
// g reads kv head g's rows from there.  Slab row (token j, head h) keeps its
// 16-byte chunk c at position c ^ slab_swz(j), which spreads the rows of four
// consecutive tokens over distinct bank groups; each DMA lane fetches the
// logical chunk that belongs at its physical position.
constexpr int kSlabTokens = 16;
// cache-policy operand of global_load_lds: the nontemporal bit (nt)
constexpr int kDmaNontemporal = 2;
__device__ __forceinline__ int slab_swz(int j) { return ((j & 3) << 2) | ((j >> 2) & 3); }

// Byte offset within a slab of the logical chunk that belongs at physical
// 16-byte position q of the slab (CPR chunks per head row).
template <int HKV, int CPR>
__device__ __forceinline__ uint32_t slab_source_offset(int q) {
  const int tok = q / (HKV * CPR);
  return (uint32_t)(((q & ~(CPR - 1)) | ((q & (CPR - 1)) ^ slab_swz(tok))) * 16);
}

// Wave g's share of one slab's DMA, K and V: PER_WAVE instructions each,
// source base (bytes from the cache start) `base`, lane offsets `off`.
template <int PER_WAVE>
__device__ __forceinline__ void slab_dma(const char* kcache, const char* vcache, uint64_t base,
                                         const uint32_t (&off)[PER_WAVE], char* kd, char* vd, int g) {
  typedef __attribute__((address_space(3))) void* lds_vptr;
  typedef __attribute__((address_space(1))) void* glb_vptr;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    __builtin_amdgcn_global_load_lds((glb_vptr)(kcache + base + off[i]), (lds_vptr)(kd + (g * PER_WAVE + i) * 1024),
                                     16, 0, kDmaNontemporal);
    __builtin_amdgcn_global_load_lds((glb_vptr)(vcache + base + off[i]), (lds_vptr)(vd + (g * PER_WAVE + i) * 1024),
                                     16, 0, kDmaNontemporal);
  }
}

// vmcnt(0), expcnt / lgkmcnt unconstrained: this wave's DMA into LDS is done
constexpr int kWaitDma = 0x0F70;

hipError_t launch_rowwise(const AttnArgs& a, hipStream_t s);
// Matrix-core split-K kernel for bf16 caches (same items, partials and
// launch shape as the vector kernel); nullptr where it has no instance.
const void* rowwise_mfma_kernel_for(int32_t D, int32_t G);
// Its whole-block form (one workgroup of Hkv waves per item, slabs of all kv
// heads staged in LDS); nullptr where it has no instance.
const void* rowwise_mfma_block_kernel_for(int32_t D, int32_t G, int32_t Hkv);
// Wave slots of one round of the split-K grid on the current device for this
// configuration (0 when the device cannot be queried).
int64_t rowwise_round_slots(bool bf16, int32_t D, int32_t G, int32_t Hkv);
hipError_t launch_chunk(const AttnArgs& a, hipStream_t s);
hipError_t launch_merge(const AttnArgs& a, hipStream_t s);
bool chunk_kernel_supports(bool bf16, int32_t D, int32_t G, int32_t B);
// Longest key segment one chunk work item may cover (its block ids live in LDS).
int32_t chunk_max_segment(int32_t B);

}  // namespace pa
