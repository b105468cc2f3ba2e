// C-ABI entry points of the paged-KV attention library (declared in pa.h).
//
// Host side only: argument checks, the step-metadata builder, the launch
// plan sizing and the kernel launch sequence
//   pa_write_kv:  write_kv
//   pa_rope_write_kv: rope_write_kv (rotary embedding of Q and K fused with the write)
//   pa_copy_blocks: copy_blocks (copy-on-write copies, swap transfers)
//   pa_attention: plan -> row-wise split-K -> chunk (matrix cores) -> merge
// all on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pa_internal.h"

namespace {

thread_local std::string g_err;
thread_local hipEvent_t g_prof[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
thread_local bool g_prof_on = false;

void prof_mark(int i, hipStream_t s) {
  if (g_prof_on) (void)hipEventRecord(g_prof[i], s);
}

pa_status fail(pa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

std::atomic<int32_t> g_tune[PA_TUNE_COUNT];

// Static scratch of pa_attention_noalloc.  In host code `scratch` names a
// host-side stand-in, not device memory: the device address comes from
// hipGetSymbolAddress, once per device (each GPU holds its own copy), and
// only that address is ever passed to kernels.
__device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on first use).
pa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(PA_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PA_OK;
}

pa_status check_geometry(int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                         int dtype) {
  if (dtype != PA_F32 && dtype != PA_BF16) return fail(PA_ERR_BAD_DTYPE, "dtype %d is not PA_F32 or PA_BF16", dtype);
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || B <= 0 || num_blocks <= 0)
    return fail(PA_ERR_BAD_SHAPE, "sizes must be positive (Hq=%d Hkv=%d D=%d B=%d num_blocks=%d)", Hq, Hkv, D, B, num_blocks);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", D);
  if (B % 16 != 0) return fail(PA_ERR_UNSUPPORTED, "block_size %d is not a multiple of 16", B);
  if (Hq % Hkv != 0) return fail(PA_ERR_UNSUPPORTED, "num_heads %d is not a multiple of num_kv_heads %d", Hq, Hkv);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(PA_ERR_UNSUPPORTED, "GQA group %d not in {1, 2, 4, 8}", G);
  return PA_OK;
}

int64_t gcd64(int64_t a, int64_t b) { return b == 0 ? a : gcd64(b, a % b); }
int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Partition lengths the split-K rule can choose for block size B: multiples of
// unit = lcm(64, B) up to cap = 64 blocks (one block id per lane of the
// wavefront); `longest` is the longest the occupancy-based rule picks (at most
// 2048 keys) and `top` the longest the device-independent rule picks (a
// power-of-two multiple of the unit, at most 1024 keys).
struct SplitLengths {
  int64_t unit, cap, longest, top;
};
SplitLengths split_lengths(int32_t B) {
  SplitLengths s;
  s.unit = 64 / gcd64(64, B) * B;
  s.cap = std::max<int64_t>(s.unit, (int64_t)64 * B);
  s.longest = std::max<int64_t>(1, std::min<int64_t>(s.cap, 2048) / s.unit) * s.unit;
  s.top = s.unit;
  while (s.top * 2 <= s.cap && s.top * 2 <= 1024) s.top *= 2;
  return s;
}

// The forced partition length of PA_TUNE_SPLIT_KEYS (0 when not forced).
int64_t forced_split(int32_t B) {
  const int64_t f = pa::tuning(PA_TUNE_SPLIT_KEYS);
  if (f <= 0) return 0;
  const SplitLengths sl = split_lengths(B);
  return std::min((f + sl.unit - 1) / sl.unit * sl.unit, sl.cap / sl.unit * sl.unit);
}

// Row-wise wavefronts of a step (all kv heads) at partition length S.
int64_t rowwise_waves(const int32_t* h_qsl, const int32_t* h_seq_lens, int32_t R, int32_t M,
                      int32_t Hkv, pa::PlanShape ps, int32_t S) {
  ps.S = S;
  int64_t n = 0;
  for (int32_t r = 0; r < R; ++r) {
    int32_t q = h_qsl[r + 1] - h_qsl[r];
    int32_t L = h_seq_lens[r];
    pa::sanitize(q, L, M, ps.B);
    if (q > 0 && pa::goes_rowwise(q, ps)) n += pa::request_counts(q, L, ps).rw;
  }
  return n * Hkv;
}

// Keys of every row that takes the split-K path (decode rows; with
// rowwise_all, every query row), or false when there are more than `limit`.
bool rowwise_row_keys(const int32_t* h_qsl, const int32_t* h_seq_lens, int32_t R, int32_t M,
                      const pa::PlanShape& ps, size_t limit, std::vector<int64_t>* keys) {
  keys->clear();
  for (int32_t r = 0; r < R; ++r) {
    int32_t q = h_qsl[r + 1] - h_qsl[r];
    int32_t L = h_seq_lens[r];
    pa::sanitize(q, L, M, ps.B);
    if (q <= 0 || !pa::goes_rowwise(q, ps)) continue;
    if (keys->size() + (size_t)q > limit) return false;
    for (int32_t i = 0; i < q; ++i) keys->push_back((int64_t)(L - q) + i + 1);
  }
  return true;
}

// Steps with more split-K rows than this keep the keys-per-slot rule (the
// simulation's host time grows with rows x candidate lengths).
constexpr size_t kLptMaxRows = 4096;

// Row-wise partition length: a multiple of lcm(64, B), at most 64 blocks (one
// block id per lane of the wavefront) and 2048 keys.  With the round's wave
// slots known (resident = min(occupancy, 8) waves per compute unit x compute
// units, so P = resident / Hkv item slots; 0 if unknown):
//  * when the whole split-K grid fits in one round at some length, the
//    shortest such length (any multiple of the unit: the grid then fills
//    nearly every slot, each wave as short as that allows);
//  * otherwise several rounds run: the length, among the multiples of the
//    unit from a quarter of the keys per slot (K / P) up to the longest, whose
//    simulated longest-first makespan is shortest (ties: the longer length,
//    fewer partials).  Measured on MI355X, best length against the old
//    choice of the keys per slot rounded down: 125 decode rows of about 2 K
//    keys 640 keys (226 us; 1024 keys 276 us); 16 x 32K + 240 short contexts
//    2048 (651 us; 1024 672 us, 512 727 us); C3's 512 decode rows 1024
//    (1107 us; 512 1179 us) -- the simulation picks each of these.  Steps
//    with more than kLptMaxRows split-K rows keep the keys per slot rounded
//    down.
// Without the slot count: a power-of-two multiple of the unit (<= 1024 keys)
// that gives the grid roughly 32 wavefronts per compute unit.
int32_t choose_split(const int32_t* h_qsl, const int32_t* h_seq_lens, int32_t R, int32_t M,
                     int64_t rowwise_keys, int32_t Hkv, int64_t resident, const pa::PlanShape& ps) {
  const SplitLengths sl = split_lengths(ps.B);
  const int64_t unit = sl.unit;
  const int64_t forced = forced_split(ps.B);
  if (forced > 0) return (int32_t)forced;
  if (resident > 0 && rowwise_keys > 0 && pa::tuning(PA_TUNE_SPLIT_RULE) != 1) {
    const int64_t longest = sl.longest;
    if (rowwise_waves(h_qsl, h_seq_lens, R, M, Hkv, ps, (int32_t)longest) <= resident) {
      // the wave count does not grow with the length: binary search for the
      // smallest multiple of the unit that fits
      int64_t lo = 1, hi = longest / unit;
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (rowwise_waves(h_qsl, h_seq_lens, R, M, Hkv, ps, (int32_t)(mid * unit)) <= resident) hi = mid;
        else lo = mid + 1;
      }
      return (int32_t)(lo * unit);
    }
    const int64_t P = std::max<int64_t>(1, resident / Hkv);
    const int64_t per_slot = rowwise_keys * Hkv / resident;
    // at least a quarter of the keys per slot, so K / S <= 4 P (the workspace bound)
    const int64_t s_min = std::max(unit, cdiv64(cdiv64(rowwise_keys * Hkv, 4 * resident), unit) * unit);
    std::vector<int64_t> keys, rem, heap;
    if (s_min < longest && rowwise_row_keys(h_qsl, h_seq_lens, R, M, ps, kLptMaxRows, &keys)) {
      int64_t best = longest, best_t = pa::lpt_makespan(keys, longest, P, &rem, &heap);
      for (int64_t S = longest - unit; S >= s_min; S -= unit) {
        const int64_t t = pa::lpt_makespan(keys, S, P, &rem, &heap);
        if (t < best_t) { best = S; best_t = t; }
      }
      return (int32_t)best;
    }
    return (int32_t)std::min(longest, std::max(unit, per_slot / unit * unit));
  }
  const int64_t target_waves = 256 * 32;
  const int64_t want = rowwise_keys * Hkv / target_waves;
  int64_t s = unit;
  while (s < want && s * 2 <= sl.top) s *= 2;
  return (int32_t)s;
}

// Key-segment lengths of the chunk kernel: multiples of 64 keys between
// kMinSegment and the kernel's limit.
constexpr int64_t kMinSegment = 512;
constexpr int64_t kSegmentItemsTarget = 256 * 2;
int64_t segment_limit(int32_t B) { return pa::chunk_max_segment(B) / 64 * 64; }
int64_t forced_segment(int32_t B) {
  const int64_t f = pa::tuning(PA_TUNE_CHUNK_SEGMENT);
  return f > 0 ? std::min<int64_t>(segment_limit(B), (f + 63) / 64 * 64) : 0;
}

// Key-segment length of the chunk kernel, sized so the chunk work spreads
// over about two workgroups per compute unit (long histories are cut into
// segments that the merge pass recombines; longer segments mean fewer
// partials to merge).
int32_t choose_segment(const int32_t* h_qsl, const int32_t* h_seq_lens, int32_t R, int32_t M,
                       int32_t B, int32_t Hkv, const pa::PlanShape& ps) {
  const int64_t limit = segment_limit(B);
  const int64_t forced = forced_segment(B);
  if (forced > 0) return (int32_t)forced;
  int64_t tiles = 0;  // 64-key tiles of all chunk work items, one kv head
  for (int32_t r = 0; r < R; ++r) {
    int32_t q = h_qsl[r + 1] - h_qsl[r];
    int32_t L = h_seq_lens[r];
    pa::sanitize(q, L, M, B);
    if (q <= 1 || pa::goes_rowwise(q, ps)) continue;
    const int32_t c = L - q;
    for (int32_t t0 = 0; t0 < q; t0 += ps.TQ) {
      const int32_t kmax = c + std::min(t0 + ps.TQ, q);
      tiles += (kmax + 63) / 64;
    }
  }
  const int64_t target = std::max<int64_t>(1, tiles * Hkv / kSegmentItemsTarget) * 64;
  // the power of two nearest the target (in ratio), or the limit when the
  // target is well above the largest power of two that fits
  int64_t seg = kMinSegment;
  while (seg * 2 <= limit && target * target > 2 * seg * seg) seg *= 2;
  if (seg * 2 > limit && target * target > 2 * seg * seg) seg = limit;
  return (int32_t)std::min(seg, limit);
}

bool plan_rowwise_all(bool bf16, int32_t D, int32_t G, int32_t B) {
  return !pa::chunk_kernel_supports(bf16, D, G, B) || pa::tuning(PA_TUNE_CHUNK_PATH) == 1;
}

// Validates the host mirrors and fills the plan shape (exact table sizes).
pa_status make_plan(const int32_t* h_qsl, const int32_t* h_seq_lens, int32_t R, int64_t T,
                    int32_t M, int32_t Hq, int32_t Hkv, int32_t D, int32_t B, bool bf16,
                    pa::PlanShape* out) {
  if (R < 0) return fail(PA_ERR_BAD_SHAPE, "R=%d < 0", R);
  if (R > 0 && (h_qsl == nullptr || h_seq_lens == nullptr))
    return fail(PA_ERR_NULL_PTR, "host query_start_loc / seq_lens mirrors are required");
  if (T < 0 || T > INT32_MAX) return fail(PA_ERR_BAD_SHAPE, "T=%lld out of range", (long long)T);
  if (R > 0 && h_qsl[0] != 0) return fail(PA_ERR_INCONSISTENT_METADATA, "query_start_loc[0]=%d != 0", h_qsl[0]);
  if (R > 0 && h_qsl[R] != T)
    return fail(PA_ERR_INCONSISTENT_METADATA, "query_start_loc[R]=%d != T=%lld", h_qsl[R], (long long)T);
  if (R == 0 && T != 0) return fail(PA_ERR_INCONSISTENT_METADATA, "T=%lld with no requests", (long long)T);
  const int64_t cap_tokens = (int64_t)M * B;
  int64_t rowwise_keys = 0;
  const int G = Hq / Hkv;
  pa::PlanShape ps{};
  ps.R = R;
  ps.T = (int32_t)T;
  ps.M = M;
  ps.B = B;
  ps.rowwise_all = plan_rowwise_all(bf16, D, G, B) ? 1 : 0;
  ps.TQ = pa::chunk_tile_tokens(G);
  ps.MT = pa::chunk_merge_tokens(G);
  ps.SEG = 1 << 30;
  for (int32_t r = 0; r < R; ++r) {
    const int32_t q = h_qsl[r + 1] - h_qsl[r];
    const int32_t L = h_seq_lens[r];
    if (q < 0) return fail(PA_ERR_INCONSISTENT_METADATA, "query_start_loc decreases at request %d", r);
    if (L < q) return fail(PA_ERR_INCONSISTENT_METADATA, "seq_lens[%d]=%d < query length %d", r, L, q);
    if ((int64_t)L > cap_tokens)
      return fail(PA_ERR_OUT_OF_RANGE, "seq_lens[%d]=%d exceeds max_blocks_per_req*block_size=%lld", r, L, (long long)cap_tokens);
    if (q > 0 && pa::goes_rowwise(q, ps)) {
      const int64_t c = L - q;
      rowwise_keys += q * (c + 1) + (int64_t)q * (q - 1) / 2;
    }
  }
  const int64_t resident = rowwise_keys > 0 ? pa::rowwise_round_slots(bf16, D, G, Hkv) : 0;
  ps.S = choose_split(h_qsl, h_seq_lens, R, M, rowwise_keys, Hkv, resident, ps);
  ps.SEG = choose_segment(h_qsl, h_seq_lens, R, M, B, Hkv, ps);
  int64_t n_rw = 0, n_ck = 0, n_mg = 0, n_parts = 0;
  for (int32_t r = 0; r < R; ++r) {
    int32_t q = h_qsl[r + 1] - h_qsl[r];
    int32_t L = h_seq_lens[r];
    pa::sanitize(q, L, M, B);
    const pa::ReqCounts n = pa::request_counts(q, L, ps);
    n_rw += n.rw;
    n_ck += n.ck;
    n_mg += n.mg;
    n_parts += n.ck_parts;
  }
  if (n_rw + n_parts > INT32_MAX / 2 || n_ck > INT32_MAX / 2 || n_mg > INT32_MAX / 2)
    return fail(PA_ERR_BAD_SHAPE, "step too large for one call");
  ps.n_rw = (int32_t)n_rw;
  // the longest-first launch order only matters when the grid takes more
  // than one round of the resident workgroups
  ps.sort_rw = resident > 0 && n_rw * Hkv <= resident ? 0 : 1;
  ps.n_ck = (int32_t)n_ck;
  ps.n_mg = (int32_t)n_mg;
  ps.n_ck_parts = (int32_t)n_parts;
  *out = ps;
  return PA_OK;
}

// Upper bounds of the plan's table sizes over every step with at most
// R_max requests, T_max query rows and sequences of at most L_max keys, for
// the partition and segment rules above.  Derivation (N = row-wise rows, K =
// their total keys, W = the chunk tiles' 64-key tiles of one kv head, Nqt =
// chunk q-tiles):
//  * row-wise items: a row of k keys has cdiv(k, S) <= k/S + 1 partitions, so
//    n_rw <= K/S + N with N <= Nmax (decode rows: min(R, T); every row when
//    multi-token requests go row-wise too) and K <= Nmax L_max.  K/S:
//    forced S: K/S directly.  Occupancy rule with R slots of waves: a
//    one-round grid has n_rw Hkv <= R; otherwise S >= a quarter of the keys
//    per slot K Hkv / R (K/S <= 4 R/Hkv), or S = the unit when that quarter
//    is below it (K/S < 4 R/Hkv too), or S = floor(keys per slot to the unit)
//    >= half the keys per slot (K/S < 3 R/Hkv), or S = longest (K/S <=
//    K/longest).  Device-independent rule:
//    S >= want = floor(K Hkv / 8192) gives K/S < 16384/Hkv, else S = top.
//  * chunk q-tiles: Nqt <= floor(T/TQ) + Rck with Rck <= min(R, T/2) chunk
//    requests; a tile has cdiv(kmax, SEG) <= cdiv(L_max, SEG) segments and
//    SEG >= 512 (or the forced length): n_ck <= Nqt cdiv(L_max, SEG_min).
//  * chunk partial slots: a split tile (nseg >= 2) has nseg < 2 kmax / SEG, so
//    the slots are < 2 TQ sum(kmax)/SEG <= 2 TQ 64 W / SEG.  The segment rule
//    takes SEG = the limit, or SEG >= target / sqrt 2 with target =
//    max(1, floor(W Hkv / 512)) 64 >= W Hkv / 16 when W Hkv >= 512, so
//    64 W / SEG < 1449 / Hkv; when W Hkv < 512, SEG >= 512 and 64 W / SEG <
//    64 / Hkv.  At the limit the tiles hold <= Nqt cdiv(L_max, limit)
//    segments.  Every case is also <= Nqt cdiv(L_max, SEG_min) per TQ.
//  * merge records: one per split row-wise row (<= Nmax) and at most
//    cdiv(TQ, MT) per chunk tile.
struct PlanBound {
  int64_t n_rw, n_ck, n_mg, n_ck_parts;
};
PlanBound plan_bound(int64_t R_max, int64_t T_max, int64_t L_max, int32_t Hq, int32_t Hkv, int32_t D,
                     int32_t B, bool bf16) {
  PlanBound b{0, 0, 0, 0};
  if (R_max <= 0 || T_max <= 0 || L_max <= 0) return b;
  const int32_t G = Hq / Hkv;
  const bool all_rw = plan_rowwise_all(bf16, D, G, B);
  const int64_t n_rows = all_rw ? T_max : std::min(R_max, T_max);
  const int64_t K = n_rows * L_max;
  const SplitLengths sl = split_lengths(B);
  const int64_t forced = forced_split(B);
  int64_t k_over_s;
  if (forced > 0) {
    k_over_s = cdiv64(K, forced);
  } else {
    const int64_t resident = pa::rowwise_round_slots(bf16, D, G, Hkv);
    if (resident > 0 && pa::tuning(PA_TUNE_SPLIT_RULE) != 1)
      k_over_s = std::max(4 * cdiv64(resident, Hkv), cdiv64(K, sl.longest));
    else
      k_over_s = std::max(cdiv64(16384, Hkv), cdiv64(K, sl.top));
  }
  b.n_rw = n_rows + k_over_s;
  b.n_mg = n_rows;
  if (!all_rw) {
    const int64_t TQ = pa::chunk_tile_tokens(G), MT = pa::chunk_merge_tokens(G);
    const int64_t r_ck = std::min(R_max, T_max / 2);
    const int64_t nqt = T_max / TQ + r_ck;
    const int64_t limit = segment_limit(B);
    const int64_t fseg = forced_segment(B);
    const int64_t seg_min = fseg > 0 ? fseg : kMinSegment;
    const int64_t segs_any = nqt * cdiv64(L_max, seg_min);
    int64_t split_segs = segs_any;
    if (fseg == 0)
      split_segs = std::min(segs_any, std::max(cdiv64(2 * 1449, Hkv), nqt * cdiv64(L_max, limit)));
    b.n_ck = segs_any;
    b.n_ck_parts = cdiv64(L_max, seg_min) > 1 ? TQ * split_segs : 0;
    b.n_mg += nqt * cdiv64(TQ, MT);
  }
  return b;
}

// Private layout of pa_step_plan (caller-owned, opaque).
constexpr uint32_t kPlanMagic = 0x50414E31u;  // "PAN1"
struct PlanRecord {
  uint32_t magic;
  int32_t device;
  pa::PlanShape ps;
  pa::WorkspaceLayout wl;
  const int32_t* block_table;
  const int32_t* qsl;
  const int32_t* seq_lens;
  const int32_t* num_computed;
  char* ws;
  int32_t Hq, Hkv, D, num_blocks;
  int32_t bf16;
};
static_assert(sizeof(PlanRecord) <= sizeof(pa_step_plan), "plan record exceeds pa_step_plan");

// Checks a step and fills the plan record on the host (nothing is enqueued).
pa_status prepare_plan(PlanRecord* pr, const int32_t* block_table, int32_t M, const int32_t* qsl,
                       const int32_t* seq_lens, const int32_t* num_computed, const int32_t* h_qsl,
                       const int32_t* h_seq_lens, int32_t R, int64_t T, int32_t Hq, int32_t Hkv,
                       int32_t D, int32_t num_blocks, int32_t B, pa_dtype dtype, void* workspace,
                       size_t workspace_bytes) {
  std::memset(pr, 0, sizeof *pr);
  pa_status st = check_geometry(Hq, Hkv, D, B, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (M <= 0) return fail(PA_ERR_BAD_SHAPE, "max_blocks_per_req=%d", M);
  const bool bf16 = dtype == PA_BF16;
  pa::PlanShape ps;
  st = make_plan(h_qsl, h_seq_lens, R, T, M, Hq, Hkv, D, B, bf16, &ps);
  if (st != PA_OK) return st;
  pr->ps = ps;
  pr->Hq = Hq;
  pr->Hkv = Hkv;
  pr->D = D;
  pr->num_blocks = num_blocks;
  pr->bf16 = bf16 ? 1 : 0;
  pr->device = -1;
  if (ps.n_rw > 0 || ps.n_ck > 0) {
    if (!block_table || !qsl || !seq_lens || !num_computed || !workspace)
      return fail(PA_ERR_NULL_PTR, "NULL device pointer");
    if ((uintptr_t)workspace & 255) return fail(PA_ERR_BAD_SHAPE, "workspace must be 256-byte aligned");
    const pa::WorkspaceLayout wl = pa::workspace_layout(ps, Hq, D);
    if (workspace_bytes < wl.total)
      return fail(PA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < needed %zu bytes", workspace_bytes, wl.total);
    pr->wl = wl;
    pr->block_table = block_table;
    pr->qsl = qsl;
    pr->seq_lens = seq_lens;
    pr->num_computed = num_computed;
    pr->ws = static_cast<char*>(workspace);
  }
  pr->magic = kPlanMagic;
  return PA_OK;
}

// Records the current device in a prepared plan that has work (after every
// host check, so that argument errors are reported as such without a device).
pa_status bind_device(PlanRecord* pr) {
  if (pr->ps.n_rw == 0 && pr->ps.n_ck == 0) return PA_OK;
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  pr->device = dev;
  return PA_OK;
}

// Enqueues the device planner of a prepared plan (it writes the work tables
// into the workspace).
pa_status enqueue_plan(const PlanRecord* pr, hipStream_t s) {
  const pa::PlanShape& ps = pr->ps;
  if (ps.n_rw == 0 && ps.n_ck == 0) return PA_OK;
  const pa::WorkspaceLayout& wl = pr->wl;
  char* ws = pr->ws;
  prof_mark(0, s);
  const hipError_t e = pa::launch_plan(pr->qsl, pr->seq_lens, ps, reinterpret_cast<int4*>(ws + wl.off_rw),
                                       reinterpret_cast<int4*>(ws + wl.off_rws),
                                       reinterpret_cast<int32_t*>(ws + wl.off_rwslot),
                                       reinterpret_cast<int4*>(ws + wl.off_ck),
                                       reinterpret_cast<int4*>(ws + wl.off_cks),
                                       reinterpret_cast<int4*>(ws + wl.off_mg), s);
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  prof_mark(1, s);
  return PA_OK;
}

// Checks one layer's arguments against a plan (nothing is enqueued); with
// same_device, also that the current device is the plan's.
pa_status check_run(const PlanRecord* pr, const void* out, const void* query, const void* key_cache,
                    const void* value_cache, float scale, bool same_device) {
  if (pr == nullptr) return fail(PA_ERR_NULL_PTR, "plan is NULL");
  if (pr->magic != kPlanMagic) return fail(PA_ERR_BAD_STATE, "plan was not filled by pa_attention_plan");
  if (!(scale > 0.f) || !(scale < 1e30f)) return fail(PA_ERR_BAD_SHAPE, "scale must be positive and finite");
  if (pr->ps.n_rw == 0 && pr->ps.n_ck == 0) return PA_OK;
  if (!out || !query || !key_cache || !value_cache) return fail(PA_ERR_NULL_PTR, "NULL device pointer");
  const uintptr_t mis = (uintptr_t)out | (uintptr_t)query | (uintptr_t)key_cache | (uintptr_t)value_cache;
  if (mis & 15) return fail(PA_ERR_BAD_SHAPE, "tensors must be 16-byte aligned");
  if (same_device) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev != pr->device) return fail(PA_ERR_BAD_STATE, "plan made on device %d, current device %d", pr->device, dev);
  }
  return PA_OK;
}

// Enqueues one layer's attention with a checked plan: row-wise split-K, chunk
// (matrix cores), merge.
pa_status run_step(const PlanRecord* pr, void* out, const void* query, const void* key_cache,
                   const void* value_cache, float scale, hipStream_t s) {
  const pa::PlanShape& ps = pr->ps;
  if (ps.n_rw == 0 && ps.n_ck == 0) return PA_OK;
  const pa::WorkspaceLayout& wl = pr->wl;
  char* ws = pr->ws;
  pa::AttnArgs a{};
  a.out = out;
  a.query = query;
  a.kcache = key_cache;
  a.vcache = value_cache;
  a.block_table = pr->block_table;
  a.qsl = pr->qsl;
  a.seq_lens = pr->seq_lens;
  a.num_computed = pr->num_computed;
  a.M = ps.M;
  a.R = ps.R;
  a.Hq = pr->Hq;
  a.Hkv = pr->Hkv;
  a.D = pr->D;
  a.B = ps.B;
  a.num_blocks = pr->num_blocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.bf16 = pr->bf16 != 0;
  a.ps = ps;
  a.items_rw = reinterpret_cast<int4*>(ws + wl.off_rw);
  a.rw_slot = reinterpret_cast<const int32_t*>(ws + wl.off_rwslot);
  a.items_ck = reinterpret_cast<int4*>(ws + wl.off_ck);
  a.merge = reinterpret_cast<int4*>(ws + wl.off_mg);
  a.ml_part = reinterpret_cast<float*>(ws + wl.off_ml);
  a.o_part = reinterpret_cast<float*>(ws + wl.off_o);

  prof_mark(1, s);
  hipError_t e = pa::launch_rowwise(a, s);
  if (e != hipSuccess) return hip_fail(e, "row-wise attention launch");
  prof_mark(2, s);
  e = pa::launch_chunk(a, s);
  if (e != hipSuccess) return hip_fail(e, "chunk attention launch");
  prof_mark(3, s);
  e = pa::launch_merge(a, s);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  prof_mark(4, s);
  return PA_OK;
}

}  // namespace

namespace pa {
int32_t tuning(int32_t knob) {
  return knob >= 0 && knob < PA_TUNE_COUNT ? g_tune[knob].load(std::memory_order_relaxed) : 0;
}
}  // namespace pa

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL_PTR: return "PA_ERR_NULL_PTR";
    case PA_ERR_BAD_SHAPE: return "PA_ERR_BAD_SHAPE";
    case PA_ERR_BAD_DTYPE: return "PA_ERR_BAD_DTYPE";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_OUT_OF_RANGE: return "PA_ERR_OUT_OF_RANGE";
    case PA_ERR_DUPLICATE_SLOT: return "PA_ERR_DUPLICATE_SLOT";
    case PA_ERR_INCONSISTENT_METADATA: return "PA_ERR_INCONSISTENT_METADATA";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_BAD_STATE: return "PA_ERR_BAD_STATE";
    default: return "PA_UNKNOWN";
  }
}

const char* pa_last_error(void) { return g_err.c_str(); }

pa_status pa_build_step_metadata(const int32_t* h_query_lens, const int32_t* h_num_computed,
                                 int32_t R, const int32_t* h_block_table,
                                 int32_t max_blocks_per_req, int32_t block_size,
                                 int32_t num_blocks, int32_t* h_query_start_loc,
                                 int32_t* h_seq_lens, int64_t* h_slot_mapping,
                                 int64_t slot_capacity) {
  g_err.clear();
  if (R < 0 || max_blocks_per_req < 0 || block_size <= 0 || num_blocks <= 0 || slot_capacity < 0)
    return fail(PA_ERR_BAD_SHAPE, "negative or zero size argument");
  if (h_query_start_loc == nullptr) return fail(PA_ERR_NULL_PTR, "h_query_start_loc is NULL");
  if (R > 0 && (h_query_lens == nullptr || h_num_computed == nullptr || h_seq_lens == nullptr))
    return fail(PA_ERR_NULL_PTR, "NULL per-request array");
  int64_t t = 0;
  h_query_start_loc[0] = 0;
  for (int32_t r = 0; r < R; ++r) {
    const int32_t q = h_query_lens[r], c = h_num_computed[r];
    if (q < 0 || c < 0) return fail(PA_ERR_BAD_SHAPE, "negative count for request %d", r);
    const int64_t L = (int64_t)q + c;
    if (L > INT32_MAX) return fail(PA_ERR_BAD_SHAPE, "sequence %d too long", r);
    const int64_t need = (L + block_size - 1) / block_size;
    if (need > max_blocks_per_req)
      return fail(PA_ERR_OUT_OF_RANGE, "request %d needs %lld blocks > %d", r, (long long)need, max_blocks_per_req);
    if (t + q > slot_capacity || t + q > INT32_MAX)
      return fail(PA_ERR_BAD_SHAPE, "scheduled tokens exceed slot_capacity %lld", (long long)slot_capacity);
    if (q > 0 && (h_block_table == nullptr || h_slot_mapping == nullptr))
      return fail(PA_ERR_NULL_PTR, "NULL block table or slot mapping");
    const int32_t* row = h_block_table + (int64_t)r * max_blocks_per_req;
    for (int32_t i = 0; i < q; ++i) {
      const int64_t p = (int64_t)c + i;
      const int32_t blk = row[p / block_size];
      if (blk < 0 || blk >= num_blocks)
        return fail(PA_ERR_OUT_OF_RANGE, "block_table[%d][%lld]=%d outside [0, %d)", r, (long long)(p / block_size), blk, num_blocks);
      h_slot_mapping[t + i] = (int64_t)blk * block_size + p % block_size;
    }
    t += q;
    h_query_start_loc[r + 1] = (int32_t)t;
    h_seq_lens[r] = (int32_t)L;
  }
  return PA_OK;
}

pa_status pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_table,
                                  int32_t max_blocks_per_req, const int32_t* query_start_loc,
                                  const int32_t* num_computed_tokens, int32_t R, int64_t T,
                                  int32_t num_blocks, int32_t block_size, void* stream) {
  g_err.clear();
  if (R < 0 || T < 0 || max_blocks_per_req < 0 || num_blocks <= 0 || block_size <= 0)
    return fail(PA_ERR_BAD_SHAPE, "bad sizes");
  if (R == 0 || T == 0) return PA_OK;
  if (!slot_mapping || !block_table || !query_start_loc || !num_computed_tokens)
    return fail(PA_ERR_NULL_PTR, "NULL device pointer");
  hipError_t e = pa::launch_slot_mapping(slot_mapping, block_table, max_blocks_per_req,
                                         query_start_loc, num_computed_tokens, R, T, num_blocks,
                                         block_size, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "slot mapping launch");
  return PA_OK;
}

pa_status pa_set_profiling_events(void* const* events, int32_t n_events) {
  g_err.clear();
  if (events == nullptr || n_events == 0) {
    g_prof_on = false;
    return PA_OK;
  }
  if (n_events != 5) return fail(PA_ERR_BAD_SHAPE, "n_events must be 5 (or 0)");
  for (int i = 0; i < 5; ++i) {
    if (events[i] == nullptr) return fail(PA_ERR_NULL_PTR, "event %d is NULL", i);
    g_prof[i] = reinterpret_cast<hipEvent_t>(events[i]);
  }
  g_prof_on = true;
  return PA_OK;
}

pa_status pa_write_kv(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int64_t T, int32_t num_blocks,
                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                      pa_dtype dtype, void* stream) {
  g_err.clear();
  pa_status st = check_geometry(num_kv_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (T < 0) return fail(PA_ERR_BAD_SHAPE, "T=%lld < 0", (long long)T);
  if (T == 0) return PA_OK;
  if (!key || !value || !key_cache || !value_cache || !slot_mapping)
    return fail(PA_ERR_NULL_PTR, "NULL tensor pointer");
  const int32_t row_bytes = num_kv_heads * head_dim * (dtype == PA_BF16 ? 2 : 4);
  const uintptr_t mis = (uintptr_t)key | (uintptr_t)value | (uintptr_t)key_cache | (uintptr_t)value_cache;
  if (mis & 15) return fail(PA_ERR_BAD_SHAPE, "tensors must be 16-byte aligned");
  hipError_t e = pa::launch_write_kv(key, value, key_cache, value_cache, slot_mapping, T,
                                     (int64_t)num_blocks * block_size, row_bytes,
                                     reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "write_kv launch");
  return PA_OK;
}

pa_status pa_rope_write_kv(void* query, const void* key, const void* value, void* key_cache,
                           void* value_cache, const int64_t* slot_mapping, const int64_t* positions,
                           const float* cos_sin_cache, int32_t max_position, int32_t rotary_dim,
                           int32_t neox_style, int64_t T, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t num_blocks, int32_t block_size,
                           pa_dtype dtype, void* stream) {
  g_err.clear();
  pa_status st = check_geometry(num_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (st != PA_OK) return st;
  if (T < 0) return fail(PA_ERR_BAD_SHAPE, "T=%lld < 0", (long long)T);
  if (T > INT32_MAX) return fail(PA_ERR_BAD_SHAPE, "T=%lld too large for one call", (long long)T);
  if (rotary_dim <= 0 || rotary_dim > head_dim || rotary_dim % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "rotary_dim %d must be a positive multiple of 16 and <= head_dim %d",
                rotary_dim, head_dim);
  if (max_position <= 0) return fail(PA_ERR_BAD_SHAPE, "max_position=%d <= 0", max_position);
  if (neox_style != 0 && neox_style != 1) return fail(PA_ERR_BAD_SHAPE, "neox_style must be 0 or 1");
  if (T == 0) return PA_OK;
  if (!query || !key || !value || !key_cache || !value_cache || !slot_mapping || !positions ||
      !cos_sin_cache)
    return fail(PA_ERR_NULL_PTR, "NULL pointer argument");
  const uintptr_t mis = (uintptr_t)query | (uintptr_t)key | (uintptr_t)value |
                        (uintptr_t)key_cache | (uintptr_t)value_cache;
  if (mis & 15) return fail(PA_ERR_BAD_SHAPE, "tensors must be 16-byte aligned");
  if ((uintptr_t)cos_sin_cache & 3) return fail(PA_ERR_BAD_SHAPE, "cos_sin_cache must be 4-byte aligned");
  pa::RopeArgs a{};
  a.query = query;
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.slots = slot_mapping;
  a.positions = positions;
  a.cos_sin = cos_sin_cache;
  a.T = T;
  a.num_slots = (int64_t)num_blocks * block_size;
  a.max_position = max_position;
  a.rotary_dim = rotary_dim;
  a.Hq = num_heads;
  a.Hkv = num_kv_heads;
  hipError_t e = pa::launch_rope_write_kv(a, dtype == PA_BF16, head_dim, neox_style != 0,
                                          reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope_write_kv launch");
  return PA_OK;
}

pa_status pa_copy_blocks(const void* src_pools, void* dst_pools, const int32_t* block_pairs,
                         int32_t num_pairs, int32_t num_pools, int64_t src_pool_stride,
                         int64_t dst_pool_stride, int32_t src_num_blocks, int32_t dst_num_blocks,
                         int64_t block_bytes, void* stream) {
  g_err.clear();
  if (num_pairs < 0 || num_pools < 0) return fail(PA_ERR_BAD_SHAPE, "negative count");
  if (num_pairs == 0 || num_pools == 0) return PA_OK;
  if (num_pools > 65535) return fail(PA_ERR_BAD_SHAPE, "num_pools %d > 65535", num_pools);
  if (!src_pools || !dst_pools || !block_pairs) return fail(PA_ERR_NULL_PTR, "NULL pointer argument");
  if (block_bytes <= 0 || block_bytes % 16 != 0)
    return fail(PA_ERR_BAD_SHAPE, "block_bytes %lld must be a positive multiple of 16", (long long)block_bytes);
  if (src_num_blocks <= 0 || dst_num_blocks <= 0) return fail(PA_ERR_BAD_SHAPE, "pool sizes must be positive");
  if (num_pools > 1 && (src_pool_stride < (int64_t)src_num_blocks * block_bytes ||
                        dst_pool_stride < (int64_t)dst_num_blocks * block_bytes))
    return fail(PA_ERR_BAD_SHAPE, "pool strides smaller than a pool");
  if ((src_pool_stride | dst_pool_stride) % 16 != 0 || (((uintptr_t)src_pools | (uintptr_t)dst_pools) & 15))
    return fail(PA_ERR_BAD_SHAPE, "pools and strides must be 16-byte aligned");
  // does the copy cross the host link (either side pinned host memory)?
  bool host_link = false;
  for (const void* p : {src_pools, static_cast<const void*>(dst_pools)}) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
      (void)hipGetLastError();
      return fail(PA_ERR_BAD_SHAPE, "pool %p is neither device memory nor pinned host memory", p);
    }
    if (at.type == hipMemoryTypeHost) host_link = true;
  }
  hipError_t e = pa::launch_copy_blocks(src_pools, dst_pools, block_pairs, num_pairs, num_pools,
                                        src_pool_stride, dst_pool_stride, src_num_blocks,
                                        dst_num_blocks, block_bytes, host_link,
                                        reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy_blocks launch");
  return PA_OK;
}

pa_status pa_swap_blocks(const void* src_pools, void* dst_pools, const int32_t* h_block_pairs,
                         int32_t num_pairs, int32_t num_pools, int64_t src_pool_stride,
                         int64_t dst_pool_stride, int32_t src_num_blocks, int32_t dst_num_blocks,
                         int64_t block_bytes, void* stream) {
  g_err.clear();
  if (num_pairs < 0 || num_pools < 0) return fail(PA_ERR_BAD_SHAPE, "negative count");
  if (num_pairs == 0 || num_pools == 0) return PA_OK;
  if (!src_pools || !dst_pools || !h_block_pairs) return fail(PA_ERR_NULL_PTR, "NULL pointer argument");
  if (block_bytes <= 0) return fail(PA_ERR_BAD_SHAPE, "block_bytes %lld must be positive", (long long)block_bytes);
  if (src_num_blocks <= 0 || dst_num_blocks <= 0) return fail(PA_ERR_BAD_SHAPE, "pool sizes must be positive");
  if (num_pools > 1 && (src_pool_stride < (int64_t)src_num_blocks * block_bytes ||
                        dst_pool_stride < (int64_t)dst_num_blocks * block_bytes))
    return fail(PA_ERR_BAD_SHAPE, "pool strides smaller than a pool");
  std::vector<int32_t> dsts((size_t)num_pairs);
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t sb = h_block_pairs[2 * i], db = h_block_pairs[2 * i + 1];
    if (sb < 0 || sb >= src_num_blocks || db < 0 || db >= dst_num_blocks)
      return fail(PA_ERR_OUT_OF_RANGE, "pair %d = (%d, %d) outside the pools (%d, %d blocks)", i, sb, db,
                  src_num_blocks, dst_num_blocks);
    dsts[(size_t)i] = db;
  }
  std::sort(dsts.begin(), dsts.end());
  for (size_t i = 1; i < dsts.size(); ++i)
    if (dsts[i] == dsts[i - 1]) return fail(PA_ERR_DUPLICATE_SLOT, "destination block %d named twice", dsts[i]);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const char* src = static_cast<const char*>(src_pools);
  char* dst = static_cast<char*>(dst_pools);
  for (int32_t i = 0; i < num_pairs;) {
    int32_t run = 1;   // consecutive source and destination blocks copy as one row
    while (i + run < num_pairs && h_block_pairs[2 * (i + run)] == h_block_pairs[2 * i] + run &&
           h_block_pairs[2 * (i + run) + 1] == h_block_pairs[2 * i + 1] + run)
      ++run;
    const size_t width = (size_t)run * (size_t)block_bytes;
    const size_t spitch = num_pools > 1 ? (size_t)src_pool_stride : width;
    const size_t dpitch = num_pools > 1 ? (size_t)dst_pool_stride : width;
    const hipError_t e = hipMemcpy2DAsync(dst + (int64_t)h_block_pairs[2 * i + 1] * block_bytes, dpitch,
                                          src + (int64_t)h_block_pairs[2 * i] * block_bytes, spitch, width,
                                          (size_t)num_pools, hipMemcpyDefault, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy2DAsync");
    i += run;
  }
  return PA_OK;
}

size_t pa_attention_workspace_bound(int32_t max_num_reqs, int64_t max_num_tokens,
                                   int32_t max_seq_len, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, pa_dtype dtype) {
  g_err.clear();
  if (check_geometry(num_heads, num_kv_heads, head_dim, block_size, 1, dtype) != PA_OK) return 0;
  if (max_num_reqs < 0 || max_num_tokens < 0 || max_seq_len < 0) {
    fail(PA_ERR_BAD_SHAPE, "negative step limit");
    return 0;
  }
  const PlanBound b = plan_bound(max_num_reqs, max_num_tokens, max_seq_len, num_heads, num_kv_heads,
                                 head_dim, block_size, dtype == PA_BF16);
  return pa::workspace_layout_counts(b.n_rw, b.n_ck, b.n_mg, b.n_ck_parts, num_heads, head_dim).total;
}

size_t pa_attention_workspace_size(const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                                   int32_t R, int32_t num_heads, int32_t num_kv_heads,
                                   int32_t head_dim, int32_t block_size, pa_dtype dtype) {
  g_err.clear();
  if (check_geometry(num_heads, num_kv_heads, head_dim, block_size, 1, dtype) != PA_OK) return 0;
  if (R < 0 || (R > 0 && (h_query_start_loc == nullptr || h_seq_lens == nullptr))) {
    fail(PA_ERR_NULL_PTR, "host mirrors are required");
    return 0;
  }
  // M does not change the plan as long as every sequence fits its row
  int32_t maxL = 0;
  for (int32_t r = 0; r < R; ++r) maxL = std::max(maxL, h_seq_lens[r]);
  const int32_t M = std::max(1, (maxL + block_size - 1) / block_size);
  pa::PlanShape ps;
  const int64_t T = R > 0 ? h_query_start_loc[R] : 0;
  if (make_plan(h_query_start_loc, h_seq_lens, R, T, M, num_heads, num_kv_heads, head_dim,
                block_size, dtype == PA_BF16, &ps) != PA_OK)
    return 0;
  return pa::workspace_layout(ps, num_heads, head_dim).total;
}

pa_status pa_attention_plan(pa_step_plan* plan, const int32_t* block_table,
                            int32_t max_blocks_per_req, const int32_t* query_start_loc,
                            const int32_t* seq_lens, const int32_t* num_computed_tokens,
                            const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                            int32_t R, int64_t T, int32_t num_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t num_blocks, int32_t block_size,
                            pa_dtype dtype, void* workspace, size_t workspace_bytes,
                            void* stream) {
  g_err.clear();
  if (plan == nullptr) return fail(PA_ERR_NULL_PTR, "plan is NULL");
  PlanRecord* pr = reinterpret_cast<PlanRecord*>(plan);
  pa_status st = prepare_plan(pr, block_table, max_blocks_per_req, query_start_loc, seq_lens,
                              num_computed_tokens, h_query_start_loc, h_seq_lens, R, T, num_heads,
                              num_kv_heads, head_dim, num_blocks, block_size, dtype, workspace,
                              workspace_bytes);
  if (st == PA_OK) st = bind_device(pr);
  if (st == PA_OK) st = enqueue_plan(pr, reinterpret_cast<hipStream_t>(stream));
  if (st != PA_OK) pr->magic = 0;
  return st;
}

pa_status pa_attention_run(const pa_step_plan* plan, void* out, const void* query,
                           const void* key_cache, const void* value_cache, float scale,
                           void* stream) {
  g_err.clear();
  const PlanRecord* pr = reinterpret_cast<const PlanRecord*>(plan);
  pa_status st = check_run(pr, out, query, key_cache, value_cache, scale, true);
  if (st != PA_OK) return st;
  return run_step(pr, out, query, key_cache, value_cache, scale, reinterpret_cast<hipStream_t>(stream));
}

pa_status pa_attention(void* out, const void* query, const void* key_cache,
                       const void* value_cache, const int32_t* block_table,
                       int32_t max_blocks_per_req, const int32_t* query_start_loc,
                       const int32_t* seq_lens, const int32_t* num_computed_tokens,
                       const int32_t* h_query_start_loc, const int32_t* h_seq_lens, int32_t R,
                       int64_t T, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                       int32_t num_blocks, int32_t block_size, float scale, pa_dtype dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PlanRecord pr;
  pa_status st = prepare_plan(&pr, block_table, max_blocks_per_req, query_start_loc, seq_lens,
                              num_computed_tokens, h_query_start_loc, h_seq_lens, R, T, num_heads,
                              num_kv_heads, head_dim, num_blocks, block_size, dtype, workspace,
                              workspace_bytes);
  if (st != PA_OK) return st;
  st = check_run(&pr, out, query, key_cache, value_cache, scale, false);
  if (st != PA_OK) return st;
  st = bind_device(&pr);
  if (st != PA_OK) return st;
  st = enqueue_plan(&pr, s);
  if (st != PA_OK) return st;
  return run_step(&pr, out, query, key_cache, value_cache, scale, s);
}

pa_status pa_attention_noalloc(void* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_table,
                               int32_t max_blocks_per_req, const int32_t* query_start_loc,
                               const int32_t* seq_lens, const int32_t* num_computed_tokens,
                               const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                               int32_t R, int64_t T, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t num_blocks, int32_t block_size,
                               float scale, pa_dtype dtype, void* stream) {
  g_err.clear();
  void* ws = nullptr;
  pa_status st = scratch_address(&ws);
  if (st != PA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  PlanRecord pr;
  st = prepare_plan(&pr, block_table, max_blocks_per_req, query_start_loc, seq_lens,
                    num_computed_tokens, h_query_start_loc, h_seq_lens, R, T, num_heads, num_kv_heads,
                    head_dim, num_blocks, block_size, dtype, ws, PA_NOALLOC_SCRATCH_BYTES);
  if (st == PA_ERR_WORKSPACE_TOO_SMALL)
    return fail(st, "the step needs %zu bytes of workspace, more than the %zu-byte static scratch of "
                "pa_attention_noalloc (use pa_attention with a caller workspace)",
                pa::workspace_layout(pr.ps, num_heads, head_dim).total, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  if (st != PA_OK) return st;
  st = check_run(&pr, out, query, key_cache, value_cache, scale, false);
  if (st != PA_OK) return st;
  st = bind_device(&pr);
  if (st != PA_OK) return st;
  st = enqueue_plan(&pr, s);
  if (st != PA_OK) return st;
  return run_step(&pr, out, query, key_cache, value_cache, scale, s);
}

pa_status pa_set_tuning(int32_t knob, int32_t value) {
  g_err.clear();
  if (knob < 0 || knob >= PA_TUNE_COUNT) return fail(PA_ERR_BAD_SHAPE, "unknown tuning knob %d", knob);
  if (value < 0) return fail(PA_ERR_BAD_SHAPE, "tuning value %d < 0", value);
  g_tune[knob].store(value, std::memory_order_relaxed);
  return PA_OK;
}

int32_t pa_get_tuning(int32_t knob) {
  return knob >= 0 && knob < PA_TUNE_COUNT ? g_tune[knob].load(std::memory_order_relaxed) : -1;
}
pa_status pa_validate_metadata(const int32_t* h_query_start_loc, const int32_t* h_seq_lens,
                               const int32_t* h_num_computed, const int32_t* h_block_table,
                               int32_t max_blocks_per_req, const int64_t* h_slot_mapping,
                               int32_t R, int64_t T, int32_t num_blocks, int32_t block_size) {
  g_err.clear();
  if (R < 0 || T < 0 || num_blocks <= 0 || block_size <= 0 || max_blocks_per_req < 0)
    return fail(PA_ERR_BAD_SHAPE, "bad sizes");
  if (h_query_start_loc == nullptr) return fail(PA_ERR_NULL_PTR, "query_start_loc is NULL");
  if (R > 0 && (h_seq_lens == nullptr || h_num_computed == nullptr || h_block_table == nullptr))
    return fail(PA_ERR_NULL_PTR, "NULL metadata array");
  if (h_query_start_loc[0] != 0) return fail(PA_ERR_INCONSISTENT_METADATA, "query_start_loc[0] != 0");
  for (int32_t r = 0; r < R; ++r) {
    const int32_t q = h_query_start_loc[r + 1] - h_query_start_loc[r];
    if (q < 0) return fail(PA_ERR_INCONSISTENT_METADATA, "query_start_loc decreases at %d", r);
    if ((int64_t)h_num_computed[r] + q != h_seq_lens[r] || h_num_computed[r] < 0)
      return fail(PA_ERR_INCONSISTENT_METADATA, "seq_lens[%d]=%d != num_computed %d + query length %d", r,
                  h_seq_lens[r], h_num_computed[r], q);
    const int64_t need = ((int64_t)h_seq_lens[r] + block_size - 1) / block_size;
    if (need > max_blocks_per_req)
      return fail(PA_ERR_OUT_OF_RANGE, "request %d needs %lld blocks > %d", r, (long long)need, max_blocks_per_req);
    for (int64_t j = 0; j < need; ++j) {
      const int32_t b = h_block_table[(int64_t)r * max_blocks_per_req + j];
      if (b < 0 || b >= num_blocks)
        return fail(PA_ERR_OUT_OF_RANGE, "block_table[%d][%lld]=%d outside [0, %d)", r, (long long)j, b, num_blocks);
    }
  }
  if (h_query_start_loc[R] != T) return fail(PA_ERR_INCONSISTENT_METADATA, "query_start_loc[R] != T");
  if (h_slot_mapping != nullptr && T > 0) {
    const int64_t nslots = (int64_t)num_blocks * block_size;
    for (int64_t t = 0; t < T; ++t) {
      const int64_t s = h_slot_mapping[t];
      if (s >= nslots) return fail(PA_ERR_OUT_OF_RANGE, "slot_mapping[%lld]=%lld >= %lld", (long long)t, (long long)s, (long long)nslots);
    }
    for (int32_t r = 0; r < R; ++r) {
      const int32_t c = h_num_computed[r];
      for (int32_t i = h_query_start_loc[r]; i < h_query_start_loc[r + 1]; ++i) {
        const int64_t s = h_slot_mapping[i];
        if (s < 0) continue;
        const int64_t p = (int64_t)c + (i - h_query_start_loc[r]);
        const int64_t want = (int64_t)h_block_table[(int64_t)r * max_blocks_per_req + p / block_size] * block_size + p % block_size;
        if (s != want)
          return fail(PA_ERR_INCONSISTENT_METADATA, "slot_mapping[%d]=%lld but the block table gives %lld", i, (long long)s, (long long)want);
      }
    }
    std::vector<int64_t> live;
    live.reserve((size_t)T);
    for (int64_t t = 0; t < T; ++t)
      if (h_slot_mapping[t] >= 0) live.push_back(h_slot_mapping[t]);
    std::sort(live.begin(), live.end());
    for (size_t i = 1; i < live.size(); ++i)
      if (live[i] == live[i - 1]) return fail(PA_ERR_DUPLICATE_SLOT, "slot %lld written twice", (long long)live[i]);
  }
  return PA_OK;
}

}  // extern "C"
