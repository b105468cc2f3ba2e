// Host check of the planner's closed forms (pa_internal.h) against their
// definitions written as plain loops over rows and q-tiles.
//
// For a row-wise request (history c, q rows, partition length S) row i sees
// keys c + i + 1 and has cdiv(c + i + 1, S) partitions; items are listed
// row by row, partition by partition; merge records are the rows with more
// than one partition.  For a chunk request (tile TQ tokens, key segments of
// SEG, merge groups of MT tokens) q-tile t has nseg(t) = cdiv(c + tok_end(t),
// SEG) segments; items are listed segment by segment and, within a segment,
// for the tiles that have it from the last tile down; every tile with more
// than one segment takes nseg * TQ partial slots, in tile order, and one
// merge record per MT tokens.
//
// It also checks lpt_makespan (the simulated longest-first schedule behind
// the split-K partition rule) against the same schedule written out item by
// item.
//
// Prints "ok <cases>" and exits 0, or prints the first mismatch and exits 1.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <vector>

#include "pa_internal.h"

using namespace pa;

struct Ref {
  std::vector<int32_t> rw_row, rw_part;                // per row-wise item
  std::vector<int32_t> mg_row;                         // per row-wise merge record
  std::vector<int64_t> mg_first_item;
  std::vector<int32_t> ck_qt, ck_seg, ck_nseg;         // per chunk item
  std::vector<int64_t> ck_slots_before;
  std::vector<int32_t> cm_qt, cm_tau0, cm_n, cm_nseg;  // per chunk merge record
  std::vector<int64_t> cm_slots_before;
  int64_t ck_parts = 0;
};

static Ref rowwise_ref(int32_t c, int32_t q, int32_t S) {
  Ref r;
  int64_t item = 0;
  for (int32_t i = 0; i < q; ++i) {
    const int32_t parts = (c + i + 1 + S - 1) / S;
    if (parts > 1) {
      r.mg_row.push_back(i);
      r.mg_first_item.push_back(item);
    }
    for (int32_t p = 0; p < parts; ++p) {
      r.rw_row.push_back(i);
      r.rw_part.push_back(p);
    }
    item += parts;
  }
  return r;
}

static Ref chunk_ref(int32_t c, int32_t q, int32_t TQ, int32_t SEG, int32_t MT) {
  Ref r;
  const int32_t nqt = (q + TQ - 1) / TQ;
  std::vector<int32_t> nseg(nqt), ntok(nqt);
  std::vector<int64_t> before(nqt);
  int64_t slots = 0;
  int32_t max_seg = 0;
  for (int32_t t = 0; t < nqt; ++t) {
    const int32_t tok_end = (t + 1) * TQ < q ? (t + 1) * TQ : q;
    nseg[t] = (c + tok_end + SEG - 1) / SEG;
    ntok[t] = tok_end - t * TQ;
    before[t] = slots;
    if (nseg[t] > 1) slots += (int64_t)nseg[t] * TQ;
    if (nseg[t] > max_seg) max_seg = nseg[t];
  }
  r.ck_parts = slots;
  for (int32_t s = 0; s < max_seg; ++s)
    for (int32_t t = nqt - 1; t >= 0; --t)
      if (nseg[t] > s) {
        r.ck_qt.push_back(t);
        r.ck_seg.push_back(s);
        r.ck_nseg.push_back(nseg[t]);
        r.ck_slots_before.push_back(before[t]);
      }
  for (int32_t t = 0; t < nqt; ++t)
    if (nseg[t] > 1)
      for (int32_t tau0 = 0; tau0 < ntok[t]; tau0 += MT) {
        r.cm_qt.push_back(t);
        r.cm_tau0.push_back(tau0);
        r.cm_n.push_back(ntok[t] - tau0 < MT ? ntok[t] - tau0 : MT);
        r.cm_nseg.push_back(nseg[t]);
        r.cm_slots_before.push_back(before[t]);
      }
  return r;
}

static bool fail(const char* what, long long a, long long b, int32_t c, int32_t q, long long j) {
  std::printf("MISMATCH %s: got %lld want %lld (c=%d q=%d j=%lld)\n", what, a, b, c, q, j);
  return false;
}

static bool check_rowwise(int32_t c, int32_t q, int32_t S) {
  const Ref r = rowwise_ref(c, q, S);
  PlanShape ps{};
  ps.S = S;
  ps.rowwise_all = 1;
  const ReqCounts n = request_counts(q, c + q, ps);
  if (n.rw != (int32_t)r.rw_row.size()) return fail("rw count", n.rw, r.rw_row.size(), c, q, -1);
  if (n.mg != (int32_t)r.mg_row.size()) return fail("rw merge count", n.mg, r.mg_row.size(), c, q, -1);
  for (size_t j = 0; j < r.rw_row.size(); ++j) {
    const int32_t i = rw_row_of_item(c, q, (int64_t)j, S);
    if (i != r.rw_row[j]) return fail("rw row", i, r.rw_row[j], c, q, j);
    const int64_t p = (int64_t)j - rw_items_before(c, i, S);
    if (p != r.rw_part[j]) return fail("rw partition", p, r.rw_part[j], c, q, j);
  }
  for (size_t j = 0; j < r.mg_row.size(); ++j) {
    const int32_t i = rw_first_split_row(c, S) + (int32_t)j;
    if (i != r.mg_row[j]) return fail("rw merge row", i, r.mg_row[j], c, q, j);
    if (rw_items_before(c, i, S) != r.mg_first_item[j])
      return fail("rw merge item", rw_items_before(c, i, S), r.mg_first_item[j], c, q, j);
  }
  return true;
}

static bool check_chunk(int32_t c, int32_t q, int32_t TQ, int32_t SEG, int32_t MT) {
  const Ref r = chunk_ref(c, q, TQ, SEG, MT);
  PlanShape ps{};
  ps.TQ = TQ;
  ps.SEG = SEG;
  ps.MT = MT;
  ps.S = 64;
  ps.rowwise_all = 0;
  const ReqCounts n = request_counts(q, c + q, ps);
  if (n.ck != (int32_t)r.ck_qt.size()) return fail("chunk count", n.ck, r.ck_qt.size(), c, q, -1);
  if (n.ck_parts != r.ck_parts) return fail("chunk slots", n.ck_parts, r.ck_parts, c, q, -1);
  if (n.mg != (int32_t)r.cm_qt.size()) return fail("chunk merge count", n.mg, r.cm_qt.size(), c, q, -1);
  for (size_t j = 0; j < r.ck_qt.size(); ++j) {
    const ChunkItem it = chunk_item_of(c, q, (int32_t)j, TQ, SEG);
    if (it.qt != r.ck_qt[j]) return fail("chunk item tile", it.qt, r.ck_qt[j], c, q, j);
    if (it.seg != r.ck_seg[j]) return fail("chunk item segment", it.seg, r.ck_seg[j], c, q, j);
    if (it.nseg != r.ck_nseg[j]) return fail("chunk item nseg", it.nseg, r.ck_nseg[j], c, q, j);
    if (it.slots_before != r.ck_slots_before[j])
      return fail("chunk item slots", it.slots_before, r.ck_slots_before[j], c, q, j);
  }
  if (chunk_item_of(c, q, (int32_t)r.ck_qt.size(), TQ, SEG).qt != -1)
    return fail("chunk item past the end", 0, -1, c, q, r.ck_qt.size());
  for (size_t j = 0; j < r.cm_qt.size(); ++j) {
    const ChunkMerge m = chunk_merge_of(c, q, (int32_t)j, TQ, SEG, MT);
    if (m.qt != r.cm_qt[j]) return fail("chunk merge tile", m.qt, r.cm_qt[j], c, q, j);
    if (m.tau0 != r.cm_tau0[j]) return fail("chunk merge tau0", m.tau0, r.cm_tau0[j], c, q, j);
    if (m.n != r.cm_n[j]) return fail("chunk merge tokens", m.n, r.cm_n[j], c, q, j);
    if (m.nseg != r.cm_nseg[j]) return fail("chunk merge nseg", m.nseg, r.cm_nseg[j], c, q, j);
    if (m.slots_before != r.cm_slots_before[j])
      return fail("chunk merge slots", m.slots_before, r.cm_slots_before[j], c, q, j);
  }
  if (chunk_merge_of(c, q, (int32_t)r.cm_qt.size(), TQ, SEG, MT).qt != -1)
    return fail("chunk merge past the end", 0, -1, c, q, r.cm_qt.size());
  return true;
}

// Longest-processing-time list scheduling written out: every item of every
// row (full items of S keys, one remainder) sorted longest first, each placed
// on the least-loaded of P slots; each costs its keys + kItemOverheadKeys.
static int64_t lpt_brute(const std::vector<int64_t>& rows, int64_t S, int64_t P) {
  std::vector<int64_t> items;
  for (const int64_t k : rows)
    for (int64_t kb = 0; kb < k; kb += S) items.push_back((k - kb < S ? k - kb : S) + kItemOverheadKeys);
  std::sort(items.begin(), items.end(), std::greater<int64_t>());
  std::vector<int64_t> load((size_t)P, 0);
  for (const int64_t c : items) *std::min_element(load.begin(), load.end()) += c;
  return *std::max_element(load.begin(), load.end());
}

int main() {
  long cases = 0;
  // simulated launch schedule of the split-K partition rule
  {
    srand(777);
    std::vector<int64_t> rem, heap;
    for (int k = 0; k < 400; ++k) {
      const int64_t P = 1 + rand() % 300;
      const int64_t S = 64 * (1 + rand() % 32);
      std::vector<int64_t> rows((size_t)(1 + rand() % 200));
      for (auto& r : rows) r = 1 + rand() % (k % 2 ? 5000 : 40000);
      const int64_t want = lpt_brute(rows, S, P), got = lpt_makespan(rows, S, P, &rem, &heap);
      if (want != got) {
        std::printf("lpt mismatch: P=%lld S=%lld rows=%zu: %lld vs %lld\n", (long long)P, (long long)S,
                    rows.size(), (long long)got, (long long)want);
        return 1;
      }
      ++cases;
    }
  }
  // exhaustive small ranges
  for (int32_t S : {64, 128, 192, 1024})
    for (int32_t c = 0; c <= 300; c += 7)
      for (int32_t q = 1; q <= 140; q += 3) {
        if (!check_rowwise(c, q, S)) return 1;
        ++cases;
      }
  for (int32_t TQ : {16, 32, 64, 128})
    for (int32_t MT : {1, 2, 4})
      for (int32_t SEG : {64, 128, 192, 512})
        for (int32_t c = 0; c <= 700; c += 37)
          for (int32_t q = 2; q <= 600; q += 29) {
            if (!check_chunk(c, q, TQ, SEG, MT)) return 1;
            ++cases;
          }
  // random large ones
  srand(12345);
  for (int k = 0; k < 3000; ++k) {
    const int32_t S = 64 * (1 + rand() % 32);
    const int32_t c = rand() % 40000, q = 1 + rand() % 3000;
    if (!check_rowwise(c, q, S)) return 1;
    const int32_t TQ = 16 << (rand() % 4), MT = 1 << (rand() % 3);
    const int32_t SEG = 64 * (1 + rand() % 128);
    const int32_t cq = 2 + rand() % 20000, cc = rand() % 60000;
    if (!check_chunk(cc, cq, TQ, SEG, MT)) return 1;
    cases += 2;
  }
  std::printf("ok %ld\n", cases);
  return 0;
}
