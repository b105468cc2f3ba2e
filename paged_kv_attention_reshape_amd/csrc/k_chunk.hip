// Prefill-chunk attention on the matrix cores (bf16 MFMA, fp32 accumulate).
//
// Method: "AI Infra入门干货总结：大模型是如何高效推理的", section "Attention
// Module": FlashAttention fuses q.k, softmax and p.v over tiles with online
// softmax; prefill attention is dense matrix work that amortises each K/V
// tile over many query rows (the compute-bound case).  "Chunked Prefill 与
// Preemption", equation M_{i,j}: a chunk's query at absolute position i sees
// keys j <= i of the cache, which already holds the chunk's own K/V.
//
// Work item: one tile of 128 (token, head) rows -- TQ = 128 / G tokens of a
// chunk times the G query heads of kv head g -- against one key segment of
// the request's cache.  Long histories are cut into segments whose partial
// results the merge pass combines, so a chunk deep into a 16K-token prompt
// spreads over many workgroups.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16; wave w owns rows 32w..32w+31):
//   S^T = K Q^T : A = 32 keys x 16 d from LDS, B = the wave's Q rows held in
//                 registers for the whole item; the accumulator gives each
//                 lane all scores of ONE query row (16 keys per 32-key block),
//                 so the row max and row sum are lane-local plus one
//                 permlane32 swap with the partner lane.
//   O^T = V^T P^T : B = the lane's own probabilities converted to bf16 in
//                 place (the K-slot order of the MFMA is permuted to match the
//                 accumulator layout, so P never moves between lanes); A = V
//                 read straight from the row-major [key][d] LDS tile with
//                 ds_read_b64_tr_b16 transposed loads.  O^T stays one query
//                 row per lane, so the online-softmax rescale is lane-local.
// K/V tiles of 64 keys are gathered through the block table by global->LDS
// DMA (16-byte chunks, rows XOR-swizzled in LDS against bank conflicts) into a
// double buffer while the previous tile is on the matrix cores.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kThreads = kChunkRows * 2;  // one wave per 32 rows
constexpr int kWaves = kThreads / 64;
constexpr int KT = 64;         // keys per tile
constexpr int kMaxSegBlocks = 1024;
constexpr int kXcds = 8;       // accelerator complex dies of an MI355X
constexpr float kNegInf = -__builtin_huge_valf();

template <int V>
struct __integral_constant {
  static constexpr int value = V;
  constexpr operator int() const { return V; }
};

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (round to nearest even; one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v_t));
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(__integral_constant<N - 1>());
  }
}

__device__ __forceinline__ float xor32(float x) {
  // value of lane l ^ 32 (permlane32 swap of x with itself)
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? p[0] : p[1]);
}

// LDS swizzle: 16-byte chunk c of key row k is stored at chunk c ^ swz(k).
// gfx950 serves 256 bytes of LDS per clock (64 banks), i.e. 16 lanes of a
// 16-byte read or 32 lanes of an 8-byte read at a time.  For 256-byte rows
// (head_dim 128) swz(k) = (k & 3) << 2 | (k >> 2) & 3 is a bijection on k mod
// 16, so the 16 consecutive key rows of a K-operand read land in 16 different
// 16-byte bank groups, and the 4 rows x 4 chunks of a 32-lane transposed V
// read (rows differing in k & 3) land in 16 different groups too.  For
// 128-byte rows (head_dim 64) two rows share a bank row and swz(k) = (k >> 1)
// & 7 separates 16 consecutive rows.
template <int CPR>
__device__ __forceinline__ int swz(int key) {
  if constexpr (CPR == 16) return ((key & 3) << 2) | ((key >> 2) & 3);
  else return (key >> 1) & 7;
}

// Lazy rescale threshold (log2 units): the running max used for the
// exponentials is only raised when a row's tile max exceeds it by more than
// this, so probabilities stay below 2^8 and are exact in fp32/bf16 range;
// numerator and denominator share the same max, so the result is unchanged.
constexpr float kRescaleSlack = 8.f;

template <int D, int G>
struct ChunkGeo {
  static constexpr int ROWB = D * 2;        // bytes per key row (one head)
  static constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  static constexpr int KSTEPS = D / 16;     // MFMA k-steps for q.k
  static constexpr int DB = D / 32;         // 32-wide d blocks of O
  static constexpr int TQ = kChunkRows / G;
  static constexpr int TILE_BYTES = KT * ROWB;
  static constexpr int LOADS = KT * CPR / kThreads;  // 16-byte chunks per thread per tile
};

template <int D, int G>
struct ChunkState {
  using Gm = ChunkGeo<D, G>;
  f32x16_t o[Gm::DB];
  float m_run;
  float l_run;
};

typedef const __attribute__((address_space(3))) char* lds_cptr;


// S^T = K Q^T for one 64-key tile: two 32-key halves, KSTEPS k-steps each.
// The K fragments are read from the swizzled LDS tile two k-steps ahead of
// the MFMAs that use them.
template <int D, int G>
__device__ __forceinline__ void chunk_qk(f32x16_t (&s)[2], lds_cptr kbuf,
                                         const u32x4_t (&qf)[ChunkGeo<D, G>::KSTEPS],
                                         const int (&koff)[ChunkGeo<D, G>::KSTEPS]) {
  using Gm = ChunkGeo<D, G>;
  constexpr int ROWB = Gm::ROWB, KSTEPS = Gm::KSTEPS;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int e = 0; e < 16; ++e) s[sub][e] = 0.f;
  }
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const u32x4_t kv = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(
          kbuf + koff[kk] + sub * 32 * ROWB);
      s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv),
                                                       __builtin_bit_cast(bf16x8_t, qf[kk]),
                                                       s[sub], 0, 0, 0);
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
  for (int kk = 0; kk < KSTEPS - 2; ++kk) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

// Mask (diagonal / segment-end tiles only), lazy online-softmax update and
// the tile's probabilities as bf16 pairs in the MFMA operand order.  The row
// max is a three-input max tree over the lane's 32 scores plus one
// permlane32 swap with the partner lane that holds the row's other keys; the
// scale (times log2 e) is applied in fp32 in the exponent's argument.
template <int D, int G>
__device__ __forceinline__ void chunk_softmax(ChunkState<D, G>& st, f32x16_t (&s)[2],
                                              uint32_t (&pk)[2][8], int kt, int qpos, int k1,
                                              int w_qpos_lo, float sl, int lane) {
  using Gm = ChunkGeo<D, G>;
  constexpr int DB = Gm::DB;
  const int grp = lane >> 5;
  if (kt + KT - 1 > w_qpos_lo || kt + KT > k1) {
    // keys < lim (relative to kt) are visible; element e of half sub holds
    // key sub*32 + 8(e/4) + 4 grp + e%4, so the lane's 4 grp moves to the
    // limit and every comparison is against an inline constant
    const int limg = min(qpos + 1, k1) - kt - 4 * grp;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        s[sub][e] = (sub * 32 + 8 * (e >> 2) + (e & 3)) < limg ? s[sub][e] : kNegInf;
  }
  float t[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int a = 3 * i, b = 3 * i + 1, c = 3 * i + 2;
    t[i] = max3f(s[a >> 4][a & 15], s[b >> 4][b & 15], s[c >> 4][c & 15]);
  }
  t[10] = fmaxf(s[1][14], s[1][15]);
  float mx = max3f(max3f(t[0], t[1], t[2]), max3f(t[3], t[4], t[5]),
                   max3f(t[6], t[7], fmaxf(t[8], fmaxf(t[9], t[10]))));
  {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1])) * sl;
  }
  if (__builtin_amdgcn_ballot_w64(mx > st.m_run + kRescaleSlack)) {
    // some row's max grew past the slack: move every row to its true max
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) st.o[db][e] *= alpha;
  }
  const float m_use = st.m_run == kNegInf ? 0.f : st.m_run;
  float psum = 0.f;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][e], sl, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][e + 1], sl, -m_use));
      pk[sub][e >> 1] = pack_bf16(p0, p1);
      // row sum of the bf16-rounded probabilities (the ones p.v uses)
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[sub][e >> 1]),
                                             __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
    }
  st.l_run += psum;
}

// O^T += V^T P^T for one tile: V^T fragments by transposed LDS reads.
template <int D, int G>
__device__ __forceinline__ void chunk_pv(ChunkState<D, G>& st, lds_cptr vbuf,
                                         const uint32_t (&pk)[2][8],
                                         const int (&voff)[ChunkGeo<D, G>::DB],
                                         const int (&voff8)[ChunkGeo<D, G>::DB]) {
  using Gm = ChunkGeo<D, G>;
  constexpr int ROWB = Gm::ROWB, DB = Gm::DB;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t pw = {pk[sub][4 * h], pk[sub][4 * h + 1], pk[sub][4 * h + 2], pk[sub][4 * h + 3]};
      const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
      const int rowoff = (sub * 32 + 16 * h) * ROWB;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(vbuf + voff[db] + rowoff));
        const s16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(vbuf + voff8[db] + rowoff));
        const s16x8_t vv = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
        st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pf,
                                                           st.o[db], 0, 0, 0);
      }
    }
}

// One whole 64-key tile in order: q.k, softmax, p.v.
template <int D, int G>
__device__ __forceinline__ void chunk_tile(ChunkState<D, G>& st, lds_cptr kbuf, lds_cptr vbuf,
                                           const u32x4_t (&qf)[ChunkGeo<D, G>::KSTEPS],
                                           const int (&koff)[ChunkGeo<D, G>::KSTEPS],
                                           const int (&voff)[ChunkGeo<D, G>::DB],
                                           const int (&voff8)[ChunkGeo<D, G>::DB], int kt,
                                           int qpos, int k1, int w_qpos_lo, float sl, int lane) {
  f32x16_t s[2];
  uint32_t pk[2][8];
  chunk_qk<D, G>(s, kbuf, qf, koff);
  chunk_softmax<D, G>(st, s, pk, kt, qpos, k1, w_qpos_lo, sl, lane);
  chunk_pv<D, G>(st, vbuf, pk, voff, voff8);
}

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 512 / kThreads) chunk_kernel(AttnArgs a) {
  using Gm = ChunkGeo<D, G>;
  constexpr int ROWB = Gm::ROWB, CPR = Gm::CPR, KSTEPS = Gm::KSTEPS, DB = Gm::DB, TQ = Gm::TQ;
  constexpr int TILE_BYTES = Gm::TILE_BYTES, LOADS = Gm::LOADS;
  static_assert(LOADS >= 1, "tile too small");

  // double-buffered K and V tiles (four distinct LDS objects, so reads of one
  // buffer need not wait for the DMA into the other) and the segment's block ids
  __shared__ __attribute__((aligned(1024))) char k_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_lds1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_lds1[TILE_BYTES];
  __shared__ int32_t bt_lds[kMaxSegBlocks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // XCD-aware work assignment: workgroups are dispatched round-robin over the
  // 8 XCDs (linear id % 8), so XCD x runs ids x, x+8, ...  Work unit
  // u = g * n_ck + item (items ordered request, segment, q-tile) is given to
  // XCD u / per_xcd, in order: every XCD gets a contiguous range of units and
  // the q-tiles that read the same K/V segment share that XCD's L2.
  const int per_xcd = (int)(gridDim.x / kXcds);
  const int u = ((int)blockIdx.x % kXcds) * per_xcd + (int)blockIdx.x / kXcds;
  if (u >= a.ps.n_ck * a.Hkv) return;
  const int g = u / a.ps.n_ck;
  const int4 it = a.items_ck[u - g * a.ps.n_ck];
  const int r = it.x;
  const int qt = it.y, seg = it.z, part_base = it.w;
  if (r < 0 || r >= a.R || qt < 0 || seg < 0) return;

  int q = a.qsl[r + 1] - a.qsl[r];
  int L = a.seq_lens[r];
  sanitize(q, L, a.M, a.B);
  const int t0 = a.qsl[r];
  const int c = L - q;
  const int tok0 = qt * TQ;
  const int tok_end = min(tok0 + TQ, q);
  const int kmax = c + tok_end;                 // exclusive key bound of the tile
  const int k0 = seg * a.ps.SEG;
  const int k1 = min(k0 + a.ps.SEG, kmax);
  if (tok0 >= q || k0 >= k1) return;

  // block ids of the segment into LDS (one-time divisions)
  const int blk_first = k0 / a.B;
  const int nblk = (k1 - 1) / a.B - blk_first + 1;
  for (int i = tid; i < nblk && i < kMaxSegBlocks; i += kThreads) {
    int b = a.block_table[(int64_t)r * a.M + blk_first + i];
    bt_lds[i] = b < 0 ? 0 : (b >= a.num_blocks ? a.num_blocks - 1 : b);
  }

  // this lane's query row
  const int rho = wave * 32 + (lane & 31);
  const int h_local = rho / TQ;
  const int tau = rho % TQ;
  const bool row_ok = tok0 + tau < q;
  const int qpos = row_ok ? c + tok0 + tau : -1;
  const int hq = g * G + h_local;
  // the wave's rows cover tokens tok0 + [tau_lo, tau_hi]
  const int w_tau_lo = (wave * 32) % TQ;
  const int w_tau_hi = min(w_tau_lo + 31, TQ - 1);
  const int w_qpos_lo = c + tok0 + w_tau_lo;
  const int w_qpos_hi = c + min(tok0 + w_tau_hi, q - 1);

  // Q fragment (B operand of S^T = K Q^T): lane holds d = 16kk + 8(lane/32) .. +8
  u32x4_t qf[KSTEPS];
  {
    const char* qrow = static_cast<const char*>(a.query) +
                       ((int64_t)(t0 + tok0 + tau) * a.Hq + hq) * ROWB + (lane >> 5) * 16;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[kk] = row_ok ? *reinterpret_cast<const u32x4_t*>(qrow + kk * 32) : u32x4_t{0, 0, 0, 0};
  }
  // lane-constant LDS read offsets within a tile buffer
  const int l32 = lane & 31, grp = lane >> 5, gam = lane >> 4, li = lane & 15;
  int koff[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) koff[kk] = l32 * ROWB + (((2 * kk + grp) ^ swz<CPR>(l32)) << 4);
  // rows r and r + 8 of a transposed read have different swizzles, so the
  // second read of each pair has its own lane offset
  int voff[DB], voff8[DB];
  {
    const int row = 4 * grp + (li >> 2);                 // row m of the 4-row transposed block
    const int d0_in = 16 * (gam & 1) + 4 * (li & 3);     // d offset within the 32-wide block
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int d0 = db * 32 + d0_in;
      voff[db] = row * ROWB + (((d0 >> 3) ^ swz<CPR>(row)) << 4) + (d0 & 7) * 2;
      voff8[db] = (row + 8) * ROWB + (((d0 >> 3) ^ swz<CPR>(row + 8)) << 4) + (d0 & 7) * 2;
    }
  }
  __syncthreads();  // bt_lds ready

  // Tile loads are direct global -> LDS DMA (global_load_lds_dwordx4): lane l
  // of a wave instruction writes 16 bytes at LDS base + 16 l, so each
  // instruction fills RPK = 1024 / ROWB consecutive key rows; lane l takes
  // row l / CPR, physical chunk l % CPR, and fetches logical chunk
  // (l % CPR) ^ swz(row) of that row from the cache, which realises the
  // swizzled layout.  Wave w loads the tile's rows WROWS w .. WROWS w + WROWS-1
  // (WROWS = 64 / waves, 8 or 16).  The block size is a multiple of 16 and
  // tiles start at multiples of 64 keys, so those rows lie in one cache block:
  // the block's address is wave-uniform (scalar registers) and each lane adds
  // a fixed 32-bit offset.
  constexpr int RPK = 1024 / ROWB;
  constexpr int WROWS = KT / kWaves;       // rows of a tile one wave loads
  static_assert(LOADS * RPK == WROWS && WROWS % 8 == 0, "a wave loads WROWS rows per tile");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const char* kcache = static_cast<const char*>(a.kcache);
  const char* vcache = static_cast<const char*>(a.vcache);
  const uint32_t block_bytes = (uint32_t)a.B * a.Hkv * ROWB;
  const int slot_stride = a.Hkv * ROWB;
  const int lb = 31 - __builtin_clz(a.B);   // block size is a power of two here
  const int bmask = a.B - 1;
  int ld_rl[LOADS], ld_off[LOADS];          // row within the wave's 16, lane offset
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int rl = i * RPK + lane / CPR;
    ld_rl[i] = rl;
    ld_off[i] = rl * slot_stride + g * ROWB + (((lane % CPR) ^ swz<CPR>(wave * WROWS + rl)) << 4);
  }
  typedef __attribute__((address_space(3))) void* lds_vptr;
  // The block id is read from LDS before the DMAs are issued: the compiler
  // cannot tell that read from the DMA's LDS writes apart and would otherwise
  // wait for the earlier DMAs to land.  In the segment's last tile a wave
  // whose rows pass the segment end starts at the last valid 16-row group and
  // clamps its rows to the last valid key (masked rows then hold finite
  // values).
#define PA_CK_DMA(KT0, KB, VB)                                                                  \
  {                                                                                             \
    const int wr0 = (KT0) + wave_u * WROWS;                                                     \
    const bool wfull = wr0 + WROWS <= k1;                                                       \
    const int wrow = wfull ? wr0 : min(wr0, (k1 - 1) & ~(WROWS - 1));                           \
    const uint32_t blk = (uint32_t)__builtin_amdgcn_readfirstlane(bt_lds[(wrow >> lb) - blk_first]); \
    const uint64_t sb = (uint64_t)blk * block_bytes + (uint32_t)((wrow & bmask) * slot_stride); \
    int off[LOADS];                                                                             \
    static_for<LOADS>([&](auto I) {                                                             \
      constexpr int i = I;                                                                      \
      off[i] = ld_off[i];                                                                       \
      if (!wfull) {                                                                             \
        const int over = wrow + ld_rl[i] - (k1 - 1);                                            \
        off[i] -= (over > 0 ? over : 0) * slot_stride;                                          \
      }                                                                                         \
    });                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    static_for<LOADS>([&](auto I) {                                                             \
      constexpr int i = I;                                                                      \
      __builtin_amdgcn_global_load_lds(kcache + sb + (uint32_t)off[i],                         \
                                       (lds_vptr)((KB) + (wave_u * LOADS + i) * 1024), 16, 0, 0); \
      __builtin_amdgcn_global_load_lds(vcache + sb + (uint32_t)off[i],                         \
                                       (lds_vptr)((VB) + (wave_u * LOADS + i) * 1024), 16, 0, 0); \
    });                                                                                         \
  }

  ChunkState<D, G> st;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.o[db][e] = 0.f;
  st.m_run = kNegInf;   // in log2 units (score * scale * log2 e)
  st.l_run = 0.f;       // this lane's share of the row sum
  const float sl = a.scale_log2;

  const int n_tiles = (k1 - k0 + KT - 1) / KT;
  const lds_cptr kb0 = (lds_cptr)k_lds0, kb1 = (lds_cptr)k_lds1;
  const lds_cptr vb0 = (lds_cptr)v_lds0, vb1 = (lds_cptr)v_lds1;
  // vmcnt(0), expcnt/lgkmcnt unconstrained: this wave's DMA into LDS is done
  constexpr int kWaitDma = 0x0F70;
  PA_CK_DMA(k0, k_lds0, v_lds0)
  for (int ti = 0; ti < n_tiles; ti += 2) {
    // even tile: buffer 0.  Wait for its DMA, then a barrier makes every
    // wave's part visible and guarantees buffer 1 is no longer being read.
    {
      const int kt = k0 + ti * KT;
      __builtin_amdgcn_s_waitcnt(kWaitDma);
      __syncthreads();
      if (ti + 1 < n_tiles) { PA_CK_DMA(kt + KT, k_lds1, v_lds1) }
      if (kt <= w_qpos_hi)
        chunk_tile<D, G>(st, kb0, vb0, qf, koff, voff, voff8, kt, qpos, k1, w_qpos_lo, sl, lane);
    }
    if (ti + 1 < n_tiles) {  // odd tile: buffer 1
      const int kt = k0 + (ti + 1) * KT;
      __builtin_amdgcn_s_waitcnt(kWaitDma);
      __syncthreads();
      if (ti + 2 < n_tiles) { PA_CK_DMA(kt + KT, k_lds0, v_lds0) }
      if (kt <= w_qpos_hi)
        chunk_tile<D, G>(st, kb1, vb1, qf, koff, voff, voff8, kt, qpos, k1, w_qpos_lo, sl, lane);
    }
  }
#undef PA_CK_DMA

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = st.l_run + xor32(st.l_run);
  if (!row_ok) return;
  const int t = t0 + tok0 + tau;
  if (part_base < 0) {
    const float inv = 1.f / l_tot;
    char* orow = static_cast<char*>(a.out) + ((int64_t)t * a.Hq + hq) * ROWB;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * grp;
        const uint2 w = make_uint2(pack_bf16(st.o[db][4 * e4] * inv, st.o[db][4 * e4 + 1] * inv),
                                   pack_bf16(st.o[db][4 * e4 + 2] * inv, st.o[db][4 * e4 + 3] * inv));
        *reinterpret_cast<uint2*>(orow + d * 2) = w;
      }
  } else {
    const int64_t slot = (int64_t)part_base + (int64_t)seg * TQ + tau;
    float* op = a.o_part + (slot * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = db * 32 + 8 * e4 + 4 * grp;
        *reinterpret_cast<float4*>(op + d) =
            make_float4(st.o[db][4 * e4], st.o[db][4 * e4 + 1], st.o[db][4 * e4 + 2], st.o[db][4 * e4 + 3]);
      }
    if (grp == 0) {
      float* mp = a.ml_part + (slot * a.Hq + hq) * 2;
      mp[0] = st.m_run;
      mp[1] = l_tot;
    }
  }
}



}  // namespace

bool chunk_kernel_supports(bool bf16, int32_t D, int32_t G, int32_t B) {
  return bf16 && (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8) &&
         (B & (B - 1)) == 0;
}

int32_t chunk_max_segment(int32_t B) { return kMaxSegBlocks * B - B; }

hipError_t launch_chunk(const AttnArgs& a, hipStream_t s) {
  if (a.ps.n_ck == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  const void* kern = nullptr;
#define PA_CK(DD, GG) \
  if (a.D == DD && G == GG) { kern = (const void*)chunk_kernel<DD, GG>; }
  PA_CK(64, 1) PA_CK(64, 2) PA_CK(64, 4) PA_CK(64, 8)
  PA_CK(128, 1) PA_CK(128, 2) PA_CK(128, 4) PA_CK(128, 8)
#undef PA_CK
  if (kern == nullptr) return hipErrorInvalidValue;
  AttnArgs args = a;
  void* params[] = {&args};
  const int64_t units = (int64_t)a.ps.n_ck * a.Hkv;
  const int64_t per_xcd = (units + kXcds - 1) / kXcds;
  return hipLaunchKernel(kern, dim3((unsigned)(per_xcd * kXcds)), dim3(kThreads), params, 0, s);
}

}  // namespace pa
