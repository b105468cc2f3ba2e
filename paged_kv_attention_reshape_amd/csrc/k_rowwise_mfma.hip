// Split-K row-wise attention on the matrix cores, for bf16 caches and GQA
// groups of 4 or 8 query heads per kv head.
//
// Method: "AI Infra入门干货总结：大模型是如何高效推理的", section "Attention
// Module": the G query heads that share a kv head read one K/V stream through
// the block table; online softmax (running max and sum) fuses q.k, softmax
// and p.v; section "总结": Flash-Decoding splits the keys of a row into
// partitions that a log-sum-exp pass merges.  The plan gives each work item
// one query row and its key range [kb, ke) (the causal limit of "Chunked
// Prefill 与 Preemption", equation M_{i,j}, is already in ke).
//
// Why matrix cores for a bandwidth-bound pass: with 8 query heads per kv head
// the q.k and p.v dot products of the vector-ALU kernel (v_dot2, 16 tokens x
// G heads per lane group) take about as long as streaming the keys and
// values, so the kernel runs below the HBM rate.  Here every 32-key tile is
// 16 MFMAs (v_mfma_f32_16x16x32_bf16, query heads padded to 16 columns) and
// about 40 vector instructions of softmax per wave, far below the time the
// tile's 16 KB take to arrive.
//
// Two forms.  The whole-block form (the default with head_dim 128 and 1, 2,
// 4 or 8 kv heads; rowwise_mfma_block_kernel below) gives an item one
// workgroup of Hkv waves reading 16-key slabs of all kv heads from LDS.  The
// per-head form (rowwise_mfma_kernel) gives each (row, key partition, kv head)
// one wavefront that streams its own rows; lane l = (grp = l / 16,
// li = l % 16):
//   S^T = K Q^T : A = K rows of the tile straight from global memory (lane
//                 holds key li of a 16-key half, d 32s + 8grp .. +7), B = the
//                 query heads (column li, zero for li >= G) held in registers;
//                 the accumulator gives lane l the scores of head li for keys
//                 4grp + r and 16 + 4grp + r, r < 4.
//   softmax     : per head over those 8 keys and the 4 lane groups (two
//                 cross-group shuffles); running max raised lazily (only past
//                 a 2^8 slack), probabilities rounded to bf16 in place.
//   O^T = V^T P^T: B = the lane's own 8 probabilities (the MFMA k-slot order
//                 is permuted to the score layout, so P never moves), A = V^T
//                 by ds_read_b64_tr_b16 transposed reads of the V tile, which
//                 the wave writes into an XOR-swizzled LDS buffer (1 KB per
//                 ds_write_b128 instruction).  O^T keeps head li per lane, so
//                 the rescale is lane-local.
// K and V are streamed into registers with the nontemporal hint (each byte is
// read once per step); the next tile's loads are issued right after the
// current tile's q.k, so they are in flight during its softmax and p.v.  V
// goes through registers rather than a global->LDS DMA: with only ordinary
// loads in flight the compiler's vmcnt waits stay exact (mixing in LDS DMA
// makes it wait for every outstanding load).  Partial results use the same
// layout as the vector kernel's, so the merge pass is shared.
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef const __attribute__((address_space(3))) char* lds_cptr;

constexpr int KT = 32;  // keys per tile
constexpr int kLdsPerWave = 20 * 1024;
constexpr float kNegInf = -__builtin_huge_valf();
// lazy rescale threshold (log2 units): probabilities stay below 2^8
constexpr float kSlack = 8.f;

template <int D>
struct MGeo {
  static constexpr int ROWB = D * 2;              // bytes of one head row
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  static constexpr int KSTEPS = D / 32;           // k-steps of q.k
  static constexpr int NB = D / 16;               // 16-wide d blocks of O^T
  static constexpr int TILE_BYTES = KT * ROWB;    // one V tile
  static constexpr int VL = TILE_BYTES / 1024;    // 16-byte V loads per lane per tile
  static constexpr int RPV = 1024 / ROWB;         // V rows per wave load instruction
};

// V tile swizzle: 16-byte chunk c of row k sits at chunk c ^ vswz(k).  A
// transposed read covers 16 rows x 32 bytes (chunks 2n, 2n+1); with 256-byte
// rows vswz = 2 (k & 7) spreads rows k, k + 8 over all 16 bank groups twice,
// with 128-byte rows (two rows per 256-byte bank row) vswz = 2 ((k >> 1) & 3).
template <int CPR>
__device__ __forceinline__ int vswz(int k) {
  if constexpr (CPR == 16) return (k & 7) << 1;
  else return ((k >> 1) & 3) << 1;
}

__device__ __forceinline__ u32x4_t load_once(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(a, fmaxf(b, c)); }

__device__ __forceinline__ float xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? p[0] : p[1]);
}

__device__ __forceinline__ float xor16(float x) { return __shfl_xor(x, 16, 64); }

template <int D, int G>
__global__ void __launch_bounds__(64, 2) rowwise_mfma_kernel(AttnArgs a) {
  using Gm = MGeo<D>;
  constexpr int ROWB = Gm::ROWB, CPR = Gm::CPR, KSTEPS = Gm::KSTEPS, NB = Gm::NB;
  constexpr int TILE_BYTES = Gm::TILE_BYTES, VL = Gm::VL, RPV = Gm::RPV;
  static_assert(G >= 1 && G <= 16, "query heads per kv head must fit 16 MFMA columns");

  // one V tile (the first TILE_BYTES); a wave's LDS accesses execute in
  // order, so the next tile's writes cannot overtake this tile's reads.  The
  // array is sized to kLdsPerWave so that at most eight of these waves share
  // a compute unit (160 KB of LDS): measured faster than the twelve its
  // 168 registers would allow (fewer concurrent K/V streams per HBM channel).
  __shared__ __attribute__((aligned(1024))) char v_lds[kLdsPerWave];
  static_assert(TILE_BYTES <= kLdsPerWave, "V tile does not fit");

  const int lane = threadIdx.x;
  const int li = lane & 15, grp = lane >> 4;
  const int4 it = a.items_rw[blockIdx.x];
  const int r = it.x;
  if (r < 0 || r >= a.R) return;
  const int g = blockIdx.y;
  const int t = it.y;
  const int kb = it.z;
  const int ke = it.w & 0x7FFFFFFF;
  const bool direct = (it.w & kDirect) != 0;
  const int slot = direct ? 0 : a.rw_slot[blockIdx.x];
  if (ke <= kb) return;

  // Q^T fragments (B operand of S^T = K Q^T): column li = query head g*G + li
  u32x4_t qf[KSTEPS];
  {
    const int hh = li < G ? li : G - 1;
    const char* qrow = static_cast<const char*>(a.query) + ((int64_t)t * a.Hq + g * G + hh) * ROWB + grp * 16;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = li < G ? *reinterpret_cast<const u32x4_t*>(qrow + s * 64) : u32x4_t{0, 0, 0, 0};
  }

  // physical block ids of the partition: lane i holds block kb / B + i
  const int blk0 = kb / a.B;
  const int nblk = (ke - 1) / a.B - blk0 + 1;
  int myblk = 0;
  if (lane < nblk) {
    myblk = a.block_table[(int64_t)r * a.M + blk0 + lane];
    myblk = myblk < 0 ? 0 : (myblk >= a.num_blocks ? a.num_blocks - 1 : myblk);
  }
  const char* kcache = static_cast<const char*>(a.kcache) + (int64_t)g * ROWB;
  const char* vcache = static_cast<const char*>(a.vcache) + (int64_t)g * ROWB;
  const uint32_t slot_stride = (uint32_t)a.Hkv * ROWB;

  // byte offset (from the head's base) of key `key` of the partition, which
  // lies in physical block `blk`; `key` must lie in [kb, ke)
  auto key_off = [&](int key, int blk) -> int64_t {
    return ((int64_t)blk * a.B + key % a.B) * slot_stride;
  };
  // lane offset of K chunk 4k + grp of row li within a 16-row half: koff + 64 k
  const uint32_t koff = li * slot_stride + grp * 16;
  // V load i of a lane: the 16 bytes that belong at LDS byte 1024 i + 16 lane
  // (physical row RPV i + lane / CPR, physical chunk lane % CPR, which holds
  // logical chunk (lane % CPR) ^ vswz(row)).  The swizzle of row RPV i + x
  // repeats with period VP in i, so the lane part takes VP registers and the
  // rest, ((RPV i) mod 16) rows, is a constant.
  constexpr int VP = CPR == 16 ? 2 : 1;
  uint32_t vlane[VP];
#pragma unroll
  for (int j = 0; j < VP; ++j) {
    const int pr = RPV * j + lane / CPR;
    vlane[j] = (lane / CPR) * slot_stride + (((lane % CPR) ^ vswz<CPR>(pr)) << 4);
  }
  auto vgoff = [&](int i) -> uint32_t { return ((RPV * i) & 15) * slot_stride + vlane[i % VP]; };
  // transposed reads: row 4 grp + li / 4 (and + 16), d 16n + 4 (li % 4), i.e.
  // chunk 2n + (li / 2) % 2 (swizzled) and byte 8 (li % 2) within it; the
  // swizzle is even, so chunk 2n + b lands at 2 (n ^ sw / 2) + b
  const int vrow = 4 * grp + (li >> 2);
  const int vsw = vswz<CPR>(vrow) >> 1;
  const int vbase = vrow * ROWB + ((li >> 1) & 1) * 16 + (li & 1) * 8;
  auto voff = [&](int n) -> int { return vbase + ((n ^ vsw) << 5); };

  // K rows (A operand: key li of half h) and V chunks of a tile into
  // registers.  A full tile uses one scalar base per 16-key half (a half
  // never crosses a block: B and the tile start are multiples of 16); the
  // last, partial tile clamps its rows to key ke - 1 (finite data; those keys
  // are masked and get zero probability).  Both paths issue the same loads.
  auto load_full = [&](int start, u32x4_t (&kr)[2][KSTEPS], u32x4_t (&vr)[VL]) {
    const int64_t base0 = key_off(start, __builtin_amdgcn_readlane(myblk, start / a.B - blk0));
    const int64_t base1 = key_off(start + 16, __builtin_amdgcn_readlane(myblk, (start + 16) / a.B - blk0));
#pragma unroll
    for (int k = 0; k < KSTEPS; ++k) {
      kr[0][k] = load_once(kcache + base0 + koff + 64 * k);
      kr[1][k] = load_once(kcache + base1 + koff + 64 * k);
    }
#pragma unroll
    for (int i = 0; i < VL; ++i) vr[i] = load_once(vcache + ((RPV * i < 16) ? base0 : base1) + vgoff(i));
  };
  auto load_tile = [&](int start, u32x4_t (&kr)[2][KSTEPS], u32x4_t (&vr)[VL]) {
    if (start + KT <= ke) {
      load_full(start, kr, vr);
    } else {
      auto row_off = [&](int row) -> int64_t {
        const int key = min(start + row, ke - 1);
        const int blk = __shfl(myblk, key / a.B - blk0, 64);
        return key_off(key, blk);
      };
      const int64_t o0 = row_off(li), o1 = row_off(16 + li);
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k) {
        kr[0][k] = load_once(kcache + o0 + (4 * k + grp) * 16);
        kr[1][k] = load_once(kcache + o1 + (4 * k + grp) * 16);
      }
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const int pr = RPV * i + lane / CPR;
        const int lc = (lane % CPR) ^ vswz<CPR>(pr);
        vr[i] = load_once(vcache + row_off(pr) + lc * 16);
      }
    }
  };

  const float sl = a.scale_log2;
  float m_run = kNegInf, l_run = 0.f;
  f32x4_t o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // The steady-state loop prefetches full tiles only and unconditionally,
  // so the compiler's vmcnt waits stay exact and the two load paths are not
  // merged into one with per-lane 64-bit addresses; the last two tiles (the
  // partial one among them) follow straight-line.
  const int n_tiles = (ke - kb + KT - 1) / KT;
  u32x4_t kr[2][KSTEPS], vr[VL];
  auto tile_step = [&](int start, auto&& prefetch) {
    // V tile into LDS (swizzled; 1 KB per instruction, conflict-free)
#pragma unroll
    for (int i = 0; i < VL; ++i)
      *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(
          (__attribute__((address_space(3))) char*)v_lds + i * 1024 + lane * 16) = vr[i];
    // S^T = K Q^T
    f32x4_t s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      s[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KSTEPS; ++k)
        s[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kr[h][k]),
                                                       __builtin_bit_cast(bf16x8_t, qf[k]), s[h], 0, 0, 0);
    }
    // next tile's loads, in flight during this tile's softmax and p.v
    prefetch();
    if (start + KT > ke) {
      // element r of half h is key 16h + 4grp + r of the tile
      const int lim = ke - start - 4 * grp;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[h][e] = (16 * h + e) < lim ? s[h][e] : kNegInf;
    }
    float mx = max3f(max3f(s[0][0], s[0][1], s[0][2]), max3f(s[0][3], s[1][0], s[1][1]),
                     fmaxf(s[1][2], s[1][3]));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx)) * sl;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) o[n] *= alpha;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    uint32_t pk[4];
    float psum = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][e], sl, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[h][e + 1], sl, -m_use));
        pk[2 * h + (e >> 1)] = pack_bf16(p0, p1);
        // the sum takes the bf16-rounded probabilities that p.v uses
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[2 * h + (e >> 1)]),
                                               __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
      }
    l_run += psum;
    // O^T += V^T P^T
    const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    lds_cptr vb = (lds_cptr)v_lds;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + voff(n)));
      const s16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vb + voff(n) + 16 * ROWB));
      const s16x8_t vv = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
      o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, vv), pf, o[n], 0, 0, 0);
    }
    };
  load_tile(kb, kr, vr);
  int tile = 0;
  for (; tile + 2 < n_tiles; ++tile) {
    const int s0 = kb + tile * KT;
    tile_step(s0, [&] { load_full(s0 + KT, kr, vr); });
  }
  const int s0 = kb + tile * KT;
  if (tile + 1 < n_tiles) {
    tile_step(s0, [&] { load_tile(s0 + KT, kr, vr); });
    tile_step(s0 + KT, [] {});
  } else {
    tile_step(s0, [] {});
  }

  // ---- finish ------------------------------------------------------------------
  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
  if (li >= G) return;
  const int hq = g * G + li;
  if (direct) {
    const float inv = 1.f / l_tot;
    char* orow = static_cast<char*>(a.out) + ((int64_t)t * a.Hq + hq) * ROWB;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int d = 16 * n + 4 * grp;
      *reinterpret_cast<uint2*>(orow + d * 2) =
          make_uint2(pack_bf16(o[n][0] * inv, o[n][1] * inv), pack_bf16(o[n][2] * inv, o[n][3] * inv));
    }
  } else {
    float* op = a.o_part + ((int64_t)slot * a.Hq + hq) * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      *reinterpret_cast<float4*>(op + 16 * n + 4 * grp) = make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
    if (grp == 0) {
      float* mp = a.ml_part + ((int64_t)slot * a.Hq + hq) * 2;
      mp[0] = m_run;
      mp[1] = l_tot;
    }
  }
}


// Whole-block form (head_dim 128): one workgroup of HKV waves per item, wave
// g computing kv head g, with the item's keys staged 16 tokens at a time as
// slabs of all kv heads in an LDS double buffer (see slab_dma); reading each
// block whole is what the whole-block vector kernel showed to stream faster.
// Per 16-key slab and wave:
//   S^T = K Q^T : four v_mfma_f32_16x16x32_bf16, A = K rows read from the
//                 slab (lane: key li, d 32s + 8grp .. +7, one ds_read_b128),
//                 B = the query heads as in the per-head kernel; lane l gets
//                 the scores of head li for keys 4grp + r, r < 4.
//   softmax     : over those 4 keys and the 4 lane groups; lazily raised max.
//   O^T = V^T P^T: v_mfma_f32_16x16x16_bf16 per 16-wide d block, B = the
//                 lane's own 4 probabilities (already in the B layout: key
//                 slots 4grp + r, head li), A = V^T by one ds_read_b64_tr_b16
//                 per block from the slab (row 4grp + li/4, d 16n + 4(li%4)
//                 give lane (li, grp) the values V[4grp + r][16n + li]).
// In the last, partial slab, keys at or past the partition end get score
// -inf and their V values are zeroed (the slab may hold NaN there).
template <int G, int HKV>
__global__ void __launch_bounds__(64 * HKV) rowwise_mfma_block_kernel(AttnArgs a) {
  constexpr int D = 128;
  using Gm = MGeo<D>;
  constexpr int ROWB = Gm::ROWB, CPR = Gm::CPR, KSTEPS = Gm::KSTEPS, NB = Gm::NB;
  constexpr int SLAB = kSlabTokens * HKV * ROWB;
  constexpr int DMA_PER_WAVE = SLAB / 1024 / HKV;
  static_assert(CPR == 16 && DMA_PER_WAVE * 1024 * HKV == SLAB, "slab geometry");
  static_assert(G >= 1 && G <= 16, "query heads per kv head must fit 16 MFMA columns");
  __shared__ __attribute__((aligned(1024))) char k_lds0[SLAB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[SLAB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[SLAB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[SLAB];

  const int lane = threadIdx.x & 63;
  const int li = lane & 15, grp = lane >> 4;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int4 it = a.items_rw[blockIdx.x];
  const int r = it.x;
  if (r < 0 || r >= a.R) return;
  const int t = it.y;
  const int kb = it.z;
  const int ke = it.w & 0x7FFFFFFF;
  const bool direct = (it.w & kDirect) != 0;
  const int slot = direct ? 0 : a.rw_slot[blockIdx.x];
  if (ke <= kb) return;

  // Q^T fragments (B operand of S^T = K Q^T): column li = query head g*G + li
  u32x4_t qf[KSTEPS];
  {
    const int hh = li < G ? li : G - 1;
    const char* qrow = static_cast<const char*>(a.query) + ((int64_t)t * a.Hq + g * G + hh) * ROWB + grp * 16;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s)
      qf[s] = li < G ? *reinterpret_cast<const u32x4_t*>(qrow + s * 64) : u32x4_t{0, 0, 0, 0};
  }

  const int blk0 = kb / a.B;
  const int nblk = (ke - 1) / a.B - blk0 + 1;
  int myblk = 0;
  if (lane < nblk) {
    myblk = a.block_table[(int64_t)r * a.M + blk0 + lane];
    myblk = myblk < 0 ? 0 : (myblk >= a.num_blocks ? a.num_blocks - 1 : myblk);
  }
  const char* kcache = static_cast<const char*>(a.kcache);
  const char* vcache = static_cast<const char*>(a.vcache);
  uint32_t dma_off[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i)
    dma_off[i] = slab_source_offset<HKV, CPR>((g * DMA_PER_WAVE + i) * 64 + lane);
  auto slab_base = [&](int start) -> uint64_t {
    const int blk = __builtin_amdgcn_readlane(myblk, start / a.B - blk0);
    return ((uint64_t)blk * a.B + (start % a.B)) * (uint64_t)(HKV * ROWB);
  };

  // LDS offsets: K row li of this head, chunk 4s + grp; V^T reads of block n
  // at row 4grp + li/4, logical chunk 2n + (li/2) % 2, byte 8 (li % 2)
  int koff[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) koff[s] = (li * HKV + g) * ROWB + (((4 * s + grp) ^ slab_swz(li)) << 4);
  const int vrow = 4 * grp + (li >> 2);
  const int vbase = (vrow * HKV + g) * ROWB + (li & 1) * 8;
  const int vsw = slab_swz(vrow);
  const int vhalf = (li >> 1) & 1;

  const float sl = a.scale_log2;
  float m_run = kNegInf, l_run = 0.f;
  f32x4_t o[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto subtile = [&](const char* kbuf, const char* vbuf, int start) __attribute__((always_inline)) {
    f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kbuf + koff[s]);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf),
                                                   __builtin_bit_cast(bf16x8_t, qf[s]), sc, 0, 0, 0);
    }
    const int lim = ke - start - 4 * grp;   // element e is key 4grp + e of the slab
    const bool tail = start + kSlabTokens > ke;
    if (tail) {
#pragma unroll
      for (int e = 0; e < 4; ++e) sc[e] = e < lim ? sc[e] : kNegInf;
    }
    float mx = max3f(sc[0], sc[1], fmaxf(sc[2], sc[3]));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx)) * sl;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int n = 0; n < NB; ++n) o[n] *= alpha;
    }
    const float m_use = m_run == kNegInf ? 0.f : m_run;
    uint32_t pk[2];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e], sl, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[e + 1], sl, -m_use));
      pk[e >> 1] = pack_bf16(p0, p1);
      // the sum takes the bf16-rounded probabilities that p.v uses
      psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[e >> 1]),
                                             __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
    }
    l_run += psum;
    const s16x4_t pf = __builtin_bit_cast(s16x4_t, make_uint2(pk[0], pk[1]));
    lds_cptr vb = (lds_cptr)vbuf;
    auto pv = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(vb + vbase + (((2 * n + vhalf) ^ vsw) << 4)));
        if constexpr (decltype(masked)::value) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = e < lim ? v[e] : (short)0;
        }
        o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, pf, o[n], 0, 0, 0);
      }
    };
    if (tail) pv(std::true_type{});
    else pv(std::false_type{});
  };

  const int n_tiles = (ke - kb + kSlabTokens - 1) / kSlabTokens;
  slab_dma(kcache, vcache, slab_base(kb), dma_off, k_lds0, v_lds0, g);
  for (int tile = 0; tile < n_tiles; tile += 2) {
    // even slab: buffer 0 (its DMA done by every wave; buffer 1 no longer read)
    __builtin_amdgcn_s_waitcnt(kWaitDma);
    __syncthreads();
    if (tile + 1 < n_tiles) slab_dma(kcache, vcache, slab_base(kb + 16 * (tile + 1)), dma_off, k_lds1, v_lds1, g);
    subtile(k_lds0, v_lds0, kb + 16 * tile);
    if (tile + 1 < n_tiles) {  // odd slab: buffer 1
      __builtin_amdgcn_s_waitcnt(kWaitDma);
      __syncthreads();
      if (tile + 2 < n_tiles) slab_dma(kcache, vcache, slab_base(kb + 16 * (tile + 2)), dma_off, k_lds0, v_lds0, g);
      subtile(k_lds1, v_lds1, kb + 16 * (tile + 1));
    }
  }

  // ---- finish ------------------------------------------------------------------
  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
  if (li >= G) return;
  const int hq = g * G + li;
  if (direct) {
    const float inv = 1.f / l_tot;
    char* orow = static_cast<char*>(a.out) + ((int64_t)t * a.Hq + hq) * ROWB;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const int d = 16 * n + 4 * grp;
      *reinterpret_cast<uint2*>(orow + d * 2) =
          make_uint2(pack_bf16(o[n][0] * inv, o[n][1] * inv), pack_bf16(o[n][2] * inv, o[n][3] * inv));
    }
  } else {
    float* op = a.o_part + ((int64_t)slot * a.Hq + hq) * D;
#pragma unroll
    for (int n = 0; n < NB; ++n)
      *reinterpret_cast<float4*>(op + 16 * n + 4 * grp) = make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
    if (grp == 0) {
      float* mp = a.ml_part + ((int64_t)slot * a.Hq + hq) * 2;
      mp[0] = m_run;
      mp[1] = l_tot;
    }
  }
}

}  // namespace

const void* rowwise_mfma_kernel_for(int32_t D, int32_t G) {
  if (D == 64 && G == 4) return (const void*)rowwise_mfma_kernel<64, 4>;
  if (D == 64 && G == 8) return (const void*)rowwise_mfma_kernel<64, 8>;
  if (D == 128 && G == 4) return (const void*)rowwise_mfma_kernel<128, 4>;
  if (D == 128 && G == 8) return (const void*)rowwise_mfma_kernel<128, 8>;
  return nullptr;
}

const void* rowwise_mfma_block_kernel_for(int32_t D, int32_t G, int32_t Hkv) {
  if (D != 128 || (G != 4 && G != 8)) return nullptr;
#define PA_MFMA_BLOCK_H(GG)                                                  \
  switch (Hkv) {                                                             \
    case 1: return (const void*)rowwise_mfma_block_kernel<GG, 1>;            \
    case 2: return (const void*)rowwise_mfma_block_kernel<GG, 2>;            \
    case 4: return (const void*)rowwise_mfma_block_kernel<GG, 4>;            \
    case 8: return (const void*)rowwise_mfma_block_kernel<GG, 8>;            \
    default: return nullptr;                                                 \
  }
  if (G == 4) { PA_MFMA_BLOCK_H(4) }
  PA_MFMA_BLOCK_H(8)
#undef PA_MFMA_BLOCK_H
}

}  // namespace pa
