// Split-K row-wise attention (decode rows) and the partition merge pass.
//
// Method: "AI Infra入门干货总结：大模型是如何高效推理的", section "Attention
// Module": attention reads each request's history through the block table and
// fuses q.k, softmax and the product with V using online softmax (a running
// max and running sum, rescaled when a new tile raises the max); section
// "总结": Flash-Decoding splits decode attention along the KV dimension and
// normalises the partitions with log-sum-exp.  The causal limit of a row at
// absolute position p is key p ("Chunked Prefill 与 Preemption", equation
// M_{i,j}); the plan gives each item its key range [kb, ke).
//
// MI355X design (no atomics, so results are deterministic).  The vector-ALU
// split-K kernels live here and share one sub-tile of math; the matrix-core
// ones (8 query heads per kv head) are in k_rowwise_mfma.hip, and
// decode_launch below picks among the four.  The whole-block vector kernel
// (bf16, head_dim 128, GQA groups up to 4: the default there) gives an item
// one workgroup of Hkv waves and stages each 16-token slab of all kv heads in
// LDS by DMA; the per-head kernel (every other case) gives each (item, kv
// head) one wavefront that loads its rows itself.  In both, per wave and kv
// head:
//   * the G query heads that share kv head g are processed together, so every
//     K/V byte is read from HBM exactly once per item;
//   * q.k: lanes are (token j, quarter c) pairs, 16 tokens per sub-tile; each
//     lane dots a quarter of the head dimension for all G heads with
//     v_dot2_f32_bf16 (two bf16 products per instruction, fp32 accumulate),
//     and two DPP quad permutations finish the sums.  K rows are loaded as
//     16-byte chunks, four lanes covering 64 contiguous bytes of a row;
//   * softmax: each lane owns one head of its token, so one v_exp covers 16
//     tokens x 4 heads; the max over tokens uses DPP row rotations and two
//     cross-row shuffles; the running sum stays per lane until the end;
//   * p.v: probabilities go through LDS as bf16 pairs of two tokens, V rows
//     are read with 16 lanes covering one 256-byte row (fully coalesced), and
//     v_dot2_f32_bf16 accumulates two tokens per instruction into fp32;
//   * the next sub-tile's K and V are loaded before the current one is used;
//     they are read with the nontemporal hint: each K/V byte is used once per
//     step, and streaming it past the caches keeps the split-K partials and
//     this step's freshly written rows resident (measured: the per-head read
//     pattern goes from about 5.8 to 6.2 TB/s with the hint, the whole-block
//     one from 5.9 to 6.4).
// fp32 caches use the per-head structure with plain FMAs.
#include <algorithm>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124;  // row_ror:4
constexpr int kRowRor8 = 0x128;  // row_ror:8

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of data read once (global_load_dwordx4 ... nt)
__device__ __forceinline__ uint4 load_once(const char* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

constexpr float kNegInf = -__builtin_huge_valf();

template <bool BF16, int D, int G>
struct Geo {
  static constexpr int E = BF16 ? 2 : 4;        // bytes per element
  static constexpr int ROWB = D * E;            // bytes of one head row
  static constexpr int LPR = 4;                 // q.k lanes per token
  static constexpr int NL = ROWB / (16 * LPR);  // 16-byte K loads per lane
  static constexpr int EPC = 16 / E;            // elements per 16-byte chunk
  static constexpr int LPRV = ROWB / 16;        // p.v lanes per V row
  static constexpr int RPI = 64 / LPRV;         // V rows per wave instruction
  static constexpr int RPL = 16 / RPI;          // V rows per lane per sub-tile
  static constexpr int HPL = (G + 3) / 4;       // softmax heads per lane
  static_assert(NL >= 1 && RPL >= 2 && RPL % 2 == 0, "unsupported geometry");
};

// One wave's online-softmax state for its G query heads: running max and sum
// (one head per lane in the softmax layout) and the unnormalised output slice
// of every head (p.v layout).
template <bool BF16, int D, int G>
struct WaveAcc {
  using Gm = Geo<BF16, D, G>;
  float m_run[Gm::HPL], l_run[Gm::HPL];
  float o[G][Gm::EPC];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int k = 0; k < Gm::HPL; ++k) { m_run[k] = kNegInf; l_run[k] = 0.f; }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < Gm::EPC; ++e) o[h][e] = 0.f;
  }
};

// Lane roles: (token j, quarter c) in the q.k layout, (first V row rsub,
// 16-byte chunk cv) in the p.v layout.
struct DecodeLanes {
  int lane, j, c, rsub, cv;
};
template <int LPRV>
__device__ __forceinline__ DecodeLanes decode_lanes(int lane) {
  return DecodeLanes{lane, lane >> 2, lane & 3, lane / LPRV, lane % LPRV};
}

// The probabilities and rescale factors handed from the q.k to the p.v lane
// layout through LDS are only exchanged among the lanes of one wave.  A
// workgroup of one wave orders the hand-off with its barrier; a wave of a
// larger workgroup needs no barrier with the other waves (the LDS accesses
// of one wave complete in order), only the compiler must keep the accesses
// on their side of the fences.
template <bool WAVE_ONLY>
__device__ __forceinline__ void lds_handoff() {
  if constexpr (WAVE_ONLY) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  } else {
    __syncthreads();
  }
}

// One 16-token sub-tile of one kv head: q.k for the G heads, online softmax,
// p.v.  kc holds the lane's K chunks (q.k layout), vc its V rows (p.v
// layout); tokens at or past ke are masked.  The query rows come from q_lds
// (QLDS) or qv.
template <bool BF16, int D, int G, bool QLDS, bool WAVE_ONLY>
__device__ __forceinline__ void decode_subtile(WaveAcc<BF16, D, G>& acc,
                                               const uint4 (&kc)[Geo<BF16, D, G>::NL],
                                               uint4 (&vc)[Geo<BF16, D, G>::RPL], const char* q_lds,
                                               const uint4 (&qv)[QLDS ? 1 : G][QLDS ? 1 : Geo<BF16, D, G>::NL],
                                               float* p_lds, float* a_lds, int start, int ke,
                                               float scale_log2, const DecodeLanes& ln) {
  using Gm = Geo<BF16, D, G>;
  constexpr int ROWB = Gm::ROWB, LPR = Gm::LPR, NL = Gm::NL, EPC = Gm::EPC;
  constexpr int RPI = Gm::RPI, RPL = Gm::RPL, HPL = Gm::HPL;
  const int j = ln.j, c = ln.c, rsub = ln.rsub;

  // ---- q.k for the G heads ------------------------------------------------
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      uint4 qq;
      if constexpr (QLDS)
        qq = *reinterpret_cast<const uint4*>(q_lds + h * ROWB + (i * LPR + c) * 16);
      else
        qq = qv[h][i];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if constexpr (BF16) {
          sum = dot2(comp(kc[i], w), comp(qq, w), sum);
        } else {
          sum = __builtin_fmaf(__uint_as_float(comp(kc[i], w)), __uint_as_float(comp(qq, w)), sum);
        }
      }
    }
    sum += dpp<kQuadXor1>(sum);
    sum += dpp<kQuadXor2>(sum);
    s[h] = sum;
  }

  // ---- online softmax: each lane owns heads c, c+4 of token j --------------
  const bool tok_ok = start + j < ke;
  bool rescale = false;
#pragma unroll
  for (int k = 0; k < HPL; ++k) {
    const int h = c + 4 * k;
    const bool hv = h < G;
    float sv = s[0];
#pragma unroll
    for (int hh = 1; hh < G; ++hh) sv = (h == hh) ? s[hh] : sv;
    const float s2 = (hv && tok_ok) ? sv * scale_log2 : kNegInf;
    float mx = s2;
    mx = fmaxf(mx, dpp<kRowRor4>(mx));
    mx = fmaxf(mx, dpp<kRowRor8>(mx));
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(acc.m_run[k], mx);
    const bool live = m_new != kNegInf;
    const float alpha = live ? __builtin_amdgcn_exp2f(acc.m_run[k] - m_new) : 1.f;
    const float p = live ? __builtin_amdgcn_exp2f(s2 - m_new) : 0.f;
    acc.l_run[k] = acc.l_run[k] * alpha + p;
    acc.m_run[k] = m_new;
    rescale |= alpha != 1.f;
    if (hv) {
      if constexpr (BF16) {
        const int rs = j % RPI, kk = j / RPI;
        const int pi = (kk >> 1) * RPI + rs;
        reinterpret_cast<uint16_t*>(p_lds)[(pi * G + h) * 2 + (kk & 1)] = to_bf16(p);
      } else {
        p_lds[j * G + h] = p;
      }
      if (j == 0) a_lds[h] = alpha;
    }
  }
  const bool any_rescale = __builtin_amdgcn_ballot_w64(rescale) != 0;
  lds_handoff<WAVE_ONLY>();

  // ---- p.v ------------------------------------------------------------------
  if (start + 16 > ke) {  // tail sub-tile: rows past the key range may hold NaN
#pragma unroll
    for (int k = 0; k < RPL; ++k)
      if (start + rsub + RPI * k >= ke) vc[k] = make_uint4(0, 0, 0, 0);
  }
  if (any_rescale) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float al = a_lds[h];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc.o[h][e] *= al;
    }
  }
  if constexpr (BF16) {
#pragma unroll
    for (int kk = 0; kk < RPL / 2; ++kk) {
      const uint32_t* pp = reinterpret_cast<const uint32_t*>(p_lds) + (kk * RPI + rsub) * G;
      uint32_t pr[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pr[h] = pp[h];
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const uint32_t lo = comp(vc[2 * kk], e >> 1);
        const uint32_t hi = comp(vc[2 * kk + 1], e >> 1);
        const uint32_t vp = __builtin_amdgcn_perm(hi, lo, (e & 1) ? 0x07060302u : 0x05040100u);
#pragma unroll
        for (int h = 0; h < G; ++h) acc.o[h][e] = dot2(vp, pr[h], acc.o[h][e]);
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < RPL; ++k) {
      const int row = rsub + RPI * k;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = p_lds[row * G + h];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc.o[h][e] = __builtin_fmaf(p, __uint_as_float(comp(vc[k], e)), acc.o[h][e]);
      }
    }
  }
  lds_handoff<WAVE_ONLY>();
}

// End of an item: sums over tokens and over V-row groups, then the G heads'
// rows of token t, kv head g, either normalised into the output (the item
// covers the whole row) or as a partial (m, l, o) in partition slot `slot`.
template <bool BF16, int D, int G, bool WAVE_ONLY>
__device__ __forceinline__ void decode_finish(WaveAcc<BF16, D, G>& acc, float* m_lds, float* l_lds,
                                              const AttnArgs& a, int t, int g, bool direct, int slot,
                                              const DecodeLanes& ln) {
  using Gm = Geo<BF16, D, G>;
  constexpr int ROWB = Gm::ROWB, EPC = Gm::EPC, LPRV = Gm::LPRV, HPL = Gm::HPL;
#pragma unroll
  for (int k = 0; k < HPL; ++k) {
    float l = acc.l_run[k];
    l += dpp<kRowRor4>(l);
    l += dpp<kRowRor8>(l);
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    const int h = ln.c + 4 * k;
    if (ln.j == 0 && h < G) {
      m_lds[h] = acc.m_run[k];
      l_lds[h] = l;
    }
  }
#pragma unroll
  for (int off = LPRV; off < 64; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc.o[h][e] += shfl_xor(acc.o[h][e], off);
  lds_handoff<WAVE_ONLY>();

  if (ln.rsub == 0) {
    const int hq0 = g * G;
    if (direct) {
      char* ob = static_cast<char*>(a.out) + ((int64_t)t * a.Hq + hq0) * ROWB + ln.cv * 16;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float inv = 1.f / l_lds[h];
        if constexpr (BF16) {
          uint32_t w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)to_bf16(acc.o[h][2 * e] * inv) | ((uint32_t)to_bf16(acc.o[h][2 * e + 1] * inv) << 16);
          *reinterpret_cast<uint4*>(ob + h * ROWB) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          *reinterpret_cast<float4*>(ob + h * ROWB) =
              make_float4(acc.o[h][0] * inv, acc.o[h][1] * inv, acc.o[h][2] * inv, acc.o[h][3] * inv);
        }
      }
    } else {
      float* op = a.o_part + ((int64_t)slot * a.Hq + hq0) * D + ln.cv * EPC;
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EPC; e += 4)
          *reinterpret_cast<float4*>(op + h * D + e) =
              make_float4(acc.o[h][e], acc.o[h][e + 1], acc.o[h][e + 2], acc.o[h][e + 3]);
    }
  }
  if (!direct && ln.lane < G) {
    float* mp = a.ml_part + ((int64_t)slot * a.Hq + g * G + ln.lane) * 2;
    mp[0] = m_lds[ln.lane];
    mp[1] = l_lds[ln.lane];
  }
}

// Per-head kernel: one wavefront per (item, kv head); its K/V rows stream
// through registers.
// QLDS: keep the G query rows in LDS (read with broadcast ds_read_b128 in the
// q.k loop) instead of registers: G * D / 4 fewer VGPRs per lane, which buys
// occupancy (more waves, more loads in flight) for the large GQA groups.
template <bool BF16, int D, int G, bool QLDS>
__global__ void __launch_bounds__(64) rowwise_kernel(AttnArgs a) {
  using Gm = Geo<BF16, D, G>;
  constexpr int ROWB = Gm::ROWB, LPR = Gm::LPR, NL = Gm::NL;
  constexpr int LPRV = Gm::LPRV, RPI = Gm::RPI, RPL = Gm::RPL;

  __shared__ __attribute__((aligned(16))) char q_lds[QLDS ? G * ROWB : 16];
  __shared__ float p_lds[16 * G];   // bf16: 8 token pairs x G dwords; fp32: 16 x G
  __shared__ float a_lds[G];        // per-head rescale factor of this sub-tile
  __shared__ float m_lds[G];
  __shared__ float l_lds[G];

  const DecodeLanes ln = decode_lanes<LPRV>(threadIdx.x);
  const int4 it = a.items_rw[blockIdx.x];
  const int r = it.x;
  if (r < 0 || r >= a.R) return;
  const int g = blockIdx.y;
  const int t = it.y;
  const int kb = it.z;
  const int ke = it.w & 0x7FFFFFFF;
  const bool direct = (it.w & kDirect) != 0;
  const int slot = direct ? 0 : a.rw_slot[blockIdx.x];   // partial slot (plan order)

  // query rows of the G heads, in the q.k lane layout (16-byte chunk
  // i * LPR + c of each row); with QLDS the G rows are staged contiguously in
  // LDS, which is the same byte order
  const char* qb = static_cast<const char*>(a.query) + ((int64_t)t * a.Hq + g * G) * ROWB;
  uint4 qv[QLDS ? 1 : G][QLDS ? 1 : NL];
  if constexpr (QLDS) {
    for (int o = ln.lane * 16; o < G * ROWB; o += 64 * 16)
      *reinterpret_cast<uint4*>(q_lds + o) = *reinterpret_cast<const uint4*>(qb + o);
    __syncthreads();
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < NL; ++i)
        qv[h][i] = *reinterpret_cast<const uint4*>(qb + h * ROWB + (i * LPR + ln.c) * 16);
  }

  // physical block ids of the partition: lane i holds block kb/B + i
  const int blk0 = kb / a.B;
  const int nblk = (ke - 1) / a.B - blk0 + 1;
  int myblk = 0;
  if (ln.lane < nblk) {
    myblk = a.block_table[(int64_t)r * a.M + blk0 + ln.lane];
    myblk = myblk < 0 ? 0 : (myblk >= a.num_blocks ? a.num_blocks - 1 : myblk);
  }

  const char* kcache = static_cast<const char*>(a.kcache);
  const char* vcache = static_cast<const char*>(a.vcache);
  const int64_t slot_stride = (int64_t)a.Hkv * ROWB;

  auto load_tile = [&](int start, uint4 (&kr)[NL], uint4 (&vr)[RPL]) {
    const int blk = __builtin_amdgcn_readlane(myblk, start / a.B - blk0);
    const int64_t slot0 = (int64_t)blk * a.B + (start % a.B);
    const char* kbp = kcache + (slot0 + ln.j) * slot_stride + (int64_t)g * ROWB;
#pragma unroll
    for (int i = 0; i < NL; ++i) kr[i] = load_once(kbp + (i * LPR + ln.c) * 16);
    const char* vbp = vcache + slot0 * slot_stride + (int64_t)g * ROWB + ln.cv * 16;
#pragma unroll
    for (int k = 0; k < RPL; ++k)
      vr[k] = load_once(vbp + (int64_t)(ln.rsub + RPI * k) * slot_stride);
  };

  WaveAcc<BF16, D, G> acc;
  acc.init();
  const int n_tiles = (ke - kb + 15) >> 4;
  uint4 kc[NL], vc[RPL];
  load_tile(kb, kc, vc);

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int start = kb + (tile << 4);
    uint4 kn[NL], vn[RPL];
    if (tile + 1 < n_tiles) load_tile(start + 16, kn, vn);
    decode_subtile<BF16, D, G, QLDS, false>(acc, kc, vc, q_lds, qv, p_lds, a_lds, start, ke,
                                            a.scale_log2, ln);
    if (tile + 1 < n_tiles) {
#pragma unroll
      for (int i = 0; i < NL; ++i) kc[i] = kn[i];
#pragma unroll
      for (int k = 0; k < RPL; ++k) vc[k] = vn[k];
    }
  }
  decode_finish<BF16, D, G, false>(acc, m_lds, l_lds, a, t, g, direct, slot, ln);
}

// Whole-block kernel (bf16, head_dim 128, GQA groups of 1, 2 or 4): one
// workgroup of HKV waves per item, wave g computing kv head g from slabs of
// all kv heads staged in LDS (see slab_dma) in a double buffer; every wave
// issues its share of the next slab's DMA, then takes its head's K and V
// rows from LDS into the same register layouts the per-head kernel loads from
// memory.  Reading each block whole, rather than as HKV separate 256-byte
// rows per token fetched by HKV unrelated waves, is what raises the stream
// (measured on MI355X: the C3 split-K pass from 6.08 to 6.37 TB/s, 256 x
// 4K-token decodes from 6.10 to 6.82 TB/s).
template <int G, int HKV>
__global__ void __launch_bounds__(64 * HKV) rowwise_block_kernel(AttnArgs a) {
  constexpr int D = 128;
  using Gm = Geo<true, D, G>;
  constexpr int ROWB = Gm::ROWB, LPR = Gm::LPR, NL = Gm::NL;
  constexpr int LPRV = Gm::LPRV, RPI = Gm::RPI, RPL = Gm::RPL;
  constexpr int CPR = ROWB / 16;                       // 16-byte chunks per head row
  constexpr int SLAB = kSlabTokens * HKV * ROWB;       // bytes of K (or V) per sub-tile
  constexpr int DMA_PER_WAVE = SLAB / 1024 / HKV;      // 1-KB DMA instructions per wave
  static_assert(CPR == 16 && DMA_PER_WAVE * 1024 * HKV == SLAB, "slab geometry");
  __shared__ __attribute__((aligned(1024))) char k_lds0[SLAB];
  __shared__ __attribute__((aligned(1024))) char k_lds1[SLAB];
  __shared__ __attribute__((aligned(1024))) char v_lds0[SLAB];
  __shared__ __attribute__((aligned(1024))) char v_lds1[SLAB];
  __shared__ __attribute__((aligned(16))) char q_lds[HKV * G * ROWB];
  __shared__ float p_lds[HKV * 16 * G];
  __shared__ float a_lds[HKV * G];
  __shared__ float m_lds[HKV * G];
  __shared__ float l_lds[HKV * G];
  const DecodeLanes ln = decode_lanes<LPRV>(threadIdx.x & 63);
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int4 it = a.items_rw[blockIdx.x];
  const int r = it.x;
  if (r < 0 || r >= a.R) return;
  const int t = it.y;
  const int kb = it.z;
  const int ke = it.w & 0x7FFFFFFF;
  const bool direct = (it.w & kDirect) != 0;
  const int slot = direct ? 0 : a.rw_slot[blockIdx.x];

  // this wave's query rows and hand-off areas
  char* qw = q_lds + g * G * ROWB;
  float* pw = p_lds + g * 16 * G;
  float* aw = a_lds + g * G;
  const char* qb = static_cast<const char*>(a.query) + ((int64_t)t * a.Hq + g * G) * ROWB;
  for (int o = ln.lane * 16; o < G * ROWB; o += 64 * 16)
    *reinterpret_cast<uint4*>(qw + o) = *reinterpret_cast<const uint4*>(qb + o);

  const int blk0 = kb / a.B;
  const int nblk = (ke - 1) / a.B - blk0 + 1;
  int myblk = 0;
  if (ln.lane < nblk) {
    myblk = a.block_table[(int64_t)r * a.M + blk0 + ln.lane];
    myblk = myblk < 0 ? 0 : (myblk >= a.num_blocks ? a.num_blocks - 1 : myblk);
  }
  const char* kcache = static_cast<const char*>(a.kcache);
  const char* vcache = static_cast<const char*>(a.vcache);

  // DMA lane offsets within a slab (wave g's instruction i, lane l: physical
  // chunk (g * DMA_PER_WAVE + i) * 64 + l)
  uint32_t dma_off[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i)
    dma_off[i] = slab_source_offset<HKV, CPR>((g * DMA_PER_WAVE + i) * 64 + ln.lane);
  auto slab_base = [&](int start) -> uint64_t {
    const int blk = __builtin_amdgcn_readlane(myblk, start / a.B - blk0);
    return ((uint64_t)blk * a.B + (start % a.B)) * (uint64_t)(HKV * ROWB);
  };

  const int sj = slab_swz(ln.j);
  int vrow_off[RPL];
#pragma unroll
  for (int k = 0; k < RPL; ++k) {
    const int row = ln.rsub + RPI * k;
    vrow_off[k] = (row * HKV + g) * ROWB + ((ln.cv ^ slab_swz(row)) << 4);
  }
  const uint4 no_qv[1][1] = {};
  WaveAcc<true, D, G> acc;
  acc.init();
  auto subtile = [&](const char* kbuf, const char* vbuf, int start) __attribute__((always_inline)) {
    uint4 kc[NL], vc[RPL];
#pragma unroll
    for (int i = 0; i < NL; ++i)
      kc[i] = *reinterpret_cast<const uint4*>(kbuf + (ln.j * HKV + g) * ROWB + (((i * LPR + ln.c) ^ sj) << 4));
#pragma unroll
    for (int k = 0; k < RPL; ++k) vc[k] = *reinterpret_cast<const uint4*>(vbuf + vrow_off[k]);
    decode_subtile<true, D, G, true, true>(acc, kc, vc, qw, no_qv, pw, aw, start, ke, a.scale_log2, ln);
  };

  const int n_tiles = (ke - kb + 15) >> 4;
  slab_dma(kcache, vcache, slab_base(kb), dma_off, k_lds0, v_lds0, g);
  for (int tile = 0; tile < n_tiles; tile += 2) {
    // even sub-tile: buffer 0.  Wait for this wave's part of its DMA, then a
    // barrier makes every wave's part visible and guarantees buffer 1 is no
    // longer being read; the next sub-tile's DMA goes out before the math.
    __builtin_amdgcn_s_waitcnt(kWaitDma);
    __syncthreads();
    if (tile + 1 < n_tiles) slab_dma(kcache, vcache, slab_base(kb + 16 * (tile + 1)), dma_off, k_lds1, v_lds1, g);
    subtile(k_lds0, v_lds0, kb + 16 * tile);
    if (tile + 1 < n_tiles) {  // odd sub-tile: buffer 1
      __builtin_amdgcn_s_waitcnt(kWaitDma);
      __syncthreads();
      if (tile + 2 < n_tiles) slab_dma(kcache, vcache, slab_base(kb + 16 * (tile + 2)), dma_off, k_lds0, v_lds0, g);
      subtile(k_lds1, v_lds1, kb + 16 * (tile + 1));
    }
  }
  decode_finish<true, D, G, true>(acc, m_lds + g * G, l_lds + g * G, a, t, g, direct, slot, ln);
}

// Merge pass: combine the partial (m, l, o) of one query row's partitions,
// rescaling each to the global max (log-sum-exp normalisation).  One
// workgroup per merge record; its waves take the record's (token, head)
// pairs in turn.  For a pair, lane p loads partition p's (m, l) so the max
// and the weighted sum of l are wave reductions, then every lane accumulates
// its slice of the head dimension over the partitions.
// Wave reductions: within each 16-lane row by DPP (quad swaps, then row
// rotations by 4 and 8), across the four rows by two shuffles.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kQuadXor1>(x));
  x = fmaxf(x, dpp<kQuadXor2>(x));
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor8>(x));
  x = fmaxf(x, shfl_xor(x, 16));
  return fmaxf(x, shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<kQuadXor1>(x);
  x += dpp<kQuadXor2>(x);
  x += dpp<kRowRor4>(x);
  x += dpp<kRowRor8>(x);
  x += shfl_xor(x, 16);
  return x + shfl_xor(x, 32);
}

template <bool BF16, int D, int G>
__global__ void __launch_bounds__(256) merge_kernel(AttnArgs a) {
  constexpr int E = BF16 ? 2 : 4;
  constexpr int PER = D / 64;  // elements per lane
  const int4 mr = a.merge[blockIdx.x];
  const int t_first = mr.x;
  if (t_first < 0) return;
  const int first = mr.y, n = mr.z, n_tok = mr.w >> 16, stride = mr.w & 0xFFFF;
  // a record must name output rows of this step and partial slots of this
  // workspace (the plan only writes such records; this keeps a table that
  // disagrees with the launch sizes from reading or writing outside them)
  const int64_t n_parts = (int64_t)a.ps.n_rw + a.ps.n_ck_parts;
  if (n < 1 || n_tok < 1 || stride < 1 || first < 0 || (int64_t)t_first + n_tok > a.ps.T ||
      (int64_t)first + (n_tok - 1) + (int64_t)(n - 1) * stride >= n_parts)
    return;
  const int g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll 1
  for (int pair = wave; pair < n_tok * G; pair += 4) {
    const int tau = pair / G;
    const int hq = g * G + pair % G;
    const int64_t p0 = first + tau;
    // (m, l) of up to 64 partitions per pass: lane p holds partition p's pair;
    // with at most 64 partitions (the usual case) one load serves both passes.
    // The first eight partitions' output slices do not depend on the max, so
    // they are loaded together with (m, l).
    const float* obase0 = a.o_part + (p0 * a.Hq + hq) * D + lane * PER;
    const int64_t pstep = (int64_t)stride * a.Hq * D;   // floats between partitions
    float v0[8][PER];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < PER; ++e) v0[u][e] = u < n ? obase0[u * pstep + e] : 0.f;
    float2 ml0 = make_float2(kNegInf, 0.f);
    if (lane < n) ml0 = *reinterpret_cast<const float2*>(a.ml_part + ((p0 + (int64_t)lane * stride) * a.Hq + hq) * 2);
    float M = ml0.x;
    for (int pb = 64; pb < n; pb += 64) {
      const int p = pb + lane;
      const float m = p < n ? a.ml_part[((p0 + (int64_t)p * stride) * a.Hq + hq) * 2] : kNegInf;
      M = fmaxf(M, m);
    }
    M = wave_max(M);
    float num[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) num[e] = 0.f;
    float den = 0.f;
    for (int pb = 0; pb < n; pb += 64) {
      const int p = pb + lane;
      float w = 0.f;
      if (p < n) {
        const float2 ml = pb == 0 ? ml0
            : *reinterpret_cast<const float2*>(a.ml_part + ((p0 + (int64_t)p * stride) * a.Hq + hq) * 2);
        w = __builtin_amdgcn_exp2f(ml.x - M);
        den += w * ml.y;
      }
      const int cnt = min(64, n - pb);
      const float* obase = a.o_part + ((p0 + (int64_t)pb * stride) * a.Hq + hq) * D + lane * PER;
      int j = 0;
      if (pb == 0) {   // the slices loaded up front (zero past the count)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), u));
#pragma unroll
          for (int e = 0; e < PER; ++e) num[e] += u < cnt ? wj * v0[u][e] : 0.f;
        }
        j = 8;
      }
      // eight partitions' slices in flight at a time
      for (; j + 8 <= cnt; j += 8) {
        float v[8][PER];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int e = 0; e < PER; ++e) v[u][e] = obase[(j + u) * pstep + e];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j + u));
#pragma unroll
          for (int e = 0; e < PER; ++e) num[e] += wj * v[u][e];
        }
      }
      for (; j < cnt; ++j) {
        const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), j));
#pragma unroll
        for (int e = 0; e < PER; ++e) num[e] += wj * obase[j * pstep + e];
      }
    }
    den = wave_sum(den);
    const float inv = 1.f / den;
    char* ob = static_cast<char*>(a.out) + (((int64_t)(t_first + tau) * a.Hq + hq) * D + lane * PER) * E;
    if constexpr (BF16) {
      if constexpr (PER == 2) {
        *reinterpret_cast<uint32_t*>(ob) =
            (uint32_t)to_bf16(num[0] * inv) | ((uint32_t)to_bf16(num[1] * inv) << 16);
      } else {
        *reinterpret_cast<uint16_t*>(ob) = to_bf16(num[0] * inv);
      }
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) reinterpret_cast<float*>(ob)[e] = num[e] * inv;
    }
  }
}

#define PA_DISPATCH_GD(FN, BF, DD)                                    \
  switch (a.Hq / a.Hkv) {                                             \
    case 1: kern = (const void*)FN<BF, DD, 1>; break;                 \
    case 2: kern = (const void*)FN<BF, DD, 2>; break;                 \
    case 4: kern = (const void*)FN<BF, DD, 4>; break;                 \
    case 8: kern = (const void*)FN<BF, DD, 8>; break;                 \
    default: return hipErrorInvalidValue;                             \
  }

#define PA_DISPATCH_GDQ(FN, BF, DD, Q)                                \
  switch (a.Hq / a.Hkv) {                                             \
    case 1: kern = (const void*)FN<BF, DD, 1, Q>; break;              \
    case 2: kern = (const void*)FN<BF, DD, 2, Q>; break;              \
    case 4: kern = (const void*)FN<BF, DD, 4, Q>; break;              \
    case 8: kern = (const void*)FN<BF, DD, 8, Q>; break;              \
    default: return hipErrorInvalidValue;                             \
  }

#define PA_SELECT_Q(FN, Q)                                            \
  if (a.bf16) {                                                       \
    if (a.D == 64) { PA_DISPATCH_GDQ(FN, true, 64, Q) }               \
    else if (a.D == 128) { PA_DISPATCH_GDQ(FN, true, 128, Q) }        \
    else return hipErrorInvalidValue;                                 \
  } else {                                                            \
    if (a.D == 64) { PA_DISPATCH_GDQ(FN, false, 64, Q) }              \
    else if (a.D == 128) { PA_DISPATCH_GDQ(FN, false, 128, Q) }       \
    else return hipErrorInvalidValue;                                 \
  }

#define PA_SELECT(FN)                                                 \
  const void* kern = nullptr;                                         \
  PA_SELECT_INTO(FN)

#define PA_SELECT_INTO(FN)                                            \
  if (a.bf16) {                                                       \
    if (a.D == 64) { PA_DISPATCH_GD(FN, true, 64) }                   \
    else if (a.D == 128) { PA_DISPATCH_GD(FN, true, 128) }            \
    else return hipErrorInvalidValue;                                 \
  } else {                                                            \
    if (a.D == 64) { PA_DISPATCH_GD(FN, false, 64) }                  \
    else if (a.D == 128) { PA_DISPATCH_GD(FN, false, 128) }           \
    else return hipErrorInvalidValue;                                 \
  }

}  // namespace

// Query rows go to LDS when that lowers the register footprint enough to
// matter (GQA groups of 4 and more: three waves per SIMD instead of two, so
// more K/V loads in flight); PA_TUNE_DECODE_Q_PLACEMENT overrides.
static bool use_qlds(int32_t G) {
  const int32_t t = tuning(PA_TUNE_DECODE_Q_PLACEMENT);
  if (t == 1) return false;
  if (t == 2) return true;
  return G >= 4;
}

// Decode is bandwidth-bound; the matrix cores are used for it only where the
// vector kernel's arithmetic measurably limits the stream: bf16 caches with
// GQA groups of 8, where the v_dot2 loops cost about as much time as the K/V
// reads (measured: 5.2 -> 5.7 TB/s on 16 x 32K + 240 short contexts).  With
// groups of 4 the two kernels are within noise of each other, and the
// vector kernel stays.  PA_TUNE_DECODE_KERNEL overrides (groups of 4 and 8).
static bool use_mfma(bool bf16, int32_t D, int32_t G) {
  if (!bf16 || rowwise_mfma_kernel_for(D, G) == nullptr) return false;
  const int32_t t = tuning(PA_TUNE_DECODE_KERNEL);
  if (t == 1) return false;
  if (t == 2) return true;
  return G >= 8;
}

// The whole-block vector kernel's instances (bf16, head_dim 128, GQA groups
// 1, 2 and 4, 1..8 kv heads); nullptr elsewhere.
static const void* block_kernel_for(int32_t G, int32_t Hkv) {
#define PA_BLOCK_G(HK)                                                   \
  switch (G) {                                                           \
    case 1: return (const void*)rowwise_block_kernel<1, HK>;             \
    case 2: return (const void*)rowwise_block_kernel<2, HK>;             \
    case 4: return (const void*)rowwise_block_kernel<4, HK>;             \
    default: return nullptr;                                             \
  }
  switch (Hkv) {
    case 1: PA_BLOCK_G(1)
    case 2: PA_BLOCK_G(2)
    case 4: PA_BLOCK_G(4)
    case 8: PA_BLOCK_G(8)
    default: return nullptr;
  }
#undef PA_BLOCK_G
}

// The split-K kernel of a configuration and its launch shape: whole-block
// kernels run one workgroup of Hkv waves per item (grid n_rw), per-head
// kernels one wavefront per (item, kv head) (grid n_rw x Hkv).  The
// whole-block forms are the default wherever they have an instance: measured
// faster than the per-head kernels on every decode mix tried (C3's split-K
// pass 4.5 %, 64 contexts of 512..4096 keys 2 %, 256 contexts of 4K keys
// 12 %).  PA_TUNE_DECODE_STAGING 1 keeps the per-head kernels.
struct DecodeLaunch {
  const void* kern;
  int threads;      // per workgroup
  bool per_item;    // one workgroup per item (whole-block) or per (item, kv head)
  int kind;         // 0/1 per-head vector (q in registers / LDS), 2 per-head matrix-core,
                    // 3 whole-block vector, 4 whole-block matrix-core
};

static hipError_t decode_launch(bool bf16, int32_t D, int32_t G, int32_t Hkv, DecodeLaunch* out) {
  const bool staged = tuning(PA_TUNE_DECODE_STAGING) != 1;
  if (use_mfma(bf16, D, G)) {
    const void* wb = staged ? rowwise_mfma_block_kernel_for(D, G, Hkv) : nullptr;
    *out = wb ? DecodeLaunch{wb, 64 * Hkv, true, 4} : DecodeLaunch{rowwise_mfma_kernel_for(D, G), 64, false, 2};
    return hipSuccess;
  }
  if (bf16 && D == 128 && staged) {
    if (const void* bk = block_kernel_for(G, Hkv)) {
      *out = DecodeLaunch{bk, 64 * Hkv, true, 3};
      return hipSuccess;
    }
  }
  AttnArgs a{};
  a.bf16 = bf16;
  a.D = D;
  a.Hkv = 1;
  a.Hq = G;
  const void* kern = nullptr;
  const bool qlds = use_qlds(G);
  if (qlds) {
    PA_SELECT_Q(rowwise_kernel, true)
  } else {
    PA_SELECT_Q(rowwise_kernel, false)
  }
  *out = DecodeLaunch{kern, 64, false, qlds ? 1 : 0};
  return hipSuccess;
}

hipError_t launch_rowwise(const AttnArgs& a, hipStream_t s) {
  if (a.ps.n_rw == 0) return hipSuccess;
  DecodeLaunch dl{};
  const hipError_t e = decode_launch(a.bf16, a.D, a.Hq / a.Hkv, a.Hkv, &dl);
  if (e != hipSuccess) return e;
  AttnArgs args = a;
  void* params[] = {&args};
  const dim3 grid = dl.per_item ? dim3(a.ps.n_rw) : dim3(a.ps.n_rw, a.Hkv);
  return hipLaunchKernel(dl.kern, grid, dim3(dl.threads), params, 0, s);
}

int64_t rowwise_round_slots(bool bf16, int32_t D, int32_t G, int32_t Hkv) {
  // wave slots of one round of the split-K grid: the kernel's occupancy per
  // compute unit in waves (workgroups times their waves: Hkv for the
  // whole-block kernels, one otherwise), at most 8 (two per SIMD), times the
  // compute units; cached per configuration.  A grid that fits in one round
  // streams faster with about 8 waves per compute unit than with the 12 the
  // per-head kernel could hold (measured on 64 contexts of 512..4096 keys:
  // 107 against 116 us; fewer concurrent K/V streams per HBM channel)
  // (per thread: the current device of the calling thread, the last device
  // seen and its entries; another device clears them)
  static thread_local int64_t cache[2][2][9][5][4] = {};
  static thread_local int cache_dev = -1;
  if (G < 1 || G > 8 || Hkv < 1) return 0;
  DecodeLaunch dl{};
  if (decode_launch(bf16, D, G, Hkv, &dl) != hipSuccess || dl.kern == nullptr) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev != cache_dev) {
    std::fill(&cache[0][0][0][0][0], &cache[0][0][0][0][0] + sizeof(cache) / sizeof(int64_t), int64_t{0});
    cache_dev = dev;
  }
  const int hi = dl.per_item ? 31 - __builtin_clz((unsigned)Hkv) : 0;   // Hkv in {1, 2, 4, 8} there
  int64_t& c = cache[bf16 ? 1 : 0][D == 128 ? 1 : 0][G][dl.kind][hi];
  if (c == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dl.kern, dl.threads, 0) != hipSuccess || cus <= 0 ||
        per_cu <= 0)
      return 0;
    c = (int64_t)cus * std::min(per_cu * (dl.threads / 64), 8);
  }
  return c;
}

hipError_t launch_merge(const AttnArgs& a, hipStream_t s) {
  if (a.ps.n_mg == 0) return hipSuccess;
  PA_SELECT(merge_kernel)
  AttnArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(kern, dim3(a.ps.n_mg, a.Hkv), dim3(256), params, 0, s);
}

}  // namespace pa
