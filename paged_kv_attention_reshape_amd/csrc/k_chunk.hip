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
// K/V tiles of 64 keys are gathered through the block table (16-byte chunks,
// rows XOR-swizzled in LDS against bank conflicts) into a double buffer while
// the previous tile is on the matrix cores.
#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kThreads = 256;  // 4 waves
constexpr int KT = 64;         // keys per tile
constexpr int kMaxSegBlocks = 512;
constexpr int kXcds = 8;       // accelerator complex dies of an MI355X
constexpr float kNegInf = -__builtin_huge_valf();

template <int V>
struct __integral_constant {
  static constexpr int value = V;
  constexpr operator int() const { return V; }
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
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

template <int D, int G>
__global__ void __launch_bounds__(kThreads, 2) chunk_kernel(AttnArgs a) {
  constexpr int ROWB = D * 2;        // bytes per key row (one head)
  constexpr int CPR = ROWB / 16;     // 16-byte chunks per row
  constexpr int KSTEPS = D / 16;     // MFMA k-steps for q.k
  constexpr int DB = D / 32;         // 32-wide d blocks of O
  constexpr int TQ = 128 / G;
  constexpr int TILE_BYTES = KT * ROWB;
  constexpr int LOADS = KT * CPR / kThreads;  // 16-byte chunks per thread per tile (K or V)
  static_assert(LOADS >= 1, "tile too small");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* k_lds = smem;                           // [2][KT][ROWB]
  char* v_lds = smem + 2 * TILE_BYTES;          // [2][KT][ROWB]
  int32_t* bt_lds = reinterpret_cast<int32_t*>(smem + 4 * TILE_BYTES);

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
  if (r < 0 || r >= a.R) return;
  const int qt = it.y, seg = it.z, part_base = it.w;

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

  // block ids of the segment into LDS
  const int blk_first = k0 / a.B;
  const int nblk = (k1 - 1) / a.B - blk_first + 1;   // (one-time divisions)
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
  __syncthreads();  // bt_lds ready

  const char* kcache = static_cast<const char*>(a.kcache);
  const char* vcache = static_cast<const char*>(a.vcache);
  const int64_t slot_stride = (int64_t)a.Hkv * ROWB;
  const int64_t head_off = (int64_t)g * ROWB;
  const int lb = 31 - __builtin_clz(a.B);   // block size is a power of two here
  const int bmask = a.B - 1;

  // This thread's 16-byte chunks of every tile: chunk i is key row
  // (i * kThreads + tid) / CPR of the tile, physical column pchunk, holding
  // logical column pchunk ^ (key % CPR) (XOR swizzle against LDS conflicts).
  int ld_key[LOADS], ld_lds[LOADS], ld_col[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int id = i * kThreads + tid;
    ld_key[i] = id / CPR;
    const int pchunk = id % CPR;
    ld_lds[i] = ld_key[i] * ROWB + pchunk * 16;
    ld_col[i] = (pchunk ^ (ld_key[i] % CPR)) * 16;
  }
  u32x4_t kst[LOADS], vst[LOADS];
#define PA_CK_LOAD(KT0)                                                                   \
  static_for<LOADS>([&](auto I) {                                                         \
    constexpr int i = I;                                                                  \
    int kabs = (KT0) + ld_key[i];                                                         \
    kabs = kabs < k1 ? kabs : k1 - 1;                                                     \
    const int blk = bt_lds[(kabs >> lb) - blk_first];                                     \
    const int64_t off = (((int64_t)blk << lb) + (kabs & bmask)) * slot_stride + head_off + ld_col[i]; \
    kst[i] = *reinterpret_cast<const u32x4_t*>(kcache + off);                             \
    vst[i] = *reinterpret_cast<const u32x4_t*>(vcache + off);                             \
  });
#define PA_CK_STORE(BUF)                                                                  \
  static_for<LOADS>([&](auto I) {                                                         \
    constexpr int i = I;                                                                  \
    *reinterpret_cast<u32x4_t*>(k_lds + (BUF) * TILE_BYTES + ld_lds[i]) = kst[i];         \
    *reinterpret_cast<u32x4_t*>(v_lds + (BUF) * TILE_BYTES + ld_lds[i]) = vst[i];         \
  });

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
  float m_run = kNegInf;   // in log2 units (score * scale * log2 e)
  float l_run = 0.f;       // this lane's share of the row sum
  const float sl = a.scale_log2;
  const int grp = lane >> 5;       // 0/1: which 4-key half of each 8-key group
  const int gam = lane >> 4;       // 16-lane group for transposed V reads
  const int li = lane & 15;        // lane within the 16-lane group

  const int n_tiles = (k1 - k0 + KT - 1) / KT;
  PA_CK_LOAD(k0)
  PA_CK_STORE(0)

  for (int ti = 0; ti < n_tiles; ++ti) {
    const int kt = k0 + ti * KT;
    const int buf = ti & 1;
    if (ti + 1 < n_tiles) { PA_CK_LOAD(kt + KT) }
    __syncthreads();

    if (kt <= w_qpos_hi) {  // some row of this wave sees part of the tile
      const char* kb = k_lds + buf * TILE_BYTES;
      const char* vb = v_lds + buf * TILE_BYTES;
      // ---- S^T = K Q^T ---------------------------------------------------
      f32x16_t s[2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int e = 0; e < 16; ++e) s[sub][e] = 0.f;
        const int key = sub * 32 + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          const int ch = (2 * kk + grp) ^ (key % CPR);
          const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(kb + key * ROWB + ch * 16);
          s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kv),
                                                           __builtin_bit_cast(bf16x8_t, qf[kk]),
                                                           s[sub], 0, 0, 0);
        }
      }
      // ---- mask, online softmax --------------------------------------------
      const bool need_mask = (kt + KT - 1 > w_qpos_lo) || (kt + KT > k1);
      float mx = kNegInf;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          if (need_mask) {
            const int key = kt + sub * 32 + 8 * (e >> 2) + 4 * grp + (e & 3);
            s[sub][e] = (key > qpos || key >= k1) ? kNegInf : s[sub][e];
          }
          mx = fmaxf(mx, s[sub][e]);
        }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx * sl);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      float psum = 0.f;
      uint32_t pk[2][8];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][e], sl, -m_use));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sub][e + 1], sl, -m_use));
          psum += p0 + p1;
          pk[sub][e >> 1] = pack_bf16(p0, p1);
        }
      l_run = l_run * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[db][e] *= alpha;
      }
      // ---- O^T += V^T P^T ----------------------------------------------------
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4_t pw = {pk[sub][4 * h], pk[sub][4 * h + 1], pk[sub][4 * h + 2], pk[sub][4 * h + 3]};
          const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
          const int kbase = sub * 32 + 16 * h + 4 * grp + (li >> 2);  // row m = li / 4
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d0 = db * 32 + 16 * (gam & 1) + 4 * (li & 3);   // 4 d values, 8 bytes
            const int key1 = kbase, key2 = kbase + 8;
            const int c1 = ((d0 >> 3) ^ (key1 % CPR)), c2 = ((d0 >> 3) ^ (key2 % CPR));
            const int in_chunk = (d0 & 7) * 2;
            const lds_s16x4_t* p1 = reinterpret_cast<const lds_s16x4_t*>(
                (__attribute__((address_space(3))) const char*)(vb + key1 * ROWB + c1 * 16 + in_chunk));
            const lds_s16x4_t* p2 = reinterpret_cast<const lds_s16x4_t*>(
                (__attribute__((address_space(3))) const char*)(vb + key2 * ROWB + c2 * 16 + in_chunk));
            const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4_t*>(p1));
            const s16x4_t v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4_t*>(p2));
            const s16x8_t vv = __builtin_shufflevector(v1, v2, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, vv);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[db], 0, 0, 0);
          }
        }
    }
    if (ti + 1 < n_tiles) { PA_CK_STORE(buf ^ 1) }
  }
#undef PA_CK_LOAD
#undef PA_CK_STORE

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = l_run + xor32(l_run);
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
        const uint2 w = make_uint2(pack_bf16(o[db][4 * e4] * inv, o[db][4 * e4 + 1] * inv),
                                   pack_bf16(o[db][4 * e4 + 2] * inv, o[db][4 * e4 + 3] * inv));
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
            make_float4(o[db][4 * e4], o[db][4 * e4 + 1], o[db][4 * e4 + 2], o[db][4 * e4 + 3]);
      }
    if (grp == 0) {
      float* mp = a.ml_part + (slot * a.Hq + hq) * 2;
      mp[0] = m_run;
      mp[1] = l_tot;
    }
  }
}

template <int D>
size_t chunk_smem() {
  return 4 * (size_t)KT * D * 2 + kMaxSegBlocks * sizeof(int32_t);
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
  size_t smem = 0;
#define PA_CK(DD, GG) \
  if (a.D == DD && G == GG) { kern = (const void*)chunk_kernel<DD, GG>; smem = chunk_smem<DD>(); }
  PA_CK(64, 1) PA_CK(64, 2) PA_CK(64, 4) PA_CK(64, 8)
  PA_CK(128, 1) PA_CK(128, 2) PA_CK(128, 4) PA_CK(128, 8)
#undef PA_CK
  if (kern == nullptr) return hipErrorInvalidValue;
  static bool attr_done[2] = {false, false};
  if (smem > 64 * 1024) {
    const int idx = a.D == 128 ? 1 : 0;
    if (!attr_done[idx]) {
      // every <D, G> instance of this D shares the size
      const void* all[4] = {nullptr, nullptr, nullptr, nullptr};
      if (a.D == 128) {
        all[0] = (const void*)chunk_kernel<128, 1>; all[1] = (const void*)chunk_kernel<128, 2>;
        all[2] = (const void*)chunk_kernel<128, 4>; all[3] = (const void*)chunk_kernel<128, 8>;
      } else {
        all[0] = (const void*)chunk_kernel<64, 1>; all[1] = (const void*)chunk_kernel<64, 2>;
        all[2] = (const void*)chunk_kernel<64, 4>; all[3] = (const void*)chunk_kernel<64, 8>;
      }
      for (const void* k : all) {
        hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
      }
      attr_done[idx] = true;
    }
  }
  AttnArgs args = a;
  void* params[] = {&args};
  const int64_t units = (int64_t)a.ps.n_ck * a.Hkv;
  const int64_t per_xcd = (units + kXcds - 1) / kXcds;
  return hipLaunchKernel(kern, dim3((unsigned)(per_xcd * kXcds)), dim3(kThreads), params, smem, s);
}

}  // namespace pa
