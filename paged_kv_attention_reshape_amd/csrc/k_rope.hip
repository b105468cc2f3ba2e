// Fused rotary embedding + cache write.
//
// "AI Infra入门干货总结：大模型是如何高效推理的", section "Attention Module
// (以标准GQA + RoPE为例)": Q and K are rotated by a block-diagonal rotation
// whose angles depend on the token position.  The rotation is applied
// elementwise with cos/sin, and the cos/sin values are not computed per call
// but read from a table cos_sin_cache [max_position, rotary_dim] prepared once
// (cos of the rotary_dim/2 angles, then their sin), indexed by each token's
// position.  The step's order is: rotate Q and K, then scatter K (rotated) and
// V into the paged cache through slot_mapping ("Paged Attention": slot =
// block * block_size + offset; the cache row of a slot holds all kv heads).
//
// One pass over the step's tokens does all of it: Q is rotated in place, the
// rotated K and the unchanged V go straight to their cache slot, so K never
// makes a round trip through HBM between the rotation and the write.  The
// kernel is bandwidth-bound: every byte of Q, K, V is read once and every
// byte of Q and of the two cache rows is written once.
//
// MI355X mapping: one workgroup per token; a work unit is one 16-byte chunk
// (or, for split-halves pairing, the two chunks whose elements pair up), so
// every load and store is a 16-byte vector and consecutive lanes cover
// consecutive chunks of a head row.  The token's cos/sin row (at most 512
// bytes) is read by every unit of the token and stays in the L1/L2 caches.
// Arithmetic is fp32 (x' = x cos - y sin, y' = y cos + x sin); results are
// rounded once to the storage type.
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// 16-byte chunk <-> EPC floats
template <bool BF16>
struct Chunk {
  static constexpr int EPC = BF16 ? 8 : 4;
  static __device__ __forceinline__ void unpack(const uint4 v, float (&f)[EPC]) {
    if constexpr (BF16) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
      f[0] = __uint_as_float(v.x);
      f[1] = __uint_as_float(v.y);
      f[2] = __uint_as_float(v.z);
      f[3] = __uint_as_float(v.w);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float (&f)[EPC]) {
    if constexpr (BF16) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = pack_bf16(f[2 * i], f[2 * i + 1]);
      return make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                        __float_as_uint(f[3]));
    }
  }
};

__device__ __forceinline__ void rotate(float& x, float& y, float c, float s) {
  const float xr = __builtin_fmaf(x, c, -(y * s));
  const float yr = __builtin_fmaf(y, c, x * s);
  x = xr;
  y = yr;
}

// Work units of one token, in order:
//   [0, NQ)            Q rotation units (head h, unit c)  -- in place
//   [NQ, NQ + NK)      K units: rotation units, then pass-through chunks
//                      (dimensions >= rotary_dim), written to the K cache
//   [NQ + NK, N)       V chunks, copied to the V cache
// A rotation unit is, for split-halves pairing, the chunk pair (c, c + UR)
// of the rotated part (elements i and i + rotary_dim/2 pair up), and for
// adjacent pairing one chunk (its elements pair up two by two).
template <bool BF16, int D, bool NEOX>
__global__ void __launch_bounds__(kThreads) rope_write_kv_kernel(RopeArgs a) {
  using C = Chunk<BF16>;
  constexpr int EPC = C::EPC;
  constexpr int CPR = D / EPC;            // chunks per head row
  const int64_t t = blockIdx.x;
  const int rd = a.rotary_dim;
  const int UR = NEOX ? rd / (2 * EPC) : rd / EPC;   // rotation units per head row
  const int UP = CPR - rd / EPC;                     // pass-through chunks per head row
  const int NQ = a.Hq * UR;
  const int NK = a.Hkv * (UR + UP);
  const int N = NQ + NK + a.Hkv * CPR;

  int64_t pos = a.positions[t];
  pos = pos < 0 ? 0 : (pos >= a.max_position ? a.max_position - 1 : pos);
  const float* __restrict__ cosv = a.cos_sin + pos * rd;
  const float* __restrict__ sinv = cosv + rd / 2;
  const int64_t slot = a.slots[t];
  const bool write = slot >= 0 && slot < a.num_slots;

  uint4* q = static_cast<uint4*>(a.query) + t * (int64_t)a.Hq * CPR;
  const uint4* __restrict__ k = static_cast<const uint4*>(a.key) + t * (int64_t)a.Hkv * CPR;
  const uint4* __restrict__ v = static_cast<const uint4*>(a.value) + t * (int64_t)a.Hkv * CPR;
  uint4* __restrict__ kc = static_cast<uint4*>(a.key_cache) + (write ? slot : 0) * (int64_t)a.Hkv * CPR;
  uint4* __restrict__ vc = static_cast<uint4*>(a.value_cache) + (write ? slot : 0) * (int64_t)a.Hkv * CPR;

  for (int u = threadIdx.x; u < N; u += kThreads) {
    if (u >= NQ + NK) {                       // V: plain copy
      if (!write) continue;
      const int i = u - NQ - NK;
      vc[i] = v[i];
      continue;
    }
    const bool is_q = u < NQ;
    const int w = is_q ? u : u - NQ;
    const int per = is_q ? UR : UR + UP;
    const int h = w / per;
    const int cu = w - h * per;
    if (!is_q && !write) continue;
    // Q is rotated in place: src and dst may be the same row
    const uint4* src = is_q ? q + h * CPR : k + h * CPR;
    uint4* dst = is_q ? q + h * CPR : kc + h * CPR;
    if (cu >= UR) {                           // K pass-through chunk
      const int c = rd / EPC + (cu - UR);
      dst[c] = src[c];
      continue;
    }
    if constexpr (NEOX) {
      const int c0 = cu, c1 = cu + UR;        // elements e0 + j and e0 + rd/2 + j pair up
      float x[EPC], y[EPC];
      C::unpack(src[c0], x);
      C::unpack(src[c1], y);
      const int e0 = cu * EPC;
#pragma unroll
      for (int j = 0; j < EPC; ++j) rotate(x[j], y[j], cosv[e0 + j], sinv[e0 + j]);
      dst[c0] = C::pack(x);
      dst[c1] = C::pack(y);
    } else {
      float x[EPC];
      C::unpack(src[cu], x);
      const int p0 = cu * (EPC / 2);          // elements 2p, 2p+1 pair up with angle p
#pragma unroll
      for (int j = 0; j < EPC / 2; ++j) rotate(x[2 * j], x[2 * j + 1], cosv[p0 + j], sinv[p0 + j]);
      dst[cu] = C::pack(x);
    }
  }
}

}  // namespace

hipError_t launch_rope_write_kv(const RopeArgs& a, bool bf16, int32_t D, bool neox, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const void* kern = nullptr;
#define PA_RK(BF, DD, NX) \
  if (bf16 == BF && D == DD && neox == NX) kern = (const void*)rope_write_kv_kernel<BF, DD, NX>;
  PA_RK(true, 64, true) PA_RK(true, 64, false) PA_RK(true, 128, true) PA_RK(true, 128, false)
  PA_RK(false, 64, true) PA_RK(false, 64, false) PA_RK(false, 128, true) PA_RK(false, 128, false)
#undef PA_RK
  if (kern == nullptr) return hipErrorInvalidValue;
  if (a.T > 0x7FFFFFFF) return hipErrorInvalidValue;
  RopeArgs args = a;
  void* params[] = {&args};
  return hipLaunchKernel(kern, dim3((unsigned)a.T), dim3(kThreads), params, 0, s);
}

}  // namespace pa
