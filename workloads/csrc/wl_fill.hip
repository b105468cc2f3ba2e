// Device side of the counter-based input generator (test and benchmark
// infrastructure, not part of the attention library).
//
// Element e of row r gets u = derive(row_key(r), e), derive(k, n) =
// mix64(k + (n + 1) * GAMMA) with the SplitMix64 output function (Steele, Lea
// and Flood, OOPSLA 2014), and is mapped to an approximately standard normal
// float32 through the Irwin-Hall sum of u's four 16-bit lanes times one float32
// constant.  bf16 storage rounds to nearest-even on the bit pattern.  Rows
// outside the valid prefix of their group hold a quiet NaN.  workloads/rng.py
// is the host mirror; the two agree bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

__device__ __forceinline__ uint64_t derive(uint64_t k, uint64_t n) {
  return mix64(k + (n + 1ull) * kGamma);
}

__device__ __forceinline__ float normal_f32(uint64_t u, float scale) {
  const int s = (int)(u & 0xFFFFull) + (int)((u >> 16) & 0xFFFFull) +
                (int)((u >> 32) & 0xFFFFull) + (int)(u >> 48) - 131070;
  return __fmul_rn((float)s, scale);
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

template <bool kBf16>
__global__ void __launch_bounds__(256) fill_rows_kernel(
    void* __restrict__ dst, int64_t n_rows, int32_t row_len, uint64_t base_key,
    const uint64_t* __restrict__ row_keys, const int32_t* __restrict__ valid,
    int32_t rows_per_group, float scale) {
  const int64_t chunks_per_row = row_len / 8;
  const int64_t total = n_rows * chunks_per_row;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = idx / chunks_per_row;
    const int64_t e0 = (idx - row * chunks_per_row) * 8;
    bool ok = true;
    if (valid != nullptr) {
      const int64_t grp = row / rows_per_group;
      ok = (row - grp * rows_per_group) < (int64_t)valid[grp];
    }
    const uint64_t rk = row_keys ? row_keys[row] : derive(base_key, (uint64_t)row);
    if (kBf16) {
      uint16_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = ok ? bf16_rne(normal_f32(derive(rk, (uint64_t)(e0 + i)), scale)) : (uint16_t)0x7FC0;
      uint4 pk;
      pk.x = v[0] | ((uint32_t)v[1] << 16);
      pk.y = v[2] | ((uint32_t)v[3] << 16);
      pk.z = v[4] | ((uint32_t)v[5] << 16);
      pk.w = v[6] | ((uint32_t)v[7] << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(dst) + row * row_len + e0) = pk;
    } else {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = ok ? normal_f32(derive(rk, (uint64_t)(e0 + i)), scale)
                  : __uint_as_float(0x7FC00000u);
      float4* p = reinterpret_cast<float4*>(reinterpret_cast<float*>(dst) + row * row_len + e0);
      p[0] = make_float4(v[0], v[1], v[2], v[3]);
      p[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

}  // namespace

extern "C" {

// Fill dst ([n_rows, row_len], row-major, device memory) with generated values.
// dtype: 0 = float32, 1 = bf16 (uint16 bit patterns).  row_keys (device,
// nullable): per-row keys; when null, row r uses derive(base_key, r).  valid
// (device, nullable): rows r with (r % rows_per_group) >= valid[r /
// rows_per_group] get NaN.  norm_scale is the float32 constant of the host
// mirror.  Returns 0 on success, 1 on bad arguments, 2 on a launch error.
int wl_fill_rows(void* dst, int dtype, int64_t n_rows, int32_t row_len, uint64_t base_key,
                 const uint64_t* row_keys, const int32_t* valid, int32_t rows_per_group,
                 float norm_scale, void* stream) {
  if (dst == nullptr || n_rows < 0 || row_len <= 0 || (row_len % 8) != 0) return 1;
  if (valid != nullptr && rows_per_group <= 0) return 1;
  if (n_rows == 0) return 0;
  const int64_t total = n_rows * (row_len / 8);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == 1)
    hipLaunchKernelGGL(fill_rows_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s, dst, n_rows,
                       row_len, base_key, row_keys, valid, rows_per_group, norm_scale);
  else if (dtype == 0)
    hipLaunchKernelGGL(fill_rows_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s, dst,
                       n_rows, row_len, base_key, row_keys, valid, rows_per_group, norm_scale);
  else
    return 1;
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
