// Quantizers on the device: MXFP4 (E2M1 + one E8M0 per 32 elements) and
// per-tensor e4m3fn.  Both are bit-exact restatements of integer rules, so the
// device and any correct host implementation agree byte for byte.
#include "qgemm_common.h"

namespace qgemm {
namespace {

// ---------------------------------------------------------------------------
// MXFP4 (MXFP4 page, section 3 quantizer, with the exponent taken exactly)
// ---------------------------------------------------------------------------
// amax is clamped to >= 1e-8f, so it is a normal fp32 a = 1.f * 2^e0.  The
// smallest e with a <= 6 * 2^e is e0 - 2 when 1.f <= 1.5 (6 * 2^(e0-2) =
// 1.5 * 2^e0) and e0 - 1 otherwise: an integer test on the mantissa field.
// An element's grid index is the number of midpoints {0.25, 0.75, 1.25, 1.75,
// 2.5, 3.5, 5} * 2^e that |x| exceeds strictly -- nearest grid point, with an
// exact tie going to the smaller magnitude.  Every threshold is exact in fp32.
// Blocks are consecutive in memory (row-major [rows, K], K % 32 == 0), so
// the input is a flat array of 128-byte blocks.  Eight lanes share a block,
// each reading 16 bytes (a wave reads 1 KB of whole cache lines per load);
// a workgroup takes kQBlocksPerLane rounds of 32 blocks and issues all its
// loads first.  The block max is reduced over the eight lanes; each lane
// forms the codes of its 4 elements (2 bytes of the block's 16) and lane
// pairs store 4 bytes.
constexpr int kQBlocksPerLane = 4;

__global__ __launch_bounds__(256) void quantize_mxfp4_kernel(const float* __restrict__ x,
                                                             uint8_t* __restrict__ codes,
                                                             uint8_t* __restrict__ e8m0,
                                                             int64_t nblocks) {
  const int part = (int)(threadIdx.x & 7);   // elements 4 part .. 4 part + 3 of a block
  const int64_t b0 = (int64_t)blockIdx.x * (32 * kQBlocksPerLane) + (threadIdx.x >> 3);
  floatx4 v[kQBlocksPerLane];
#pragma unroll
  for (int j = 0; j < kQBlocksPerLane; ++j) {
    const int64_t b = b0 + 32 * j;   // uniform over the 8 lanes of a block
    v[j] = b < nblocks ? __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(x) + 8 * b + part)
                       : floatx4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int j = 0; j < kQBlocksPerLane; ++j) {
    const int64_t b = b0 + 32 * j;
    float amax = fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3])));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    amax = fmaxf(amax, 1e-8f);
    const uint32_t bits = __builtin_bit_cast(uint32_t, amax);
    const int e0 = (int)(bits >> 23) - 127;
    const int e = e0 - 2 + ((bits & 0x7fffffu) > 0x400000u ? 1 : 0);
    const float p2 = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);  // 2^e, normal
    const float t0 = 0.25f * p2, t1 = 0.75f * p2, t2 = 1.25f * p2, t3 = 1.75f * p2;
    const float t4 = 2.5f * p2, t5 = 3.5f * p2, t6 = 5.0f * p2;
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float a = fabsf(v[j][i]);
      const uint32_t idx =
          (a > t0) + (a > t1) + (a > t2) + (a > t3) + (a > t4) + (a > t5) + (a > t6);
      w |= (idx | (v[j][i] < 0.f ? 8u : 0u)) << (4 * i);   // element 2j -> low nibble of byte j
    }
    // lanes 2q and 2q + 1 hold bytes 4q .. 4q + 3 of the block's codes
    const uint32_t pair = w | (__shfl_xor(w, 1, 64) << 16);
    if (b < nblocks && (part & 1) == 0)
      __builtin_nontemporal_store(pair, reinterpret_cast<uint32_t*>(codes + 16 * b + 2 * part));
    if (b < nblocks && part == 0) e8m0[b] = (uint8_t)(e + 127);
  }
}

// ---------------------------------------------------------------------------
// e4m3fn (FP8 page, precision management): scale = fp32(amax / 448),
// code = RNE(fp32(x / scale)) saturated at 448.
// ---------------------------------------------------------------------------

// Round a finite fp32 to e4m3fn, nearest-even, saturating at +-448.
__device__ __forceinline__ uint32_t e4m3fn_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                                 // below 2^-6: step 2^-9
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // exact scale, 0..8
  }
  const uint32_t ua = __builtin_bit_cast(uint32_t, a);
  // keep 3 mantissa bits, round to nearest even on the 20 dropped bits
  const uint32_t r = (ua + 0x7ffffu + ((ua >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));                     // rebias 127 -> 7
}

__global__ void fp8_init_kernel(float* __restrict__ scale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *reinterpret_cast<uint32_t*>(scale) = 0u;
}

// max |x| into *scale (as its bit pattern; non-negative floats order as ints)
__global__ __launch_bounds__(256) void fp8_amax_kernel(const float* __restrict__ x, int64_t n,
                                                       float* __restrict__ scale) {
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    m = fmaxf(m, fabsf(x[i]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float bm = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(scale), __builtin_bit_cast(unsigned int, bm));
  }
}

__device__ __forceinline__ float fp8_scale_of(float amax) {
  // fp32 quotient via fp64: double rounding of a quotient of two floats
  // through binary64 equals the correctly rounded fp32 quotient
  return amax == 0.f ? 1.0f : (float)((double)amax / 448.0);
}

__global__ __launch_bounds__(256) void fp8_cast_kernel(const float* __restrict__ x, int64_t n,
                                                       const float* __restrict__ amax_in,
                                                       uint8_t* __restrict__ codes) {
  const float s = fp8_scale_of(*amax_in);
  const double sd = (double)s;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const float v = (float)((double)x[i] / sd);
    codes[i] = (uint8_t)e4m3fn_rne(v);
  }
}

__global__ void fp8_finish_kernel(float* __restrict__ scale) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *scale = fp8_scale_of(*scale);
}

// With a workspace: the same scale and codes in two launches and no
// atomics.  Pass 1 writes one partial max |x| per block; in pass 2 every
// block reduces all partials itself (at most kFp8Partials floats), forms the
// scale and casts its share, four elements per thread; block 0 stores the
// scale.  count % 4 == 0 and x 16-byte aligned.
__global__ __launch_bounds__(256) void fp8_partial_amax_kernel(const float* __restrict__ x,
                                                               int64_t n4,
                                                               float* __restrict__ partials) {
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const floatx4* x4 = reinterpret_cast<const floatx4*>(x);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const floatx4 v = x4[i];
    m = fmaxf(fmaxf(m, fmaxf(fabsf(v[0]), fabsf(v[1]))), fmaxf(fabsf(v[2]), fabsf(v[3])));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    partials[blockIdx.x] = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
}

__global__ __launch_bounds__(256) void fp8_cast_partials_kernel(
    const float* __restrict__ x, int64_t n4, const float* __restrict__ partials, int np,
    uint32_t* __restrict__ codes4, float* __restrict__ scale) {
  float m = (int)threadIdx.x < np ? partials[threadIdx.x] : 0.f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  const float s = fp8_scale_of(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3])));
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale = s;
  const double sd = (double)s;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const floatx4* x4 = reinterpret_cast<const floatx4*>(x);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const floatx4 v = x4[i];
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= e4m3fn_rne((float)((double)v[j] / sd)) << (8 * j);
    codes4[i] = w;
  }
}

}  // namespace

hipError_t launch_quantize_fp8_ws(const float* x, int64_t count, uint8_t* codes, float* scale,
                                  float* partials, hipStream_t stream) {
  const int64_t n4 = count / 4;
  const int64_t want = cdiv(n4, 256);
  const int np = (int)(want < kFp8Partials ? want : kFp8Partials);
  if (np > 0) {
    hipLaunchKernelGGL(fp8_partial_amax_kernel, dim3((unsigned)np), dim3(256), 0, stream, x, n4,
                       partials);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t grid = want < 1 ? 1 : (want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fp8_cast_partials_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, n4,
                     (const float*)partials, np, reinterpret_cast<uint32_t*>(codes), scale);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const float* x, int64_t rows, int64_t K, uint8_t* codes,
                                 uint8_t* e8m0, hipStream_t stream) {
  const int64_t blocks = rows * (K / 32);
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp4_kernel, dim3((unsigned)cdiv(blocks, 32 * kQBlocksPerLane)),
                     dim3(256), 0, stream, x, codes, e8m0, blocks);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(const float* x, int64_t count, uint8_t* codes, float* scale,
                               hipStream_t stream) {
  hipLaunchKernelGGL(fp8_init_kernel, dim3(1), dim3(64), 0, stream, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (count > 0) {
    const int64_t want = cdiv(count, 256);
    const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(fp8_amax_kernel, dim3(grid), dim3(256), 0, stream, x, count, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(fp8_cast_kernel, dim3(grid), dim3(256), 0, stream, x, count,
                       (const float*)scale, codes);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fp8_finish_kernel, dim3(1), dim3(64), 0, stream, scale);
  return hipGetLastError();
}

}  // namespace qgemm
