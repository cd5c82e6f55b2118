// Weight prepack: canonical layouts of the pages -> fragment tiles.
//
// Offline, once per weight; one thread per output 32-bit word, so every
// output byte (padding included) is written exactly once.  The tile geometry
// is described in qgemm_common.h.
#include "qgemm_common.h"

namespace qgemm {
namespace {

// W4A16 canonical input: uint8 [K/2, N], byte (j, n) holds k = 2j (low nibble)
// and k = 2j + 1 (high nibble) -- W4A16 page, section 2.
__device__ __forceinline__ uint32_t w4_code(const uint8_t* __restrict__ in, int64_t k,
                                            int64_t n, int64_t K, int64_t N) {
  if (k >= K || n >= N) return 8u;  // zero point: dequantizes to 0
  const uint32_t b = in[(k >> 1) * N + n];
  return (b >> (4 * (k & 1))) & 0xfu;
}

__global__ void prepack_w4_kernel(const uint8_t* __restrict__ in, uint32_t* __restrict__ out,
                                  int64_t K, int64_t N, int64_t KT, int64_t words) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= words) return;
  const int64_t tile = d >> 8;       // 256 words per 1 KB tile
  const int within = (int)(d & 255);
  const int lane = within >> 2;
  const int j = within & 3;
  const int64_t cg = tile / KT;
  const int64_t kt = tile - cg * KT;
  const int64_t n = cg * kTileN + (lane & 15);
  // word j of lane l feeds matrix step j: k = 32 j + 8 (l >> 4) + [0, 8)
  const int64_t kbase = kt * kTileK8 + 32 * j + 8 * (lane >> 4);
  // nibble p holds k offset (0, 2, 4, 6, 1, 3, 5, 7)[p]
  uint32_t word = 0;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int koff = (p < 4) ? 2 * p : 2 * (p - 4) + 1;
    word |= w4_code(in, kbase + koff, n, K, N) << (4 * p);
  }
  out[d] = word;
}

// W8A16 (int8 [K, N], stored biased by +128, bytes in matrix-step order) and
// FP8 (e4m3fn [K, N], as is, lane l holding k = 32 (l >> 4) + [0, 32)).
template <bool BIAS>
__global__ void prepack_k8_kernel(const uint8_t* __restrict__ in, uint32_t* __restrict__ out,
                                  int64_t K, int64_t N, int64_t KT, int64_t words) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= words) return;
  const int64_t tile = d >> 9;       // 512 words per 2 KB tile
  const int off = (int)(d & 511) * 4;
  const int h = off >> 10;
  const int lane = (off & 1023) >> 4;
  const int b0 = off & 15;
  const int64_t cg = tile / KT;
  const int64_t kt = tile - cg * KT;
  const int64_t n = cg * kTileN + (lane & 15);
  // W8A16: byte b of half h feeds step s = 2h + b/8: k = 32 s + 8 (l >> 4) + b % 8
  // FP8:    byte b of half h is k = 32 (l >> 4) + 16 h + b
  const int64_t k0 = BIAS ? kt * kTileK8 + 32 * (2 * h + (b0 >> 3)) + 8 * (lane >> 4) + (b0 & 7)
                          : kt * kTileK8 + 32 * (lane >> 4) + 16 * h + b0;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t k = k0 + i;
    uint32_t b = 0;
    if (k < K && n < N) b = in[k * N + n];
    if (BIAS) b = (b + 128u) & 0xffu;  // w + 128; padding becomes 0x80 (= 0)
    word |= b << (8 * i);
  }
  out[d] = word;
}

// MXFP4 codes: canonical uint8 [N, K/2] (element 2j low nibble of byte j).
// A tile byte holds elements k, k+1 with k even, exactly as the canonical
// byte (n, k/2) does, so this is a byte gather.
__global__ void prepack_mxfp4_codes_kernel(const uint8_t* __restrict__ in,
                                           uint32_t* __restrict__ out, int64_t K, int64_t N,
                                           int64_t KT, int64_t words) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= words) return;
  const int64_t tile = d >> 9;
  const int off = (int)(d & 511) * 4;
  const int h = off >> 10;
  const int lane = (off & 1023) >> 4;
  const int b0 = off & 15;
  const int64_t cg = tile / KT;
  const int64_t kt = tile - cg * KT;
  const int64_t n = cg * kTileN + (lane & 15);
  const int64_t kbyte0 = (kt * kTileK4 + 128 * h + 32 * (lane >> 4)) / 2 + b0;
  const int64_t row_bytes = K / 2;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t kb = kbyte0 + i;
    const uint32_t b = (kb < row_bytes && n < N) ? in[n * row_bytes + kb] : 0u;
    word |= b << (8 * i);
  }
  out[d] = word;
}

// MXFP4 scales: canonical uint8 [N, K/32]; tile byte 2l + h is block
// 8kt + 4h + (l >> 4) of column cg*16 + (l & 15).  Padding: 127 (= 1.0).
// Scale segment: for each group of 8 column tiles (128 columns) and each
// 128-element K step ks (two steps per code tile), 512 bytes ordered
// [lane 64][tile 8]: byte (lane, j) is the E8M0 of column 128*c8 + 16*j +
// (lane & 15) for block 4*ks + (lane >> 4).
__global__ void prepack_mxfp4_scales_kernel(const uint8_t* __restrict__ in,
                                            uint32_t* __restrict__ out, int64_t K, int64_t N,
                                            int64_t KS, int64_t words) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= words) return;
  const int64_t chunk = d >> 7;      // 128 words per 512 B (group, step) chunk
  const int w = (int)(d & 127);
  const int64_t c8 = chunk / KS;
  const int64_t ks = chunk - c8 * KS;
  const int lane = w >> 1;
  const int64_t blocks = K / 32;
  const int64_t blk = 4 * ks + (lane >> 4);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = 4 * (w & 1) + i;
    const int64_t n = (8 * c8 + j) * kTileN + (lane & 15);
    const uint32_t e = (blk < blocks && n < N) ? in[n * blocks + blk] : (uint32_t)kE8M0One;
    word |= e << (8 * i);
  }
  out[d] = word;
}

// Metadata segment of the grouped formats: one thread per 4-byte entry
// ((cg * KT + kt) * 16 + c) * NGT + j (layout in qgemm_common.h).
__global__ void prepack_group_meta_kernel(const uint16_t* __restrict__ scales,
                                          const uint8_t* __restrict__ zeros, bool w4,
                                          uint32_t* __restrict__ out, int64_t K, int64_t N,
                                          int64_t KT, int64_t group_k, int64_t group_n, int ngt,
                                          int64_t entries) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= entries) return;
  const int j = (int)(d % ngt);
  const int64_t col = d / ngt;              // (cg * KT + kt) * 16 + c
  const int c = (int)(col & 15);
  const int64_t tile = col >> 4;
  const int64_t cg = tile / KT;
  const int64_t kt = tile - cg * KT;
  const int64_t n = cg * kTileN + c;
  const int64_t k0 = kt * kTileK8 + j * (kTileK8 / ngt);
  const int64_t ng_count = cdiv(N, group_n);
  int z = w4 ? 8 : 0;
  uint16_t s_bits = 0;                      // padding: scale 0
  if (n < N && k0 < K) {
    const int64_t e = (k0 / group_k) * ng_count + n / group_n;
    s_bits = scales[e];
    if (zeros != nullptr) z = w4 ? (int)zeros[e] : (int)(int8_t)zeros[e];
  }
  const float zc = (float)((w4 ? 1024 : 1152) + z);   // exact in fp16
  out[d] = (uint32_t)f32_to_f16_bits(zc) | ((uint32_t)s_bits << 16);
}

// NVFP4 codes: one thread per output word; word s of lane l of tile (cg, kt)
// = the 4 source bytes holding k = kt*128 + 32s + 8g + [0, 8) of column n.
__global__ void prepack_nvfp4_codes_kernel(const uint8_t* __restrict__ in,
                                           uint32_t* __restrict__ out, int64_t K, int64_t N,
                                           int64_t KT, int64_t words) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= words) return;
  const int64_t tile = d >> 8;               // 256 words per 1 KB tile
  const int within = (int)(d & 255);
  const int lane = within >> 2, s = within & 3;
  const int64_t cg = tile / KT, kt = tile - cg * KT;
  const int64_t n = cg * kTileN + (lane & 15);
  const int64_t k0 = kt * kTileK8 + 32 * s + 8 * (lane >> 4);
  uint32_t word = 0;
  if (n < N && k0 < K) {                      // K % 16 == 0: all 8 in range or none
    const uint8_t* src = in + n * (K / 2) + k0 / 2;
    word = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) |
           ((uint32_t)src[3] << 24);
  }
  out[d] = word;
}

// NVFP4 block scales: one thread per output word; word w of tile (cg, kt) is
// column w / 2, half h = w % 2, bytes s = 0..3: block kt*8 + 2s + h.
__global__ void prepack_nvfp4_scales_kernel(const uint8_t* __restrict__ in,
                                            uint32_t* __restrict__ out, int64_t K, int64_t N,
                                            int64_t KT, int64_t words) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d >= words) return;
  const int64_t tile = d >> 5;                // 32 words per 128 B
  const int w = (int)(d & 31);
  const int c = w >> 1, h = w & 1;
  const int64_t cg = tile / KT, kt = tile - cg * KT;
  const int64_t n = cg * kTileN + c;
  const int64_t blocks = K / 16;
  uint32_t word = 0;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t b = kt * 8 + 2 * s + h;
    const uint32_t e = (n < N && b < blocks) ? in[n * blocks + b] : 0u;
    word |= e << (8 * s);
  }
  out[d] = word;
}

__global__ void zero_words_kernel(uint32_t* __restrict__ out, int64_t words) {
  const int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (d < words) out[d] = 0u;
}

inline unsigned grid_for(int64_t words, int block) { return (unsigned)cdiv(words, block); }

}  // namespace

hipError_t launch_prepack(int fmt, const void* w, const void* w_scales, void* packed, int64_t K,
                          int64_t N, hipStream_t stream) {
  const PackGeom g = pack_geom(fmt, K, N);
  const int block = 256;
  const int64_t words = g.codes / 4;
  if (words == 0) return hipSuccess;
  const uint8_t* in = static_cast<const uint8_t*>(w);
  uint32_t* out = static_cast<uint32_t*>(packed);
  switch (fmt) {
    case 1:
      hipLaunchKernelGGL(prepack_w4_kernel, dim3(grid_for(words, block)), dim3(block), 0,
                         stream, in, out, K, N, g.kt, words);
      break;
    case 2:
      hipLaunchKernelGGL(prepack_k8_kernel<true>, dim3(grid_for(words, block)), dim3(block), 0,
                         stream, in, out, K, N, g.kt, words);
      break;
    case 4:
      hipLaunchKernelGGL(prepack_k8_kernel<false>, dim3(grid_for(words, block)), dim3(block), 0,
                         stream, in, out, K, N, g.kt, words);
      break;
    case 3: {
      hipLaunchKernelGGL(prepack_mxfp4_codes_kernel, dim3(grid_for(words, block)), dim3(block),
                         0, stream, in, out, K, N, g.kt, words);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      // zero the alignment gap between the segments, then the scale tiles
      const int64_t gap_words = (g.scales - g.codes) / 4;
      if (gap_words > 0) {
        hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, out + words,
                           gap_words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      const int64_t swords = (g.total - g.scales) / 4;
      hipLaunchKernelGGL(prepack_mxfp4_scales_kernel, dim3(grid_for(swords, block)),
                         dim3(block), 0, stream, static_cast<const uint8_t*>(w_scales),
                         out + g.scales / 4, K, N, 2 * g.kt, swords);
      break;
    }
    case 7: {
      hipLaunchKernelGGL(prepack_nvfp4_codes_kernel, dim3(grid_for(words, block)), dim3(block),
                         0, stream, in, out, K, N, g.kt, words);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t gap_words = (g.scales - g.codes) / 4;
      if (gap_words > 0) {
        hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, out + words,
                           gap_words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      const int64_t swords = (g.total - g.scales) / 4;
      hipLaunchKernelGGL(prepack_nvfp4_scales_kernel, dim3(grid_for(swords, block)),
                         dim3(block), 0, stream, static_cast<const uint8_t*>(w_scales),
                         out + g.scales / 4, K, N, g.kt, swords);
      break;
    }
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prepack_grouped(int fmt, const void* w, const void* scales, const void* zeros,
                                  int64_t group_k, int64_t group_n, void* packed, int64_t K,
                                  int64_t N, hipStream_t stream) {
  const PackGeom g = grouped_geom(fmt, K, N, group_k);
  hipError_t e = launch_prepack(fmt == 5 ? 1 : 2, w, nullptr, packed, K, N, stream);
  if (e != hipSuccess) return e;
  uint32_t* out = static_cast<uint32_t*>(packed);
  const int64_t gap_words = (g.scales - g.codes) / 4;
  if (gap_words > 0) {
    hipLaunchKernelGGL(zero_words_kernel, dim3(1), dim3(64), 0, stream, out + g.codes / 4,
                       gap_words);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int ngt = grouped_ngt(group_k);
  const int64_t entries = (g.total - g.scales) / 4;
  if (entries == 0) return hipSuccess;
  const int block = 256;
  hipLaunchKernelGGL(prepack_group_meta_kernel, dim3(grid_for(entries, block)), dim3(block), 0,
                     stream, static_cast<const uint16_t*>(scales),
                     static_cast<const uint8_t*>(zeros), fmt == 5, out + g.scales / 4, K, N,
                     g.kt, group_k, group_n, ngt, entries);
  return hipGetLastError();
}

}  // namespace qgemm
