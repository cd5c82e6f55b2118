// Measurement reference kernels (not part of any GEMM).
//
// Streaming read: how fast this GPU reads a buffer of a given size from HBM, measured with the access pattern of the weight stream
// (16-byte non-temporal loads per lane, several in flight per lane, whole
// contiguous chunks per workgroup).  The W8A16 page's performance analysis
// compares INT8 and FP16 weight read bandwidth; this kernel gives the plain
// read rate that such a comparison (and the decode GEMMs' roofline fraction)
// is read against.  It moves no data anywhere but one word per workgroup.
#include "qgemm_common.h"

namespace qgemm {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;    // 16-byte loads in flight per lane

// Workgroup b reads 16-byte words [b * per_wg, min((b + 1) * per_wg, n16))
// and folds them into one word so that no load can be dropped.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(
    const uintx4* __restrict__ buf, int64_t n16, int64_t per_wg, uint32_t* __restrict__ sink) {
  const int64_t begin = (int64_t)blockIdx.x * per_wg;
  const int64_t end = begin + per_wg < n16 ? begin + per_wg : n16;
  uint32_t acc = 0;
  for (int64_t i = begin + threadIdx.x; i < end; i += kProbeThreads * kProbeUnroll) {
    uintx4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + (int64_t)kProbeThreads * u;
      v[u] = j < end ? __builtin_nontemporal_load(buf + j) : uintx4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// Matrix pipe: back-to-back v_mfma_scale_f32_32x32x64_f8f6f4 on operands
// held in registers, nothing else issued.  Each lane loads 4 A and 4 B
// fragments (and, for FP4, 8 E8M0 scale bytes) of random data once, then
// every iteration runs all 16 (A, B) pairs into 16 independent accumulators,
// so consecutive instructions see different operands and the matrix pipe
// toggles the way it does on real data.  The accumulators fold into one word
// per workgroup.  This gives the practical ceiling of the instruction on this
// GPU, clock throttling under the power the pipe draws included.
template <bool FP4>
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(
    const uintx4* __restrict__ ops, int64_t iters, float* __restrict__ sink) {
  constexpr int fmt = FP4 ? kFmtFP4 : kFmtFP8;
  const uintx4* p = ops + (int64_t)(blockIdx.x * kProbeThreads + threadIdx.x) * 17;
  intx8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uintx4 lo = p[2 * i], hi = p[2 * i + 1];
    const uintx4 lo2 = p[8 + 2 * i], hi2 = p[8 + 2 * i + 1];
    // FP4 operands use 16 bytes of a fragment, FP8 all 32
    a[i] = intx8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 FP4 ? 0 : (int)hi[0], FP4 ? 0 : (int)hi[1], FP4 ? 0 : (int)hi[2],
                 FP4 ? 0 : (int)hi[3]};
    b[i] = intx8{(int)lo2[0], (int)lo2[1], (int)lo2[2], (int)lo2[3],
                 FP4 ? 0 : (int)hi2[0], FP4 ? 0 : (int)hi2[1], FP4 ? 0 : (int)hi2[2],
                 FP4 ? 0 : (int)hi2[3]};
  }
  // E8M0 scales 120..127 (FP4) keep every product finite; unit scales (FP8)
  const uintx4 sv = p[16];
  const int sa = FP4 ? (int)(0x78787878u | (sv[0] & 0x07070707u)) : (int)0x7f7f7f7f;
  const int sb = FP4 ? (int)(0x78787878u | (sv[1] & 0x07070707u)) : (int)0x7f7f7f7f;
  floatx16 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[4 * i + j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a[i], b[j], acc[4 * i + j], fmt, fmt, 0, sa, 0, sb);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  __shared__ float part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] + part[1] + part[2] + part[3];
}

}  // namespace

hipError_t launch_mfma_probe(bool fp4, const void* ops, int64_t iters, float* sink,
                             int64_t workgroups, hipStream_t stream) {
  if (fp4)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3((unsigned)workgroups), dim3(kProbeThreads),
                       0, stream, static_cast<const uintx4*>(ops), iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3((unsigned)workgroups), dim3(kProbeThreads),
                       0, stream, static_cast<const uintx4*>(ops), iters, sink);
  return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int64_t workgroups,
                             hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  // whole 1 KB pieces per workgroup, so every chunk starts on a cache line
  const int64_t per_wg = cdiv(cdiv(n16, workgroups), 64) * 64;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, stream,
                     static_cast<const uintx4*>(buf), n16, per_wg, sink);
  return hipGetLastError();
}

}  // namespace qgemm
