// Streaming-read reference kernel: how fast this GPU reads a buffer of a
// given size from HBM, measured with the access pattern of the weight stream
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

}  // namespace

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
