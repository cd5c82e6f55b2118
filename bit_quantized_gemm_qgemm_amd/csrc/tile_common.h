// Device helpers shared by the 256 x 256 tile kernels (the weight-only
// pipeline in tile_wo256.hip, the MXFP4 / FP8 kernels in tile_mx256.hip) and
// the host-side range check in tile_gemm.hip: buffer resources, global->LDS
// copies, barrier macros, launch arguments and the XCD-aware tile walk.
#pragma once

#include "qgemm_common.h"

namespace qgemm {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBig = 256;                       // output rows and columns per workgroup
constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset past every buffer
constexpr int kCTileBytes = kBig * kBig * 2;    // one bf16 / fp16 output tile

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer, 32-bit data format; offsets >= bytes read as zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// lane l of the wave deposits its 16 (or 4) bytes at lds_wave_base + 16 l (4 l)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base,
                                      uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voffset, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base,
                                     uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 4, voffset, 0, 0, 0);
}

// s_waitcnt with vmcnt = n (expcnt and lgkmcnt left alone), then a bare
// workgroup barrier; the scheduler may move nothing across either.
#define QG_WAIT_VM_BARRIER(n)                                                           \
  do {                                                                                  \
    __builtin_amdgcn_sched_barrier(0);                                                  \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | 0x70 | 0xF00);  \
    __builtin_amdgcn_s_barrier();                                                       \
    __builtin_amdgcn_sched_barrier(0);                                                  \
  } while (0)

// vmcnt = n and lgkmcnt = 0, then a bare workgroup barrier
#define QG_WAIT_VM_LGKM_BARRIER(n)                                              \
  do {                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                          \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | 0x70);  \
    __builtin_amdgcn_s_barrier();                                               \
    __builtin_amdgcn_sched_barrier(0);                                          \
  } while (0)

// Launch arguments of the 256 x 256 kernels (byte sizes bound the buffer
// resources; KS counts the kernel's K steps).
struct PipeArgs {
  int M, N, K, KT, KS, CG, tiles_m, tiles_n;
  uint32_t a_bytes, w_bytes, asc_bytes, wsc_bytes;
};

// First output row and first 16-column group of this workgroup's tile.
// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Give each XCD a contiguous range of tile ids, and walk that range in
// groups of 4 tile rows so the tiles resident on one XCD share A rows and W
// columns in its L2.
struct TileOrigin {
  int m0, cg0;
};

__device__ __forceinline__ TileOrigin tile_origin(const PipeArgs& g) {
  const int T = g.tiles_m * g.tiles_n;
  const int bid = blockIdx.x;
  const int id = (T % 8 == 0) ? (bid % 8) * (T / 8) + bid / 8 : bid;
  constexpr int GM = 4;
  const int group = id / (GM * g.tiles_n);
  const int first_m = group * GM;
  const int gsize = min(g.tiles_m - first_m, GM);
  const int in_group = id - group * GM * g.tiles_n;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  return TileOrigin{tm * kBig, tn * (kBig / 16)};
}

}  // namespace
}  // namespace qgemm
