// LDS-tiled matrix-core GEMM for MXFP4 x MXFP4 and FP8 e4m3fn (any M).
//
// The MXFP4 page (section 2) tiles C into B_M x B_N blocks per workgroup and
// sums, per 32-element micro-block, S_A * S_W * dot(A, W) (eq. 1) with the
// scale product done as an exponent add (eq. 2).  On gfx950 that whole step is
// one instruction: v_mfma_scale_f32_16x16x128_f8f6f4 takes 128 K-elements of
// FP4 (or FP8) codes per lane group and one E8M0 byte per lane, applies
// 2^(E_A-127) * 2^(E_W-127) to each 32-element block product in hardware and
// accumulates in fp32.  FP8 (FP8 page) uses the same instruction with e4m3
// operands and unit scales; its per-tensor scales multiply the fp32 result
// once in the epilogue.
//
// Data flow per K step (128 bytes of K per row: 256 FP4 or 128 FP8 elements):
//   A (row-major activations) -> LDS, 16-byte chunks XOR-swizzled by row so
//     that both the row-wise stores and the fragment reads are bank-conflict
//     free;
//   W (prepacked fragment tiles) -> LDS as is: already in lane order, so the
//     fragment reads are linear;
//   MXFP4 scales -> LDS, rearranged for A into the same [fragment][lane][h]
//     order the W scale tiles already have, so each lane reads one 16-bit
//     word per fragment holding the scales of both 128-element halves.
// Double-buffered: the global loads of step k+1 are in flight while the
// matrix cores work on step k; one barrier per step.
#include "qgemm_common.h"

namespace qgemm {
namespace {

constexpr int kKBytes = 128;                 // bytes of K per row per step
constexpr int kThreads = 256;                // 4 waves, 2 x 2

template <int FM, int FN>
struct TileCfg {
  static constexpr int BM = 2 * 16 * FM;     // rows per workgroup
  static constexpr int BN = 2 * 16 * FN;     // columns per workgroup
  static constexpr int A_BYTES = BM * kKBytes;
  static constexpr int B_BYTES = BN * kKBytes;
  static constexpr int SA_BYTES = BM * 8;    // MXFP4: 8 scale bytes per row
  static constexpr int SB_BYTES = BN * 8;
  static constexpr int A_LOADS = A_BYTES / 16 / kThreads;
  static constexpr int B_LOADS = B_BYTES / 16 / kThreads;
  static_assert(A_LOADS * 16 * kThreads == A_BYTES, "A tile must split evenly");
  static_assert(B_LOADS * 16 * kThreads == B_BYTES, "B tile must split evenly");
};

template <bool FP4, int FM, int FN>
struct StageRegs {
  uintx4 a[TileCfg<FM, FN>::A_LOADS];
  uintx4 b[TileCfg<FM, FN>::B_LOADS];
  uintx2 sa;   // FP4: 8 A scale bytes of one row (threads < BM)
  uintx4 sb;   // FP4: 16 W scale bytes (threads < SB_BYTES / 16)
};

template <bool FP4, int FM, int FN>
__device__ __forceinline__ void global_load_stage(
    StageRegs<FP4, FM, FN>& r, const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ w_sc, int m0, int cg0, int kt,
    int M, int row_bytes, int sc_cols, int KT, int CG) {
  using C = TileCfg<FM, FN>;
  const int t = threadIdx.x;
  const int kbyte0 = kt * kKBytes;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int c = t + kThreads * j;
    const int row = c >> 3;
    const int ch = c & 7;
    const int gm = m0 + row;
    const int kb = kbyte0 + 16 * ch;
    if (gm < M && kb < row_bytes)
      r.a[j] = *reinterpret_cast<const uintx4*>(a + (int64_t)gm * row_bytes + kb);
    else
      r.a[j] = uintx4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int c = t + kThreads * j;
    const int tile = c >> 7;            // 128 chunks per 2 KB tile
    const int off = (c & 127) * 16;
    const int cg = min(cg0 + tile, CG - 1);   // past-the-end groups: discarded
    r.b[j] = *reinterpret_cast<const uintx4*>(wp + ((int64_t)cg * KT + kt) * kTileBytes + off);
  }
  if constexpr (FP4) {
    if (t < C::BM) {
      const int gm = m0 + t;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int blk = 8 * kt + i;
        const uint32_t e = (gm < M && blk < sc_cols) ? a_sc[(int64_t)gm * sc_cols + blk]
                                                     : (uint32_t)kE8M0One;
        if (i < 4) lo |= e << (8 * i);
        else hi |= e << (8 * (i - 4));
      }
      r.sa = uintx2{lo, hi};
    }
    if (t < C::SB_BYTES / 16) {
      const int tile = t >> 3;          // 8 x 16 B per 128 B scale tile
      const int cg = min(cg0 + tile, CG - 1);
      r.sb = *reinterpret_cast<const uintx4*>(w_sc + ((int64_t)cg * KT + kt) * kScaleTileBytes +
                                              16 * (t & 7));
    }
  }
}

template <bool FP4, int FM, int FN>
__device__ __forceinline__ void lds_store_stage(const StageRegs<FP4, FM, FN>& r, uint8_t* lds_a,
                                                uint8_t* lds_b, uint8_t* lds_sa,
                                                uint8_t* lds_sb) {
  using C = TileCfg<FM, FN>;
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < C::A_LOADS; ++j) {
    const int c = t + kThreads * j;
    const int row = c >> 3;
    const int ch = c & 7;
    *reinterpret_cast<uintx4*>(lds_a + row * kKBytes + 16 * (ch ^ (row & 7))) = r.a[j];
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int c = t + kThreads * j;
    *reinterpret_cast<uintx4*>(lds_b + 16 * c) = r.b[j];
  }
  if constexpr (FP4) {
    if (t < C::BM) {
      // row t, block i -> fragment t/16, lane 16*(i%4) + t%16, half i/4
      const int frag = t >> 4;
      const int rl = t & 15;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t e = ((i < 4 ? r.sa[0] : r.sa[1]) >> (8 * (i & 3))) & 0xffu;
        lds_sa[frag * 128 + 2 * (16 * (i & 3) + rl) + (i >> 2)] = (uint8_t)e;
      }
    }
    if (t < C::SB_BYTES / 16) *reinterpret_cast<uintx4*>(lds_sb + 16 * t) = r.sb;
  }
}

template <bool FP4, int FM, int FN>
__device__ __forceinline__ void compute_stage(const uint8_t* lds_a, const uint8_t* lds_b,
                                              const uint8_t* lds_sa, const uint8_t* lds_sb,
                                              floatx4 (&acc)[FM][FN], int wm, int wn,
                                              int lane) {
  const int g = lane >> 4;
  if constexpr (!FP4) {
    intx8 af[FM];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int row = wm * 16 * FM + fm * 16 + (lane & 15);
      const uint8_t* rp = lds_a + row * kKBytes;
      const uintx4 lo = *reinterpret_cast<const uintx4*>(rp + 16 * ((2 * g) ^ (row & 7)));
      const uintx4 hi = *reinterpret_cast<const uintx4*>(rp + 16 * ((2 * g + 1) ^ (row & 7)));
      af[fm] = intx8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const uint8_t* tp = lds_b + (wn * FN + fn) * kTileBytes + 16 * lane;
      const uintx4 lo = *reinterpret_cast<const uintx4*>(tp);
      const uintx4 hi = *reinterpret_cast<const uintx4*>(tp + 1024);
      const intx8 bf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[fm], bf, acc[fm][fn], kFmtFP8, kFmtFP8, 0, kE8M0One, 0, kE8M0One);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      intx8 af[FM];
      int sa[FM];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int frag = wm * FM + fm;
        const int row = frag * 16 + (lane & 15);
        const uintx4 v = *reinterpret_cast<const uintx4*>(lds_a + row * kKBytes +
                                                          16 * ((g + 4 * h) ^ (row & 7)));
        af[fm] = intx8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(lds_sa + frag * 128 + 2 * lane);
        sa[fm] = (int)((s2 >> (8 * h)) & 0xffu);
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int tile = wn * FN + fn;
        const uintx4 v =
            *reinterpret_cast<const uintx4*>(lds_b + tile * kTileBytes + 1024 * h + 16 * lane);
        const intx8 bf = {(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(lds_sb + tile * 128 + 2 * lane);
        const int sb = (int)((s2 >> (8 * h)) & 0xffu);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[fm], bf, acc[fm][fn], kFmtFP4, kFmtFP4, 0, sa[fm], 0, sb);
      }
    }
  }
}

template <bool FP4, int FM, int FN>
__global__ __launch_bounds__(kThreads) void tile_gemm_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ w_sc,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b,
    uint16_t* __restrict__ c, int M, int N, int K, int KT, int CG, int tiles_n) {
  using C = TileCfg<FM, FN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][C::A_BYTES + C::B_BYTES +
                                                       (FP4 ? C::SA_BYTES + C::SB_BYTES : 0)];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int tm = blockIdx.x / tiles_n;
  const int tn = blockIdx.x - tm * tiles_n;
  const int m0 = tm * C::BM;
  const int cg0 = tn * (C::BN / 16);
  const int row_bytes = FP4 ? K / 2 : K;
  const int sc_cols = K / 32;

  floatx4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto lds = [&](int buf, int part) -> uint8_t* {
    uint8_t* base = &smem[buf][0];
    if (part == 0) return base;
    if (part == 1) return base + C::A_BYTES;
    if (part == 2) return base + C::A_BYTES + C::B_BYTES;
    return base + C::A_BYTES + C::B_BYTES + C::SA_BYTES;
  };

  StageRegs<FP4, FM, FN> regs;
  if (KT > 0) {
    global_load_stage<FP4, FM, FN>(regs, a, a_sc, wp, w_sc, m0, cg0, 0, M, row_bytes, sc_cols,
                                   KT, CG);
    lds_store_stage<FP4, FM, FN>(regs, lds(0, 0), lds(0, 1), lds(0, 2), lds(0, 3));
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < KT;
    if (more)
      global_load_stage<FP4, FM, FN>(regs, a, a_sc, wp, w_sc, m0, cg0, kt + 1, M, row_bytes,
                                     sc_cols, KT, CG);
    compute_stage<FP4, FM, FN>(lds(cur, 0), lds(cur, 1), lds(cur, 2), lds(cur, 3), acc, wm, wn,
                               lane);
    if (more) lds_store_stage<FP4, FM, FN>(regs, lds(cur ^ 1, 0), lds(cur ^ 1, 1),
                                           lds(cur ^ 1, 2), lds(cur ^ 1, 3));
    __syncthreads();
  }

  // epilogue: lane holds rows 4*(lane>>4)+i, column lane&15 of each fragment
  const float s = FP4 ? 1.0f : (*scale_a) * (*scale_b);
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int gn = (cg0 + wn * FN + fn) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gm = m0 + wm * 16 * FM + fm * 16 + 4 * (lane >> 4) + i;
        if (gm < M && gn < N) c[(int64_t)gm * N + gn] = f32_to_bf16_rne(acc[fm][fn][i] * s);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Large tiles: 256 x 256 per workgroup, 128 x 128 per wave (8 x 8 fragments,
// 256 fp32 accumulators per lane), operands moved global -> LDS by the
// buffer unit directly (no VGPR staging, no LDS store instructions).  Buffer
// resources bound every operand, so rows past M, column groups past N and K
// chunks past K read as zero without predication.  Two LDS stages; the loads
// of step k+1 run while the matrix cores work on step k.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBig = 256;

template <bool FP4>
struct BigCfg {
  static constexpr int A = kBig * kKBytes;                      // 32 KB
  static constexpr int B = kBig * kKBytes;                      // 32 KB
  static constexpr int SA = FP4 ? kBig * 8 : 0;                 // [row][8 blocks]
  static constexpr int SB = FP4 ? (kBig / 16) * kScaleTileBytes : 0;
  static constexpr int STAGE = A + B + SA + SB;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  // raw buffer, 32-bit data format; offsets >= bytes read as zero
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}

// lane l of the wave deposits its `size` bytes at lds_wave_base + size * l
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t r, uint8_t* lds_wave_base,
                                           uint32_t voffset, int size) {
  if (size == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voffset, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 4, voffset, 0, 0, 0);
}

constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset past every buffer

struct BigArgs {
  int M, N, K, KT, CG, tiles_m, tiles_n;
  uint32_t a_bytes, w_bytes, asc_bytes, wsc_bytes;
};

template <bool FP4>
__device__ __forceinline__ void big_issue_stage(uint8_t* stage, int kt, int wave, int lane,
                                                int m0, int cg0, const BigArgs& g,
                                                __amdgpu_buffer_rsrc_t ra,
                                                __amdgpu_buffer_rsrc_t rw,
                                                __amdgpu_buffer_rsrc_t rsa,
                                                __amdgpu_buffer_rsrc_t rsw) {
  using C = BigCfg<FP4>;
  const int row_bytes = FP4 ? g.K / 2 : g.K;
  // A: 32 chunks of 1 KB (8 rows x 128 B); chunk 16-byte slots XOR-swizzled by row
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = wave * 8 + j;
    const int r = q * 8 + (lane >> 3);
    const int chunk = (lane & 7) ^ (r & 7);
    const int kb = kt * kKBytes + 16 * chunk;
    const uint32_t off = (kb < row_bytes) ? (uint32_t)(m0 + r) * (uint32_t)row_bytes + kb
                                          : kOutOfRange;
    dma_to_lds(ra, stage + q * 1024, off, 16);
  }
  // W: 16 fragment tiles of 2 KB, copied as is
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int q = wave * 8 + j;
    const uint32_t off =
        ((uint32_t)(cg0 + (q >> 1)) * g.KT + kt) * kTileBytes + 1024u * (q & 1) + 16u * lane;
    dma_to_lds(rw, stage + C::A + q * 1024, off, 16);
  }
  if constexpr (FP4) {
    // A scales: 256 rows x 8 bytes, row-major, in 4-byte pieces (K % 128 == 0)
    const int sc_cols = g.K / 32;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = wave * 2 + j;
      const int d = q * 64 + lane;
      const int r = d >> 1;
      const int blk = 8 * kt + 4 * (d & 1);
      const uint32_t off = (blk < sc_cols) ? (uint32_t)(m0 + r) * (uint32_t)sc_cols + blk
                                           : kOutOfRange;
      dma_to_lds(rsa, stage + C::A + C::B + q * 256, off, 4);
    }
    // W scales: 16 tiles x 128 B
    if (wave < 2) {
      const int t = 8 * wave + (lane >> 3);
      const uint32_t off =
          ((uint32_t)(cg0 + t) * g.KT + kt) * kScaleTileBytes + 16u * (lane & 7);
      dma_to_lds(rsw, stage + C::A + C::B + C::SA + wave * 1024, off, 16);
    }
  }
}

template <bool FP4>
__device__ __forceinline__ void big_compute_stage(const uint8_t* stage, floatx4 (&acc)[8][8],
                                                  int wm, int wn, int lane) {
  using C = BigCfg<FP4>;
  const uint8_t* la = stage;
  const uint8_t* lb = stage + C::A;
  const int g = lane >> 4;
  if constexpr (!FP4) {
    intx8 af[8];
#pragma unroll
    for (int fm = 0; fm < 8; ++fm) {
      const int row = wm * 128 + fm * 16 + (lane & 15);
      const uint8_t* rp = la + row * kKBytes;
      const uintx4 lo = *reinterpret_cast<const uintx4*>(rp + 16 * ((2 * g) ^ (row & 7)));
      const uintx4 hi = *reinterpret_cast<const uintx4*>(rp + 16 * ((2 * g + 1) ^ (row & 7)));
      af[fm] = intx8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int fn = 0; fn < 8; ++fn) {
      const uint8_t* tp = lb + (wn * 8 + fn) * kTileBytes + 16 * lane;
      const uintx4 lo = *reinterpret_cast<const uintx4*>(tp);
      const uintx4 hi = *reinterpret_cast<const uintx4*>(tp + 1024);
      const intx8 bf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
      for (int fm = 0; fm < 8; ++fm)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            af[fm], bf, acc[fm][fn], kFmtFP8, kFmtFP8, 0, kE8M0One, 0, kE8M0One);
    }
  } else {
    const uint8_t* lsa = stage + C::A + C::B;
    const uint8_t* lsb = lsa + C::SA;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      intx8 af[8];
      int sa[8];
#pragma unroll
      for (int fm = 0; fm < 8; ++fm) {
        const int row = wm * 128 + fm * 16 + (lane & 15);
        const uintx4 v = *reinterpret_cast<const uintx4*>(la + row * kKBytes +
                                                          16 * ((g + 4 * h) ^ (row & 7)));
        af[fm] = intx8{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        sa[fm] = lsa[row * 8 + g + 4 * h];
      }
#pragma unroll
      for (int fn = 0; fn < 8; ++fn) {
        const int t = wn * 8 + fn;
        const uintx4 v =
            *reinterpret_cast<const uintx4*>(lb + t * kTileBytes + 1024 * h + 16 * lane);
        const intx8 bf = {(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(lsb + t * 128 + 2 * lane);
        const int sb = (int)((s2 >> (8 * h)) & 0xffu);
#pragma unroll
        for (int fm = 0; fm < 8; ++fm)
          acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af[fm], bf, acc[fm][fn], kFmtFP4, kFmtFP4, 0, sa[fm], 0, sb);
      }
    }
  }
}

template <bool FP4>
__global__ __launch_bounds__(kThreads) void tile256_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ w_sc,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b,
    uint16_t* __restrict__ c, BigArgs g) {
  using C = BigCfg<FP4>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGE];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  // Workgroups are dispatched round-robin over the 8 XCDs (each with its own
  // L2).  Give each XCD a contiguous range of tile ids, and walk that range in
  // groups of 4 tile rows so the tiles resident on one XCD share A rows and W
  // columns in its L2.
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
  const int m0 = tm * kBig;
  const int cg0 = tn * (kBig / 16);

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, g.a_bytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wp, g.w_bytes);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(FP4 ? a_sc : a, FP4 ? g.asc_bytes : 0u);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(FP4 ? w_sc : wp, FP4 ? g.wsc_bytes : 0u);

  floatx4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  if (g.KT > 0) big_issue_stage<FP4>(smem, 0, wave, lane, m0, cg0, g, ra, rw, rsa, rsw);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < g.KT; ++kt) {
    uint8_t* cur = smem + (kt & 1) * C::STAGE;
    if (kt + 1 < g.KT)
      big_issue_stage<FP4>(smem + ((kt + 1) & 1) * C::STAGE, kt + 1, wave, lane, m0, cg0, g, ra,
                           rw, rsa, rsw);
    big_compute_stage<FP4>(cur, acc, wm, wn, lane);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  const float s = FP4 ? 1.0f : (*scale_a) * (*scale_b);
#pragma unroll
  for (int fm = 0; fm < 8; ++fm) {
#pragma unroll
    for (int fn = 0; fn < 8; ++fn) {
      const int gn = (cg0 + wn * 8 + fn) * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gm = m0 + wm * 128 + fm * 16 + 4 * (lane >> 4) + i;
        if (gm < g.M && gn < g.N) c[(int64_t)gm * g.N + gn] = f32_to_bf16_rne(acc[fm][fn][i] * s);
      }
    }
  }
}

template <bool FP4>
hipError_t launch_big(const void* a, const void* a_sc, const void* wp, const float* sa,
                      const float* sb, void* c, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
  const PackGeom pg = pack_geom(FP4 ? 3 : 4, K, N);
  BigArgs g;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.KT = (int)pg.kt;
  g.CG = (int)pg.cg;
  g.tiles_m = (int)cdiv(M, kBig);
  g.tiles_n = (int)cdiv(N, kBig);
  g.a_bytes = (uint32_t)(M * (FP4 ? K / 2 : K));
  g.w_bytes = (uint32_t)pg.codes;
  g.asc_bytes = FP4 ? (uint32_t)(M * (K / 32)) : 0u;
  g.wsc_bytes = FP4 ? (uint32_t)(pg.total - pg.scales) : 0u;
  const uint8_t* w_sc = FP4 ? static_cast<const uint8_t*>(wp) + pg.scales : nullptr;
  hipLaunchKernelGGL((tile256_kernel<FP4>), dim3((unsigned)(g.tiles_m * g.tiles_n)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(a),
                     static_cast<const uint8_t*>(a_sc), static_cast<const uint8_t*>(wp), w_sc,
                     sa, sb, static_cast<uint16_t*>(c), g);
  return hipGetLastError();
}

template <bool FP4, int FM, int FN>
hipError_t launch_tiles(const void* a, const void* a_sc, const void* wp, const float* sa,
                        const float* sb, void* c, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
  using C = TileCfg<FM, FN>;
  const PackGeom g = pack_geom(FP4 ? 3 : 4, K, N);
  const int64_t tiles_m = cdiv(M, C::BM);
  const int64_t tiles_n = cdiv(N, C::BN);
  const uint8_t* w_sc = FP4 ? static_cast<const uint8_t*>(wp) + g.scales : nullptr;
  hipLaunchKernelGGL((tile_gemm_kernel<FP4, FM, FN>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(a),
                     static_cast<const uint8_t*>(a_sc), static_cast<const uint8_t*>(wp), w_sc,
                     sa, sb, static_cast<uint16_t*>(c), (int)M, (int)N, (int)K, (int)g.kt,
                     (int)g.cg, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_tile_gemm(int fmt, const void* a, const void* a_e8m0, const void* w_packed,
                            const float* scale_a, const float* scale_b, void* c, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream) {
  // large tiles once both output dimensions fill them; the 128 x 128 kernel
  // covers the rest (and MXFP4 K that is not a multiple of 128)
  const bool big = M > 128 && N > 128;
  if (fmt == 3) {
    if (big && K % 128 == 0)
      return launch_big<true>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
    return launch_tiles<true, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  if (fmt == 4) {
    if (big) return launch_big<false>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
    return launch_tiles<false, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qgemm
