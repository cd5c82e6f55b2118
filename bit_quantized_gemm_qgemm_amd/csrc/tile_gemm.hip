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
      // the 128 columns form one scale group; its two 512 B steps of this kt
      r.sb = *reinterpret_cast<const uintx4*>(
          w_sc + ((int64_t)(cg0 / 8) * (2 * KT) + 2 * kt) * 512 + 16 * t);
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
        const int sb = lds_sb[512 * h + 8 * lane + tile];
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
  static_assert(!FP4 || C::BN == 128, "an MXFP4 tile spans exactly one 128-column scale group");
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
// Large tiles: 256 x 256 per workgroup, 128 x 128 per wave (256 fp32
// accumulators per lane, all in AGPRs).  K advances in steps of 64 bytes per
// row (128 FP4 or 64 FP8 elements) through a 4-deep ring of LDS stages that
// the buffer unit fills directly from global memory (no VGPR staging).
// Buffer resources bound every operand, so rows past M, column tiles past N
// and K chunks past K read as zero without predication.
//
// Schedule per step ks (one barrier per step):
//   - issue the global->LDS copies of step ks+3;
//   - run the step's matrix instructions from registers, and in between read
//     the fragments of step ks+1 from LDS into a second register set, so the
//     LDS latency hides behind matrix work;
//   - wait until this wave's copies of step ks+2 have landed (those of ks+3
//     stay in flight) and meet at the barrier.
// The barrier is issued without the full memory drain that __syncthreads()
// implies, which would also wait for the copies still in flight.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBig = 256;
constexpr int kStepBytes = 64;      // bytes of K per row per step
constexpr int kStages = 4;
constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset past every buffer

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

struct PipeArgs {
  int M, N, K, KT, KS, CG, tiles_m, tiles_n;
  uint32_t a_bytes, w_bytes, asc_bytes, wsc_bytes;
};

// Stage layout (both formats):
//   A   [256 rows][64 B]; 16-byte chunk c of row r sits in slot c ^ swizzle(r),
//       with swizzle(r) = (r >> 1) & 3 for MXFP4 and (r >> 2) & 3 for FP8: the
//       row bits that keep each format's fragment reads free of bank
//       conflicts (16 rows x 4 lane groups for MXFP4, 32 rows x 2 for FP8)
//   W   16 column tiles x 1 KB
//   MXFP4 only: A scales [256 rows][4 blocks]; W scales [wn 2][lane 64][tile 8]
template <bool FP4>
struct PipeCfg {
  static constexpr int A = kBig * kStepBytes;
  static constexpr int B = kBig * kStepBytes;
  static constexpr int SA = FP4 ? kBig * 4 : 0;
  static constexpr int SB = FP4 ? 2 * 512 : 0;
  static constexpr int STAGE = A + B + SA + SB;
  static constexpr int DMA = FP4 ? 10 : 8;        // copies per wave per stage
};

template <bool FP4>
__device__ __forceinline__ int pipe_swizzle(int r) {
  return FP4 ? (r >> 1) & 3 : (r >> 2) & 3;
}

template <bool FP4>
__device__ __forceinline__ void pipe_issue(uint8_t* st, int ks, int wave, int lane, int m0,
                                           int cg0, const PipeArgs& g,
                                           __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rw,
                                           __amdgpu_buffer_rsrc_t rsa,
                                           __amdgpu_buffer_rsrc_t rsw) {
  using C = PipeCfg<FP4>;
  const int row_bytes = FP4 ? g.K / 2 : g.K;
  const int kt = ks >> 1, h = ks & 1;
  // A: 16 slices of 16 rows x 64 B; wave w copies slices 4w .. 4w+3
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 4 * wave + j;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ pipe_swizzle<FP4>(r);
    const int kb = ks * kStepBytes + 16 * c;
    const uint32_t off = kb < row_bytes ? (uint32_t)(m0 + r) * (uint32_t)row_bytes + kb
                                        : kOutOfRange;
    dma16(ra, st + q * 1024, off);
  }
  // W: the 1 KB of column tile t = 4w + j that belongs to this step
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * wave + j;
    const uint32_t base = ((uint32_t)(cg0 + t) * g.KT + kt) * kTileBytes;
    // FP4: half h of the tile as is.  FP8: bytes [16h, 16h + 16) of each
    // lane group pair 2h, 2h + 1, from both 1 KB halves of the tile.
    const uint32_t off = FP4 ? base + 1024u * h + 16u * lane
                             : base + 1024u * (lane >> 5) + 512u * h + 16u * (lane & 31);
    dma16(rw, st + C::A + t * 1024, off);
  }
  if constexpr (FP4) {
    const int sc_cols = g.K / 32;   // K % 128 == 0: four blocks per row are one dword
    const int r = 64 * wave + lane;
    const int blk = 4 * ks;
    const uint32_t off = blk < sc_cols ? (uint32_t)(m0 + r) * (uint32_t)sc_cols + blk
                                       : kOutOfRange;
    dma4(rsa, st + C::A + C::B + 256 * wave, off);
    const uint32_t soff = ((uint32_t)(cg0 / 8 + (wave >> 1)) * g.KS + ks) * 512u +
                          256u * (wave & 1) + 4u * lane;
    dma4(rsw, st + C::A + C::B + C::SA + 256 * wave, soff);
  }
}

// MXFP4: 8 x 8 fragments of 16 x 16 per wave; one step = 128 K elements =
// one v_mfma_scale_f32_16x16x128_f8f6f4 per fragment pair.
struct Fp4Pipe {
  static constexpr bool FP4 = true;
  static constexpr int PARTS = 8;
  typedef floatx4 Acc[8][8];
  struct Frags {
    uintx4 a[8];
    uintx4 b[8];
    uint32_t sa[8];
    uintx2 sb;
  };
  struct Lane {
    int a, sa, b, sb;
  };
  __device__ __forceinline__ static Lane lane_offsets(int wm, int wn, int lane) {
    using C = PipeCfg<true>;
    const int r = wm * 128 + (lane & 15), grp = lane >> 4;
    Lane L;
    L.a = r * kStepBytes + 16 * (grp ^ pipe_swizzle<true>(r));
    L.sa = C::A + C::B + r * 4 + grp;
    L.b = C::A + wn * 8 * 1024 + 16 * lane;
    L.sb = C::A + C::B + C::SA + wn * 512 + 8 * lane;
    return L;
  }
  template <int P>
  __device__ __forceinline__ static void read(Frags& F, const uint8_t* st, const Lane& L) {
    F.a[P] = *reinterpret_cast<const uintx4*>(st + L.a + P * 1024);
    F.sa[P] = st[L.sa + P * 64];
    F.b[P] = *reinterpret_cast<const uintx4*>(st + L.b + P * 1024);
    if (P == 0) F.sb = *reinterpret_cast<const uintx2*>(st + L.sb);
  }
  // column fragment P against all 8 row fragments
  template <int P>
  __device__ __forceinline__ static void mma(const Frags& F, Acc& acc) {
    const intx8 bf = {(int)F.b[P][0], (int)F.b[P][1], (int)F.b[P][2], (int)F.b[P][3], 0, 0, 0, 0};
    const int sb = (int)F.sb[P >> 2];
#pragma unroll
    for (int fm = 0; fm < 8; ++fm) {
      const intx8 af = {(int)F.a[fm][0], (int)F.a[fm][1], (int)F.a[fm][2], (int)F.a[fm][3],
                        0, 0, 0, 0};
      // byte P & 3 of sb is the scale of column tile P
      acc[fm][P] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          af, bf, acc[fm][P], kFmtFP4, kFmtFP4, 0, (int)F.sa[fm], P & 3, sb);
    }
  }
  __device__ __forceinline__ static void zero(Acc& acc) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  // lane holds rows 4 (lane >> 4) + i, column lane & 15 of each fragment
  __device__ __forceinline__ static void store(const Acc& acc, uint16_t* __restrict__ c, int m0, int n0, int wm,
                               int wn, int lane, int M, int N, float s) {
#pragma unroll
    for (int fm = 0; fm < 8; ++fm)
#pragma unroll
      for (int fn = 0; fn < 8; ++fn) {
        const int gn = n0 + wn * 128 + fn * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int gm = m0 + wm * 128 + fm * 16 + 4 * (lane >> 4) + i;
          if (gm < M && gn < N) c[(int64_t)gm * N + gn] = f32_to_bf16_rne(acc[fm][fn][i] * s);
        }
      }
  }
};

// FP8: 4 x 4 fragments of 32 x 32 per wave; one step = 64 K elements = one
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) per fragment pair.
// Lane l feeds row (or column) l & 31 with K elements 32 (l >> 5) + [0, 32)
// of the step, the same K order on both sides.
struct Fp8Pipe {
  static constexpr bool FP4 = false;
  static constexpr int PARTS = 4;
  typedef floatx16 Acc[4][4];
  struct Frags {
    uintx4 alo[4], ahi[4];
    uintx4 blo[4], bhi[4];
  };
  struct Lane {
    int alo, ahi, b;
  };
  __device__ __forceinline__ static Lane lane_offsets(int wm, int wn, int lane) {
    using C = PipeCfg<false>;
    const int r = wm * 128 + (lane & 31), hh = lane >> 5, swz = pipe_swizzle<false>(r);
    Lane L;
    L.alo = r * kStepBytes + 16 * ((2 * hh) ^ swz);
    L.ahi = r * kStepBytes + 16 * ((2 * hh + 1) ^ swz);
    // column tile wn*8 + 2P + ((lane >> 4) & 1); lane group pair half hh
    L.b = C::A + (wn * 8 + ((lane >> 4) & 1)) * 1024 + 256 * hh + 16 * (lane & 15);
    return L;
  }
  template <int P>
  __device__ __forceinline__ static void read(Frags& F, const uint8_t* st, const Lane& L) {
    F.alo[P] = *reinterpret_cast<const uintx4*>(st + L.alo + P * 2048);
    F.ahi[P] = *reinterpret_cast<const uintx4*>(st + L.ahi + P * 2048);
    F.blo[P] = *reinterpret_cast<const uintx4*>(st + L.b + P * 2048);
    F.bhi[P] = *reinterpret_cast<const uintx4*>(st + L.b + P * 2048 + 512);
  }
  template <int P>
  __device__ __forceinline__ static void mma(const Frags& F, Acc& acc) {
    const intx8 bf = {(int)F.blo[P][0], (int)F.blo[P][1], (int)F.blo[P][2], (int)F.blo[P][3],
                      (int)F.bhi[P][0], (int)F.bhi[P][1], (int)F.bhi[P][2], (int)F.bhi[P][3]};
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const intx8 af = {(int)F.alo[fm][0], (int)F.alo[fm][1], (int)F.alo[fm][2],
                        (int)F.alo[fm][3], (int)F.ahi[fm][0], (int)F.ahi[fm][1],
                        (int)F.ahi[fm][2], (int)F.ahi[fm][3]};
      acc[fm][P] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          af, bf, acc[fm][P], kFmtFP8, kFmtFP8, 0, kE8M0One, 0, kE8M0One);
    }
  }
  __device__ __forceinline__ static void zero(Acc& acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  }
  // lane holds rows 8 (e >> 2) + 4 (lane >> 5) + (e & 3), column lane & 31
  __device__ __forceinline__ static void store(const Acc& acc, uint16_t* __restrict__ c, int m0, int n0, int wm,
                               int wn, int lane, int M, int N, float s) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
#pragma unroll
      for (int fn = 0; fn < 4; ++fn) {
        const int gn = n0 + wn * 128 + fn * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int gm = m0 + wm * 128 + fm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (gm < M && gn < N) c[(int64_t)gm * N + gn] = f32_to_bf16_rne(acc[fm][fn][e] * s);
        }
      }
  }
};

// One part: read fragment P of the next step (RD), then the matrix work of
// fragment P of the current step; the scheduler keeps the two together.
template <class Ops, int P, bool RD>
__device__ __forceinline__ void pipe_part(typename Ops::Frags& cur, typename Ops::Frags& nxt,
                                          const uint8_t* nx, const typename Ops::Lane& L,
                                          typename Ops::Acc& acc) {
  if (RD) Ops::template read<P>(nxt, nx, L);
  Ops::template mma<P>(cur, acc);
  __builtin_amdgcn_sched_barrier(0);
}

template <class Ops, bool RD>
__device__ __forceinline__ void pipe_step(typename Ops::Frags& cur, typename Ops::Frags& nxt,
                                          const uint8_t* nx, const typename Ops::Lane& L,
                                          typename Ops::Acc& acc) {
  pipe_part<Ops, 0, RD>(cur, nxt, nx, L, acc);
  pipe_part<Ops, 1, RD>(cur, nxt, nx, L, acc);
  pipe_part<Ops, 2, RD>(cur, nxt, nx, L, acc);
  pipe_part<Ops, 3, RD>(cur, nxt, nx, L, acc);
  if constexpr (Ops::PARTS == 8) {
    pipe_part<Ops, 4, RD>(cur, nxt, nx, L, acc);
    pipe_part<Ops, 5, RD>(cur, nxt, nx, L, acc);
    pipe_part<Ops, 6, RD>(cur, nxt, nx, L, acc);
    pipe_part<Ops, 7, RD>(cur, nxt, nx, L, acc);
  }
}

template <class Ops>
__device__ __forceinline__ void pipe_read_all(typename Ops::Frags& F, const uint8_t* st,
                                              const typename Ops::Lane& L) {
  Ops::template read<0>(F, st, L);
  Ops::template read<1>(F, st, L);
  Ops::template read<2>(F, st, L);
  Ops::template read<3>(F, st, L);
  if constexpr (Ops::PARTS == 8) {
    Ops::template read<4>(F, st, L);
    Ops::template read<5>(F, st, L);
    Ops::template read<6>(F, st, L);
    Ops::template read<7>(F, st, L);
  }
}

// Requires KS even and >= 4 (checked on the host).
template <class Ops>
__global__ __launch_bounds__(kThreads) void pipe256_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ w_sc,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b,
    uint16_t* __restrict__ c, PipeArgs g) {
  constexpr bool FP4 = Ops::FP4;
  using C = PipeCfg<FP4>;
  constexpr int PER = C::DMA;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * C::STAGE];
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
  const typename Ops::Lane L = Ops::lane_offsets(wm, wn, lane);

  typename Ops::Acc acc;
  Ops::zero(acc);
  const int KS = g.KS;
  auto stage = [&](int s) { return smem + (s & (kStages - 1)) * C::STAGE; };
  auto issue = [&](int s) { pipe_issue<FP4>(stage(s), s, wave, lane, m0, cg0, g, ra, rw, rsa, rsw); };

  issue(0);
  issue(1);
  issue(2);
  QG_WAIT_VM_BARRIER(PER);   // steps 0 and 1 landed; 2 may be in flight
  typename Ops::Frags F0, F1;
  pipe_read_all<Ops>(F0, stage(0), L);

  // Two steps per iteration, F0 and F1 trading roles.  Every copy issued in
  // here is in range (ks + 4 < KS).
  int ks = 0;
  for (; ks + 4 < KS; ks += 2) {
    issue(ks + 3);
    pipe_step<Ops, true>(F0, F1, stage(ks + 1), L, acc);
    QG_WAIT_VM_BARRIER(PER);   // step ks+2 landed
    issue(ks + 4);
    pipe_step<Ops, true>(F1, F0, stage(ks + 2), L, acc);
    QG_WAIT_VM_BARRIER(PER);   // step ks+3 landed
  }
  // last four steps: ks == KS - 4, copies issued up to step KS - 2
  issue(ks + 3);
  pipe_step<Ops, true>(F0, F1, stage(ks + 1), L, acc);
  QG_WAIT_VM_BARRIER(PER);
  pipe_step<Ops, true>(F1, F0, stage(ks + 2), L, acc);
  QG_WAIT_VM_BARRIER(0);
  pipe_step<Ops, true>(F0, F1, stage(ks + 3), L, acc);
  pipe_step<Ops, false>(F1, F0, stage(ks + 3), L, acc);

  const float s = FP4 ? 1.0f : (*scale_a) * (*scale_b);
  Ops::store(acc, c, m0, cg0 * 16, wm, wn, lane, g.M, g.N, s);
}

template <class Ops>
hipError_t launch_pipe(const void* a, const void* a_sc, const void* wp, const float* sa,
                       const float* sb, void* c, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream) {
  constexpr bool FP4 = Ops::FP4;
  const PackGeom pg = pack_geom(FP4 ? 3 : 4, K, N);
  PipeArgs g;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.KT = (int)pg.kt;
  g.KS = 2 * (int)pg.kt;
  g.CG = (int)pg.cg;
  g.tiles_m = (int)cdiv(M, kBig);
  g.tiles_n = (int)cdiv(N, kBig);
  g.a_bytes = (uint32_t)(M * (FP4 ? K / 2 : K));
  g.w_bytes = (uint32_t)pg.codes;
  g.asc_bytes = FP4 ? (uint32_t)(M * (K / 32)) : 0u;
  g.wsc_bytes = FP4 ? (uint32_t)(pg.total - pg.scales) : 0u;
  const uint8_t* w_sc = FP4 ? static_cast<const uint8_t*>(wp) + pg.scales : nullptr;
  hipLaunchKernelGGL((pipe256_kernel<Ops>), dim3((unsigned)(g.tiles_m * g.tiles_n)),
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
  // large tiles once both output dimensions fill them and K spans at least
  // two 256-element tiles; the 128 x 128 kernel covers the rest (and MXFP4 K
  // that is not a multiple of 128, whose scale rows the 4-byte copies of the
  // large kernel cannot split)
  const bool big = M > 128 && N > 128 && cdiv(K, kTileK8) >= 2;
  if (fmt == 3) {
    if (big && K % 128 == 0 && cdiv(K, kTileK4) >= 2)
      return launch_pipe<Fp4Pipe>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
    return launch_tiles<true, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  if (fmt == 4) {
    if (big) return launch_pipe<Fp8Pipe>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
    return launch_tiles<false, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qgemm
