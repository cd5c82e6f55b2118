// LDS-tiled matrix-core GEMMs for MXFP4 x MXFP4 and FP8 e4m3fn: the 128 x 128
// kernel (any M; small or ragged shapes) and the dispatch between it and the
// 256 x 256 kernels of tile_mx256.hip.
//
// The MXFP4 page (section 2) tiles C into B_M x B_N blocks per workgroup and
// sums, per 32-element micro-block, S_A * S_W * dot(A, W) (eq. 1) with the
// scale product done as an exponent add (eq. 2).  On gfx950 that whole step is
// one instruction: v_mfma_scale_f32_16x16x128_f8f6f4 (here; the 256 x 256
// kernels use its 32 x 32 x 64 form) takes FP4
// (or FP8) codes and one E8M0 byte per lane, applies 2^(E_A-127) *
// 2^(E_W-127) to each 32-element block product in hardware and accumulates in
// fp32.  FP8 (FP8 page) uses the same instruction with e4m3 operands and unit
// scales; its per-tensor scales multiply the fp32 result once in the
// epilogue.
//
// 128 x 128 kernel, data flow per K step (128 bytes of K per row: 256 FP4 or
// 128 FP8 elements):
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
#include "tile_common.h"

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

bool pipe_fits(int fmt, int64_t M, int64_t N, int64_t K, int64_t group_k) {
  const int64_t lim = kOutOfRange;
  const int64_t a_row = fmt == 3 ? K / 2 : fmt == 4 ? K : 2 * K;
  if (M * a_row >= lim || (fmt == 3 && M * (K / 32) >= lim)) return false;
  const PackGeom g =
      fmt == 5 || fmt == 6 ? grouped_geom(fmt, K, N, group_k) : pack_geom(fmt, K, N);
  return g.total < lim;   // the code segment and any scale or metadata segment
}

// Large tiles once N exceeds 128, M exceeds 64 (the dispatch sends M <= 128
// here only for wide N, where one row of 256 x 256 tiles beats both the
// small-M kernel and 128 x 128 tiles) and K spans at least two 128-element
// tiles; the 128 x 128 kernel covers the rest (and MXFP4 K that is not a
// multiple of 128, whose scale rows the 4-byte copies of the large kernel
// cannot split, or that spans a single 256-element step).
bool tile_is_big(int fmt, int64_t M, int64_t N, int64_t K) {
  const bool big = M > 64 && N > 128 && cdiv(K, kTileK8) >= 2 && pipe_fits(fmt, M, N, K, 0);
  return fmt == 3 ? big && K % 128 == 0 && cdiv(K, kTileK4) >= 2 : big;
}

hipError_t launch_tile_gemm(int fmt, const void* a, const void* a_e8m0, const void* w_packed,
                            const float* scale_a, const float* scale_b, void* c, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream) {
  const bool big = tile_is_big(fmt, M, N, K);
  if (fmt == 3) {
    if (big) return launch_mxfp4_256(a, a_e8m0, w_packed, c, M, N, K, stream);
    return launch_tiles<true, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  if (fmt == 4) {
    if (big) return launch_fp8_256(a, w_packed, scale_a, scale_b, c, M, N, K, stream);
    return launch_tiles<false, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qgemm
