// LDS-tiled matrix-core GEMMs: MXFP4 x MXFP4 and FP8 e4m3fn at any M, and the
// weight-only formats (INT4 / INT8 per column or grouped, NVFP4 weights; fp16
// X) at large M.
//
// The MXFP4 page (section 2) tiles C into B_M x B_N blocks per workgroup and
// sums, per 32-element micro-block, S_A * S_W * dot(A, W) (eq. 1) with the
// scale product done as an exponent add (eq. 2).  On gfx950 that whole step is
// one instruction: v_mfma_scale_f32_16x16x128_f8f6f4 (here in the 128 x 128
// kernel; the 256 x 256 kernels below use its 32 x 32 x 64 form) takes FP4
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
#include "qgemm_dequant.h"

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
//   - run the step's matrix instructions from registers, and in between read
//     the fragments of step ks+1 from LDS into a second register set, so the
//     LDS latency hides behind matrix work;
//   - in the step's first two parts, issue the global->LDS copies of step
//     ks+3 (into the stage whose fragments were read one step earlier);
//   - wait until this wave's copies of step ks+2 have landed (those of ks+3
//     stay in flight) and meet at the barrier.
// The barrier is issued without the full memory drain that __syncthreads()
// implies, which would also wait for the copies still in flight.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBig = 256;
constexpr int kStepBytes = 64;      // bytes of K per row per step
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

// Stage layout, common part: A [256 rows][64 B] at offset 0; the 16-byte
// chunk c of row r sits in slot c ^ Ops::swizzle(r), the row bits that keep
// that format's fragment reads free of LDS bank conflicts (checked with the
// bank-conflict counter: rows 1-2 for 16-row x 4-group reads, rows 2-3 for
// 32-row x 2-group reads).  The weight part (and the MXFP4 scales) follow.
constexpr int kStageA = kBig * kStepBytes;

// A copies of step ks: 16 slices of 16 rows x 64 B; wave w takes 4w .. 4w+3.
template <class Ops>
__device__ __forceinline__ void pipe_issue_a(uint8_t* st, int ks, int wave, int lane, int m0,
                                             int row_bytes, __amdgpu_buffer_rsrc_t ra) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = 4 * wave + j;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ Ops::swizzle(r);
    const int kb = ks * kStepBytes + 16 * c;
    const uint32_t off = kb < row_bytes ? (uint32_t)(m0 + r) * (uint32_t)row_bytes + kb
                                        : kOutOfRange;
    dma16(ra, st + q * 1024, off);
  }
}

// Operand rsrcs of one workgroup.
struct PipeRsrc {
  __amdgpu_buffer_rsrc_t a, w, sa, sw;
};

// Everything an epilogue may need besides the accumulators.
struct PipeOut {
  uint16_t* c;
  const uint16_t* col_scale;   // W4A16 / W8A16: fp16 scale per output column
  float s;                     // FP8: scale_a * scale_b
  int M, N;
};

// A fragment of a 16 x 16 x K matrix step: lane l reads row l & 15, 16-byte
// chunk l >> 4 of the step's 64 bytes.
__device__ __forceinline__ int a16_lane_offset(int wm, int lane, int swz) {
  const int r = wm * 128 + (lane & 15);
  return r * kStepBytes + 16 * ((lane >> 4) ^ swz);
}

// ---- epilogue: the 256 x 256 output tile goes through LDS -----------------
// Each lane rounds its scaled accumulators (hardware RNE conversion) into a
// row-major [256][512 B] tile in LDS; then the workgroup copies it out with
// 16-byte row-contiguous stores.  16-byte chunk k of row r sits in slot
// k ^ (((r >> 2) & 3) << 2): the rows that one 2-byte write instruction
// touches (4 apart for 16 x 16 fragments, 4 apart for 32 x 32) land in
// different banks.
constexpr int kCTileBytes = kBig * kBig * 2;

__device__ __forceinline__ int c_tile_offset(int row, int col) {
  return row * (kBig * 2) + 16 * ((col >> 3) ^ (((row >> 2) & 3) << 2)) + 2 * (col & 7);
}

template <bool F16_OUT>
__device__ __forceinline__ uint16_t round_out(float v) {
  if constexpr (F16_OUT) return f32_to_f16_bits(v);
  else return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// 16 x 16 accumulators: lane holds rows 4 (lane >> 4) + i, column lane & 15.
template <bool F16_OUT, bool COL_SCALE = F16_OUT>
__device__ __forceinline__ void stage16(const floatx4 (&acc)[8][8], uint8_t* ct, const PipeOut& o,
                                        int n0, int wm, int wn, int lane) {
#pragma unroll
  for (int fn = 0; fn < 8; ++fn) {
    const int col = wn * 128 + fn * 16 + (lane & 15);
    float s = o.s;
    if constexpr (COL_SCALE) {
      const int gn = n0 + col;
      s = (float)__builtin_bit_cast(_Float16, o.col_scale[gn < o.N ? gn : o.N - 1]);
    }
#pragma unroll
    for (int fm = 0; fm < 8; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + fm * 16 + 4 * (lane >> 4) + i;
        *reinterpret_cast<uint16_t*>(ct + c_tile_offset(row, col)) =
            round_out<F16_OUT>(acc[fm][fn][i] * s);
      }
  }
}

// Copy the staged tile to C (rows past M and columns past N are dropped).
template <int NT = kThreads>
__device__ __forceinline__ void pipe_copy_out(const uint8_t* ct, const PipeOut& o, int m0,
                                              int n0) {
  const bool vec = (o.N & 7) == 0;
#pragma unroll 4
  for (int j = 0; j < kCTileBytes / 16 / NT; ++j) {
    const int q = (int)threadIdx.x + NT * j;
    const int row = q >> 5, ch = q & 31;
    const int gm = m0 + row, gn = n0 + 8 * ch;
    if (gm >= o.M || gn >= o.N) continue;
    const uintx4 v =
        *reinterpret_cast<const uintx4*>(ct + row * (kBig * 2) + 16 * (ch ^ (((row >> 2) & 3) << 2)));
    uint16_t* dst = o.c + (int64_t)gm * o.N + gn;
    if (vec) {
      *reinterpret_cast<uintx4*>(dst) = v;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (gn + t < o.N) dst[t] = (uint16_t)(v[t >> 1] >> (16 * (t & 1)));
    }
  }
}

// 32 x 32 accumulator layout of v_mfma_*_32x32x*: lane holds rows
// 8 (e >> 2) + 4 (lane >> 5) + (e & 3) of its fragment, column lane & 31.
__device__ __forceinline__ void stage32(const floatx16 (&acc)[4][4], uint8_t* ct,
                                        const PipeOut& o, int wm, int wn, int lane) {
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < 4; ++fn) {
      const int col = wn * 128 + fn * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * 128 + fm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        *reinterpret_cast<uint16_t*>(ct + c_tile_offset(row, col)) =
            round_out<false>(acc[fm][fn][e] * o.s);
      }
    }
}

// FP8: 4 x 4 fragments of 32 x 32 per wave; one step = 64 K elements = one
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) per fragment pair.
// Lane l feeds row (or column) l & 31 with K elements 32 (l >> 5) + [0, 32)
// of the step, the same K order on both sides.
// Stage: A | W 16 tiles x 1 KB: bytes [16h, 16h + 16) of the lane group pair
// 2s, 2s + 1 (s = step within the tile) from both 1 KB halves h.
struct Fp8Pipe {
  static constexpr int FMT = 4;
  template <class F>
  __device__ __forceinline__ static void init(F&, F&) {}
  static constexpr int GROUP_WORDS = 0;
  static constexpr int PARTS = 4;
  static constexpr int STEPS_PER_TILE = 2;
  static constexpr int B = 16 * 1024;
  static constexpr int STAGE = kStageA + B;
  static constexpr int DMA = 8;
  static constexpr int NST = 4;                  // 4 x 32 KB
  static constexpr bool CP_INTERLEAVE = true;
  static constexpr int CP_PIN_PAIRS = 4;         // copies of parts 0 / 1: 4 / 4
  typedef floatx16 Acc[4][4];
  struct Frags {
    uintx4 alo[4], ahi[4];
    uintx4 blo[4], bhi[4];
  };
  struct Lane {
    int alo, ahi, b;
  };
  __device__ __forceinline__ static int swizzle(int r) { return (r >> 2) & 3; }
  __device__ __forceinline__ static int row_bytes(int K) { return K; }
  __device__ __forceinline__ static void issue_rest(uint8_t* st, int ks, int wave, int lane,
                                                    int, int cg0, const PipeArgs& g,
                                                    const PipeRsrc& rs) {
    const int kt = ks >> 1, h = ks & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * wave + j;
      const uint32_t off = ((uint32_t)(cg0 + t) * g.KT + kt) * kTileBytes +
                           1024u * (lane >> 5) + 512u * h + 16u * (lane & 31);
      dma16(rs.w, st + kStageA + t * 1024, off);
    }
  }
  __device__ __forceinline__ static Lane lane_offsets(int wm, int wn, int lane) {
    const int r = wm * 128 + (lane & 31), hh = lane >> 5, swz = swizzle(r);
    Lane L;
    L.alo = r * kStepBytes + 16 * ((2 * hh) ^ swz);
    L.ahi = r * kStepBytes + 16 * ((2 * hh + 1) ^ swz);
    // column tile wn*8 + 2P + ((lane >> 4) & 1); lane group pair half hh
    L.b = kStageA + (wn * 8 + ((lane >> 4) & 1)) * 1024 + 256 * hh + 16 * (lane & 15);
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
  __device__ __forceinline__ static void mma(const Frags& F, const Lane&, Acc& acc) {
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
  __device__ __forceinline__ static void stage(const Acc& acc, uint8_t* ct, const PipeOut& o,
                                               int, int wm, int wn, int lane) {
    stage32(acc, ct, o, wm, wn, lane);
  }
};

// W4A16 / W8A16 with fp16 X: 8 x 8 fragments of 16 x 16 per wave; one step =
// 32 K elements = one v_mfma_f32_16x16x32_f16 per fragment pair.  The step's
// weight bytes of a lane (the word of matrix step s = ks % 4 of its packed
// 128-wide tile: 4 bytes for W4, 8 for W8) are gathered into LDS with 4-byte
// copies, read back as one or two words and dequantized in registers right
// before the matrix instructions that use them (W4A16 page section 2, W8A16
// page Steps 1-2: the dequantized weight never leaves the registers).  The
// per-column scale multiplies the fp32 sum in the epilogue.
// Grouped formats (NGT > 0 metadata words per column and 128-wide tile, the
// layout of the grouped prepack): each step also gathers the lane's word
// {fp16 1024 + z (1152 + z for INT8), fp16 s} of its column and the step's K
// group, and the dequant forms fp16((w - z) * s) with one rounding, as the
// small-M kernel does; the epilogue then rounds the fp32 sum alone.
// NVFP4 weights (WFMT 7: E2M1 codes in the INT4 tile geometry, natural
// nibble order): each step also gathers the dword of the lane's column that
// holds its 16-element block's e4m3 scale for all four steps of the tile
// (byte s for step s; the register set counts its steps to pick the byte);
// each weight is formed exactly in fp16 (E2M1 value times e4m3 scale) and
// the per-tensor scale multiplies the fp32 sum in the epilogue.
// Stage: A (fp16 X) | W: [tile 16][part WV][lane 64][4 B] | metadata (grouped
// or NVFP4): [tile 16][lane 64][4 B].
template <int WFMT, int NGT = 0>
struct F16Pipe {
  static constexpr int FMT = WFMT;
  static constexpr int GROUP_WORDS = NGT;
  static constexpr bool META = NGT > 0 || WFMT == 7;
  static constexpr int WV = WFMT == 2 ? 2 : 1;        // weight words per lane per step
  static constexpr int PARTS = 8;
  static constexpr int STEPS_PER_TILE = 4;
  static constexpr int B = 16 * WV * 256;
  static constexpr int MB = META ? 16 * 256 : 0;
  static constexpr int STAGE = kStageA + B + MB;
  static constexpr int DMA = 4 + 4 * WV + (META ? 4 : 0);
  // 8 x 20 KB or 6 x 24 KB; with metadata: 6 x 24 KB or 4 x 28 KB
  static constexpr int NST = META ? (WV == 1 ? 6 : 4) : (WV == 1 ? 8 : 6);
  // copies issued inside parts 0 and 1 but not pinned between the matrix
  // instructions (pinning made the register allocator spill); 2-5% faster
  // than issuing them ahead of the step
  static constexpr bool CP_INTERLEAVE = true;
  static constexpr int CP_PIN_PAIRS = 0;
  typedef floatx4 Acc[8][8];
  struct Frags {
    uintx4 a[8];
    half8_t b[8];   // dequantized right after the LDS read
    int step;       // NVFP4: the step these registers are read for next
  };
  struct Lane {
    int a, b, m;
  };
  // the two register sets take the even and the odd steps
  __device__ __forceinline__ static void init(Frags& F0, Frags& F1) {
    F0.step = 0;
    F1.step = 1;
  }
  __device__ __forceinline__ static int swizzle(int r) { return (r >> 1) & 3; }
  __device__ __forceinline__ static int row_bytes(int K) { return 2 * K; }
  __device__ __forceinline__ static void issue_rest(uint8_t* st, int ks, int wave, int lane,
                                                    int, int cg0, const PipeArgs& g,
                                                    const PipeRsrc& rs) {
    const int kt = ks >> 2, s = ks & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * wave + j;
#pragma unroll
      for (int p = 0; p < WV; ++p) {
        // W4: word s of the lane's 16 bytes.  W8: bytes 8 (s & 1) + 4p of
        // the lane's 16 bytes in half s >> 1.
        const uint32_t off = WV == 1
            ? ((uint32_t)(cg0 + t) * g.KT + kt) * kTileBytesW4 + 16u * lane + 4u * s
            : ((uint32_t)(cg0 + t) * g.KT + kt) * kTileBytes + 1024u * (s >> 1) + 16u * lane +
                  8u * (s & 1) + 4u * p;
        dma4(rs.w, st + kStageA + (t * WV + p) * 256, off);
      }
    }
    if constexpr (WFMT == 7) {
      // the scale dword of the lane's column (lane & 15) and 16-element
      // block pair (lane >> 5): bytes c*8 + 4(g >> 1) + s of the tile
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t = 4 * wave + jj;
        const uint32_t off = ((uint32_t)(cg0 + t) * g.KT + kt) * (uint32_t)kScaleTileBytes +
                             8u * (uint32_t)(lane & 15) + 4u * (uint32_t)(lane >> 5);
        dma4(rs.sw, st + kStageA + B + t * 256, off);
      }
    }
    if constexpr (NGT > 0) {
      // the word of the lane's column (lane & 15) for the step's K group
      const int j = (s * NGT) >> 2;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int t = 4 * wave + jj;
        const uint32_t off =
            ((((uint32_t)(cg0 + t) * g.KT + kt) * 16u + (uint32_t)(lane & 15)) * NGT + j) * 4u;
        dma4(rs.sw, st + kStageA + B + t * 256, off);
      }
    }
  }
  __device__ __forceinline__ static Lane lane_offsets(int wm, int wn, int lane) {
    const int r = wm * 128 + (lane & 15);
    Lane L;
    L.a = a16_lane_offset(wm, lane, swizzle(r));
    L.b = kStageA + wn * 8 * WV * 256 + 4 * lane;
    L.m = kStageA + B + wn * 8 * 256 + 4 * lane;
    return L;
  }
  template <int P>
  __device__ __forceinline__ static void read(Frags& F, const uint8_t* st, const Lane& L) {
    F.a[P] = *reinterpret_cast<const uintx4*>(st + L.a + P * 1024);
    const uint32_t w0 = *reinterpret_cast<const uint32_t*>(st + L.b + P * WV * 256);
    if constexpr (WFMT == 7) {
      const uint32_t e = *reinterpret_cast<const uint32_t*>(st + L.m + P * 256);
      F.b[P] = dequant_nvfp4(w0, e >> (8 * (F.step & 3)));
      if constexpr (P == PARTS - 1) F.step += 2;
    } else if constexpr (NGT > 0) {
      const uint32_t e = *reinterpret_cast<const uint32_t*>(st + L.m + P * 256);
      if constexpr (WFMT == 1) {
        F.b[P] = dequant_w4_group(w0, e);
      } else {
        const uint32_t w1 = *reinterpret_cast<const uint32_t*>(st + L.b + (P * WV + 1) * 256);
        F.b[P] = dequant_w8_group(w0, w1, e);
      }
    } else if constexpr (WFMT == 1) {
      F.b[P] = dequant_w4_shift(w0);
    } else {
      const uint32_t w1 = *reinterpret_cast<const uint32_t*>(st + L.b + (P * WV + 1) * 256);
      F.b[P] = dequant_w8(w0, w1);
    }
  }
  template <int P>
  __device__ __forceinline__ static void mma(const Frags& F, const Lane&, Acc& acc) {
#pragma unroll
    for (int fm = 0; fm < 8; ++fm)
      acc[fm][P] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, F.a[fm]),
                                                          F.b[P], acc[fm][P], 0, 0, 0);
  }
  __device__ __forceinline__ static void zero(Acc& acc) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ static void stage(const Acc& acc, uint8_t* ct, const PipeOut& o,
                                               int n0, int wm, int wn, int lane) {
    stage16<true, NGT == 0 && WFMT != 7>(acc, ct, o, n0, wm, wn, lane);
  }
};

// No copies in this step (the last steps, or copies issued before it).
struct NoCopies {
  __device__ __forceinline__ void operator()(int) const {}
};

// One part: read fragment P of the next step (RD), then the matrix work of
// fragment P of the current step; the scheduler keeps the two together.
// With CP, parts 0 and 1 also issue the copies of a later step (cp(0): the A
// slices, cp(1): the rest), after the part's matrix instructions in program
// order and, where the policy asks (CP_PIN_PAIRS), pinned to alternate with
// them: issuing them all ahead of the step kept the matrix pipe idle after
// every barrier.
template <class Ops, int P, bool RD, bool CP, class Copies>
__device__ __forceinline__ void pipe_part(typename Ops::Frags& cur, typename Ops::Frags& nxt,
                                          const uint8_t* nx, const typename Ops::Lane& L,
                                          typename Ops::Acc& acc, const Copies& cp) {
  if (RD) Ops::template read<P>(nxt, nx, L);
  Ops::template mma<P>(cur, L, acc);
  if constexpr (CP && P <= 1) {
    cp(P);
#pragma unroll
    for (int i = 0; i < Ops::CP_PIN_PAIRS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one vector memory read
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

template <class Ops, bool RD, bool CP = false, class Copies = NoCopies>
__device__ __forceinline__ void pipe_step(typename Ops::Frags& cur, typename Ops::Frags& nxt,
                                          const uint8_t* nx, const typename Ops::Lane& L,
                                          typename Ops::Acc& acc, const Copies& cp = Copies{}) {
  pipe_part<Ops, 0, RD, CP>(cur, nxt, nx, L, acc, cp);
  pipe_part<Ops, 1, RD, CP>(cur, nxt, nx, L, acc, cp);
  pipe_part<Ops, 2, RD, CP>(cur, nxt, nx, L, acc, cp);
  pipe_part<Ops, 3, RD, CP>(cur, nxt, nx, L, acc, cp);
  if constexpr (Ops::PARTS == 8) {
    pipe_part<Ops, 4, RD, CP>(cur, nxt, nx, L, acc, cp);
    pipe_part<Ops, 5, RD, CP>(cur, nxt, nx, L, acc, cp);
    pipe_part<Ops, 6, RD, CP>(cur, nxt, nx, L, acc, cp);
    pipe_part<Ops, 7, RD, CP>(cur, nxt, nx, L, acc, cp);
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

// Last steps of the pipeline, J = 0 .. NST-1 of them, unrolled: step J
// computes one register set and reads the other (except the very last), and
// waits until the copies of step J+2 have landed while those still issued
// after it stay in flight.
template <class Ops, int NST, int PER, int J>
__device__ __forceinline__ void pipe_tail(typename Ops::Frags& F0, typename Ops::Frags& F1,
                                          uint8_t* smem, int ks, const typename Ops::Lane& L,
                                          typename Ops::Acc& acc) {
  if constexpr (J < NST) {
    constexpr bool RD = J + 1 < NST;
    const uint8_t* nx = smem + ((ks + J + 1) % NST) * Ops::STAGE;
    if constexpr (J % 2 == 0) pipe_step<Ops, RD>(F0, F1, nx, L, acc);
    else pipe_step<Ops, RD>(F1, F0, nx, L, acc);
    if constexpr (J + 3 <= NST) QG_WAIT_VM_BARRIER((NST - 3 - J) * PER);
    pipe_tail<Ops, NST, PER, J + 1>(F0, F1, smem, ks, L, acc);
  }
}

// NST LDS stages (even, >= 4); requires KS even and >= NST (checked on the
// host).
template <class Ops, int NST>
__global__ __launch_bounds__(kThreads) void pipe256_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ w_sc,
    const float* __restrict__ scale_a, const float* __restrict__ scale_b,
    const uint16_t* __restrict__ col_scale, uint16_t* __restrict__ c, PipeArgs g) {
  constexpr int PER = Ops::DMA;
  static_assert(NST % 2 == 0 && NST >= 4, "stage ring");
  constexpr int LDS_BYTES = NST * Ops::STAGE > kCTileBytes ? NST * Ops::STAGE : kCTileBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
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

  PipeRsrc rs;
  rs.a = make_rsrc(a, g.a_bytes);
  rs.w = make_rsrc(wp, g.w_bytes);
  rs.sa = make_rsrc(g.asc_bytes ? a_sc : a, g.asc_bytes);
  rs.sw = make_rsrc(g.wsc_bytes ? w_sc : wp, g.wsc_bytes);
  const int row_bytes = Ops::row_bytes(g.K);
  const typename Ops::Lane L = Ops::lane_offsets(wm, wn, lane);

  typename Ops::Acc acc;
  Ops::zero(acc);
  const int KS = g.KS;
  auto stage = [&](int s) { return smem + (s % NST) * Ops::STAGE; };
  auto issue = [&](int s) {
    uint8_t* st = stage(s);
    pipe_issue_a<Ops>(st, s, wave, lane, m0, row_bytes, rs.a);
    Ops::issue_rest(st, s, wave, lane, m0, cg0, g, rs);
  };

  // Step s lives in stage s % NST; the copies of step s are issued NST - 1
  // steps ahead, into the stage whose fragments were consumed one step ago.
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue(s);
  QG_WAIT_VM_BARRIER((NST - 3) * PER);   // steps 0 and 1 landed
  typename Ops::Frags F0, F1;
  Ops::init(F0, F1);
  pipe_read_all<Ops>(F0, stage(0), L);

  // Two steps per iteration, F0 and F1 trading roles; every copy issued in
  // here is in range (ks + NST < KS).  At the end of step ks the copies of
  // step ks+2 must have landed (its fragments are read during step ks+1).
  // step_issuing(cur, nxt, r, s): compute with cur, read step r into nxt,
  // issue the copies of step s
  auto step_issuing = [&](typename Ops::Frags& cur, typename Ops::Frags& nxt, int r, int s) {
    // the 4-stage fallback ring of the unpinned (weight-only) kernels keeps
    // its copies ahead of the step: interleaving them made one spill
    if constexpr (Ops::CP_INTERLEAVE && !(Ops::CP_PIN_PAIRS == 0 && NST == 4)) {
      uint8_t* st = stage(s);
      auto cp = [&](int part) {
        if (part == 0) pipe_issue_a<Ops>(st, s, wave, lane, m0, row_bytes, rs.a);
        if (part == 1) Ops::issue_rest(st, s, wave, lane, m0, cg0, g, rs);
      };
      pipe_step<Ops, true, true>(cur, nxt, stage(r), L, acc, cp);
    } else {
      issue(s);
      pipe_step<Ops, true>(cur, nxt, stage(r), L, acc);
    }
  };
  int ks = 0;
  for (; ks + NST < KS; ks += 2) {
    step_issuing(F0, F1, ks + 1, ks + NST - 1);
    QG_WAIT_VM_BARRIER((NST - 3) * PER);
    step_issuing(F1, F0, ks + 2, ks + NST);
    QG_WAIT_VM_BARRIER((NST - 3) * PER);
  }
  // last NST steps (ks == KS - NST), copies issued up to step KS - 2
  issue(ks + NST - 1);
  pipe_tail<Ops, NST, PER, 0>(F0, F1, smem, ks, L, acc);

  PipeOut o;
  o.c = c;
  o.col_scale = col_scale;
  o.s = (Ops::FMT == 4) ? (*scale_a) * (*scale_b) : (Ops::FMT == 7) ? *scale_a : 1.0f;
  o.M = g.M;
  o.N = g.N;
  __syncthreads();   // every wave has finished with the last stage
  Ops::stage(acc, smem, o, cg0 * 16, wm, wn, lane);
  __syncthreads();
  pipe_copy_out(smem, o, m0, cg0 * 16);
}

// ---- MXFP4, 256 x 256 tiles, 256-element K steps ------------------------
// 256 x 256 output tile per workgroup, NW waves (4: one per SIMD, each owning
// a 128 x 128 block of C, 4 x 4 fragments of 32 x 32; 8: two per SIMD, 128 x
// 64 each).  A K step is one packed W tile: 256 elements, 128 bytes of an A
// row, so every A copy reads whole 128-byte lines (8 rows x 128 B per
// instruction).  The earlier 64-byte step read halves of 16 lines per
// instruction, which the vector memory path serves several times slower; at
// M = N = K = 8192 the move took the GEMM from 296 to 274 us.  Four and eight
// waves measured the same (274 / 277 us), and so did issuing all of a step's
// copies in one quarter or spreading them over two; with no copies in the loop
// at all the kernel takes 205 us, so the copies and the compute side (matrix
// instructions, LDS fragment reads, the per-step barrier) each hold part of
// the time.
//
// LDS, two stages s = 0, 1 of each part (the A and W parts of both stages
// sit below 64 KB and 128 KB so that one address register per quarter and a
// constant offset reach every fragment):
//   A  [s][256 rows][128 B] at 32 KB s, 16-byte chunk c of row r at slot
//      c ^ ((r >> 1) & 7): a fragment read (32 rows, one chunk each) then
//      hits 16 distinct 16-byte bank groups per 16 lanes;
//   W  [s][16 tiles][2 KB] at 64 KB + 32 KB s: the packed tiles of the step as
//      they are ([chunk 8][column 16][16 B], chunk c = K elements 32c + [0,
//      32) of the step);
//   SA [s][256 rows][8 B] at 128 KB + 2 KB s: the eight E8M0 bytes of each A
//      row;
//   SB [s][2][1 KB] at 132 KB + 2 KB s: the packed W scale chunks of the step
//      for the two 128-column halves ([chunk 8][column 16][tile 8]).
// Quarter u (0..3) of a step is one matrix instruction per fragment pair;
// lane l feeds row (column) l & 31 with chunk 4j + u (j = l >> 5), so the
// instruction covers blocks u and 4 + u and each lane's scale is byte u of
// dword j of its row's (column's) eight scale bytes.
template <int NW>
struct Mx256 {
  static constexpr int FN = 16 / NW;                    // 32-column fragments per wave
  static constexpr int THREADS = 64 * NW;
  static constexpr int ROW = 128;                         // A bytes per row and step
  static constexpr int A_STAGE = kBig * ROW;              // 32 KB
  static constexpr int W_OFF = 2 * A_STAGE;               // 64 KB
  static constexpr int W_STAGE = 16 * kTileBytes;         // 32 KB
  static constexpr int SA_OFF = W_OFF + 2 * W_STAGE;      // 128 KB
  static constexpr int SA_STAGE = kBig * 8;               // 2 KB
  static constexpr int SB_OFF = SA_OFF + 2 * SA_STAGE;    // 132 KB
  static constexpr int SB_STAGE = 2048;
  static constexpr int LDS = SB_OFF + 2 * SB_STAGE;       // 136 KB
  typedef floatx16 Acc[4][FN];
  struct Quarter {
    uintx4 a[4];
    uintx4 b[FN];
    uint32_t sb[FN / 2];   // the scale bytes of the lane's column in this wave's tiles
  };
  struct Lane {
    int a[4], b[4], sb, sa;   // stage 0; quarter u of sb is 128 u further
    uint32_t shb;
  };
  __device__ __forceinline__ static int swizzle(int r) { return (r >> 1) & 7; }
  // wave (wm, wn): rows 128 wm + [0, 128), columns 32 FN wn + [0, 32 FN) =
  // column tiles 2 FN wn .. 2 FN wn + 2 FN - 1
  __device__ __forceinline__ static Lane lane_offsets(int wm, int wn, int lane) {
    const int r = wm * 128 + (lane & 31), j = lane >> 5;
    const int par = (lane >> 4) & 1;
    Lane L;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 4 * j + u;
      L.a[u] = r * ROW + 16 * (c ^ swizzle(r));
      L.b[u] = W_OFF + (wn * 2 * FN + par) * kTileBytes + c * 256 + 16 * (lane & 15);
    }
    // the wave's tiles are dwords (2 FN wn / 4 ..) of its column's 8-byte
    // entry in 128-column half 2 FN wn / 8
    L.sb = SB_OFF + (2 * FN * wn / 8) * 1024 + 4 * j * 128 + 8 * (lane & 15) +
           4 * ((2 * FN * wn / 4) & 1);
    L.sa = SA_OFF + 8 * r + 4 * j;
    L.shb = 8u * par;
    return L;
  }
  template <int S, int U>
  __device__ __forceinline__ static void read(Quarter& X, const uint8_t* lds, const Lane& L) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
      X.a[fm] = *reinterpret_cast<const uintx4*>(lds + L.a[U] + (S * A_STAGE + fm * 32 * ROW));
#pragma unroll
    for (int p = 0; p < FN; ++p)
      X.b[p] =
          *reinterpret_cast<const uintx4*>(lds + L.b[U] + (S * W_STAGE + p * 2 * kTileBytes));
#pragma unroll
    for (int d = 0; d < FN / 2; ++d)
      X.sb[d] = *reinterpret_cast<const uint32_t*>(lds + L.sb + (S * SB_STAGE + U * 128 + 4 * d));
  }
  template <int S>
  __device__ __forceinline__ static void read_sa(uint32_t (&sa)[4], const uint8_t* lds,
                                                 const Lane& L) {
#pragma unroll
    for (int fm = 0; fm < 4; ++fm)
      sa[fm] = *reinterpret_cast<const uint32_t*>(lds + L.sa + (S * SA_STAGE + fm * 32 * 8));
  }
  template <int U, int P>
  __device__ __forceinline__ static void mma_pair(const Quarter& X, const uint32_t (&sa)[4],
                                                  const Lane& L, Acc& acc) {
    const intx8 bf = {(int)X.b[P][0], (int)X.b[P][1], (int)X.b[P][2], (int)X.b[P][3],
                      0, 0, 0, 0};
    // byte 2 (P & 1) of the shifted word P / 2: tile 2P + par of the wave's
    const int sb = (int)(X.sb[P >> 1] >> L.shb);
#pragma unroll
    for (int fm = 0; fm < 4; ++fm) {
      const intx8 af = {(int)X.a[fm][0], (int)X.a[fm][1], (int)X.a[fm][2], (int)X.a[fm][3],
                        0, 0, 0, 0};
      acc[fm][P] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          af, bf, acc[fm][P], kFmtFP4, kFmtFP4, U, (int)sa[fm], 2 * (P & 1), sb);
    }
  }
  template <int U>
  __device__ __forceinline__ static void mma(const Quarter& X, const uint32_t (&sa)[4],
                                             const Lane& L, Acc& acc) {
    mma_pair<U, 0>(X, sa, L, acc);
    mma_pair<U, 1>(X, sa, L, acc);
    if constexpr (FN == 4) {
      mma_pair<U, 2>(X, sa, L, acc);
      mma_pair<U, 3>(X, sa, L, acc);
    }
  }

  // The copies of a step (32 of A: 8 rows x 128 B each; 16 W tiles: two 1 KB
  // halves each; 8 of A scales: 32 rows x 8 B each; 8 of W scales: 256 B
  // each), split evenly over the waves.  Everything but the step's own
  // offset is fixed per wave and lane.
  static constexpr int NA = 32 / NW, NT = 16 / NW, NS = 8 / NW;
  static constexpr int COPIES = NA + 2 * NT + 2 * NS;
  struct Copies {
    __amdgpu_buffer_rsrc_t ra, rw, rsa, rsw;
    uint32_t a_base[NA];   // A: row offset plus the lane's chunk
    int a_kb[NA];          // A: the chunk's byte within a step
    uint32_t w_base[NT];   // W: the tile's first K tile plus the lane's 16 B
    uint32_t sa_base[NS];  // A scales: the lane's row and dword
    int sa_kb;             // A scales: the dword's byte within a step (0 or 4)
    uint32_t sw_base[NS];  // W scales: the copy's 256 B in step 0
    int row_bytes, sc_cols, KT;
    int a_lds[NA], w_lds[NT], sa_lds[NS], sw_lds[NS];
  };
  __device__ __forceinline__ static Copies plan(int wave, int lane, int m0, int cg0,
                                                const PipeArgs& g, const PipeRsrc& rs) {
    Copies C;
    C.ra = rs.a;
    C.rw = rs.w;
    C.rsa = rs.sa;
    C.rsw = rs.sw;
    C.row_bytes = g.K / 2;
    C.sc_cols = g.K / 32;
    C.KT = g.KT;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int q = NA * wave + i;
      const int r = 8 * q + (lane >> 3);
      const int c = (lane & 7) ^ swizzle(r);
      C.a_kb[i] = 16 * c;
      C.a_base[i] = (uint32_t)(m0 + r) * (uint32_t)C.row_bytes + 16u * c;
      C.a_lds[i] = q * 1024;
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = NT * wave + i;
      C.w_base[i] = (uint32_t)(cg0 + t) * (uint32_t)g.KT * kTileBytes + 16u * lane;
      C.w_lds[i] = t * kTileBytes;
    }
    C.sa_kb = 4 * (lane & 1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int q = NS * wave + i;   // 0 .. 7
      C.sa_base[i] = (uint32_t)(m0 + 32 * q + (lane >> 1)) * (uint32_t)C.sc_cols + C.sa_kb;
      C.sa_lds[i] = 256 * q;
      C.sw_base[i] = (uint32_t)(cg0 / 8 + (q >> 2)) * (uint32_t)g.KS * 512u + 256u * (q & 3) +
                     4u * lane;
      C.sw_lds[i] = 256 * q;
    }
    return C;
  }
  // K % 128 == 0, so a 16-byte A chunk or a 4-byte scale word is wholly
  // inside K or past it; past it the copy reads zeros, and so does every copy
  // of a step s >= KT (all-zero codes and scales: such a step adds exactly 0)
  // Part H (0 or 1) of the copies of step s: half of the A and W copies and
  // half of the scale copies (with one scale copy of each kind per wave, the
  // A scales go in part 0 and the W scales in part 1).
  static constexpr int PART_COPIES = COPIES / 2;
  template <int S, int H>
  __device__ __forceinline__ static void issue(uint8_t* lds, int s, const Copies& C) {
    uint8_t* const sta = lds + S * A_STAGE;
    uint8_t* const stw = lds + W_OFF + S * W_STAGE;
#pragma unroll
    for (int i = H * NA / 2; i < (H + 1) * NA / 2; ++i) {
      const int kb = s * ROW + C.a_kb[i];
      dma16(C.ra, sta + C.a_lds[i],
            kb < C.row_bytes ? C.a_base[i] + (uint32_t)s * ROW : kOutOfRange);
    }
    const bool in_kt = s < C.KT;
#pragma unroll
    for (int i = H * NT / 2; i < (H + 1) * NT / 2; ++i) {
      const uint32_t off = in_kt ? C.w_base[i] + (uint32_t)s * kTileBytes : kOutOfRange;
      dma16(C.rw, stw + C.w_lds[i], off);
      dma16(C.rw, stw + C.w_lds[i] + 1024, off + 1024u);
    }
    const bool sa_in = 8 * s + C.sa_kb < C.sc_cols;
    if constexpr (NS == 1) {
      if constexpr (H == 0)
        dma4(C.rsa, lds + SA_OFF + S * SA_STAGE + C.sa_lds[0],
             sa_in ? C.sa_base[0] + 8u * s : kOutOfRange);
      else
        dma4(C.rsw, lds + SB_OFF + S * SB_STAGE + C.sw_lds[0],
             in_kt ? C.sw_base[0] + 1024u * s : kOutOfRange);
    } else {
#pragma unroll
      for (int i = H * NS / 2; i < (H + 1) * NS / 2; ++i) {
        dma4(C.rsa, lds + SA_OFF + S * SA_STAGE + C.sa_lds[i],
             sa_in ? C.sa_base[i] + 8u * s : kOutOfRange);
        dma4(C.rsw, lds + SB_OFF + S * SB_STAGE + C.sw_lds[i],
             in_kt ? C.sw_base[i] + 1024u * s : kOutOfRange);
      }
    }
  }
};

// 32 x 32 accumulators of a 128 x 32 FN wave block -> the LDS C tile.
template <int NW>
__device__ __forceinline__ void mx256_stage(const typename Mx256<NW>::Acc& acc, uint8_t* ct,
                                          int wm, int wn, int lane) {
  constexpr int FN = Mx256<NW>::FN;
#pragma unroll
  for (int fm = 0; fm < 4; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int col = wn * 32 * FN + fn * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = wm * 128 + fm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        *reinterpret_cast<uint16_t*>(ct + c_tile_offset(row, col)) =
            round_out<false>(acc[fm][fn][e]);
      }
    }
}

// vmcnt(0) and lgkmcnt(0), then a bare workgroup barrier: this wave's copies
// have landed and its LDS reads have returned
#define QG_WAIT_ALL_BARRIER()                          \
  do {                                                 \
    __builtin_amdgcn_sched_barrier(0);                 \
    __builtin_amdgcn_s_waitcnt(0x0070);                \
    __builtin_amdgcn_s_barrier();                      \
    __builtin_amdgcn_sched_barrier(0);                 \
  } while (0)

// Step s, in stage S = s % 2.  Quarters 0-2 compute from registers while
// the next quarter's fragments arrive; then every wave waits for its copies
// of step s + 1 and for its reads of stage S, and meets the others.  Quarter 3
// reads quarter 0 of step s + 1 and, as stage S is now free, issues the first
// half of the copies of step s + 2 into it; quarter 0 of step s + 1 issues the
// second half (the same time was measured with all of them in quarter 3).
// Each copy is pinned beside a matrix instruction.  (In the last two steps
// these read and copy steps past K: zeros, never used.)
template <class P, int N>
__device__ __forceinline__ void pin_copies() {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix instruction
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one vector memory read
  }
}

template <int NW, int S, class P = Mx256<NW>>
__device__ __forceinline__ void mx256_step(typename P::Quarter& X0, typename P::Quarter& X1,
                                           uint32_t (&sc)[4], uint32_t (&sn)[4], uint8_t* lds,
                                           int s, const typename P::Lane& L,
                                           typename P::Acc& acc, const typename P::Copies& C) {
  constexpr int PAIRS = P::PART_COPIES < 4 * P::FN ? P::PART_COPIES : 4 * P::FN;
  P::template read<S, 1>(X1, lds, L);
  P::template mma<0>(X0, sc, L, acc);
  P::template issue<1 - S, 1>(lds, s + 1, C);   // second half of step s + 1
  pin_copies<P, PAIRS>();
  __builtin_amdgcn_sched_barrier(0);
  P::template read<S, 2>(X0, lds, L);
  P::template mma<1>(X1, sc, L, acc);
  __builtin_amdgcn_sched_barrier(0);
  P::template read<S, 3>(X1, lds, L);
  P::template mma<2>(X0, sc, L, acc);
  QG_WAIT_ALL_BARRIER();
  P::template read<1 - S, 0>(X0, lds, L);
  P::template read_sa<1 - S>(sn, lds, L);
  P::template mma<3>(X1, sc, L, acc);
  P::template issue<S, 0>(lds, s + 2, C);       // first half of step s + 2
  pin_copies<P, PAIRS>();
  __builtin_amdgcn_sched_barrier(0);
}

// MXFP4, M and N > 128, K % 128 == 0, at least two 256-element K tiles.
template <int NW>
__global__ __launch_bounds__(64 * NW) void mx256_kernel(
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ a_sc,
    const uint8_t* __restrict__ wp, const uint8_t* __restrict__ w_sc,
    uint16_t* __restrict__ c, PipeArgs g) {
  using P = Mx256<NW>;
  constexpr int LDS_BYTES = P::LDS > kCTileBytes ? P::LDS : kCTileBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / (NW / 2);
  const int wn = wave % (NW / 2);

  // XCD-aware tile walk, as in pipe256_kernel
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

  PipeRsrc rs;
  rs.a = make_rsrc(a, g.a_bytes);
  rs.w = make_rsrc(wp, g.w_bytes);
  rs.sa = make_rsrc(a_sc, g.asc_bytes);
  rs.sw = make_rsrc(w_sc, g.wsc_bytes);
  const typename P::Copies C = P::plan(wave, lane, m0, cg0, g, rs);
  const typename P::Lane L = P::lane_offsets(wm, wn, lane);

  typename P::Acc acc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < P::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int KT = g.KT;

  // step s lives in stage s % 2; its copies go out in quarter 3 of step s - 2
  P::template issue<0, 0>(smem, 0, C);
  P::template issue<0, 1>(smem, 0, C);
  P::template issue<1, 0>(smem, 1, C);   // its other half goes out in step 0
  QG_WAIT_VM_BARRIER(P::PART_COPIES);    // step 0 landed
  typename P::Quarter X0, X1;
  uint32_t sa0[4], sa1[4];
  P::template read<0, 0>(X0, smem, L);
  P::template read_sa<0>(sa0, smem, L);

  // an even number of steps: for odd KT the last one is all zeros
  const int KP = KT + (KT & 1);
  for (int s = 0; s < KP; s += 2) {
    mx256_step<NW, 0>(X0, X1, sa0, sa1, smem, s, L, acc, C);
    mx256_step<NW, 1>(X0, X1, sa1, sa0, smem, s + 1, L, acc, C);
  }
  // the copies of steps KP and KP + 1 (all zeros) land before the LDS is
  // reused for the output tile
  __builtin_amdgcn_s_waitcnt(0x0F70);

  PipeOut o;
  o.c = c;
  o.M = g.M;
  o.N = g.N;
  __syncthreads();   // every wave has finished with the last stage
  mx256_stage<NW>(acc, smem, wm, wn, lane);
  __syncthreads();
  pipe_copy_out<64 * NW>(smem, o, m0, cg0 * 16);
}

// waves per workgroup (four and eight measured the same)
constexpr int kMx256Waves = 4;

hipError_t launch_mx256(const void* a, const void* a_sc, const void* wp, void* c, int64_t M,
                        int64_t N, int64_t K, hipStream_t stream) {
  const PackGeom pg = pack_geom(3, K, N);
  PipeArgs g;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.KT = (int)pg.kt;
  g.KS = 2 * (int)pg.kt;
  g.CG = (int)pg.cg;
  g.tiles_m = (int)cdiv(M, kBig);
  g.tiles_n = (int)cdiv(N, kBig);
  g.a_bytes = (uint32_t)(M * (K / 2));
  g.w_bytes = (uint32_t)pg.codes;
  g.asc_bytes = (uint32_t)(M * (K / 32));
  g.wsc_bytes = (uint32_t)(pg.total - pg.scales);
  const uint8_t* w_sc = static_cast<const uint8_t*>(wp) + pg.scales;
  hipLaunchKernelGGL(mx256_kernel<kMx256Waves>, dim3((unsigned)(g.tiles_m * g.tiles_n)),
                     dim3(64 * kMx256Waves), 0,
                     stream, static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(a_sc),
                     static_cast<const uint8_t*>(wp), w_sc, static_cast<uint16_t*>(c), g);
  return hipGetLastError();
}

// a_sc: MXFP4 activation scales; col_scale: W4A16/W8A16 column scales;
// sa, sb: FP8 per-tensor scales (unused arguments may be null).
template <class Ops, int NST>
hipError_t launch_pipe_nst(const PipeArgs& g, const void* a, const void* a_sc, const void* wp,
                           const uint8_t* w_sc, const float* sa, const float* sb,
                           const void* col_scale, void* c, hipStream_t stream) {
  hipLaunchKernelGGL((pipe256_kernel<Ops, NST>), dim3((unsigned)(g.tiles_m * g.tiles_n)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(a),
                     static_cast<const uint8_t*>(a_sc), static_cast<const uint8_t*>(wp), w_sc,
                     sa, sb, static_cast<const uint16_t*>(col_scale), static_cast<uint16_t*>(c), g);
  return hipGetLastError();
}

// group_k: grouped weight-only formats (their metadata segment is the second
// weight buffer); 0 otherwise.
template <class Ops>
hipError_t launch_pipe(const void* a, const void* a_sc, const void* wp, const float* sa,
                       const float* sb, const void* col_scale, void* c, int64_t M, int64_t N,
                       int64_t K, hipStream_t stream, int64_t group_k = 0) {
  constexpr int FMT = Ops::FMT;
  const PackGeom pg = pack_geom(FMT, K, N);
  PipeArgs g;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.KT = (int)pg.kt;
  g.KS = Ops::STEPS_PER_TILE * (int)pg.kt;
  g.CG = (int)pg.cg;
  g.tiles_m = (int)cdiv(M, kBig);
  g.tiles_n = (int)cdiv(N, kBig);
  const int64_t a_row = FMT == 3 ? K / 2 : FMT == 4 ? K : 2 * K;
  g.a_bytes = (uint32_t)(M * a_row);
  g.w_bytes = (uint32_t)pg.codes;
  g.asc_bytes = FMT == 3 ? (uint32_t)(M * (K / 32)) : 0u;
  g.wsc_bytes = FMT == 3 || FMT == 7 ? (uint32_t)(pg.total - pg.scales) : 0u;
  const uint8_t* w_sc =
      FMT == 3 || FMT == 7 ? static_cast<const uint8_t*>(wp) + pg.scales : nullptr;
  if constexpr (Ops::GROUP_WORDS > 0) {
    const PackGeom gg = grouped_geom(FMT == 1 ? 5 : 6, K, N, group_k);
    g.wsc_bytes = (uint32_t)(gg.total - gg.scales);
    w_sc = static_cast<const uint8_t*>(wp) + gg.scales;
  }
  // the deepest ring that fits in LDS, when K has at least that many steps
  if (Ops::NST > 4 && g.KS >= Ops::NST)
    return launch_pipe_nst<Ops, Ops::NST>(g, a, a_sc, wp, w_sc, sa, sb, col_scale, c, stream);
  return launch_pipe_nst<Ops, 4>(g, a, a_sc, wp, w_sc, sa, sb, col_scale, c, stream);
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

hipError_t launch_weight_only_tile(int fmt, const void* x, const void* w_packed,
                                  const void* scales, void* y, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream) {
  if (fmt == 1)
    return launch_pipe<F16Pipe<1>>(x, nullptr, w_packed, nullptr, nullptr, scales, y, M, N, K,
                                   stream);
  if (fmt == 2)
    return launch_pipe<F16Pipe<2>>(x, nullptr, w_packed, nullptr, nullptr, scales, y, M, N, K,
                                   stream);
  return hipErrorInvalidValue;
}

hipError_t launch_weight_only_tile_grouped(int fmt, const void* x, const void* w_packed, void* y,
                                          int64_t M, int64_t N, int64_t K, int64_t group_k,
                                          hipStream_t stream) {
#define QG_GROUPED(W, NG)                                                                   \
  return launch_pipe<F16Pipe<W, NG>>(x, nullptr, w_packed, nullptr, nullptr, nullptr, y, M, N, \
                                     K, stream, group_k);
  const int ngt = grouped_ngt(group_k);
  if (fmt == 5) {
    if (ngt == 1) QG_GROUPED(1, 1)
    if (ngt == 2) QG_GROUPED(1, 2)
    QG_GROUPED(1, 4)
  }
  if (fmt == 6) {
    if (ngt == 1) QG_GROUPED(2, 1)
    if (ngt == 2) QG_GROUPED(2, 2)
    QG_GROUPED(2, 4)
  }
#undef QG_GROUPED
  return hipErrorInvalidValue;
}

hipError_t launch_weight_only_tile_nvfp4(const void* x, const void* w_packed,
                                        const float* global_scale, void* y, int64_t M, int64_t N,
                                        int64_t K, hipStream_t stream) {
  return launch_pipe<F16Pipe<7>>(x, nullptr, w_packed, global_scale, nullptr, nullptr, y, M, N, K,
                                 stream);
}

hipError_t launch_tile_gemm(int fmt, const void* a, const void* a_e8m0, const void* w_packed,
                            const float* scale_a, const float* scale_b, void* c, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream) {
  // large tiles once both output dimensions fill them and K spans at least
  // two 256-element tiles; the 128 x 128 kernel covers the rest (and MXFP4 K
  // that is not a multiple of 128, whose scale rows the 4-byte copies of the
  // large kernel cannot split)
  const bool big = M > 128 && N > 128 && cdiv(K, kTileK8) >= 2 && pipe_fits(fmt, M, N, K, 0);
  if (fmt == 3) {
    if (big && K % 128 == 0 && cdiv(K, kTileK4) >= 2)
      return launch_mx256(a, a_e8m0, w_packed, c, M, N, K, stream);
    return launch_tiles<true, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  if (fmt == 4) {
    if (big)
      return launch_pipe<Fp8Pipe>(a, a_e8m0, w_packed, scale_a, scale_b, nullptr, c, M, N, K,
                                  stream);
    return launch_tiles<false, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qgemm
