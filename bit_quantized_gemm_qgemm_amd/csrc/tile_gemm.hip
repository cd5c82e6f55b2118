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
// Large tiles for the weight-only formats (fp16 X; MXFP4 and FP8 have their
// own 256 x 256 kernels further down): 256 x 256 per workgroup, 128 x 128
// per wave (256 fp32 accumulators per lane, all in AGPRs).  K advances in
// steps of 64 bytes per row (32 fp16 elements) through a ring of LDS stages
// that the buffer unit fills directly from global memory (no VGPR staging).
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
  float s;                     // NVFP4 weights: the per-tensor scale
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
  o.s = (Ops::FMT == 7) ? *scale_a : 1.0f;
  o.M = g.M;
  o.N = g.N;
  __syncthreads();   // every wave has finished with the last stage
  Ops::stage(acc, smem, o, cg0 * 16, wm, wn, lane);
  __syncthreads();
  pipe_copy_out(smem, o, m0, cg0 * 16);
}

// ---- MXFP4, 256 x 256 tiles, W fragments straight to registers -----------
// Each of the 4 waves owns all 256 rows and 64 columns (4 column tiles) of
// the workgroup's output tile: 8 x 2 fragments of 32 x 32.  No other wave
// reads a wave's W columns, so its W fragments go from global memory straight
// into registers (the packed tiles are already in lane order; one 16-byte
// load per lane and fragment feeds one matrix instruction), and only A and
// its E8M0 bytes pass through LDS, 34 KB per 256-element K step.  That fits a
// ring of four LDS stages, so the copies of step s + 3 go out spread evenly
// over all four quarters of step s instead of in bursts.
//
// The matrix instruction takes W as its first operand and A as its second,
// which yields C transposed in the accumulators: lane l holds C row
// (l & 31) of its 32-row fragment and, for each e >> 2, four consecutive
// columns 8 (e >> 2) + 4 (l >> 5) + [0, 4) of its 32-column fragment, so the
// epilogue writes 8 bytes per lane.
//
// Per quarter u of a step (one 64-element K slice, blocks u and 4 + u of the
// step; lane l feeds chunk 4 (l >> 5) + u of its row or column):
//   - LDS reads of the next quarter's 8 A fragments (and in quarter 3, after
//     the barrier, those of quarter 0 of step s + 1 plus its A scales);
//   - 16 matrix instructions, each beside one memory instruction: the 2 W
//     fragment loads and the W scale dword of the same quarter of step
//     s + WB - 1, then this quarter's share of the copies of step s + 3
//     (8 A copies of 8 rows x 128 B, 2 A-scale copies of 32 rows x 8 B);
//   - after quarter 2: wait until this wave's copies of step s + 1 have
//     landed and its LDS reads have returned, and meet the other waves.
//
// Measured at M = N = K = 8192 against the earlier kernel (2 x 2 waves of
// 128 x 128, A and W both through a two-stage LDS ring with the copies in two
// of the four quarters): 257-270 us against 266-277 us, box to box; a
// three-step W register ring measured the same as two.  Counters on this
// kernel: the matrix pipe 57% busy at 1.76-1.82 GHz, and the clock falls as
// that share rises (1.95 GHz at 45% busy with K = 4096, 1.70 GHz at 63% with
// K = 16384), so part of the remaining gap is the power the operand traffic
// and the matrix pipe draw together.  A persistent form (one workgroup per
// CU, the copy ring running across tile boundaries, results stored straight
// from the accumulators) took the same kernel time and was not kept.
namespace mxw {
constexpr int kRow = 128;                     // A bytes per row and step
constexpr int kAStage = kBig * kRow;          // 32 KB
constexpr int kStage = kAStage + kBig * 8;    // + 8 scale bytes per row
constexpr int kStages = 4;
constexpr int kLds = kStages * kStage;        // 136 KB
constexpr int kOps[4] = {6, 6, 5, 5};         // memory instructions per quarter
// ops issued after the copies of step s + 1 when the wait after quarter 2 of
// step s runs: all of step s - 1 and quarters 0-2 of step s
constexpr int kCopyWait = 22 + 6 + 6 + 5;
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
}  // namespace mxw

// vmcnt = n and lgkmcnt = 0, then a bare workgroup barrier
#define QG_WAIT_VM_LGKM_BARRIER(n)                                              \
  do {                                                                          \
    __builtin_amdgcn_sched_barrier(0);                                          \
    __builtin_amdgcn_s_waitcnt(((n) & 15) | ((((n) >> 4) & 3) << 14) | 0x70);  \
    __builtin_amdgcn_s_barrier();                                               \
    __builtin_amdgcn_sched_barrier(0);                                          \
  } while (0)

struct MxwPlan {
  __amdgpu_buffer_rsrc_t ra, rsa, rw, rsw;
  int rd_a[4];          // LDS: A chunk of quarter u within a stage (fragment fm: + 4096 fm)
  int rd_sa;            // LDS: the lane's row's scale dword (fragment fm: + 256 fm)
  uint32_t w[2];        // W fragment f of step 0 (step s: + 2048 s; quarter u: + 256 u)
  uint32_t ws;          // W scale dword of step 0 (step s: + 1024 s; quarter u: + 128 u)
  uint32_t a_g[8];      // A copy i of step 0 (step s: + 128 s)
  int a_kb[8];          // its chunk's byte within a step
  uint32_t sa_g[2];     // A scale copy i of step 0 (step s: + 8 s)
  int sa_kb;
  int a_lds[8], sa_lds[2];
  uint32_t shb;         // 8 * ((lane >> 4) & 1): the W scale byte of the lane's tile
  int row_bytes, sc_cols, KT;
};

struct MxwW {
  uintx4 b[4][2];       // [quarter][fragment]
  uint32_t s[4];        // [quarter] W scale dword (the wave's 4 tiles)
};

typedef floatx16 MxwAcc[8][2];

template <int U>
__device__ __forceinline__ void mxw_read_a(uintx4 (&x)[8], const uint8_t* st, const MxwPlan& P) {
#pragma unroll
  for (int fm = 0; fm < 8; ++fm)
    x[fm] = *reinterpret_cast<const uintx4*>(st + P.rd_a[U] + fm * 4096);
}

__device__ __forceinline__ void mxw_read_sa(uint32_t (&sa)[8], const uint8_t* st,
                                            const MxwPlan& P) {
#pragma unroll
  for (int fm = 0; fm < 8; ++fm)
    sa[fm] = *reinterpret_cast<const uint32_t*>(st + P.rd_sa + fm * 256);
}

template <int U>
__device__ __forceinline__ void mxw_load_w(MxwW& W, int s, const MxwPlan& P) {
  const bool in = s < P.KT;
#pragma unroll
  for (int f = 0; f < 2; ++f)
    W.b[U][f] = __builtin_amdgcn_raw_buffer_load_b128(
        P.rw, in ? P.w[f] + (uint32_t)s * 2048u + 256u * U : kOutOfRange, 0, 0);
  W.s[U] = __builtin_amdgcn_raw_buffer_load_b32(
      P.rsw, in ? P.ws + (uint32_t)s * 1024u + 128u * U : kOutOfRange, 0, 0);
}

// quarter U's share of the copies of step s into stage memory cst
template <int U>
__device__ __forceinline__ void mxw_copies(uint8_t* cst, int s, const MxwPlan& P) {
#pragma unroll
  for (int i = 2 * U; i < 2 * U + 2; ++i) {
    const int kb = s * mxw::kRow + P.a_kb[i];
    dma16(P.ra, cst + P.a_lds[i], kb < P.row_bytes ? P.a_g[i] + (uint32_t)s * mxw::kRow
                                                   : kOutOfRange);
  }
  if constexpr (U < 2) {
    const bool in = 8 * s + P.sa_kb < P.sc_cols;
    dma4(P.rsa, cst + mxw::kAStage + P.sa_lds[U], in ? P.sa_g[U] + 8u * s : kOutOfRange);
  }
}

template <int U, int F>
__device__ __forceinline__ void mxw_mma_f(const uintx4 (&x)[8], const MxwW& W,
                                          const uint32_t (&sa)[8], int sw, MxwAcc& acc) {
  const intx8 wf = {(int)W.b[U][F][0], (int)W.b[U][F][1], (int)W.b[U][F][2],
                    (int)W.b[U][F][3], 0, 0, 0, 0};
#pragma unroll
  for (int fm = 0; fm < 8; ++fm) {
    const intx8 af = {(int)x[fm][0], (int)x[fm][1], (int)x[fm][2], (int)x[fm][3], 0, 0, 0, 0};
    acc[fm][F] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        wf, af, acc[fm][F], kFmtFP4, kFmtFP4, 2 * F, sw, U, (int)sa[fm]);
  }
}

template <int U>
__device__ __forceinline__ void mxw_mma(const uintx4 (&x)[8], const MxwW& W,
                                        const uint32_t (&sa)[8], uint32_t shb, MxwAcc& acc) {
  const int sw = (int)(W.s[U] >> shb);   // byte 2 f: the lane's tile of fragment f
  mxw_mma_f<U, 0>(x, W, sa, sw, acc);
  mxw_mma_f<U, 1>(x, W, sa, sw, acc);
}

// the quarter's LDS reads first, then one matrix instruction beside one
// memory instruction, N times
template <int N, int R = 8>
__device__ __forceinline__ void mxw_pin() {
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// step s; W[B] holds its W fragments, sa[B] its A scales, x[0] its quarter-0
// A fragments
template <int WB, int B>
__device__ __forceinline__ void mxw_step(int s, uint8_t* lds, MxwW (&W)[WB],
                                         uintx4 (&x)[2][8], uint32_t (&sa)[WB][8],
                                         const MxwPlan& P, MxwAcc& acc) {
  constexpr int BN = (B + WB - 1) % WB;   // W of step s + WB - 1
  constexpr int BS = (B + 1) % WB;        // A scales of step s + 1
  const uint8_t* st = lds + (s & 3) * mxw::kStage;
  const uint8_t* nst = lds + ((s + 1) & 3) * mxw::kStage;
  uint8_t* cst = lds + ((s + 3) & 3) * mxw::kStage;
  const int sw = s + WB - 1;

  mxw_read_a<1>(x[1], st, P);
  mxw_mma<0>(x[0], W[B], sa[B], P.shb, acc);
  mxw_load_w<0>(W[BN], sw, P);
  mxw_copies<0>(cst, s + 3, P);
  mxw_pin<mxw::kOps[0]>();
  __builtin_amdgcn_sched_barrier(0);

  mxw_read_a<2>(x[0], st, P);
  mxw_mma<1>(x[1], W[B], sa[B], P.shb, acc);
  mxw_load_w<1>(W[BN], sw, P);
  mxw_copies<1>(cst, s + 3, P);
  mxw_pin<mxw::kOps[1]>();
  __builtin_amdgcn_sched_barrier(0);

  mxw_read_a<3>(x[1], st, P);
  mxw_mma<2>(x[0], W[B], sa[B], P.shb, acc);
  mxw_load_w<2>(W[BN], sw, P);
  mxw_copies<2>(cst, s + 3, P);
  mxw_pin<mxw::kOps[2]>();
  QG_WAIT_VM_LGKM_BARRIER(mxw::kCopyWait);

  mxw_read_a<0>(x[0], nst, P);
  mxw_read_sa(sa[BS], nst, P);
  mxw_mma<3>(x[1], W[B], sa[B], P.shb, acc);
  mxw_load_w<3>(W[BN], sw, P);
  mxw_copies<3>(cst, s + 3, P);
  mxw_pin<mxw::kOps[3], 16>();
  __builtin_amdgcn_sched_barrier(0);
}

// C tile in LDS for this kernel: row-major [256][512 B], 16-byte chunk k of
// row r at slot k ^ (r & 15), so the 8-byte writes of 32 consecutive rows
// fall into 16 different bank groups.
__device__ __forceinline__ int mxw_c_offset(int row, int col) {
  return row * (kBig * 2) + 16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// MXFP4, M and N > 128, K % 128 == 0, at least two 256-element K tiles.
template <int WB>
__global__ __launch_bounds__(256) void mxw_kernel(const uint8_t* __restrict__ a,
                                                  const uint8_t* __restrict__ a_sc,
                                                  const uint8_t* __restrict__ wp,
                                                  const uint8_t* __restrict__ w_sc,
                                                  uint16_t* __restrict__ c, PipeArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[mxw::kLds];
  static_assert(mxw::kLds >= kCTileBytes, "the C tile reuses the stage memory");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // XCD-aware tile walk, as in the other 256 x 256 kernels
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

  MxwPlan P;
  P.ra = make_rsrc(a, g.a_bytes);
  P.rsa = make_rsrc(a_sc, g.asc_bytes);
  P.rw = make_rsrc(wp, g.w_bytes);
  P.rsw = make_rsrc(w_sc, g.wsc_bytes);
  P.row_bytes = g.K / 2;
  P.sc_cols = g.K / 32;
  P.KT = g.KT;
  {
    const int cl = lane & 31, j = lane >> 5, par = (lane >> 4) & 1;
#pragma unroll
    for (int u = 0; u < 4; ++u) P.rd_a[u] = cl * mxw::kRow + 16 * ((4 * j + u) ^ mxw::swz(cl));
    P.rd_sa = mxw::kAStage + 8 * cl + 4 * j;
#pragma unroll
    for (int f = 0; f < 2; ++f)
      P.w[f] = (uint32_t)(cg0 + 4 * wave + 2 * f + par) * (uint32_t)g.KT * 2048u +
               1024u * j + 16u * (lane & 15);
    P.ws = (uint32_t)(cg0 / 8 + (wave >> 1)) * (uint32_t)g.KS * 512u + 512u * j +
           8u * (lane & 15) + 4u * (wave & 1);
    P.shb = 8u * par;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = 8 * wave + i;
      const int r = 8 * q + (lane >> 3);
      const int ch = (lane & 7) ^ mxw::swz(r);
      P.a_kb[i] = 16 * ch;
      P.a_g[i] = (uint32_t)(m0 + r) * (uint32_t)P.row_bytes + 16u * ch;
      P.a_lds[i] = q * 1024;
    }
    P.sa_kb = 4 * (lane & 1);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = 2 * wave + i;
      P.sa_g[i] = (uint32_t)(m0 + 32 * q + (lane >> 1)) * (uint32_t)P.sc_cols + P.sa_kb;
      P.sa_lds[i] = 256 * q;
    }
  }

  MxwAcc acc;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][f][e] = 0.f;

  // prologue: the W of steps 0 .. WB - 2, then the copies of steps 0, 1, 2.
  // The W loads go first so that, as in the loop, plenty of memory
  // instructions follow each of them: the compiler's waits for these
  // registers at the loop head take the smaller count of the two paths.
  MxwW W[WB];
#pragma unroll
  for (int b = 0; b < WB - 1; ++b) {
    mxw_load_w<0>(W[b], b, P);
    mxw_load_w<1>(W[b], b, P);
    mxw_load_w<2>(W[b], b, P);
    mxw_load_w<3>(W[b], b, P);
  }
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    uint8_t* cst = smem + s * mxw::kStage;
    mxw_copies<0>(cst, s, P);
    mxw_copies<1>(cst, s, P);
    mxw_copies<2>(cst, s, P);
    mxw_copies<3>(cst, s, P);
  }
  QG_WAIT_VM_BARRIER(20);   // the W loads and step 0's copies landed
  uintx4 x[2][8];
  uint32_t sa[WB][8];
  mxw_read_a<0>(x[0], smem, P);
  mxw_read_sa(sa[0], smem, P);
  // nothing of the lgkm counter left pending on the way into the loop (the
  // kernel-argument loads count there too, out of order), so the compiler's
  // wait at the loop head is the loop's own
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)

  const int KS = g.KT;   // one step per 256-element K tile
  int s = 0;
  for (; s + WB <= KS; s += WB) {
    mxw_step<WB, 0>(s, smem, W, x, sa, P, acc);
    mxw_step<WB, 1>(s + 1, smem, W, x, sa, P, acc);
    if constexpr (WB == 3) mxw_step<WB, 2>(s + 2, smem, W, x, sa, P, acc);
  }
  if (s < KS) mxw_step<WB, 0>(s, smem, W, x, sa, P, acc);
  if constexpr (WB == 3)
    if (s + 1 < KS) mxw_step<WB, 1>(s + 1, smem, W, x, sa, P, acc);

  // every copy and load (those past K read zeros) has landed before the stage
  // memory becomes the C tile
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < 8; ++fm)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 32 * fm + (lane & 31);
        const int col = 64 * wave + 32 * f + 8 * q + 4 * (lane >> 5);
        const uintx2 v = {pack_bf16x2(acc[fm][f][4 * q], acc[fm][f][4 * q + 1]),
                          pack_bf16x2(acc[fm][f][4 * q + 2], acc[fm][f][4 * q + 3])};
        *reinterpret_cast<uintx2*>(smem + mxw_c_offset(row, col)) = v;
      }
  __syncthreads();
  const bool vec = (g.N & 7) == 0;
  const int n0 = cg0 * 16;
#pragma unroll 4
  for (int jj = 0; jj < kCTileBytes / 16 / 256; ++jj) {
    const int q = (int)threadIdx.x + 256 * jj;
    const int row = q >> 5, ch = q & 31;
    const int gm = m0 + row, gn = n0 + 8 * ch;
    if (gm >= g.M || gn >= g.N) continue;
    const uintx4 v = *reinterpret_cast<const uintx4*>(smem + row * (kBig * 2) +
                                                      16 * (ch ^ (row & 15)));
    uint16_t* dst = c + (int64_t)gm * g.N + gn;
    if (vec) {
      *reinterpret_cast<uintx4*>(dst) = v;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (gn + t < g.N) dst[t] = (uint16_t)(v[t >> 1] >> (16 * (t & 1)));
    }
  }
}

template <int WB>
hipError_t launch_mxw(const void* a, const void* a_sc, const void* wp, void* c, int64_t M,
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
  hipLaunchKernelGGL(mxw_kernel<WB>, dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(256), 0,
                     stream, static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(a_sc),
                     static_cast<const uint8_t*>(wp), w_sc, static_cast<uint16_t*>(c), g);
  return hipGetLastError();
}

// ---- FP8, 256 x 256 tiles, B fragments straight to registers -------------
// The MXFP4 kernel's design with e4m3 operands: each of the 4 waves owns all
// 256 rows and 64 columns (4 column tiles) of the output tile, loads its B
// fragments straight from the packed tiles into a two-step register ring, and
// reads A from a four-stage LDS ring of 128-byte steps (128 K elements: one
// cache line of every A row, 32 KB per step).  A step is two matrix
// instructions per fragment pair (64 K elements each); lane l feeds row
// (column) l & 31 with the 32-element chunk q = 2 (l >> 5) + u of the step in
// instruction u, i.e. 16-byte chunks 2q, 2q + 1 of the A row and halves 0, 1
// of the packed B tile's lane group q.  An FP8 fragment is 32 bytes per lane,
// so the step runs in four quarters (instruction u, row fragments 4 v ..
// 4 v + 3) to keep the A registers at two quarters' worth.  B is the first
// operand, so the accumulators hold C transposed and the epilogue writes
// 8 bytes per lane; s_a * s_b multiplies the fp32 result.
namespace f8w {
constexpr int kRow = 128;                     // A bytes per row and step
constexpr int kStage = kBig * kRow;           // 32 KB
constexpr int kStages = 4;
constexpr int kLds = kStages * kStage;        // 128 KB
constexpr int kOps = 4;                       // memory instructions per quarter
// ops issued after the copies of step s + 1 when the wait after quarter 2 of
// step s runs: all of step s - 1 and quarters 0-2 of step s
constexpr int kCopyWait = 16 + 3 * kOps;
}  // namespace f8w

struct F8wPlan {
  __amdgpu_buffer_rsrc_t ra, rb;
  int rd_a;             // LDS: A chunk 4 (l >> 5) of the lane's row (XOR 16 (2u + h))
  uint32_t b[2];        // B fragment f of step 0 (step s: + 2048 s; instruction u: + 256 u,
                        // half h: + 1024 h)
  uint32_t a_g[2];      // A copies i = 0, 1 of step 0; copy i: + (i >> 1) * a_step
  int a_kb[2];          // their chunk's byte within a step
  uint32_t a_step;
  int row_bytes, KT;
};

struct F8wB {
  uintx4 b[2][2][2];    // [instruction u][fragment f][half h]
};

typedef floatx16 F8wAcc[8][2];

// quarter Q: instruction u = Q >> 1, row fragments 4 (Q & 1) + [0, 4)
template <int Q>
__device__ __forceinline__ void f8w_read_a(uintx4 (&x)[4][2], const uint8_t* st,
                                           const F8wPlan& P) {
  constexpr int U = Q >> 1, V = Q & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      x[i][h] = *reinterpret_cast<const uintx4*>(st + (P.rd_a ^ (16 * (2 * U + h))) +
                                                 (4 * V + i) * 4096);
}

// B fragment f of instruction U of step s (two 16-byte loads)
template <int U, int F>
__device__ __forceinline__ void f8w_load_b(F8wB& B, int s, const F8wPlan& P) {
  const bool in = s < P.KT;
#pragma unroll
  for (int h = 0; h < 2; ++h)
    B.b[U][F][h] = __builtin_amdgcn_raw_buffer_load_b128(
        P.rb, in ? P.b[F] + (uint32_t)s * 2048u + 256u * U + 1024u * h : kOutOfRange, 0, 0);
}

// copies 2 Q, 2 Q + 1 of this wave for step s (8 rows x 128 B each)
// (a chunk past K reads zeros: the bytes there belong to the next row and
// could be NaN codes, which would survive a multiply by B's zero padding)
template <int Q>
__device__ __forceinline__ void f8w_copies(uint8_t* cst, int s, int wave, const F8wPlan& P) {
#pragma unroll
  for (int i = 2 * Q; i < 2 * Q + 2; ++i) {
    const uint32_t off = P.a_g[i & 1] + (uint32_t)(i >> 1) * P.a_step + (uint32_t)s * f8w::kRow;
    dma16(P.ra, cst + (8 * wave + i) * 1024,
          s * f8w::kRow + P.a_kb[i & 1] < P.row_bytes ? off : kOutOfRange);
  }
}

template <int Q>
__device__ __forceinline__ void f8w_mma(const uintx4 (&x)[4][2], const F8wB& B, F8wAcc& acc) {
  constexpr int U = Q >> 1, V = Q & 1;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const intx8 bf = {(int)B.b[U][f][0][0], (int)B.b[U][f][0][1], (int)B.b[U][f][0][2],
                      (int)B.b[U][f][0][3], (int)B.b[U][f][1][0], (int)B.b[U][f][1][1],
                      (int)B.b[U][f][1][2], (int)B.b[U][f][1][3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const intx8 af = {(int)x[i][0][0], (int)x[i][0][1], (int)x[i][0][2], (int)x[i][0][3],
                        (int)x[i][1][0], (int)x[i][1][1], (int)x[i][1][2], (int)x[i][1][3]};
      acc[4 * V + i][f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          bf, af, acc[4 * V + i][f], kFmtFP8, kFmtFP8, 0, kE8M0One, 0, kE8M0One);
    }
  }
}

template <int N>
__device__ __forceinline__ void f8w_pin() {
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the quarter's LDS reads first
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// step s, in stage S = s % 4; B[S % 2] holds its B fragments, x[0] its
// quarter-0 A fragments
template <int S>
__device__ __forceinline__ void f8w_step(int s, uint8_t* lds, F8wB (&B)[2], uintx4 (&x)[2][4][2],
                                         int wave, const F8wPlan& P, F8wAcc& acc) {
  constexpr int BC = S & 1, BN = 1 - BC;
  const uint8_t* st = lds + S * f8w::kStage;
  const uint8_t* nst = lds + ((S + 1) & 3) * f8w::kStage;
  uint8_t* cst = lds + ((S + 3) & 3) * f8w::kStage;

  f8w_read_a<1>(x[1], st, P);
  f8w_mma<0>(x[0], B[BC], acc);
  f8w_load_b<0, 0>(B[BN], s + 1, P);
  f8w_copies<0>(cst, s + 3, wave, P);
  f8w_pin<f8w::kOps>();
  __builtin_amdgcn_sched_barrier(0);

  f8w_read_a<2>(x[0], st, P);
  f8w_mma<1>(x[1], B[BC], acc);
  f8w_load_b<0, 1>(B[BN], s + 1, P);
  f8w_copies<1>(cst, s + 3, wave, P);
  f8w_pin<f8w::kOps>();
  __builtin_amdgcn_sched_barrier(0);

  f8w_read_a<3>(x[1], st, P);
  f8w_mma<2>(x[0], B[BC], acc);
  f8w_load_b<1, 0>(B[BN], s + 1, P);
  f8w_copies<2>(cst, s + 3, wave, P);
  f8w_pin<f8w::kOps>();
  QG_WAIT_VM_LGKM_BARRIER(f8w::kCopyWait);

  f8w_read_a<0>(x[0], nst, P);
  f8w_mma<3>(x[1], B[BC], acc);
  f8w_load_b<1, 1>(B[BN], s + 1, P);
  f8w_copies<3>(cst, s + 3, wave, P);
  f8w_pin<f8w::kOps>();
  __builtin_amdgcn_sched_barrier(0);
}

// FP8, M and N > 128, at least two 128-element K tiles (K % 16 == 0).
__global__ __launch_bounds__(256) void f8w_kernel(const uint8_t* __restrict__ a,
                                                  const uint8_t* __restrict__ bp,
                                                  const float* __restrict__ scale_a,
                                                  const float* __restrict__ scale_b,
                                                  uint16_t* __restrict__ c, PipeArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[f8w::kLds];
  static_assert(f8w::kLds >= kCTileBytes, "the C tile reuses the stage memory");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

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

  F8wPlan P;
  P.ra = make_rsrc(a, g.a_bytes);
  P.rb = make_rsrc(bp, g.w_bytes);
  P.row_bytes = g.K;
  P.KT = g.KT;
  {
    const int cl = lane & 31, j = lane >> 5, par = (lane >> 4) & 1;
    P.rd_a = cl * f8w::kRow + 16 * ((4 * j) ^ mxw::swz(cl));
#pragma unroll
    for (int f = 0; f < 2; ++f)
      P.b[f] = (uint32_t)(cg0 + 4 * wave + 2 * f + par) * (uint32_t)g.KT * 2048u + 512u * j +
               16u * (lane & 15);
    // copy i covers rows 64 wave + 8 i + [0, 8); copies i and i + 2 differ by
    // 16 rows and share the chunk swizzle
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 64 * wave + 8 * i + (lane >> 3);
      const int ch = (lane & 7) ^ mxw::swz(r);
      P.a_g[i] = (uint32_t)(m0 + r) * (uint32_t)P.row_bytes + 16u * ch;
      P.a_kb[i] = 16 * ch;
    }
    P.a_step = 16u * (uint32_t)P.row_bytes;
  }

  F8wAcc acc;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][f][e] = 0.f;

  // prologue: the B of step 0, then the copies of steps 0, 1, 2.  The B
  // loads go first so that, as in the loop, at least 14 memory instructions
  // follow each of them: the compiler's waits for these registers at the
  // loop head take the smaller count of the two paths into it.
  F8wB B[2];
  f8w_load_b<0, 0>(B[0], 0, P);
  f8w_load_b<0, 1>(B[0], 0, P);
  f8w_load_b<1, 0>(B[0], 0, P);
  f8w_load_b<1, 1>(B[0], 0, P);
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    uint8_t* cst = smem + s * f8w::kStage;
    f8w_copies<0>(cst, s, wave, P);
    f8w_copies<1>(cst, s, wave, P);
    f8w_copies<2>(cst, s, wave, P);
    f8w_copies<3>(cst, s, wave, P);
  }
  QG_WAIT_VM_BARRIER(16);   // B and step 0's copies landed
  uintx4 x[2][4][2];
  f8w_read_a<0>(x[0], smem, P);
  // nothing of the lgkm counter left pending on the way into the loop (the
  // kernel-argument loads count there too, out of order), so the compiler's
  // wait at the loop head is the loop's own
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)

  const int KS = g.KT;   // one step per 128-element K tile
  int s = 0;
  for (; s + 4 <= KS; s += 4) {
    f8w_step<0>(s, smem, B, x, wave, P, acc);
    f8w_step<1>(s + 1, smem, B, x, wave, P, acc);
    f8w_step<2>(s + 2, smem, B, x, wave, P, acc);
    f8w_step<3>(s + 3, smem, B, x, wave, P, acc);
  }
  if (s < KS) f8w_step<0>(s, smem, B, x, wave, P, acc);
  if (s + 1 < KS) f8w_step<1>(s + 1, smem, B, x, wave, P, acc);
  if (s + 2 < KS) f8w_step<2>(s + 2, smem, B, x, wave, P, acc);

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const float sc = (*scale_a) * (*scale_b);
#pragma unroll
  for (int fm = 0; fm < 8; ++fm)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 32 * fm + (lane & 31);
        const int col = 64 * wave + 32 * f + 8 * q + 4 * (lane >> 5);
        const uintx2 v = {pack_bf16x2(acc[fm][f][4 * q] * sc, acc[fm][f][4 * q + 1] * sc),
                          pack_bf16x2(acc[fm][f][4 * q + 2] * sc, acc[fm][f][4 * q + 3] * sc)};
        *reinterpret_cast<uintx2*>(smem + mxw_c_offset(row, col)) = v;
      }
  __syncthreads();
  const bool vec = (g.N & 7) == 0;
  const int n0 = cg0 * 16;
#pragma unroll 4
  for (int jj = 0; jj < kCTileBytes / 16 / 256; ++jj) {
    const int q = (int)threadIdx.x + 256 * jj;
    const int row = q >> 5, ch = q & 31;
    const int gm = m0 + row, gn = n0 + 8 * ch;
    if (gm >= g.M || gn >= g.N) continue;
    const uintx4 v = *reinterpret_cast<const uintx4*>(smem + row * (kBig * 2) +
                                                      16 * (ch ^ (row & 15)));
    uint16_t* dst = c + (int64_t)gm * g.N + gn;
    if (vec) {
      *reinterpret_cast<uintx4*>(dst) = v;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (gn + t < g.N) dst[t] = (uint16_t)(v[t >> 1] >> (16 * (t & 1)));
    }
  }
}

hipError_t launch_f8w(const void* a, const void* bp, const float* sa, const float* sb, void* c,
                      int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const PackGeom pg = pack_geom(4, K, N);
  PipeArgs g;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.KT = (int)pg.kt;
  g.KS = (int)pg.kt;
  g.CG = (int)pg.cg;
  g.tiles_m = (int)cdiv(M, kBig);
  g.tiles_n = (int)cdiv(N, kBig);
  g.a_bytes = (uint32_t)(M * K);
  g.w_bytes = (uint32_t)pg.codes;
  g.asc_bytes = 0;
  g.wsc_bytes = 0;
  hipLaunchKernelGGL(f8w_kernel, dim3((unsigned)(g.tiles_m * g.tiles_n)), dim3(256), 0, stream,
                     static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(bp), sa, sb,
                     static_cast<uint16_t*>(c), g);
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
      return launch_mxw<2>(a, a_e8m0, w_packed, c, M, N, K, stream);
    return launch_tiles<true, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  if (fmt == 4) {
    if (big) return launch_f8w(a, w_packed, scale_a, scale_b, c, M, N, K, stream);
    return launch_tiles<false, 4, 4>(a, a_e8m0, w_packed, scale_a, scale_b, c, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace qgemm
