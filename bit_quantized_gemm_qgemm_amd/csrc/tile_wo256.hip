// LDS-tiled matrix-core GEMM for the weight-only formats at large M (INT4 /
// INT8 per column or grouped, NVFP4 weights; fp16 X): the W4A16 page's
// section 2 and the W8A16 page's Steps 1-2 with the dequantization done in
// registers between the LDS read and the matrix instruction.
#include "qgemm_common.h"
#include "qgemm_dequant.h"
#include "tile_common.h"

namespace qgemm {
namespace {

constexpr int kThreads = 256;        // 4 waves, 2 x 2
// ---------------------------------------------------------------------------
// Large tiles for the weight-only formats (fp16 X): 256 x 256 per workgroup, 128 x 128
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

constexpr int kStepBytes = 64;      // bytes of K per row per step

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

// Operand rsrcs of one workgroup: X, the packed weight codes, and the scale
// or metadata segment (NVFP4, grouped).
struct PipeRsrc {
  __amdgpu_buffer_rsrc_t a, w, sw;
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
// Each lane rounds its scaled accumulators to fp16 (round to nearest even)
// into a row-major [256][512 B] tile in LDS; then the workgroup copies it out
// with 16-byte row-contiguous stores.  16-byte chunk k of row r sits in slot
// k ^ (((r >> 2) & 3) << 2): the rows that one 2-byte write instruction
// touches (4 apart in a 16 x 16 fragment) land in different banks.
__device__ __forceinline__ int c_tile_offset(int row, int col) {
  return row * (kBig * 2) + 16 * ((col >> 3) ^ (((row >> 2) & 3) << 2)) + 2 * (col & 7);
}

// 16 x 16 accumulators: lane holds rows 4 (lane >> 4) + i, column lane & 15.
// COL_SCALE: multiply by the column's fp16 scale (per-column formats), else
// by the per-tensor o.s.
template <bool COL_SCALE>
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
            f32_to_f16_bits(acc[fm][fn][i] * s);
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
    stage16<NGT == 0 && WFMT != 7>(acc, ct, o, n0, wm, wn, lane);
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
    const uint8_t* __restrict__ a, const uint8_t* __restrict__ wp,
    const uint8_t* __restrict__ w_sc, const float* __restrict__ scale_a,
    const uint16_t* __restrict__ col_scale, uint16_t* __restrict__ c, PipeArgs g) {
  constexpr int PER = Ops::DMA;
  static_assert(NST % 2 == 0 && NST >= 4, "stage ring");
  constexpr int LDS_BYTES = NST * Ops::STAGE > kCTileBytes ? NST * Ops::STAGE : kCTileBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1;
  const int wn = wave & 1;

  const TileOrigin to = tile_origin(g);   // XCD-aware tile walk
  const int m0 = to.m0;
  const int cg0 = to.cg0;

  PipeRsrc rs;
  rs.a = make_rsrc(a, g.a_bytes);
  rs.w = make_rsrc(wp, g.w_bytes);
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

// w_sc: the scale or metadata segment (NVFP4, grouped); sa: the NVFP4
// per-tensor scale; col_scale: the W4A16 / W8A16 column scales (unused
// arguments may be null).
template <class Ops, int NST>
hipError_t launch_pipe_nst(const PipeArgs& g, const void* a, const void* wp, const uint8_t* w_sc,
                           const float* sa, const void* col_scale, void* c, hipStream_t stream) {
  hipLaunchKernelGGL((pipe256_kernel<Ops, NST>), dim3((unsigned)(g.tiles_m * g.tiles_n)),
                     dim3(kThreads), 0, stream, static_cast<const uint8_t*>(a),
                     static_cast<const uint8_t*>(wp), w_sc, sa,
                     static_cast<const uint16_t*>(col_scale), static_cast<uint16_t*>(c), g);
  return hipGetLastError();
}

// group_k: grouped weight-only formats (their metadata segment is the second
// weight buffer); 0 otherwise.
template <class Ops>
hipError_t launch_pipe(const void* a, const void* wp, const float* sa, const void* col_scale,
                       void* c, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                       int64_t group_k = 0) {
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
  g.a_bytes = (uint32_t)(M * 2 * K);   // fp16 X
  g.w_bytes = (uint32_t)pg.codes;
  g.asc_bytes = 0;
  g.wsc_bytes = FMT == 7 ? (uint32_t)(pg.total - pg.scales) : 0u;
  const uint8_t* w_sc = FMT == 7 ? static_cast<const uint8_t*>(wp) + pg.scales : nullptr;
  if constexpr (Ops::GROUP_WORDS > 0) {
    const PackGeom gg = grouped_geom(FMT == 1 ? 5 : 6, K, N, group_k);
    g.wsc_bytes = (uint32_t)(gg.total - gg.scales);
    w_sc = static_cast<const uint8_t*>(wp) + gg.scales;
  }
  // the deepest ring that fits in LDS, when K has at least that many steps
  if (Ops::NST > 4 && g.KS >= Ops::NST)
    return launch_pipe_nst<Ops, Ops::NST>(g, a, wp, w_sc, sa, col_scale, c, stream);
  return launch_pipe_nst<Ops, 4>(g, a, wp, w_sc, sa, col_scale, c, stream);
}

}  // namespace

hipError_t launch_weight_only_tile(int fmt, const void* x, const void* w_packed,
                                  const void* scales, void* y, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream) {
  if (fmt == 1)
    return launch_pipe<F16Pipe<1>>(x, w_packed, nullptr, scales, y, M, N, K, stream);
  if (fmt == 2)
    return launch_pipe<F16Pipe<2>>(x, w_packed, nullptr, scales, y, M, N, K, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_weight_only_tile_grouped(int fmt, const void* x, const void* w_packed, void* y,
                                          int64_t M, int64_t N, int64_t K, int64_t group_k,
                                          hipStream_t stream) {
#define QG_GROUPED(W, NG)                                                                   \
  return launch_pipe<F16Pipe<W, NG>>(x, w_packed, nullptr, nullptr, y, M, N, K, stream, group_k);
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
  return launch_pipe<F16Pipe<7>>(x, w_packed, global_scale, nullptr, y, M, N, K, stream);
}

}  // namespace qgemm
