// 256 x 256 matrix-core kernels for MXFP4 x MXFP4 and FP8 e4m3fn (M above 64,
// N above 128).
//
// The MXFP4 page (section 2) tiles C into B_M x B_N blocks per workgroup and
// sums, per 32-element micro-block, S_A * S_W * dot(A, W) (eq. 1) with the
// scale product done as an exponent add (eq. 2).  On gfx950 that whole step is
// one instruction: v_mfma_scale_f32_32x32x64_f8f6f4 takes FP4 (or FP8) codes
// and one E8M0 byte per lane and block, applies 2^(E_A-127) * 2^(E_W-127) to
// each 32-element block product in hardware and accumulates in fp32.  FP8
// (FP8 page) uses the same instruction with e4m3 operands and unit scales;
// its per-tensor scales multiply the fp32 result once in the epilogue.
#include "qgemm_common.h"
#include "tile_common.h"

namespace qgemm {
namespace {

// The C tile in LDS of both kernels: row-major [256][512 B], 16-byte chunk k of
// row r at slot k ^ (r & 15), so the 8-byte writes of 32 consecutive rows
// fall into 16 different bank groups.
__device__ __forceinline__ int mxw_c_offset(int row, int col) {
  return row * (kBig * 2) + 16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// Copy the staged C tile to C with 16-byte row-contiguous stores (rows past
// M and columns past N are dropped).
__device__ __forceinline__ void mx_copy_out(const uint8_t* smem, uint16_t* __restrict__ c,
                                            const PipeArgs& g, int m0, int n0) {
  const bool vec = (g.N & 7) == 0;
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
//   - 16 matrix instructions;
//   - between the first four of them, the LDS reads of the next quarter's 8 A
//     fragments (in quarter 3, after the barrier, those of quarter 0 of step
//     s + 1 plus its A scales);
//   - beside the first five or six, one memory instruction each: the 2 W
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
// and the matrix pipe draw together.  Builds with the A copies, or the W
// loads, left out ran about 10% faster with the matrix pipe still 56-59%
// busy, so most of the idle share is in the issue schedule of the one wave
// per SIMD rather than in operand traffic.  A persistent form (one workgroup
// per CU, the copy ring running across tile boundaries, results stored
// straight from the accumulators) took the same kernel time and was not kept.
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

struct MxwPlan {
  __amdgpu_buffer_rsrc_t rsa;
  const uint8_t *a_base, *w_base, *wsc_base;   // A codes, W codes, W scales
  uint32_t a_n, w_n, wsc_n;     // their sizes in bytes
  int rd_a[4];          // LDS: A chunk of quarter u within a stage (fragment fm: + 4096 fm)
  int rd_sa;            // LDS: the lane's row's scale dword (fragment fm: + 256 fm)
  uint32_t w[2];        // W fragment f of step 0 (step s: + 2048 s; quarter u: + 256 u)
  uint32_t ws;          // W scale dword of step 0 (step s: + 1024 s; quarter u: + 128 u)
  uint32_t a_g[8];      // A copy i of step 0 (step s: + 128 s)
  uint32_t sa_g[2];     // A scale copy i of step 0 (step s: + 8 s)
  int sa_kb;
  int a_lds[8], sa_lds[2];
  uint32_t shb;         // 8 * ((lane >> 4) & 1): the W scale byte of the lane's tile
  int row_bytes, sc_cols;
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

// A buffer resource over p + off .. p + n (empty once off >= n): the step
// offset lives in the resource, so the lane offsets stay constant and the
// range check still bounds every read
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_from(const uint8_t* p, uint32_t n,
                                                           uint32_t off) {
  // readfirstlane: the clamped difference would otherwise become a VALU
  // saturating subtract and the resource a per-lane value
  const uint32_t left = __builtin_amdgcn_readfirstlane(n > off ? n - off : 0u);
  return make_rsrc(p + off, left);
}

// (a step past the last K tile reads the next column group's tiles, or
// zeros past the end; those registers are never used)
template <int U>
__device__ __forceinline__ void mxw_load_w(MxwW& W, int s, const MxwPlan& P) {
  const __amdgpu_buffer_rsrc_t rw = rsrc_from(P.w_base, P.w_n, (uint32_t)s * 2048u);
  const __amdgpu_buffer_rsrc_t rsw = rsrc_from(P.wsc_base, P.wsc_n, (uint32_t)s * 1024u);
#pragma unroll
  for (int f = 0; f < 2; ++f)
    W.b[U][f] = __builtin_amdgcn_raw_buffer_load_b128(rw, P.w[f] + 256u * U, 0, 0);
  W.s[U] = __builtin_amdgcn_raw_buffer_load_b32(rsw, P.ws + 128u * U, 0, 0);
}

// quarter U's share of the copies of step s into stage memory cst
// (in a last K tile of 128 elements, chunks 4-7 of a row copy the next row's
// first codes: they meet W's zero padding, and E2M1 has no NaN or infinity,
// so their products are exactly zero)
template <int U>
__device__ __forceinline__ void mxw_copies(uint8_t* cst, int s, const MxwPlan& P) {
  const __amdgpu_buffer_rsrc_t ra = rsrc_from(P.a_base, P.a_n, (uint32_t)s * mxw::kRow);
#pragma unroll
  for (int i = 2 * U; i < 2 * U + 2; ++i) dma16(ra, cst + P.a_lds[i], P.a_g[i]);
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

// The quarter's 16 matrix instructions, the first N each followed by one
// global memory instruction and the first four by a quarter of its R LDS
// reads.  A 32 x 32 x 64 FP4 instruction keeps the matrix pipe busy for only
// 32 cycles, so the reads go out between matrix instructions rather than as
// a burst ahead of them (measured at M = N = K = 8192: 255-260 us against
// 265-267 us with the burst).
template <int N, int R = 8>
__device__ __forceinline__ void mxw_pin() {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < 4) __builtin_amdgcn_sched_group_barrier(0x100, R / 4, 0);
    if (i < N) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
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

  const TileOrigin to = tile_origin(g);   // XCD-aware tile walk
  const int m0 = to.m0;
  const int cg0 = to.cg0;

  MxwPlan P;
  P.rsa = make_rsrc(a_sc, g.asc_bytes);
  P.a_base = a;
  P.w_base = wp;
  P.wsc_base = w_sc;
  P.a_n = g.a_bytes;
  P.w_n = g.w_bytes;
  P.wsc_n = g.wsc_bytes;
  P.row_bytes = g.K / 2;
  P.sc_cols = g.K / 32;
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
  mx_copy_out(smem, c, g, m0, cg0 * 16);
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
//
// Counters at M = N = K = 8192: the matrix pipe 71% busy at 1.86 GHz.  Builds
// with the A copies, or the B loads, left out ran 17% and 10% faster, at 2.16
// and 2.05 GHz with the pipe as busy as before: under the power limit, moving
// operands into the CU costs clock.  The bytes per step are already the
// least a workgroup can move (256 x 256 is the largest output tile whose fp32
// accumulators fit the register file), and copying A through registers
// (global load, then LDS store) instead of the buffer-to-LDS path measured
// the same.
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
  __amdgpu_buffer_rsrc_t ra;
  const uint8_t* b_base;   // packed B and its size in bytes
  uint32_t b_n;
  int rd_a;             // LDS: A chunk 4 (l >> 5) of the lane's row (XOR 16 (2u + h))
  uint32_t b[2];        // B fragment f of step 0 (step s: + 2048 s; instruction u: + 256 u,
                        // half h: + 1024 h)
  uint32_t a_g[2];      // A copies i = 0, 1 of step 0; copy i: + (i >> 1) * a_step
  int a_kb[2];          // their chunk's byte within a step
  uint32_t a_step;
  int row_bytes;
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

// B fragment f of instruction U of step s (two 16-byte loads; a step past
// the last K tile reads the next column group's tiles, or zeros past the
// end, into registers that are never used)
template <int U, int F>
__device__ __forceinline__ void f8w_load_b(F8wB& B, int s, const F8wPlan& P) {
  const __amdgpu_buffer_rsrc_t rb = rsrc_from(P.b_base, P.b_n, (uint32_t)s * 2048u);
#pragma unroll
  for (int h = 0; h < 2; ++h)
    B.b[U][F][h] = __builtin_amdgcn_raw_buffer_load_b128(rb, P.b[F] + 256u * U + 1024u * h, 0, 0);
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

// The quarter's 8 matrix instructions, the first N each followed by one
// global memory instruction and the first four by two of its 8 LDS reads
// (spread out as in the MXFP4 kernel: 394-400 us against 413-415 us with the
// reads as a burst ahead of the quarter, M = N = K = 8192, same box).
template <int N>
__device__ __forceinline__ void f8w_pin() {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < 4) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    if (i < N) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
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

  const TileOrigin to = tile_origin(g);   // XCD-aware tile walk
  const int m0 = to.m0;
  const int cg0 = to.cg0;

  F8wPlan P;
  P.ra = make_rsrc(a, g.a_bytes);
  P.b_base = bp;
  P.b_n = g.w_bytes;
  P.row_bytes = g.K;
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
  mx_copy_out(smem, c, g, m0, cg0 * 16);
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

}  // namespace

hipError_t launch_mxfp4_256(const void* a, const void* a_e8m0, const void* w_packed, void* c,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return launch_mxw<2>(a, a_e8m0, w_packed, c, M, N, K, stream);
}

hipError_t launch_fp8_256(const void* a, const void* b_packed, const float* scale_a,
                          const float* scale_b, void* c, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream) {
  return launch_f8w(a, b_packed, scale_a, scale_b, c, M, N, K, stream);
}

}  // namespace qgemm
