// Small-M GEMM with in-register dequantization (W4A16 and W8A16 with per-column
// or group-wise scales, NVFP4 weights, FP8).
//
// The bandwidth-bound shape of the W4A16 page (section 1: every decode step
// streams the whole weight) and of the W8A16 page (Steps 1-2: load the low-bit
// tile, convert and scale on chip, feed the dot product; never write W_fp16
// back).  On gfx950 the multiply runs on the matrix cores
// (v_mfma_f32_16x16x32_f16 for the fp16 formats, the scaled f8f6f4 16x16x128
// instruction with unit scales for e4m3fn), with the M <= 16 rows of X in the
// A operand and a 16-column fragment tile of W in the B operand.
//
// Work split: a workgroup owns G column groups (16 columns each) and S
// 16-row slabs of X; its NW waves split the K tiles round-robin, so at any
// time the waves of a workgroup read neighbouring tiles.  Each wave keeps D K
// tiles of loads in flight in a register ring (above eight rows, unless one
// slab meets more than four column groups, the activation part of a tile
// goes to a wave-private LDS slot instead, copied with whole-row DMA reads)
// and its fp32 partial sums in registers; the workgroup reduces them through
// LDS in a fixed order (deterministic, no atomics, no workspace) and the
// epilogue applies the per-column scale (or the per-tensor FP8 / NVFP4
// scales) once to the fp32 sum before rounding to the output type; the
// grouped formats apply their scales in the dequant, before the matrix
// instruction.
//
// K order inside a 128-wide tile (fp16 formats): matrix step s (0..3) of lane
// group g = lane >> 4 covers k = 32 s + 8 g + [0, 8).  Both operands use the
// same order, so the product is unchanged, and the four lanes of one X row
// read 64 contiguous bytes per load.
//
// Dequantization without conversions: an fp16 with exponent field 25 and
// mantissa field m has value 1024 + m, so OR-ing a code into the mantissa of
// 0x6400 and subtracting a constant gives the exact small integer.  Two
// nibbles (or bytes) become two fp16 lanes of one register per operation.
#include "qgemm_common.h"
#include "qgemm_dequant.h"

#include <algorithm>

namespace qgemm {
namespace {

template <int FMT> struct DecodeTraits;
// W4A16: 16 B of W per lane per tile, 64 B of fp16 X per lane per tile.
template <> struct DecodeTraits<1> {
  static constexpr int WV = 1, XV = 4, TB = kTileBytesW4;
};
// W8A16: 32 B of W (two 1 KB halves), 64 B of fp16 X.
template <> struct DecodeTraits<2> {
  static constexpr int WV = 2, XV = 4, TB = kTileBytes;
};
// NVFP4 weights: 16 B of E2M1 codes per lane per tile, 64 B of fp16 X.
template <> struct DecodeTraits<7> {
  static constexpr int WV = 1, XV = 4, TB = kTileBytesW4;
};
// FP8: 32 B of W, 32 B of e4m3 A (lane holds k = 32 g + [0, 32)).
template <> struct DecodeTraits<4> {
  static constexpr int WV = 2, XV = 2, TB = kTileBytes;
};
// MXFP4: a 256-wide tile = two 128-element blocks h; per lane 16 B of W codes
// and 16 B of A codes per block (k = 128 h + 32 g + [0, 32)), plus one E8M0
// byte of each operand per block.
template <> struct DecodeTraits<3> {
  static constexpr int WV = 2, XV = 2, TB = kTileBytes;
};

// K elements per tile and activation bytes per row and tile.
template <int FMT> constexpr int tile_k() { return FMT == 3 ? kTileK4 : kTileK8; }
template <int FMT> constexpr int tile_x_bytes() { return FMT == 3 ? 128 : FMT == 4 ? 128 : 256; }

// NGT > 0: grouped formats, NGT metadata words {1024 + z (+128), s} per
// column and K tile (layout in qgemm_common.h).
// S: 16-row slabs of X per workgroup (each weight tile, loaded and
// dequantized once, multiplies the rows of all S slabs).
template <int FMT, int G, int NGT = 0, int S = 1>
struct Chunk {
  uintx4 x[S][DecodeTraits<FMT>::XV];
  uintx4 w[G][DecodeTraits<FMT>::WV];
  uint32_t meta[G][NGT > 0 ? NGT : (FMT == 3 ? 2 : 1)];   // MXFP4: W scale word per block
  uint32_t asc[FMT == 3 ? S : 1][2];                        // MXFP4: A scale byte per block
};

// Per-lane and per-workgroup addressing of one launch.  Scalar (wave-uniform)
// parts stay in SGPRs; each lane adds a 32-bit offset.  Activation and A
// scale offsets count from row m0, the workgroup's first row.
struct DecodeAddr {
  const uint8_t* x;       // activations, row m0
  uint32_t xrows;         // bytes of X from row m0 to its end
  uint32_t xlane[4];      // per slab: byte offset of this lane's row and first K piece
  const uint8_t* w;       // first weight tile of this workgroup
  int64_t cg_stride;      // bytes between column groups
  uint32_t wspan;         // record count of a tile's weight buffer: G groups' bytes, capped
                          // at 2^31 - 1 (above every offset a tile reads)
  int cg_last;            // last valid group index relative to this workgroup
  uint32_t wlane;         // 16 * lane
  int K;
  int g;                  // lane group, lane >> 4
  const uint8_t* meta;    // grouped / NVFP4: first metadata tile of this workgroup;
                          // MXFP4: the W scales of the 8-group band holding cg0
  const uint8_t* asc;     // MXFP4: A scales, E8M0 [M, K/32], row m0
  uint32_t arows;         // MXFP4: bytes of A scales from row m0 to their end
  uint32_t alane[4];      // MXFP4, per slab: this lane's row and block g in asc
  int cg0, KT;            // MXFP4: first column group, K tiles
  uint32_t wsh[8];        // MXFP4, per group: bit shift of its tile's scale byte
  int64_t meta_cg_stride; // bytes between column groups of metadata
  int meta_kt_stride;     // bytes of metadata per K tile
  uint32_t mlane;         // this lane's entries within a tile
  uint32_t mspan;         // the same for a tile's metadata buffer
  // activations staged through LDS: per (slab, copy instruction) the byte
  // offset of this lane's 16 B from a tile's first byte in row m0, and per
  // operand piece this lane's byte offset within a staged slab
  uint32_t xdma[8];
  uint32_t xrd[4];
};

// A raw buffer of `bytes` bytes at p.  Reads at or past `bytes` return zero
// without touching memory; with bytes = 0 every read does.  The prologue
// fills a ring slot whose K tile lies past the end through such an empty
// buffer instead of skipping its loads under a branch: where the paths of a
// branch around loads merge, the compiler waits for every load in flight.
// `bytes` is wave-uniform and is chosen between run-time values (a choice
// between constants such as ~0 and 0 is compiled into a vector register, and
// each load then loops over its distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dec_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr int kStreamLoad = 2;               // cache policy of the weight stream: nt

typedef __attribute__((address_space(3))) void lds_void_t;
constexpr uint32_t kXOutOfRange = 0x80000000u;   // past any staged tile's activation buffer

// Activation tiles staged through LDS.  A staged slab is the 16 rows x RB
// bytes (RB = tile_x_bytes: 256 for fp16 X, 128 for e4m3 / E2M1 codes) of
// one K tile, row-major, with 16-byte chunk c of row r stored at chunk
// position c ^ swz(r).  The copy reads RB contiguous bytes per row (whole
// cache lines: 4 rows x 256 B or 8 rows x 128 B per instruction), which the
// vector memory path serves about three times faster than the 16 rows x 64 B
// that the matrix-operand layout would read directly; the swizzle makes the
// operand reads (16 rows, one chunk column each) hit 16 distinct 16-byte bank
// groups.
template <int FMT> __device__ __forceinline__ int x_swz(int r) {
  return tile_x_bytes<FMT>() == 256 ? r : (r >> 1) & 7;
}
template <int FMT> constexpr int x_copy_instrs() { return tile_x_bytes<FMT>() == 256 ? 4 : 2; }

// K index of the first element of X piece p of lane group g in tile kt.
template <int FMT>
__device__ __forceinline__ int piece_k(int kt, int g, int p) {
  if constexpr (FMT == 4) return kt * kTileK8 + 32 * g + 16 * p;   // e4m3: contiguous 32
  else if constexpr (FMT == 3) return kt * kTileK4 + 128 * p + 32 * g;   // FP4: block p
  else return kt * kTileK8 + 32 * p + 8 * g;                        // fp16: step p
}

// Load lane data of K tile `kt`: the lane's X (or A) pieces and each of the G
// weight tiles; with live = false (a tile past the end) the same loads read
// nothing.  X pieces past K read as zero when staged (and in the last rows
// of X); loaded into registers they may hold the next row's values and are
// cleared before that tile's compute (cut_chunk).  Rows past M load row M-1
// instead (their outputs are never stored); groups past the last column load
// the last group (likewise discarded).
template <int FMT, int G, bool X_ELEMENTWISE, int NGT = 0, int S = 1, bool XL = false>
__device__ __forceinline__ void load_chunk(Chunk<FMT, G, NGT, S>& ch, const DecodeAddr& ad,
                                           int kt, bool live, uint8_t* xs = nullptr) {
  constexpr int TB = DecodeTraits<FMT>::TB;
  constexpr int RB = tile_x_bytes<FMT>();
  constexpr int PSTRIDE = (FMT == 4) ? 16 : 64;    // bytes between a lane's pieces
  // the slots' loads are issued in ring order (the wait before a slot's
  // compute then counts only the later slots' loads)
  __builtin_amdgcn_sched_barrier(0);
  // this tile's activations: from column kt * RB of row m0 to the end of X,
  // at most 2^31 - 1 bytes (the host keeps every offset below that)
  const __amdgpu_buffer_rsrc_t xr = dec_rsrc(
      ad.x + (int64_t)kt * RB, live ? min(ad.xrows - (uint32_t)kt * RB, 0x7fffffffu) : 0u);
  if constexpr (XL) {
    // copy the S staged slabs of tile kt into this wave's LDS slot `xs`; in
    // a partial last tile, chunks past K take an offset past the buffer and
    // land as zeros (K % 8 == 0 for fp16, % 16 for e4m3, % 32 for E2M1: a
    // chunk is wholly in or out).  Issued before the weight loads of the
    // chunk, with nothing scheduled across: the weight loads complete after
    // them.
    constexpr int NI = x_copy_instrs<FMT>();
    constexpr int LPR = RB / 16;                  // lanes per row
    constexpr int KPC = tile_k<FMT>() / LPR;      // K elements per chunk
    const bool full = (kt + 1) * tile_k<FMT>() <= ad.K;   // uniform
    const int lane = __lane_id();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        uint32_t off = ad.xdma[q * NI + i];
        if (!full) {
          const int r = i * (64 / LPR) + lane / LPR;
          const int c = (lane % LPR) ^ x_swz<FMT>(r);
          if (kt * tile_k<FMT>() + c * KPC >= ad.K) off = kXOutOfRange;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t*)(xs + q * 16 * RB + i * 1024),
                                                 16, off, 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
  } else if constexpr (!X_ELEMENTWISE) {
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int p = 0; p < DecodeTraits<FMT>::XV; ++p)
        ch.x[q][p] = __builtin_amdgcn_raw_buffer_load_b128(xr, ad.xlane[q] + PSTRIDE * p, 0, 0);
  } else {
    // K % 8 != 0 (fp16 only): rows are not 16-byte aligned; go element-wise
    // (K and the tile decide each element; a tile past the end loads none)
    static_assert(S == 1 && FMT != 3 && FMT != 4, "the element-wise path: fp16 X, one slab");
    const uint16_t* xr16 =
        reinterpret_cast<const uint16_t*>(ad.x + (int64_t)kt * RB + ad.xlane[0]);
#pragma unroll
    for (int p = 0; p < DecodeTraits<FMT>::XV; ++p) {
      uint32_t d[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = piece_k<FMT>(kt, ad.g, p) + 2 * j;
        const int e = (PSTRIDE / 2) * p + 2 * j;
        const uint32_t lo = (k < ad.K) ? xr16[e] : 0u;
        const uint32_t hi = (k + 1 < ad.K) ? xr16[e + 1] : 0u;
        d[j] = lo | (hi << 16);
      }
      ch.x[0][p] = uintx4{d[0], d[1], d[2], d[3]};
    }
  }
  if constexpr (FMT == 3) {
    // the E8M0 byte of block 8 kt + 4 h + g of each slab row (blocks past K
    // are replaced at use)
    const __amdgpu_buffer_rsrc_t ar =
        dec_rsrc(ad.asc + 8 * (int64_t)kt, live ? ad.arows - 8u * (uint32_t)kt : 0u);
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ch.asc[q][h] = __builtin_amdgcn_raw_buffer_load_b8(ar, ad.alane[q] + 4 * h, 0, 0);
  }
  const __amdgpu_buffer_rsrc_t wr = dec_rsrc(ad.w + (int64_t)kt * TB, live ? ad.wspan : 0u);
  // grouped / NVFP4: this tile's metadata; MXFP4: the W scales of blocks
  // 8 kt .. 8 kt + 7 (512 B per 8 column groups and 128-element block,
  // [lane][group], 2 KT blocks per band of 8 groups)
  const __amdgpu_buffer_rsrc_t mr =
      dec_rsrc(ad.meta + (int64_t)kt * (FMT == 3 ? 1024 : ad.meta_kt_stride),
               live ? ad.mspan : 0u);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int gg = g < ad.cg_last ? g : ad.cg_last;                // uniform
    const uint32_t wo = (uint32_t)(gg * ad.cg_stride);             // uniform
    ch.w[g][0] = __builtin_amdgcn_raw_buffer_load_b128(wr, ad.wlane, wo, kStreamLoad);
    if constexpr (DecodeTraits<FMT>::WV == 2)
      ch.w[g][1] = __builtin_amdgcn_raw_buffer_load_b128(wr, ad.wlane + 1024, wo, kStreamLoad);
    if constexpr (FMT == 3) {
      const int cg = ad.cg0 + gg;
      const int band = (cg >> 3) - (ad.cg0 >> 3);                  // 0 or 1
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t mo = (uint32_t)(band * 1024 * ad.KT + 512 * h + 4 * ((cg >> 2) & 1));
        ch.meta[g][h] = __builtin_amdgcn_raw_buffer_load_b32(mr, ad.wlane / 2, mo, 0);
      }
    }
    if constexpr (NGT > 0) {
      const uint32_t mo = (uint32_t)(gg * ad.meta_cg_stride);
      if constexpr (FMT == 7) {
        ch.meta[g][0] = __builtin_amdgcn_raw_buffer_load_b32(mr, ad.mlane, mo, 0);   // 4 block scales
      } else if constexpr (NGT == 4) {
        const uintx4 v = __builtin_amdgcn_raw_buffer_load_b128(mr, ad.mlane, mo, 0);
        ch.meta[g][0] = v[0]; ch.meta[g][1] = v[1]; ch.meta[g][2] = v[2]; ch.meta[g][3] = v[3];
      } else if constexpr (NGT == 2) {
        const uintx2 v = __builtin_amdgcn_raw_buffer_load_b64(mr, ad.mlane, mo, 0);
        ch.meta[g][0] = v[0]; ch.meta[g][1] = v[1];
      } else {
        ch.meta[g][0] = __builtin_amdgcn_raw_buffer_load_b32(mr, ad.mlane, mo, 0);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Operand piece p of slab q: from the chunk's registers or, staged, from the
// LDS slot.
template <int FMT, int G, int NGT, int S, bool XL>
__device__ __forceinline__ uintx4 x_piece(const Chunk<FMT, G, NGT, S>& ch, const DecodeAddr& ad,
                                          const uint8_t* xs, int q, int p) {
  if constexpr (XL)
    return *reinterpret_cast<const uintx4*>(xs + q * 16 * tile_x_bytes<FMT>() + ad.xrd[p]);
  else
    return ch.x[q][p];
}

// Tile kt reaches past K (the last tile, when K is not a multiple of the
// tile): clear the X pieces past K that were loaded into registers (they
// hold the next row's values) and give MXFP4 blocks past K the unit A scale
// (their codes are zero; the bytes after a row's last block belong to the
// next row).  Staged pieces past K arrived as zeros.
template <int FMT, int G, int NGT, int S, bool XL>
__device__ __forceinline__ void cut_chunk(Chunk<FMT, G, NGT, S>& ch, const DecodeAddr& ad,
                                          int kt) {
  if constexpr (!XL) {
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int p = 0; p < DecodeTraits<FMT>::XV; ++p)
        if (piece_k<FMT>(kt, ad.g, p) >= ad.K) ch.x[q][p] = uintx4{0, 0, 0, 0};
  }
  if constexpr (FMT == 3) {
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (8 * kt + 4 * h + ad.g >= ad.K / 32) ch.asc[q][h] = kE8M0One;
  }
}

template <int FMT, int G, int NGT = 0, int S = 1, bool XL = false>
__device__ __forceinline__ void compute_chunk(const Chunk<FMT, G, NGT, S>& ch,
                                              floatx4 (&acc)[S][G], W4Masks mk,
                                              const DecodeAddr& ad, const uint8_t* xs = nullptr) {
  if constexpr (XL) {
    // the staged copies of this tile were issued before its weight loads and
    // loads complete in order: once the first weight register has landed, so
    // has the slot.  The empty asm makes the compiler wait for that register
    // here and keeps the LDS reads after the wait.
    asm volatile("" ::"v"(ch.w[0][0][0]) : "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (FMT == 3) {
    // two scaled FP4 instructions per group (blocks h = 0, 1); the lane's
    // scale bytes sit in the low byte (A) and at byte (cg & 3) of the loaded
    // word (W)
    uintx4 xv[S][2];
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) xv[q][h] = x_piece<FMT, G, NGT, S, XL>(ch, ad, xs, q, h);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uintx4& wb = ch.w[g][h];
        const intx8 b = {(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3], 0, 0, 0, 0};
        const int sb = (int)(ch.meta[g][h] >> ad.wsh[g]);
#pragma unroll
        for (int q = 0; q < S; ++q) {
          const uintx4& xa = xv[q][h];
          const intx8 a = {(int)xa[0], (int)xa[1], (int)xa[2], (int)xa[3], 0, 0, 0, 0};
          acc[q][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a, b, acc[q][g], kFmtFP4, kFmtFP4, 0, (int)ch.asc[q][h], 0, sb);
        }
      }
  } else if constexpr (FMT == 4) {
    uintx4 xv[S][2];
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int p = 0; p < 2; ++p) xv[q][p] = x_piece<FMT, G, NGT, S, XL>(ch, ad, xs, q, p);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const intx8 b = {(int)ch.w[g][0][0], (int)ch.w[g][0][1], (int)ch.w[g][0][2],
                       (int)ch.w[g][0][3], (int)ch.w[g][1][0], (int)ch.w[g][1][1],
                       (int)ch.w[g][1][2], (int)ch.w[g][1][3]};
#pragma unroll
      for (int q = 0; q < S; ++q) {
        const uintx4& x0 = xv[q][0];
        const uintx4& x1 = xv[q][1];
        const intx8 a = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                         (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        acc[q][g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a, b, acc[q][g], kFmtFP8, kFmtFP8, 0, kE8M0One, 0, kE8M0One);
      }
    }
  } else {
    // grouped INT4 / INT8 with group 128 or 64 (one or two groups per column
    // and tile): the matrix steps of a group accumulate (w - z) unscaled
    // (exact in fp16) into a group sum, and one fp32 fma per accumulator
    // applies the group's scale; each dequantized weight then costs no
    // multiply.  (w - z) * s is exact in fp32, so a single weight still
    // reaches the output as (w - z) * s rounded once.  (Group 128 with one
    // slab or staged activations, group 64 with one slab: otherwise the
    // group sums would not fit beside the ring.)
    constexpr bool TILE_SCALE =
        (FMT == 1 || FMT == 2) && ((NGT == 1 && (S == 1 || XL)) || (NGT == 2 && S == 1));
    constexpr int SPG = NGT == 2 ? 2 : 4;   // matrix steps per scale group
    floatx4 tile[TILE_SCALE ? S : 1][TILE_SCALE ? G : 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      half8_t xv[S];
#pragma unroll
      for (int q = 0; q < S; ++q)
        xv[q] = __builtin_bit_cast(half8_t, (x_piece<FMT, G, NGT, S, XL>(ch, ad, xs, q, s)));
#pragma unroll
      for (int g = 0; g < G; ++g) {
        half8_t b;
        if constexpr (FMT == 7) {
          b = dequant_nvfp4(ch.w[g][0][s], ch.meta[g][0] >> (8 * s));
        } else if constexpr (TILE_SCALE) {
          const uint32_t e = ch.meta[g][(s * NGT) >> 2];
          if constexpr (FMT == 1) {
            b = dequant_w4_group_unscaled(ch.w[g][0][s], e, mk);
          } else {
            const uintx4& h = ch.w[g][s >> 1];
            b = dequant_w8_group_unscaled(h[2 * (s & 1)], h[2 * (s & 1) + 1], e);
          }
        } else if constexpr (NGT > 0) {
          // (w - z) * s rounded once to fp16, z and s of this step's group
          const uint32_t e = ch.meta[g][(s * NGT) >> 2];
          if constexpr (FMT == 1) {
            b = dequant_w4_group(ch.w[g][0][s], e);
          } else {
            const uintx4& h = ch.w[g][s >> 1];
            b = dequant_w8_group(h[2 * (s & 1)], h[2 * (s & 1) + 1], e);
          }
        } else if constexpr (FMT == 1) {
          b = dequant_w4(ch.w[g][0][s], mk);
        } else {
          const uintx4& h = ch.w[g][s >> 1];
          b = dequant_w8(h[2 * (s & 1)], h[2 * (s & 1) + 1]);
        }
#pragma unroll
        for (int q = 0; q < S; ++q) {
          if constexpr (TILE_SCALE)
            tile[q][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                xv[q], b, s % SPG == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : tile[q][g], 0, 0, 0);
          else
            acc[q][g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv[q], b, acc[q][g], 0, 0, 0);
        }
      }
      if constexpr (TILE_SCALE) {
        if (s % SPG == SPG - 1) {
          // the lane's accumulator column is its B-operand column (lane & 15),
          // whose word holds the group's scale in its high half
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const uint32_t e = ch.meta[g][(s * NGT) >> 2];
            const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16));
            const floatx4 sv = {sc, sc, sc, sc};
#pragma unroll
            for (int q = 0; q < S; ++q)
              acc[q][g] = __builtin_elementwise_fma(tile[q][g], sv, acc[q][g]);
          }
        }
      }
    }
  }
}

// Workgroup -> (column block, row block).  Workgroups are handed to the eight
// XCDs round-robin by linear index, and each XCD has its own L2.  With one
// row block the linear index is the column block.  With R > 1 row blocks,
// the R row blocks of one column block take R consecutive slots of one XCD
// (slot = index / 8, XCD = index % 8), so they start together and read the
// same weight tiles through the same L2: the weight streams from HBM about
// once instead of R times.  The column blocks are padded to a multiple of 8;
// workgroups of the padding exit at once.
struct DecodeBlock {
  int cb, rb;
  bool valid;
};
__device__ __forceinline__ DecodeBlock decode_block(int b, int CG, int G, int M, int rows) {
  const int nrb = (M + rows - 1) / rows;
  if (nrb <= 1) return DecodeBlock{b, 0, true};
  const int slot = b >> 3;
  const int cb = (slot / nrb) * 8 + (b & 7);
  return DecodeBlock{cb, slot % nrb, cb * G < CG};
}

// Grid of the small-M kernel: see decode_block.
inline unsigned decode_grid(int64_t CG, int G, int64_t M, int rows) {
  const int64_t ncb = cdiv(CG, G), nrb = cdiv(M, rows);
  return (unsigned)(nrb <= 1 ? ncb : cdiv(ncb, 8) * 8 * nrb);
}

// NGT > 0: grouped W4A16 / W8A16 (scales and zero points in the metadata
// segment at wp + meta_offset; `scales` unused).
// S: 16-row slabs per workgroup (rows m0 .. m0 + 16 S - 1).
// XL: activation tiles staged through LDS (each wave owns D slots of S
// staged slabs); the host guarantees that X spans fewer than 2^31 bytes.
template <int FMT, int G, int NW, int D, bool X_ELEMENTWISE, int NGT = 0, int S = 1,
          bool XL = false>
__global__ __launch_bounds__(NW * kWave) void decode_gemm_kernel(
    const uint8_t* __restrict__ x, const uint8_t* __restrict__ wp,
    const _Float16* __restrict__ scales, const float* __restrict__ scale_a,
    const float* __restrict__ scale_b, uint16_t* __restrict__ y, int M, int N, int K, int KT,
    int CG, int64_t meta_offset) {
  static_assert(NW >= 2, "the K split needs at least two waves");
  static_assert(D >= 2 && D <= 4, "prefetch depth 2..4");
  static_assert(S == 1 || S == 2 || S == 4, "1, 2 or 4 slabs");
  static_assert(!XL || (!X_ELEMENTWISE && S * x_copy_instrs<FMT>() <= 8),
                "staged activations: aligned rows, at most 8 copy instructions per tile");
  constexpr int TB = DecodeTraits<FMT>::TB;
  constexpr int RB = tile_x_bytes<FMT>();
  constexpr int XSLOT = S * 16 * RB;             // one staged tile (S slabs)
  constexpr int XWAVE = D * XSLOT;               // one wave's ring of slots
  constexpr int RED_BYTES = NW * G * kWave * 16;
  constexpr int SMEM = XL && NW * XWAVE > RED_BYTES ? NW * XWAVE : RED_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  floatx4 (*red)[G][kWave] = reinterpret_cast<floatx4 (*)[G][kWave]>(smem);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const DecodeBlock blk = decode_block(blockIdx.x, CG, G, M, 16 * S);
  if (!blk.valid) return;   // padding of the column blocks (whole workgroup)
  const int cg0 = blk.cb * G;
  const int m0 = blk.rb * 16 * S;

  DecodeAddr ad;
  ad.g = lane >> 4;
  // X from row m0 (rows past M load row M - 1: their outputs are never stored)
  const int64_t rowbytes = FMT == 3 ? K / 2 : FMT == 4 ? (int64_t)K : 2 * (int64_t)K;
  ad.x = x + (int64_t)m0 * rowbytes;
  ad.xrows = (uint32_t)((int64_t)(M - m0) * rowbytes);
#pragma unroll
  for (int q = 0; q < S; ++q) {
    const int r = min(m0 + 16 * q + (lane & 15), M - 1) - m0;
    if constexpr (FMT == 3) {   // 16 B of codes at k = 32 g of a block
      ad.xlane[q] = (uint32_t)((int64_t)r * rowbytes + 16 * ad.g);
      ad.alane[q] = (uint32_t)((int64_t)r * (K / 32) + ad.g);
    } else {
      const int xb = FMT == 4 ? 1 : 2;
      ad.xlane[q] = (uint32_t)((int64_t)r * rowbytes + (FMT == 4 ? 32 : 8) * ad.g * xb);
    }
  }
  if constexpr (FMT == 3) {
    // `scales` carries the A E8M0 bytes; meta_offset locates the W scales
    ad.asc = reinterpret_cast<const uint8_t*>(scales) + (int64_t)m0 * (K / 32);
    ad.arows = (uint32_t)((int64_t)(M - m0) * (K / 32));
    ad.cg0 = cg0;
    ad.KT = KT;
#pragma unroll
    for (int g = 0; g < G && g < 8; ++g) {
      const int cg = cg0 + min(g, CG - 1 - cg0);
      ad.wsh[g] = 8u * (uint32_t)(cg & 3);
    }
  }
  ad.cg_stride = (int64_t)KT * TB;
  ad.w = wp + (int64_t)cg0 * ad.cg_stride;
  ad.cg_last = CG - 1 - cg0;
  ad.wlane = 16u * lane;
  ad.K = K;
  // grouped: NGT words per column and tile; NVFP4: 8 scale bytes per column
  // and tile, the lanes of group g reading the dword of blocks 2s + (g >> 1);
  // MXFP4: the band of 8 column groups holding cg0 (2 KT blocks of 512 B)
  ad.meta_kt_stride = FMT == 7 ? kScaleTileBytes : 16 * (NGT > 0 ? NGT : 1) * 4;
  ad.meta_cg_stride = (int64_t)KT * ad.meta_kt_stride;
  ad.meta = FMT == 3 ? wp + meta_offset + (int64_t)(cg0 >> 3) * 1024 * KT
                     : wp + meta_offset + (int64_t)cg0 * ad.meta_cg_stride;
  ad.mlane = FMT == 7 ? (uint32_t)((lane & 15) * 8 + 4 * (ad.g >> 1))
                      : (uint32_t)((lane & 15) * (NGT > 0 ? NGT : 1) * 4);
  constexpr int64_t kSpanCap = 0x7fffffff;
  ad.wspan = (uint32_t)min((int64_t)G * ad.cg_stride, kSpanCap);
  ad.mspan = (uint32_t)min(FMT == 3 ? 2048 * (int64_t)KT : (int64_t)G * ad.meta_cg_stride,
                           kSpanCap);
  if constexpr (XL) {
    constexpr int NI = x_copy_instrs<FMT>();
    constexpr int LPR = RB / 16;
    // copy instruction i of slab q: row i * (64 / LPR) + lane / LPR of the
    // slab, chunk (lane % LPR) ^ swz(row); rows past M copy row M - 1
#pragma unroll
    for (int q = 0; q < S; ++q)
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = i * (64 / LPR) + lane / LPR;
        const int row = min(m0 + 16 * q + r, M - 1) - m0;
        const int c = (lane % LPR) ^ x_swz<FMT>(r);
        ad.xdma[q * NI + i] = (uint32_t)(row * rowbytes + 16 * c);
      }
    // operand piece p of lane (row r = lane & 15, group g): chunk 4 p + g
    // (fp16 step p; E2M1 block p) or 2 g + p (e4m3 half p)
    const int r = lane & 15;
#pragma unroll
    for (int p = 0; p < DecodeTraits<FMT>::XV; ++p) {
      const int c = FMT == 4 ? 2 * ad.g + p : 4 * p + ad.g;
      ad.xrd[p] = (uint32_t)(r * RB + 16 * (c ^ x_swz<FMT>(r)));
    }
  }

  W4Masks mk{};
  if constexpr (FMT == 1) mk = W4Masks{vgpr_const(0x000f000fu), vgpr_const(0x00f000f0u)};

  floatx4 acc[S][G];
#pragma unroll
  for (int q = 0; q < S; ++q)
#pragma unroll
    for (int g = 0; g < G; ++g) acc[q][g] = floatx4{0.f, 0.f, 0.f, 0.f};

  // K tiles wave, wave + NW, ...; a ring of D register buffers keeps D tiles
  // of loads in flight per wave.  The prologue fills every slot (a slot past
  // the end through an empty buffer); the steady loop runs while every
  // compute and every reload of its round is a real tile, with no branch
  // around a load, so each compute waits only for its own slot; the last
  // 2 D - 1 tiles at most take the guarded loop (which holds the last tile,
  // the only one K can cut: X pieces loaded into registers and MXFP4 scales
  // past K are replaced there).
  constexpr bool CUTS = (!XL && !X_ELEMENTWISE) || FMT == 3;
  Chunk<FMT, G, NGT, S> ring[D];
  uint8_t* const xw = smem + wave * XWAVE;   // this wave's staging slots (XL)
#pragma unroll
  for (int d = 0; d < D; ++d)
    load_chunk<FMT, G, X_ELEMENTWISE, NGT, S, XL>(ring[d], ad, wave + d * NW, wave + d * NW < KT,
                                                  xw + d * XSLOT);
  int base = wave;
  for (; base + (2 * D - 1) * NW < KT; base += D * NW) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute_chunk<FMT, G, NGT, S, XL>(ring[d], acc, mk, ad, xw + d * XSLOT);
      load_chunk<FMT, G, X_ELEMENTWISE, NGT, S, XL>(ring[d], ad, base + (d + D) * NW, true,
                                                    xw + d * XSLOT);
    }
  }
  for (; base < KT; base += D * NW) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int kt = base + d * NW;
      if (kt < KT) {
        if (CUTS && (kt + 1) * tile_k<FMT>() > K) cut_chunk<FMT, G, NGT, S, XL>(ring[d], ad, kt);
        compute_chunk<FMT, G, NGT, S, XL>(ring[d], acc, mk, ad, xw + d * XSLOT);
        if (kt + D * NW < KT)
          load_chunk<FMT, G, X_ELEMENTWISE, NGT, S, XL>(ring[d], ad, kt + D * NW, true,
                                                        xw + d * XSLOT);
      }
    }
  }
  // the partial-sum buffer reuses the staging slots of every wave: the
  // empty copies of the slots past the end must have landed as well
  if constexpr (XL) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // ---- reduce the NW partial tiles in a fixed order, one slab at a time
  const float fp8_scale = (FMT == 4) ? (*scale_a) * (*scale_b) : (FMT == 7) ? *scale_a : 1.0f;
  const float* redf = reinterpret_cast<const float*>(smem);
  constexpr int OUT = 16 * 16 * G;
#pragma unroll
  for (int q = 0; q < S; ++q) {
    if (q > 0) __syncthreads();   // every thread has read the previous slab's partials
#pragma unroll
    for (int g = 0; g < G; ++g) red[wave][g][lane] = acc[q][g];
    __syncthreads();
    // consecutive threads take consecutive columns of one row (coalesced
    // store); the 16x16 accumulator of a wave holds row 4*(lane>>4)+i,
    // column lane&15
    for (int o = threadIdx.x; o < OUT; o += NW * kWave) {
      const int m = o / (16 * G);
      const int nl = o - m * (16 * G);
      const int g = nl >> 4;
      const int c = nl & 15;
      const int src_lane = 16 * (m >> 2) + c;
      const int i = m & 3;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += redf[((w * G + g) * kWave + src_lane) * 4 + i];
      const int gm = m0 + 16 * q + m;
      const int gn = (cg0 + g) * 16 + c;
      if (gm < M && gn < N) {
        if constexpr (FMT == 3) {
          y[(int64_t)gm * N + gn] = f32_to_bf16_rne(sum);   // scales applied in the MFMA
        } else if constexpr (FMT == 4) {
          y[(int64_t)gm * N + gn] = f32_to_bf16_rne(sum * fp8_scale);
        } else if constexpr (FMT == 7) {
          y[(int64_t)gm * N + gn] = f32_to_f16_bits(sum * fp8_scale);   // per-tensor scale
        } else if constexpr (NGT > 0) {
          y[(int64_t)gm * N + gn] = f32_to_f16_bits(sum);   // scales already applied
        } else {
          y[(int64_t)gm * N + gn] = f32_to_f16_bits((float)scales[gn] * sum);
        }
      }
    }
  }
}

struct DecodeConfig {
  int g;   // column groups (of 16) per workgroup
  int nw;  // waves per workgroup (K split)
  int d;   // K tiles in flight per wave
  int s;   // 16-row slabs per workgroup
  bool xl; // activation tiles staged through LDS
};

// Whether a launch may stage its activation tiles through LDS: with more
// than eight rows, eight waves (or four with at least 16 K tiles: the
// launches with several row blocks), and at most 8 copy instructions per
// tile (fp16 X: up to two slabs); X must span fewer than 2^31 bytes (32-bit
// buffer offsets).  With one slab the callers stage only up to four column
// groups.  Measured on MI355X, each shape timed staged and direct in
// alternation: one slab, one or two groups, staging wins (W4A16 K = N = 4096,
// M = 12 / 16: 5.0 / 5.3 us against 5.9 / 6.4 direct; W4A16, NVFP4 and
// grouped W4A16 with two groups, K = N = 8192, M = 16: 10.0 / 10.8 / 11.3
// against 11.5 / 12.5 / 12.8); FP8 and INT8 with two to four groups run
// within 3 % either way; with more than four groups the weight loads
// outnumber the activation loads and direct loads win (W4A16 N = 28672,
// seven groups: K = 8192, M = 9 / 12 / 16 21.3 / 21.2 / 22.0 against
// 22.1 / 22.5 / 22.5; K = 4096, M = 12 / 16 13.0 / 13.3 against 14.3 / 14.3;
// eight groups, N = 32768, M = 12 / 16 28.0 / 28.0 against 29.3 / 28.4).
// From two slabs on staging saved 8 % (INT4) to 11 % (grouped INT8) at
// M = 32 and up to 21 % at M = 64 .. 128 (FP8) with an earlier form of the
// main loop.
bool use_x_lds(int fmt, int64_t M, int nw, int s, int64_t KT) {
  const int rb = fmt == 3 || fmt == 4 ? 128 : 256;
  const int ni = rb == 256 ? 4 : 2;
  return M > 8 && (nw == 8 || (nw == 4 && KT >= 16)) && s * ni <= 8 &&
         M * KT * rb < ((int64_t)1 << 31);
}

// Waves per workgroup: eight, or four when K has fewer than 16 tiles.  A
// launch with several row blocks (above 16 S rows) also takes four: its
// staging slots then need 64 KB of LDS instead of 128, so two workgroups
// share a CU and one's start (the first weight tiles arriving from HBM) and
// end (the reduction and stores) overlap the other's K loop.  Measured on
// MI355X at M = 64 / 96 / 128: W8A16 K = 4096, N = 11008 21.6 / 29.4 / 36.4
// us with eight waves, 19.9 / 26.7 / 32.6 with four; at M = 128: grouped
// W8A16 (group 128, same shape) 39.8 -> 34.0, grouped W4A16 (group 128,
// K = 8192, N = 28672) 115 -> 109, MXFP4 K = N = 8192 29.8 -> 27.3, FP8
// 30.5 -> 29.1, W4A16 K = 8192, N = 28672 89.5 -> 88.0.  Two waves (four
// workgroups per CU) ran M = 64 slower (W4A16 71 us against 50).
int decode_waves(int64_t M, int s, int64_t KT) {
  return KT < 16 || (s > 1 && M > 16 * s) ? 4 : 8;
}

// Launch shape with one row block: about one workgroup per CU.  Measured on
// MI355X at the decode workloads (W8A16 K=4096 N=11008, W4A16 K=8192
// N=28672, FP8 K=N=8192, M = 1 .. 16): the weight streams fastest when the
// grid has close to 256 workgroups, each owning G = ceil(column groups / 256)
// column groups; more, smaller workgroups leave the CUs unevenly loaded and
// fewer leave CUs idle.
// G is capped by the register budget (8 for INT4, 4 for the byte formats);
// every format keeps two K tiles in flight per wave (INT8 at M <= 16 with
// three: 9.7 / 9.8 / 10.9 us at M = 1 / 4 / 16, K = 4096, N = 11008, against
// 9.4 / 9.5 / 10.6 with two); short K uses four waves.  Above 16 rows a workgroup takes 2 (M <= 32) or 4 slabs, so each
// weight tile is streamed and dequantized once for up to 64 rows instead of
// once per 16; the activations of all slabs then share the register ring,
// which caps G and the ring at two tiles.  The fp16-activation formats keep
// 2 slabs at every M, staged through LDS (four would need 16 copy
// instructions and 256 KB of slots, so they would load X directly): INT4
// with 4 slabs could keep only 3 groups and its grid grew to 2.3 workgroups
// per CU (K = 8192, N = 28672, M = 64: 106 us against 68 us); INT8 at
// K = 4096, N = 11008 ran M = 64 / 96 / 128 in 24.2 / 43.8 / 44.0 us with
// 4 direct slabs and 21.6 / 29.5 / 36.3 us with 2 staged ones.  The extra
// row blocks cost little HBM traffic: decode_block puts the row blocks of
// one column block on one XCD.
DecodeConfig pick_decode_config(int fmt, int64_t M, int64_t CG, int64_t KT) {
  const int s = M <= 16 ? 1 : (M <= 32 || fmt == 1 || fmt == 2) ? 2 : 4;
  // MXFP4 carries its scale words in the ring too: 2 groups with 4 slabs
  const int64_t gmax = s == 1 ? (fmt == 1 ? 8 : 4) : s == 2 ? (fmt == 1 ? 7 : 4) : fmt == 3 ? 2 : 3;
  int64_t g = cdiv(CG, 256);
  g = g < 1 ? 1 : (g > gmax ? gmax : g);
  DecodeConfig c{(int)g, decode_waves(M, s, KT), 2, s, false};
  c.xl = use_x_lds(fmt, M, c.nw, c.s, KT) && (c.s > 1 || c.g <= 4);
  // e4m3 activations, one slab, at least 16 K tiles and two column groups:
  // four waves loading A directly, each with twice the tiles (most of them
  // in the steady loop).  Measured on MI355X against eight staged waves,
  // K = 8192: N = 8192 M = 1 / 8 / 16 11.9 / 12.1 / 12.2 us against 12.1 /
  // 12.5 / 12.6; N = 16384 M = 1 / 16 23.5 / 23.8 against 25.4 / 25.4; with
  // one group (K = N = 4096, M = 16) 5.35 against 5.15, and the other
  // formats ran as fast or faster with eight.
  if (fmt == 4 && s == 1 && KT >= 16 && g >= 2) {
    c.nw = 4;
    c.xl = false;
  }
  // e4m3 activations with up to eight rows: one column group per workgroup
  // (two to seven workgroups per CU; the activation bytes each re-reads are
  // few).  Measured on MI355X against the rule above, M = 1 / 8: K = 8192,
  // N = 8192 11.6 / 11.6 us against 12.0 / 12.1, N = 16384 21.0 / 21.1
  // against 23.4 / 23.6, N = 28672 36.7 / 38.1 against 39.2 / 38.3; K = 4096,
  // N = 8192 6.8 / 7.1 against 7.2 / 7.4.  At 16 rows it lost (N = 8192:
  // 13.4 against 12.2).
  if (fmt == 4 && M <= 8) {
    c.g = 1;
    c.nw = decode_waves(M, s, KT);
    c.xl = false;
  }
  // E2M1 activations, one slab, at least 16 K tiles, and more than 256
  // workgroups of the largest G: four waves loading A directly, so that two
  // workgroups share a CU and one's start and end overlap the other's K loop.
  // Measured on MI355X against eight staged waves, M = 1 / 16: K = 8192,
  // N = 20480 19.9 / 22.3 us against 20.6 / 23.0, N = 28672 22.2 / 23.4
  // against 23.2 / 24.8; K = 4096, N = 28672 13.0 / 13.5 against 13.8 / 15.5.
  // With at most 256 workgroups it ran as fast (N = 12288, 16384) or slower
  // (N = 8192: 9.1 / 9.6 against 8.6 / 9.2).
  if (fmt == 3 && s == 1 && KT >= 16 && cdiv(CG, c.g) > 256) {
    c.nw = 4;
    c.xl = false;
  }
  // INT8 weights on the same wide grids take four waves only up to eight
  // rows (activations loaded directly either way): M = 1, K = 4096, N = 20480
  // 18.1 / 18.2 us against 18.8, N = 28672 20.6 / 20.8 against 21.5; K = 8192,
  // N = 28672 39.2 against 43.1.  At 16 rows, direct loads cost more than
  // the overlap gains (N = 20480: 21.0 against 20.2 staged).
  if (fmt == 2 && s == 1 && M <= 8 && KT >= 16 && cdiv(CG, c.g) > 256) c.nw = 4;
  return c;
}

// MXFP4 (FMT 3): `s` is the A E8M0 array and meta_offset the offset of the W
// scale segment in the packed weight.
template <int FMT, int G, int NW, int D, bool ELEMENTWISE, int S = 1, bool XL = false>
hipError_t launch_cfg(const void* x, const void* w, const void* s, const float* sa,
                      const float* sb, void* y, int64_t M, int64_t N, int64_t K, int64_t KT,
                      int64_t CG, hipStream_t stream, int64_t meta_offset = 0) {
  dim3 grid(decode_grid(CG, G, M, 16 * S));
  dim3 block(NW * kWave);
  hipLaunchKernelGGL((decode_gemm_kernel<FMT, G, NW, D, ELEMENTWISE, 0, S, XL>), grid, block, 0,
                     stream,
                     (const uint8_t*)x, (const uint8_t*)w, (const _Float16*)s, sa, sb,
                     (uint16_t*)y, (int)M, (int)N, (int)K, (int)KT, (int)CG, meta_offset);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt_cfg(const DecodeConfig& c, const void* x, const void* w, const void* s,
                          const float* sa, const float* sb, void* y, int64_t M, int64_t N,
                          int64_t K, int64_t KT, int64_t CG, int64_t meta_offset,
                          hipStream_t stream) {
  // fp16 X rows that are not 16-byte aligned (K % 8 != 0) take one
  // element-wise configuration
  if constexpr (FMT == 1 || FMT == 2) {
    if (K % 8 != 0)
      return launch_cfg<FMT, 1, 4, 2, true>(x, w, s, sa, sb, y, M, N, K, KT, CG, stream);
  }
#define QG_CASE(GG, WW, DD, SS, XX)                                                         \
  if (c.g == GG && c.nw == WW && c.d == DD && c.s == SS && c.xl == XX)                      \
    return launch_cfg<FMT, GG, WW, DD, false, SS, XX>(x, w, s, sa, sb, y, M, N, K, KT, CG,  \
                                                      stream, meta_offset);
#define QG_G(GG) \
  QG_CASE(GG, 8, DEPTH, 1, false) QG_CASE(GG, 4, DEPTH, 1, false) QG_CASE(GG, 8, DEPTH, 1, true)
#define QG_GS(GG, SS) QG_CASE(GG, 8, 2, SS, false) QG_CASE(GG, 4, 2, SS, false) \
  if constexpr (SS * (FMT == 3 || FMT == 4 ? 2 : 4) <= 8) {                                \
    QG_CASE(GG, 8, 2, SS, true) QG_CASE(GG, 4, 2, SS, true)                               \
  }
  constexpr int DEPTH = 2;
  QG_G(1) QG_G(2) QG_G(3) QG_G(4)
  if constexpr (FMT == 1) {   // up to eight INT4 column groups fit in registers
    QG_G(5) QG_G(6) QG_G(7) QG_G(8)
  }
  QG_GS(1, 2) QG_GS(2, 2) QG_GS(3, 2) QG_GS(4, 2)
  if constexpr (FMT == 1) {   // two INT4 slabs leave room for seven groups
    QG_GS(5, 2) QG_GS(6, 2) QG_GS(7, 2)
  }
  if constexpr (FMT == 3 || FMT == 4) {   // four slabs: the e4m3 / E2M1 activations
    QG_GS(1, 4) QG_GS(2, 4)
  }
  if constexpr (FMT == 4) {
    QG_GS(3, 4)
  }
#undef QG_GS
#undef QG_G
#undef QG_CASE
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_fmt(const void* x, const void* w, const void* s, const float* sa,
                      const float* sb, void* y, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
  const PackGeom pg = pack_geom(FMT, K, N);
  const DecodeConfig c = pick_decode_config(FMT, M, pg.cg, pg.kt);
  return launch_fmt_cfg<FMT>(c, x, w, s, sa, sb, y, M, N, K, pg.kt, pg.cg, pg.scales, stream);
}

// Slabs per workgroup for the grouped and NVFP4 launches: two above 16 rows
// (as for INT4: each weight tile dequantized once for 32 rows), one with
// short K (four waves).
int slab_count(int64_t M, int nw) { return M > 16 && nw == 8 ? 2 : 1; }

// Column groups per workgroup for the grouped and NVFP4 launches: the same
// one-workgroup-per-CU rule, rounded down to an instantiated value (1, 2, 3,
// 4, or 7 where gmax allows it); short K (four waves) uses 1 or 2.
int slab_groups(int64_t CG, int gmax, int64_t KT) {
  int64_t g = cdiv(CG, 256);
  if (KT < 16) return g >= 2 ? 2 : 1;
  if (g >= 7 && gmax >= 7) return 7;
  g = g < 1 ? 1 : (g > 4 ? 4 : g);
  return (int)g;
}

// Grouped formats: the same kernel with NGT metadata words per column and K
// tile, D = 2; G and NW as for the per-column formats with fewer rows.
template <int FMT, int NGT, int G, int NW, int S, bool XL>
hipError_t launch_grouped_cfg(const void* x, const void* w, void* y, int64_t M, int64_t N,
                              int64_t K, int64_t KT, int64_t CG, int64_t meta_offset,
                              hipStream_t stream) {
  dim3 grid(decode_grid(CG, G, M, 16 * S));
  dim3 block(NW * kWave);
  hipLaunchKernelGGL((decode_gemm_kernel<FMT, G, NW, 2, false, NGT, S, XL>), grid, block, 0,
                     stream,
                     (const uint8_t*)x, (const uint8_t*)w, (const _Float16*)nullptr,
                     (const float*)nullptr, (const float*)nullptr, (uint16_t*)y, (int)M, (int)N,
                     (int)K, (int)KT, (int)CG, meta_offset);
  return hipGetLastError();
}

template <int FMT, int NGT>
hipError_t launch_grouped_ngt(const void* x, const void* w, void* y, int64_t M, int64_t N,
                              int64_t K, int64_t KT, int64_t CG, int64_t meta_offset,
                              hipStream_t stream) {
  const int s = slab_count(M, KT < 16 ? 4 : 8);
  // two slabs with four metadata words per tile leave room for four INT4
  // groups (seven spill)
  const int g = slab_groups(CG, FMT == 1 && !(s == 2 && NGT == 4) ? 7 : 4, KT);
  // seven groups with two metadata words keep eight waves: with four they
  // would need more than 256 registers per lane (one wave per SIMD)
  int nw = g == 7 && NGT > 1 ? (KT < 16 ? 4 : 8) : decode_waves(M, s, KT);
  // grouped INT8 up to eight rows with more than 256 workgroups: four waves,
  // as for per-column INT8 (K = 4096, N = 28672, group 128, M = 1 / 8: 21.1 /
  // 21.3-21.4 us against 21.6-22.1 / 22.3-22.5; K = 8192: M = 1 40.2 against
  // 43.5)
  if (FMT == 2 && s == 1 && M <= 8 && KT >= 16 && cdiv(CG, g) > 256) nw = 4;
  // one slab with more than four groups loads X directly (see use_x_lds)
  const bool xl = use_x_lds(FMT, M, nw, s, KT) && (s > 1 || g <= 4);
#define QG_GCASE(GG, WW, SS, XX)                                                            \
  if (g == GG && nw == WW && s == SS && xl == XX)                                           \
    return launch_grouped_cfg<FMT, NGT, GG, WW, SS, XX>(x, w, y, M, N, K, KT, CG,           \
                                                        meta_offset, stream);
#define QG_GCASE2(GG, SS) QG_GCASE(GG, 8, SS, false) QG_GCASE(GG, 8, SS, true)
#define QG_GCASE4(GG) QG_GCASE2(GG, 2) QG_GCASE(GG, 4, 2, true)
  QG_GCASE(1, 4, 1, false) QG_GCASE(2, 4, 1, false)
  if constexpr (FMT == 2) {
    QG_GCASE(3, 4, 1, false) QG_GCASE(4, 4, 1, false)
  }
  QG_GCASE2(1, 1) QG_GCASE2(2, 1) QG_GCASE2(3, 1) QG_GCASE2(4, 1)
  QG_GCASE4(1) QG_GCASE4(2) QG_GCASE4(3) QG_GCASE4(4)
  if constexpr (FMT == 1) {
    QG_GCASE(7, 8, 1, false)
  }
  if constexpr (FMT == 1 && NGT == 1) {
    QG_GCASE4(7)
  }
  if constexpr (FMT == 1 && NGT == 2) {
    QG_GCASE2(7, 2)
  }
#undef QG_GCASE4
#undef QG_GCASE2
#undef QG_GCASE
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_grouped_fmt(const void* x, const void* w, void* y, int64_t M, int64_t N,
                              int64_t K, int64_t group_k, hipStream_t stream) {
  const PackGeom g = grouped_geom(FMT == 1 ? 5 : 6, K, N, group_k);
  switch (grouped_ngt(group_k)) {
    case 1: return launch_grouped_ngt<FMT, 1>(x, w, y, M, N, K, g.kt, g.cg, g.scales, stream);
    case 2: return launch_grouped_ngt<FMT, 2>(x, w, y, M, N, K, g.kt, g.cg, g.scales, stream);
    default: return launch_grouped_ngt<FMT, 4>(x, w, y, M, N, K, g.kt, g.cg, g.scales, stream);
  }
}

template <int G, int NW, int S, bool XL>
hipError_t launch_nvfp4_cfg(const void* x, const void* w, const float* gs, void* y, int64_t M,
                            int64_t N, int64_t K, int64_t KT, int64_t CG, int64_t meta_offset,
                            hipStream_t stream) {
  dim3 grid(decode_grid(CG, G, M, 16 * S));
  dim3 block(NW * kWave);
  hipLaunchKernelGGL((decode_gemm_kernel<7, G, NW, 2, false, 1, S, XL>), grid, block, 0, stream,
                     (const uint8_t*)x, (const uint8_t*)w, (const _Float16*)nullptr, gs,
                     (const float*)nullptr, (uint16_t*)y, (int)M, (int)N, (int)K, (int)KT,
                     (int)CG, meta_offset);
  return hipGetLastError();
}

// A lane's activation offset inside the kernel is 32-bit and counts from its
// workgroup's first row (row * row bytes + a few hundred bytes), so it stays
// below 2^31 while (rows per workgroup - 1) * row bytes does.  A call whose
// activation rows are longer than that allows runs as consecutive launches
// over row chunks short enough (each launch streams the whole weight; it
// takes rows of over 2^31 / 63 bytes, K in the tens of millions).
constexpr int64_t kRowOffsetLimit = ((int64_t)1 << 31) - 4096;

template <class Launch>
hipError_t in_row_chunks(int64_t M, int64_t row_bytes, Launch launch) {
  int64_t r = M;
  if ((std::min<int64_t>(M, 64) - 1) * row_bytes >= kRowOffsetLimit)
    r = (kRowOffsetLimit - 1) / row_bytes + 1;   // (r - 1) * row_bytes < limit
  for (int64_t m = 0; m < M; m += r) {
    const hipError_t e = launch(m, std::min(r, M - m));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <class T>
const T* rows_at(const void* p, int64_t m, int64_t row_bytes) {
  return reinterpret_cast<const T*>(static_cast<const uint8_t*>(p) + m * row_bytes);
}

}  // namespace

hipError_t launch_decode_nvfp4(const void* x, const void* w_packed, const float* global_scale,
                               void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if ((std::min<int64_t>(M, 64) - 1) * 2 * K >= kRowOffsetLimit)
    return in_row_chunks(M, 2 * K, [&](int64_t m, int64_t rows) {
      return launch_decode_nvfp4(rows_at<uint8_t>(x, m, 2 * K), w_packed, global_scale,
                                 static_cast<uint8_t*>(y) + m * 2 * N, rows, N, K, stream);
    });
  const PackGeom pg = pack_geom(7, K, N);
  const int g = slab_groups(pg.cg, 7, pg.kt);
  const int s = slab_count(M, pg.kt < 16 ? 4 : 8);
  // seven groups keep eight waves (with four: 264 registers per lane)
  const int nw = g == 7 ? (pg.kt < 16 ? 4 : 8) : decode_waves(M, s, pg.kt);
  const bool xl = use_x_lds(7, M, nw, s, pg.kt) && (s > 1 || g <= 4);   // see use_x_lds
#define QG_NCASE(GG, WW, SS, XX)                                                           \
  if (g == GG && nw == WW && s == SS && xl == XX)                                          \
    return launch_nvfp4_cfg<GG, WW, SS, XX>(x, w_packed, global_scale, y, M, N, K, pg.kt,  \
                                            pg.cg, pg.scales, stream);
#define QG_NCASE2(GG, SS) QG_NCASE(GG, 8, SS, false) QG_NCASE(GG, 8, SS, true)
#define QG_NCASE4(GG) QG_NCASE2(GG, 2) QG_NCASE(GG, 4, 2, true)
  QG_NCASE(1, 4, 1, false) QG_NCASE(2, 4, 1, false)
  QG_NCASE2(1, 1) QG_NCASE2(2, 1) QG_NCASE2(3, 1) QG_NCASE2(4, 1) QG_NCASE(7, 8, 1, false)
  QG_NCASE4(1) QG_NCASE4(2) QG_NCASE4(3) QG_NCASE4(4) QG_NCASE2(7, 2)
#undef QG_NCASE4
#undef QG_NCASE2
#undef QG_NCASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_grouped(int fmt, const void* x, const void* w_packed, void* y,
                                 int64_t M, int64_t N, int64_t K, int64_t group_k,
                                 hipStream_t stream) {
  if ((std::min<int64_t>(M, 64) - 1) * 2 * K >= kRowOffsetLimit)
    return in_row_chunks(M, 2 * K, [&](int64_t m, int64_t rows) {
      return launch_decode_grouped(fmt, rows_at<uint8_t>(x, m, 2 * K), w_packed,
                                   static_cast<uint8_t*>(y) + m * 2 * N, rows, N, K, group_k,
                                   stream);
    });
  if (fmt == 5) return launch_grouped_fmt<1>(x, w_packed, y, M, N, K, group_k, stream);
  if (fmt == 6) return launch_grouped_fmt<2>(x, w_packed, y, M, N, K, group_k, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_gemm(int fmt, const void* x, const void* w_packed, const void* scales,
                              const float* scale_a, const float* scale_b, void* y, int64_t M,
                              int64_t N, int64_t K, hipStream_t stream) {
  const int64_t row_bytes = fmt == 3 ? K / 2 : fmt == 4 ? K : 2 * K;
  if ((std::min<int64_t>(M, 64) - 1) * row_bytes >= kRowOffsetLimit)
    return in_row_chunks(M, row_bytes, [&](int64_t m, int64_t rows) {
      // MXFP4: `scales` are A's E8M0 bytes, K / 32 per row
      const void* s = fmt == 3 ? rows_at<uint8_t>(scales, m, K / 32) : scales;
      return launch_decode_gemm(fmt, rows_at<uint8_t>(x, m, row_bytes), w_packed, s, scale_a,
                                scale_b, static_cast<uint8_t*>(y) + m * 2 * N, rows, N, K,
                                stream);
    });
  switch (fmt) {
    case 1: return launch_fmt<1>(x, w_packed, scales, scale_a, scale_b, y, M, N, K, stream);
    case 2: return launch_fmt<2>(x, w_packed, scales, scale_a, scale_b, y, M, N, K, stream);
    case 3: return launch_fmt<3>(x, w_packed, scales, scale_a, scale_b, y, M, N, K, stream);
    case 4: return launch_fmt<4>(x, w_packed, scales, scale_a, scale_b, y, M, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qgemm
