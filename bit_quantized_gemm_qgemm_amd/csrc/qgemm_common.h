// Internal definitions shared by the libqgemm HIP sources (gfx950 only).
//
// Packed weight layouts (produced by qgemm_prepack, private to the library)
// -------------------------------------------------------------------------
// All weight formats are stored as "fragment tiles": a tile covers 16 output
// columns and a fixed span of K, and is laid out in exactly the order in which
// the 64 lanes of a wavefront feed it to a 16x16 matrix-core instruction, so a
// wave fetches a tile with fully coalesced 16-byte-per-lane loads and needs no
// shuffling afterwards.  Tiles are ordered column-group-major:
//   tile(cg, kt) at byte offset (cg * KT + kt) * TILE_BYTES.
// Lane l of a wave owns column cg*16 + (l & 15); g = l >> 4 is its lane group.
//
//   W4A16: TK = 128, 1024 B/tile.  Lane l's 16 bytes = four 32-bit words; word
//          s feeds f16 matrix step s and holds k = kt*128 + 32s + 8g + [0, 8)
//          as eight nibbles in the order (k0, k2, k4, k6, k1, k3, k5, k7) from
//          the least significant nibble up, which lets one AND-OR with an fp16
//          exponent pattern turn two nibbles into two fp16 values at once.
//          Padding code: 8 (value 0).
//   W8A16: TK = 128, 2048 B/tile, two 1 KB halves; lane l's 16 bytes of half
//          h (at offset 1024h + 16l) feed steps 2h and 2h+1, 8 bytes each:
//          byte b holds k = kt*128 + 32(2h + b/8) + 8g + b%8.  Bytes are
//          stored biased (w + 128) so that a byte permute with an fp16
//          exponent pattern yields 1024 + w + 128 exactly.  Padding: 0x80.
//   FP8:   TK = 128, 2048 B/tile, same geometry; lane l holds the 32-element
//          segment k = kt*128 + 32g + [0, 32): bytes 16h + [0, 16) of it at
//          offset 1024h + 16l.  e4m3fn bytes unbiased.  Padding: 0.
//   MXFP4: TK = 256, 2048 B/tile of codes; half h (h = 0, 1) holds, at offset
//          1024h + 16l, the 32 E2M1 codes k = kt*256 + 128h + 32(l>>4) +
//          [0, 32) (even element in the low nibble).  Each half is one
//          128-element K step ks = 2kt + h.  A separate scale segment follows
//          the code segment (256-byte aligned), ordered by groups of 8 column
//          tiles c8 = cg / 8: for each (c8, ks), 512 B at (c8 * 2KT + ks) * 512
//          laid out [lane 64][j 8]; byte (l, j) = E8M0 of column
//          (8 c8 + j) * 16 + (l & 15), block 4ks + (l >> 4).  A lane reads the
//          scales of all 8 tiles of a step with one 8-byte load.
//          Padding: code 0, scale 127 (= 1.0).
//   NVFP4 (weight-only, format 7): TK = 128, 1 KB/tile like W4A16, but word s
//          of lane l holds the 8 E2M1 codes k = kt*128 + 32s + 8g + [0, 8) in
//          natural order (byte j: elements 2j low nibble, 2j+1 high), which
//          is the order the gfx950 FP4 -> fp16 conversion consumes.  A block
//          scale segment follows (256-byte aligned): 128 B per tile, byte
//          c*8 + 4h + s = e4m3 scale of column c of the tile for the 16-element
//          block kt*8 + 2s + h, so the lanes of group g read the dword
//          c*8 + 4*(g >> 1).  Padding: code 0, scale 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qgemm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef unsigned int uintx2 __attribute__((ext_vector_type(2)));
typedef unsigned int uintx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTileN = 16;                 // columns per fragment tile
constexpr int kTileK8 = 128;               // K per tile for W4, W8, FP8
constexpr int kTileK4 = 256;               // K per tile for MXFP4
constexpr int kTileBytesW4 = 1024;
constexpr int kTileBytes = 2048;           // W8, FP8, MXFP4 code tiles
constexpr int kScaleTileBytes = 128;       // MXFP4 scale bytes per tile
constexpr int kE8M0One = 127;              // E8M0 encoding of 1.0

// Matrix-core operand formats of the scaled f8f6f4 instructions.
constexpr int kFmtFP8 = 0;                 // e4m3 (OCP e4m3fn on gfx950)
constexpr int kFmtFP4 = 4;                 // e2m1

__host__ __device__ constexpr int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Geometry of a packed weight (host and device).
struct PackGeom {
  int64_t cg;      // column groups of 16
  int64_t kt;      // K tiles
  int64_t tile;    // bytes per code tile
  int64_t codes;   // bytes of the code segment
  int64_t scales;  // offset of the scale (MXFP4, NVFP4) or metadata (grouped) segment, or 0
  int64_t total;   // total bytes
};

inline PackGeom pack_geom(int fmt, int64_t K, int64_t N) {
  PackGeom g{};
  g.cg = cdiv(N, kTileN);
  if (fmt == 1 || fmt == 7) {  // W4A16, NVFP4 weights
    g.kt = cdiv(K, kTileK8);
    g.tile = kTileBytesW4;
  } else if (fmt == 3) {     // MXFP4
    g.kt = cdiv(K, kTileK4);
    g.tile = kTileBytes;
  } else {                   // W8A16, FP8
    g.kt = cdiv(K, kTileK8);
    g.tile = kTileBytes;
  }
  g.codes = g.cg * g.kt * g.tile;
  if (fmt == 3) {
    g.scales = cdiv(g.codes, 256) * 256;
    g.total = g.scales + cdiv(g.cg, 8) * g.kt * 8 * kScaleTileBytes;
  } else if (fmt == 7) {
    g.scales = cdiv(g.codes, 256) * 256;
    g.total = g.scales + g.cg * g.kt * kScaleTileBytes;
  } else {
    g.scales = 0;
    g.total = g.codes;
  }
  return g;
}

// Grouped weight-only formats (5 = W4A16, 6 = W8A16 with group-wise scales
// and zero points): the code segment of format 1 / 2, then, 256-byte
// aligned, a metadata segment.  For each tile (cg, kt) and column c of it
// (16 per tile) there are NGT 4-byte entries at
//   ((cg * KT + kt) * 16 + c) * NGT + j,
// entry j covering the 128 / NGT K elements kt*128 + j*128/NGT + [0, 128/NGT)
// of column cg*16 + c: low half fp16 (1024 + z) for W4 or (1152 + z) for W8
// (the exponent-pattern subtrahend that leaves w - z), high half the fp16
// scale.  NGT = 1 when group_k is a multiple of 128, 2 when it is 64,
// otherwise 4 (one entry per 32-element matrix step; group_k % 32 == 0, so a
// step never straddles two groups).  Padding entries have scale 0.
inline int grouped_ngt(int64_t group_k) {
  return group_k % 128 == 0 ? 1 : group_k == 64 ? 2 : 4;
}

inline PackGeom grouped_geom(int fmt, int64_t K, int64_t N, int64_t group_k) {
  PackGeom g = pack_geom(fmt == 5 ? 1 : 2, K, N);
  g.scales = cdiv(g.codes, 256) * 256;
  g.total = g.scales + g.cg * g.kt * 16 * grouped_ngt(group_k) * 4;
  return g;
}

// ---- launchers (defined in the .hip files; all enqueue on `stream`) -------
// Each returns hipSuccess or the launch error.

hipError_t launch_prepack(int fmt, const void* w, const void* w_scales, void* packed,
                          int64_t K, int64_t N, hipStream_t stream);
hipError_t launch_prepack_grouped(int fmt, const void* w, const void* scales, const void* zeros,
                                  int64_t group_k, int64_t group_n, void* packed, int64_t K,
                                  int64_t N, hipStream_t stream);

hipError_t launch_quantize_mxfp4(const float* x, int64_t rows, int64_t K, uint8_t* codes,
                                 uint8_t* e8m0, hipStream_t stream);
hipError_t launch_quantize_fp8(const float* x, int64_t count, uint8_t* codes, float* scale,
                               hipStream_t stream);
// Per-block partial maxima of the two-launch FP8 quantizer (workspace form).
constexpr int kFp8Partials = 256;
// count % 4 == 0, x 16-byte aligned; partials holds kFp8Partials floats.
hipError_t launch_quantize_fp8_ws(const float* x, int64_t count, uint8_t* codes, float* scale,
                                  float* partials, hipStream_t stream);

// Small-M path (M rows handled in 16-row slabs) for W4A16 / W8A16 / FP8 /
// MXFP4; for MXFP4 `scales` is the A E8M0 array [M, K/32].
hipError_t launch_decode_gemm(int fmt, const void* x, const void* w_packed, const void* scales,
                              const float* scale_a, const float* scale_b, void* y,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream);

// NVFP4 weights (format 7) with fp16 X: M rows in 16-row slabs;
// global_scale is a device fp32 scalar.
hipError_t launch_decode_nvfp4(const void* x, const void* w_packed, const float* global_scale,
                               void* y, int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Grouped W4A16 / W8A16 (formats 5, 6): M rows in 16-row slabs.
hipError_t launch_decode_grouped(int fmt, const void* x, const void* w_packed, void* y,
                                 int64_t M, int64_t N, int64_t K, int64_t group_k,
                                 hipStream_t stream);

// Whether the operands of a format-`fmt` GEMM (group_k for formats 5 and 6)
// fit the 256 x 256 kernels, whose buffer descriptors take 32-bit offsets
// (every operand below 2^31 bytes).  Larger ones take the kernels that
// address with 64 bits (the 128 x 128 tile kernel, the small-M kernel).
bool pipe_fits(int fmt, int64_t M, int64_t N, int64_t K, int64_t group_k);
// Whether launch_tile_gemm takes a 256 x 256 kernel (else 128 x 128 tiles).
bool tile_is_big(int fmt, int64_t M, int64_t N, int64_t K);

// LDS-tiled matrix-core path for W4A16 / W8A16 at large M (fp16 X with K a
// positive multiple of 8; 256 x 256 output tiles).
hipError_t launch_weight_only_tile(int fmt, const void* x, const void* w_packed,
                                  const void* scales, void* y, int64_t M, int64_t N, int64_t K,
                                  hipStream_t stream);
// NVFP4 weights with fp16 X (format 7) through the same tiled kernel.
hipError_t launch_weight_only_tile_nvfp4(const void* x, const void* w_packed,
                                        const float* global_scale, void* y, int64_t M, int64_t N,
                                        int64_t K, hipStream_t stream);
// Grouped W4A16 / W8A16 (formats 5, 6) through the same tiled kernel.
hipError_t launch_weight_only_tile_grouped(int fmt, const void* x, const void* w_packed, void* y,
                                          int64_t M, int64_t N, int64_t K, int64_t group_k,
                                          hipStream_t stream);

// LDS-tiled matrix-core path for MXFP4 / FP8 (any M).
hipError_t launch_tile_gemm(int fmt, const void* a, const void* a_e8m0, const void* w_packed,
                            const float* scale_a, const float* scale_b, void* c,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);
// Its 256 x 256 kernels (M and N > 128, operands within pipe_fits): MXFP4
// with K % 128 == 0 and at least two 256-element K tiles, FP8 with at least
// two 128-element K tiles.
hipError_t launch_mxfp4_256(const void* a, const void* a_e8m0, const void* w_packed, void* c,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);
hipError_t launch_fp8_256(const void* a, const void* b_packed, const float* scale_a,
                          const float* scale_b, void* c, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream);

// Streaming read of `bytes` bytes (a multiple of 16, buf 16-byte aligned) by
// `workgroups` workgroups; one word per workgroup goes to sink.
hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int64_t workgroups,
                             hipStream_t stream);
// Back-to-back scaled 32 x 32 x 64 matrix instructions (FP4 or FP8 operands)
// on register-held data: `iters` rounds of 16 per wave; ops holds 272 bytes
// per thread (workgroups x 256 threads); one float per workgroup to sink.
hipError_t launch_mfma_probe(bool fp4, const void* ops, int64_t iters, float* sink,
                             int64_t workgroups, hipStream_t stream);

// ---- device helpers --------------------------------------------------------

// fp32 -> bf16 bits, round to nearest even (inputs are finite here; a NaN
// stays a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

}  // namespace qgemm
