/*
 * qgemm.h -- C ABI of libqgemm: GEMMs whose low-bit operands are dequantized
 * inside the kernel, for AMD Instinct MI355X (gfx950).
 *
 * Four variants:
 *   W4A16  Y[M,N] = X[M,K] * ((code - 8) * s[n])   two INT4 codes per byte
 *   W8A16  Y[M,N] = X[M,K] * (w * s[n])            INT8 weights
 *   MXFP4  C[M,N] = A[M,K] * W[N,K]^T              E2M1 codes, one E8M0
 *                                                  exponent per 32 K-elements
 *   FP8    C[M,N] = (A[M,K] * B[K,N]) * sa * sb    e4m3fn, per-tensor scales
 * and their extensions: W4A16 / W8A16 with group-wise scales and zero points
 * (qgemm_w4a16_grouped, qgemm_w8a16_grouped), NVFP4 weights with fp16
 * activations (qgemm_nvfp4), and MXFP4 / FP8 GEMMs that quantize fp32
 * activations on the device inside the call (qgemm_mxfp4_act,
 * qgemm_fp8_act).
 *
 * Sources (short names):
 *   W4A16 page -- "Triton W4A16 blocked GEMM and Blackwell NVFP4"
 *                 (dreamvfia.cn), section 2: INT4 packing and dequant.
 *   W8A16 page -- "Triton quantization: W8A16 weight-quantized fused GEMM"
 *                 (datawhalechina llm-algo-leetcode, chapter 10), Steps 1-3.
 *   MXFP4 page -- "MXFP4 matrix-multiplication kernel principle" (pwwt.cn),
 *                 sections 1-3, eqs. (1) and (2).
 *   FP8 page   -- "FP8 GEMM kernel in Triton via CUTLASS naming"
 *                 (blog.hotdry.top), kernel and parameter list.
 *
 * Conventions for every entry point
 *   - Array pointers are DEVICE pointers owned by the caller; one may be NULL
 *     only when its array holds no elements.  The library
 *     never allocates device memory and never synchronises; it enqueues its
 *     kernels on `stream` (a hipStream_t; NULL means the null stream) and
 *     returns.  Scalar-scale pointers (FP8) are device pointers too, so a
 *     scale computed on the device never forces a host round trip.
 *   - Matrices are dense and row-major with no padding between rows.
 *   - Every array pointer must be 16-byte aligned (the kernels move 128-bit
 *     words; MXFP4 page, section 1); fp32 scale pointers 4-byte aligned.
 *   - Arguments are checked on the host before anything is launched.  A
 *     status < 0 means nothing was enqueued (except QGEMM_ERR_LAUNCH, which
 *     reports a failed launch).  No entry point prints or throws.
 *   - M == 0 or N == 0 is a valid no-op; K == 0 writes the empty sum, an
 *     all-zero output.  Results are deterministic: the same inputs give
 *     bit-identical outputs (no atomics in any GEMM).
 *   - Accumulation is fp32; the output is rounded to nearest-even once.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight formats accepted by qgemm_prepack / qgemm_prepack_bytes (1-4, 7)
 * and by qgemm_prepack_grouped / qgemm_prepack_grouped_bytes (5, 6). */
enum qgemm_format {
  QGEMM_W4A16 = 1,
  QGEMM_W8A16 = 2,
  QGEMM_MXFP4 = 3,
  QGEMM_FP8 = 4,
  QGEMM_W4A16_GROUPED = 5,   /* INT4 codes, group-wise scales, zero points */
  QGEMM_W8A16_GROUPED = 6,   /* INT8 weights, group-wise scales, zero points */
  QGEMM_NVFP4 = 7            /* E2M1 weights, e4m3 per-16 block scales      */
};

/* Status codes. */
enum qgemm_status {
  QGEMM_OK = 0,
  QGEMM_ERR_NULL = -1,    /* a required pointer is NULL                     */
  QGEMM_ERR_SHAPE = -2,   /* negative size, or K not a multiple the format
                             needs, or a size too large for 32-bit indexing */
  QGEMM_ERR_ALIGN = -3,   /* a pointer is not 16-byte (scales: 4-byte)
                             aligned                                         */
  QGEMM_ERR_ARCH = -4,    /* the current device is not gfx950 (if the
                             environment variable QGEMM_ARCH_OVERRIDE is
                             set, its value is taken as the device's
                             architecture name and no device is queried)  */
  QGEMM_ERR_LAUNCH = -5,  /* the HIP runtime reported a launch error        */
  QGEMM_ERR_FORMAT = -6,  /* unknown format id                               */
  QGEMM_ERR_DEVICE = -7,  /* no HIP device could be queried                  */
  QGEMM_ERR_TOO_LARGE = -8  /* the input exceeds an entry point's fixed
                               scratch (qgemm_fp8_act_noalloc)              */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* qgemm_status_string(int status);

/* ABI version of this header (major * 100 + minor). */
int qgemm_abi_version(void);

/* The kernels a GEMM call can launch (qgemm_dispatch_kernel). */
enum qgemm_kernel {
  QGEMM_KERNEL_NONE = 0,            /* M = 0 or N = 0: nothing is launched          */
  QGEMM_KERNEL_SMALL_M = 1,         /* register-dequant kernel in 16-row slabs      */
  QGEMM_KERNEL_WEIGHT_ONLY_256 = 2, /* weight-only formats: 256 x 256 matrix tiles  */
  QGEMM_KERNEL_MXFP4_256 = 3,       /* MXFP4: 256 x 256 matrix tiles                */
  QGEMM_KERNEL_FP8_256 = 4,         /* FP8: 256 x 256 matrix tiles                  */
  QGEMM_KERNEL_TILE_128 = 5         /* MXFP4 / FP8: 128 x 128 matrix tiles          */
};

/*
 * qgemm_dispatch_kernel -- which kernel a GEMM call of format fmt with these
 * sizes launches: the dispatch by M, N and K that every GEMM entry point
 * applies (the W8A16 page's performance and autotune notes and the FP8
 * page's parameter list choose a tile configuration per M, N, K; here a
 * fixed rule fitted to measurements does).  qgemm_mxfp4_act and
 * qgemm_fp8_act(_noalloc) dispatch as QGEMM_MXFP4 and QGEMM_FP8.  group_k is
 * read for the grouped formats only.  Host-only: touches no device.  Returns
 * a qgemm_kernel value, or a negative status for a format or sizes the entry
 * point would reject (QGEMM_ERR_FORMAT, QGEMM_ERR_SHAPE).
 */
int qgemm_dispatch_kernel(int fmt, int64_t M, int64_t N, int64_t K, int64_t group_k);

/*
 * qgemm_prepack_bytes -- size in bytes of the opaque packed weight buffer for
 * a K x N weight (N output columns; for MXFP4, N rows of W[N,K]).  Host-only,
 * never touches the device.  Returns < 0 (a qgemm_status) on bad arguments.
 */
int64_t qgemm_prepack_bytes(int fmt, int64_t K, int64_t N);

/*
 * qgemm_prepack -- convert a weight from the pages' canonical layout into the
 * kernel-native packed layout (offline; not part of the timed GEMM).
 *
 *   fmt = QGEMM_W4A16: w = uint8 [K/2, N]; byte (j, n) holds k = 2j in its low
 *         nibble and k = 2j+1 in its high nibble (W4A16 page, section 2).
 *         K must be even.  w_scales must be NULL (scales go to the GEMM).
 *   fmt = QGEMM_W8A16: w = int8 [K, N] (W8A16 page, Step 3).  w_scales NULL.
 *   fmt = QGEMM_MXFP4: w = uint8 codes [N, K/2] (element 2j in the low nibble
 *         of byte j), w_scales = uint8 E8M0 [N, K/32] (MXFP4 page, sections
 *         2-3; data and scale segments kept apart as in section 1).
 *         K % 32 == 0.
 *   fmt = QGEMM_FP8:   w = e4m3fn bytes B [K, N] (FP8 page kernel, B indexed
 *         by k then n).  K % 16 == 0.  w_scales NULL (the per-tensor scale
 *         goes to the GEMM).
 *   fmt = QGEMM_NVFP4: w = uint8 E2M1 codes [N, K/2] (element 2j in the low
 *         nibble of byte j), w_scales = uint8 e4m3fn block scales [N, K/16],
 *         one per 16 consecutive K elements (W4A16 page, section 3: two-level
 *         block scaling; the block size and scale format are this library's
 *         reading).  K % 16 == 0.  NaN scale codes are not checked.
 *
 * w_packed must hold qgemm_prepack_bytes(fmt, K, N) bytes; the library fills
 * all of it (padding included).  The packed layout is private to the library
 * and is consumed only by the matching qgemm_* GEMM with the same K and N.
 */
int qgemm_prepack(int fmt, const void* w, const void* w_scales, void* w_packed,
                  int64_t K, int64_t N, void* stream);

/*
 * qgemm_quantize_mxfp4 -- quantize fp32 x[rows, K] to MXFP4, bit-identical to
 * the MXFP4 page's section-3 quantizer read exactly: per row and 32-element K
 * block, amax = max(max|x|, 1e-8f); e = ceil(log2(amax / 6)) taken exactly;
 * E8M0 byte E = e + 127; each element goes to the nearest of
 * {0, .5, 1, 1.5, 2, 3, 4, 6} * 2^e (ties to the smaller magnitude) with the
 * sign bit set when x < 0.  codes: uint8 [rows, K/2], element 2j in the low
 * nibble of byte j; e8m0: uint8 [rows, K/32].  K % 32 == 0.  Inputs must be
 * finite (non-finite input gives unspecified codes).
 */
int qgemm_quantize_mxfp4(const float* x, int64_t rows, int64_t K,
                         uint8_t* codes, uint8_t* e8m0, void* stream);

/*
 * qgemm_quantize_fp8 -- per-tensor e4m3fn quantization of fp32 x[count]
 * (FP8 page, precision management: e4m3fn, range +-448, per-tensor scale).
 * scale = fp32(max|x| / 448) (1.0 for an all-zero tensor) is written to the
 * device float *scale; codes[i] = e4m3fn(fp32(x[i] / scale)), rounded to
 * nearest-even and saturated at +-448.  Inputs must be finite.  *scale is
 * also used as scratch between the kernels this enqueues: do not read it
 * before the stream reaches the end of this call.
 */
int qgemm_quantize_fp8(const float* x, int64_t count, uint8_t* codes,
                       float* scale, void* stream);

/*
 * qgemm_w4a16 -- Y[M,N] fp16 = X[M,K] fp16 * W_deq, W_deq[k,n] =
 * (code[k,n] - 8) * scales[n] (W4A16 page, section 2), fp32 accumulation.
 * w_packed comes from qgemm_prepack(QGEMM_W4A16, ..., K, N); scales is fp16
 * [N].  K even.  The scale is applied to the fp32 column sum (equal in exact
 * arithmetic to scaling each weight).
 */
int qgemm_w4a16(const void* x, const void* w_packed, const void* scales,
                void* y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qgemm_w8a16 -- Y[M,N] fp16 = X[M,K] fp16 * (W_int8 * S) (W8A16 page,
 * Step 1), fp32 accumulation.  w_packed from qgemm_prepack(QGEMM_W8A16, ...),
 * scales fp16 [N].  Any K >= 0.
 */
int qgemm_w8a16(const void* x, const void* w_packed, const void* scales,
                void* y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qgemm_mxfp4 -- C[M,N] bf16 = A_deq[M,K] * W_deq[N,K]^T (MXFP4 page,
 * section 2, eqs. 1-2), each 32-element block scaled by 2^(E_A + E_W - 254)
 * inside the matrix cores, fp32 accumulation.  a_codes uint8 [M, K/2] and
 * a_e8m0 uint8 [M, K/32] as produced by qgemm_quantize_mxfp4; w_packed from
 * qgemm_prepack(QGEMM_MXFP4, ..., K, N).  K % 32 == 0.
 */
int qgemm_mxfp4(const void* a_codes, const void* a_e8m0, const void* w_packed,
                void* c, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qgemm_fp8 -- C[M,N] bf16 = (A[M,K] * B[K,N]) * (*scale_a) * (*scale_b)
 * (FP8 page: e4m3fn inputs, fp32 accumulator, per-tensor scales, bf16 out).
 * a: e4m3fn [M, K]; b_packed from qgemm_prepack(QGEMM_FP8, ..., K, N);
 * scale_a / scale_b: device fp32 scalars.  K % 16 == 0.
 */
int qgemm_fp8(const void* a, const void* b_packed, const float* scale_a,
              const float* scale_b, void* c, int64_t M, int64_t N, int64_t K,
              void* stream);

/*
 * Activation quantization enqueued before the GEMM, on the same stream and
 * without a host round trip (MXFP4 page, section 3: per-32 E8M0 quantization
 * of A; FP8 page: per-tensor amax scaling and e4m3fn cast of A).  The caller
 * passes fp32 activations and a device workspace of
 * qgemm_act_workspace_bytes(fmt, M, K) bytes (16-byte aligned), which after
 * the call (in stream order) holds the quantized A exactly as
 * qgemm_quantize_mxfp4 / qgemm_quantize_fp8 produce it:
 *   MXFP4: codes [M, K/2] at offset 0, E8M0 [M, K/32] at round_up(M*K/2, 16);
 *   FP8:   e4m3fn codes [M, K] at offset 0, the fp32 scale at
 *          round_up(M*K, 16); 1 KB of per-block partial maxima follows at
 *          round_up(M*K, 16) + 16 (scratch of the quantizer).
 * The result equals quantizing with those entry points and calling
 * qgemm_mxfp4 / qgemm_fp8 on the quantized A (bit for bit).  The library
 * allocates nothing.  Calls that share a workspace must not overlap.
 *
 * qgemm_act_workspace_bytes -- fmt QGEMM_MXFP4 or QGEMM_FP8; < 0 on bad
 * arguments.  Host-only.
 */
int64_t qgemm_act_workspace_bytes(int fmt, int64_t M, int64_t K);

/* C[M,N] bf16 = MXFP4(a)[M,K] * W_deq^T, a fp32 [M, K]; K % 32 == 0. */
int qgemm_mxfp4_act(const float* a, const void* w_packed, void* c, void* workspace, int64_t M,
                    int64_t N, int64_t K, void* stream);

/* C[M,N] bf16 = (FP8(a) * B) * s_a * (*scale_b), a fp32 [M, K]; K % 16 == 0. */
int qgemm_fp8_act(const float* a, const void* b_packed, const float* scale_b, void* c,
                  void* workspace, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qgemm_fp8_act_noalloc -- qgemm_fp8_act without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments,
 * same kernels and bit-identical output; the quantized A, its scale and the
 * quantizer's partial maxima go to a fixed scratch array that the library
 * holds on each GPU (QGEMM_FP8_ACT_NOALLOC_MAX_ELEMS bytes of codes plus
 * 1040 bytes), so the call allocates nothing.  M * K above
 * QGEMM_FP8_ACT_NOALLOC_MAX_ELEMS returns QGEMM_ERR_TOO_LARGE and enqueues
 * nothing.  Every call on one GPU uses that GPU's one scratch array: calls
 * that may overlap on the same GPU (other streams, other host threads) race
 * and must be ordered by the caller.  The scratch is not readable by the
 * caller.
 */
#define QGEMM_FP8_ACT_NOALLOC_MAX_ELEMS ((int64_t)16 * 1024 * 1024)
int qgemm_fp8_act_noalloc(const float* a, const void* b_packed, const float* scale_b, void* c,
                          int64_t M, int64_t N, int64_t K, void* stream);

/*
 * qgemm_nvfp4 -- Y[M,N] fp16 = X[M,K] fp16 * W_deq^T with
 * W_deq[n,k] = e2m1(code[n,k]) * e4m3(scale[n, k/16]) * (*global_scale)
 * (W4A16 page, section 3: NVFP4's two-level block scaling; the second level
 * is the fp32 per-tensor scale, a device scalar).  Each weight is formed
 * exactly in fp16 (an E2M1 value times an e4m3 value), the products
 * accumulate in fp32 and the global scale multiplies the fp32 sum.
 * w_packed from qgemm_prepack(QGEMM_NVFP4, ..., K, N).  K % 16 == 0.
 */
int qgemm_nvfp4(const void* x, const void* w_packed, const float* global_scale, void* y,
                int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Group-wise scales and asymmetric zero points (W4A16 page, section 1: the
 * dequant (w - zero_point) * scale; W8A16 page, extensions: scales shared by
 * groups of columns, and zero points for asymmetric quantization).  The scale
 * and zero point of weight (k, n) are entry (k / group_k, n / group_n) of
 * row-major tables with KG = ceil(K / group_k) rows and NG = ceil(N / group_n)
 * columns; group_k = K, group_n = 1 is the per-column scheme of
 * qgemm_w4a16 / qgemm_w8a16.
 *
 * qgemm_prepack_grouped_bytes -- size of the packed buffer (host-only).
 * group_k must be a positive multiple of 32 and K a multiple of 32.
 */
int64_t qgemm_prepack_grouped_bytes(int fmt, int64_t K, int64_t N, int64_t group_k);

/*
 * qgemm_prepack_grouped -- pack codes, scales and zero points into one
 * buffer for qgemm_w4a16_grouped / qgemm_w8a16_grouped.
 *
 *   fmt = QGEMM_W4A16_GROUPED: w = uint8 [K/2, N] as for QGEMM_W4A16;
 *         zeros = uint8 [KG, NG] with values 0..15, or NULL for 8.
 *   fmt = QGEMM_W8A16_GROUPED: w = int8 [K, N]; zeros = int8 [KG, NG], or
 *         NULL for 0.
 *   scales = fp16 [KG, NG], any finite values.  group_n >= 1.
 *
 * W_deq[k, n] = (w[k, n] - z) * s with (s, z) the entry of (k, n).  The
 * GEMMs form each dequantized weight in fp16 as (w - z) * s rounded once to
 * nearest-even (the W4A16 page's section-1 arithmetic) and accumulate in
 * fp32.  Zero points are device data and are not range-checked (that would
 * need a host sync): W4 values outside 0..15 give unspecified results.
 */
int qgemm_prepack_grouped(int fmt, const void* w, const void* scales, const void* zeros,
                          int64_t group_k, int64_t group_n, void* w_packed, int64_t K,
                          int64_t N, void* stream);

/*
 * qgemm_w4a16_grouped / qgemm_w8a16_grouped -- Y[M,N] fp16 = X[M,K] fp16 *
 * W_deq with the grouped W_deq above; w_packed from qgemm_prepack_grouped with
 * the same K, N and group_k.  K % 32 == 0.
 */
int qgemm_w4a16_grouped(const void* x, const void* w_packed, void* y, int64_t M, int64_t N,
                        int64_t K, int64_t group_k, void* stream);
int qgemm_w8a16_grouped(const void* x, const void* w_packed, void* y, int64_t M, int64_t N,
                        int64_t K, int64_t group_k, void* stream);

/*
 * qgemm_read_probe -- measurement reference, not part of any GEMM: reads the
 * `bytes` bytes of buf once with the weight stream's access pattern (16-byte
 * non-temporal loads per lane, eight in flight per lane, one contiguous chunk
 * of whole 1 KB pieces per workgroup, `workgroups` workgroups of 256 threads)
 * and writes one 32-bit fold of its chunk per workgroup to sink[workgroups].
 * Timed around a launch it gives the plain HBM read rate for that byte
 * count, against which the decode GEMMs' weight streaming is compared (W8A16
 * page, performance analysis: weight read bandwidth).  bytes % 16 == 0; buf
 * 16-byte aligned; 1 <= workgroups <= 2^20.
 */
int qgemm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int64_t workgroups,
                     void* stream);

/*
 * qgemm_mfma_probe -- measurement reference, not part of any GEMM: the
 * practical rate of the scaled matrix instruction that the MXFP4 and FP8 tile
 * GEMMs are built on (MXFP4 page, section 2: the block dot product with the
 * exponent-add scale product in one step).  Each of `workgroups` workgroups
 * (256 threads, 4 waves) loads register operands from `operands` (272 bytes
 * per thread, 16-byte aligned: random bytes give operand data like the
 * GEMMs'), then issues iters x 16 v_mfma_scale_f32_32x32x64_f8f6f4 per wave
 * with nothing else in the loop (fmt QGEMM_MXFP4: E2M1 operands and E8M0
 * scales 120..127; QGEMM_FP8: e4m3 operands, unit scales) and writes one
 * float per workgroup to sink[workgroups].  Flops per launch =
 * workgroups * 4 * iters * 16 * 131072.  1 <= workgroups <= 2^20.
 */
int qgemm_mfma_probe(int fmt, const void* operands, int64_t iters, float* sink,
                     int64_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
