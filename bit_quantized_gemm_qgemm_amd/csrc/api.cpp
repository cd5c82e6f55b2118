// libqgemm C ABI: argument checks, dispatch by format and M, launch on the
// caller's stream.  Every check that needs no device runs first, so a bad
// call returns its status without touching the HIP runtime.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/qgemm.h"
#include "qgemm_common.h"

namespace {

using qgemm::PackGeom;
using qgemm::pack_geom;
using qgemm::grouped_geom;

constexpr int64_t kMaxIndex = (int64_t)1 << 31;   // kernels index with 32-bit ints
// The weight-only GEMMs take the 256 x 256 tiled kernel from M = 256 on once
// its grid fills three quarters of the CUs (192 tiles), or from M = 640 with
// at least 48 tiles; otherwise the small-M kernel.  A round of tiles costs
// about the same whatever M is, while the small-M kernel's time grows with M.
// Measured on MI355X (us, small-M kernel / tiled kernel):
//   W8A16 K = 4096 N = 11008 (43 tile columns): M = 512 114 / 132, 768 189 / 134
//   W4A16 K = 8192 N = 28672 (112): M = 256 177 / 219, 384 267 / 223
//   W8A16 K = 4096 N = 4096 (16): M = 512 75 / 132, 768 165 / 132
//   grouped W4A16 g128 K = 8192 N = 28672: M = 256 214 / 257, 384 318 / 258
//   grouped W8A16 g128 K = 4096 N = 11008: M = 512 115 / 151, 768 186 / 153
//   NVFP4 K = 8192 N = 28672: M = 256 198 / 247, 384 303 / 249
constexpr int64_t kWeightOnlyTileMinM = 256;
constexpr int64_t kWeightOnlyTileFullGrid = 192;
constexpr int64_t kWeightOnlyTileLongM = 640;
constexpr int64_t kWeightOnlyTileLongMinTiles = 48;
bool weight_only_tiled(int64_t M, int64_t N) {
  if (M < kWeightOnlyTileMinM || N <= 128) return false;
  const int64_t tiles = qgemm::cdiv(M, 256) * qgemm::cdiv(N, 256);
  return tiles >= kWeightOnlyTileFullGrid ||
         (M >= kWeightOnlyTileLongM && tiles >= kWeightOnlyTileLongMinTiles);
}
// FP8 and MXFP4 GEMMs take the small-M kernel (16-row slabs, up to four per
// workgroup) up to M = 64; from 65 to 128 rows unless N is wide (FP8 N >=
// 24576, MXFP4 N >= 16384), where one row of 256 x 256 tiles is faster; and
// above that while the tiled kernels' grid stays small: FP8 up to M = 512
// while M * N <= 2.6e6 (5 * 2^19), MXFP4 up to M = 256 while M * N <= 2^21.
// Otherwise the tile kernels.  The small-M kernel's time grows with M * N * K,
// while the tiled kernels take about one 256 x 256 x K tile per CU whatever M
// is.  Measured on MI355X (us, small-M kernel / tile kernels):
//   FP8 K = N = 8192:   M = 128 30 / 68, 144 47 / 69, 256 48 / 73, 384 71 / 70,
//                       512 95 / 73
//   FP8 K = N = 4096:   M = 512 37 / 40, 768 54 / 40
//   FP8 K = 8192, N = 28672: M = 72 92 / 78, 128 86 / 72, 144 123 / 80
//   FP8 K = 4096, N = 16384: M = 96 28 / 38
//   MXFP4 K = N = 8192: M = 128 27 / 44, 192 39 / 50, 256 49 / 56, 384 70 / 46
//   MXFP4 K = N = 4096: M = 256 24 / 26, 384 34 / 25
//   MXFP4 K = 8192, N = 28672: M = 72 87 / 48, 128 85 / 51, 144 117 / 52
//   MXFP4 K = 4096, N = 16384: M = 72 27.6 / 24.7, 128 27.8 / 27.0
bool scaled_small_m(int fmt, int64_t M, int64_t N) {
  if (M <= 64) return true;
  if (M <= 128) return N < (fmt == QGEMM_FP8 ? 24576 : 16384);
  if (fmt == QGEMM_FP8) return M <= 512 && M * N <= 2621440;
  return M <= 256 && M * N <= 2097152;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// formats of qgemm_prepack (the grouped ones have their own prepack)
bool valid_format(int fmt) {
  return (fmt >= QGEMM_W4A16 && fmt <= QGEMM_FP8) || fmt == QGEMM_NVFP4;
}

// K constraints per format (see qgemm.h).
bool k_ok(int fmt, int64_t K) {
  switch (fmt) {
    case QGEMM_W4A16: return K % 2 == 0;
    case QGEMM_W8A16: return true;
    case QGEMM_MXFP4: return K % 32 == 0;
    case QGEMM_FP8: return K % 16 == 0;
    case QGEMM_NVFP4: return K % 16 == 0;
    default: return false;
  }
}

// Sizes must be non-negative and every array the kernels index must stay
// addressable with 32-bit element offsets.
int check_sizes(int fmt, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return QGEMM_ERR_SHAPE;
  if (!k_ok(fmt, K)) return QGEMM_ERR_SHAPE;
  if (M >= kMaxIndex || N >= kMaxIndex || K >= kMaxIndex) return QGEMM_ERR_SHAPE;
  if (M * K * 2 >= kMaxIndex * 2 || M * N >= kMaxIndex || K * N >= kMaxIndex * 2)
    return QGEMM_ERR_SHAPE;
  return QGEMM_OK;
}

// Device architecture check, cached per device ordinal.  The environment
// variable QGEMM_ARCH_OVERRIDE, when set, stands in for the current device's
// architecture name and no device is queried (host-side tests of the
// ERR_ARCH path on machines without the GPU).
int check_device() {
  if (const char* forced = std::getenv("QGEMM_ARCH_OVERRIDE"))
    return std::strncmp(forced, "gfx950", 6) == 0 ? QGEMM_OK : QGEMM_ERR_ARCH;
  static std::mutex mu;
  static int cached[64];
  static bool init = false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QGEMM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!init) {
    for (int& c : cached) c = 1;  // 1 = unknown
    init = true;
  }
  if (dev < 0 || dev >= 64) return QGEMM_ERR_DEVICE;
  if (cached[dev] == 1) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QGEMM_ERR_DEVICE;
    cached[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? QGEMM_OK : QGEMM_ERR_ARCH;
  }
  return cached[dev];
}

int launched(hipError_t e) { return e == hipSuccess ? QGEMM_OK : QGEMM_ERR_LAUNCH; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// A pointer may be NULL only when its array holds no elements.
bool present(const void* p, int64_t elems) { return p != nullptr || elems == 0; }

// The kernel a GEMM call of format fmt launches (M, N, K and group_k already
// validated): the one dispatch every entry point and qgemm_dispatch_kernel
// apply.  The fused-quantization calls dispatch as their GEMM format.
int kernel_for(int fmt, int64_t M, int64_t N, int64_t K, int64_t group_k) {
  if (M == 0 || N == 0) return QGEMM_KERNEL_NONE;
  switch (fmt) {
    case QGEMM_W4A16:
    case QGEMM_W8A16:   // fp16 X rows of the tile kernel must be 16-byte aligned
      return weight_only_tiled(M, N) && K > 0 && K % 8 == 0 &&
                     qgemm::pipe_fits(fmt, M, N, K, 0)
                 ? QGEMM_KERNEL_WEIGHT_ONLY_256
                 : QGEMM_KERNEL_SMALL_M;
    case QGEMM_NVFP4:   // K % 16 == 0
      return weight_only_tiled(M, N) && K > 0 && qgemm::pipe_fits(fmt, M, N, K, 0)
                 ? QGEMM_KERNEL_WEIGHT_ONLY_256
                 : QGEMM_KERNEL_SMALL_M;
    case QGEMM_W4A16_GROUPED:
    case QGEMM_W8A16_GROUPED:   // K % 32 == 0
      return weight_only_tiled(M, N) && K > 0 && qgemm::pipe_fits(fmt, M, N, K, group_k)
                 ? QGEMM_KERNEL_WEIGHT_ONLY_256
                 : QGEMM_KERNEL_SMALL_M;
    case QGEMM_MXFP4:
    case QGEMM_FP8:
      if (scaled_small_m(fmt, M, N)) return QGEMM_KERNEL_SMALL_M;
      if (!qgemm::tile_is_big(fmt, M, N, K)) return QGEMM_KERNEL_TILE_128;
      return fmt == QGEMM_MXFP4 ? QGEMM_KERNEL_MXFP4_256 : QGEMM_KERNEL_FP8_256;
    default:
      return QGEMM_ERR_FORMAT;
  }
}

int weight_only(int fmt, const void* x, const void* w_packed, const void* scales, void* y,
                int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_sizes(fmt, M, N, K);
  if (st != QGEMM_OK) return st;
  if (!present(x, M * K) || !present(w_packed, K * N) || !present(scales, N) ||
      !present(y, M * N))
    return QGEMM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(scales, 16) || !aligned(y, 16))
    return QGEMM_ERR_ALIGN;
  if (M == 0 || N == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  // Large M: LDS-tiled matrix-core kernel (each weight byte is read once per
  // 256 rows).  Otherwise the register-dequant kernel in 16-row slabs, the
  // bandwidth path of decode.
  if (kernel_for(fmt, M, N, K, 0) == QGEMM_KERNEL_WEIGHT_ONLY_256)
    return launched(qgemm::launch_weight_only_tile(fmt, x, w_packed, scales, y, M, N, K,
                                                   as_stream(stream)));
  return launched(qgemm::launch_decode_gemm(fmt, x, w_packed, scales, nullptr, nullptr, y, M, N,
                                            K, as_stream(stream)));
}

// Grouped weight-only formats: K and group_k multiples of 32 (a 32-element
// matrix step never straddles two groups), the sizes of the per-column format.
int check_grouped(int fmt, int64_t M, int64_t N, int64_t K, int64_t group_k) {
  if (fmt != QGEMM_W4A16_GROUPED && fmt != QGEMM_W8A16_GROUPED) return QGEMM_ERR_FORMAT;
  if (group_k <= 0 || group_k % 32 != 0 || K % 32 != 0) return QGEMM_ERR_SHAPE;
  if (group_k >= kMaxIndex) return QGEMM_ERR_SHAPE;
  return check_sizes(fmt == QGEMM_W4A16_GROUPED ? QGEMM_W4A16 : QGEMM_W8A16, M, N, K);
}

int grouped_gemm(int fmt, const void* x, const void* w_packed, void* y, int64_t M, int64_t N,
                 int64_t K, int64_t group_k, void* stream) {
  int st = check_grouped(fmt, M, N, K, group_k);
  if (st != QGEMM_OK) return st;
  if (!present(x, M * K) || !present(w_packed, K * N) || !present(y, M * N))
    return QGEMM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 16)) return QGEMM_ERR_ALIGN;
  if (M == 0 || N == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  // K % 32 == 0 here, so fp16 X rows are 16-byte aligned
  if (kernel_for(fmt, M, N, K, group_k) == QGEMM_KERNEL_WEIGHT_ONLY_256)
    return launched(qgemm::launch_weight_only_tile_grouped(fmt, x, w_packed, y, M, N, K, group_k,
                                                           as_stream(stream)));
  return launched(qgemm::launch_decode_grouped(fmt, x, w_packed, y, M, N, K, group_k,
                                               as_stream(stream)));
}

// ---- FP8 GEMM with fp32 A quantized on the device --------------------------

// Checks shared by qgemm_fp8_act and qgemm_fp8_act_noalloc (everything but
// the workspace).
int check_fp8_act(const float* a, const void* b_packed, const float* scale_b, void* c,
                  int64_t M, int64_t N, int64_t K) {
  int st = check_sizes(QGEMM_FP8, M, N, K);
  if (st != QGEMM_OK) return st;
  if (!present(a, M * K) || !present(b_packed, K * N) || !present(c, M * N) || !scale_b)
    return QGEMM_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b_packed, 16) || !aligned(c, 16) || !aligned(scale_b, 4))
    return QGEMM_ERR_ALIGN;
  return QGEMM_OK;
}

// Quantize A into ws (codes [M*K], the fp32 scale at round_up(M*K, 16), the
// partial maxima 16 bytes after it), then the GEMM; everything on `stream`.
int fp8_act_run(const float* a, const void* b_packed, const float* scale_b, void* c, uint8_t* ws,
                int64_t M, int64_t N, int64_t K, void* stream) {
  uint8_t* codes = ws;
  float* scale_a = reinterpret_cast<float*>(codes + qgemm::cdiv(M * K, 16) * 16);
  float* partials = scale_a + 4;
  // an empty A still gets its scale (1.0, the all-zero rule); K % 16 == 0,
  // so A is whole 16-byte pieces
  int st = launched(
      qgemm::launch_quantize_fp8_ws(a, M * K, codes, scale_a, partials, as_stream(stream)));
  if (st != QGEMM_OK || N == 0) return st;
  if (kernel_for(QGEMM_FP8, M, N, K, 0) == QGEMM_KERNEL_SMALL_M)
    return launched(qgemm::launch_decode_gemm(QGEMM_FP8, codes, b_packed, nullptr, scale_a,
                                              scale_b, c, M, N, K, as_stream(stream)));
  return launched(qgemm::launch_tile_gemm(QGEMM_FP8, codes, nullptr, b_packed, scale_a, scale_b,
                                          c, M, N, K, as_stream(stream)));
}

// Fixed scratch of qgemm_fp8_act_noalloc, one copy per GPU, held from the
// moment the code object is loaded on that GPU until the process ends: the
// codes of A (at most QGEMM_FP8_ACT_NOALLOC_MAX_ELEMS bytes), 16 bytes holding
// the fp32 scale, then the partial maxima of the quantizer.  Every call on a
// GPU shares that GPU's copy.  Nothing in it needs to start at zero: each
// call writes every byte it later reads.
constexpr int64_t kNoAllocScratchBytes =
    QGEMM_FP8_ACT_NOALLOC_MAX_ELEMS + 16 + 4 * qgemm::kFp8Partials;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// The device address of this GPU's copy of `scratch`.  In host code the
// array's name is only a host-side stand-in, so kernels receive the address
// hipGetSymbolAddress returns, looked up once per device with that device
// current.
int scratch_of_current_device(uint8_t** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return QGEMM_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
      return QGEMM_ERR_DEVICE;
    addr[dev] = p;
  }
  *out = static_cast<uint8_t*>(addr[dev]);
  return QGEMM_OK;
}

}  // namespace

extern "C" {

const char* qgemm_status_string(int status) {
  switch (status) {
    case QGEMM_OK: return "ok";
    case QGEMM_ERR_NULL: return "a required pointer is NULL";
    case QGEMM_ERR_SHAPE: return "invalid shape (negative, K not a multiple the format needs, or too large)";
    case QGEMM_ERR_ALIGN: return "pointer not aligned (16 bytes for arrays, 4 for scalar scales)";
    case QGEMM_ERR_ARCH: return "current device is not gfx950";
    case QGEMM_ERR_LAUNCH: return "kernel launch failed";
    case QGEMM_ERR_FORMAT: return "unknown format id";
    case QGEMM_ERR_DEVICE: return "no HIP device available";
    case QGEMM_ERR_TOO_LARGE: return "input larger than the entry point's fixed scratch";
    default: return "unknown status";
  }
}

int qgemm_abi_version(void) { return 103; }

int qgemm_dispatch_kernel(int fmt, int64_t M, int64_t N, int64_t K, int64_t group_k) {
  int st;
  if (fmt == QGEMM_W4A16_GROUPED || fmt == QGEMM_W8A16_GROUPED)
    st = check_grouped(fmt, M, N, K, group_k);
  else if (valid_format(fmt))
    st = check_sizes(fmt, M, N, K);
  else
    return QGEMM_ERR_FORMAT;
  if (st != QGEMM_OK) return st;
  return kernel_for(fmt, M, N, K, group_k);
}

int64_t qgemm_prepack_bytes(int fmt, int64_t K, int64_t N) {
  if (!valid_format(fmt)) return QGEMM_ERR_FORMAT;
  const int st = check_sizes(fmt, 0, N, K);
  if (st != QGEMM_OK) return st;
  return pack_geom(fmt, K, N).total;
}

int qgemm_prepack(int fmt, const void* w, const void* w_scales, void* w_packed, int64_t K,
                  int64_t N, void* stream) {
  if (!valid_format(fmt)) return QGEMM_ERR_FORMAT;
  if (!w_packed) return QGEMM_ERR_NULL;
  int st = check_sizes(fmt, 0, N, K);
  if (st != QGEMM_OK) return st;
  const bool empty = (K == 0 || N == 0);
  if (!empty && !w) return QGEMM_ERR_NULL;
  if ((fmt == QGEMM_MXFP4 || fmt == QGEMM_NVFP4) && !empty && !w_scales) return QGEMM_ERR_NULL;
  if (!aligned(w_packed, 16)) return QGEMM_ERR_ALIGN;
  if (pack_geom(fmt, K, N).total == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  return launched(qgemm::launch_prepack(fmt, w, w_scales, w_packed, K, N, as_stream(stream)));
}

int64_t qgemm_prepack_grouped_bytes(int fmt, int64_t K, int64_t N, int64_t group_k) {
  const int st = check_grouped(fmt, 0, N, K, group_k);
  if (st != QGEMM_OK) return st;
  return grouped_geom(fmt, K, N, group_k).total;
}

int qgemm_prepack_grouped(int fmt, const void* w, const void* scales, const void* zeros,
                          int64_t group_k, int64_t group_n, void* w_packed, int64_t K,
                          int64_t N, void* stream) {
  int st = check_grouped(fmt, 0, N, K, group_k);
  if (st != QGEMM_OK) return st;
  if (group_n < 1 || group_n >= kMaxIndex) return QGEMM_ERR_SHAPE;
  if (!w_packed) return QGEMM_ERR_NULL;
  const bool empty = (K == 0 || N == 0);
  if (!empty && (!w || !scales)) return QGEMM_ERR_NULL;
  if (!aligned(w_packed, 16) || !aligned(w, 16) || !aligned(scales, 16) || !aligned(zeros, 16))
    return QGEMM_ERR_ALIGN;
  if (grouped_geom(fmt, K, N, group_k).total == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  return launched(qgemm::launch_prepack_grouped(fmt, w, scales, zeros, group_k, group_n,
                                                w_packed, K, N, as_stream(stream)));
}

int qgemm_nvfp4(const void* x, const void* w_packed, const float* global_scale, void* y,
                int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_sizes(QGEMM_NVFP4, M, N, K);
  if (st != QGEMM_OK) return st;
  if (!present(x, M * K) || !present(w_packed, K * N) || !present(y, M * N) || !global_scale)
    return QGEMM_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 16) || !aligned(global_scale, 4))
    return QGEMM_ERR_ALIGN;
  if (M == 0 || N == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  // K % 16 == 0 here, so fp16 X rows are 16-byte aligned
  if (kernel_for(QGEMM_NVFP4, M, N, K, 0) == QGEMM_KERNEL_WEIGHT_ONLY_256)
    return launched(qgemm::launch_weight_only_tile_nvfp4(x, w_packed, global_scale, y, M, N, K,
                                                         as_stream(stream)));
  return launched(qgemm::launch_decode_nvfp4(x, w_packed, global_scale, y, M, N, K,
                                             as_stream(stream)));
}

int qgemm_w4a16_grouped(const void* x, const void* w_packed, void* y, int64_t M, int64_t N,
                        int64_t K, int64_t group_k, void* stream) {
  return grouped_gemm(QGEMM_W4A16_GROUPED, x, w_packed, y, M, N, K, group_k, stream);
}

int qgemm_w8a16_grouped(const void* x, const void* w_packed, void* y, int64_t M, int64_t N,
                        int64_t K, int64_t group_k, void* stream) {
  return grouped_gemm(QGEMM_W8A16_GROUPED, x, w_packed, y, M, N, K, group_k, stream);
}

int qgemm_quantize_mxfp4(const float* x, int64_t rows, int64_t K, uint8_t* codes, uint8_t* e8m0,
                         void* stream) {
  if (rows < 0 || K < 0 || K % 32 != 0) return QGEMM_ERR_SHAPE;
  if (!present(x, rows * K) || !present(codes, rows * K) || !present(e8m0, rows * K))
    return QGEMM_ERR_NULL;
  if (rows >= kMaxIndex || K >= kMaxIndex || rows * K >= kMaxIndex * 4) return QGEMM_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(codes, 16)) return QGEMM_ERR_ALIGN;
  if (rows == 0 || K == 0) return QGEMM_OK;
  int st = check_device();
  if (st != QGEMM_OK) return st;
  return launched(qgemm::launch_quantize_mxfp4(x, rows, K, codes, e8m0, as_stream(stream)));
}

int qgemm_quantize_fp8(const float* x, int64_t count, uint8_t* codes, float* scale,
                       void* stream) {
  if (!scale) return QGEMM_ERR_NULL;
  if (count < 0) return QGEMM_ERR_SHAPE;
  if (count > 0 && (!x || !codes)) return QGEMM_ERR_NULL;
  if (!aligned(scale, 4)) return QGEMM_ERR_ALIGN;
  int st = check_device();
  if (st != QGEMM_OK) return st;
  return launched(qgemm::launch_quantize_fp8(x, count, codes, scale, as_stream(stream)));
}

int qgemm_w4a16(const void* x, const void* w_packed, const void* scales, void* y, int64_t M,
                int64_t N, int64_t K, void* stream) {
  return weight_only(QGEMM_W4A16, x, w_packed, scales, y, M, N, K, stream);
}

int qgemm_w8a16(const void* x, const void* w_packed, const void* scales, void* y, int64_t M,
                int64_t N, int64_t K, void* stream) {
  return weight_only(QGEMM_W8A16, x, w_packed, scales, y, M, N, K, stream);
}

int qgemm_mxfp4(const void* a_codes, const void* a_e8m0, const void* w_packed, void* c,
                int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_sizes(QGEMM_MXFP4, M, N, K);
  if (st != QGEMM_OK) return st;
  if (!present(a_codes, M * K) || !present(a_e8m0, M * K) || !present(w_packed, K * N) ||
      !present(c, M * N))
    return QGEMM_ERR_NULL;
  if (!aligned(a_codes, 16) || !aligned(w_packed, 16) || !aligned(c, 16)) return QGEMM_ERR_ALIGN;
  if (M == 0 || N == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  if (kernel_for(QGEMM_MXFP4, M, N, K, 0) == QGEMM_KERNEL_SMALL_M)
    return launched(qgemm::launch_decode_gemm(QGEMM_MXFP4, a_codes, w_packed, a_e8m0, nullptr,
                                              nullptr, c, M, N, K, as_stream(stream)));
  return launched(qgemm::launch_tile_gemm(QGEMM_MXFP4, a_codes, a_e8m0, w_packed, nullptr,
                                          nullptr, c, M, N, K, as_stream(stream)));
}

int qgemm_fp8(const void* a, const void* b_packed, const float* scale_a, const float* scale_b,
              void* c, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_sizes(QGEMM_FP8, M, N, K);
  if (st != QGEMM_OK) return st;
  if (!present(a, M * K) || !present(b_packed, K * N) || !present(c, M * N) || !scale_a ||
      !scale_b)
    return QGEMM_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b_packed, 16) || !aligned(c, 16)) return QGEMM_ERR_ALIGN;
  if (!aligned(scale_a, 4) || !aligned(scale_b, 4)) return QGEMM_ERR_ALIGN;
  if (M == 0 || N == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  if (kernel_for(QGEMM_FP8, M, N, K, 0) == QGEMM_KERNEL_SMALL_M)
    return launched(qgemm::launch_decode_gemm(QGEMM_FP8, a, b_packed, nullptr, scale_a, scale_b,
                                              c, M, N, K, as_stream(stream)));
  return launched(qgemm::launch_tile_gemm(QGEMM_FP8, a, nullptr, b_packed, scale_a, scale_b, c, M,
                                          N, K, as_stream(stream)));
}

// ---- activation quantization enqueued before the GEMM ----------------------

int64_t qgemm_act_workspace_bytes(int fmt, int64_t M, int64_t K) {
  if (fmt != QGEMM_MXFP4 && fmt != QGEMM_FP8) return QGEMM_ERR_FORMAT;
  if (M < 0 || K < 0 || !k_ok(fmt, K)) return QGEMM_ERR_SHAPE;
  if (M >= kMaxIndex || K >= kMaxIndex || M * K >= kMaxIndex * 2) return QGEMM_ERR_SHAPE;
  if (fmt == QGEMM_MXFP4) return qgemm::cdiv(M * K / 2, 16) * 16 + M * (K / 32);
  return qgemm::cdiv(M * K, 16) * 16 + 16 + 4 * qgemm::kFp8Partials;
}

int qgemm_mxfp4_act(const float* a, const void* w_packed, void* c, void* workspace, int64_t M,
                    int64_t N, int64_t K, void* stream) {
  int st = check_sizes(QGEMM_MXFP4, M, N, K);
  if (st != QGEMM_OK) return st;
  if (!present(a, M * K) || !present(w_packed, K * N) || !present(c, M * N) ||
      !present(workspace, M * K))
    return QGEMM_ERR_NULL;
  if (!aligned(a, 16) || !aligned(w_packed, 16) || !aligned(c, 16) || !aligned(workspace, 16))
    return QGEMM_ERR_ALIGN;
  if (M == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  uint8_t* codes = static_cast<uint8_t*>(workspace);
  uint8_t* e8m0 = codes + qgemm::cdiv(M * K / 2, 16) * 16;
  if (K > 0) {
    st = launched(qgemm::launch_quantize_mxfp4(a, M, K, codes, e8m0, as_stream(stream)));
    if (st != QGEMM_OK) return st;
  }
  if (N == 0) return QGEMM_OK;
  if (kernel_for(QGEMM_MXFP4, M, N, K, 0) == QGEMM_KERNEL_SMALL_M)
    return launched(qgemm::launch_decode_gemm(QGEMM_MXFP4, codes, w_packed, e8m0, nullptr,
                                              nullptr, c, M, N, K, as_stream(stream)));
  return launched(qgemm::launch_tile_gemm(QGEMM_MXFP4, codes, e8m0, w_packed, nullptr, nullptr, c,
                                          M, N, K, as_stream(stream)));
}

int qgemm_fp8_act(const float* a, const void* b_packed, const float* scale_b, void* c,
                  void* workspace, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_fp8_act(a, b_packed, scale_b, c, M, N, K);
  if (st != QGEMM_OK) return st;
  if (!workspace) return QGEMM_ERR_NULL;
  if (!aligned(workspace, 16)) return QGEMM_ERR_ALIGN;
  if (M == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  return fp8_act_run(a, b_packed, scale_b, c, static_cast<uint8_t*>(workspace), M, N, K, stream);
}

int qgemm_fp8_act_noalloc(const float* a, const void* b_packed, const float* scale_b, void* c,
                          int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_fp8_act(a, b_packed, scale_b, c, M, N, K);
  if (st != QGEMM_OK) return st;
  if (M * K > QGEMM_FP8_ACT_NOALLOC_MAX_ELEMS) return QGEMM_ERR_TOO_LARGE;
  if (M == 0) return QGEMM_OK;
  if ((st = check_device()) != QGEMM_OK) return st;
  uint8_t* ws = nullptr;
  if ((st = scratch_of_current_device(&ws)) != QGEMM_OK) return st;
  return fp8_act_run(a, b_packed, scale_b, c, ws, M, N, K, stream);
}

int qgemm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int64_t workgroups,
                     void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || workgroups < 1 || workgroups > (1 << 20))
    return QGEMM_ERR_SHAPE;
  if (!present(buf, bytes) || !sink) return QGEMM_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QGEMM_ERR_ALIGN;
  int st = check_device();
  if (st != QGEMM_OK) return st;
  return launched(qgemm::launch_read_probe(buf, bytes, sink, workgroups, as_stream(stream)));
}

int qgemm_mfma_probe(int fmt, const void* operands, int64_t iters, float* sink,
                     int64_t workgroups, void* stream) {
  if (fmt != QGEMM_MXFP4 && fmt != QGEMM_FP8) return QGEMM_ERR_FORMAT;
  if (iters < 0 || workgroups < 1 || workgroups > (1 << 20)) return QGEMM_ERR_SHAPE;
  if (!operands || !sink) return QGEMM_ERR_NULL;
  if (!aligned(operands, 16) || !aligned(sink, 4)) return QGEMM_ERR_ALIGN;
  int st = check_device();
  if (st != QGEMM_OK) return st;
  return launched(qgemm::launch_mfma_probe(fmt == QGEMM_MXFP4, operands, iters, sink, workgroups,
                                           as_stream(stream)));
}

}  // extern "C"
