// C-ABI layer of libfp8blk.so: argument validation (host only, before any HIP
// call or write), then dispatch to the kernel launchers. The interface and its
// numerics are documented in include/fp8blk.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/fp8blk.h"
#include "internal.h"

namespace {

thread_local char g_last_error[512] = "";

fp8blk_status fail(fp8blk_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

fp8blk_status ok() {
  g_last_error[0] = '\0';
  return FP8BLK_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Scale strides are bounded so that every grid offset fits comfortably in
// 64 bits (and in any real allocation).
constexpr int64_t kMaxScaleStride = (int64_t)1 << 40;

// True when the cells of a written scale grid [gr][gc] with element strides
// (sr, sc) are distinct floats: one stride must step over the whole extent of
// the other axis (row-major, column-major and padded layouts all do), so that
// no two workgroups store to the same float.
bool grid_cells_distinct(int64_t gr, int64_t gc, int64_t sr, int64_t sc) {
  if (gr <= 1 && gc <= 1) return true;
  if (gr <= 1) return sc > 0;
  if (gc <= 1) return sr > 0;
  return (sc > 0 && (__int128)sr >= (__int128)gc * sc) || (sr > 0 && (__int128)sc >= (__int128)gr * sr);
}

// Byte range [lo, hi) of a strided 2-D array with rows >= 1 and cols >= 1.
struct Range {
  uintptr_t lo, hi;
};
Range range2d(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t elem) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return {b, b + (uintptr_t)(((rows - 1) * ld + cols) * elem)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// Byte range covered by a scale grid [gr][gc] with element strides (sr, sc) >= 0.
Range range_grid(const float* p, int64_t gr, int64_t gc, int64_t sr, int64_t sc) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  const int64_t last = (gr - 1) * sr + (gc - 1) * sc;
  return {b, b + (uintptr_t)((last + 1) * 4)};
}

fp8blk_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FP8BLK_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // indices are kept in 32 bits inside kernels
// the GEMM addresses a 256-row operand tile with 32-bit byte offsets
constexpr int64_t kMaxLdCodes = (int64_t)1 << 23;
// ... and a scale grid with 32-bit byte offsets from its base
constexpr int64_t kMaxScaleGridBytes = (int64_t)1 << 32;

fp8blk_status check_format(fp8blk_format fmt, const char* what) {
  if (fmt == FP8BLK_E4M3 || fmt == FP8BLK_E5M2) return FP8BLK_OK;
  return fail(FP8BLK_EINVAL, "%s: unknown fp8 format %d", what, (int)fmt);
}

}  // namespace

extern "C" {

int fp8blk_abi_version(void) { return FP8BLK_ABI_VERSION; }

const char* fp8blk_last_error(void) { return g_last_error; }

const char* fp8blk_status_string(fp8blk_status s) {
  switch (s) {
    case FP8BLK_OK: return "FP8BLK_OK";
    case FP8BLK_EINVAL: return "FP8BLK_EINVAL";
    case FP8BLK_EALIGN: return "FP8BLK_EALIGN";
    case FP8BLK_EUNSUPPORTED: return "FP8BLK_EUNSUPPORTED";
    case FP8BLK_EHIP: return "FP8BLK_EHIP";
  }
  return "FP8BLK_UNKNOWN";
}

fp8blk_status fp8_quantize(const void* x, fp8blk_dtype x_dtype, int64_t rows, int64_t cols,
                           int64_t ld_x, fp8blk_granularity gran, fp8blk_format fmt, uint8_t* q,
                           int64_t ld_q, float* scales, int64_t scale_stride_row,
                           int64_t scale_stride_col, void* stream) {
  const char* fn = "fp8_quantize";
  if (!x || !q || !scales) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (x_dtype != FP8BLK_BF16 && x_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown input dtype %d", fn, (int)x_dtype);
  if (gran != FP8BLK_PER_TENSOR && gran != FP8BLK_GROUP_1x128 && gran != FP8BLK_BLOCK_128x128)
    return fail(FP8BLK_EINVAL, "%s: unknown granularity %d", fn, (int)gran);
  if (fp8blk_status st = check_format(fmt, fn)) return st;
  if (rows < 0 || cols < 0) return fail(FP8BLK_EINVAL, "%s: negative size", fn);
  if (rows >= kMaxDim || cols >= kMaxDim || ld_x >= kMaxDim || ld_q >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: dimension above 2^31", fn);
  if (ld_x < cols || ld_q < cols) return fail(FP8BLK_EINVAL, "%s: leading dimension < cols", fn);
  if (scale_stride_row < 0 || scale_stride_col < 0)
    return fail(FP8BLK_EINVAL, "%s: negative scale stride", fn);
  if (scale_stride_row >= kMaxScaleStride || scale_stride_col >= kMaxScaleStride)
    return fail(FP8BLK_EUNSUPPORTED, "%s: scale stride above 2^40", fn);
  const int64_t esz = x_dtype == FP8BLK_BF16 ? 2 : 4;
  if (!aligned16(x) || !aligned16(q)) return fail(FP8BLK_EALIGN, "%s: x and q must be 16-byte aligned", fn);
  if (!aligned4(scales)) return fail(FP8BLK_EALIGN, "%s: scales must be 4-byte aligned", fn);
  if ((ld_x * esz) % 16 != 0 || ld_q % 16 != 0)
    return fail(FP8BLK_EALIGN, "%s: ld_x * elem_size and ld_q must be multiples of 16 bytes", fn);
  if (gran == FP8BLK_GROUP_1x128) {
    const int64_t groups = rows * ((cols + 127) / 128);
    if (groups >= kMaxDim) return fail(FP8BLK_EUNSUPPORTED, "%s: more than 2^31 groups", fn);
  }
  if (rows > 0 && cols > 0) {
    const Range rx = range2d(x, rows, cols, ld_x, esz);
    const Range rq = range2d(q, rows, cols, ld_q, 1);
    int64_t gr = 1, gc = 1;
    if (gran == FP8BLK_GROUP_1x128) { gr = rows; gc = (cols + 127) / 128; }
    if (gran == FP8BLK_BLOCK_128x128) { gr = (rows + 127) / 128; gc = (cols + 127) / 128; }
    const Range rs = gran == FP8BLK_PER_TENSOR ? range_grid(scales, 1, 1, 0, 0)
                                               : range_grid(scales, gr, gc, scale_stride_row, scale_stride_col);
    if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs))
      return fail(FP8BLK_EINVAL, "%s: x, q and scales must not overlap", fn);
    if (gran != FP8BLK_PER_TENSOR && !grid_cells_distinct(gr, gc, scale_stride_row, scale_stride_col))
      return fail(FP8BLK_EINVAL, "%s: scale strides map two grid cells to one float", fn);
  } else if (gran != FP8BLK_PER_TENSOR) {
    return ok();   // empty grid: nothing to write
  }
  fp8blk::QuantArgs a;
  a.x = x;
  a.x_dtype = (int)x_dtype;
  a.rows = rows;
  a.cols = cols;
  a.ld_x = ld_x;
  a.gran = (int)gran;
  a.fmt = (int)fmt;
  a.q = q;
  a.ld_q = ld_q;
  a.scales = scales;
  a.ss_row = scale_stride_row;
  a.ss_col = scale_stride_col;
  return hip_status(fp8blk::launch_quantize(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"

namespace {

// Validation shared by both GEMM entry points: everything about the inputs.
// Fills `g` with the inputs and the byte ranges of the four input arrays.
fp8blk_status check_gemm_inputs(const char* fn, int64_t M, int64_t N, int64_t K, const uint8_t* a,
                                int64_t lda, const float* scale_a, fp8blk_granularity gran_a,
                                int64_t sa_stride_m, int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                                const float* scale_b, fp8blk_granularity gran_b, int64_t sb_stride_n,
                                int64_t sb_stride_k, fp8blk_format fmt_a, fp8blk_format fmt_b,
                                fp8blk::GemmArgs& g, Range (&in)[4]) {
  if (!a || !b || !scale_a || !scale_b) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (gran_a != FP8BLK_PER_TENSOR && gran_a != FP8BLK_GROUP_1x128)
    return fail(FP8BLK_EINVAL, "%s: gran_a must be PER_TENSOR or GROUP_1x128", fn);
  if (gran_b != FP8BLK_PER_TENSOR && gran_b != FP8BLK_BLOCK_128x128)
    return fail(FP8BLK_EINVAL, "%s: gran_b must be PER_TENSOR or BLOCK_128x128", fn);
  if (fp8blk_status st = check_format(fmt_a, fn)) return st;
  if (fp8blk_status st = check_format(fmt_b, fn)) return st;
  if (M < 0 || N <= 0 || K <= 0) return fail(FP8BLK_EINVAL, "%s: need M >= 0, N > 0, K > 0", fn);
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: dimension above 2^31", fn);
  if (N % 128 != 0 || K % 128 != 0)
    return fail(FP8BLK_EUNSUPPORTED, "%s: N and K must be multiples of 128", fn);
  if (lda < K || ldb < K) return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  if (lda >= kMaxLdCodes || ldb >= kMaxLdCodes)
    return fail(FP8BLK_EUNSUPPORTED, "%s: lda and ldb must be below 2^23", fn);
  if (sa_stride_m < 0 || sa_stride_k < 0 || sb_stride_n < 0 || sb_stride_k < 0)
    return fail(FP8BLK_EINVAL, "%s: negative scale stride", fn);
  if (sa_stride_m >= kMaxScaleStride || sa_stride_k >= kMaxScaleStride || sb_stride_n >= kMaxScaleStride ||
      sb_stride_k >= kMaxScaleStride)
    return fail(FP8BLK_EUNSUPPORTED, "%s: scale stride above 2^40", fn);
  if (!aligned16(a) || !aligned16(b)) return fail(FP8BLK_EALIGN, "%s: a and b must be 16-byte aligned", fn);
  if (!aligned4(scale_a) || !aligned4(scale_b))
    return fail(FP8BLK_EALIGN, "%s: scale_a and scale_b must be 4-byte aligned", fn);
  if (lda % 16 != 0 || ldb % 16 != 0) return fail(FP8BLK_EALIGN, "%s: lda and ldb must be multiples of 16 bytes", fn);
  if (M > 0) {
    // The prefill kernel reads each scale grid through one buffer resource
    // with 32-bit byte offsets from the grid's base, so a grid must span less
    // than 4 GiB (its largest cell's byte offset + 4).
    const int64_t nk = K / 128;
    if (gran_a != FP8BLK_PER_TENSOR &&
        ((M - 1) * sa_stride_m + (nk - 1) * sa_stride_k + 1) * 4 >= kMaxScaleGridBytes)
      return fail(FP8BLK_EUNSUPPORTED, "%s: scale_a grid spans 4 GiB or more", fn);
    if (gran_b != FP8BLK_PER_TENSOR &&
        ((N / 128 - 1) * sb_stride_n + (nk - 1) * sb_stride_k + 1) * 4 >= kMaxScaleGridBytes)
      return fail(FP8BLK_EUNSUPPORTED, "%s: scale_b grid spans 4 GiB or more", fn);
    in[0] = range2d(a, M, K, lda, 1);
    in[1] = range2d(b, N, K, ldb, 1);
    in[2] = gran_a == FP8BLK_PER_TENSOR ? range_grid(scale_a, 1, 1, 0, 0)
                                        : range_grid(scale_a, M, K / 128, sa_stride_m, sa_stride_k);
    in[3] = gran_b == FP8BLK_PER_TENSOR ? range_grid(scale_b, 1, 1, 0, 0)
                                        : range_grid(scale_b, N / 128, K / 128, sb_stride_n, sb_stride_k);
  }
  g = fp8blk::GemmArgs{};
  g.M = M;
  g.N = N;
  g.K = K;
  g.a = a;
  g.lda = lda;
  g.sa = scale_a;
  g.gran_a = (int)gran_a;
  g.sa_m = sa_stride_m;
  g.sa_k = sa_stride_k;
  g.b = b;
  g.ldb = ldb;
  g.sb = scale_b;
  g.gran_b = (int)gran_b;
  g.sb_n = sb_stride_n;
  g.sb_k = sb_stride_k;
  g.fmt_a = (int)fmt_a;
  g.fmt_b = (int)fmt_b;
  return FP8BLK_OK;
}

bool overlaps_any(Range r, const Range (&in)[4]) {
  for (const Range& x : in)
    if (overlap(r, x)) return true;
  return false;
}

}  // namespace

extern "C" {

fp8blk_status fp8_block_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                             const float* scale_a, fp8blk_granularity gran_a, int64_t sa_stride_m,
                             int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                             const float* scale_b, fp8blk_granularity gran_b, int64_t sb_stride_n,
                             int64_t sb_stride_k, fp8blk_format fmt_a, fp8blk_format fmt_b,
                             void* c, fp8blk_dtype c_dtype, int64_t ldc, void* stream) {
  const char* fn = "fp8_block_gemm";
  fp8blk::GemmArgs g;
  Range in[4] = {};
  if (fp8blk_status st = check_gemm_inputs(fn, M, N, K, a, lda, scale_a, gran_a, sa_stride_m, sa_stride_k, b,
                                           ldb, scale_b, gran_b, sb_stride_n, sb_stride_k, fmt_a, fmt_b, g, in))
    return st;
  if (!c) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (c_dtype != FP8BLK_BF16 && c_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown output dtype %d", fn, (int)c_dtype);
  if (ldc < N) return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  const int64_t csz = c_dtype == FP8BLK_BF16 ? 2 : 4;
  if (!aligned16(c)) return fail(FP8BLK_EALIGN, "%s: c must be 16-byte aligned", fn);
  if ((ldc * csz) % 16 != 0) return fail(FP8BLK_EALIGN, "%s: ldc * elem_size must be a multiple of 16 bytes", fn);
  if (M == 0) return ok();
  if (overlaps_any(range2d(c, M, N, ldc, csz), in)) return fail(FP8BLK_EINVAL, "%s: c must not overlap the inputs", fn);
  g.c = c;
  g.c_dtype = (int)c_dtype;
  g.ldc = ldc;
  g.quant_out = 0;
  g.mx = 0;
  return hip_status(fp8blk::launch_block_gemm(g, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_quantize_gemm_decode(const void* x, fp8blk_dtype x_dtype, int64_t M, int64_t N, int64_t K,
                                       int64_t ld_x, fp8blk_granularity gran_a, fp8blk_format fmt_a,
                                       const uint8_t* b, int64_t ldb, int b_packed, const float* scale_b,
                                       fp8blk_granularity gran_b, int64_t sb_stride_n, int64_t sb_stride_k,
                                       fp8blk_format fmt_b, void* c, fp8blk_dtype c_dtype, int64_t ldc,
                                       uint8_t* q_out, int64_t ld_q, float* scale_out, int64_t so_stride_m,
                                       int64_t so_stride_k, void* stream) {
  const char* fn = "fp8_quantize_gemm_decode";
  if (!x || !b || !scale_b || !c) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (x_dtype != FP8BLK_BF16 && x_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown input dtype %d", fn, (int)x_dtype);
  if (c_dtype != FP8BLK_BF16 && c_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown output dtype %d", fn, (int)c_dtype);
  if (gran_a != FP8BLK_PER_TENSOR && gran_a != FP8BLK_GROUP_1x128)
    return fail(FP8BLK_EINVAL, "%s: gran_a must be PER_TENSOR or GROUP_1x128", fn);
  if (gran_b != FP8BLK_PER_TENSOR && gran_b != FP8BLK_BLOCK_128x128)
    return fail(FP8BLK_EINVAL, "%s: gran_b must be PER_TENSOR or BLOCK_128x128", fn);
  if (b_packed != 0 && b_packed != 1) return fail(FP8BLK_EINVAL, "%s: b_packed must be 0 or 1", fn);
  if (fp8blk_status st = check_format(fmt_a, fn)) return st;
  if (fp8blk_status st = check_format(fmt_b, fn)) return st;
  if (M < 1 || N <= 0 || K <= 0) return fail(FP8BLK_EINVAL, "%s: need M >= 1, N > 0, K > 0", fn);
  if (M > 64 || N >= kMaxDim || K >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: M must be at most 64 and N, K below 2^31", fn);
  if (N % 128 != 0 || K % 128 != 0) return fail(FP8BLK_EUNSUPPORTED, "%s: N and K must be multiples of 128", fn);
  if (gran_a == FP8BLK_PER_TENSOR && M * K > 65536)
    return fail(FP8BLK_EUNSUPPORTED, "%s: per-tensor M * K above 65536 (quantize and multiply in two calls)", fn);
  if (b_packed) ldb = K;   // the packed operand spans N * K contiguous bytes
  if (ld_x < K || ldb < K || ldc < N || (q_out && ld_q < K))
    return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  if (ld_x >= kMaxDim || ldb >= kMaxLdCodes || ldc >= kMaxDim || ld_q >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: leading dimension too large", fn);
  if (sb_stride_n < 0 || sb_stride_k < 0 || so_stride_m < 0 || so_stride_k < 0)
    return fail(FP8BLK_EINVAL, "%s: negative scale stride", fn);
  if (sb_stride_n >= kMaxScaleStride || sb_stride_k >= kMaxScaleStride || so_stride_m >= kMaxScaleStride ||
      so_stride_k >= kMaxScaleStride)
    return fail(FP8BLK_EUNSUPPORTED, "%s: scale stride above 2^40", fn);
  const bool group = gran_a == FP8BLK_GROUP_1x128;
  if (group && scale_out && !grid_cells_distinct(M, K / 128, so_stride_m, so_stride_k))
    return fail(FP8BLK_EINVAL, "%s: scale_out strides map distinct scales to one float", fn);
  const int64_t xsz = x_dtype == FP8BLK_BF16 ? 2 : 4;
  const int64_t csz = c_dtype == FP8BLK_BF16 ? 2 : 4;
  if (!aligned16(x) || !aligned16(b) || !aligned16(c) || (q_out && !aligned16(q_out)))
    return fail(FP8BLK_EALIGN, "%s: x, b, c and q_out must be 16-byte aligned", fn);
  if (!aligned4(scale_b) || (scale_out && !aligned4(scale_out)))
    return fail(FP8BLK_EALIGN, "%s: scale_b and scale_out must be 4-byte aligned", fn);
  if ((ld_x * xsz) % 16 != 0 || ldb % 16 != 0 || (ldc * csz) % 16 != 0 || (q_out && ld_q % 16 != 0))
    return fail(FP8BLK_EALIGN, "%s: ld_x, ldb, ldc and ld_q must span multiples of 16 bytes", fn);
  const Range in[4] = {range2d(x, M, K, ld_x, xsz), range2d(b, N, K, ldb, 1),
                       gran_b == FP8BLK_PER_TENSOR ? range_grid(scale_b, 1, 1, 0, 0)
                                                   : range_grid(scale_b, N / 128, K / 128, sb_stride_n, sb_stride_k),
                       Range{0, 0}};
  const Range rc = range2d(c, M, N, ldc, csz);
  const Range rq = q_out ? range2d(q_out, M, K, ld_q, 1) : Range{0, 0};
  const Range rs = !scale_out ? Range{0, 0}
                   : group    ? range_grid(scale_out, M, K / 128, so_stride_m, so_stride_k)
                              : range_grid(scale_out, 1, 1, 0, 0);
  if (overlaps_any(rc, in) || overlaps_any(rq, in) || overlaps_any(rs, in) || overlap(rc, rq) || overlap(rc, rs) ||
      overlap(rq, rs))
    return fail(FP8BLK_EINVAL, "%s: outputs must not overlap the inputs or each other", fn);
  fp8blk::QuantGemmDecodeArgs a{};
  a.g.M = M;
  a.g.N = N;
  a.g.K = K;
  a.g.b = b;
  a.g.ldb = ldb;
  a.g.sb = scale_b;
  a.g.gran_b = (int)gran_b;
  a.g.sb_n = sb_stride_n;
  a.g.sb_k = sb_stride_k;
  a.g.fmt_a = (int)fmt_a;
  a.g.fmt_b = (int)fmt_b;
  a.g.c = c;
  a.g.c_dtype = (int)c_dtype;
  a.g.ldc = ldc;
  a.x = x;
  a.x_dtype = (int)x_dtype;
  a.ld_x = ld_x;
  a.gran_a = (int)gran_a;
  a.packed = b_packed;
  a.q_out = q_out;
  a.ld_q = q_out ? ld_q : 0;
  a.s_out = scale_out;
  a.so_m = group ? so_stride_m : 0;
  a.so_k = group ? so_stride_k : 0;
  return hip_status(fp8blk::launch_quant_gemm_decode(a, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_pack_weights_decode(const uint8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                                      void* stream) {
  const char* fn = "fp8_pack_weights_decode";
  if (!w || !packed) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (N <= 0 || K <= 0) return fail(FP8BLK_EINVAL, "%s: need N > 0 and K > 0", fn);
  if (N >= kMaxDim || K >= kMaxDim || ldw >= kMaxDim) return fail(FP8BLK_EUNSUPPORTED, "%s: dimension above 2^31", fn);
  if (N % 128 != 0 || K % 128 != 0) return fail(FP8BLK_EUNSUPPORTED, "%s: N and K must be multiples of 128", fn);
  if (N * K > ((int64_t)1 << 40)) return fail(FP8BLK_EUNSUPPORTED, "%s: more than 2^40 weights", fn);
  if (ldw < K) return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  if (!aligned16(w) || !aligned16(packed) || ldw % 16 != 0)
    return fail(FP8BLK_EALIGN, "%s: w and packed must be 16-byte aligned and ldw a multiple of 16", fn);
  const uintptr_t pb = reinterpret_cast<uintptr_t>(packed);
  if (overlap(range2d(w, N, K, ldw, 1), Range{pb, pb + (uintptr_t)(N * K)}))
    return fail(FP8BLK_EINVAL, "%s: packed must not overlap w", fn);
  return hip_status(fp8blk::launch_pack_decode_weights(w, N, K, ldw, packed, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_block_gemm_packed(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                    const float* scale_a, fp8blk_granularity gran_a, int64_t sa_stride_m,
                                    int64_t sa_stride_k, const uint8_t* b_packed, const float* scale_b,
                                    fp8blk_granularity gran_b, int64_t sb_stride_n, int64_t sb_stride_k,
                                    fp8blk_format fmt_a, fp8blk_format fmt_b, void* c, fp8blk_dtype c_dtype,
                                    int64_t ldc, void* stream) {
  const char* fn = "fp8_block_gemm_packed";
  fp8blk::GemmArgs g;
  Range in[4] = {};
  // the packed operand holds N * K contiguous bytes, the range of a row-major
  // [N][K] array with ldb = K
  if (fp8blk_status st = check_gemm_inputs(fn, M, N, K, a, lda, scale_a, gran_a, sa_stride_m, sa_stride_k,
                                           b_packed, K, scale_b, gran_b, sb_stride_n, sb_stride_k, fmt_a, fmt_b,
                                           g, in))
    return st;
  if (M > 64) return fail(FP8BLK_EUNSUPPORTED, "%s: packed weights serve M <= 64 (decode); got M = %lld", fn,
                          (long long)M);
  if (!c) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (c_dtype != FP8BLK_BF16 && c_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown output dtype %d", fn, (int)c_dtype);
  if (ldc < N) return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  const int64_t csz = c_dtype == FP8BLK_BF16 ? 2 : 4;
  if (!aligned16(c)) return fail(FP8BLK_EALIGN, "%s: c must be 16-byte aligned", fn);
  if ((ldc * csz) % 16 != 0) return fail(FP8BLK_EALIGN, "%s: ldc * elem_size must be a multiple of 16 bytes", fn);
  if (M == 0) return ok();
  if (overlaps_any(range2d(c, M, N, ldc, csz), in)) return fail(FP8BLK_EINVAL, "%s: c must not overlap the inputs", fn);
  g.c = c;
  g.c_dtype = (int)c_dtype;
  g.ldc = ldc;
  g.quant_out = 0;
  g.mx = 0;
  g.b_packed = 1;
  return hip_status(fp8blk::launch_block_gemm(g, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_block_gemm_quant(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                   const float* scale_a, fp8blk_granularity gran_a, int64_t sa_stride_m,
                                   int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                                   const float* scale_b, fp8blk_granularity gran_b, int64_t sb_stride_n,
                                   int64_t sb_stride_k, fp8blk_format fmt_a, fp8blk_format fmt_b,
                                   fp8blk_format fmt_c, uint8_t* qc, int64_t ldqc, float* scale_c,
                                   int64_t sc_stride_m, int64_t sc_stride_n, void* stream) {
  const char* fn = "fp8_block_gemm_quant";
  fp8blk::GemmArgs g;
  Range in[4] = {};
  if (fp8blk_status st = check_gemm_inputs(fn, M, N, K, a, lda, scale_a, gran_a, sa_stride_m, sa_stride_k, b,
                                           ldb, scale_b, gran_b, sb_stride_n, sb_stride_k, fmt_a, fmt_b, g, in))
    return st;
  if (!qc || !scale_c) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (fp8blk_status st = check_format(fmt_c, fn)) return st;
  if (ldqc < N) return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  if (sc_stride_m < 0 || sc_stride_n < 0) return fail(FP8BLK_EINVAL, "%s: negative scale stride", fn);
  if (sc_stride_m >= kMaxScaleStride || sc_stride_n >= kMaxScaleStride)
    return fail(FP8BLK_EUNSUPPORTED, "%s: scale stride above 2^40", fn);
  if (!aligned16(qc) || ldqc % 16 != 0)
    return fail(FP8BLK_EALIGN, "%s: qc must be 16-byte aligned and ldqc a multiple of 16", fn);
  if (!aligned4(scale_c)) return fail(FP8BLK_EALIGN, "%s: scale_c must be 4-byte aligned", fn);
  if (M == 0) return ok();
  const int64_t groups = N / 128;
  if (!grid_cells_distinct(M, groups, sc_stride_m, sc_stride_n))
    return fail(FP8BLK_EINVAL, "%s: scale strides map two grid cells to one float", fn);
  const Range rq = range2d(qc, M, N, ldqc, 1);
  const Range rs = range_grid(scale_c, M, groups, sc_stride_m, sc_stride_n);
  if (overlaps_any(rq, in) || overlaps_any(rs, in) || overlap(rq, rs))
    return fail(FP8BLK_EINVAL, "%s: qc and scale_c must not overlap each other or the inputs", fn);
  g.c = nullptr;
  g.c_dtype = (int)FP8BLK_F32;
  g.ldc = ldqc;
  g.quant_out = 1;
  g.mx = 0;
  g.fmt_c = (int)fmt_c;
  g.qc = qc;
  g.sc = scale_c;
  g.sc_m = sc_stride_m;
  g.sc_n = sc_stride_n;
  return hip_status(fp8blk::launch_block_gemm(g, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_quantize_static(const void* x, fp8blk_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                  fp8blk_format fmt, const float* scale, uint8_t* q, int64_t ld_q, float* amax_out,
                                  void* stream) {
  const char* fn = "fp8_quantize_static";
  if (!scale || ((!x || !q) && rows > 0 && cols > 0)) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (x_dtype != FP8BLK_BF16 && x_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown input dtype %d", fn, (int)x_dtype);
  if (fp8blk_status st = check_format(fmt, fn)) return st;
  if (rows < 0 || cols < 0) return fail(FP8BLK_EINVAL, "%s: negative size", fn);
  if (rows >= kMaxDim || cols >= kMaxDim || ld_x >= kMaxDim || ld_q >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: dimension above 2^31", fn);
  if (ld_x < cols || ld_q < cols) return fail(FP8BLK_EINVAL, "%s: leading dimension < cols", fn);
  const int64_t esz = x_dtype == FP8BLK_BF16 ? 2 : 4;
  if (!aligned16(x) || !aligned16(q)) return fail(FP8BLK_EALIGN, "%s: x and q must be 16-byte aligned", fn);
  if ((ld_x * esz) % 16 != 0 || ld_q % 16 != 0)
    return fail(FP8BLK_EALIGN, "%s: ld_x * elem_size and ld_q must be multiples of 16 bytes", fn);
  if (!aligned4(scale) || !aligned4(amax_out))
    return fail(FP8BLK_EALIGN, "%s: scale and amax_out must be 4-byte aligned", fn);
  const Range rsc = range_grid(scale, 1, 1, 0, 0);
  const Range ram = amax_out ? range_grid(amax_out, 1, 1, 0, 0) : Range{0, 0};
  if (amax_out && overlap(rsc, ram)) return fail(FP8BLK_EINVAL, "%s: amax_out must not overlap scale", fn);
  if (rows > 0 && cols > 0) {
    const Range rx = range2d(x, rows, cols, ld_x, esz);
    const Range rq = range2d(q, rows, cols, ld_q, 1);
    if (overlap(rx, rq) || overlap(rq, rsc) || (amax_out && (overlap(rx, ram) || overlap(rq, ram))))
      return fail(FP8BLK_EINVAL, "%s: x, q, scale and amax_out must not overlap", fn);
  }
  fp8blk::QuantArgs a = {};
  a.x = x;
  a.x_dtype = (int)x_dtype;
  a.rows = rows;
  a.cols = cols;
  a.ld_x = ld_x;
  a.fmt = (int)fmt;
  a.q = q;
  a.ld_q = ld_q;
  return hip_status(fp8blk::launch_quantize_static(a, scale, amax_out, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_scale_from_amax_history(const float* history, int64_t n, fp8blk_format fmt, float* scale_out,
                                          void* stream) {
  const char* fn = "fp8_scale_from_amax_history";
  if (!history || !scale_out) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (fp8blk_status st = check_format(fmt, fn)) return st;
  if (n <= 0) return fail(FP8BLK_EINVAL, "%s: the history must hold at least one value", fn);
  if (n >= kMaxDim) return fail(FP8BLK_EUNSUPPORTED, "%s: history longer than 2^31", fn);
  if (!aligned4(history) || !aligned4(scale_out))
    return fail(FP8BLK_EALIGN, "%s: pointers must be 4-byte aligned", fn);
  if (overlap(range_grid(history, 1, n, 0, 1), range_grid(scale_out, 1, 1, 0, 0)))
    return fail(FP8BLK_EINVAL, "%s: scale_out must not overlap the history", fn);
  return hip_status(fp8blk::launch_scale_from_history(history, n, (int)fmt, scale_out, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_quantize_mx(const void* x, fp8blk_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              fp8blk_format fmt, uint8_t* q, int64_t ld_q, uint8_t* scales, int64_t ld_s,
                              void* stream) {
  const char* fn = "fp8_quantize_mx";
  if (!x || !q || !scales) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (x_dtype != FP8BLK_BF16 && x_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown input dtype %d", fn, (int)x_dtype);
  if (fp8blk_status st = check_format(fmt, fn)) return st;
  if (rows < 0 || cols < 0) return fail(FP8BLK_EINVAL, "%s: negative size", fn);
  if (rows >= kMaxDim || cols >= kMaxDim || ld_x >= kMaxDim || ld_q >= kMaxDim || ld_s >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: dimension above 2^31", fn);
  const int64_t nblk = (cols + 31) / 32;
  if (ld_x < cols || ld_q < cols || ld_s < nblk) return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  if (rows * nblk >= kMaxDim) return fail(FP8BLK_EUNSUPPORTED, "%s: more than 2^31 blocks", fn);
  const int64_t esz = x_dtype == FP8BLK_BF16 ? 2 : 4;
  if (!aligned16(x) || !aligned16(q)) return fail(FP8BLK_EALIGN, "%s: x and q must be 16-byte aligned", fn);
  if ((ld_x * esz) % 16 != 0 || ld_q % 16 != 0)
    return fail(FP8BLK_EALIGN, "%s: ld_x * elem_size and ld_q must be multiples of 16 bytes", fn);
  if (rows == 0 || cols == 0) return ok();
  const Range rx = range2d(x, rows, cols, ld_x, esz);
  const Range rq = range2d(q, rows, cols, ld_q, 1);
  const Range rs = range2d(scales, rows, nblk, ld_s, 1);
  if (overlap(rx, rq) || overlap(rx, rs) || overlap(rq, rs))
    return fail(FP8BLK_EINVAL, "%s: x, q and scales must not overlap", fn);
  fp8blk::QuantArgs a = {};
  a.x = x;
  a.x_dtype = (int)x_dtype;
  a.rows = rows;
  a.cols = cols;
  a.ld_x = ld_x;
  a.fmt = (int)fmt;
  a.q = q;
  a.ld_q = ld_q;
  a.scales = reinterpret_cast<float*>(scales);
  a.ss_row = ld_s;
  return hip_status(fp8blk::launch_quantize_mx(a, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* scale_a,
                          int64_t ld_sa, const uint8_t* b, int64_t ldb, const uint8_t* scale_b, int64_t ld_sb,
                          fp8blk_format fmt_a, fp8blk_format fmt_b, void* c, fp8blk_dtype c_dtype, int64_t ldc,
                          void* stream) {
  const char* fn = "fp8_mx_gemm";
  if (!a || !b || !scale_a || !scale_b || !c) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (fp8blk_status st = check_format(fmt_a, fn)) return st;
  if (fp8blk_status st = check_format(fmt_b, fn)) return st;
  if (c_dtype != FP8BLK_BF16 && c_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown output dtype %d", fn, (int)c_dtype);
  if (M < 0 || N <= 0 || K <= 0) return fail(FP8BLK_EINVAL, "%s: need M >= 0, N > 0, K > 0", fn);
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: dimension above 2^31", fn);
  if (N % 128 != 0 || K % 128 != 0)
    return fail(FP8BLK_EUNSUPPORTED, "%s: N and K must be multiples of 128", fn);
  if (lda < K || ldb < K || ldc < N || ld_sa < K / 32 || ld_sb < K / 32)
    return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  if (lda >= kMaxLdCodes || ldb >= kMaxLdCodes || ld_sa >= kMaxLdCodes || ld_sb >= kMaxLdCodes)
    return fail(FP8BLK_EUNSUPPORTED, "%s: leading dimensions must be below 2^23", fn);
  const int64_t csz = c_dtype == FP8BLK_BF16 ? 2 : 4;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c))
    return fail(FP8BLK_EALIGN, "%s: a, b and c must be 16-byte aligned", fn);
  if (lda % 16 != 0 || ldb % 16 != 0 || (ldc * csz) % 16 != 0)
    return fail(FP8BLK_EALIGN, "%s: lda, ldb and ldc * elem_size must be multiples of 16 bytes", fn);
  if ((reinterpret_cast<uintptr_t>(scale_a) & 3u) != 0 || (reinterpret_cast<uintptr_t>(scale_b) & 3u) != 0 ||
      ld_sa % 4 != 0 || ld_sb % 4 != 0)
    return fail(FP8BLK_EALIGN, "%s: scale arrays and their row strides must be 4-byte aligned", fn);
  if (M == 0) return ok();
  const Range in[4] = {range2d(a, M, K, lda, 1), range2d(b, N, K, ldb, 1), range2d(scale_a, M, K / 32, ld_sa, 1),
                       range2d(scale_b, N, K / 32, ld_sb, 1)};
  if (overlaps_any(range2d(c, M, N, ldc, csz), in)) return fail(FP8BLK_EINVAL, "%s: c must not overlap the inputs", fn);
  fp8blk::GemmArgs g = {};
  g.M = M;
  g.N = N;
  g.K = K;
  g.a = a;
  g.lda = lda;
  g.b = b;
  g.ldb = ldb;
  g.gran_a = (int)FP8BLK_PER_TENSOR;
  g.gran_b = (int)FP8BLK_PER_TENSOR;
  g.fmt_a = (int)fmt_a;
  g.fmt_b = (int)fmt_b;
  g.c = c;
  g.c_dtype = (int)c_dtype;
  g.ldc = ldc;
  g.mx = 1;
  g.sa8 = scale_a;
  g.sb8 = scale_b;
  g.ld_sa8 = ld_sa;
  g.ld_sb8 = ld_sb;
  return hip_status(fp8blk::launch_block_gemm(g, static_cast<hipStream_t>(stream)), fn);
}

size_t fp8_kv_decode_attention_workspace_size(int64_t heads_q, int64_t tokens) {
  if (heads_q <= 0 || tokens <= 0) return 0;
  return (size_t)heads_q * (size_t)fp8blk::attention_splits(tokens) * (size_t)fp8blk::attention_partial_floats() *
         sizeof(float);
}

}  // extern "C"

namespace {

// Validation shared by both decode-attention entry points. `workspace` is the
// caller's workspace of `workspace_bytes` bytes, or null for the fixed one
// (then only its capacity is checked). Fills `a` except for a.ws.
fp8blk_status check_attention(const char* fn, const void* q, int64_t ld_q, int64_t heads_q, int64_t heads_kv,
                              int64_t tokens, int64_t head_dim, const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales, int64_t token_block,
                              fp8blk_format fmt, float softmax_scale, void* out, fp8blk_dtype out_dtype,
                              int64_t ld_o, const void* workspace, size_t workspace_bytes, fp8blk::AttnArgs& a) {
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !out)
    return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (fp8blk_status st = check_format(fmt, fn)) return st;
  if (out_dtype != FP8BLK_BF16 && out_dtype != FP8BLK_F32)
    return fail(FP8BLK_EINVAL, "%s: unknown output dtype %d", fn, (int)out_dtype);
  if (heads_q <= 0 || heads_kv <= 0 || tokens <= 0)
    return fail(FP8BLK_EINVAL, "%s: heads_q, heads_kv and tokens must be positive", fn);
  if (heads_q % heads_kv != 0) return fail(FP8BLK_EINVAL, "%s: heads_q must be a multiple of heads_kv", fn);
  if (heads_q / heads_kv > 16) return fail(FP8BLK_EUNSUPPORTED, "%s: more than 16 query heads per kv head", fn);
  if (head_dim != 128) return fail(FP8BLK_EUNSUPPORTED, "%s: head_dim must be 128", fn);
  if (token_block != 128) return fail(FP8BLK_EUNSUPPORTED, "%s: token_block must be 128", fn);
  if (heads_kv >= 65536 || heads_q >= kMaxDim || tokens * 128 >= ((int64_t)1 << 32))
    return fail(FP8BLK_EUNSUPPORTED, "%s: tensor too large", fn);
  if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
    return fail(FP8BLK_EINVAL, "%s: softmax_scale must be finite", fn);
  if (ld_q < head_dim || ld_o < head_dim) return fail(FP8BLK_EINVAL, "%s: leading dimension too small", fn);
  if (!aligned16(q) || ld_q % 8 != 0)
    return fail(FP8BLK_EALIGN, "%s: q must be 16-byte aligned and ld_q a multiple of 8", fn);
  if (!aligned4(out) || !aligned4(workspace) || !aligned4(k_scales) || !aligned4(v_scales))
    return fail(FP8BLK_EALIGN, "%s: out, workspace and scales must be 4-byte aligned", fn);
  const size_t need = fp8_kv_decode_attention_workspace_size(heads_q, tokens);
  if (workspace == nullptr) {
    if (need > fp8blk::attention_scratch_bytes())
      return fail(FP8BLK_EUNSUPPORTED, "%s: needs %zu bytes of workspace; the fixed workspace holds %zu "
                  "(heads_q * ceil(tokens / 1408) <= %zu)", fn, need, fp8blk::attention_scratch_bytes(),
                  fp8blk::attention_scratch_bytes() / ((size_t)fp8blk::attention_partial_floats() * sizeof(float)));
  } else if (workspace_bytes < need) {
    return fail(FP8BLK_EINVAL, "%s: workspace smaller than %zu bytes", fn, need);
  }
  const int64_t nb = (tokens + 127) / 128;
  const int64_t osz = out_dtype == FP8BLK_BF16 ? 2 : 4;
  const Range in[5] = {range2d(q, heads_q, head_dim, ld_q, 2),
                       {reinterpret_cast<uintptr_t>(k_codes), reinterpret_cast<uintptr_t>(k_codes) + (uintptr_t)(heads_kv * tokens * head_dim)},
                       {reinterpret_cast<uintptr_t>(v_codes), reinterpret_cast<uintptr_t>(v_codes) + (uintptr_t)(heads_kv * tokens * head_dim)},
                       range_grid(k_scales, heads_kv, nb, nb, 1), range_grid(v_scales, heads_kv, nb, nb, 1)};
  const Range ro = range2d(out, heads_q, head_dim, ld_o, osz);
  for (const Range& r : in)
    if (overlap(r, ro)) return fail(FP8BLK_EINVAL, "%s: out must not overlap the inputs", fn);
  if (workspace != nullptr) {
    const Range rw = {reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + need};
    for (const Range& r : in)
      if (overlap(r, rw)) return fail(FP8BLK_EINVAL, "%s: workspace must not overlap the inputs", fn);
    if (overlap(ro, rw)) return fail(FP8BLK_EINVAL, "%s: out must not overlap the workspace", fn);
  }
  a = fp8blk::AttnArgs{};
  a.q = q;
  a.ld_q = ld_q;
  a.heads_q = heads_q;
  a.heads_kv = heads_kv;
  a.tokens = tokens;
  a.k = k_codes;
  a.v = v_codes;
  a.sk = k_scales;
  a.sv = v_scales;
  a.fmt = (int)fmt;
  a.softmax_scale = softmax_scale;
  a.out = out;
  a.out_dtype = (int)out_dtype;
  a.ld_o = ld_o;
  return FP8BLK_OK;
}

}  // namespace

extern "C" {

fp8blk_status fp8_kv_decode_attention(const void* q, int64_t ld_q, int64_t heads_q, int64_t heads_kv,
                                      int64_t tokens, int64_t head_dim, const uint8_t* k_codes,
                                      const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                                      int64_t token_block, fp8blk_format fmt, float softmax_scale, void* out,
                                      fp8blk_dtype out_dtype, int64_t ld_o, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const char* fn = "fp8_kv_decode_attention";
  if (!workspace) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  fp8blk::AttnArgs a;
  if (fp8blk_status st = check_attention(fn, q, ld_q, heads_q, heads_kv, tokens, head_dim, k_codes, k_scales,
                                         v_codes, v_scales, token_block, fmt, softmax_scale, out, out_dtype, ld_o,
                                         workspace, workspace_bytes, a))
    return st;
  a.ws = static_cast<float*>(workspace);
  return hip_status(fp8blk::launch_kv_decode_attention(a, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_kv_decode_attention_noalloc(const void* q, int64_t ld_q, int64_t heads_q, int64_t heads_kv,
                                              int64_t tokens, int64_t head_dim, const uint8_t* k_codes,
                                              const float* k_scales, const uint8_t* v_codes,
                                              const float* v_scales, int64_t token_block, fp8blk_format fmt,
                                              float softmax_scale, void* out, fp8blk_dtype out_dtype, int64_t ld_o,
                                              void* stream) {
  const char* fn = "fp8_kv_decode_attention_noalloc";
  fp8blk::AttnArgs a;
  if (fp8blk_status st = check_attention(fn, q, ld_q, heads_q, heads_kv, tokens, head_dim, k_codes, k_scales,
                                         v_codes, v_scales, token_block, fmt, softmax_scale, out, out_dtype, ld_o,
                                         nullptr, 0, a))
    return st;
  // the fixed workspace of the current device (its address is looked up on
  // the first call on each device)
  float* ws = nullptr;
  if (fp8blk_status st = hip_status(fp8blk::attention_scratch(&ws), fn)) return st;
  a.ws = ws;
  return hip_status(fp8blk::launch_kv_decode_attention(a, static_cast<hipStream_t>(stream)), fn);
}

static fp8blk_status check_kv_common(const char* fn, int64_t heads, int64_t tokens, int64_t head_dim,
                                     int64_t token_block, fp8blk_format fmt) {
  if (fp8blk_status st = check_format(fmt, fn)) return st;
  if (heads < 0 || tokens < 0) return fail(FP8BLK_EINVAL, "%s: negative size", fn);
  if (head_dim <= 0 || token_block <= 0)
    return fail(FP8BLK_EINVAL, "%s: head_dim and token_block must be positive", fn);
  if (head_dim % 8 != 0) return fail(FP8BLK_EUNSUPPORTED, "%s: head_dim must be a multiple of 8", fn);
  if (token_block * head_dim > 16384)
    return fail(FP8BLK_EUNSUPPORTED, "%s: token_block * head_dim must be <= 16384", fn);
  if (heads >= 65536 || tokens >= kMaxDim || heads * tokens * head_dim >= ((int64_t)1 << 40))
    return fail(FP8BLK_EUNSUPPORTED, "%s: tensor too large", fn);
  if ((tokens + token_block - 1) / token_block >= kMaxDim)
    return fail(FP8BLK_EUNSUPPORTED, "%s: too many token blocks", fn);
  return FP8BLK_OK;
}

fp8blk_status fp8_kv_quantize(const void* kv, int64_t heads, int64_t tokens, int64_t head_dim,
                              int64_t stride_head, int64_t stride_token, int64_t token_block,
                              fp8blk_format fmt, uint8_t* q, float* scales, void* stream) {
  const char* fn = "fp8_kv_quantize";
  if (!kv || !q || !scales) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (fp8blk_status st = check_kv_common(fn, heads, tokens, head_dim, token_block, fmt)) return st;
  if (stride_token < head_dim || stride_head < 0)
    return fail(FP8BLK_EINVAL, "%s: stride_token must be >= head_dim and stride_head >= 0", fn);
  if (!aligned16(kv) || !aligned16(q)) return fail(FP8BLK_EALIGN, "%s: kv and q must be 16-byte aligned", fn);
  if (!aligned4(scales)) return fail(FP8BLK_EALIGN, "%s: scales must be 4-byte aligned", fn);
  if (stride_head % 8 != 0 || stride_token % 8 != 0)
    return fail(FP8BLK_EALIGN, "%s: strides must be multiples of 8 elements", fn);
  if (heads == 0 || tokens == 0) return ok();
  const int64_t nb = (tokens + token_block - 1) / token_block;
  const uintptr_t kb = reinterpret_cast<uintptr_t>(kv);
  const Range rkv = {kb, kb + (uintptr_t)(((heads - 1) * stride_head + (tokens - 1) * stride_token + head_dim) * 2)};
  const Range rq = {reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + (uintptr_t)(heads * tokens * head_dim)};
  const Range rs = range_grid(scales, heads, nb, nb, 1);
  if (overlap(rkv, rq) || overlap(rkv, rs) || overlap(rq, rs))
    return fail(FP8BLK_EINVAL, "%s: kv, q and scales must not overlap", fn);
  fp8blk::KvArgs a = {};
  a.kv = kv;
  a.heads = heads;
  a.tokens = tokens;
  a.head_dim = head_dim;
  a.stride_head = stride_head;
  a.stride_token = stride_token;
  a.token_block = token_block;
  a.fmt = (int)fmt;
  a.q = q;
  a.scales = scales;
  return hip_status(fp8blk::launch_kv_quantize(a, static_cast<hipStream_t>(stream)), fn);
}

fp8blk_status fp8_kv_dequantize(const uint8_t* q, const float* scales, int64_t heads,
                                int64_t tokens, int64_t head_dim, int64_t token_block,
                                fp8blk_format fmt, void* out_bf16, void* stream) {
  const char* fn = "fp8_kv_dequantize";
  if (!q || !scales || !out_bf16) return fail(FP8BLK_EINVAL, "%s: null pointer", fn);
  if (fp8blk_status st = check_kv_common(fn, heads, tokens, head_dim, token_block, fmt)) return st;
  if (!aligned16(q) || !aligned16(out_bf16))
    return fail(FP8BLK_EALIGN, "%s: q and out must be 16-byte aligned", fn);
  if (!aligned4(scales)) return fail(FP8BLK_EALIGN, "%s: scales must be 4-byte aligned", fn);
  if (heads == 0 || tokens == 0) return ok();
  const int64_t nb = (tokens + token_block - 1) / token_block;
  const int64_t n = heads * tokens * head_dim;
  const Range rq = {reinterpret_cast<uintptr_t>(q), reinterpret_cast<uintptr_t>(q) + (uintptr_t)n};
  const Range ro = {reinterpret_cast<uintptr_t>(out_bf16), reinterpret_cast<uintptr_t>(out_bf16) + (uintptr_t)(2 * n)};
  const Range rs = range_grid(scales, heads, nb, nb, 1);
  if (overlap(ro, rq) || overlap(ro, rs)) return fail(FP8BLK_EINVAL, "%s: out must not overlap q or scales", fn);
  fp8blk::KvArgs a = {};
  a.q_in = q;
  a.scales_in = scales;
  a.heads = heads;
  a.tokens = tokens;
  a.head_dim = head_dim;
  a.token_block = token_block;
  a.fmt = (int)fmt;
  a.out = out_bf16;
  return hip_status(fp8blk::launch_kv_dequantize(a, static_cast<hipStream_t>(stream)), fn);
}

}  // extern "C"
