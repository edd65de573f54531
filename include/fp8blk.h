/*
 * fp8blk -- W8A8 FP8 quantization and block-scaled FP8 GEMM for AMD MI355X (gfx950).
 *
 * C ABI of libfp8blk.so. Plain pointers and sizes only; every device pointer is
 * caller-owned HIP device memory, every call is asynchronous on `stream`
 * (a hipStream_t; NULL means the default stream) and stateless.
 *
 * Sources (the web pages this library implements):
 *   [FP8]   wangyu.me, "大语言模型量化技术（五）：FP8" (LLM quantization part 5: FP8)
 *   [MIXED] charles2530.github.io, "量化：FP8 与混合精度推理：它不是一个 dtype 开关"
 *   [LONG]  pwwt.cn, Llama-3 FP8 and long-context practice notes
 *   [VS]    api.makesence.top, "LLM推理量化:FP8 versus INT8"
 *
 * Numerics shared by every entry point:
 *   - FP8 formats ([FP8] section "FP8 是什么", format table): OCP E4M3 (bias 7,
 *     subnormals, no infinity, S.1111.111 = NaN), largest finite value
 *     MAX = 448; and OCP E5M2 (bias 15, subnormals, S.11111.00 = infinity,
 *     S.11111.{01,10,11} = NaN), largest finite value MAX = 57344.
 *   - Scale of a group: s = fl32(amax / MAX), an IEEE fp32 correctly rounded
 *     division; the stored scale is the dequantization multiplier, x ~ q * s
 *     ([FP8] section "什么是 FP8 量化"; section "权重量化：128×128 分块 FP8").
 *   - Code of an element: the value of the format nearest to fl32(x / s) (the
 *     IEEE fp32 correctly rounded quotient), ties to even, magnitudes >= MAX
 *     saturate to +-MAX (no infinity or NaN code is ever written), the sign of
 *     a zero result is the sign of x. A group with s == 0 gets sign-only zero
 *     codes.
 *   - Denormals are honoured, never flushed.
 *   - Inputs must be finite; non-finite inputs give unspecified codes but never
 *     out-of-bounds accesses.
 *
 * Error behaviour: every argument is checked on the host before any HIP call
 * and before any write, so a call that returns an error leaves all outputs
 * untouched. FP8BLK_EHIP reports a failed kernel launch; device faults surface
 * at the caller's next synchronisation. fp8blk_last_error() gives a per-thread
 * message for the last failing call. No C++ exception crosses this interface.
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BLK_ABI_VERSION 1

typedef enum fp8blk_status {
  FP8BLK_OK = 0,
  FP8BLK_EINVAL = 1,       /* null pointer, negative size, ld < cols, bad enum, aliasing */
  FP8BLK_EALIGN = 2,       /* base pointer or leading dimension not 16-byte aligned */
  FP8BLK_EUNSUPPORTED = 3, /* valid request this version does not implement (e.g. N % 128 != 0) */
  FP8BLK_EHIP = 4          /* the HIP runtime rejected a launch */
} fp8blk_status;

/* FP8 encodings ([FP8] section "FP8 是什么", format table; [VS] section 2 keeps
 * weights and activations in E4M3 and the KV cache in E5M2). Every entry point
 * takes either; the GEMM takes each operand in its own format. */
typedef enum fp8blk_format { FP8BLK_E4M3 = 0, FP8BLK_E5M2 = 1 } fp8blk_format;

/* Scale granularity ([MIXED] section "scale 是控制面"; [FP8] sections
 * "权重量化：128×128 分块 FP8" and "激活动态量化"). */
typedef enum fp8blk_granularity {
  FP8BLK_PER_TENSOR = 0,    /* one scale for the whole tensor; grid [1] */
  FP8BLK_GROUP_1x128 = 1,   /* one row x 128 consecutive columns; grid [rows][ceil(cols/128)] */
  FP8BLK_BLOCK_128x128 = 2  /* 128 rows x 128 columns; grid [ceil(rows/128)][ceil(cols/128)] */
} fp8blk_granularity;

typedef enum fp8blk_dtype { FP8BLK_BF16 = 0, FP8BLK_F32 = 1 } fp8blk_dtype;

/*
 * fp8_quantize -- dynamic quantization of a 2-D tensor to FP8 codes (fmt) plus fp32 scales.
 *
 * Defined by [FP8] section "什么是 FP8 量化" (scale max|x|/448, divide, round to
 * nearest, saturate, keep codes and scale), section "权重量化：128×128 分块 FP8"
 * (128x128 weight blocks, ceil-sized scale grid, fp32 scales) and section
 * "激活动态量化" (per-token activation scales, optionally one per 128-channel
 * group, computed at run time).
 *
 *   x       device, [rows][cols] of x_dtype (bf16 or fp32), row stride ld_x elements.
 *   q       device, uint8 codes of format fmt [rows][cols], row stride ld_q bytes.
 *   scales  device, fp32 scale grid; element (i, j) of the grid lives at
 *           scales[i * scale_stride_row + j * scale_stride_col] (strides in
 *           elements; ignored for PER_TENSOR, whose single scale is scales[0]).
 *           For GROUP_1x128, scale_stride_row = 1 and scale_stride_col = rows
 *           gives the K-block-major layout fp8_block_gemm reads fastest.
 *   Ragged edges (cols or rows not a multiple of 128) form smaller groups.
 *   rows == 0 or cols == 0 is a no-op, except that PER_TENSOR sets scales[0] = 0.
 *
 * Requirements: x, q, scales non-null; rows, cols >= 0; ld_x >= cols and
 * ld_q >= cols; x and q 16-byte aligned, scales 4-byte aligned; ld_x *
 * sizeof(x_dtype) and ld_q multiples of 16 (else FP8BLK_EALIGN); scale strides
 * >= 0 and below 2^40, and such that distinct grid cells are distinct floats
 * (one stride at least the other axis's extent times its stride, as in
 * row-major, K-block-major or padded layouts; else FP8BLK_EINVAL); x, q and
 * scales must not overlap.
 * PER_TENSOR on more than 64K elements keeps per-workgroup maxima in q
 * (below 4 columns: the raw amax in scales[0]) between the call's kernels;
 * codes and scale replace them before the call ends.
 */
fp8blk_status fp8_quantize(const void* x, fp8blk_dtype x_dtype, int64_t rows, int64_t cols,
                           int64_t ld_x, fp8blk_granularity gran, fp8blk_format fmt,
                           uint8_t* q, int64_t ld_q, float* scales, int64_t scale_stride_row,
                           int64_t scale_stride_col, void* stream);

/*
 * fp8_block_gemm -- C[M][N] = A[M][K] . B[N][K]^T from FP8 codes and their scales.
 *
 * Defined by [FP8] section "激活动态量化" (the product is a sum over 128-wide K
 * blocks j of activation scale x weight-block scale x FP8 block product, the
 * scales multiplied back while accumulating) and section "FP8 矩阵乘" (128x128
 * weight blocks, 1x128 activation groups, FP8 products with fp32
 * accumulation); [MIXED] section "混合精度才是生产形态" (low-precision products,
 * higher-precision sums). Computed as
 *   C[m][n] = sum_j s_a(m, j) * s_b(n / 128, j) * P_j[m][n],
 *   P_j[m][n] = sum over the 128 k of block j of dec(a[m][k]) * dec(b[n][k]),
 * with every P_j summed in fp32 from zero and promoted into an fp32 accumulator
 * with one fused multiply-add per K block; the result is rounded once to c_dtype.
 *
 *   a       device, uint8 codes [M][K] of format fmt_a, row stride lda bytes (activations).
 *   scale_a device, fp32. gran_a = PER_TENSOR: scale_a[0]. gran_a = GROUP_1x128:
 *           s_a(m, j) = scale_a[m * sa_stride_m + j * sa_stride_k].
 *   b       device, uint8 codes [N][K] of format fmt_b, row stride ldb bytes (weights W in R^{N x K}).
 *   scale_b device, fp32. gran_b = PER_TENSOR: scale_b[0]. gran_b = BLOCK_128x128:
 *           s_b(nb, j) = scale_b[nb * sb_stride_n + j * sb_stride_k]
 *           (the ceil(N/128) x ceil(K/128) weight_scale_inv grid).
 *   c       device, [M][N] of c_dtype (BF16 output, or F32 for verification),
 *           row stride ldc elements.
 *
 * Requirements: pointers non-null; M >= 0 (M == 0 is a no-op); N > 0, K > 0,
 * N % 128 == 0 and K % 128 == 0 (else FP8BLK_EUNSUPPORTED); lda, ldb >= K and
 * below 2^23 (else FP8BLK_EUNSUPPORTED);
 * ldc >= N; a, b, c 16-byte aligned and lda, ldb, ldc * sizeof(c_dtype)
 * multiples of 16; scale_a and scale_b 4-byte aligned, their strides >= 0 and
 * below 2^40 (a zero stride broadcasts one scale along that axis), and each
 * block-scaled grid spanning less than 4 GiB, i.e. (offset of its last cell +
 * 1) * 4 < 2^32 (else FP8BLK_EUNSUPPORTED);
 * gran_a in {PER_TENSOR, GROUP_1x128}; gran_b in {PER_TENSOR,
 * BLOCK_128x128}; fmt_a, fmt_b in {E4M3, E5M2} (independently); codes must be
 * finite (E4M3: not S.1111.111; E5M2: exponent field not 11111), as every
 * code fp8_quantize writes is; c must not overlap the inputs.
 */
fp8blk_status fp8_block_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                             const float* scale_a, fp8blk_granularity gran_a, int64_t sa_stride_m,
                             int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                             const float* scale_b, fp8blk_granularity gran_b, int64_t sb_stride_n,
                             int64_t sb_stride_k, fp8blk_format fmt_a, fp8blk_format fmt_b,
                             void* c, fp8blk_dtype c_dtype, int64_t ldc, void* stream);

/*
 * fp8_block_gemm_quant -- fp8_block_gemm whose output is quantized in the same
 * kernel: C = A . B^T computed exactly as fp8_block_gemm computes its fp32
 * output, then written as FP8 codes of format fmt_c with one fp32 scale per
 * row and 128-column group, i.e. the 1 x 128 activation quantization of
 * fp8_quantize (GROUP_1x128) applied to that fp32 C.
 *
 * Defined by [FP8] section "激活动态量化" (activations of the next matrix
 * multiply get one scale per token and 128-channel group, computed at run
 * time) on top of the product fp8_block_gemm defines; the output of one layer
 * is the activation of the next, so quantizing it where it is produced
 * replaces a separate pass over a bf16 copy of it.
 *
 *   Inputs, their layouts and requirements: as fp8_block_gemm.
 *   qc      device, uint8 codes [M][N] of format fmt_c, row stride ldqc bytes.
 *   scale_c device, fp32 grid [M][N / 128]; element (m, g) at
 *           scale_c[m * sc_stride_m + g * sc_stride_n]. sc_stride_m = 1 and
 *           sc_stride_n = M give the K-block-major layout fp8_block_gemm reads
 *           fastest when qc is the next GEMM's A.
 *
 * Requirements: as fp8_block_gemm for the inputs; qc and scale_c non-null; qc
 * 16-byte aligned, ldqc >= N and a multiple of 16; scale_c 4-byte aligned;
 * strides >= 0 and below 2^40, and such that distinct grid cells are distinct
 * floats (as for fp8_quantize); qc and scale_c must not overlap each other or
 * the inputs. For M > 64 the results are bit-identical to fp8_quantize(GROUP_1x128)
 * of the fp32 output of fp8_block_gemm on the same inputs (the same kernel
 * and summation order). For M <= 64 this entry point still runs that kernel,
 * while fp8_block_gemm takes a split-K kernel whose fp32 sums may differ in
 * the last bits; both meet the same tolerance.
 */
fp8blk_status fp8_block_gemm_quant(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                   const float* scale_a, fp8blk_granularity gran_a, int64_t sa_stride_m,
                                   int64_t sa_stride_k, const uint8_t* b, int64_t ldb,
                                   const float* scale_b, fp8blk_granularity gran_b, int64_t sb_stride_n,
                                   int64_t sb_stride_k, fp8blk_format fmt_a, fp8blk_format fmt_b,
                                   fp8blk_format fmt_c, uint8_t* qc, int64_t ldqc, float* scale_c,
                                   int64_t sc_stride_m, int64_t sc_stride_n, void* stream);

/*
 * fp8_quantize_gemm_decode -- dynamic quantization of a decode step's
 * activations inside the block-scaled GEMM that consumes them, in one launch
 * (M <= 64): C = fp8_block_gemm(fp8_quantize(x, gran_a, fmt_a), W).
 *
 * The activation scales are taken at run time, just before the matmul that
 * consumes the codes ([FP8] wangyu.me, "大语言模型量化技术（五）：FP8", section
 * "激活动态量化"): per tensor, or per token and 128-channel group; s =
 * fl32(amax(|x|) / MAX) and q = FP8(fl32(x / s)) with the saturating
 * round-to-nearest-even cast. At decode shapes the GEMM is bound by streaming
 * the weights from HBM, and each of its workgroups quantizes the activation
 * fragments it multiplies in registers: a 1x128 group lies within one
 * fragment, and a per-tensor max is taken by every workgroup over the whole,
 * small, tensor. Codes, scales and C are bit-identical to fp8_quantize(x,
 * gran_a, fmt_a) followed by fp8_block_gemm (row-major weights) or
 * fp8_block_gemm_packed (b_packed = 1) on those codes and scales.
 *
 *   x          device, [M][ld_x] of x_dtype (BF16 or F32), row-major.
 *   gran_a     PER_TENSOR or GROUP_1x128.
 *   fmt_a      format of the activation codes.
 *   b, ldb     device weight codes: row-major [N][ldb] bytes (b_packed = 0),
 *              or the decode-packed layout of fp8_pack_weights_decode
 *              (b_packed = 1; ldb is then ignored).
 *   scale_b, gran_b, sb_stride_n, sb_stride_k, fmt_b
 *              the weight scales and format, as for fp8_block_gemm.
 *   c          device, [M][ldc] of c_dtype (BF16 or F32).
 *   q_out      device, [M][ld_q] uint8, or NULL: if given, the activation
 *              codes, as fp8_quantize writes them.
 *   scale_out  device fp32, or NULL: if given, the activation scales, as
 *              fp8_quantize writes them: scale_out[0] for PER_TENSOR; for
 *              GROUP_1x128 the [M][K / 128] grid at
 *              scale_out[m * so_stride_m + j * so_stride_k] (the strides are
 *              ignored for PER_TENSOR).
 *
 * Requirements: x, b, scale_b, c non-null; 1 <= M <= 64 (M < 1: FP8BLK_EINVAL;
 * M > 64: FP8BLK_EUNSUPPORTED, prefill shapes take the two calls); N, K
 * positive multiples of 128 below 2^31; PER_TENSOR needs M * K <= 65536 (else
 * FP8BLK_EUNSUPPORTED); b_packed 0 or 1; ld_x >= K, x 16-byte aligned and
 * ld_x * elem_size a multiple of 16; the weights' and C's requirements of
 * fp8_block_gemm; q_out, if given, 16-byte aligned with ld_q >= K a multiple
 * of 16; scale_out 4-byte aligned, its strides >= 0, below 2^40 and mapping
 * distinct grid cells to distinct floats. The outputs must not overlap the
 * inputs or each other. Any failure is reported before anything is written.
 */
fp8blk_status fp8_quantize_gemm_decode(const void* x, fp8blk_dtype x_dtype, int64_t M, int64_t N, int64_t K,
                                       int64_t ld_x, fp8blk_granularity gran_a, fp8blk_format fmt_a,
                                       const uint8_t* b, int64_t ldb, int b_packed, const float* scale_b,
                                       fp8blk_granularity gran_b, int64_t sb_stride_n, int64_t sb_stride_k,
                                       fp8blk_format fmt_b, void* c, fp8blk_dtype c_dtype, int64_t ldc,
                                       uint8_t* q_out, int64_t ld_q, float* scale_out, int64_t so_stride_m,
                                       int64_t so_stride_k, void* stream);

/*
 * fp8_pack_weights_decode -- copy row-major weight codes into the
 * decode-packed layout read by fp8_block_gemm_packed.
 *
 * The weights of a decode step (a handful of tokens, M <= 64) are streamed
 * from HBM once per call, so their memory order decides the GEMM's speed. The
 * method fixes the codes and their 128 x 128 block scales ([FP8] section
 * "FP8 矩阵乘": the weights are cut into 128 x 128 blocks and quantized ahead
 * of time, offline) but not their order in memory; this is a one-time, offline
 * reordering of the same bytes, done after fp8_quantize(BLOCK_128x128). The
 * scales are unchanged.
 *
 *   w       device, uint8 codes [N][K], row stride ldw bytes.
 *   packed  device, N * K bytes, caller-owned. One 2 KB block per (16-row
 *           group rg, 128-wide K block kb), blocks stored K-block-major at byte
 *           (kb * N / 16 + rg) * 2048. Inside a block, byte e (0..15) of half h
 *           (0, 1) of lane l = r + 16 g (r 0..15, g 0..3) is at h * 1024 + 16 l + e
 *           and holds w[16 rg + r][128 kb + 32 g + 16 h + e].
 *
 * Requirements: pointers non-null; N > 0, K > 0, both multiples of 128 and
 * below 2^31, N * K <= 2^40 (else FP8BLK_EUNSUPPORTED); ldw >= K; w, packed
 * 16-byte aligned and ldw a multiple of 16; packed must not overlap w.
 */
fp8blk_status fp8_pack_weights_decode(const uint8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                                      void* stream);

/*
 * fp8_block_gemm_packed -- fp8_block_gemm for M <= 64 with the weights in the
 * decode-packed layout of fp8_pack_weights_decode.
 *
 * The product, its numerics and every other argument are those of
 * fp8_block_gemm ([FP8] sections "激活动态量化" and "FP8 矩阵乘"); the result
 * is bit-identical to fp8_block_gemm on the row-major codes the packed array
 * was made from (the same kernel and summation order, only the weight loads
 * are addressed differently). In the packed order all workgroups read one
 * K block's N * 128 bytes at a time instead of reads spread over the whole
 * matrix.
 *
 *   b_packed device, N * K bytes written by fp8_pack_weights_decode(N, K).
 *
 * Requirements: as fp8_block_gemm, with ldb taken as K; M <= 64 (else
 * FP8BLK_EUNSUPPORTED: prefill shapes take fp8_block_gemm); M == 0 is a no-op.
 */
fp8blk_status fp8_block_gemm_packed(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda,
                                    const float* scale_a, fp8blk_granularity gran_a, int64_t sa_stride_m,
                                    int64_t sa_stride_k, const uint8_t* b_packed, const float* scale_b,
                                    fp8blk_granularity gran_b, int64_t sb_stride_n, int64_t sb_stride_k,
                                    fp8blk_format fmt_a, fp8blk_format fmt_b, void* c, fp8blk_dtype c_dtype,
                                    int64_t ldc, void* stream);

/*
 * fp8_kv_quantize -- FP8 KV-cache quantization with one scale per (head, token block).
 *
 * Defined by [LONG] section 1 (K and V quantized to FP8 with separate scales)
 * and section 3 (finer KV granularity: per head and per 128-token block, so
 * that small late-position keys keep their precision); [MIXED] section
 * "scale 是控制面" (per-head scales). Same per-group arithmetic as fp8_quantize,
 * in format fmt (E5M2 is the KV format of [VS] section 2). Call once for K
 * and once for V.
 *
 *   kv      device, bf16 [heads][tokens][head_dim]; element (h, t, d) at
 *           kv[h * stride_head + t * stride_token + d] (strides in elements,
 *           head_dim contiguous).
 *   q       device, dense uint8 codes of format fmt [heads][tokens][head_dim].
 *   scales  device, dense fp32 [heads][ceil(tokens / token_block)].
 *   A group is one head, token_block consecutive tokens (fewer in the ragged
 *   last block) and all of head_dim.
 *
 * Requirements: pointers non-null; heads, tokens >= 0 (0 is a no-op);
 * head_dim > 0 and a multiple of 8; token_block > 0 and token_block * head_dim
 * <= 16384 (else FP8BLK_EUNSUPPORTED); kv and q 16-byte aligned, scales
 * 4-byte aligned; stride_head and stride_token multiples of 8 with
 * stride_token >= head_dim; outputs must not overlap the input.
 */
fp8blk_status fp8_kv_quantize(const void* kv, int64_t heads, int64_t tokens, int64_t head_dim,
                              int64_t stride_head, int64_t stride_token, int64_t token_block,
                              fp8blk_format fmt, uint8_t* q, float* scales, void* stream);

/*
 * fp8_kv_dequantize -- out = bf16(fl32(dec(q) * s)), round to nearest even.
 *
 * Defined by [MIXED] section "E4M3 和 E5M2 是范围与格点的取舍" (dequantization
 * multiplies the FP8 value by its scale) and [FP8] section "什么是 FP8 量化"
 * (x ~ q * s). Layouts are those fp8_kv_quantize writes; fmt must be the
 * format the codes were written in; out is dense bf16 [heads][tokens][head_dim].
 *
 * Requirements as fp8_kv_quantize; out must not overlap q or scales.
 */
fp8blk_status fp8_kv_dequantize(const uint8_t* q, const float* scales, int64_t heads,
                                int64_t tokens, int64_t head_dim, int64_t token_block,
                                fp8blk_format fmt, void* out_bf16, void* stream);

/*
 * fp8_quantize_static -- quantization with a caller-supplied per-tensor scale
 * (static scaling, or delayed scaling with a scale derived from past amax
 * values), optionally recording the tensor's own amax.
 *
 * Defined by [MIXED] section "scale 是控制面" (the scale can come from recorded
 * history instead of the current batch: Transformer Engine's delayed scaling
 * updates it from past amax statistics) and [VS] section 2 (delayed scaling in
 * the FP8 forward pass); the cast is that of fp8_quantize: the code of the
 * format value nearest to fl32(x / s), ties to even, saturating at +-MAX, the
 * sign of a zero result that of x. s = scale[0] is read on the device and must
 * be positive and finite (0 gives sign-only zero codes; other values give
 * unspecified codes).
 *
 *   x, q        as fp8_quantize.
 *   scale       device, one float, the dequantization multiplier s.
 *   amax_out    device, one float, or NULL: receives max |x| over the tensor
 *               (0 for an empty tensor), to append to the caller's history.
 *
 * Requirements: as fp8_quantize for x and q, except that x and q may be NULL
 * when rows or cols is 0 (then only amax_out is written); scale and amax_out
 * 4-byte aligned and not overlapping each other, x or q. With amax_out, q
 * holds per-workgroup maxima in a few 4-byte slots between the call's two
 * kernels; the final codes replace them before the call ends.
 */
fp8blk_status fp8_quantize_static(const void* x, fp8blk_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                  fp8blk_format fmt, const float* scale, uint8_t* q, int64_t ld_q, float* amax_out,
                                  void* stream);

/*
 * fp8_scale_from_amax_history -- scale_out[0] = fl32(max_i history[i] / MAX)
 * (MAX = 448 for E4M3, 57344 for E5M2): the delayed-scaling scale from a
 * window of recorded amax values ([MIXED] section "scale 是控制面"; the same
 * division as fp8_quantize's per-tensor scale).
 *
 *   history     device, n >= 1 non-negative floats.
 *   scale_out   device, one float.
 */
fp8blk_status fp8_scale_from_amax_history(const float* history, int64_t n, fp8blk_format fmt, float* scale_out,
                                          void* stream);

/*
 * fp8_quantize_mx -- MX quantization: FP8 codes with one power-of-two scale per
 * 32 consecutive elements of a row.
 *
 * Defined by [VS] section 3 (Microscaling formats: blocks of 32 elements share
 * one scale; block-scaled hardware runs them natively) and [FP8] section
 * "什么是 FP8 量化" (map into the format's range, round to nearest even,
 * saturate). The scale of a block is X = 2^k with k the smallest integer such
 * that max|x| <= MAX * 2^k over the block (MAX = 448 for E4M3, 57344 for
 * E5M2), clamped to [-127, 127] (an all-zero block gets k = -127); it is stored
 * as the E8M0 byte k + 127. Codes are FP8(x * 2^-k): the scaling is exact, so
 * the encoder's rounding (nearest, ties to even) is the only one.
 *
 *   x       device, [rows][cols] of x_dtype, row stride ld_x elements.
 *   q       device, uint8 codes of format fmt [rows][cols], row stride ld_q bytes.
 *   scales  device, uint8 E8M0 bytes [rows][ceil(cols / 32)], row stride ld_s bytes
 *           (the ragged last block of a row uses its valid elements).
 *
 * Requirements: pointers non-null; rows, cols >= 0 (0 is a no-op); ld_x, ld_q
 * >= cols and ld_s >= ceil(cols / 32); x and q 16-byte aligned with
 * ld_x * sizeof(x_dtype) and ld_q multiples of 16; x, q and scales must not
 * overlap.
 */
fp8blk_status fp8_quantize_mx(const void* x, fp8blk_dtype x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              fp8blk_format fmt, uint8_t* q, int64_t ld_q, uint8_t* scales, int64_t ld_s,
                              void* stream);

/*
 * fp8_mx_gemm -- C[M][N] = A[M][K] . B[N][K]^T from MX operands: each operand's
 * codes with one E8M0 scale per 32 K elements of each row (as fp8_quantize_mx
 * writes them for A [M][K] and for the weights B [N][K]).
 *
 * Defined by [VS] section 3 (block-32 scaled formats multiplied natively by
 * the hardware) on the product of [FP8] section "FP8 矩阵乘" (FP8 products,
 * fp32 accumulation):
 *   C[m][n] = sum_k dec(a[m][k]) 2^(sa[m][k/32] - 127) * dec(b[n][k]) 2^(sb[n][k/32] - 127),
 * the scales applied inside the matrix instruction (gfx950's scaled FP8 MFMA),
 * summed in fp32 and rounded once to c_dtype.
 *
 *   a, b     device, uint8 codes of formats fmt_a / fmt_b, row strides lda / ldb bytes.
 *   scale_a  device, uint8 [M][ld_sa] (ld_sa >= K / 32); scale_b likewise [N][ld_sb].
 *   c        device, [M][N] of c_dtype (BF16 or F32), row stride ldc elements.
 *
 * Requirements: pointers non-null; M >= 0 (0 is a no-op), N > 0, K > 0, N and K
 * multiples of 128 (else FP8BLK_EUNSUPPORTED); lda, ldb >= K, ldc >= N, all
 * leading dimensions below 2^23; a, b, c 16-byte aligned with lda, ldb and
 * ldc * sizeof(c_dtype) multiples of 16; scale arrays 4-byte aligned with ld_sa
 * and ld_sb multiples of 4; codes finite; scale bytes not 0xFF; c must not
 * overlap the inputs.
 */
fp8blk_status fp8_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a, int64_t lda, const uint8_t* scale_a,
                          int64_t ld_sa, const uint8_t* b, int64_t ldb, const uint8_t* scale_b, int64_t ld_sb,
                          fp8blk_format fmt_a, fp8blk_format fmt_b, void* c, fp8blk_dtype c_dtype, int64_t ldc,
                          void* stream);

/*
 * fp8_kv_decode_attention -- one decode step of attention over the FP8 KV cache
 * that fp8_kv_quantize writes (grouped-query attention, one query token).
 *
 * Defined by [LONG] section 1 (K and V kept in FP8, each with its own scales,
 * and dequantized where attention reads them) and section 3 (per head and
 * per 128-token scales); [MIXED] section "scale 是控制面" (per-head KV scales
 * read by the attention backend). For query head g (kv head h = g / G,
 * G = heads_q / heads_kv):
 *   s_t  = softmax_scale * sum_d q[g][d] * dec(k[h][t][d]) * k_scales[h][t / 128]
 *   p_t  = exp(s_t - max_t s_t) / sum_t exp(s_t - max_t s_t)
 *   o[g][d] = sum_t p_t * dec(v[h][t][d]) * v_scales[h][t / 128]
 * computed in fp32 (scores, softmax, accumulation) from exactly converted
 * codes; each output is within 1e-3 * sum_t p_t |dec(v[h][t][d]) * v_scale|
 * of the exact value (plus half a bf16 ulp for bf16 output).
 *
 *   q          device, bf16 [heads_q][ld_q] (head_dim contiguous).
 *   k_codes, v_codes
 *              device, dense uint8 codes [heads_kv][tokens][head_dim] of format fmt.
 *   k_scales, v_scales
 *              device, dense fp32 [heads_kv][ceil(tokens / token_block)].
 *   out        device, [heads_q][ld_o] of out_dtype (BF16 or F32).
 *   workspace  device, caller-owned scratch of at least
 *              fp8_kv_decode_attention_workspace_size(heads_q, tokens) bytes;
 *              its contents on entry do not matter and on return are unspecified.
 *
 * Requirements: pointers non-null; heads_q, heads_kv, tokens > 0; heads_q a
 * multiple of heads_kv with at most 16 query heads per kv head; head_dim == 128
 * and token_block == 128 (else FP8BLK_EUNSUPPORTED); softmax_scale finite;
 * q 16-byte aligned, ld_q >= 128 and a multiple of 8; out, scales and
 * workspace 4-byte aligned; ld_o >= 128; out and workspace must not overlap
 * the inputs or each other. Calls that share a workspace must not overlap in
 * time.
 */
size_t fp8_kv_decode_attention_workspace_size(int64_t heads_q, int64_t tokens);
fp8blk_status fp8_kv_decode_attention(const void* q, int64_t ld_q, int64_t heads_q, int64_t heads_kv,
                                      int64_t tokens, int64_t head_dim, const uint8_t* k_codes,
                                      const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                                      int64_t token_block, fp8blk_format fmt, float softmax_scale, void* out,
                                      fp8blk_dtype out_dtype, int64_t ld_o, void* workspace,
                                      size_t workspace_bytes, void* stream);

/*
 * fp8_kv_decode_attention_noalloc -- fp8_kv_decode_attention with a fixed
 * workspace inside the library instead of a caller-owned one, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops that must not call the allocator, harnesses that forbid it). It calls
 * no allocator: the split partials live in a file-scope device array of
 * 12 MiB, one per device, kept until the process ends.
 *
 * Arguments, numerics, results and requirements: those of
 * fp8_kv_decode_attention without the workspace (the same kernels, so the
 * outputs are bit-identical). The partials need
 * fp8_kv_decode_attention_workspace_size(heads_q, tokens) <= 12 MiB, i.e.
 * heads_q * ceil(tokens / 1408) <= 24197 (else FP8BLK_EUNSUPPORTED, before any
 * HIP call). The first call on a device looks up the array's address there
 * (FP8BLK_EHIP if that fails). Every call on one device uses the same array:
 * calls that overlap in time on one device (other streams, other threads)
 * race and give unspecified results; its contents between calls do not matter.
 */
fp8blk_status fp8_kv_decode_attention_noalloc(const void* q, int64_t ld_q, int64_t heads_q, int64_t heads_kv,
                                              int64_t tokens, int64_t head_dim, const uint8_t* k_codes,
                                              const float* k_scales, const uint8_t* v_codes,
                                              const float* v_scales, int64_t token_block, fp8blk_format fmt,
                                              float softmax_scale, void* out, fp8blk_dtype out_dtype, int64_t ld_o,
                                              void* stream);

/* Human-readable name of a status code (static storage). */
const char* fp8blk_status_string(fp8blk_status s);
/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* fp8blk_last_error(void);
/* FP8BLK_ABI_VERSION of the loaded library. */
int fp8blk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
