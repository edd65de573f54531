// Internal interface between the C-ABI layer (api.hip) and the kernel
// launchers (quantize.hip, gemm.hip). Arguments reaching a launcher have been
// validated on the host.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

enum Gran : int { GRAN_PER_TENSOR = 0, GRAN_GROUP_1x128 = 1, GRAN_BLOCK_128x128 = 2 };
enum DType : int { DTYPE_BF16 = 0, DTYPE_F32 = 1 };
// FP8 encodings; the values are also the operand-format selectors of the
// gfx950 f8f6f4 MFMA (0 = E4M3, 1 = E5M2).
enum Fmt : int { FMT_E4M3 = 0, FMT_E5M2 = 1 };

struct QuantArgs {
  const void* x;
  int x_dtype;
  int64_t rows, cols, ld_x;
  int gran;
  int fmt;
  uint8_t* q;
  int64_t ld_q;
  float* scales;
  int64_t ss_row, ss_col;
};

struct KvArgs {
  const void* kv;        // quantize input
  const uint8_t* q_in;   // dequantize input
  int64_t heads, tokens, head_dim, stride_head, stride_token, token_block;
  int fmt;
  uint8_t* q;            // quantize output
  float* scales;         // quantize output / dequantize input
  const float* scales_in;
  void* out;             // dequantize output
};

struct GemmArgs {
  int64_t M, N, K;
  const uint8_t* a;
  int64_t lda;
  const float* sa;
  int gran_a;
  int64_t sa_m, sa_k;
  const uint8_t* b;
  int64_t ldb;
  const float* sb;
  int gran_b;
  int64_t sb_n, sb_k;
  void* c;
  int c_dtype;
  int64_t ldc;          // row stride of c, or of qc (bytes) when quant_out
  int fmt_a, fmt_b;
  // quant_out: instead of c, write the output as FP8 codes of format fmt_c
  // (qc) with one fp32 scale per row and 128-column group at
  // sc[row * sc_m + group * sc_n]
  // mx: operands carry E8M0 scale bytes (one per 32 K elements) in sa8 / sb8
  // with row strides ld_sa8 / ld_sb8 bytes; sa, sb, gran_a, gran_b unused
  int mx;
  const uint8_t* sa8;
  const uint8_t* sb8;
  int64_t ld_sa8, ld_sb8;
  int quant_out;
  int fmt_c;
  uint8_t* qc;
  float* sc;
  int64_t sc_m, sc_n;
  // b_packed: b is in the decode-packed layout written by
  // launch_pack_decode_weights (ldb unused); M <= 64, bf16 or fp32 output
  int b_packed;
};

// Dynamic activation quantization inside the decode GEMM: g holds M (<= 64),
// N, K, the weights (row-major, or decode-packed with packed != 0), their
// scales and the output as for launch_block_gemm (g.fmt_a is the format of
// the activation codes); x [M][ld_x] of x_dtype; gran_a GRAN_PER_TENSOR
// (M * K <= 65536) or GRAN_GROUP_1x128; q_out (row stride ld_q) and s_out
// (per tensor: s_out[0]; 1x128: s_out[m * so_m + j * so_k]) may be null.
struct QuantGemmDecodeArgs {
  GemmArgs g;
  const void* x;
  int x_dtype;
  int64_t ld_x;
  int gran_a;
  int packed;
  uint8_t* q_out;
  int64_t ld_q;
  float* s_out;
  int64_t so_m;
  int64_t so_k;
};

struct AttnArgs {
  const void* q;          // bf16 [heads_q][ld_q]
  int64_t ld_q;
  int64_t heads_q, heads_kv, tokens;
  const uint8_t* k;       // codes [heads_kv][tokens][128]
  const uint8_t* v;
  const float* sk;        // [heads_kv][ceil(tokens / 128)]
  const float* sv;
  int fmt;
  float softmax_scale;
  float* ws;              // attention_splits(tokens) * heads_q * attention_partial_floats() floats
  void* out;              // [heads_q][ld_o] of out_dtype
  int out_dtype;
  int64_t ld_o;
};

// Token splits of the decode attention and the workspace floats per (query
// head, split).
int attention_splits(int64_t tokens);
int64_t attention_partial_floats();
// The fixed decode-attention workspace (a device array of attention_scratch_bytes()
// bytes, one per device): its device address on the current device.
size_t attention_scratch_bytes();
hipError_t attention_scratch(float** ptr);

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);
// MX blocks of 32 along the rows: a.scales points at uint8 E8M0 bytes, a.ss_row
// is the byte stride between their rows.
hipError_t launch_quantize_mx(const QuantArgs& a, hipStream_t st);
// Codes under a caller-supplied scale (scale[0], device); amax_out (device,
// may be null) receives max|x| of the tensor.
hipError_t launch_quantize_static(const QuantArgs& a, const float* scale, float* amax_out, hipStream_t st);
hipError_t launch_scale_from_history(const float* history, int64_t n, int fmt, float* scale_out, hipStream_t st);
hipError_t launch_kv_decode_attention(const AttnArgs& a, hipStream_t st);
hipError_t launch_kv_quantize(const KvArgs& a, hipStream_t st);
hipError_t launch_kv_dequantize(const KvArgs& a, hipStream_t st);
hipError_t launch_block_gemm(const GemmArgs& a, hipStream_t st);
hipError_t launch_quant_gemm_decode(const QuantGemmDecodeArgs& a, hipStream_t st);
// Row-major weight codes [N][ldw] (N % 16 == 0, K % 128 == 0) to the
// decode-packed layout: 2 KB per (16-row group rg, K block kb) at
// (kb * N / 16 + rg) * 2048.
hipError_t launch_pack_decode_weights(const uint8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                                      hipStream_t st);

}  // namespace fp8blk
