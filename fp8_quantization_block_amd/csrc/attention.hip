// Decode attention over an FP8 KV cache (one query token per head).
//
// o[g] = sum_t softmax_t(c * q[g] . k_hat[h, t]) v_hat[h, t], h = g / G, with
// k_hat = dec(k codes) * s_k(h, t / 128) and v_hat likewise: the consumer of
// the KV cache that fp8_kv_quantize writes. [LONG] pwwt.cn Llama-3 FP8 notes,
// section 1 (K and V stored in FP8 with their own scales, dequantized when
// attention reads them) and section 3 (per head and per 128-token scales);
// [MIXED] charles2530.github.io, "量化：FP8 与混合精度推理", section "scale 是控制面"
// (KV-cache scales per head, read by the attention backend).
//
// Design (gfx950), one workgroup of 4 waves per (kv head, 1408-token split),
// 48 KB of LDS each, three workgroups per compute unit (for the 8 x 131072
// cache: 94 splits x 8 heads = 752 workgroups, one round on 256 compute
// units; measured 48.1 us against 51.7 us for 2048-token splits with K and V
// both staged in the LDS, two workgroups per compute unit):
// * Each wave streams its 352 tokens in 32-token units, two units ahead of
//   the one it computes (16 KB of codes in flight per wave, 192 KB per compute
//   unit): the K codes of a unit go straight into registers (each lane loads
//   the 32 bytes of a key that it multiplies), the V codes into a ring of 3
//   LDS stages of the wave's own by direct global -> LDS copies; both carry
//   the non-temporal hint. Keeping K out of the LDS is what lets three
//   workgroups share a compute unit. V rows are 128 bytes; logical 16-byte
//   chunk c of row r is stored at c ^ (r % 8), so that 16 lanes reading one
//   chunk of 16 consecutive rows hit distinct banks. The kernel is bound by
//   reading the codes from HBM.
// * Scores S^T = K Q^T on the bf16 MFMA (16 x 16 x 32): FP8 codes convert to
//   bf16 exactly and the query is bf16; the 16 MFMA columns are the G query
//   heads that share the kv head (G <= 16). Head_dim is permuted the same way
//   in both operands, so that a lane reads 32 contiguous bytes of a key.
// * Softmax in fp32, base 2 (scores multiplied by c * s_k * log2 e), online
//   over units: running max m, running sum l, rescaled output.
// * O^T += V^T P^T on the bf16 MFMA: V codes are read transposed from LDS by
//   ds_read_b64_tr_b8 (in each 16-lane group, lane j receives byte j % 8 of
//   the 8-byte rows addressed by lanes 2 i + j / 8, i = 0..7); P' = P * s_v is
//   split into two bf16 terms (hi + lo: 16 significant bits), so that the
//   products carry the fp32 softmax weights to within 2^-16 relative.
// * The 4 waves' (m, l, O) are merged through LDS into one partial per
//   workgroup; a second kernel merges the splits of each query head.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace fp8blk {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v2i lds_v2i;

constexpr int kD = 128;                    // head_dim
constexpr int kWaves = 4;
constexpr int kThreadsA = kWaves * 64;
constexpr int kUnit = 32;                  // tokens per unit
constexpr int kSub = kUnit / 16;           // 16-token subtiles per unit
constexpr int kUnitsPerWave = 11;          // 352 tokens per wave
constexpr int kStages = 3;                 // V stages per wave (2 units in flight)
constexpr int kSplitTokens = kWaves * kUnitsPerWave * kUnit;   // 1408
constexpr int kUnitBytes = kUnit * kD;     // 4 KB of codes per tensor
constexpr int kCopies = kUnitBytes / 1024; // 1 KB copies per tensor and unit
constexpr int kPartial = kD + 2;           // floats per (query head, split): O[128], m, l
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;        // running max before any token (finite)

struct AttnParams {
  const __hip_bfloat16* q;   // [Hq][ld_q]
  const uint8_t* k;          // [Hkv][T][128]
  const uint8_t* v;
  const float* sk;           // [Hkv][nb]
  const float* sv;
  float* ws;                 // [Hq][splits][kPartial]
  void* out;                 // [Hq][ld_o]
  int64_t ld_q, ld_o;
  int T, nb, G, splits;
  float c_log2;              // softmax scale * log2 e
};

// 8 codes (two words) -> 8 bf16, exact (an FP8 value has at most 4
// significant bits and an exponent inside bf16's range): gfx950's packed
// conversion, two codes per instruction, with a unit scale (checked against
// the decode tables on every code of both formats).
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

template <int kFmt>
__device__ __forceinline__ v2bf cvt2_bf16(uint32_t w, bool hi) {
  if constexpr (kFmt == FMT_E4M3)
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  else
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, false);
}

template <int kFmt>
__device__ __forceinline__ v8bf codes_to_bf16(uint32_t w0, uint32_t w1) {
  const v2bf a = cvt2_bf16<kFmt>(w0, false), b = cvt2_bf16<kFmt>(w0, true);
  const v2bf c = cvt2_bf16<kFmt>(w1, false), d = cvt2_bf16<kFmt>(w1, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Upper halves of two fp32 values as two bf16 (exact when the low halves are
// zero; otherwise truncation).
__device__ __forceinline__ uint32_t hi2(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// V codes of one unit (32 token rows of 128 bytes) into an LDS buffer: 4
// copies of 1 KB. Lane l of copy i fills row 8 i + l / 8, physical chunk l % 8,
// i.e. logical chunk (l % 8) ^ (row % 8). Every offset is in the VGPR offset,
// which the buffer's range check covers (rows past T read zero). The codes
// are read once per call, so the copies carry the non-temporal hint.
__device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t r, uint32_t unit_off, uint32_t lane_voff,
                                          uint8_t* buf) {
#pragma unroll
  for (int i = 0; i < kCopies; ++i) dma16_nt(r, unit_off + (uint32_t)(i * 1024) + lane_voff, 0u, buf + i * 1024);
}

// K codes of one unit in registers: for subtile i, the lane's A operand of
// the score MFMAs, i.e. bytes 32 g .. 32 g + 31 of token row 16 i + c (g =
// lane / 16, c = lane % 16), as two 16-byte words. Loaded through the buffer
// resource (rows past T read zero) with the non-temporal hint.
struct KRegs {
  v4u w[kSub][2];
};

__device__ __forceinline__ void load_k(__amdgpu_buffer_rsrc_t r, uint32_t unit_off, uint32_t k_voff, KRegs& k) {
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      k.w[i][h] = __builtin_amdgcn_raw_buffer_load_b128(r, unit_off + (uint32_t)(i * 16 * kD + 16 * h) + k_voff, 0, 2);
}

// Byte offset of logical byte `b` of row `row` in a swizzled buffer.
__device__ __forceinline__ int swz_off(int row, int b) {
  return row * kD + ((((b >> 4) ^ (row & 7))) << 4) + (b & 15);
}

// Running state of one wave for its query columns (lane % 16).
struct Run {
  float m;        // running max (base-2 scores), same in the 4 lane groups
  float l;        // this lane's share of the running sum (its own tokens)
  v4f o[8];       // O^T, dims 16 j + 4 g + v, query column lane % 16
};

// One unit: scores, softmax update, P V. `kr` holds the unit's K codes (in
// registers), `vb` its V codes in LDS. unit_t0: first token of the unit; s_scale: c * s_k *
// log2 e of the unit's token block; s_v: its V scale.
template <int kFmt>
__device__ __forceinline__ void unit_step(const KRegs& kr, const uint8_t* vb, const v8bf (&qb)[4], Run& st,
                                          int unit_t0, int T, float s_scale, float s_v, int lane) {
  const int g = lane >> 4, c = lane & 15;
  // ---- scores: S^T[token 16 i + 4 g + v][query c]; the lane's A operand is
  // token 16 i + c, dims 32 g .. 32 g + 31 (two 16-byte chunks)
  v4f s[kSub];
#pragma unroll
  for (int i = 0; i < kSub; ++i) {
    const v4u w0 = kr.w[i][0];
    const v4u w1 = kr.w[i][1];
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const v4u& w = sl < 2 ? w0 : w1;
      const v8bf a = codes_to_bf16<kFmt>(w[(sl & 1) * 2], w[(sl & 1) * 2 + 1]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[sl], acc, 0, 0, 0);
    }
    s[i] = acc;
  }
  // ---- softmax update (base 2)
  float mx = kNegBig;
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = unit_t0 + 16 * i + 4 * g + v;
      s[i][v] = t < T ? s[i][v] * s_scale : -__builtin_inff();
      mx = fmaxf(mx, s[i][v]);
    }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st.m, mx);
  const float corr = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;
  float psum = 0.f;
  float p[kSub][4];
#pragma unroll
  for (int i = 0; i < kSub; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[i][v] = __builtin_amdgcn_exp2f(s[i][v] - m_new);
      psum += p[i][v];
    }
  st.l = st.l * corr + psum;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] *= corr;
  // ---- O^T += V^T P'^T over the unit's 32-token steps; k element e of lane
  // group g is token 4 g + e (e < 4) or 16 + 4 g + e - 4 of the step
#pragma unroll
  for (int st32 = 0; st32 < kUnit / 32; ++st32) {
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      // elements 2 e2, 2 e2 + 1
      const int e0 = 2 * e2, e1 = 2 * e2 + 1;
      const float p0 = (e0 < 4 ? p[2 * st32][e0] : p[2 * st32 + 1][e0 - 4]) * s_v;
      const float p1 = (e1 < 4 ? p[2 * st32][e1] : p[2 * st32 + 1][e1 - 4]) * s_v;
      const uint32_t b0 = __float_as_uint(p0) & 0xffff0000u, b1 = __float_as_uint(p1) & 0xffff0000u;
      hw[e2] = hi2(b0, b1);
      lw[e2] = hi2(__float_as_uint(p0 - __uint_as_float(b0)), __float_as_uint(p1 - __uint_as_float(b1)));
    }
    const v8bf ph = __builtin_bit_cast(v8bf, v4u{hw[0], hw[1], hw[2], hw[3]});
    const v8bf pl = __builtin_bit_cast(v8bf, v4u{lw[0], lw[1], lw[2], lw[3]});
    // transposed read: lane r of the 16-lane group addresses token
    // index r / 2 (mapped as above) and dims 8 (r % 2) .. +7 of the subtile
    const int r = c;
    const int ti = r >> 1;
    const int tok = 32 * st32 + (ti < 4 ? 4 * g + ti : 16 + 4 * g + ti - 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v2i w = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)(vb + swz_off(tok, 16 * j + 8 * (r & 1))));
      const v8bf a = codes_to_bf16<kFmt>((uint32_t)w[0], (uint32_t)w[1]);
      st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph, st.o[j], 0, 0, 0);
      st.o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl, st.o[j], 0, 0, 0);
    }
  }
}

// The wave's loop over its units, two units ahead: unit u + 2 is issued (K
// into register slot (u + 2) % 3, V into LDS stage (u + 2) % 3) before unit u
// is computed, after a wait that leaves only the 2 later units' memory
// operations in flight. The issues and waits run in every step of the loop,
// up to 2 steps past the wave's last unit (those steps compute nothing), and
// past the last unit the issue reads at an offset beyond the resource's end:
// the range check makes those loads return zeros without touching memory.
// So every path has the same operations in flight, the compiler's own waits
// for the K registers keep the same depth, and no load sits in a conditional
// block next to its use (where the compiler would sink it, to just before
// the unit that needs it). A slot or stage is refilled only after its
// previous unit has been computed, every LDS read and register use of which
// has completed. Distinct __restrict__ stages and arrays, and resources built
// here, let the compiler see that reading one stage does not wait for the
// copies into the others.
template <int kFmt>
__device__ __forceinline__ void wave_loop(const AttnParams& p, const uint8_t* __restrict__ kh,
                                          const uint8_t* __restrict__ vh, uint32_t head_bytes,
                                          uint8_t* __restrict__ v0, uint8_t* __restrict__ v1,
                                          uint8_t* __restrict__ v2, const v8bf (&qb)[4], Run& st, int h,
                                          int t_begin, int nunits, int lane) {
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kh, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(vh, head_bytes);
  const int crow = lane >> 3;
  const uint32_t lane_voff = (uint32_t)(crow * kD + (((lane & 7) ^ (crow & 7)) << 4));
  const uint32_t k_voff = (uint32_t)((lane & 15) * kD + 32 * (lane >> 4));
  // per-token-block scales, read through the constant address space (scalar
  // loads: they are inputs the kernel never writes)
  typedef const __attribute__((address_space(4))) float* cf_ptr;
  const cf_ptr skh = (cf_ptr)(p.sk + (int64_t)h * p.nb);
  const cf_ptr svh = (cf_ptr)(p.sv + (int64_t)h * p.nb);
  constexpr int kOps = kSub * 2 + kCopies;   // memory operations per unit
  // units past the wave's last read at the resource's end (zeros, no memory
  // access). The lanes add less than 4 KB to it; only for T > 2^25 - 32 can the
  // 32-bit sum wrap, and then it addresses the head's own codes (in bounds),
  // whose values go into a slot that is never computed.
  auto unit_off = [&](int u) { return u < nunits ? (uint32_t)(t_begin + u * kUnit) * kD : head_bytes; };
  auto issue = [&](int u, KRegs& kr, uint8_t* vb) {
    load_k(rk, unit_off(u), k_voff, kr);
    load_unit(rv, unit_off(u), lane_voff, vb);
  };
  // issue unit u + 2 into (kn, vn), wait for unit u, compute it from (kc, vc)
  auto step = [&](int u, const KRegs& kc, const uint8_t* vc, KRegs& kn, uint8_t* vn) {
    issue(u + 2, kn, vn);
    wait_vm<2 * kOps>();
    asm volatile("" ::: "memory");
    if (u < nunits) {
      const int t0 = t_begin + u * kUnit;
      const int blk = t0 >> 7;
      unit_step<kFmt>(kc, vc, qb, st, t0, p.T, skh[blk] * p.c_log2, svh[blk], lane);
    }
  };
  KRegs k0, k1, k2;
  issue(0, k0, v0);
  issue(1, k1, v1);
  for (int u = 0; u < nunits; u += 3) {
    step(u, k0, v0, k2, v2);
    step(u + 1, k1, v1, k0, v0);
    step(u + 2, k2, v2, k1, v1);
  }
  wait_vm<0>();
}

// grid (splits, Hkv), 256 threads.
template <int kFmt>
__global__ __launch_bounds__(kThreadsA) void k_fp8kv_decode_attn(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWaves * kStages * kUnitBytes];   // 48 KB
  const int split = blockIdx.x, h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;

  // query fragments (B operand): column c = query head h G + c, dims
  // 32 g + 8 sl .. +7 for slab sl; zero columns past G
  v8bf qb[4];
  {
    const bool live = c < p.G;
    const __hip_bfloat16* qrow = p.q + (int64_t)(h * p.G + (live ? c : 0)) * p.ld_q + 32 * g;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const v4u w = live ? *reinterpret_cast<const v4u*>(qrow + 8 * sl) : v4u{0u, 0u, 0u, 0u};
      qb[sl] = __builtin_bit_cast(v8bf, w);
    }
  }
  Run st;
  st.m = kNegBig;
  st.l = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) st.o[j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int t_begin = split * kSplitTokens + wave * (kUnitsPerWave * kUnit);
  const int left = p.T - t_begin;
  const int nunits = left <= 0 ? 0 : min(kUnitsPerWave, (left + kUnit - 1) / kUnit);
  const uint32_t head_bytes = (uint32_t)p.T * kD;
  uint8_t* const b = smem + wave * kStages * kUnitBytes;
  if (nunits > 0)
    wave_loop<kFmt>(p, p.k + (int64_t)h * p.T * kD, p.v + (int64_t)h * p.T * kD, head_bytes, b, b + kUnitBytes,
                    b + 2 * kUnitBytes, qb, st, h, t_begin, nunits, lane);

  // ---- merge the 4 waves through LDS (the stages are free: every wave
  // has waited for its last copies and passes this barrier first)
  float lsum = st.l;
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  raw_barrier();
  static_assert(kWaves * 16 * kPartial * sizeof(float) <= sizeof(smem), "merge buffer exceeds the LDS");
  float* const red = reinterpret_cast<float*>(smem);      // [wave][16 q][kPartial]
  float* const mine = red + wave * 16 * kPartial;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) mine[c * kPartial + 16 * j + 4 * g + v] = st.o[j][v];
  if (g == 0) {
    mine[c * kPartial + kD] = st.m;
    mine[c * kPartial + kD + 1] = lsum;
  }
  raw_barrier();
  // thread t: query column t / 16, dims (t % 16) * 8 .. +7
  const int qc = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
  if (qc < p.G) {
    float mw[kWaves], M = kNegBig;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = red[(w * 16 + qc) * kPartial + kD];
      M = fmaxf(M, mw[w]);
    }
    float L = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(mw[w] - M);
      L += red[(w * 16 + qc) * kPartial + kD + 1] * f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += red[(w * 16 + qc) * kPartial + d0 + e] * f;
    }
    float* const dst = p.ws + ((int64_t)(h * p.G + qc) * p.splits + split) * kPartial;
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[d0 + e] = o[e];
    if (d0 == 0) {
      dst[kD] = M;
      dst[kD + 1] = L;
    }
  }
}

// Merge of the splits of each query head; grid (Hq, 4), 512 threads: a
// workgroup takes 32 dims of one query head, thread t dim t % 32 over the
// splits s = t / 32 (mod 16). Each thread merges its splits online (running
// max, sum and output, rescaled by exp2 of the change of max), with the loads of all
// its splits independent of the arithmetic, so one round trip to memory; the
// 16 parts of a dim are then merged through LDS.
constexpr int kCombThreads = 512;
constexpr int kCombDims = 32;
constexpr int kCombParts = kCombThreads / kCombDims;

template <bool kBf16Out>
__global__ __launch_bounds__(kCombThreads) void k_fp8kv_attn_combine(AttnParams p) {
  __shared__ float pm[kCombParts][kCombDims], pl[kCombParts][kCombDims], po[kCombParts][kCombDims];
  const int hq = blockIdx.x, t = threadIdx.x;
  const int dl = t % kCombDims, part = t / kCombDims, d = blockIdx.y * kCombDims + dl;
  const float* base = p.ws + (int64_t)hq * p.splits * kPartial;
  // online merge of the part's splits: running max M, sum L and output o
  float M = kNegBig, L = 0.f, o = 0.f;
#pragma unroll 4
  for (int s = part; s < p.splits; s += kCombParts) {
    const float* ps = base + (int64_t)s * kPartial;
    const float m = ps[kD], l = ps[kD + 1], v = ps[d];
    const float mn = fmaxf(M, m);
    const float a = __builtin_amdgcn_exp2f(M - mn), b = __builtin_amdgcn_exp2f(m - mn);
    L = L * a + l * b;
    o = o * a + v * b;
    M = mn;
  }
  pm[part][dl] = M;
  pl[part][dl] = L;
  po[part][dl] = o;
  __syncthreads();
  if (part == 0) {
    float mx = kNegBig;
#pragma unroll
    for (int i = 0; i < kCombParts; ++i) mx = fmaxf(mx, pm[i][dl]);
    float os = 0.f, ls = 0.f;
#pragma unroll
    for (int i = 0; i < kCombParts; ++i) {
      const float w = __builtin_amdgcn_exp2f(pm[i][dl] - mx);
      os += po[i][dl] * w;
      ls += pl[i][dl] * w;
    }
    const float r = os / ls;
    if (kBf16Out)
      static_cast<__hip_bfloat16*>(p.out)[(int64_t)hq * p.ld_o + d] = __float2bfloat16(r);
    else
      static_cast<float*>(p.out)[(int64_t)hq * p.ld_o + d] = r;
  }
}

}  // namespace

int attention_splits(int64_t tokens) { return (int)((tokens + kSplitTokens - 1) / kSplitTokens); }
int64_t attention_partial_floats() { return kPartial; }

// ---------------------------------------------------------------------------
// The fixed workspace of fp8_kv_decode_attention_noalloc, for callers that
// cannot allocate device memory: a file-scope device array, 12 MiB (the split
// partials of heads_q * ceil(tokens / 1408) <= 24197 query-head splits, e.g.
// 64 query heads over 512K tokens), one copy on every device the library runs
// on, held until the process ends. In host code the array's name is only a
// stand-in for it: its device address is looked up once per device with that
// device current and cached, and only that address is handed to kernels.
// Calls on one device share the array, so calls that overlap in time on one
// device race.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)12 << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

size_t attention_scratch_bytes() { return kScratchBytes; }

hipError_t attention_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_kv_decode_attention(const AttnArgs& a, hipStream_t st) {
  AttnParams p;
  p.q = static_cast<const __hip_bfloat16*>(a.q);
  p.k = a.k;
  p.v = a.v;
  p.sk = a.sk;
  p.sv = a.sv;
  p.ws = a.ws;
  p.out = a.out;
  p.ld_q = a.ld_q;
  p.ld_o = a.ld_o;
  p.T = (int)a.tokens;
  p.nb = (int)((a.tokens + 127) / 128);
  p.G = (int)(a.heads_q / a.heads_kv);
  p.splits = attention_splits(a.tokens);
  p.c_log2 = a.softmax_scale * kLog2e;
  const dim3 grid((unsigned)p.splits, (unsigned)a.heads_kv);
  if (a.fmt == FMT_E5M2)
    hipLaunchKernelGGL(k_fp8kv_decode_attn<FMT_E5M2>, grid, dim3(kThreadsA), 0, st, p);
  else
    hipLaunchKernelGGL(k_fp8kv_decode_attn<FMT_E4M3>, grid, dim3(kThreadsA), 0, st, p);
  if (a.out_dtype == DTYPE_BF16)
    hipLaunchKernelGGL(k_fp8kv_attn_combine<true>, dim3((unsigned)a.heads_q, kD / kCombDims), dim3(kCombThreads), 0,
                       st, p);
  else
    hipLaunchKernelGGL(k_fp8kv_attn_combine<false>, dim3((unsigned)a.heads_q, kD / kCombDims), dim3(kCombThreads), 0,
                       st, p);
  return hipGetLastError();
}

}  // namespace fp8blk
