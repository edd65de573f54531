// Device helpers shared by the fp8blk HIP kernels (gfx950 only).
//
// The FP8 formats are OCP E4M3 and OCP E5M2 as fixed by [FP8] (wangyu.me,
// "大语言模型量化技术（五）：FP8"), section "FP8 是什么", format table: E4M3 has
// largest finite 448, smallest normal 2^-6, smallest subnormal 2^-9, no
// infinity, saturation at +-448; E5M2 has largest finite 57344, smallest
// normal 2^-14, smallest subnormal 2^-16 (its infinity and NaN codes are never
// produced: the quantizer saturates at +-57344 as well).
#pragma once

#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace fp8blk {

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

// ---------------------------------------------------------------------------
// bf16 <-> fp32 bit helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// Buffer resources, direct global -> LDS copies, waits and barriers.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over `bytes` bytes from `base` (raw loads; reads at or past
// `bytes` return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct global -> LDS copy through a buffer resource: lane l writes `size`
// bytes at lds + size * l (lds must be wave-uniform); reads past the
// resource's end write zeros.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}
// The same with the non-temporal hint (nt), for data read once.
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 2);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt with vmcnt(n) only (expcnt and lgkmcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(((n >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (n & 15));
}

// s_waitcnt with lgkmcnt(n) only (vmcnt and expcnt left at their maxima).
template <int n>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(n >= 0 && n < 16, "lgkmcnt");
  __builtin_amdgcn_s_waitcnt((3 << 14) | (n << 8) | (0x7 << 4) | 0xF);
}

// Workgroup barrier. s_barrier alone does not wait for the wave's own LDS
// accesses, so the wave first waits for them (lgkmcnt(0)): LDS writes made
// before the barrier are then complete when other waves read after it, and
// LDS reads made before it are complete when other waves overwrite the data.
// Vector memory operations, the direct global -> LDS copies among them, are
// waited for separately (wait_vm). The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  wait_lgkm<0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The same barrier after this wave's vector memory operations (the direct
// copies into LDS among them) have also completed: one s_waitcnt vmcnt(0)
// lgkmcnt(0), then s_barrier.
__device__ __forceinline__ void copies_done_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((0x7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Max reductions over non-negative fp32 bit patterns (which order like uints).
// ---------------------------------------------------------------------------
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)0, (int)v, kCtrl, 0xf, 0xf, false);
  return o > v ? o : v;
}

// Max over the 16 lanes of a DPP row; every lane of the row gets the result.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  v = dpp_max_step<0x140>(v);  // row_mirror
  return v;
}

// Max over the whole 64-lane wave; every lane gets the result.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = row16_max(v);
  uint32_t o = (uint32_t)__shfl_xor((int)v, 16);
  v = o > v ? o : v;
  o = (uint32_t)__shfl_xor((int)v, 32);
  return o > v ? o : v;
}

// ---------------------------------------------------------------------------
// fp32 -> FP8 with round-to-nearest-even and saturation, and FP8 -> fp32.
//
// The hardware conversions v_cvt_pk_fp8_f32 (E4M3) and v_cvt_pk_bf8_f32 (E5M2)
// of gfx950 write OCP codes with round-to-nearest-even; clamping to the
// format's largest value first (v_med3_f32) gives the saturating behaviour of
// the quantizer. tests/test_gpu_quantize.py and tests/test_gpu_e5m2.py check
// this against the CPU oracle on every fp32 value in [-448, 448] and
// [-57344, 57344]. v_cvt_pk_f32_fp8 / v_cvt_pk_f32_bf8 decode codes exactly.
// ---------------------------------------------------------------------------
template <int kFmt>
struct Fp8;

template <>
struct Fp8<FMT_E4M3> {
  static constexpr float kMax = kE4M3Max;
  // four values with |v| <= 448 (or a hair above) -> four codes, no clamp
  static __device__ __forceinline__ uint32_t pack4_raw(float a, float b, float c, float d) {
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)w, true);
  }
  // codes 0,1 (kHi = false) or 2,3 (kHi = true) of a word -> fp32
  template <bool kHi>
  static __device__ __forceinline__ auto decode2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
  }
};

template <>
struct Fp8<FMT_E5M2> {
  static constexpr float kMax = kE5M2Max;
  static __device__ __forceinline__ uint32_t pack4_raw(float a, float b, float c, float d) {
    uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c, d, (int)w, true);
  }
  template <bool kHi>
  static __device__ __forceinline__ auto decode2(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_bf8((int)w, kHi);
  }
};

template <int kFmt>
__device__ __forceinline__ float clamp_max(float v) {
  return __builtin_amdgcn_fmed3f(v, -Fp8<kFmt>::kMax, Fp8<kFmt>::kMax);
}

// Four fp32 values -> four codes packed little-endian in one word, saturating.
template <int kFmt>
__device__ __forceinline__ uint32_t pack4_sat(float a, float b, float c, float d) {
  return Fp8<kFmt>::pack4_raw(clamp_max<kFmt>(a), clamp_max<kFmt>(b), clamp_max<kFmt>(c), clamp_max<kFmt>(d));
}

// ---------------------------------------------------------------------------
// Group scale and the bit-exact cast of a group's elements.
//
// The code of x is FP8(fl32(x / s)) with the IEEE correctly rounded fp32
// quotient; the per-element division is replaced by multiplications with a
// per-group reciprocal r: v_rcp_f32(s) (1 ulp) refined by one Newton step.
//
// bf16 inputs (cast4_bf16): q = fl32(x r), then one residual correction
// q' = q - fl32(s q - x) r with fused multiply-adds. For each format, an
// exhaustive sweep over every bf16 amax whose scale lies in [2^-64, 2^64] and,
// under each, every bf16 |x| <= amax in both signs finds the code of q' equal
// to the code of fl32(x / s) (the quotient itself can differ by one ulp, never
// across a code boundary of either grid); tests/test_gpu_quantize.py runs the
// sweep against the CPU oracle for E4M3 and E5M2. The residual is negated so
// that x = -0 keeps its sign. E5M2 quotients are clamped to +-57344 before the
// conversion (saturation). Groups whose scale lies outside that range, or is
// zero, divide exactly.
//
// fp32 inputs (cast4_f32), either format: the products fl32(x rl) and fl32(x rh) with
// rl = r (1 - 2^-20), rh = r (1 + 2^-20) bracket fl32(x / s) strictly in
// magnitude (their relative offsets exceed 2^-20 - 2^-22 - 3 * 2^-24 > 2^-24,
// the fp32 rounding bound) whenever the quotient is an fp32 normal.
// Round-to-nearest is monotone, so when both brackets give the same code it is
// the code of fl32(x / s); otherwise the element takes the exact division.
// For E4M3 the brackets are converted without a clamp: the lower one never
// exceeds 448 (|x| <= amax), where the hardware conversion is exact; the upper
// one may exceed it by a hair, and if the conversion then disagrees the exact
// path decides. For E5M2 both are clamped to +-57344 first (a monotone,
// saturating conversion), so the argument holds unchanged. Quotients below the
// fp32 normal range give code 0 (signed) on every path. Groups whose scale is
// zero or an fp32 subnormal always take the exact division.
// ---------------------------------------------------------------------------
struct GroupScale {
  float s;  // fl32(amax / max_fmt)
  float r;  // ~ 1 / s, Newton-refined
};

template <int kFmt>
__device__ __forceinline__ GroupScale make_group_scale(uint32_t amax_bits) {
  GroupScale g;
  g.s = __uint_as_float(amax_bits) / Fp8<kFmt>::kMax;   // IEEE correctly rounded division
  const float r0 = __builtin_amdgcn_rcpf(g.s);   // 1 ulp
  g.r = __builtin_fmaf(__builtin_fmaf(-g.s, r0, 1.0f), r0, r0);
  return g;
}

// Exact path for one element: sign-only zero when s == 0.
__device__ __forceinline__ float exact_quotient(float x, float s) {
  if (s == 0.0f) return __uint_as_float(__float_as_uint(x) & 0x80000000u);
  return x / s;   // IEEE correctly rounded division
}

template <int kFmt>
__device__ __forceinline__ uint32_t exact4(const GroupScale& g, float a, float b, float c, float d) {
  return pack4_sat<kFmt>(exact_quotient(a, g.s), exact_quotient(b, g.s), exact_quotient(c, g.s),
                         exact_quotient(d, g.s));
}

__device__ __forceinline__ bool bf16_fast_ok(const GroupScale& g) {
  return g.s >= 0x1.0p-64f && g.s <= 0x1.0p64f;
}

__device__ __forceinline__ float quotient_bf16(const GroupScale& g, float x) {
  const float q = x * g.r;
  const float e = __builtin_fmaf(g.s, q, -x);
  return __builtin_fmaf(-e, g.r, q);
}

// Codes of four elements of one group of arbitrary fp32 values.
template <int kFmt>
__device__ __forceinline__ uint32_t cast4_f32(const GroupScale& g, float a, float b, float c, float d) {
  if (g.s >= 0x1.0p-126f) {
    const float rl = g.r * (1.0f - 0x1.0p-20f);
    const float rh = g.r * (1.0f + 0x1.0p-20f);
    uint32_t lo, hi;
    if constexpr (kFmt == FMT_E4M3) {
      lo = Fp8<kFmt>::pack4_raw(a * rl, b * rl, c * rl, d * rl);
      hi = Fp8<kFmt>::pack4_raw(a * rh, b * rh, c * rh, d * rh);
    } else {
      lo = pack4_sat<kFmt>(a * rl, b * rl, c * rl, d * rl);
      hi = pack4_sat<kFmt>(a * rh, b * rh, c * rh, d * rh);
    }
    if (__builtin_expect(lo == hi, 1)) return lo;
  }
  return exact4<kFmt>(g, a, b, c, d);
}

// A caller-supplied scale s (static or delayed scaling): the same reciprocal
// as make_group_scale computes.
__device__ __forceinline__ GroupScale make_given_scale(float s) {
  GroupScale g;
  g.s = s;
  const float r0 = __builtin_amdgcn_rcpf(s);
  g.r = __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
  return g;
}

// Codes of four elements under a caller-supplied scale, where |x / s| may lie
// anywhere (saturation is real): the bracket of cast4_f32 with both brackets
// clamped to +-MAX first for either format (a monotone, saturating
// conversion, so the bracket argument holds), else the exact division. The
// bracket needs a normal reciprocal, so s above 2^125 takes the exact path.
template <int kFmt>
__device__ __forceinline__ uint32_t cast4_sat(const GroupScale& g, float a, float b, float c, float d) {
  if (g.s >= 0x1.0p-126f && g.s <= 0x1.0p125f) {
    const float rl = g.r * (1.0f - 0x1.0p-20f);
    const float rh = g.r * (1.0f + 0x1.0p-20f);
    const uint32_t lo = pack4_sat<kFmt>(a * rl, b * rl, c * rl, d * rl);
    const uint32_t hi = pack4_sat<kFmt>(a * rh, b * rh, c * rh, d * rh);
    if (__builtin_expect(lo == hi, 1)) return lo;
  }
  return exact4<kFmt>(g, a, b, c, d);
}

// Codes of four elements of one group whose values are bf16 numbers, given
// bf16_fast_ok(g) (for callers that check it once for many elements).
template <int kFmt>
__device__ __forceinline__ uint32_t cast4_bf16_fast(const GroupScale& g, float a, float b, float c, float d) {
  const float qa = quotient_bf16(g, a), qb = quotient_bf16(g, b), qc = quotient_bf16(g, c),
              qd = quotient_bf16(g, d);
  if constexpr (kFmt == FMT_E4M3)
    return Fp8<kFmt>::pack4_raw(qa, qb, qc, qd);
  else
    return pack4_sat<kFmt>(qa, qb, qc, qd);
}

// Codes of four elements of one group whose values are bf16 numbers.
template <int kFmt>
__device__ __forceinline__ uint32_t cast4_bf16(const GroupScale& g, float a, float b, float c, float d) {
  if (__builtin_expect(bf16_fast_ok(g), 1)) return cast4_bf16_fast<kFmt>(g, a, b, c, d);
  return exact4<kFmt>(g, a, b, c, d);
}

// Max over the 8 lanes of each half of a DPP row; every lane of the half gets it.
__device__ __forceinline__ uint32_t row8_max(uint32_t v) {
  v = dpp_max_step<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141>(v);  // row_half_mirror
  return v;
}

// q = n / d for n < 2^31 with a precomputed multiplier (Granlund and
// Montgomery, "Division by invariant integers using multiplication", PLDI
// 1994): l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, and
// q = (umulhi(m, n) + n) >> l; the sum cannot overflow because n < 2^31.
struct FastDiv {
  uint32_t m;
  uint32_t l;
};
__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv d) {
  return (__umulhi(d.m, n) + n) >> d.l;
}
// Multiplier and shift for fastdiv by d >= 1 (host side).
inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  FastDiv f;
  f.m = (uint32_t)((((1ull << l) - d) << 32) / d + 1);
  f.l = l;
  return f;
}

// |x| bit patterns of eight bf16 values held in four words, as fp32 bit
// patterns, reduced to their max.
__device__ __forceinline__ uint32_t amax_bf16x8(uint4 w) {
  uint32_t m = 0;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = ws[i] & 0x7fff7fffu;
    const uint32_t hi = a & 0xffff0000u;
    const uint32_t lo = a << 16;
    m = hi > m ? hi : m;
    m = lo > m ? lo : m;
  }
  return m;
}

__device__ __forceinline__ uint32_t amax_f32(float v, uint32_t m) {
  const uint32_t a = __float_as_uint(v) & 0x7fffffffu;
  return a > m ? a : m;
}

// ---------------------------------------------------------------------------
// Eight consecutive input elements of one lane.
//
// Loads are streaming (nontemporal) by default: every quantizer reads its
// input exactly once, and keeping it out of the caches measured 8-17% faster
// on the large passes. The per-tensor amax pass reads with normal loads so
// that its second (cast) pass can hit the Infinity Cache.
// ---------------------------------------------------------------------------
typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

template <bool kStream>
__device__ __forceinline__ uint4 load16(const void* p) {
  if (kStream) {
    const v4u32 t = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
    return make_uint4(t[0], t[1], t[2], t[3]);
  }
  return *reinterpret_cast<const uint4*>(p);
}

template <typename T>
struct Vec8;

template <>
struct Vec8<__hip_bfloat16> {
  uint4 w;
  template <bool kStream = true>
  __device__ __forceinline__ void load(const __hip_bfloat16* p, uint32_t nvalid) {
    if (nvalid >= 8) {
      w = load16<kStream>(p);
    } else {
      const uint16_t* h = reinterpret_cast<const uint16_t*>(p);
      uint32_t e[8];
#pragma unroll
      for (uint32_t i = 0; i < 8; ++i) e[i] = i < nvalid ? (uint32_t)h[i] : 0u;
      w.x = e[0] | (e[1] << 16);
      w.y = e[2] | (e[3] << 16);
      w.z = e[4] | (e[5] << 16);
      w.w = e[6] | (e[7] << 16);
    }
  }
  __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ uint32_t amax_bits() const { return amax_bf16x8(w); }
  template <int kFmt>
  __device__ __forceinline__ uint2 cast(const GroupScale& g) const {
    uint2 r;
    r.x = cast4_bf16<kFmt>(g, bf16_lo_to_f32(w.x), bf16_hi_to_f32(w.x), bf16_lo_to_f32(w.y), bf16_hi_to_f32(w.y));
    r.y = cast4_bf16<kFmt>(g, bf16_lo_to_f32(w.z), bf16_hi_to_f32(w.z), bf16_lo_to_f32(w.w), bf16_hi_to_f32(w.w));
    return r;
  }
  // cast() when the caller has checked bf16_fast_ok(g)
  template <int kFmt>
  __device__ __forceinline__ uint2 cast_fast(const GroupScale& g) const {
    uint2 r;
    r.x = cast4_bf16_fast<kFmt>(g, bf16_lo_to_f32(w.x), bf16_hi_to_f32(w.x), bf16_lo_to_f32(w.y),
                                bf16_hi_to_f32(w.y));
    r.y = cast4_bf16_fast<kFmt>(g, bf16_lo_to_f32(w.z), bf16_hi_to_f32(w.z), bf16_lo_to_f32(w.w),
                                bf16_hi_to_f32(w.w));
    return r;
  }
  template <int kFmt>
  __device__ __forceinline__ uint2 cast_sat(const GroupScale& g) const {
    uint2 r;
    r.x = cast4_sat<kFmt>(g, bf16_lo_to_f32(w.x), bf16_hi_to_f32(w.x), bf16_lo_to_f32(w.y), bf16_hi_to_f32(w.y));
    r.y = cast4_sat<kFmt>(g, bf16_lo_to_f32(w.z), bf16_hi_to_f32(w.z), bf16_lo_to_f32(w.w), bf16_hi_to_f32(w.w));
    return r;
  }
  // codes of x * 2^e (exact scaling), saturating
  template <int kFmt>
  __device__ __forceinline__ uint2 cast_pow2(int e) const {
    uint2 r;
    r.x = pack4_sat<kFmt>(__builtin_amdgcn_ldexpf(bf16_lo_to_f32(w.x), e), __builtin_amdgcn_ldexpf(bf16_hi_to_f32(w.x), e),
                          __builtin_amdgcn_ldexpf(bf16_lo_to_f32(w.y), e), __builtin_amdgcn_ldexpf(bf16_hi_to_f32(w.y), e));
    r.y = pack4_sat<kFmt>(__builtin_amdgcn_ldexpf(bf16_lo_to_f32(w.z), e), __builtin_amdgcn_ldexpf(bf16_hi_to_f32(w.z), e),
                          __builtin_amdgcn_ldexpf(bf16_lo_to_f32(w.w), e), __builtin_amdgcn_ldexpf(bf16_hi_to_f32(w.w), e));
    return r;
  }
};

template <>
struct Vec8<float> {
  float4 a, b;
  template <bool kStream = true>
  __device__ __forceinline__ void load(const float* p, uint32_t nvalid) {
    if (nvalid >= 8) {
      const uint4 ua = load16<kStream>(p), ub = load16<kStream>(p + 4);
      a = make_float4(__uint_as_float(ua.x), __uint_as_float(ua.y), __uint_as_float(ua.z), __uint_as_float(ua.w));
      b = make_float4(__uint_as_float(ub.x), __uint_as_float(ub.y), __uint_as_float(ub.z), __uint_as_float(ub.w));
    } else {
      float e[8];
#pragma unroll
      for (uint32_t i = 0; i < 8; ++i) e[i] = i < nvalid ? p[i] : 0.0f;
      a = make_float4(e[0], e[1], e[2], e[3]);
      b = make_float4(e[4], e[5], e[6], e[7]);
    }
  }
  __device__ __forceinline__ void zero() {
    a = make_float4(0, 0, 0, 0);
    b = a;
  }
  __device__ __forceinline__ uint32_t amax_bits() const {
    uint32_t m = 0;
    m = amax_f32(a.x, m); m = amax_f32(a.y, m); m = amax_f32(a.z, m); m = amax_f32(a.w, m);
    m = amax_f32(b.x, m); m = amax_f32(b.y, m); m = amax_f32(b.z, m); m = amax_f32(b.w, m);
    return m;
  }
  template <int kFmt>
  __device__ __forceinline__ uint2 cast(const GroupScale& g) const {
    uint2 r;
    r.x = cast4_f32<kFmt>(g, a.x, a.y, a.z, a.w);
    r.y = cast4_f32<kFmt>(g, b.x, b.y, b.z, b.w);
    return r;
  }
  template <int kFmt>
  __device__ __forceinline__ uint2 cast_sat(const GroupScale& g) const {
    uint2 r;
    r.x = cast4_sat<kFmt>(g, a.x, a.y, a.z, a.w);
    r.y = cast4_sat<kFmt>(g, b.x, b.y, b.z, b.w);
    return r;
  }
  template <int kFmt>
  __device__ __forceinline__ uint2 cast_pow2(int e) const {
    uint2 r;
    r.x = pack4_sat<kFmt>(__builtin_amdgcn_ldexpf(a.x, e), __builtin_amdgcn_ldexpf(a.y, e),
                          __builtin_amdgcn_ldexpf(a.z, e), __builtin_amdgcn_ldexpf(a.w, e));
    r.y = pack4_sat<kFmt>(__builtin_amdgcn_ldexpf(b.x, e), __builtin_amdgcn_ldexpf(b.y, e),
                          __builtin_amdgcn_ldexpf(b.z, e), __builtin_amdgcn_ldexpf(b.w, e));
    return r;
  }
};

__device__ __forceinline__ void store_codes8(uint8_t* p, uint2 c, uint32_t nvalid) {
  if (nvalid >= 8) {
    *reinterpret_cast<uint2*>(p) = c;
  } else {
#pragma unroll
    for (uint32_t i = 0; i < 8; ++i) {
      const uint32_t word = i < 4 ? c.x : c.y;
      if (i < nvalid) p[i] = (uint8_t)(word >> (8 * (i & 3)));
    }
  }
}

}  // namespace fp8blk
