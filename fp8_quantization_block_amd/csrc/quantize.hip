// Quantization kernels: per-tensor, 1x128 groups, 128x128 blocks, KV
// (head x token block) groups, the KV dequantizer, MX blocks of 32 with
// power-of-two scales, and the static / delayed-scaling cast under a
// caller-supplied scale.
//
// Method ([FP8] wangyu.me, "大语言模型量化技术（五）：FP8"): per group, amax = max|x|,
// s = amax / max_fmt, code = FP8(x / s) rounded to nearest even and saturated
// (section "什么是 FP8 量化"; section "权重量化：128×128 分块 FP8" for 128x128
// blocks; section "激活动态量化" for per-token 1x128 groups). KV groups are one
// head x 128 tokens x head_dim ([LONG] pwwt.cn Llama-3 FP8 notes, section 3).
// Dequantization is x ~ q * s ([MIXED] charles2530.github.io, "量化：FP8 与混合精度推理",
// section "E4M3 和 E5M2 是范围与格点的取舍"). Every kernel is instantiated for both
// FP8 formats ([FP8] section "FP8 是什么", format table): E4M3 (max_fmt = 448)
// and E5M2 (max_fmt = 57344; [VS] api.makesence.top, "LLM推理量化:FP8 versus INT8",
// section 2, serves a W8A8 E4M3 model with an E5M2 KV cache).
//
// All passes are HBM-bound: 16-byte loads, a max reduction in registers / DPP
// / LDS, then packed code stores.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace fp8blk {

// The per-tensor, static and MX casts store their codes with the
// non-temporal hint: measured bit-identical and faster at 4096 x 4096 (static
// 19.7 -> 18.0 us, per tensor 18.1 -> 17.7 us, MX unchanged). The 1x128,
// 128x128 and KV kernels keep cached stores: with the hint they measured the
// same or slower (1x128 at 8192 x 8192 33.0 -> 34.4 us, 128x128 at
// 10240 x 8192 41.8 -> 44.0 us, KV K + V 124.3 -> 127.2 us).
constexpr bool kStreamCastCodes = true;

// store_codes8 with, for kStream and a full chunk, the non-temporal hint.
template <bool kStream>
__device__ __forceinline__ void store_codes8_hint(uint8_t* p, uint2 c, uint32_t nvalid) {
  if (kStream && nvalid >= 8) {
    typedef uint32_t v2u32_t __attribute__((ext_vector_type(2)));
    v2u32_t t;
    t[0] = c.x;
    t[1] = c.y;
    __builtin_nontemporal_store(t, reinterpret_cast<v2u32_t*>(p));
  } else {
    store_codes8(p, c, nvalid);
  }
}

// Block-wide max over non-negative fp32 bit patterns (blockDim.x == 256).
__device__ __forceinline__ uint32_t block256_max(uint32_t m) {
  __shared__ uint32_t red[4];
  m = wave_max(m);
  const uint32_t wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63u) == 0) red[wave] = m;
  __syncthreads();
  uint32_t r = red[0];
  r = red[1] > r ? red[1] : r;
  r = red[2] > r ? red[2] : r;
  r = red[3] > r ? red[3] : r;
  return r;
}

// ---------------------------------------------------------------------------
// 1x128 groups: 8 lanes (half a DPP row) per group, 16 elements per lane in
// two 16-byte chunks (elements 8 l .. 8 l + 7 and 64 + 8 l .. 64 + 8 l + 7),
// kUnroll units of 32 groups per workgroup with all loads issued before any
// arithmetic.
// * kColumns = false (scales row-major): a unit is 32 consecutive groups of
//   the flat (row, group) index space, row = g / ngroups, so a workgroup's
//   scales are contiguous.
// * kColumns = true (scales K-block-major, consecutive rows' scales of one
//   group adjacent): a unit is 8 rows x 4 groups; wave w takes group 4 gb + w
//   of the 8 rows, so its 8 scale stores are one contiguous 32-byte run
//   (row by row they would be 4-byte writes 4 * rows bytes apart), and the
//   workgroup reads 1 KB of each row.
// ---------------------------------------------------------------------------
template <typename T, int kUnroll, int kFmt, bool kColumns>
__global__ __launch_bounds__(256) void k_quant_group_1x128(
    const T* __restrict__ x, int64_t ld_x, uint32_t rows, uint32_t cols, uint32_t ngroups, uint32_t total_units,
    FastDiv div_units, uint32_t units_per_row, uint8_t* __restrict__ q, int64_t ld_q, float* __restrict__ sc,
    int64_t ss_row, int64_t ss_col) {
  const uint32_t lane8 = threadIdx.x & 7u;
  const uint32_t slot = threadIdx.x >> 3;
  Vec8<T> v[kUnroll][2];
  uint32_t row[kUnroll], grp[kUnroll], nv[kUnroll][2];
  bool live[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    if constexpr (kColumns) {
      const uint32_t unit = blockIdx.x * kUnroll + u;   // (row block of 8, group block of 4)
      const uint32_t rb = fastdiv(unit, div_units);
      row[u] = rb * 8u + (slot & 7u);
      grp[u] = (unit - rb * units_per_row) * 4u + (slot >> 3);
      live[u] = unit < total_units && row[u] < rows && grp[u] < ngroups;
      if (!live[u]) row[u] = grp[u] = 0u;
    } else {
      const uint32_t g = (blockIdx.x * kUnroll + u) * 32u + slot;
      live[u] = g < total_units;
      row[u] = live[u] ? fastdiv(g, div_units) : 0u;
      grp[u] = g - row[u] * ngroups;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t col0 = grp[u] * 128u + h * 64u + lane8 * 8u;
      nv[u][h] = (live[u] && col0 < cols) ? min(8u, cols - col0) : 0u;
      if (nv[u][h] > 0)
        v[u][h].load(x + (int64_t)row[u] * ld_x + col0, nv[u][h]);
      else
        v[u][h].zero();
    }
  }
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const uint32_t a0 = v[u][0].amax_bits(), a1 = v[u][1].amax_bits();
    const uint32_t amax = row8_max(a0 > a1 ? a0 : a1);
    const GroupScale gs = make_group_scale<kFmt>(amax);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint2 codes = v[u][h].template cast<kFmt>(gs);
      const uint32_t col0 = grp[u] * 128u + h * 64u + lane8 * 8u;
      if (nv[u][h] > 0) store_codes8(q + (int64_t)row[u] * ld_q + col0, codes, nv[u][h]);
    }
    if (live[u] && lane8 == 0) sc[(int64_t)row[u] * ss_row + (int64_t)grp[u] * ss_col] = gs.s;
  }
}

// ---------------------------------------------------------------------------
// Tile groups held in registers by one 256-thread workgroup: a 128x128 weight
// block, or one KV head x token block x head_dim. Up to 2048 chunks of 8
// elements (16384 elements, 32 KB of bf16), 8 chunks per thread.
// ---------------------------------------------------------------------------
struct TileGroup {
  int64_t in_off;      // element offset of the group's first element
  int64_t in_ld;       // element stride between the group's rows
  int64_t out_off;     // byte offset of the first code
  int64_t out_ld;      // byte stride between rows of codes
  int64_t scale_off;   // index of the group's scale
  uint32_t rows;       // valid rows in this group
  uint32_t cols;       // valid columns in this group
};

// A full group (128 rows of 128 elements): thread t takes chunk t % 16 of
// rows t / 16 + 16 i, so one base address and a fixed row stride cover its 8
// chunks. The general path below keeps a row, column and length per chunk
// and needs 100 VGPRs (4 workgroups per compute unit); a kernel built on this
// one alone needs 80 (6 per compute unit), so the launchers pick it when
// every group of the call is full.
template <typename T, int kFmt>
__device__ __forceinline__ void quant_tile_group_full(const T* __restrict__ x, uint8_t* __restrict__ q,
                                                      float* __restrict__ sc, const TileGroup& tg) {
  const uint32_t r0 = threadIdx.x >> 4, c0 = (threadIdx.x & 15u) * 8u;
  const T* xp = x + tg.in_off + (int64_t)r0 * tg.in_ld + c0;
  uint8_t* qp = q + tg.out_off + (int64_t)r0 * tg.out_ld + c0;
  const int64_t xs = 16 * tg.in_ld, qs = 16 * tg.out_ld;
  Vec8<T> v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i].load(xp + i * xs, 8u);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = v[i].amax_bits();
    m = a > m ? a : m;
  }
  const GroupScale gs = make_group_scale<kFmt>(block256_max(m));
#pragma unroll
  for (int i = 0; i < 8; ++i) store_codes8(qp + i * qs, v[i].template cast<kFmt>(gs), 8u);
  if (threadIdx.x == 0) sc[tg.scale_off] = gs.s;
}

template <typename T, int kFmt>
__device__ __forceinline__ void quant_tile_group(const T* __restrict__ x, uint8_t* __restrict__ q,
                                                 float* __restrict__ sc, const TileGroup& tg) {
  const uint32_t cpr = (tg.cols + 7u) >> 3;   // chunks per row
  const uint32_t nchunks = tg.rows * cpr;
  Vec8<T> v[8];
  uint32_t r[8], cc[8], nv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = threadIdx.x + 256u * i;
    r[i] = c / cpr;
    cc[i] = c - r[i] * cpr;
    nv[i] = c < nchunks ? min(8u, tg.cols - cc[i] * 8u) : 0u;
    if (nv[i] > 0)
      v[i].load(x + tg.in_off + (int64_t)r[i] * tg.in_ld + cc[i] * 8u, nv[i]);
    else
      v[i].zero();
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t a = v[i].amax_bits();
    m = a > m ? a : m;
  }
  const GroupScale gs = make_group_scale<kFmt>(block256_max(m));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (nv[i] > 0)
      store_codes8(q + tg.out_off + (int64_t)r[i] * tg.out_ld + cc[i] * 8u, v[i].template cast<kFmt>(gs), nv[i]);
  }
  if (threadIdx.x == 0) sc[tg.scale_off] = gs.s;
}

// 128x128 blocks of a [rows][cols] matrix; grid (ceil(cols/128), ceil(rows/128)).
// kFull: rows and cols are multiples of 128.
template <typename T, int kFmt, bool kFull>
__global__ __launch_bounds__(256) void k_quant_block_128x128(
    const T* __restrict__ x, int64_t ld_x, uint32_t rows, uint32_t cols, uint8_t* __restrict__ q,
    int64_t ld_q, float* __restrict__ sc, int64_t ss_row, int64_t ss_col) {
  TileGroup tg;
  const uint32_t gx = blockIdx.x, gy = blockIdx.y;
  tg.in_off = (int64_t)gy * 128 * ld_x + (int64_t)gx * 128;
  tg.in_ld = ld_x;
  tg.out_off = (int64_t)gy * 128 * ld_q + (int64_t)gx * 128;
  tg.out_ld = ld_q;
  tg.scale_off = (int64_t)gy * ss_row + (int64_t)gx * ss_col;
  tg.rows = min(128u, rows - gy * 128u);
  tg.cols = min(128u, cols - gx * 128u);
  if constexpr (kFull)
    quant_tile_group_full<T, kFmt>(x, q, sc, tg);
  else
    quant_tile_group<T, kFmt>(x, q, sc, tg);
}

// KV groups; grid (ceil(tokens/token_block), heads). kFull: token_block and
// head_dim are 128 and tokens a multiple of 128.
template <int kFmt, bool kFull>
__global__ __launch_bounds__(256) void k_kv_quant(
    const __hip_bfloat16* __restrict__ kv, int64_t stride_head, int64_t stride_token,
    uint32_t tokens, uint32_t head_dim, uint32_t token_block, uint8_t* __restrict__ q,
    float* __restrict__ sc) {
  TileGroup tg;
  const uint32_t b = blockIdx.x, h = blockIdx.y, nb = gridDim.x;
  const uint32_t t0 = b * token_block;
  tg.in_off = (int64_t)h * stride_head + (int64_t)t0 * stride_token;
  tg.in_ld = stride_token;
  tg.out_off = ((int64_t)h * tokens + t0) * head_dim;
  tg.out_ld = head_dim;
  tg.scale_off = (int64_t)h * nb + b;
  tg.rows = min(token_block, tokens - t0);
  tg.cols = head_dim;
  if constexpr (kFull)
    quant_tile_group_full<__hip_bfloat16, kFmt>(kv, q, sc, tg);
  else
    quant_tile_group<__hip_bfloat16, kFmt>(kv, q, sc, tg);
}

// KV dequantize: one workgroup per group, 8 codes per chunk (contiguous run
// of rows * head_dim codes in the dense layout), up to 2048 chunks per group.
template <int kFmt>
__global__ __launch_bounds__(256) void k_kv_dequant(
    const uint8_t* __restrict__ q, const float* __restrict__ sc, uint32_t tokens,
    uint32_t head_dim, uint32_t token_block, __hip_bfloat16* __restrict__ out) {
  const uint32_t b = blockIdx.x, h = blockIdx.y, nb = gridDim.x;
  const uint32_t t0 = b * token_block;
  const uint32_t rows = min(token_block, tokens - t0);
  const int64_t off = ((int64_t)h * tokens + t0) * head_dim;
  const float s = sc[(int64_t)h * nb + b];
  const uint32_t nchunks = (rows * head_dim) >> 3;   // head_dim % 8 == 0
  const uint2* src = reinterpret_cast<const uint2*>(q + off);
  uint4* dst = reinterpret_cast<uint4*>(out + off);
  uint2 w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = threadIdx.x + 256u * i;
    w[i] = c < nchunks ? src[c] : make_uint2(0, 0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t c = threadIdx.x + 256u * i;
    if (c >= nchunks) continue;
    uint32_t o[4];
    const uint32_t ws[2] = {w[i].x, w[i].y};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const auto lo = Fp8<kFmt>::template decode2<false>(ws[k]);
      const auto hi = Fp8<kFmt>::template decode2<true>(ws[k]);
      const __hip_bfloat16 e0 = __float2bfloat16(lo[0] * s);
      const __hip_bfloat16 e1 = __float2bfloat16(lo[1] * s);
      const __hip_bfloat16 e2 = __float2bfloat16(hi[0] * s);
      const __hip_bfloat16 e3 = __float2bfloat16(hi[1] * s);
      o[2 * k] = (uint32_t)__bfloat16_as_ushort(e0) | ((uint32_t)__bfloat16_as_ushort(e1) << 16);
      o[2 * k + 1] = (uint32_t)__bfloat16_as_ushort(e2) | ((uint32_t)__bfloat16_as_ushort(e3) << 16);
    }
    // streaming store: the output is written once (measured 22% faster)
    v4u32 t;
    t[0] = o[0]; t[1] = o[1]; t[2] = o[2]; t[3] = o[3];
    __builtin_nontemporal_store(t, reinterpret_cast<v4u32*>(dst + c));
  }
}

// ---------------------------------------------------------------------------
// Streaming passes over a whole [rows, cols] tensor in chunks of 8 elements
// (16 B of bf16): each thread of a 256-thread workgroup loads U chunks that
// lie 256 chunks apart before it converts any of them, so that U loads per
// thread are in flight.
// ---------------------------------------------------------------------------

// Row and chunk column of flat chunk c: a 32-bit multiply-shift division below
// 2^31 chunks, a 64-bit division above.
template <bool kWide>
struct ChunkMap {
  uint32_t cpr;   // chunks per row
  FastDiv fd;     // division by cpr
  __device__ __forceinline__ void at(uint64_t c, uint64_t& r, uint32_t& cc) const {
    if constexpr (kWide) {
      r = c / cpr;
      cc = (uint32_t)(c - r * cpr);
    } else {
      const uint32_t rr = fastdiv((uint32_t)c, fd);
      r = rr;
      cc = (uint32_t)c - rr * cpr;
    }
  }
};

template <typename T, int U, bool kWide, bool kStream, typename F>
__device__ __forceinline__ void for_chunks(const T* __restrict__ x, int64_t ld_x, uint32_t cols, uint64_t nchunks,
                                           const ChunkMap<kWide>& map, F&& f) {
  const uint64_t stride = (uint64_t)gridDim.x * 256u * U;
  for (uint64_t base = (uint64_t)blockIdx.x * 256u * U + threadIdx.x; base < nchunks; base += stride) {
    Vec8<T> v[U];
    uint64_t r[U];
    uint32_t cc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t c = base + (uint64_t)u * 256u;
      if (c < nchunks) {
        map.at(c, r[u], cc[u]);
        v[u].template load<kStream>(x + (int64_t)r[u] * ld_x + cc[u] * 8u, min(8u, cols - cc[u] * 8u));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + (uint64_t)u * 256u < nchunks) f(v[u], r[u], cc[u], min(8u, cols - cc[u] * 8u));
  }
}

// ---------------------------------------------------------------------------
// Per tensor: max |x| over the whole tensor, s = amax / MAX into scales[0],
// then the cast with s. The max is taken in two steps and needs no buffer of
// the library's own: each workgroup leaves its max in a 4-byte slot of the
// code buffer q, which the cast rewrites afterwards, and one workgroup reduces
// the slots. (Same-address atomics from thousands of workgroups serialize at
// ~10 ns each, several times the pass itself.)
// ---------------------------------------------------------------------------
__global__ void k_store_zero(float* __restrict__ p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *reinterpret_cast<uint32_t*>(p) = 0u;
}

// Slot b: 4 bytes at row b / per_row, byte 4 * (b % per_row), of a row-major
// byte buffer with row pitch ld (4-byte aligned rows).
struct SlotMap {
  uint8_t* base;
  uint32_t per_row;
  int64_t ld;
  __device__ __forceinline__ uint32_t* at(uint32_t b) const {
    return reinterpret_cast<uint32_t*>(base + (int64_t)(b / per_row) * ld + (int64_t)(b % per_row) * 4);
  }
};

template <typename T, int U, bool kWide>
__global__ __launch_bounds__(256) void k_amax_slots(const T* __restrict__ x, int64_t ld_x, uint32_t cols,
                                                    uint64_t nchunks, ChunkMap<kWide> map, SlotMap slots) {
  uint32_t m = 0;
  for_chunks<T, U, kWide, false>(x, ld_x, cols, nchunks, map, [&](const Vec8<T>& v, uint64_t, uint32_t, uint32_t) {
    const uint32_t a = v.amax_bits();
    m = a > m ? a : m;
  });
  m = block256_max(m);
  if (threadIdx.x == 0) *slots.at(blockIdx.x) = m;
}

// scales[0] = max over the n <= 1024 * kSlotsPerThread slots / MAX (the same
// correctly rounded division as the group quantizers); one workgroup of 1024
// threads, each with all of its slot loads in flight together.
constexpr int kSlotsPerThread = 8;

template <int kFmt>
__global__ __launch_bounds__(1024) void k_reduce_slots(SlotMap slots, uint32_t n, float* __restrict__ scales) {
  uint32_t v[kSlotsPerThread];
#pragma unroll
  for (int k = 0; k < kSlotsPerThread; ++k) {
    const uint32_t b = threadIdx.x + 1024u * k;
    v[k] = b < n ? *slots.at(b) : 0u;
  }
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < kSlotsPerThread; ++k) m = v[k] > m ? v[k] : m;
  __shared__ uint32_t red[16];
  m = wave_max(m);
  if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) r = red[i] > r ? red[i] : r;
    scales[0] = make_group_scale<kFmt>(r).s;
  }
}

template <typename T, int kFmt, int U, bool kWide>
__global__ __launch_bounds__(256) void k_cast_tensor(const T* __restrict__ x, int64_t ld_x, uint32_t cols,
                                                     uint64_t nchunks, ChunkMap<kWide> map,
                                                     const float* __restrict__ scales, uint8_t* __restrict__ q,
                                                     int64_t ld_q) {
  // s = amax / MAX, so |x / s| <= MAX and the group quantizers' cast applies
  const GroupScale gs = make_given_scale(scales[0]);
  for_chunks<T, U, kWide, true>(x, ld_x, cols, nchunks, map, [&](const Vec8<T>& v, uint64_t r, uint32_t cc, uint32_t nv) {
    store_codes8_hint<kStreamCastCodes>(q + (int64_t)r * ld_q + cc * 8u, v.template cast<kFmt>(gs), nv);
  });
}

// Per tensor, small tensors (at most kSmallChunks * 1024 chunks of 8, 64K
// elements): one workgroup of 1024 threads holds the whole tensor in
// registers, takes the max, stores s = amax / MAX and the codes, in one
// launch instead of three. Same scale and cast as the three-kernel path.
constexpr int kSmallChunks = 8;

template <typename T, int kFmt>
__global__ __launch_bounds__(1024) void k_quant_tensor_small(const T* __restrict__ x, int64_t ld_x, uint32_t cols,
                                                             uint32_t nchunks, FastDiv div_cpr, uint32_t cpr,
                                                             uint8_t* __restrict__ q, int64_t ld_q,
                                                             float* __restrict__ scales) {
  Vec8<T> v[kSmallChunks];
  uint32_t r[kSmallChunks], cc[kSmallChunks], nv[kSmallChunks];
#pragma unroll
  for (int i = 0; i < kSmallChunks; ++i) {
    const uint32_t c = threadIdx.x + 1024u * i;
    r[i] = c < nchunks ? fastdiv(c, div_cpr) : 0u;
    cc[i] = c - r[i] * cpr;
    nv[i] = c < nchunks ? min(8u, cols - cc[i] * 8u) : 0u;
    if (nv[i] > 0)
      v[i].template load<false>(x + (int64_t)r[i] * ld_x + cc[i] * 8u, nv[i]);
    else
      v[i].zero();
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kSmallChunks; ++i) {
    const uint32_t a = v[i].amax_bits();
    m = a > m ? a : m;
  }
  __shared__ uint32_t red[16];
  m = wave_max(m);
  if ((threadIdx.x & 63u) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = red[i] > m ? red[i] : m;
  const GroupScale gs = make_group_scale<kFmt>(m);
#pragma unroll
  for (int i = 0; i < kSmallChunks; ++i)
    if (nv[i] > 0) store_codes8(q + (int64_t)r[i] * ld_q + cc[i] * 8u, v[i].template cast<kFmt>(gs), nv[i]);
  if (threadIdx.x == 0) scales[0] = gs.s;
}

// ---------------------------------------------------------------------------
// MX blocks: 32 consecutive elements of a row share one power-of-two scale
// X = 2^k, stored as the byte k + 127 (E8M0), with k the smallest integer such
// that amax <= MAX * 2^k ([VS] api.makesence.top, "LLM推理量化:FP8 versus INT8",
// section 3: Microscaling with block size 32; the pages' s = amax / MAX rounded
// up to a power of two, so that the block max never saturates). With
// MAX = 0.875 * 2^E and amax = m * 2^e (m in [0.5, 1), frexp), k = e - E +
// (m > 0.875); an all-zero block takes k = -127; k is clamped to [-127, 127].
// The codes are FP8(x * 2^-k), the scaling exact, so only the encoder rounds.
// Four lanes (a DPP quad) per block, 8 elements each; one block per quad.
// ---------------------------------------------------------------------------
template <int kFmt>
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  const float a = __uint_as_float(amax_bits);
  const int e = __builtin_amdgcn_frexp_expf(a);
  const float m = __builtin_amdgcn_frexp_mantf(a);
  constexpr int kE = kFmt == FMT_E4M3 ? 9 : 16;   // MAX = 0.875 * 2^kE
  const int k = e - kE + (m > 0.875f ? 1 : 0);
  return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// 64-block units per workgroup, each thread's loads all in flight before any
// arithmetic: 2 measured 10.5 against 11.1 us for 1 at 4096 x 4096 (4: 10.6)
constexpr int kMxUnroll = 2;

template <typename T, int kFmt>
__global__ __launch_bounds__(256) void k_quant_mx(const T* __restrict__ x, int64_t ld_x, uint32_t cols,
                                                   uint32_t nblk, uint32_t total_blocks, FastDiv div_nblk,
                                                   uint8_t* __restrict__ q, int64_t ld_q,
                                                   uint8_t* __restrict__ sc, int64_t ld_s) {
  const uint32_t sub = threadIdx.x & 3u;
  Vec8<T> v[kMxUnroll];
  uint32_t row[kMxUnroll], blk[kMxUnroll], col0[kMxUnroll], nv[kMxUnroll];
  bool live[kMxUnroll];
  // all loads first: block b of unit u is blockIdx.x * 64 kMxUnroll + 64 u + thread / 4
#pragma unroll
  for (int u = 0; u < kMxUnroll; ++u) {
    const uint32_t b = (blockIdx.x * kMxUnroll + u) * 64u + (threadIdx.x >> 2);
    live[u] = b < total_blocks;
    row[u] = live[u] ? fastdiv(b, div_nblk) : 0u;
    blk[u] = b - row[u] * nblk;
    col0[u] = blk[u] * 32u + sub * 8u;
    nv[u] = (live[u] && col0[u] < cols) ? min(8u, cols - col0[u]) : 0u;
    if (nv[u] > 0)
      v[u].load(x + (int64_t)row[u] * ld_x + col0[u], nv[u]);
    else
      v[u].zero();
  }
#pragma unroll
  for (int u = 0; u < kMxUnroll; ++u) {
    uint32_t m = v[u].amax_bits();
    m = dpp_max_step<0xB1>(m);   // quad_perm [1,0,3,2]
    m = dpp_max_step<0x4E>(m);   // quad_perm [2,3,0,1]
    const int k = mx_exponent<kFmt>(m);
    if (nv[u] > 0) {
      const uint2 codes = v[u].template cast_pow2<kFmt>(-k);
      store_codes8_hint<kStreamCastCodes>(q + (int64_t)row[u] * ld_q + col0[u], codes, nv[u]);
    }
    if (live[u] && sub == 0) sc[(int64_t)row[u] * ld_s + blk[u]] = (uint8_t)(k + 127);
  }
}

// ---------------------------------------------------------------------------
// Static / delayed scaling ([MIXED] charles2530.github.io, "量化：FP8 与混合精度推理",
// section "scale 是控制面": the scale may come from history instead of the
// current batch, as Transformer Engine's delayed scaling updates it from
// recorded amax values; [VS] api.makesence.top section 2 trains with delayed
// scaling). The codes use a scale read from device memory; the pass can record
// the tensor's own amax for the caller's history. The scale from a history is
// max(history) / MAX.
// ---------------------------------------------------------------------------
// How the static cast records the tensor's amax.
enum AmaxMode { AMAX_NONE = 0, AMAX_SLOTS = 1, AMAX_ATOMIC = 2 };

// The slot of workgroup b of a streaming pass: 4 code bytes of its first chunk
// c0 = b * 256 * U, or of the next chunk when c0 ends a row with fewer than 4
// elements (the next chunk then starts a row, and rows hold >= 4 elements
// where slots are used). None (~0) when c0 is the tensor's last chunk and
// short; that workgroup then converts c0 alone.
template <bool kWide>
__device__ __forceinline__ uint64_t slot_chunk(uint64_t c0, uint64_t nchunks, const ChunkMap<kWide>& map,
                                               uint32_t cols) {
  uint64_t r;
  uint32_t cc;
  map.at(c0, r, cc);
  if (cols - cc * 8u >= 4u) return c0;
  if (c0 + 1 < nchunks) return c0 + 1;
  return ~0ull;
}

// AMAX_SLOTS: each workgroup overwrites its slot (4 codes it has just written)
// with its max; k_static_amax_restore then reduces the slots into amax_out and
// writes the 4 codes of every slot again. No atomics and no buffer beyond q.
// AMAX_ATOMIC (tensors narrower than 4 columns, which have no slots): an
// atomic max after an agent-scope read of the current value.
template <typename T, int kFmt, int U, bool kWide, int kAmax>
__global__ __launch_bounds__(256) void k_cast_static(const T* __restrict__ x, int64_t ld_x, uint32_t cols,
                                                     uint64_t nchunks, ChunkMap<kWide> map,
                                                     const float* __restrict__ scale, uint8_t* __restrict__ q,
                                                     int64_t ld_q, float* __restrict__ amax_out) {
  const GroupScale gs = make_given_scale(*scale);
  if constexpr (kAmax == AMAX_SLOTS) {
    // k_static_amax_restore merges into amax_out after this kernel
    if (blockIdx.x == 0 && threadIdx.x == 0) *reinterpret_cast<uint32_t*>(amax_out) = 0u;
  }
  uint32_t m = 0;
  for_chunks<T, U, kWide, true>(x, ld_x, cols, nchunks, map, [&](const Vec8<T>& v, uint64_t r, uint32_t cc, uint32_t nv) {
    if constexpr (kAmax != AMAX_NONE) {
      const uint32_t a = v.amax_bits();
      m = a > m ? a : m;
    }
    store_codes8_hint<kStreamCastCodes>(q + (int64_t)r * ld_q + cc * 8u, v.template cast_sat<kFmt>(gs), nv);
  });
  if constexpr (kAmax == AMAX_SLOTS) {
    m = block256_max(m);
    const uint64_t c0 = (uint64_t)blockIdx.x * 256u * U;
    const uint64_t sc = slot_chunk(c0, nchunks, map, cols);
    // the thread that wrote the slot's codes (thread 0 or 1) overwrites them
    if (sc != ~0ull && threadIdx.x == (uint32_t)(sc - c0)) {
      uint64_t r;
      uint32_t cc;
      map.at(sc, r, cc);
      *reinterpret_cast<uint32_t*>(q + (int64_t)r * ld_q + cc * 8u) = m;
    }
  } else if constexpr (kAmax == AMAX_ATOMIC) {
    // the value only grows from the zero stored before this kernel, so a
    // workgroup whose max does not exceed the current value skips its atomic
    m = block256_max(m);
    if (threadIdx.x == 0) {
      unsigned int* p = reinterpret_cast<unsigned int*>(amax_out);
      if (m > __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(p, m);
    }
  }
}

// amax_out[0] = max over the slots of the nblocks workgroups of
// k_cast_static<..., AMAX_SLOTS> (or over the lone short chunk of a workgroup
// without a slot), and the 4 codes of every slot written again with the same
// conversion. One thread per slot; each workgroup merges its max into
// amax_out (zeroed by the cast kernel) with one atomic, so a few atomics in
// all.
template <typename T, int kFmt, int U, bool kWide>
__global__ __launch_bounds__(256) void k_static_amax_restore(const T* __restrict__ x, int64_t ld_x, uint32_t cols,
                                                             uint64_t nchunks, ChunkMap<kWide> map, uint32_t nblocks,
                                                             const float* __restrict__ scale,
                                                             uint8_t* __restrict__ q, int64_t ld_q,
                                                             float* __restrict__ amax_out) {
  const uint32_t b = blockIdx.x * 256u + threadIdx.x;
  uint32_t m = 0;
  if (b < nblocks) {
    const uint64_t c0 = (uint64_t)b * 256u * U;
    const uint64_t sc = slot_chunk(c0, nchunks, map, cols);
    uint64_t r;
    uint32_t cc;
    map.at(sc != ~0ull ? sc : c0, r, cc);
    Vec8<T> v;
    v.template load<false>(x + (int64_t)r * ld_x + cc * 8u, min(8u, cols - cc * 8u));
    if (sc != ~0ull) {
      uint32_t* p = reinterpret_cast<uint32_t*>(q + (int64_t)r * ld_q + cc * 8u);
      m = *p;
      *p = v.template cast_sat<kFmt>(make_given_scale(*scale)).x;
    } else {
      m = v.amax_bits();   // a workgroup without a slot had this one short chunk only
    }
  }
  m = block256_max(m);
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(amax_out), m);
}

// scale_out[0] = max(history[0 .. n)) / MAX (one workgroup; history >= 0).
template <int kFmt>
__global__ __launch_bounds__(256) void k_scale_from_history(const float* __restrict__ history, uint32_t n,
                                                            float* __restrict__ scale_out) {
  uint32_t m = 0;
  for (uint32_t i = threadIdx.x; i < n; i += 256u) {
    const uint32_t a = __float_as_uint(history[i]) & 0x7fffffffu;
    m = a > m ? a : m;
  }
  m = block256_max(m);
  if (threadIdx.x == 0) scale_out[0] = __uint_as_float(m) / Fp8<kFmt>::kMax;
}

// ---------------------------------------------------------------------------
// Host launchers (arguments already validated by the API layer).
// ---------------------------------------------------------------------------
namespace {
constexpr int kGroupUnroll = 1;   // 1 group per 8 lanes: measured 6-10% faster than 2 or 4
// calls whose groups are all full take the kFull kernels (bit-identical; K + V
// [8, 131072, 128] 124.0 -> 120.5 us, weights [14336, 4096] 31.6 -> 30.4 us)
constexpr bool kTileFull = true;

// Chunks in flight per thread: the amax-only pass, the cast passes (per-tensor
// cast and static cast without an amax record; 4 measured 15.5 against 17.7 us
// for 2 and 18.3 us for 8 per tensor at 4096 x 4096), and the static cast that
// records the amax (2 and 4 within 2%, 8 slower).
constexpr int kAmaxUnroll = 4;
constexpr int kCastUnroll = 4;
constexpr int kStaticUnroll = 4;
constexpr uint64_t kMaxStreamGrid = 8192;  // workgroups of a streaming pass (grid-stride beyond)

uint32_t stream_grid(uint64_t nchunks, int unroll) {
  const uint64_t want = (nchunks + 256ull * unroll - 1) / (256ull * unroll);
  return (uint32_t)(want < kMaxStreamGrid ? want : kMaxStreamGrid);
}

template <bool kWide>
ChunkMap<kWide> make_chunk_map(uint32_t cols) {
  ChunkMap<kWide> m;
  m.cpr = (cols + 7u) >> 3;
  m.fd = make_fastdiv(m.cpr);
  return m;
}

// amax into slots of q, slots into the scale, cast. Tensors with fewer than 4
// columns have no slot in q; one workgroup then uses scales[0] as its slot.
template <typename T, int kFmt, bool kWide>
void per_tensor_passes(const QuantArgs& a, const T* x, uint64_t nchunks, hipStream_t st) {
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const ChunkMap<kWide> map = make_chunk_map<kWide>(cols);
  const uint64_t per_row = cols / 4u;
  const uint64_t nslots = (uint64_t)rows * per_row;
  uint32_t g = stream_grid(nchunks, kAmaxUnroll);
  if (g > 1024u * kSlotsPerThread) g = 1024u * kSlotsPerThread;
  SlotMap sm;
  if (nslots == 0) {
    g = 1;
    sm.base = reinterpret_cast<uint8_t*>(a.scales);
    sm.per_row = 1;
    sm.ld = 4;
  } else {
    if (g > nslots) g = (uint32_t)nslots;
    sm.base = a.q;
    sm.per_row = (uint32_t)per_row;
    sm.ld = a.ld_q;
  }
  hipLaunchKernelGGL((k_amax_slots<T, kAmaxUnroll, kWide>), dim3(g), dim3(256), 0, st, x, a.ld_x, cols, nchunks,
                     map, sm);
  hipLaunchKernelGGL(k_reduce_slots<kFmt>, dim3(1), dim3(1024), 0, st, sm, g, a.scales);
  hipLaunchKernelGGL((k_cast_tensor<T, kFmt, kCastUnroll, kWide>), dim3(stream_grid(nchunks, kCastUnroll)), dim3(256),
                     0, st, x, a.ld_x, cols, nchunks, map, a.scales, a.q, a.ld_q);
}

template <typename T, int kFmt>
hipError_t quantize_typed(const QuantArgs& a, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  if (a.gran == GRAN_PER_TENSOR) {
    if (rows == 0 || cols == 0) {
      hipLaunchKernelGGL(k_store_zero, dim3(1), dim3(64), 0, st, a.scales);
      return hipGetLastError();
    }
    const uint64_t nchunks = (uint64_t)rows * ((cols + 7u) >> 3);
    if (nchunks <= 1024ull * kSmallChunks) {
      const uint32_t cpr = (cols + 7u) >> 3;
      hipLaunchKernelGGL((k_quant_tensor_small<T, kFmt>), dim3(1), dim3(1024), 0, st, x, a.ld_x, cols,
                         (uint32_t)nchunks, make_fastdiv(cpr), cpr, a.q, a.ld_q, a.scales);
    } else if (nchunks < (1ull << 31))
      per_tensor_passes<T, kFmt, false>(a, x, nchunks, st);
    else
      per_tensor_passes<T, kFmt, true>(a, x, nchunks, st);
    return hipGetLastError();
  }
  if (rows == 0 || cols == 0) return hipSuccess;
  if (a.gran == GRAN_GROUP_1x128) {
    const uint32_t ngroups = (cols + 127u) / 128u;
    if (a.ss_row == 1 && ngroups > 1 && rows >= 8) {
      // K-block-major scales: units of 8 rows x 4 groups
      const uint32_t gunits = (ngroups + 3u) / 4u;
      const uint32_t total = ((rows + 7u) / 8u) * gunits;
      const uint32_t grid = (total + kGroupUnroll - 1) / kGroupUnroll;
      hipLaunchKernelGGL((k_quant_group_1x128<T, kGroupUnroll, kFmt, true>), dim3(grid), dim3(256), 0, st, x,
                         a.ld_x, rows, cols, ngroups, total, make_fastdiv(gunits), gunits, a.q, a.ld_q, a.scales,
                         a.ss_row, a.ss_col);
    } else {
      const uint32_t total = rows * ngroups;
      const uint32_t per_block = 32u * kGroupUnroll;
      const uint32_t grid = (total + per_block - 1) / per_block;
      hipLaunchKernelGGL((k_quant_group_1x128<T, kGroupUnroll, kFmt, false>), dim3(grid), dim3(256), 0, st, x,
                         a.ld_x, rows, cols, ngroups, total, make_fastdiv(ngroups), ngroups, a.q, a.ld_q, a.scales,
                         a.ss_row, a.ss_col);
    }
    return hipGetLastError();
  }
  // 128x128 blocks
  const dim3 grid((cols + 127u) / 128u, (rows + 127u) / 128u);
  if (kTileFull && rows % 128u == 0 && cols % 128u == 0)
    hipLaunchKernelGGL((k_quant_block_128x128<T, kFmt, true>), grid, dim3(256), 0, st, x, a.ld_x, rows, cols, a.q,
                       a.ld_q, a.scales, a.ss_row, a.ss_col);
  else
    hipLaunchKernelGGL((k_quant_block_128x128<T, kFmt, false>), grid, dim3(256), 0, st, x, a.ld_x, rows, cols, a.q,
                       a.ld_q, a.scales, a.ss_row, a.ss_col);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
  if (a.fmt == FMT_E5M2) {
    if (a.x_dtype == DTYPE_BF16) return quantize_typed<__hip_bfloat16, FMT_E5M2>(a, st);
    return quantize_typed<float, FMT_E5M2>(a, st);
  }
  if (a.x_dtype == DTYPE_BF16) return quantize_typed<__hip_bfloat16, FMT_E4M3>(a, st);
  return quantize_typed<float, FMT_E4M3>(a, st);
}

hipError_t launch_quantize_mx(const QuantArgs& a, hipStream_t st) {
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  if (rows == 0 || cols == 0) return hipSuccess;
  const uint32_t nblk = (cols + 31u) / 32u;
  const uint32_t total = rows * nblk;
  const dim3 grid((total + 64u * kMxUnroll - 1u) / (64u * kMxUnroll));
  uint8_t* const sc = reinterpret_cast<uint8_t*>(a.scales);
  const FastDiv fd = make_fastdiv(nblk);
  if (a.x_dtype == DTYPE_BF16) {
    const __hip_bfloat16* x = static_cast<const __hip_bfloat16*>(a.x);
    if (a.fmt == FMT_E5M2)
      hipLaunchKernelGGL((k_quant_mx<__hip_bfloat16, FMT_E5M2>), grid, dim3(256), 0, st, x, a.ld_x, cols, nblk, total, fd, a.q, a.ld_q, sc, a.ss_row);
    else
      hipLaunchKernelGGL((k_quant_mx<__hip_bfloat16, FMT_E4M3>), grid, dim3(256), 0, st, x, a.ld_x, cols, nblk, total, fd, a.q, a.ld_q, sc, a.ss_row);
  } else {
    const float* x = static_cast<const float*>(a.x);
    if (a.fmt == FMT_E5M2)
      hipLaunchKernelGGL((k_quant_mx<float, FMT_E5M2>), grid, dim3(256), 0, st, x, a.ld_x, cols, nblk, total, fd, a.q, a.ld_q, sc, a.ss_row);
    else
      hipLaunchKernelGGL((k_quant_mx<float, FMT_E4M3>), grid, dim3(256), 0, st, x, a.ld_x, cols, nblk, total, fd, a.q, a.ld_q, sc, a.ss_row);
  }
  return hipGetLastError();
}

namespace {
template <typename T, int kFmt, bool kWide>
void static_pass(const QuantArgs& a, uint64_t nchunks, const float* scale, float* amax_out, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  const uint32_t cols = (uint32_t)a.cols;
  const ChunkMap<kWide> map = make_chunk_map<kWide>(cols);
  if (!amax_out) {
    hipLaunchKernelGGL((k_cast_static<T, kFmt, kCastUnroll, kWide, AMAX_NONE>), dim3(stream_grid(nchunks, kCastUnroll)),
                       dim3(256), 0, st, x, a.ld_x, cols, nchunks, map, scale, a.q, a.ld_q, amax_out);
  } else if (cols >= 4) {
    // at most 2048 workgroups: at most 8 restore workgroups and atomics
    uint32_t g = stream_grid(nchunks, kStaticUnroll);
    if (g > 2048u) g = 2048u;
    hipLaunchKernelGGL((k_cast_static<T, kFmt, kStaticUnroll, kWide, AMAX_SLOTS>), dim3(g), dim3(256), 0, st, x,
                       a.ld_x, cols, nchunks, map, scale, a.q, a.ld_q, amax_out);
    hipLaunchKernelGGL((k_static_amax_restore<T, kFmt, kStaticUnroll, kWide>), dim3((g + 255u) / 256u), dim3(256), 0, st,
                       x, a.ld_x, cols, nchunks, map, g, scale, a.q, a.ld_q, amax_out);
  } else {
    hipLaunchKernelGGL(k_store_zero, dim3(1), dim3(64), 0, st, amax_out);
    hipLaunchKernelGGL((k_cast_static<T, kFmt, kAmaxUnroll, kWide, AMAX_ATOMIC>), dim3(stream_grid(nchunks, kAmaxUnroll)),
                       dim3(256), 0, st, x, a.ld_x, cols, nchunks, map, scale, a.q, a.ld_q, amax_out);
  }
}

template <typename T, int kFmt>
void static_typed(const QuantArgs& a, uint64_t nchunks, const float* scale, float* amax_out, hipStream_t st) {
  if (nchunks < (1ull << 31))
    static_pass<T, kFmt, false>(a, nchunks, scale, amax_out, st);
  else
    static_pass<T, kFmt, true>(a, nchunks, scale, amax_out, st);
}
}  // namespace

hipError_t launch_quantize_static(const QuantArgs& a, const float* scale, float* amax_out, hipStream_t st) {
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  if (rows == 0 || cols == 0) {
    if (!amax_out) return hipSuccess;
    hipLaunchKernelGGL(k_store_zero, dim3(1), dim3(64), 0, st, amax_out);
    return hipGetLastError();
  }
  const uint64_t nchunks = (uint64_t)rows * ((cols + 7u) >> 3);
  if (a.x_dtype == DTYPE_BF16) {
    if (a.fmt == FMT_E5M2)
      static_typed<__hip_bfloat16, FMT_E5M2>(a, nchunks, scale, amax_out, st);
    else
      static_typed<__hip_bfloat16, FMT_E4M3>(a, nchunks, scale, amax_out, st);
  } else {
    if (a.fmt == FMT_E5M2)
      static_typed<float, FMT_E5M2>(a, nchunks, scale, amax_out, st);
    else
      static_typed<float, FMT_E4M3>(a, nchunks, scale, amax_out, st);
  }
  return hipGetLastError();
}

hipError_t launch_scale_from_history(const float* history, int64_t n, int fmt, float* scale_out, hipStream_t st) {
  if (fmt == FMT_E5M2)
    hipLaunchKernelGGL(k_scale_from_history<FMT_E5M2>, dim3(1), dim3(256), 0, st, history, (uint32_t)n, scale_out);
  else
    hipLaunchKernelGGL(k_scale_from_history<FMT_E4M3>, dim3(1), dim3(256), 0, st, history, (uint32_t)n, scale_out);
  return hipGetLastError();
}

hipError_t launch_kv_quantize(const KvArgs& a, hipStream_t st) {
  if (a.heads == 0 || a.tokens == 0) return hipSuccess;
  const dim3 grid((uint32_t)((a.tokens + a.token_block - 1) / a.token_block), (uint32_t)a.heads);
  const bool full = kTileFull && a.token_block == 128 && a.head_dim == 128 && a.tokens % 128 == 0;
  auto kernel = a.fmt == FMT_E5M2 ? (full ? k_kv_quant<FMT_E5M2, true> : k_kv_quant<FMT_E5M2, false>)
                                  : (full ? k_kv_quant<FMT_E4M3, true> : k_kv_quant<FMT_E4M3, false>);
  hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st,
                     static_cast<const __hip_bfloat16*>(a.kv), a.stride_head, a.stride_token,
                     (uint32_t)a.tokens, (uint32_t)a.head_dim, (uint32_t)a.token_block, a.q,
                     a.scales);
  return hipGetLastError();
}

hipError_t launch_kv_dequantize(const KvArgs& a, hipStream_t st) {
  if (a.heads == 0 || a.tokens == 0) return hipSuccess;
  const dim3 grid((uint32_t)((a.tokens + a.token_block - 1) / a.token_block), (uint32_t)a.heads);
  auto kernel = a.fmt == FMT_E5M2 ? k_kv_dequant<FMT_E5M2> : k_kv_dequant<FMT_E4M3>;
  hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, a.q_in, a.scales_in, (uint32_t)a.tokens,
                     (uint32_t)a.head_dim, (uint32_t)a.token_block,
                     static_cast<__hip_bfloat16*>(a.out));
  return hipGetLastError();
}

}  // namespace fp8blk
