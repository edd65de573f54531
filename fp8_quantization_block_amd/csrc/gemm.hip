// Block-scaled FP8 GEMM on CDNA4 FP8 MFMA.
//
// C[m][n] = sum_j s_a(m, j) * s_b(n / 128, j) * P_j[m][n], with
// P_j = the FP8 x FP8 product of the 128-wide K block j summed in fp32.
// [FP8] wangyu.me, "大语言模型量化技术（五）：FP8", section "激活动态量化" (sum over
// K blocks of activation scale x weight-block scale x FP8 block product) and
// section "FP8 矩阵乘" (FP8 products, fp32 accumulation, partial results
// multiplied by their scales); [MIXED] charles2530.github.io, "量化：FP8 与混合精度推理",
// section "混合精度才是生产形态" (low-precision products, higher-precision sums).
//
// Design (gfx950):
// * One v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep scale block,
//   so every MFMA starts from zero and its 16x16 fp32 result is promoted into
//   the fp32 accumulator with one FMA per element: acc += P_j * s_a * s_b.
// * Workgroup tile 256 x 256, K step 128; 8 waves in a 4 x 2 grid, each wave
//   owning 64 rows x 128 columns (so a wave's columns are exactly one weight
//   scale block and s_b is one scalar per K block).
// * A and B tiles (and the K block's 256 activation scales and 2 weight-block
//   scales) are double buffered in LDS, one barrier per K block. The next
//   block's tiles travel through 16 registers per thread in two halves: the A
//   tile is loaded while the first half of the block's MFMAs run and written
//   to LDS after them, then the B tile the same way around the second half.
//   (Direct global-to-LDS copies did not overlap with the MFMA work on this
//   chip; the register route does.) Rows are stored with their eight 16-byte
//   chunks XOR-swizzled so the MFMA operand reads are conflict free.
// * Workgroup ids are remapped so that neighbouring tiles (which share A rows
//   or B columns) run on the same XCD and share its L2.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 512;
constexpr int kTileBytes = BM * BK;                 // one operand tile, 32 KB

struct GemmParams {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  void* c;
  int64_t lda, ldb, ldc;
  int64_t sa_m, sa_k, sb_n, sb_k;
  int M, N, K;
  int tiles_m, tiles_n;
};

// A 128-byte operand row holds eight 16-byte chunks; logical chunk c of row r
// is stored at physical chunk c ^ swz(r). Any 16 consecutive rows then hit 16
// distinct (row parity, chunk) pairs and any 8 consecutive rows 8 distinct
// chunks, so the fragment reads (16 rows, same logical chunk) and the tile
// writes (8 lanes per row) are free of bank conflicts whether the LDS serves
// 8 or 16 lanes of a 128-bit access per cycle.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Buffer resource over `bytes` bytes from `base` (raw, untyped loads; reads
// at or past `bytes` return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// Operand fragment of one 16-row (or 16-column) subtile: lane l takes row
// base + l % 16 and the 32 bytes at K offset 32 * (l / 16). A and B use the
// same K assignment, so the MFMA sums exactly the 128 products of the block.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int lane) {
  const int lc0 = (lane >> 4) * 2;
  const int sw = swz(row);
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * 128 + ((lc0 ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * 128 + (((lc0 + 1) ^ sw) << 4));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Multiply the four 16-column subtiles ni0 .. ni0 + 3 of this wave against
// its four 16-row A fragments and promote every 16 x 16 partial into acc.
template <int ni0>
__device__ __forceinline__ void mma_half(const uint8_t* tb, int wn, int lane, const v8i (&af)[4],
                                         const v4f (&comb)[4], v4f (&acc)[4][8]) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ni = ni0; ni < ni0 + 4; ++ni) {
    const v8i bf = read_frag(tb, wn * 128 + ni * 16 + (lane & 15), lane);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bf, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mi][ni][v] = __builtin_fmaf(part[v], comb[mi][v], acc[mi][ni][v]);
    }
  }
}

// One K block's operands in flight in registers: thread t holds chunks
// c = t + 512 i (i = 0..3) of the A and the B tile (row c / 8, logical chunk
// c % 8), and one scale (an activation scale for t < 256, a weight-block
// scale for t = 256, 257).
struct Regs {
  uint4 a[4];
  uint4 b[4];
  float s;
};

// Per-thread copy plan. Global offsets are relative to the tile's first row
// (so they fit 32 bits: 256 * ld < 2^31 is checked on the host); rows past the
// operand's end fall outside the buffer resource and read as zero. The four
// LDS destinations of a thread are 64 rows apart, which keeps the same swizzle,
// so one offset plus immediates addresses them.
struct Copier {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t goa[4], gob[4];
  uint32_t loff;      // LDS byte offset of chunk 0; chunk i adds 8192 * i
  const float* sp;    // this thread's scale for K block 0 (threads 0..257)
  int64_t s_kstep;    // element step of that scale per K block
  int tid;
};

__device__ __forceinline__ void load_a(const Copier& c, int kb, Regs& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.a[i] = buf_load16(c.ra, c.goa[i], (uint32_t)kb * BK);
}
__device__ __forceinline__ void load_b(const Copier& c, int kb, Regs& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) r.b[i] = buf_load16(c.rb, c.gob[i], (uint32_t)kb * BK);
  r.s = c.tid < 258 ? c.sp[(int64_t)kb * c.s_kstep] : 0.f;
}
__device__ __forceinline__ void store_a(const Copier& c, const Regs& r, uint8_t* ta) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(ta + c.loff + 8192 * i) = r.a[i];
}
__device__ __forceinline__ void store_b(const Copier& c, const Regs& r, uint8_t* tb, float* ts) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(tb + c.loff + 8192 * i) = r.b[i];
  if (c.tid < 258) ts[c.tid] = r.s;
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier that waits for this wave's LDS writes but not for its
// global loads in flight; the empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  wait_lds();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One K block. On entry `r` holds block kb + 1 (loaded during the previous
// block) and stage nxt_* is free. The A half of r goes to LDS and is reloaded
// with block kb + 2, the first half of block kb's MFMAs runs, then the B half
// and the scales move the same way before the second half of the MFMAs. The
// LDS writes thus arrive as two 32 KB bursts between fragment reads, and every
// load has a whole block of work to arrive. Block indices are clamped to the
// last block (the tail re-copies it into a stage nobody reads again), so every
// step has the same shape.
__device__ __forceinline__ void block_step(const Copier& cp, Regs& r, int kb, int nk, int wm,
                                           int wn, int lane, bool active, const uint8_t* cur_a,
                                           const uint8_t* cur_b, const float* cur_s,
                                           uint8_t* nxt_a, uint8_t* nxt_b, float* nxt_s,
                                           v4f (&acc)[4][8]) {
  const int kl = min(kb + 2, nk - 1);
  v8i af[4];
  v4f comb[4];
  if (active) {
    const float sbv = cur_s[256 + wn];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      af[mi] = read_frag(cur_a, wm * 64 + mi * 16 + (lane & 15), lane);
      const v4f s4 = *reinterpret_cast<const v4f*>(cur_s + wm * 64 + mi * 16 + 4 * (lane >> 4));
      comb[mi] = s4 * sbv;
    }
  }
  store_a(cp, r, nxt_a);
  load_a(cp, kl, r);
  __builtin_amdgcn_sched_barrier(0);
  if (active) mma_half<0>(cur_b, wn, lane, af, comb, acc);
  __builtin_amdgcn_sched_barrier(0);
  store_b(cp, r, nxt_b, nxt_s);
  load_b(cp, kl, r);
  __builtin_amdgcn_sched_barrier(0);
  if (active) mma_half<4>(cur_b, wn, lane, af, comb, acc);
  lds_barrier();
}

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_fp8_block(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t a0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[kTileBytes];
  __shared__ __attribute__((aligned(16))) float s0[BM + 4];
  __shared__ __attribute__((aligned(1024))) uint8_t a1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t b1[kTileBytes];
  __shared__ __attribute__((aligned(16))) float s1[BM + 4];

  // ---- tile assignment: XCD-major remap, then grouped row-major order ----
  const int nwg = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  constexpr int kGroupM = 8;
  const int group = bid / (kGroupM * p.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(p.tiles_m - first_m, kGroupM);
  const int in_group = bid - group * kGroupM * p.tiles_n;
  const int m0 = (first_m + in_group % gm) * BM;
  const int n0 = (in_group / gm) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wm = wave >> 1;          // 0..3 : 64-row slab
  const int wn = wave & 1;           // 0..1 : 128-column slab
  const bool active = (n0 + wn * 128) < p.N;

  Copier cp;
  cp.tid = tid;
  const int rows_a = min(p.M - m0, BM), rows_b = min(p.N - n0, BN);
  cp.ra = make_rsrc(p.a + (int64_t)m0 * p.lda, (uint32_t)(rows_a * p.lda));
  cp.rb = make_rsrc(p.b + (int64_t)n0 * p.ldb, (uint32_t)(rows_b * p.ldb));
  {
    const int row = tid >> 3, lc = tid & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      cp.goa[i] = (uint32_t)((row + 64 * i) * (int)p.lda + lc * 16);
      cp.gob[i] = (uint32_t)((row + 64 * i) * (int)p.ldb + lc * 16);
    }
    cp.loff = (uint32_t)(row * 128 + ((lc ^ swz(row)) << 4));
  }
  // scales: threads 0..255 copy the activation scale of tile row tid, threads
  // 256 and 257 the weight-block scales of the tile's two 128-column halves
  if (tid < 256) {
    cp.sp = p.sa + (int64_t)min(m0 + tid, p.M - 1) * p.sa_m;
    cp.s_kstep = p.sa_k;
  } else {
    cp.sp = p.sb + (int64_t)min((n0 >> 7) + (tid - 256), (p.N >> 7) - 1) * p.sb_n;
    cp.s_kstep = p.sb_k;
  }

  v4f acc[4][8];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / BK;
  Regs r;
  load_a(cp, 0, r);
  load_b(cp, 0, r);
  store_a(cp, r, a0);
  store_b(cp, r, b0, s0);
  load_a(cp, min(1, nk - 1), r);
  load_b(cp, min(1, nk - 1), r);
  lds_barrier();

  for (int kb = 0; kb < nk; kb += 2) {
    block_step(cp, r, kb, nk, wm, wn, lane, active, a0, b0, s0, a1, b1, s1, acc);
    if (kb + 1 < nk) block_step(cp, r, kb + 1, nk, wm, wn, lane, active, a1, b1, s1, a0, b0, s0, acc);
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no load outstanding past the loop

  if (!active) return;
  // ---- epilogue: lane holds rows 4 * (lane / 16) + v, column lane % 16 ----
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + wm * 64 + mi * 16 + 4 * (lane >> 4) + v;
      if (row >= p.M) continue;
#pragma unroll
      for (int ni = 0; ni < 8; ++ni) {
        const int col = n0 + wn * 128 + ni * 16 + (lane & 15);
        if (kBf16Out) {
          __hip_bfloat16* c = static_cast<__hip_bfloat16*>(p.c);
          c[(int64_t)row * p.ldc + col] = __float2bfloat16(acc[mi][ni][v]);
        } else {
          float* c = static_cast<float*>(p.c);
          c[(int64_t)row * p.ldc + col] = acc[mi][ni][v];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode-shaped GEMM (M <= 64): bound by streaming the weights from HBM once.
//
// A workgroup owns 64 output columns (four 16-column subtiles) for every
// row of C and splits K eight ways over its waves. Weight fragments go from
// global memory straight into MFMA operand registers (each weight byte is
// used once, so LDS staging would only add traffic); the next K block's
// fragments are loaded while the current one is multiplied. The MFMA's first
// operand is the weight subtile and its second the activations, so a lane's
// four results share one activation row (one s_a) and the subtile shares one
// s_b. The eight partial sums are added through LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 512;
constexpr int kDecSplit = kDecThreads / 64;
constexpr int kDecBN = 64;

template <int MT>
struct DecFrags {
  v8i w[4];
  v8i a[MT];
  float sa[MT];
  float sw;
};

__device__ __forceinline__ v8i load_frag32(const uint8_t* p) {
  const uint4 lo = reinterpret_cast<const uint4*>(p)[0];
  const uint4 hi = reinterpret_cast<const uint4*>(p)[1];
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

template <int MT, bool kBf16Out>
__global__ __launch_bounds__(kDecThreads) void k_gemm_fp8_decode(GemmParams p) {
  __shared__ float red[kDecSplit][4 * MT * 64 * 4];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kDecBN;
  const int nk = p.K / 128;
  const int kb0 = (nk * wave) / kDecSplit;
  const int kb1 = (nk * (wave + 1)) / kDecSplit;
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 32;          // this lane's 32 bytes of a K block

  const uint8_t* wrow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) wrow[ns] = p.b + (int64_t)(n0 + ns * 16 + r16) * p.ldb + kq;
  const uint8_t* arow[MT];
  const float* sarow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r16, p.M - 1);
    arow[mt] = p.a + (int64_t)m * p.lda + kq;
    sarow[mt] = p.sa + (int64_t)m * p.sa_m;
  }
  const float* swrow = p.sb + (int64_t)(n0 >> 7) * p.sb_n;

  auto load = [&](int kb) {
    DecFrags<MT> f;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) f.w[ns] = load_frag32(wrow[ns] + (int64_t)kb * 128);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f.a[mt] = load_frag32(arow[mt] + (int64_t)kb * 128);
      f.sa[mt] = sarow[mt][(int64_t)kb * p.sa_k];
    }
    f.sw = swrow[(int64_t)kb * p.sb_k];
    return f;
  };

  v4f acc[4][MT];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[ns][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if (kb0 < kb1) {
    DecFrags<MT> cur = load(kb0);
    for (int kb = kb0; kb < kb1; ++kb) {
      DecFrags<MT> nxt = cur;
      if (kb + 1 < kb1) nxt = load(kb + 1);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const float comb = cur.sa[mt] * cur.sw;
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) {
          const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cur.w[ns], cur.a[mt], zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[ns][mt][v] = __builtin_fmaf(part[v], comb, acc[ns][mt][v]);
        }
      }
      cur = nxt;
    }
  }

  // partial sums to LDS: index ((ns * MT + mt) * 64 + lane) * 4 + v
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<v4f*>(&red[wave][((ns * MT + mt) * 64 + lane) * 4]) = acc[ns][mt];
  __syncthreads();

  for (int o = threadIdx.x; o < 4 * MT * 64 * 4; o += kDecThreads) {
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kDecSplit; ++w) sum += red[w][o];
    const int v = o & 3;
    const int ln = (o >> 2) & 63;
    const int mt = (o >> 8) % MT;
    const int ns = (o >> 8) / MT;
    const int m = mt * 16 + (ln & 15);
    const int n = n0 + ns * 16 + 4 * (ln >> 4) + v;
    if (m < p.M) {
      if (kBf16Out)
        static_cast<__hip_bfloat16*>(p.c)[(int64_t)m * p.ldc + n] = __float2bfloat16(sum);
      else
        static_cast<float*>(p.c)[(int64_t)m * p.ldc + n] = sum;
    }
  }
}

template <int MT>
void launch_decode(const GemmParams& p, bool bf16, hipStream_t st) {
  const dim3 grid((unsigned)(p.N / kDecBN));
  if (bf16)
    hipLaunchKernelGGL((k_gemm_fp8_decode<MT, true>), grid, dim3(kDecThreads), 0, st, p);
  else
    hipLaunchKernelGGL((k_gemm_fp8_decode<MT, false>), grid, dim3(kDecThreads), 0, st, p);
}

}  // namespace

hipError_t launch_block_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.M == 0) return hipSuccess;
  GemmParams p;
  p.a = g.a;
  p.b = g.b;
  p.sa = g.sa;
  p.sb = g.sb;
  p.c = g.c;
  p.lda = g.lda;
  p.ldb = g.ldb;
  p.ldc = g.ldc;
  p.sa_m = g.gran_a == GRAN_PER_TENSOR ? 0 : g.sa_m;
  p.sa_k = g.gran_a == GRAN_PER_TENSOR ? 0 : g.sa_k;
  p.sb_n = g.gran_b == GRAN_PER_TENSOR ? 0 : g.sb_n;
  p.sb_k = g.gran_b == GRAN_PER_TENSOR ? 0 : g.sb_k;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.tiles_m = (p.M + BM - 1) / BM;
  p.tiles_n = (p.N + BN - 1) / BN;
  const bool bf16 = g.c_dtype == DTYPE_BF16;
  if (p.M <= 16) {
    launch_decode<1>(p, bf16, st);
    return hipGetLastError();
  }
  if (p.M <= 32) {
    launch_decode<2>(p, bf16, st);
    return hipGetLastError();
  }
  if (p.M <= 64) {
    launch_decode<4>(p, bf16, st);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
  if (g.c_dtype == DTYPE_BF16)
    hipLaunchKernelGGL(k_gemm_fp8_block<true>, grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(k_gemm_fp8_block<false>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace fp8blk
