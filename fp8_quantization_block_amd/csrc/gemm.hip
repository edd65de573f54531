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
//   scales) are copied
//   global -> LDS with global_load_lds_dwordx4 / _dword, double buffered, one
//   barrier per K block. Rows are stored with their eight 16-byte chunks
//   XOR-swizzled by (row & 7) so the MFMA operand reads are conflict free.
// * Workgroup ids are remapped so that neighbouring tiles (which share A rows
//   or B columns) run on the same XCD and share its L2.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

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

__device__ __forceinline__ void lds_copy16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void lds_copy4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)g, (lds_ptr_t)lds, 4, 0, 0);
}

// Issue the copies of K block kb into one LDS stage. Each wave instruction
// fills 1 KB = 8 rows of 128 bytes; lane l fills physical chunk l % 8 of row
// l / 8, which holds logical chunk (l % 8) ^ (row & 7).
struct Stage {
  uint8_t* a;      // [256][128] codes, swizzled
  uint8_t* b;      // [256][128] codes, swizzled
  float* s;        // [256] activation scales, then 2 weight-block scales
};

__device__ __forceinline__ void issue_stage(const GemmParams& p, const Stage& stage, int m0, int n0,
                                            int kb, int wave, int lane) {
  const int sub_row = lane >> 3;
  const int pchunk = lane & 7;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int blk = wave * 4 + i;                // 0..31
    const int row = blk * 8 + sub_row;           // 0..255
    const int lchunk = pchunk ^ (row & 7);
    const int ra = min(m0 + row, p.M - 1);
    const int rb = min(n0 + row, p.N - 1);
    lds_copy16(p.a + (int64_t)ra * p.lda + (int64_t)kb * BK + lchunk * 16, stage.a + blk * 1024);
    lds_copy16(p.b + (int64_t)rb * p.ldb + (int64_t)kb * BK + lchunk * 16, stage.b + blk * 1024);
  }
  if (wave < 4) {
    const int r = min(m0 + wave * 64 + lane, p.M - 1);
    lds_copy4(p.sa + (int64_t)r * p.sa_m + (int64_t)kb * p.sa_k, stage.s + wave * 64);
  } else if (wave == 4 && lane < 2) {
    const int nb = min((n0 >> 7) + lane, (p.N >> 7) - 1);
    lds_copy4(p.sb + (int64_t)nb * p.sb_n + (int64_t)kb * p.sb_k, stage.s + 256);
  }
}

// Operand fragment of one 16-row (or 16-column) subtile: lane l takes row
// base + l % 16 and the 32 bytes at K offset 32 * (l / 16). A and B use the
// same K assignment, so the MFMA sums exactly the 128 products of the block.
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, int row, int lane) {
  const int lc0 = (lane >> 4) * 2;
  const int sw = row & 7;
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + row * 128 + ((lc0 ^ sw) << 4));
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + row * 128 + (((lc0 + 1) ^ sw) << 4));
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// One K block: prefetch block kb + 1 into `next` (if any), then multiply the
// tiles of block kb held in `cur` and promote into acc.
struct WaveCtx {
  int m0, n0, wave, lane, wm, wn;
  bool active;
};

__device__ __forceinline__ void k_block_step(const GemmParams& p, const WaveCtx& w, int kb, int nk,
                                             const Stage& cur, const Stage& next, v4f (&acc)[4][8]) {
  if (kb + 1 < nk) issue_stage(p, next, w.m0, w.n0, kb + 1, w.wave, w.lane);
  if (w.active) {
    const float sbv = cur.s[256 + w.wn];
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* ta = cur.a;
    const uint8_t* tb = cur.b;
    const float* ssa = cur.s;
    const int lane = w.lane;
    v8i af[4];
    v4f comb[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      af[mi] = read_frag(ta, w.wm * 64 + mi * 16 + (lane & 15), lane);
      const v4f s4 = *reinterpret_cast<const v4f*>(ssa + w.wm * 64 + mi * 16 + 4 * (lane >> 4));
      comb[mi] = s4 * sbv;
    }
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) {
      const v8i bf = read_frag(tb, w.wn * 128 + ni * 16 + (lane & 15), lane);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bf, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[mi][ni][v] = __builtin_fmaf(part[v], comb[mi][v], acc[mi][ni][v]);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's prefetch landed
  __syncthreads();                      // ... and every other wave's
}

template <bool kBf16Out>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_fp8_block(GemmParams p) {
  // two LDS stages as distinct objects, so the compiler can tell reads of one
  // stage from the asynchronous copies into the other
  __shared__ __attribute__((aligned(1024))) uint8_t a0[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[kTileBytes];
  __shared__ __attribute__((aligned(16))) float s0[BM + 4];
  __shared__ __attribute__((aligned(1024))) uint8_t a1[kTileBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t b1[kTileBytes];
  __shared__ __attribute__((aligned(16))) float s1[BM + 4];
  const Stage stage0 = {a0, b0, s0};
  const Stage stage1 = {a1, b1, s1};

  // ---- tile assignment: XCD-major remap, then grouped row-major order ----
  const int nwg = p.tiles_m * p.tiles_n;
  int bid = blockIdx.x;
  if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  constexpr int kGroupM = 8;
  const int group = bid / (kGroupM * p.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(p.tiles_m - first_m, kGroupM);
  const int in_group = bid - group * kGroupM * p.tiles_n;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;

  WaveCtx w;
  w.m0 = tm * BM;
  w.n0 = tn * BN;
  w.lane = threadIdx.x & 63;
  w.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  w.wm = w.wave >> 1;          // 0..3 : 64-row slab
  w.wn = w.wave & 1;           // 0..1 : 128-column slab
  w.active = (w.n0 + w.wn * 128) < p.N;
  const int m0 = w.m0, n0 = w.n0, lane = w.lane, wm = w.wm, wn = w.wn;
  const bool wave_active = w.active;

  v4f acc[4][8];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

  const int nk = p.K / BK;
  issue_stage(p, stage0, m0, n0, 0, w.wave, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies landed
  __syncthreads();

  for (int kb = 0; kb < nk; kb += 2) {
    k_block_step(p, w, kb, nk, stage0, stage1, acc);
    if (kb + 1 < nk) k_block_step(p, w, kb + 1, nk, stage1, stage0, acc);
  }

  if (!wave_active) return;
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
