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
// Operands are E4M3 or E5M2 codes, each operand in its own format ([FP8]
// section "FP8 是什么", format table): the f8f6f4 MFMA decodes either format, so
// the kernels are instantiated per (format of A, format of B) pair.
//
// Prefill kernel design (gfx950):
// * One v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep scale block,
//   so every MFMA starts from zero and its 16x16 fp32 result is promoted into
//   the fp32 accumulator with one FMA per element: acc += P_j * s_a * s_b.
// * Workgroup tile 256 x 256 (the largest whose fp32 accumulators fit the
//   register file next to the operands: 256 KB per CU), K step 128; 8 waves in
//   a 4 x 2 grid, each owning 64 rows x 128 columns (one weight scale block,
//   so s_b is one scalar per wave and K block).
// * Both operand tiles (32 KB each) and the K block's scales go global -> LDS
//   by direct copies (no staging registers), double buffered: the copies of
//   block kb + 1 are issued at the start of block kb and waited for at its
//   end, one barrier per block.
// * The 32 products of a wave's K block are software pipelined: the MFMA of
//   product t is issued before the promotion FMAs of product t - 2, so the
//   FMAs run under the matrix unit's work.
// * Fragment K order: lane group q = lane / 16 holds K bytes [16q, 16q + 16)
//   and [64 + 16q, 64 + 16q + 16) of the block for both operands, so the MFMA
//   sums exactly the block's 128 products.
// * LDS rows hold eight 16-byte chunks, logical chunk c of row r at physical
//   chunk c ^ swz(r), so the operand reads are free of bank conflicts.
// * Workgroup ids are remapped so that neighbouring tiles (which share A rows
//   or B columns) run on the same XCD and share its L2.
// * Output: bf16, fp32, or (fused quantization) FP8 codes with one scale per
//   row and 128-column group. A wave owns 64 rows x 128 columns, i.e. exactly
//   one 1 x 128 group of each of its rows, so the group amax is a max over the
//   wave's own registers and one 16-lane DPP reduction: the next GEMM's
//   activation quantization ([FP8] section "激活动态量化": one scale per token
//   and 128-channel group, computed at run time) runs in this epilogue instead
//   of as a separate pass over the bf16 output.
#include <hip/hip_bf16.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 512;
constexpr int kTileBytes = BM * BK;    // one operand tile, 32 KB
constexpr int kScaleSlots = BM + 64;   // 256 activation scales, then 64 weight-scale slots
// bf16 output staging after the K loop: per wave 64 rows of 128 values, 256
// bytes per row (the row-contiguous read-back is then a linear, conflict-free
// LDS read)
constexpr int kOutPitch = 256;
constexpr int kLoopSmem = 4 * kTileBytes + (2 * kScaleSlots + 64) * 4;
// MX operands: per stage 1 KB of activation scale bytes (4 per row), then 1 KB
// of weight scale bytes
constexpr int kMxScaleStage = 2048;
constexpr int kLoopSmemMx = 4 * kTileBytes + 2 * kMxScaleStage;
constexpr int kOutSmem = 8 * 64 * kOutPitch;
constexpr int kSmemA = kLoopSmem > kOutSmem ? kLoopSmem : kOutSmem;
constexpr int kSmemBytes = kSmemA > kLoopSmemMx ? kSmemA : kLoopSmemMx;

struct GemmParams {
  const uint8_t* a;
  const uint8_t* b;
  const float* sa;
  const float* sb;
  void* c;
  int64_t lda, ldb, ldc;
  int64_t sa_m, sa_k, sb_n, sb_k;
  const uint8_t* sa8;   // MX operands: E8M0 scale bytes [M][ld_sa8] ...
  const uint8_t* sb8;   // ... and [N][ld_sb8], one per 32 K elements
  int64_t ld_sa8, ld_sb8;
  uint8_t* qc;          // fused quantization: codes (row stride ldc bytes) ...
  float* sc;            // ... and scales, sc[row * sc_m + group * sc_n]
  int64_t sc_m, sc_n;
  int M, N, K;
  int tiles_m, tiles_n;
  // Tail balancing: the last n_half tiles (in tile order) are computed as two
  // 256 x 128 halves by two workgroups each, so that a last round that would
  // occupy only part of the chip fills it. n_full + n_half = tiles; when
  // n_half > 0 both n_full and 2 n_half are multiples of 8 (one share per XCD).
  int n_full, n_half;
};

// LDS rows are 128 bytes (eight 16-byte chunks); logical chunk c of row r is
// stored at physical chunk c ^ swz(r). With swz(r) = r % 8 the 128-bit
// fragment reads (16 consecutive rows, one logical chunk per 16 lanes) are
// free of bank conflicts on gfx950 (measured: 243 B/clk per CU, as a linear
// read; the swizzle (r % 8) ^ (r / 8 % 2) measured 2-way conflicted).
__device__ __forceinline__ int swz(int row) { return row & 7; }

__device__ __forceinline__ v8i pack_frag(uint4 lo, uint4 hi) {
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Fragment of a 16-row subtile from an LDS tile: lane l takes the row at
// byte offset `row_off` (subtile base + l % 16, precomputed with its
// swizzled chunk offsets lo/hi for chunks q and 4 + q, q = l / 16).
__device__ __forceinline__ v8i read_frag(const uint8_t* tile, uint32_t lo_off, uint32_t hi_off) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + lo_off);
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + hi_off);
  return pack_frag(lo, hi);
}

// Per-thread copy and read plan.
// * Operand tiles, K block kb, into an LDS stage: wave w fills rows 32 w ..
//   32 w + 31 of each tile, 8 rows (1 KB) per instruction; lane l fills
//   physical chunk l % 8 of row 8 (4 w + i) + l / 8, i.e. logical chunk
//   (l % 8) ^ swz(row). Activation rows past M read as zero.
// * Scales of K block kb: lane l of wave w < 4 copies the activation scale of
//   tile row 64 w + l (rows past M re-read row M - 1; their results are never
//   stored) into slot 64 w + l; lane l of wave 4 copies the weight-block scale
//   of the tile's 128-column half l % 2 into slot 256 + l; waves 5..7 copy the
//   same into a sink (so that every wave issues the same instructions).
struct Plan {
  // Byte offsets of this lane's chunk in copy instruction i (block 0). The
  // row offset of an activation copy stays in the VGPR offset, which the
  // buffer's range check covers (a ragged last tile must read zeros past M);
  // weight rows past the end come in whole 32-row groups of one wave, so the
  // weight copies carry the 8-row step of instruction i in the scalar offset.
  uint32_t a_voff[4], b_voff;
  uint32_t b_istep;            // bytes between consecutive weight copy instructions (8 rows)
  uint32_t s_voff;      // byte offset of this lane's scale (block 0)
  uint32_t s_kstep;     // bytes between consecutive K blocks' scales
  uint32_t a_lo, a_hi;  // this lane's activation fragment chunks (subtile 0 of its slab)
  uint32_t b_lo, b_hi;  // this lane's weight fragment chunks (subtile 0 of its slab)
  uint32_t s_rd;        // this lane's four activation scales (subtile 0)
  uint32_t w_rd;        // the wave's weight-block scale slot
  int wave;
};

// Copies of K block kb into one stage: 4 + 4 + 1 vector memory instructions.
__device__ __forceinline__ void issue(const Plan& pl, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                      __amdgpu_buffer_rsrc_t rs, int kb, uint8_t* ta, uint8_t* tb,
                                      float* ts, float* sink) {
  const uint32_t soff = (uint32_t)kb * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dma16(ra, pl.a_voff[i], soff, ta + (pl.wave * 4 + i) * 1024);
    dma16(rb, pl.b_voff, soff + (uint32_t)i * pl.b_istep, tb + (pl.wave * 4 + i) * 1024);
  }
  float* sdst = pl.wave <= 4 ? ts + pl.wave * 64 : sink;
  dma4(rs, pl.s_voff, (uint32_t)kb * pl.s_kstep, sdst);
}

// The MFMA / promotion pipeline of a wave, continuous across K blocks.
// Products are numbered t = 0..31 per block, (ni, mi) = (t / 4, t % 4). Step t
// issues the MFMA of product t into partial register t % kRing and promotes
// the product issued kLag steps earlier (for t < kLag the last products of the
// previous block, with that block's scales), so a promotion never waits for
// its MFMA and the matrix unit keeps running across the block boundary, while
// the first LDS reads of the new block are in flight.
constexpr int kLag = 5;
constexpr int kRing = 8;   // > kLag and a divisor of 32: ring slots are the same in every block

struct Pipe {
  v4f part[kRing];
  v4f comb[4];   // scales of the block whose products are being promoted
};

__device__ __forceinline__ void promote(const Pipe& pp, const v4f (&comb)[4], int u, v4f (&acc)[4][8]) {
#pragma unroll
  for (int v = 0; v < 4; ++v)
    acc[u & 3][u >> 2][v] = __builtin_fmaf(pp.part[u % kRing][v], comb[u & 3][v], acc[u & 3][u >> 2][v]);
}

// One K block of a wave: 4 activation subtiles x 8 weight subtiles. `first`:
// no previous block to finish.
template <bool first, int kFa, int kFb>
__device__ __forceinline__ void mma_block(const Plan& pl, const uint8_t* ta, const uint8_t* tb,
                                          const float* ts, Pipe& pp, v4f (&acc)[4][8]) {
  // reads for the first MFMA first, then the rest of the activation fragments
  // and the scales; the weight fragment of subtile ni + 1 is read while
  // subtile ni is in use
  v8i af[4], bf[2];
  af[0] = read_frag(ta, pl.a_lo, pl.a_hi);
  bf[0] = read_frag(tb, pl.b_lo, pl.b_hi);
#pragma unroll
  for (int mi = 1; mi < 4; ++mi) af[mi] = read_frag(ta, pl.a_lo + mi * 2048, pl.a_hi + mi * 2048);
  v4f s4[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) s4[mi] = *reinterpret_cast<const v4f*>(ts + pl.s_rd + mi * 16);
  const float sw = ts[pl.w_rd];
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int ni = t >> 2, mi = t & 3;
    if (mi == 0 && ni < 7)
      bf[(ni + 1) & 1] = read_frag(tb, pl.b_lo + (ni + 1) * 2048, pl.b_hi + (ni + 1) * 2048);
    pp.part[t % kRing] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bf[ni & 1], zero, kFa, kFb, 0, 0, 0, 0);
    if (t >= kLag) {
      promote(pp, pp.comb, t - kLag, acc);
    } else if (!first) {
      promote(pp, pp.comb, t - kLag + 32, acc);   // previous block's product, its scales
    }
    if (t == kLag - 1) {
      // from here on the promotions belong to this block
#pragma unroll
      for (int m = 0; m < 4; ++m) pp.comb[m] = s4[m] * sw;
    }
    // keep the program order: the scheduler would otherwise pair FMAs with the
    // MFMA that produces their operand and stall on it
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Promotions of the last block's final kLag products.
__device__ __forceinline__ void drain(const Pipe& pp, v4f (&acc)[4][8]) {
#pragma unroll
  for (int u = 32 - kLag; u < 32; ++u) promote(pp, pp.comb, u, acc);
}

// One K block kb: copy block kb + 1 into the other stage, multiply block kb,
// wait for the copies (the only vector memory operations in flight), barrier.
// The block index of the copy is clamped to the last block (the tail copy
// lands in a stage nobody reads again).
template <bool first, int kFa, int kFb>
__device__ __forceinline__ void k_step(const Plan& pl, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                       __amdgpu_buffer_rsrc_t rs, int kb, int nk, const uint8_t* ca,
                                       const uint8_t* cb, const float* cs, uint8_t* na, uint8_t* nb,
                                       float* ns, float* sink, bool active, Pipe& pp, v4f (&acc)[4][8]) {
  issue(pl, ra, rb, rs, min(kb + 1, nk - 1), na, nb, ns, sink);
  if (active) mma_block<first, kFa, kFb>(pl, ca, cb, cs, pp, acc);
  copies_done_barrier();
}

// The K loop over the two stages. Every pointer the copies touch (both
// stages' tiles and scale slots, the sink, and the arrays they read) is a
// distinct non-aliasing parameter, so that the compiler can tell that reading
// one stage does not depend on the copies in flight into the other.
template <int kFa, int kFb>
__device__ __forceinline__ void k_loop(const Plan& pl, const uint8_t* __restrict__ ga, uint32_t ga_bytes,
                                       const uint8_t* __restrict__ gb, uint32_t gb_bytes,
                                       const float* __restrict__ gs, uint32_t gs_bytes,
                                       uint8_t* __restrict__ a0, uint8_t* __restrict__ a1,
                                       uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                       float* __restrict__ s0, float* __restrict__ s1,
                                       float* __restrict__ sink, int nk, bool active, v4f (&acc)[4][8]) {
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(ga, ga_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(gb, gb_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(gs, gs_bytes);
  Pipe pp;
  issue(pl, ra, rb, rs, 0, a0, b0, s0, sink);
  copies_done_barrier();
  k_step<true, kFa, kFb>(pl, ra, rb, rs, 0, nk, a0, b0, s0, a1, b1, s1, sink, active, pp, acc);
  int kb = 1;
  for (; kb + 1 < nk; kb += 2) {
    k_step<false, kFa, kFb>(pl, ra, rb, rs, kb, nk, a1, b1, s1, a0, b0, s0, sink, active, pp, acc);
    k_step<false, kFa, kFb>(pl, ra, rb, rs, kb + 1, nk, a0, b0, s0, a1, b1, s1, sink, active, pp, acc);
  }
  if (kb < nk) k_step<false, kFa, kFb>(pl, ra, rb, rs, kb, nk, a1, b1, s1, a0, b0, s0, sink, active, pp, acc);
  if (active) drain(pp, acc);
}

// ---------------------------------------------------------------------------
// MX operands ([VS] api.makesence.top, "LLM推理量化:FP8 versus INT8", section 3:
// one power-of-two scale per 32 elements of a row, applied by block-scaled
// hardware). gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 takes one E8M0 byte
// per lane for each operand: lane group g = lane / 16 supplies the scale of
// the lane's row (A) or column (B) for the 32-element K block g of the
// instruction's 128; with the fragment K order above (lane group g holds K
// bytes 16 g .. and 64 + 16 g ..) that block is K [32 g, 32 g + 32). Both
// established on the device. The scaled products accumulate in the MFMA
// itself: no promotion FMAs.
// ---------------------------------------------------------------------------
// Copies of K block kb: the operand tiles as issue(), and the scale dwords
// (4 bytes = the block's 4 scales) of 64 rows per wave: waves 0..3 activation
// rows 64 w .., waves 4..7 weight rows 64 (w - 4) .., landing at stage bytes
// 256 w (activation rows at 4 r, weight rows at 1024 + 4 r). Row offsets and
// the K step are in the VGPR offset (rows past the tile read zero).
__device__ __forceinline__ void issue_mx(const Plan& pl, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                         __amdgpu_buffer_rsrc_t rs, int kb, uint8_t* ta, uint8_t* tb, uint8_t* ts) {
  const uint32_t soff = (uint32_t)kb * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dma16(ra, pl.a_voff[i], soff, ta + (pl.wave * 4 + i) * 1024);
    dma16(rb, pl.b_voff, soff + (uint32_t)i * pl.b_istep, tb + (pl.wave * 4 + i) * 1024);
  }
  dma4(rs, pl.s_voff + (uint32_t)kb * 4u, 0u, ts + pl.wave * 256);
}

// One K block of a wave, MX operands: 32 scaled MFMAs accumulating in place.
// pl.s_rd / pl.w_rd: byte offsets of this lane's activation / weight scale
// (subtile 0) in the stage. Weight fragments are read two subtiles ahead
// (three-deep ring) and the program order is pinned per step: with no
// promotion work between the MFMAs, a one-subtile lead left them waiting on
// the LDS reads.
template <int kFa, int kFb>
__device__ __forceinline__ void mma_block_mx(const Plan& pl, const uint8_t* ta, const uint8_t* tb, const uint8_t* ts,
                                             v4f (&acc)[4][8]) {
  v8i af[4], bf[3];
  af[0] = read_frag(ta, pl.a_lo, pl.a_hi);
  bf[0] = read_frag(tb, pl.b_lo, pl.b_hi);
#pragma unroll
  for (int mi = 1; mi < 4; ++mi) af[mi] = read_frag(ta, pl.a_lo + mi * 2048, pl.a_hi + mi * 2048);
  bf[1] = read_frag(tb, pl.b_lo + 2048, pl.b_hi + 2048);
  int sa[4], sb[8];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) sa[mi] = ts[pl.s_rd + mi * 64];
#pragma unroll
  for (int ni = 0; ni < 8; ++ni) sb[ni] = ts[pl.w_rd + ni * 64];
#pragma unroll
  for (int t = 0; t < 32; ++t) {
    const int ni = t >> 2, mi = t & 3;
    if (mi == 0 && ni < 6)
      bf[(ni + 2) % 3] = read_frag(tb, pl.b_lo + (ni + 2) * 2048, pl.b_hi + (ni + 2) * 2048);
    acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[mi], bf[ni % 3], acc[mi][ni], kFa, kFb, 0,
                                                                  sa[mi], 0, sb[ni]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int kFa, int kFb>
__device__ __forceinline__ void k_step_mx(const Plan& pl, __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                          __amdgpu_buffer_rsrc_t rs, int kb, int nk, const uint8_t* ca,
                                          const uint8_t* cb, const uint8_t* cs, uint8_t* na, uint8_t* nb, uint8_t* ns,
                                          bool active, v4f (&acc)[4][8]) {
  issue_mx(pl, ra, rb, rs, min(kb + 1, nk - 1), na, nb, ns);
  if (active) mma_block_mx<kFa, kFb>(pl, ca, cb, cs, acc);
  copies_done_barrier();
}

// The MX K loop over two stages (distinct __restrict__ stages and arrays, as
// k_loop).
template <int kFa, int kFb>
__device__ __forceinline__ void k_loop_mx(const Plan& pl, const uint8_t* __restrict__ ga, uint32_t ga_bytes,
                                          const uint8_t* __restrict__ gb, uint32_t gb_bytes,
                                          const uint8_t* __restrict__ gs, uint32_t gs_bytes,
                                          uint8_t* __restrict__ a0, uint8_t* __restrict__ a1,
                                          uint8_t* __restrict__ b0, uint8_t* __restrict__ b1,
                                          uint8_t* __restrict__ s0, uint8_t* __restrict__ s1, int nk, bool active,
                                          v4f (&acc)[4][8]) {
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(ga, ga_bytes);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(gb, gb_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(gs, gs_bytes);
  issue_mx(pl, ra, rb, rs, 0, a0, b0, s0);
  copies_done_barrier();
  int kb = 0;
  for (; kb + 1 < nk; kb += 2) {
    k_step_mx<kFa, kFb>(pl, ra, rb, rs, kb, nk, a0, b0, s0, a1, b1, s1, active, acc);
    k_step_mx<kFa, kFb>(pl, ra, rb, rs, kb + 1, nk, a1, b1, s1, a0, b0, s0, active, acc);
  }
  if (kb < nk) k_step_mx<kFa, kFb>(pl, ra, rb, rs, kb, nk, a0, b0, s0, a1, b1, s1, active, acc);
}

// Output modes of the prefill kernel.
enum OutMode : int { OUT_BF16 = 0, OUT_F32 = 1, OUT_Q_E4M3 = 2, OUT_Q_E5M2 = 3 };
// quantized output staging: per wave 64 rows of 128 codes, 144-byte pitch
constexpr int kQPitch = 144;
static_assert(8 * 64 * kQPitch <= kSmemBytes, "quantized output staging exceeds the LDS");

template <int kOut, int kFa, int kFb, bool kMx = false>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_fp8_block(GemmParams p) {
  // LDS: two stages of operand tiles and scales during the K loop; afterwards
  // the same memory stages the bf16 output for coalesced stores
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kSmemBytes];
  uint8_t* const ta0 = smem;
  uint8_t* const ta1 = smem + kTileBytes;
  uint8_t* const tb0 = smem + 2 * kTileBytes;
  uint8_t* const tb1 = smem + 3 * kTileBytes;
  float* const ts0 = reinterpret_cast<float*>(smem + 4 * kTileBytes);
  float* const ts1 = ts0 + kScaleSlots;
  float* const sink = ts1 + kScaleSlots;

  // ---- tile assignment --------------------------------------------------
  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8); each XCD
  // is given a contiguous share of the tile order (neighbouring tiles share A
  // rows or B columns in its L2): first its full tiles, then its halves.
  int bid = blockIdx.x, half = -1;
  if (p.n_half == 0) {
    const int nwg = p.tiles_m * p.tiles_n;
    if ((nwg & 7) == 0) bid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  } else {
    const int x = bid & 7, pos = bid >> 3;
    const int fpx = p.n_full >> 3, hpx = (2 * p.n_half) >> 3;
    if (pos < fpx) {
      bid = x * fpx + pos;
    } else {
      const int h = x * hpx + (pos - fpx);
      bid = p.n_full + (h >> 1);
      half = h & 1;
    }
  }
  // grouped row-major order: 8 tile rows at a time
  constexpr int kGroupM = 8;
  const int group = bid / (kGroupM * p.tiles_n);
  const int first_m = group * kGroupM;
  const int gm = min(p.tiles_m - first_m, kGroupM);
  const int in_group = bid - group * kGroupM * p.tiles_n;
  const int m0 = (first_m + in_group % gm) * BM;
  // a half tile is the 256 x 128 block n0 + 128 half .. + 127, computed by the
  // waves of column slab 0 (one on each SIMD); the other four idle
  const int n0 = (in_group / gm) * BN + (half > 0 ? 128 : 0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
  const int wm = wave & 3;           // 0..3 : 64-row slab (waves 4 apart share a SIMD)
  const int wn = wave >> 2;          // 0..1 : 128-column slab
  const bool active = (n0 + wn * 128) < p.N && (half < 0 || wn == 0);
  const int nk = p.K / BK;
  const int rows_a = min(p.M - m0, BM), rows_b = min(p.N - n0, half < 0 ? BN : 128);

  Plan pl;
  pl.wave = wave;
  {
    // copy instruction i fills rows 8 (4 w + i) + l / 8, whose swizzle is
    // l / 8: every instruction uses the same chunk pattern, 8 rows further on
    const int sub_row = lane >> 3, pchunk = lane & 7;
    const int row0 = wave * 32 + sub_row;
    const int chunk = (pchunk ^ swz(row0)) << 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) pl.a_voff[i] = (uint32_t)((row0 + 8 * i) * (int)p.lda + chunk);
    pl.b_voff = (uint32_t)(row0 * (int)p.ldb + chunk);
    pl.b_istep = (uint32_t)(8 * p.ldb);
    const int rrow = lane & 15, q = lane >> 4;
    const uint32_t lo = (uint32_t)(rrow * 128 + ((q ^ swz(rrow)) << 4));
    const uint32_t hi = (uint32_t)(rrow * 128 + (((4 + q) ^ swz(rrow)) << 4));
    pl.a_lo = lo + wm * 64 * 128;
    pl.a_hi = hi + wm * 64 * 128;
    pl.b_lo = lo + wn * 128 * 128;
    pl.b_hi = hi + wn * 128 * 128;
    pl.s_rd = (uint32_t)(wm * 64 + 4 * q);
    pl.w_rd = (uint32_t)(BM + wn);
  }
  v4f acc[4][8];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
#pragma unroll
    for (int ni = 0; ni < 8; ++ni) acc[mi][ni] = v4f{0.f, 0.f, 0.f, 0.f};

  if constexpr (kMx) {
    // scale copy plan: waves 0..3 activation rows 64 w + lane, waves 4..7
    // weight rows 64 (w - 4) + lane of the tile; reads: this lane's row of
    // subtile 0 (r = lane % 16) and scale byte g = lane / 16
    const int rl = (wave & 3) * 64 + lane;
    const uint8_t* gs8;
    uint32_t gs8_bytes;
    if (wave < 4) {
      gs8 = p.sa8 + (int64_t)m0 * p.ld_sa8;
      gs8_bytes = (uint32_t)(rows_a * p.ld_sa8);
      pl.s_voff = (uint32_t)(rl * p.ld_sa8);
    } else {
      gs8 = p.sb8 + (int64_t)n0 * p.ld_sb8;
      gs8_bytes = (uint32_t)(rows_b * p.ld_sb8);
      pl.s_voff = (uint32_t)(rl * p.ld_sb8);
    }
    const int rrow = lane & 15, q = lane >> 4;
    pl.s_rd = (uint32_t)((wm * 64 + rrow) * 4 + q);
    pl.w_rd = (uint32_t)(1024 + (wn * 128 + rrow) * 4 + q);
    uint8_t* const s0 = smem + 4 * kTileBytes;
    k_loop_mx<kFa, kFb>(pl, p.a + (int64_t)m0 * p.lda, (uint32_t)(rows_a * (int)p.lda), p.b + (int64_t)n0 * p.ldb,
                        (uint32_t)(rows_b * (int)p.ldb), gs8, gs8_bytes, ta0, ta1, tb0, tb1, s0,
                        s0 + kMxScaleStage, nk, active, acc);
  } else {
  // scale copy plan: waves 0..3 activation scales, waves 4..7 weight-block scales
  const float* gs;
  uint32_t gs_bytes;
  if (wave < 4) {
    const int64_t s_last = (int64_t)(p.M - 1) * p.sa_m + (int64_t)(nk - 1) * p.sa_k;
    gs = p.sa;
    gs_bytes = (uint32_t)((s_last + 1) * 4);
    pl.s_voff = (uint32_t)((int64_t)min(m0 + wave * 64 + lane, p.M - 1) * p.sa_m * 4);
    pl.s_kstep = (uint32_t)(p.sa_k * 4);
  } else {
    const int nblk = p.N >> 7;
    const int64_t s_last = (int64_t)(nblk - 1) * p.sb_n + (int64_t)(nk - 1) * p.sb_k;
    gs = p.sb;
    gs_bytes = (uint32_t)((s_last + 1) * 4);
    pl.s_voff = (uint32_t)((int64_t)min((n0 >> 7) + (lane & 1), nblk - 1) * p.sb_n * 4);
    pl.s_kstep = (uint32_t)(p.sb_k * 4);
  }

  k_loop<kFa, kFb>(pl, p.a + (int64_t)m0 * p.lda, (uint32_t)(rows_a * (int)p.lda), p.b + (int64_t)n0 * p.ldb,
         (uint32_t)(rows_b * (int)p.ldb), gs, gs_bytes, ta0, ta1, tb0, tb1, ts0, ts1, sink, nk, active, acc);
  }

  if (!active) return;
  // ---- epilogue: lane holds rows 4 * (lane / 16) + v, column lane % 16 ----
  const int q = lane >> 4, c16 = lane & 15;
  if constexpr (kOut == OUT_Q_E4M3 || kOut == OUT_Q_E5M2) {
    // Row (mi, v) of this lane has its 128-column group in the 16 lanes of the
    // lane's DPP row (8 values each): group amax, scale, codes as the
    // stand-alone 1 x 128 quantizer computes them for fp32 inputs; codes are
    // staged in the idle LDS and stored row by row, 16 bytes per lane.
    constexpr int kFc = kOut == OUT_Q_E4M3 ? FMT_E4M3 : FMT_E5M2;
    uint8_t* const ep = smem + wave * (64 * kQPitch);
    const int64_t grp = (n0 + wn * 128) >> 7;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        uint32_t m = 0;
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) m = amax_f32(acc[mi][ni][v], m);
        const GroupScale gs = make_group_scale<kFc>(row16_max(m));
        const uint32_t w0 = cast4_f32<kFc>(gs, acc[mi][0][v], acc[mi][1][v], acc[mi][2][v], acc[mi][3][v]);
        const uint32_t w1 = cast4_f32<kFc>(gs, acc[mi][4][v], acc[mi][5][v], acc[mi][6][v], acc[mi][7][v]);
        const int r = mi * 16 + 4 * q + v;
        uint8_t* const rowp = ep + r * kQPitch + c16;
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          rowp[ni * 16] = (uint8_t)(w0 >> (8 * ni));
          rowp[(ni + 4) * 16] = (uint8_t)(w1 >> (8 * ni));
        }
        const int row = m0 + wm * 64 + r;
        if (c16 == 0 && row < p.M) p.sc[(int64_t)row * p.sc_m + grp * p.sc_n] = gs.s;
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = i * 64 + lane;
      const int r = idx >> 3, ch = idx & 7;
      const v4i val = *reinterpret_cast<const v4i*>(ep + r * kQPitch + ch * 16);
      const int row = m0 + wm * 64 + r;
      if (row < p.M)
        __builtin_nontemporal_store(val, reinterpret_cast<v4i*>(p.qc + (int64_t)row * p.ldc + n0 + wn * 128 + ch * 16));
    }
  } else if constexpr (kOut == OUT_BF16) {
    // Every wave is past the loop's last barrier and no copy is in flight, so
    // the LDS is free: stage the wave's 64 x 128 block as bf16, then store it
    // row by row, 16 bytes per lane (16 lanes per 256-byte row).
    uint8_t* const ep = smem + wave * (64 * kOutPitch);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int ni = 0; ni < 8; ++ni)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<__hip_bfloat16*>(ep + (mi * 16 + 4 * q + v) * kOutPitch + (ni * 16 + c16) * 2) =
              __float2bfloat16(acc[mi][ni][v]);
    __hip_bfloat16* const c = static_cast<__hip_bfloat16*>(p.c);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = i * 64 + lane;
      const int r = idx >> 4, ch = idx & 15;
      const v4i val = *reinterpret_cast<const v4i*>(ep + r * kOutPitch + ch * 16);
      const int row = m0 + wm * 64 + r;
      if (row < p.M)
        __builtin_nontemporal_store(val, reinterpret_cast<v4i*>(c + (int64_t)row * p.ldc + n0 + wn * 128 + ch * 8));
    }
  } else {
    float* const c = static_cast<float*>(p.c);
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + wm * 64 + mi * 16 + 4 * q + v;
        if (row >= p.M) continue;
#pragma unroll
        for (int ni = 0; ni < 8; ++ni) c[(int64_t)row * p.ldc + n0 + wn * 128 + ni * 16 + c16] = acc[mi][ni][v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Decode-shaped GEMM (M <= 64): bound by streaming the weights from HBM once.
//
// A workgroup owns 64 output columns (four 16-column subtiles) for every
// row of C and splits K four ways over its waves. Weight fragments go from
// global memory straight into MFMA operand registers (each weight byte is
// used once, so LDS staging would only add traffic); the next K block's
// fragments are loaded while the current one is multiplied. The MFMA's first
// operand is the weight subtile and its second the activations, so a lane's
// four results share one activation row (one s_a) and the subtile shares one
// s_b. The four partial sums are added through LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kDecThreads = 256;   // 4 waves: 5-6% faster than 8 at M = 16..64 (weights streamed from HBM)
constexpr int kDecSplit = kDecThreads / 64;
constexpr int kDecBN = 64;

template <int MT>
struct DecFrags {
  v8i w[4];
  v8i a[MT];
  float sa[MT];
  float sw;
};

// A lane's 32 fragment bytes: the low 16 at p, the high 16 at p + hi_off.
__device__ __forceinline__ v8i load_frag32(const uint8_t* p, int hi_off = 16) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + hi_off);
  v8i f;
  f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
  f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
  return f;
}

// Two floats to bf16 (the same rounding as __float2bfloat16), low one first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__bfloat16_as_ushort(__float2bfloat16(lo)) |
         ((uint32_t)__bfloat16_as_ushort(__float2bfloat16(hi)) << 16);
}

// The decode kernels' K loop, split-K merge and stores for the 64 output
// columns at n0. The loader has three stages: fetch(kb) issues the loads of K
// block kb that go to HBM (a block ahead) and returns them raw; near(kb)
// issues block kb's loads that hit in L2, before the next fetch, so that
// waiting for them (load counters drain in issue order) leaves that fetch in
// flight; frags(raw, near, kb) makes the block's MFMA fragments and scales.
// `first` is block kb0's fetch, made by the caller (who may issue it early).
// With kFetchAlways the fetch is made on the last block too (again of that
// block): a branch around it would leave the compiler unable to count the
// loads in flight, and it would then wait for all of them before the
// multiply; and the loop alternates two named buffers, so that no register
// copy at its back edge waits for the fetch either. The arithmetic (MFMA per block, promotion FMAs, the fixed order of the four
// waves' sums) does not depend on the loader. red: kDecSplit x (4 MT 64 4)
// floats of LDS.
__device__ __forceinline__ int decode_kb0(int K, int wave) { return ((K / 128) * wave) / kDecSplit; }
__device__ __forceinline__ int decode_kb1(int K, int wave) { return ((K / 128) * (wave + 1)) / kDecSplit; }

template <int MT, bool kBf16Out, int kFa, int kFb, bool kFetchAlways, typename Raw, typename Fetch, typename Near,
          typename Frags>
__device__ __forceinline__ void decode_tile(const GemmParams& p, int n0, float* red, Raw first, Fetch&& fetch,
                                            Near&& near, Frags&& frags) {
  constexpr int kRed = 4 * MT * 64 * 4;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb0 = decode_kb0(p.K, wave);
  const int kb1 = decode_kb1(p.K, wave);

  v4f acc[4][MT];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[ns][mt] = v4f{0.f, 0.f, 0.f, 0.f};

  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  auto multiply = [&](const DecFrags<MT>& f) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const float comb = f.sa[mt] * f.sw;
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        // weights are the first MFMA operand here
        const v4f part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.w[ns], f.a[mt], zero, kFb, kFa, 0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[ns][mt][v] = __builtin_fmaf(part[v], comb, acc[ns][mt][v]);
      }
    }
  };
  if constexpr (kFetchAlways) {
    Raw ra = first;
    Raw rb;
    for (int kb = kb0; kb < kb1;) {
      const auto na = near(kb);
      rb = fetch(min(kb + 1, kb1 - 1));
      multiply(frags(ra, na, kb));
      if (++kb >= kb1) break;
      const auto nb = near(kb);
      ra = fetch(min(kb + 1, kb1 - 1));
      multiply(frags(rb, nb, kb));
      ++kb;
    }
  } else if (kb0 < kb1) {
    Raw cur = first;
    for (int kb = kb0; kb < kb1; ++kb) {
      const auto nr = near(kb);
      Raw nxt = cur;
      if (kb + 1 < kb1) nxt = fetch(kb + 1);
      multiply(frags(cur, nr, kb));
      cur = nxt;
    }
  }

  // partial sums to LDS: index ((ns * MT + mt) * 64 + lane) * 4 + v
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<v4f*>(&red[wave * kRed + ((ns * MT + mt) * 64 + lane) * 4]) = acc[ns][mt];
  __syncthreads();

  // each thread adds the four waves' v4f of one (ns, mt, lane) slot, in wave
  // order, and stores the 4 adjacent outputs at once (c is 16-byte aligned
  // with a 16-byte row pitch; n is a multiple of 4)
  static_assert((kRed / 4) % kDecThreads == 0, "merge slots must split evenly over the threads");
#pragma unroll
  for (int i = 0; i < kRed / 4 / kDecThreads; ++i) {
    const int o = i * kDecThreads + threadIdx.x;
    v4f sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kDecSplit; ++w) {
      const v4f r = *reinterpret_cast<const v4f*>(&red[w * kRed + o * 4]);
#pragma unroll
      for (int v = 0; v < 4; ++v) sum[v] += r[v];
    }
    const int ln = o & 63;
    const int mt = (o >> 6) % MT;
    const int ns = (o >> 6) / MT;
    const int m = mt * 16 + (ln & 15);
    const int n = n0 + ns * 16 + 4 * (ln >> 4);
    if (m < p.M) {
      if (kBf16Out) {
        uint2 pk;
        pk.x = pack_bf16x2(sum[0], sum[1]);
        pk.y = pack_bf16x2(sum[2], sum[3]);
        *reinterpret_cast<uint2*>(static_cast<__hip_bfloat16*>(p.c) + (int64_t)m * p.ldc + n) = pk;
      } else {
        *reinterpret_cast<v4f*>(static_cast<float*>(p.c) + (int64_t)m * p.ldc + n) = sum;
      }
    }
  }
}

// kPacked: the weights are in the decode-packed layout (see
// k_pack_decode_weights) instead of row-major [N][ldb].
template <int MT, bool kBf16Out, int kFa, int kFb, bool kPacked>
__global__ __launch_bounds__(kDecThreads) void k_gemm_fp8_decode(GemmParams p) {
  __shared__ float red[kDecSplit * 4 * MT * 64 * 4];

  const int lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * kDecBN;
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 32;          // this lane's 32 bytes of a K block

  // weight fragment of column subtile ns and K block kb: row-major, this
  // lane's 32 bytes of row n0 + 16 ns + r16 at byte 128 kb + kq; packed, the
  // 2 KB block of (row group n0 / 16 + ns, kb) with this lane's halves at
  // 16 lane and 1024 + 16 lane
  const uint8_t* wrow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
    wrow[ns] = kPacked ? p.b + (int64_t)((n0 >> 4) + ns) * 2048 + lane * 16
                       : p.b + (int64_t)(n0 + ns * 16 + r16) * p.ldb + kq;
  const int64_t w_kstep = kPacked ? (int64_t)(p.N >> 4) * 2048 : 128;
  constexpr int kWHi = kPacked ? 1024 : 16;
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
    for (int ns = 0; ns < 4; ++ns) f.w[ns] = load_frag32(wrow[ns] + (int64_t)kb * w_kstep, kWHi);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f.a[mt] = load_frag32(arow[mt] + (int64_t)kb * 128);
      f.sa[mt] = sarow[mt][(int64_t)kb * p.sa_k];
    }
    f.sw = swrow[(int64_t)kb * p.sb_k];
    return f;
  };
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kb0 = decode_kb0(p.K, wave);
  DecFrags<MT> first;
  if (kb0 < decode_kb1(p.K, wave)) first = load(kb0);
  decode_tile<MT, kBf16Out, kFa, kFb, false>(
      p, n0, red, first, load, [](int) { return 0; }, [](const DecFrags<MT>& f, int, int) { return f; });
}

// The 32 codes of a lane's A fragment, four chunks of values of one group
// with scale g. With kHoist and bf16 values the scale's fast-path check is
// made once for all 32 rather than per four (the same codes: Vec8::cast_fast
// is the fast branch of Vec8::cast); it costs registers, which four M tiles
// do not have to spare below 256.
template <int kFmt, bool kHoist, typename T>
__device__ __forceinline__ void quant_frag(const Vec8<T> (&v)[4], const GroupScale& g, v8i& a) {
  if constexpr (kHoist && std::is_same<T, __hip_bfloat16>::value) {
    if (__builtin_expect(bf16_fast_ok(g), 1)) {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const uint2 cd = v[ch].template cast_fast<kFmt>(g);
        a[2 * ch] = (int)cd.x;
        a[2 * ch + 1] = (int)cd.y;
      }
      return;
    }
  }
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    const uint2 cd = v[ch].template cast<kFmt>(g);
    a[2 * ch] = (int)cd.x;
    a[2 * ch + 1] = (int)cd.y;
  }
}

// Dynamic activation quantization inside the decode GEMM (M <= 64): x is read
// as bf16 or fp32 and each A fragment is quantized in registers just before
// the MFMAs that consume it. [FP8] wangyu.me, "大语言模型量化技术（五）：FP8",
// section "激活动态量化" (activation scales taken at run time, just before the
// matmul, per tensor or per token and 128-channel group). The weights stream
// from HBM as in k_gemm_fp8_decode (row-major or decode-packed), which leaves
// the vector ALUs time to quantize.
//   kGroup (1x128): lane l's 32 values of a fragment (row 16 mt + l % 16, K
//   block kb, from value 32 (l / 16)) are a quarter of one group; lanes l ^ 16,
//   l ^ 32 and l ^ 48 hold the rest, so the group's max is two lane exchanges
//   away, and its scale is the s_a of that lane's MFMA results.
//   Per tensor: every workgroup takes the max over the whole (small) tensor
//   itself (at most 64K elements, 128 KB of bf16, mostly read from L2), so no
//   workgroup waits for another.
// Scales and casts are the quantizer's own (make_group_scale, Vec8::cast), so
// codes, scales and C equal those of fp8_quantize followed by the decode GEMM
// bit for bit. With q_out / s_out the codes and scales are stored as well:
// K block kb by workgroup kb % gridDim.x, from the fragments it multiplies.
template <int MT, bool kBf16Out, int kFa, int kFb, typename T, bool kGroup>
__global__ __launch_bounds__(kDecThreads) void k_quant_gemm_decode(GemmParams p, const T* __restrict__ x,
                                                                   int64_t ld_x, FastDiv div_cpr, int packed,
                                                                   uint8_t* __restrict__ q_out, int64_t ld_q,
                                                                   float* __restrict__ s_out, int64_t so_m,
                                                                   int64_t so_k) {
  __shared__ float red[kDecSplit * 4 * MT * 64 * 4];
  __shared__ uint32_t mred[kDecSplit];
  const int tid = threadIdx.x;
  const int lane = tid & 63;

  // the weights do not depend on the activation scales: this wave's first K
  // block of them is fetched before anything else, and the per-tensor max's
  // latency then covers theirs. Addresses as in k_gemm_fp8_decode.
  const int n0 = blockIdx.x * kDecBN;
  const int r16 = lane & 15;
  const int kq = (lane >> 4) * 32;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb0 = decode_kb0(p.K, wave);
  const uint8_t* wrow[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns)
    wrow[ns] = packed ? p.b + (int64_t)((n0 >> 4) + ns) * 2048 + lane * 16
                      : p.b + (int64_t)(n0 + ns * 16 + r16) * p.ldb + kq;
  const int64_t w_kstep = packed ? (int64_t)(p.N >> 4) * 2048 : 128;
  const int w_hi = packed ? 1024 : 16;
  const float* swrow = p.sb + (int64_t)(n0 >> 7) * p.sb_n;
  struct WFrags {
    v8i w[4];
    float sw;
  };
  auto fetch = [&](int kb) {
    WFrags r;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) r.w[ns] = load_frag32(wrow[ns] + (int64_t)kb * w_kstep, w_hi);
    r.sw = swrow[(int64_t)kb * p.sb_k];
    return r;
  };
  WFrags first;
  if (kb0 < decode_kb1(p.K, wave)) first = fetch(kb0);

  GroupScale gs_tensor{};
  if constexpr (!kGroup) {
    // max |x| over the tensor: batches of 16 chunk loads per thread, all
    // issued before the first is used; past the end a thread reads the last
    // chunk again (no branch, and a repeat cannot change a max)
    const uint32_t cpr = (uint32_t)p.K >> 3;   // chunks of 8 elements per row (K % 128 == 0)
    const uint32_t nchunks = (uint32_t)p.M * cpr;
    uint32_t m = 0;
    constexpr int kBatch = 16;
    for (uint32_t c0 = tid; c0 < nchunks; c0 += kBatch * kDecThreads) {
      Vec8<T> v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t c = min(c0 + (uint32_t)u * kDecThreads, nchunks - 1);
        const uint32_t r = fastdiv(c, div_cpr);
        v[u].template load<false>(x + (int64_t)r * ld_x + (c - r * cpr) * 8u, 8u);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const uint32_t a = v[u].amax_bits();
        m = a > m ? a : m;
      }
    }
    m = wave_max(m);
    if (lane == 0) mred[wave] = m;
    __syncthreads();
    m = 0;
#pragma unroll
    for (int w = 0; w < kDecSplit; ++w) m = mred[w] > m ? mred[w] : m;
    gs_tensor = make_group_scale<kFa>(m);
    if (s_out != nullptr && blockIdx.x == 0 && tid == 0) *s_out = gs_tensor.s;
  }

  // the A fragments, quantized from x (lane l: values 32 (l / 16) .. + 31 of
  // the K block of row 16 mt + l % 16; rows past M repeat row M - 1 and are
  // neither stored nor multiplied into C)
  const T* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xrow[mt] = x + (int64_t)min(mt * 16 + r16, p.M - 1) * ld_x + kq;
  const bool store_any = q_out != nullptr || (kGroup && s_out != nullptr);
  struct XRaw {
    Vec8<T> v[MT][4];
  };
  auto near = [&](int kb) {
    XRaw xr;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) xr.v[mt][ch].template load<false>(xrow[mt] + (int64_t)kb * 128 + ch * 8, 8u);
    return xr;
  };
  auto frags = [&](const WFrags& r, const XRaw& xr, int kb) {
    DecFrags<MT> f;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) f.w[ns] = r.w[ns];
    const bool store = store_any && (uint32_t)kb % gridDim.x == blockIdx.x;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      GroupScale g = gs_tensor;
      if constexpr (kGroup) {
        uint32_t m = 0;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
          const uint32_t a = xr.v[mt][ch].amax_bits();
          m = a > m ? a : m;
        }
        uint32_t o = (uint32_t)__shfl_xor((int)m, 16);
        m = o > m ? o : m;
        o = (uint32_t)__shfl_xor((int)m, 32);
        m = o > m ? o : m;
        g = make_group_scale<kFa>(m);
      }
      quant_frag<kFa, MT <= 2>(xr.v[mt], g, f.a[mt]);
      f.sa[mt] = g.s;
      if (store) {
        const int row = mt * 16 + r16;
        if (row < p.M) {
          if (q_out != nullptr) {
            uint4* dst = reinterpret_cast<uint4*>(q_out + (int64_t)row * ld_q + (int64_t)kb * 128 + kq);
            dst[0] = make_uint4((uint32_t)f.a[mt][0], (uint32_t)f.a[mt][1], (uint32_t)f.a[mt][2],
                                (uint32_t)f.a[mt][3]);
            dst[1] = make_uint4((uint32_t)f.a[mt][4], (uint32_t)f.a[mt][5], (uint32_t)f.a[mt][6],
                                (uint32_t)f.a[mt][7]);
          }
          if (kGroup && s_out != nullptr && kq == 0) s_out[(int64_t)row * so_m + (int64_t)kb * so_k] = g.s;
        }
      }
    }
    f.sw = r.sw;
    return f;
  };
  decode_tile<MT, kBf16Out, kFa, kFb, true>(p, n0, red, first, fetch, near, frags);
}

template <int MT, int kFa, int kFb>
void launch_decode(const GemmParams& p, bool bf16, bool packed, hipStream_t st) {
  const dim3 grid((unsigned)(p.N / kDecBN));
  if (packed) {
    if (bf16)
      hipLaunchKernelGGL((k_gemm_fp8_decode<MT, true, kFa, kFb, true>), grid, dim3(kDecThreads), 0, st, p);
    else
      hipLaunchKernelGGL((k_gemm_fp8_decode<MT, false, kFa, kFb, true>), grid, dim3(kDecThreads), 0, st, p);
  } else {
    if (bf16)
      hipLaunchKernelGGL((k_gemm_fp8_decode<MT, true, kFa, kFb, false>), grid, dim3(kDecThreads), 0, st, p);
    else
      hipLaunchKernelGGL((k_gemm_fp8_decode<MT, false, kFa, kFb, false>), grid, dim3(kDecThreads), 0, st, p);
  }
}

// Kernel choice for one (format of A, format of B) pair: the decode kernel for
// M <= 64 (bf16 / fp32 output), else the prefill kernel on a grid of
// n_full + 2 n_half workgroups. The fused quantized output always takes the
// prefill kernel (its epilogue needs a wave's whole 128-column group).
template <int kFa, int kFb>
void launch_formats(const GemmParams& p, int out, bool packed, hipStream_t st) {
  if (out == OUT_BF16 || out == OUT_F32) {
    const bool bf16 = out == OUT_BF16;
    if (p.M <= 16) return launch_decode<1, kFa, kFb>(p, bf16, packed, st);
    if (p.M <= 32) return launch_decode<2, kFa, kFb>(p, bf16, packed, st);
    if (p.M <= 64) return launch_decode<4, kFa, kFb>(p, bf16, packed, st);
  }
  const dim3 grid((unsigned)(p.n_full + 2 * p.n_half));
  switch (out) {
    case OUT_BF16: hipLaunchKernelGGL((k_gemm_fp8_block<OUT_BF16, kFa, kFb>), grid, dim3(kThreads), 0, st, p); break;
    case OUT_F32: hipLaunchKernelGGL((k_gemm_fp8_block<OUT_F32, kFa, kFb>), grid, dim3(kThreads), 0, st, p); break;
    case OUT_Q_E4M3: hipLaunchKernelGGL((k_gemm_fp8_block<OUT_Q_E4M3, kFa, kFb>), grid, dim3(kThreads), 0, st, p); break;
    default: hipLaunchKernelGGL((k_gemm_fp8_block<OUT_Q_E5M2, kFa, kFb>), grid, dim3(kThreads), 0, st, p); break;
  }
}

}  // namespace

// MX operands: always the prefill kernel (bf16 or fp32 output).
template <int kFa, int kFb>
void launch_mx(const GemmParams& p, int out, hipStream_t st) {
  const dim3 grid((unsigned)(p.n_full + 2 * p.n_half));
  if (out == OUT_BF16)
    hipLaunchKernelGGL((k_gemm_fp8_block<OUT_BF16, kFa, kFb, true>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((k_gemm_fp8_block<OUT_F32, kFa, kFb, true>), grid, dim3(kThreads), 0, st, p);
}

// Compute units of the current device (cached per device; 0 if unknown).
int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {
template <int MT, int kFa, int kFb, typename T, bool kGroup>
void launch_quant_gemm_decode_mt(const GemmParams& p, const QuantGemmDecodeArgs& a, FastDiv fd, bool bf16,
                                 hipStream_t st) {
  const dim3 grid((unsigned)(p.N / kDecBN));
  const T* x = static_cast<const T*>(a.x);
  if (bf16)
    hipLaunchKernelGGL((k_quant_gemm_decode<MT, true, kFa, kFb, T, kGroup>), grid, dim3(kDecThreads), 0, st, p, x,
                       a.ld_x, fd, a.packed, a.q_out, a.ld_q, a.s_out, a.so_m, a.so_k);
  else
    hipLaunchKernelGGL((k_quant_gemm_decode<MT, false, kFa, kFb, T, kGroup>), grid, dim3(kDecThreads), 0, st, p, x,
                       a.ld_x, fd, a.packed, a.q_out, a.ld_q, a.s_out, a.so_m, a.so_k);
}

template <int kFa, int kFb, typename T, bool kGroup>
void launch_quant_gemm_decode_gran(const GemmParams& p, const QuantGemmDecodeArgs& a, FastDiv fd, bool bf16,
                                   hipStream_t st) {
  if (p.M <= 16) launch_quant_gemm_decode_mt<1, kFa, kFb, T, kGroup>(p, a, fd, bf16, st);
  else if (p.M <= 32) launch_quant_gemm_decode_mt<2, kFa, kFb, T, kGroup>(p, a, fd, bf16, st);
  else launch_quant_gemm_decode_mt<4, kFa, kFb, T, kGroup>(p, a, fd, bf16, st);
}

template <int kFa, int kFb>
void launch_quant_gemm_decode_fmt(const GemmParams& p, const QuantGemmDecodeArgs& a, FastDiv fd, bool bf16,
                                  hipStream_t st) {
  const bool group = a.gran_a == GRAN_GROUP_1x128;
  if (a.x_dtype == DTYPE_BF16) {
    if (group) launch_quant_gemm_decode_gran<kFa, kFb, __hip_bfloat16, true>(p, a, fd, bf16, st);
    else launch_quant_gemm_decode_gran<kFa, kFb, __hip_bfloat16, false>(p, a, fd, bf16, st);
  } else {
    if (group) launch_quant_gemm_decode_gran<kFa, kFb, float, true>(p, a, fd, bf16, st);
    else launch_quant_gemm_decode_gran<kFa, kFb, float, false>(p, a, fd, bf16, st);
  }
}
}  // namespace

hipError_t launch_quant_gemm_decode(const QuantGemmDecodeArgs& a, hipStream_t st) {
  const GemmArgs& g = a.g;
  GemmParams p{};
  p.b = g.b;
  p.sb = g.sb;
  p.c = g.c;
  p.ldb = g.ldb;
  p.ldc = g.ldc;
  p.sb_n = g.gran_b == GRAN_PER_TENSOR ? 0 : g.sb_n;
  p.sb_k = g.gran_b == GRAN_PER_TENSOR ? 0 : g.sb_k;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  const FastDiv fd = make_fastdiv((uint32_t)(g.K / 8));
  const bool bf16 = g.c_dtype == DTYPE_BF16;
  const bool a5 = g.fmt_a == FMT_E5M2, b5 = g.fmt_b == FMT_E5M2;
  if (!a5 && !b5) launch_quant_gemm_decode_fmt<FMT_E4M3, FMT_E4M3>(p, a, fd, bf16, st);
  else if (!a5 && b5) launch_quant_gemm_decode_fmt<FMT_E4M3, FMT_E5M2>(p, a, fd, bf16, st);
  else if (a5 && !b5) launch_quant_gemm_decode_fmt<FMT_E5M2, FMT_E4M3>(p, a, fd, bf16, st);
  else launch_quant_gemm_decode_fmt<FMT_E5M2, FMT_E5M2>(p, a, fd, bf16, st);
  return hipGetLastError();
}

hipError_t launch_block_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.M == 0) return hipSuccess;
  GemmParams p;
  p.a = g.a;
  p.b = g.b;
  p.sa = g.sa;
  p.sb = g.sb;
  p.c = g.c;
  p.sa8 = g.sa8;
  p.sb8 = g.sb8;
  p.ld_sa8 = g.ld_sa8;
  p.ld_sb8 = g.ld_sb8;
  p.qc = g.qc;
  p.sc = g.sc;
  p.sc_m = g.sc_m;
  p.sc_n = g.sc_n;
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
  const int out = g.quant_out ? (g.fmt_c == FMT_E5M2 ? OUT_Q_E5M2 : OUT_Q_E4M3)
                              : (g.c_dtype == DTYPE_BF16 ? OUT_BF16 : OUT_F32);
  // tail balancing (see GemmParams)
  const int tiles = p.tiles_m * p.tiles_n;
  const int cus = (p.M > 64 || g.quant_out || g.mx) ? device_cu_count() : 0;
  const int rem = cus > 0 ? tiles % cus : 0;
  p.n_full = tiles;
  p.n_half = 0;
  if (rem > 0 && 2 * rem <= cus && rem % 4 == 0 && (tiles - rem) % 8 == 0) {
    p.n_full = tiles - rem;
    p.n_half = rem;
  }
  const bool a5 = g.fmt_a == FMT_E5M2, b5 = g.fmt_b == FMT_E5M2;
  if (g.mx) {
    if (!a5 && !b5) launch_mx<FMT_E4M3, FMT_E4M3>(p, out, st);
    else if (!a5 && b5) launch_mx<FMT_E4M3, FMT_E5M2>(p, out, st);
    else if (a5 && !b5) launch_mx<FMT_E5M2, FMT_E4M3>(p, out, st);
    else launch_mx<FMT_E5M2, FMT_E5M2>(p, out, st);
    return hipGetLastError();
  }
  // packed weights are read by the decode kernel only (the entry point
  // admits them for M <= 64 with a bf16 or fp32 output)
  const bool packed = g.b_packed != 0;
  if (packed && (p.M > 64 || g.quant_out)) return hipErrorInvalidValue;
  if (!a5 && !b5) launch_formats<FMT_E4M3, FMT_E4M3>(p, out, packed, st);
  else if (!a5 && b5) launch_formats<FMT_E4M3, FMT_E5M2>(p, out, packed, st);
  else if (a5 && !b5) launch_formats<FMT_E5M2, FMT_E4M3>(p, out, packed, st);
  else launch_formats<FMT_E5M2, FMT_E5M2>(p, out, packed, st);
  return hipGetLastError();
}

namespace {

// Decode-packed weight layout, for the decode kernel: one 2 KB block per
// (16-row group rg, K block kb), stored K-block-major at (kb * N / 16 + rg) *
// 2048. Inside a block, the 16 bytes that MFMA lane l = r + 16 g takes as the
// low (h = 0) or high (h = 1) half of its operand -- row r, bytes 32 g + 16 h
// .. + 15 of the K block -- sit at h * 1024 + 16 l, so each load instruction
// of a wave reads 1 KB contiguous. All workgroups of the decode kernel then
// stream one K block's region of N * 128 bytes at a time (39.7 us against
// 47.6 us at 16 x 28672 x 8192 for row-major weights, whose concurrent reads
// span the whole matrix). A thread per 16-byte chunk of the packed output,
// grid-stride over a capped grid (N * K may reach 2^40 bytes).
constexpr uint64_t kPackMaxGrid = 1u << 20;

__global__ __launch_bounds__(256) void k_pack_decode_weights(const uint8_t* __restrict__ w, int64_t ldw,
                                                             uint64_t row_groups, uint64_t chunks,
                                                             uint8_t* __restrict__ out) {
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  for (uint64_t t = (uint64_t)blockIdx.x * 256 + threadIdx.x; t < chunks; t += stride) {
    const uint64_t l = t & 63, h = (t >> 6) & 1;
    const uint64_t block = t >> 7;   // kb * row_groups + rg
    const uint64_t kb = block / row_groups, rg = block - kb * row_groups;
    const uint64_t row = rg * 16 + (l & 15);
    const uint64_t col = kb * 128 + 32 * (l >> 4) + 16 * h;
    *reinterpret_cast<uint4*>(out + t * 16) = *reinterpret_cast<const uint4*>(w + row * (uint64_t)ldw + col);
  }
}

}  // namespace

hipError_t launch_pack_decode_weights(const uint8_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* packed,
                                      hipStream_t st) {
  const uint64_t chunks = (uint64_t)N * (uint64_t)K / 16;
  if (chunks == 0) return hipSuccess;
  const uint64_t grid = min((chunks + 255) / 256, kPackMaxGrid);
  hipLaunchKernelGGL(k_pack_decode_weights, dim3((unsigned)grid), dim3(256), 0, st, w, ldw, (uint64_t)N / 16,
                     chunks, packed);
  return hipGetLastError();
}

}  // namespace fp8blk
