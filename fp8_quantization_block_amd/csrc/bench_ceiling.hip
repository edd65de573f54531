// Measurement-only kernel (not part of the product library): the throughput
// ceiling of the FP8 MFMA used by the block-scaled GEMM on this chip, with no
// memory traffic, for given operand bytes and a given number of independent
// fp32 FMAs issued per MFMA (the GEMM's per-K-block promotion issues 4 per
// MFMA). The chip's clock under MFMA load depends on power, and power on the
// operand bits, so the ceiling is measured on the workload's own codes.
//
// Each wave keeps its operand fragments in registers (taken from `a_codes` /
// `b_codes`, 64 lanes x 32 bytes each) and issues 8 v_mfma_scale 16x16x128
// FP8 per iteration into 4 independent accumulators; `fmas` (0, 2, 4 or 8)
// independent FMAs follow each MFMA. One workgroup is 4 waves, one per SIMD.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int kFma>
__global__ __launch_bounds__(256) void k_mfma_ceiling(const int32_t* a_codes, const int32_t* b_codes, float* out,
                                                      int iters) {
  const int lane = threadIdx.x & 63;
  v8i a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = a_codes[lane * 8 + i];
    b[i] = b_codes[lane * 8 + i];
  }
  v4f p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, p2 = p0, p3 = p0;
  float f[8];
  for (int i = 0; i < 8; ++i) f[i] = (float)(lane + i);
  const float c = 1.0001f, d = 0.999f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v4f& pj = (j & 3) == 0 ? p0 : (j & 3) == 1 ? p1 : (j & 3) == 2 ? p2 : p3;
      pj = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, pj, 0, 0, 0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < kFma; ++q) f[q] = __builtin_fmaf(f[q], c, d);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const v4f pp = p0 + p1 + p2 + p3;
  float s = pp[0] + pp[1] + pp[2] + pp[3];
  for (int i = 0; i < 8; ++i) s += f[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// a_codes, b_codes: device pointers to at least 512 int32 each (2 KB of FP8
// codes; codes 0x7F / 0xFF must not occur). out: device, blocks * 256 floats.
// Launches `blocks` workgroups of 256 threads running `iters` iterations of 8
// MFMAs per wave. Returns 0, or -1 for an unsupported `fmas` / bad sizes, or
// the HIP error code of the launch.
extern "C" int fp8blk_bench_mfma_ceiling(const int32_t* a_codes, const int32_t* b_codes, float* out, int fmas,
                                         int blocks, int iters, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || !a_codes || !b_codes || !out) return -1;
  const dim3 grid(blocks), block(256);
  switch (fmas) {
    case 0: hipLaunchKernelGGL(k_mfma_ceiling<0>, grid, block, 0, stream, a_codes, b_codes, out, iters); break;
    case 2: hipLaunchKernelGGL(k_mfma_ceiling<2>, grid, block, 0, stream, a_codes, b_codes, out, iters); break;
    case 4: hipLaunchKernelGGL(k_mfma_ceiling<4>, grid, block, 0, stream, a_codes, b_codes, out, iters); break;
    case 8: hipLaunchKernelGGL(k_mfma_ceiling<8>, grid, block, 0, stream, a_codes, b_codes, out, iters); break;
    default: return -1;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
