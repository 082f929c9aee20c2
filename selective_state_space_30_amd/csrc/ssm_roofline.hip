// ssm_roofline.hip -- gfx950 microbenchmarks that measure the two ceilings
// the scan kernels are held against, on the machine and in the run that
// measures the kernels:
//   * HBM: a non-temporal 16-byte copy, an in-place read-modify-write (the
//     decode step's access pattern) and a read-only pass over buffers much
//     larger than the last-level cache;
//   * VALU issue: long chains of v_exp_f32 (the transcendental every state
//     update needs once), of v_fma_f32, and of the two interleaved (whether
//     a transcendental overlaps other VALU work).
// None of this is part of the method; the benchmark calls it to report the
// scan's fraction of what the hardware sustains.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int kRoofThreads = 256;
constexpr int kRoofPer = 4;  // 16-byte pieces per thread

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 nt_load(const float4 *p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store(float4 v, float4 *p) {
  const f32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4_t *>(p));
}

// Each workgroup covers kRoofThreads * kRoofPer consecutive 16-byte pieces,
// thread-interleaved so every load instruction of a wave is one contiguous
// 1 KB span; n16 is a multiple of that span (checked by the host).
__global__ __launch_bounds__(kRoofThreads) void roof_copy_kernel(
    const float4 *__restrict__ src, float4 *__restrict__ dst) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kRoofThreads * kRoofPer +
                       threadIdx.x;
  float4 v[kRoofPer];
#pragma unroll
  for (int k = 0; k < kRoofPer; ++k) v[k] = nt_load(src + base + k * kRoofThreads);
#pragma unroll
  for (int k = 0; k < kRoofPer; ++k) nt_store(v[k], dst + base + k * kRoofThreads);
}

__global__ __launch_bounds__(kRoofThreads) void roof_rmw_kernel(float4 *__restrict__ buf,
                                                                float a, float b) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kRoofThreads * kRoofPer +
                       threadIdx.x;
  float4 v[kRoofPer];
#pragma unroll
  for (int k = 0; k < kRoofPer; ++k) v[k] = nt_load(buf + base + k * kRoofThreads);
#pragma unroll
  for (int k = 0; k < kRoofPer; ++k) {
    v[k].x = fmaf(v[k].x, a, b);
    v[k].y = fmaf(v[k].y, a, b);
    v[k].z = fmaf(v[k].z, a, b);
    v[k].w = fmaf(v[k].w, a, b);
    nt_store(v[k], buf + base + k * kRoofThreads);
  }
}

// Read only: the sum of every loaded value is kept live by a store that
// happens only when it equals a value no input of the benchmark produces.
__global__ __launch_bounds__(kRoofThreads) void roof_read_kernel(
    const float4 *__restrict__ src, float *__restrict__ sink) {
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kRoofThreads * kRoofPer +
                       threadIdx.x;
  float acc = 0.0f;
#pragma unroll
  for (int k = 0; k < kRoofPer; ++k) {
    const float4 v = nt_load(src + base + k * kRoofThreads);
    acc += (v.x + v.y) + (v.z + v.w);
  }
  if (acc == -1.25e-30f) sink[0] = acc;
}

// VALU issue rate: eight independent chains per thread so that the issue
// rate, not the latency of one chain, bounds the loop.  kind 0: x = 2^-x
// (one v_exp_f32 with a negated source, values stay in [0.5, 1]); kind 1:
// x = x * a + b (one v_fma_f32); kind 2: four chains of each, interleaved.
constexpr int kChains = 8;

template <int kKind>
__global__ __launch_bounds__(kRoofThreads) void roof_valu_kernel(float *__restrict__ out,
                                                                 int iters, float a,
                                                                 float b) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kRoofThreads + threadIdx.x;
  float x[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
    x[k] = 0.5f + 0.0625f * static_cast<float>((threadIdx.x + k) & 7);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) {
      const bool is_exp = kKind == 0 || (kKind == 2 && (k & 1) == 0);
      x[k] = is_exp ? __builtin_amdgcn_exp2f(-x[k]) : fmaf(x[k], a, b);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += x[k];
  out[tid] = s;
}

}  // namespace

int launch_roofline_hbm(int kind, void *a, void *b, int64_t n16, int repeats,
                        void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t span = static_cast<int64_t>(kRoofThreads) * kRoofPer;
  const dim3 grid(static_cast<unsigned>(n16 / span));
  for (int r = 0; r < repeats; ++r) {
    if (kind == 0)
      hipLaunchKernelGGL(roof_copy_kernel, grid, dim3(kRoofThreads), 0, s,
                         static_cast<const float4 *>(a), static_cast<float4 *>(b));
    else if (kind == 1)
      hipLaunchKernelGGL(roof_rmw_kernel, grid, dim3(kRoofThreads), 0, s,
                         static_cast<float4 *>(a), 0.5f, 0.25f);
    else
      hipLaunchKernelGGL(roof_read_kernel, grid, dim3(kRoofThreads), 0, s,
                         static_cast<const float4 *>(a), static_cast<float *>(b));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return static_cast<int>(e);
  }
  return 0;
}

int launch_roofline_valu(int kind, float *out, int64_t threads, int iters, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(threads / kRoofThreads));
  using Fn = void (*)(float *, int, float, float);
  static constexpr Fn fns[3] = {roof_valu_kernel<0>, roof_valu_kernel<1>,
                                roof_valu_kernel<2>};
  hipLaunchKernelGGL(fns[kind], grid, dim3(kRoofThreads), 0, s, out, iters, 0.999f,
                     0.001f);
  return static_cast<int>(hipGetLastError());
}

}  // namespace ssm
