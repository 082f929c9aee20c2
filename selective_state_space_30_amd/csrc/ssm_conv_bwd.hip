// ssm_conv_bwd.hip -- gfx950 kernels of the conv prologue's backward pass.
//
// The Mamba block feeds the SSM with u = silu(conv_b + depthwise causal
// conv1d(x)) ("Mamba & State Space Models - Guide Complet", section 4
// architecture figure Conv1D -> SiLU -> SSM, section 7 Mamba block; d_conv
// = 4 on the inferownia.pl page).  The forward fuses that prologue into the
// scan and never writes u; its backward runs in three steps:
//   1. conv_fwd_kernel writes u (activation dtype) into the workspace;
//   2. the scan's backward (ssm_bwd.hip) takes that u and writes du;
//   3. conv_bwd_kernel recomputes the pre-activation, forms g = du *
//      silu'(pre), and writes dx[s] = sum_k w[k] g[s + K-1-k]; each
//      workgroup (one (batch, channel) row) sums g x and g for the taps and
//      the bias in a fixed order, and conv_reduce_kernel sums those over the
//      batch -- no atomics, so results are bitwise reproducible.
// A thread handles 16 consecutive tokens; the K-1 inputs before its first
// token and the K-1 gradients after its last are read or recomputed by the
// thread itself.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using namespace dev;

constexpr int kConvThreads = 256;
constexpr int kConvTokens = 16;  // per thread
constexpr int kConvTile = kConvThreads * kConvTokens;

template <typename T>
__device__ __forceinline__ float ld(const T *row, int64_t t, int64_t L) {
  return (t >= 0 && t < L) ? to_f32<T>(row[t]) : 0.0f;
}

// u[row, t] = silu(cb + sum_k w[k] x[row, t-(K-1)+k]), x = 0 before t = 0.
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_fwd_kernel(ConvBwdArgs p) {
  const int64_t row = blockIdx.x;  // b * dim + d
  const int64_t d = row % p.dim;
  const int K = p.d_conv;
  float w[kMaxConv];
#pragma unroll
  for (int k = 0; k < kMaxConv; ++k) w[k] = k < K ? p.conv_w[d * K + k] : 0.0f;
  const float cb = p.conv_b ? p.conv_b[d] : 0.0f;
  const T *xr = static_cast<const T *>(p.x) + row * p.L;
  T *ur = static_cast<T *>(p.u) + row * p.L;
  for (int64_t t0 = static_cast<int64_t>(threadIdx.x) * kConvTokens; t0 < p.L;
       t0 += kConvTile) {
    float xs[kConvTokens + kMaxConv - 1];  // x[t0 - 3 .. t0 + 15]
#pragma unroll
    for (int i = 0; i < kConvTokens + kMaxConv - 1; ++i)
      xs[i] = ld(xr, t0 - (kMaxConv - 1) + i, p.L);
#pragma unroll
    for (int j = 0; j < kConvTokens; ++j) {
      if (t0 + j >= p.L) break;
      float acc = cb;
#pragma unroll
      for (int k = 0; k < kMaxConv; ++k)
        if (k < K) acc = fmaf(w[k], xs[j + (kMaxConv - 1) - (K - 1) + k], acc);
      ur[t0 + j] = from_f32<T>(silu_f(acc));
    }
  }
}

// dx, and per-row sums of g * x (taps) and g (bias).
template <typename T>
__global__ __launch_bounds__(kConvThreads) void conv_bwd_kernel(ConvBwdArgs p) {
  __shared__ float red[kConvThreads / kWaveLanes][kMaxConv + 1];
  const int64_t row = blockIdx.x;
  const int64_t d = row % p.dim;
  const int K = p.d_conv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float w[kMaxConv];
#pragma unroll
  for (int k = 0; k < kMaxConv; ++k) w[k] = k < K ? p.conv_w[d * K + k] : 0.0f;
  const float cb = p.conv_b ? p.conv_b[d] : 0.0f;
  const T *xr = static_cast<const T *>(p.x) + row * p.L;
  const T *dur = static_cast<const T *>(p.du) + row * p.L;
  T *dxr = static_cast<T *>(p.dx) + row * p.L;
  float sw[kMaxConv] = {0.0f, 0.0f, 0.0f, 0.0f};
  float sb = 0.0f;
  constexpr int kG = kConvTokens + kMaxConv - 1;  // g for t0 .. t0 + 18
  for (int64_t t0 = static_cast<int64_t>(threadIdx.x) * kConvTokens; t0 < p.L;
       t0 += kConvTile) {
    // x[t0 - 3 .. t0 + 18]: the inputs of the pre-activations of t0 .. t0 + 18
    float xs[kG + kMaxConv - 1];
#pragma unroll
    for (int i = 0; i < kG + kMaxConv - 1; ++i) xs[i] = ld(xr, t0 - (kMaxConv - 1) + i, p.L);
    float g[kG];
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      float pre = cb;
#pragma unroll
      for (int k = 0; k < kMaxConv; ++k)
        if (k < K) pre = fmaf(w[k], xs[i + (kMaxConv - 1) - (K - 1) + k], pre);
      g[i] = ld(dur, t0 + i, p.L) * dsilu_f(pre);  // 0 past the end
    }
#pragma unroll
    for (int j = 0; j < kConvTokens; ++j) {
      if (t0 + j >= p.L) break;
      // x[s] feeds the outputs s + (K-1) - k through tap k
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < kMaxConv; ++k)
        if (k < K) acc = fmaf(w[k], g[j + (K - 1) - k], acc);
      dxr[t0 + j] = from_f32<T>(acc);
      // output t0 + j used x[t0 + j - (K-1) + k] through tap k
#pragma unroll
      for (int k = 0; k < kMaxConv; ++k)
        if (k < K) sw[k] = fmaf(g[j], xs[j + (kMaxConv - 1) - (K - 1) + k], sw[k]);
      sb += g[j];
    }
  }
  // the workgroup's sums, in a fixed order: within each wave by the DPP
  // prefix sum, then the waves in order
#pragma unroll
  for (int k = 0; k < kMaxConv + 1; ++k) {
    const float v = k < kMaxConv ? sw[k] : sb;
    const float s = lane_broadcast(wave_inclusive_sum(v), kWaveLanes - 1);
    if (lane == 0) red[wave][k] = s;
  }
  __syncthreads();
  if (threadIdx.x <= kMaxConv) {
    float acc = 0.0f;
    for (int i = 0; i < kConvThreads / kWaveLanes; ++i) acc += red[i][threadIdx.x];
    p.part[row * (kMaxConv + 1) + threadIdx.x] = acc;
  }
}

// dconv_w[d, k] and dconv_b[d]: the rows' sums added over the batch in order.
__global__ __launch_bounds__(256) void conv_reduce_kernel(ConvBwdArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= p.dim * (kMaxConv + 1)) return;
  const int64_t d = i / (kMaxConv + 1);
  const int k = static_cast<int>(i % (kMaxConv + 1));
  float acc = 0.0f;
  for (int64_t b = 0; b < p.batch; ++b) acc += p.part[(b * p.dim + d) * (kMaxConv + 1) + k];
  if (k < p.d_conv)
    p.dconv_w[d * p.d_conv + k] = acc;
  else if (k == kMaxConv && p.dconv_b)
    p.dconv_b[d] = acc;
}

template <typename T>
hipError_t launch_conv_fwd_t(const ConvBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(conv_fwd_kernel<T>, dim3(static_cast<unsigned>(a.batch * a.dim)),
                     dim3(kConvThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_conv_bwd_t(const ConvBwdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL(conv_bwd_kernel<T>, dim3(static_cast<unsigned>(a.batch * a.dim)),
                     dim3(kConvThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = a.dim * (kMaxConv + 1);
  hipLaunchKernelGGL(conv_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int launch_conv_fwd(const ConvBwdArgs &a, bool bf16, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return bf16 ? launch_conv_fwd_t<uint16_t>(a, s) : launch_conv_fwd_t<float>(a, s);
}

int launch_conv_bwd(const ConvBwdArgs &a, bool bf16, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return bf16 ? launch_conv_bwd_t<uint16_t>(a, s) : launch_conv_bwd_t<float>(a, s);
}

}  // namespace ssm
