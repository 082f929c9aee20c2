// ssm_step.hip -- gfx950 (CDNA4) kernel of the selective SSM's single-token
// decoding step.
//
// One token advances every (batch, channel) state in place: dt =
// softplus(delta + bias), h = exp(dt*A) (.) h + dt*B*x, y = (C . h + D*x) *
// silu(z).  Sources: "Mamba & State Space Models - Guide Complet", section 4
// "Implementation du SSM selectif (S6)" (one iteration of its per-token
// loop); the johe.ru page "Mamba и State Space Models", section "SSM as RNN"
// (the recurrent view used for generation).
//
// The fp32 state (batch, dim, 16) is read and written once per step, so the
// kernel is bound by HBM: it is laid out for coalesced 16-byte accesses and
// enough loads in flight, and its arithmetic is a few dozen instructions per
// channel.  Other state counts (up to 256) take a plainer
// one-wave-per-channel kernel.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using namespace dev;

// Four lanes per (batch, channel), four states each: the fp32 state is read
// and written with 16-byte accesses, fully coalesced; the 4-lane readout is
// a two-step DPP reduction inside each quad.  A thread serves one channel
// for kStepBatch batch entries, so A, D and the bias are read once for
// them, and the loads of both states are in flight together.  The state is
// touched once per step: its loads and stores are non-temporal.
constexpr int kStepBatch = 2;
constexpr int kStepThreads = 256;
constexpr int kStepChannels = kStepThreads / 4;  // per workgroup

typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <bool kVec>
__device__ __forceinline__ void load_state4(const float *p, float (&h)[4]) {
  if constexpr (kVec) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(p));
    h[0] = v[0]; h[1] = v[1]; h[2] = v[2]; h[3] = v[3];
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = __builtin_nontemporal_load(p + i);
  }
}

template <bool kVec>
__device__ __forceinline__ void store_state4(float *p, const float (&h)[4]) {
  if constexpr (kVec) {
    const f32x4_t v = {h[0], h[1], h[2], h[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t *>(p));
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(h[i], p + i);
  }
}

// Four consecutive activations (B or C states) as fp32: one 8- or 16-byte
// load when kVec (the caller has checked the alignment).
template <typename T, bool kVec>
__device__ __forceinline__ void load_act4(const T *p, float (&v)[4]) {
  if constexpr (kVec && sizeof(T) == 2) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  } else if constexpr (kVec) {
    const float4 w = *reinterpret_cast<const float4 *>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = to_f32<T>(p[i]);
  }
}

// grid: (ceil(dim / kStepChannels), ceil(batch / kStepBatch)); thread =
// (channel d, states 4q .. 4q+3) for batch entries kStepBatch*blockIdx.y + u.
// kConv: the input x passes through the causal conv1d + SiLU first (the
// same prologue as the scan's), its window carried in conv_state.
template <typename T, bool kVec, bool kConv>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs p) {
  constexpr int U = kStepBatch;
  const uint32_t dim = static_cast<uint32_t>(p.dim);
  const uint32_t batch = static_cast<uint32_t>(p.batch);
  const int q = threadIdx.x & 3;
  const uint32_t d_raw = blockIdx.x * kStepChannels + (threadIdx.x >> 2);
  const bool d_ok = d_raw < dim;
  const uint32_t d = d_ok ? d_raw : dim - 1;  // clamped for reads
  uint32_t bc[U];  // batch entry, clamped for reads
  size_t ch[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t b = blockIdx.y * U + u;
    ok[u] = d_ok && b < batch;
    bc[u] = b < batch ? b : batch - 1;
    ch[u] = static_cast<size_t>(bc[u]) * dim + d;
  }

  float h[U][4], a4[4];
  if constexpr (kVec) {
    const float4 av = *reinterpret_cast<const float4 *>(p.A + d * kStates + 4 * q);
    a4[0] = av.x; a4[1] = av.y; a4[2] = av.z; a4[3] = av.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) a4[i] = p.A[d * kStates + 4 * q + i];
  }
  // conv prologue.  Slots 0..kMaxConv-1 of a channel's conv input are the
  // kMaxConv - 1 window positions, then x; the taps are aligned to the last
  // slots and the kept inputs to the last window positions, so with d_conv
  // taps the first kMaxConv - d_conv slots have neither (zeros).  Lane q of
  // the quad loads tap q and window position q, once for the whole quad, at
  // a clamped valid address; the values reach the other lanes by DPP
  // broadcast and the absent slots are zeroed there, on a condition uniform
  // across the wave (a per-lane select right after a load would make the
  // compiler wait for it before the state loads are issued).
  float wq = 0.0f, cb = 0.0f, wl[U];
  int K = 0, H = 0;
  if constexpr (kConv) {
    K = p.d_conv;
    H = K - 1;
    const int ti = q - (kMaxConv - K);       // tap of lane q, or none
    const int wi = q - (kMaxConv - 1 - H);   // kept input of lane q, or none
    const float cb_raw = (p.conv_b ? p.conv_b : p.conv_w)[d];
    wq = p.conv_w[d * K + (ti < 0 ? 0 : ti)];
    // H = 0: no window; every lane reads x (stride 1, a valid address).  One
    // address form for both, so the load is not branched.
    const T *cs = static_cast<const T *>(H > 0 ? p.conv_state : p.x);
    const uint32_t hs = H > 0 ? H : 1;
    const int hmax = H > 0 ? H - 1 : 0;
    const uint32_t idx = wi < 0 ? 0 : (wi > hmax ? hmax : wi);
#pragma unroll
    for (int u = 0; u < U; ++u) wl[u] = to_f32<T>(cs[ch[u] * hs + idx]);
    cb = p.conv_b ? cb_raw : 0.0f;
  }

  // Every load is unconditional (an absent bias, D or gate reads some other
  // valid input and is zeroed at its use): a load under a branch would make
  // the merge wait for every load in flight, the state's included, before
  // the rest are issued.
  const float bias_raw = (p.bias ? p.bias : p.A)[d];
  const float D_raw = (p.D ? p.D : p.A)[d];
  const T *zsrc = static_cast<const T *>(p.z ? p.z : p.x);
  float x[U], dr[U], zz[U], b4[U][4], c4[U][4];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const size_t bsel = bc[u];
    x[u] = to_f32<T>(static_cast<const T *>(p.x)[ch[u]]);
    dr[u] = to_f32<T>(static_cast<const T *>(p.delta)[ch[u]]);
    zz[u] = to_f32<T>(zsrc[ch[u]]);
    load_act4<T, kVec>(static_cast<const T *>(p.B) + bsel * kStates + 4 * q, b4[u]);
    load_act4<T, kVec>(static_cast<const T *>(p.C) + bsel * kStates + 4 * q, c4[u]);
  }
  // the state last: the wait counter retires loads in order, so the
  // arithmetic on the small inputs can start while the state is in flight
#pragma unroll
  for (int u = 0; u < U; ++u) load_state4<kVec>(p.state + ch[u] * kStates + 4 * q, h[u]);
  const float bias = p.bias ? bias_raw : 0.0f;
  const float Dd = p.D ? D_raw : 0.0f;
  float xin[U], wnew[U];  // the raw input; this lane's next window entry
  if constexpr (kConv) {
    static_assert(kMaxConv == 4, "one slot per lane of a quad");
    const int lead = kMaxConv - K;  // slots with no tap and no kept input
    const float wc[kMaxConv] = {lead > 0 ? 0.0f : dpp<0x00>(wq, wq),
                                lead > 1 ? 0.0f : dpp<0x55>(wq, wq),
                                lead > 2 ? 0.0f : dpp<0xAA>(wq, wq),
                                dpp<0xFF>(wq, wq)};
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float s0 = lead > 0 ? 0.0f : dpp<0x00>(wl[u], wl[u]);
      const float s1 = lead > 1 ? 0.0f : dpp<0x55>(wl[u], wl[u]);
      const float s2 = lead > 2 ? 0.0f : dpp<0xAA>(wl[u], wl[u]);
      float acc = fmaf(wc[0], s0, cb);
      acc = fmaf(wc[1], s1, acc);
      acc = fmaf(wc[2], s2, acc);
      acc = fmaf(wc[3], x[u], acc);
      xin[u] = x[u];
      x[u] = silu_f(acc);
      // the window moves by one: kept input q becomes slot kMaxConv - H + q
      // of (window, x)
      const int sl = kMaxConv - H + q;
      wnew[u] = sl == 1 ? s1 : (sl == 2 ? s2 : xin[u]);
    }
  }
  float part[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const float xr = dr[u] + bias;
    const float dt = p.softplus ? softplus_f(xr) : xr;
    const float dx = dt * x[u];
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float arg = dt * a4[i] * kLog2e;
      const float e = fast_exp2(arg);
      float inp = dx * b4[u][i];
      if (p.zoh)  // exact ZOH: coefficient (e - 1)/A in place of dt
        inp = zoh_coeff(arg, e, dt * kLog2e, 1.0f / a4[i]) * (x[u] * b4[u][i]);
      h[u][i] = fmaf(e, h[u][i], inp);
      acc = fmaf(c4[u][i], h[u][i], acc);
    }
    acc += dpp<kQuadXor1>(acc, acc);
    acc += dpp<kQuadXor2>(acc, acc);
    asm volatile("" : "+v"(acc));  // reduced by all four lanes before any branch
    part[u] = acc;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!ok[u]) continue;
    store_state4<kVec>(p.state + ch[u] * kStates + 4 * q, h[u]);
    if constexpr (kConv) {
      if (q < H) static_cast<T *>(p.conv_state)[ch[u] * H + q] = from_f32<T>(wnew[u]);
    }
    if (q == 0) {
      float yv = fmaf(Dd, x[u], part[u]);
      if (p.z) yv *= silu_f(zz[u]);
      static_cast<T *>(p.y)[ch[u]] = from_f32<T>(yv);
    }
  }
}

// Any other d_state up to 256: one wave per (batch, channel), state n in
// lane n % 64 (up to four per lane); the readout is a wave sum.  The same
// arithmetic per state as step_kernel (and its conv window: the d_conv - 1
// kept inputs, oldest first, then x; the window moves by one).
constexpr int kLaneStepWaves = 4;  // channels per workgroup
constexpr int kLaneStepStates = 4;  // states per lane at most

template <typename T, bool kConv>
__global__ __launch_bounds__(kLaneStepWaves * kWaveLanes) void step_lanes_kernel(StepArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kLaneStepWaves + (threadIdx.x >> 6);
  const int64_t b = blockIdx.y;
  const bool d_ok = d_raw < p.dim;
  const int64_t d = d_ok ? d_raw : p.dim - 1;  // clamped for reads
  const int N = p.N;
  const int64_t ch = b * p.dim + d;
  float x = to_f32<T>(static_cast<const T *>(p.x)[ch]);
  const float dr = to_f32<T>(static_cast<const T *>(p.delta)[ch]);
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  float wnew = 0.0f;  // lane k < d_conv - 1: the window's next entry k
  int H = 0;
  if constexpr (kConv) {
    const int K = p.d_conv;
    H = K - 1;
    const T *cs = static_cast<const T *>(p.conv_state) + ch * (H > 0 ? H : 0);
    float acc = p.conv_b ? p.conv_b[d] : 0.0f;
    for (int k = 0; k < H; ++k) acc = fmaf(p.conv_w[d * K + k], to_f32<T>(cs[k]), acc);
    acc = fmaf(p.conv_w[d * K + H], x, acc);
    if (lane < H) wnew = lane + 1 < H ? to_f32<T>(cs[lane + 1]) : x;
    x = silu_f(acc);
  }
  const float xr = dr + bias;
  const float dt = p.softplus ? softplus_f(xr) : xr;
  float h[kLaneStepStates], part = 0.0f;
#pragma unroll
  for (int i = 0; i < kLaneStepStates; ++i) {
    const int n = kWaveLanes * i + lane;
    const bool on = n < N;
    const int ns = on ? n : 0;  // clamped for reads
    const float An = p.A[d * N + ns];
    const float Bn = to_f32<T>(static_cast<const T *>(p.B)[b * N + ns]);
    const float Cn = to_f32<T>(static_cast<const T *>(p.C)[b * N + ns]);
    h[i] = p.state[ch * N + ns];
    const float arg = dt * An * kLog2e;
    const float e = fast_exp2(arg);
    float inp = dt * x * Bn;
    if (p.zoh)  // exact ZOH: coefficient (e - 1)/A in place of dt
      inp = zoh_coeff(arg, e, dt * kLog2e, 1.0f / An) * (x * Bn);
    h[i] = fmaf(e, h[i], inp);
    part += on ? Cn * h[i] : 0.0f;
  }
  float sum = lane_broadcast(wave_inclusive_sum(part), kWaveLanes - 1);
  asm volatile("" : "+s"(sum));  // formed by the whole wave first
  if (!d_ok) return;
#pragma unroll
  for (int i = 0; i < kLaneStepStates; ++i) {
    const int n = kWaveLanes * i + lane;
    if (n < N) p.state[ch * N + n] = h[i];
  }
  if (kConv && lane < H) static_cast<T *>(p.conv_state)[ch * H + lane] = from_f32<T>(wnew);
  if (lane == 0) {
    float yv = fmaf(Dd, x, sum);
    if (p.z) yv *= silu_f(to_f32<T>(static_cast<const T *>(p.z)[ch]));
    static_cast<T *>(p.y)[ch] = from_f32<T>(yv);
  }
}

template <typename T, bool kVec>
hipError_t launch_step_t(const StepArgs &a, hipStream_t s) {
  if (a.N != kStates) {
    const dim3 lgrid(static_cast<unsigned>((a.dim + kLaneStepWaves - 1) / kLaneStepWaves),
                     static_cast<unsigned>(a.batch));
    if (a.d_conv > 0)
      hipLaunchKernelGGL((step_lanes_kernel<T, true>), lgrid, dim3(kLaneStepWaves * kWaveLanes),
                         0, s, a);
    else
      hipLaunchKernelGGL((step_lanes_kernel<T, false>), lgrid, dim3(kLaneStepWaves * kWaveLanes),
                         0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((a.dim + kStepChannels - 1) / kStepChannels),
                  static_cast<unsigned>((a.batch + kStepBatch - 1) / kStepBatch));
  if (a.d_conv > 0)
    hipLaunchKernelGGL((step_kernel<T, kVec, true>), grid, dim3(kStepThreads), 0, s, a);
  else
    hipLaunchKernelGGL((step_kernel<T, kVec, false>), grid, dim3(kStepThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int launch_step(const StepArgs &a, bool bf16, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch_step_t<uint16_t, true>(a, s) : launch_step_t<uint16_t, false>(a, s);
  return vec ? launch_step_t<float, true>(a, s) : launch_step_t<float, false>(a, s);
}

}  // namespace ssm
