// ssm_device.h -- device-side building blocks shared by the gfx950 scan
// kernels (forward, decode, backward): transcendental helpers, bf16
// packing, run loads and stores (16-byte vector loads in full blocks, buffer
// views with hardware range checks in partial ones), the DPP wave scans and
// the B/C staging runs.  Included by the .hip sources only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_internal.h"

namespace ssm {
namespace dev {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// DPP controls (GFX9 encoding).
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]

// Value of `src` from another lane.  Where the source lane does not exist
// (row shifts at the row edge) the result is 0 when kZero, otherwise `old`.
template <int kCtrl, int kRowMask = 0xF, int kBankMask = 0xF, bool kZero = false>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      __float_as_int(old), __float_as_int(src), kCtrl, kRowMask, kBankMask,
      kZero));
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// softplus(x) = log(1 + e^x) = max(x, 0) + log1p(e^-|x|).  log1p(e) is
// log(w) with w = fl(1 + e), corrected by the exactly representable rounding
// error r = e - (w - 1): log(1 + e) = log(w) + r/w + O(r^2) and r/w ~ r.
__device__ __forceinline__ float softplus_f(float x) {
  const float e = fast_exp2(-fabsf(x) * kLog2e);
  const float w = 1.0f + e;
  const float r = e - (w - 1.0f);
  const float l = fmaf(__builtin_amdgcn_logf(w), kLn2, r);
  return fmaxf(x, 0.0f) + l;
}

// silu(z) = z * sigmoid(z) = z / (1 + e^-z); for z -> -inf the reciprocal of
// +inf is 0 and the result is -0.
__device__ __forceinline__ float silu_f(float z) {
  const float e = fast_exp2(-z * kLog2e);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// sigmoid(x) = 1 / (1 + e^-x), the derivative of softplus.
__device__ __forceinline__ float sigmoid_f(float x) {
  return __builtin_amdgcn_rcpf(1.0f + fast_exp2(-x * kLog2e));
}

// d silu(z) / dz = sigmoid(z) (1 + z (1 - sigmoid(z))).
__device__ __forceinline__ float dsilu_f(float z) {
  const float s = sigmoid_f(z);
  return s * fmaf(z, 1.0f - s, 1.0f);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// Two fp32 -> one word of two bf16 (lo = first), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r.x = static_cast<__bf16>(lo);
  r.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, r);
}

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) {
  return static_cast<uint16_t>(f32_to_bf16_bits(v));
}

// Buffer resource (V#) word 3 for gfx9-family untyped buffer access: 32-bit
// data format, no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;

// Wave-uniform byte view of row[t0, tend) for buffer loads and stores.  The
// hardware range check makes a load past the end return 0 and drops a store
// past it, so the last, partial block of a chunk needs no per-element
// bounds arithmetic.  `row + t0` must be the same in every lane.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_view(const T *row,
                                                           int64_t t0,
                                                           int64_t tend) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<T *>(row + t0), 0,
      static_cast<int>((tend - t0) * static_cast<int64_t>(sizeof(T))),
      kBufferWord3);
}

// Loads K consecutive activations row[t .. t+K) as fp32.  kInRange: the run
// lies wholly inside the data, fetched with 16-byte loads under kVec (the
// caller guarantees 16-byte alignment of row + t), else element by element.
// Otherwise the run belongs to the partial block [t0, tend) (t0 wave-uniform)
// and is read through its buffer view: positions >= tend read as 0.
template <typename T, int K, bool kVec, bool kInRange>
__device__ __forceinline__ void load_run(const T *__restrict__ row, int64_t t0,
                                         int64_t t, int64_t tend,
                                         float (&v)[K]) {
  if constexpr (kInRange && kVec) {
    if constexpr (sizeof(T) == 2) {
      const uint4 *p = reinterpret_cast<const uint4 *>(row + t);
#pragma unroll
      for (int q = 0; q < K / 8; ++q) {
        const uint4 w = p[q];
        v[8 * q + 0] = bf16_lo(w.x);
        v[8 * q + 1] = bf16_hi(w.x);
        v[8 * q + 2] = bf16_lo(w.y);
        v[8 * q + 3] = bf16_hi(w.y);
        v[8 * q + 4] = bf16_lo(w.z);
        v[8 * q + 5] = bf16_hi(w.z);
        v[8 * q + 6] = bf16_lo(w.w);
        v[8 * q + 7] = bf16_hi(w.w);
      }
    } else {
      const float4 *p = reinterpret_cast<const float4 *>(row + t);
#pragma unroll
      for (int q = 0; q < K / 4; ++q) {
        const float4 w = p[q];
        v[4 * q + 0] = w.x;
        v[4 * q + 1] = w.y;
        v[4 * q + 2] = w.z;
        v[4 * q + 3] = w.w;
      }
    }
  } else if constexpr (kInRange) {
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = to_f32<T>(row[t + j]);
  } else {
    const __amdgpu_buffer_rsrc_t r = row_view(row, t0, tend);
    const int off = static_cast<int>(t - t0) * static_cast<int>(sizeof(T));
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if constexpr (sizeof(T) == 2)
        v[j] = __uint_as_float(static_cast<uint32_t>(
                                   __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * j, 0, 0))
                               << 16);
      else
        v[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * j, 0, 0));
    }
  }
}

// Stores a K-token run; the counterpart of load_run (positions >= tend of a
// partial block are dropped).
template <typename T, int K, bool kVec, bool kInRange>
__device__ __forceinline__ void store_run(T *__restrict__ row, int64_t t0,
                                          int64_t t, int64_t tend,
                                          const float (&v)[K]) {
  if constexpr (kInRange && kVec) {
    if constexpr (sizeof(T) == 2) {
      uint4 *p = reinterpret_cast<uint4 *>(row + t);
#pragma unroll
      for (int q = 0; q < K / 8; ++q) {
        uint4 w;
        w.x = pack_bf16x2(v[8 * q + 0], v[8 * q + 1]);
        w.y = pack_bf16x2(v[8 * q + 2], v[8 * q + 3]);
        w.z = pack_bf16x2(v[8 * q + 4], v[8 * q + 5]);
        w.w = pack_bf16x2(v[8 * q + 6], v[8 * q + 7]);
        p[q] = w;
      }
    } else {
      float4 *p = reinterpret_cast<float4 *>(row + t);
#pragma unroll
      for (int q = 0; q < K / 4; ++q)
        p[q] = make_float4(v[4 * q + 0], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
  } else if constexpr (kInRange) {
#pragma unroll
    for (int j = 0; j < K; ++j) row[t + j] = from_f32<T>(v[j]);
  } else {
    const __amdgpu_buffer_rsrc_t r = row_view(static_cast<const T *>(row), t0, tend);
    const int off = static_cast<int>(t - t0) * static_cast<int>(sizeof(T));
#pragma unroll
    for (int j = 0; j < K; ++j) {
      if constexpr (sizeof(T) == 2)
        __builtin_amdgcn_raw_buffer_store_b16(
            static_cast<unsigned short>(f32_to_bf16_bits(v[j])), r, off + 2 * j, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[j]), r, off + 4 * j, 0, 0);
    }
  }
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_sum(float v) {
  v += dpp<kRowShr1, 0xF, 0xF, true>(0.0f, v);
  v += dpp<kRowShr2, 0xF, 0xF, true>(0.0f, v);
  v += dpp<kRowShr4, 0xF, 0xF, true>(0.0f, v);
  v += dpp<kRowShr8, 0xF, 0xF, true>(0.0f, v);
  v += dpp<kRowBcast15, 0xA, 0xF, false>(0.0f, v);
  v += dpp<kRowBcast31, 0xC, 0xF, false>(0.0f, v);
  return v;
}

// ---------------------------------------------------------------- scan ---
// Inclusive scan of affine maps h -> P*h + H over the 64 lanes of a wave,
// earlier lanes composed into later ones:
//   (P, H)_i <- (P_i * P_j, P_i * H_j + H_i),  j = i - s,  s = 1, 2, 4, 8
// inside each 16-lane row, then across rows (lane 15 -> rows 1 and 3, lane
// 31 -> rows 2 and 3).  Each step is one DPP-fused VALU operation: where the
// source lane does not exist, H adds 0 (bound_ctrl) and P is left unwritten.
// `s_nop 1` gives every DPP read the two wait states it needs after a VALU
// write of its source.  On return H_i is the composition of lanes 0..i; P is
// not meaningful any more.
__device__ __forceinline__ void wave_affine_scan(float &P, float &H) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "v_mul_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %1, %1, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      : "+v"(P), "+v"(H));
}

// Lane i receives H of lane i - 1; lane 0 receives `first`.
__device__ __forceinline__ float wave_shift_in(float H, float first) {
  float r = first;
  asm volatile(
      "s_nop 1\n\t"
      "v_mov_b32_dpp %0, %1 wave_shr:1 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(r)
      : "v"(H));
  return r;
}

__device__ __forceinline__ float lane_broadcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Exact zero-order-hold input coefficient of one state, (exp(dt*A) - 1) / A
// ("Mamba & State Space Models - Guide Complet", section 1: B_bar =
// (exp(dt A) - I) A^-1 B; for a diagonal A, per state).  `arg` = dt*A*log2(e)
// (the exp2 argument), `a` = exp2(arg), `dtl` = dt*log2(e), `inv_a` = 1/A.
// Where |arg| < 2^-5 the difference a - 1 would lose up to ~2^-18 relative
// accuracy, so the series dt * (1 + x/2 + x^2/6), x = dt*A = arg*ln2, is
// used instead (truncation below 4e-7 relative there), written in dtl and
// arg: dtl * (ln2 + arg ln2^2/2 + arg^2 ln2^3/6).  A = 0 takes the series
// (arg = 0) and gives dt, the limit; the infinite inv_a of the other operand
// is not selected.  The direct form is one fused a*(1/A) - 1/A: the exact
// a/A - 1/A rounded once (a - 1 itself is exact for a in [1/2, 2]).
__device__ __forceinline__ float zoh_coeff(float arg, float a, float dtl,
                                           float inv_a) {
  constexpr float c0 = 0.69314718055994531f;   // ln2
  constexpr float c1 = 0.24022650695910071f;   // ln2^2 / 2
  constexpr float c2 = 0.055504108664821580f;  // ln2^3 / 6
  const float q = fmaf(arg, fmaf(arg, c2, c1), c0);
  const float series = dtl * q;
  const float direct = fmaf(a, inv_a, -inv_a);  // (a - 1) / A, rounded once
  return fabsf(arg) < 0x1p-5f ? series : direct;
}

// One thread's share of a B or C tile: K consecutive tokens of one state.
// bf16 runs of full blocks stay packed (K/2 words) until they are written to
// LDS as fp32; otherwise the run is held as fp32.
template <typename T, int K, bool kVec, bool kInRange>
struct TileRun {
  static constexpr bool kPacked = kVec && kInRange && sizeof(T) == 2;
  static constexpr int kWords = kPacked ? K / 2 : K;
  uint32_t w[kWords];

  __device__ __forceinline__ void load(const T *__restrict__ row, int64_t t0,
                                       int64_t t, int64_t tend) {
    if constexpr (kPacked && K == 4) {
      const uint2 v = *reinterpret_cast<const uint2 *>(row + t);
      w[0] = v.x;
      w[1] = v.y;
    } else if constexpr (kPacked) {
      static_assert(K % 8 == 0, "packed runs of 4 or a multiple of 8 tokens");
      const uint4 *q = reinterpret_cast<const uint4 *>(row + t);
#pragma unroll
      for (int i = 0; i < K / 8; ++i) {
        const uint4 v = q[i];
        w[4 * i + 0] = v.x;
        w[4 * i + 1] = v.y;
        w[4 * i + 2] = v.z;
        w[4 * i + 3] = v.w;
      }
    } else {
      float v[K];
      load_run<T, K, kVec, kInRange>(row, t0, t, tend, v);
#pragma unroll
      for (int j = 0; j < K; ++j) w[j] = __float_as_uint(v[j]);
    }
  }
  __device__ __forceinline__ float at(int j) const {
    if constexpr (kPacked)
      return (j & 1) ? bf16_hi(w[j / 2]) : bf16_lo(w[j / 2]);
    else
      return __uint_as_float(w[j]);
  }
  // Writes the run as fp32 at tile + off (16-byte aligned).
  __device__ __forceinline__ void store(float *tile, int off) const {
    float4 *dst = reinterpret_cast<float4 *>(tile + off);
#pragma unroll
    for (int j = 0; j < K / 4; ++j)
      dst[j] = make_float4(at(4 * j), at(4 * j + 1), at(4 * j + 2), at(4 * j + 3));
  }
};

// Float offset, inside one LDS tile buffer, of the run that lane `lane` of
// wave `wave` stages: state (wave >> 1) of the phase's pair, matrix B (even
// waves) or C (odd), run `lane`, padded stride KP.
static_assert(kWavesPerGroup == 2 * kPhaseStates, "one staging row per wave");
template <int KP>
__device__ __forceinline__ int staging_offset(int wave, int lane) {
  return (wave * kWaveLanes + lane) * KP;
}

}  // namespace dev
}  // namespace ssm
