// ssm_kernels.hip -- gfx950 (CDNA4) kernels of the selective state-space scan.
//
// The method (Mamba's selective SSM, "S6"): for every (batch, channel) with a
// diagonal A of 16 states, every token t is discretised with its own step
// dt_t = softplus(delta_t + bias) -- dA = exp(dt*A), dB*u = dt*B_t*u_t --,
// the state advances h_t = dA (.) h_{t-1} + dB*u_t, and the output is
// y_t = (C_t . h_t + D*u_t) * silu(z_t).
// Sources: "Mamba & State Space Models - Guide Complet", section 4
// "Implementation du SSM selectif (S6)" and its "Parallel Associative Scan"
// (the operator on affine pairs is associative, so a scan runs in O(log n)
// parallel steps); the johe.ru page "Mamba и State Space Models", sections
// "SSM as RNN", "Selective SSM" and "Hardware-Aware Scan" (block-wise
// processing); the inferownia.pl page, section on the selective scan
// (discretise and recur on chip, fuse the steps, never write the expanded
// (token x state) quantities to HBM).
//
// Work layout of the scan kernel (one workgroup = 4 waves = 16 channels of
// one batch entry; one wave = 4 channel rows of 16 lanes; one lane = 16
// consecutive tokens of its row's channel; a block = 256 tokens):
//   * B and C of the block (16 states x 256 tokens) are read from HBM once per
//     workgroup, widened to fp32 and kept in LDS, shared by its 16 channels;
//   * per lane and state n: dA and dB*u of its 16 tokens stay in registers;
//     the lane folds them into one affine pair (P, H); a 4-step DPP scan over
//     the 16 lanes of the row composes the pairs (the state carried in from
//     the previous block enters lane 0 first); each lane then replays its 16
//     tokens from its true incoming state and accumulates C_t,n * h into y;
//   * the epilogue applies the gate and writes y; the state after the last
//     token goes to h_final.
// All arithmetic is fp32.  No MFMA: the work is a recurrence, not a dense
// contraction.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// DPP controls (GFX9 encoding).
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowRor1 = 0x121;
constexpr int kRowRor2 = 0x122;
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
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

// Loads K consecutive activations row[t .. t+K) as fp32; positions >= tend
// read as 0.  With kVec the run is fetched with 16-byte loads when it is
// wholly in range (the caller guarantees 16-byte alignment of row + t).
template <typename T, int K, bool kVec>
__device__ __forceinline__ void load_run(const T *__restrict__ row, int64_t t,
                                         int64_t tend, float (&v)[K]) {
  if (kVec && t + K <= tend) {
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
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j)
      v[j] = (t + j < tend) ? to_f32<T>(row[t + j]) : 0.0f;
  }
}

// Stores the in-range part (positions < tend) of a K-token run.
template <typename T, int K, bool kVec>
__device__ __forceinline__ void store_run(T *__restrict__ row, int64_t t,
                                          int64_t tend, const float (&v)[K]) {
  if (kVec && t + K <= tend) {
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
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (t + j < tend) row[t + j] = from_f32<T>(v[j]);
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
// Value of lane 15 of the row in lane 0, zero in the other lanes.
__device__ __forceinline__ float row_last_to_first(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x10F,
                                                 0xF, 0xF, true));
}
// x from lane i - s of the row, zero where that lane does not exist.
template <int kCtrl>
__device__ __forceinline__ float row_shift_zero(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl,
                                                 0xF, 0xF, true));
}

struct ScanLane {
  int tid, wave, lane, row, li, ch;
};

// One block of 256 tokens for the 16 channels of the workgroup.  kFull:
// the block lies wholly inside [ct0, ct1) (no masking); otherwise positions
// past ct1 act as identity steps (dt = 0, u = 0) and are not stored.
template <typename T, bool kVec, bool kFull>
__device__ __forceinline__ void scan_block(
    const ScanArgs &p, const ScanLane &L, int64_t t0, int64_t ct1,
    const T *__restrict__ Bb, const T *__restrict__ Cb,
    const T *__restrict__ urow, const T *__restrict__ drow,
    const T *__restrict__ zrow, T *__restrict__ yrow, bool row_ok,
    float bias, float Dd, float *sB, float *sC, const float *sA,
    float (&hlast)[kStates], float &sdt_total) {
  constexpr int K = kTokensPerLane;
  constexpr int KP = K + 4;
  const int64_t tend = kFull ? t0 + kBlockTokens : ct1;
  // B and C of this block: thread (n, q) fetches state n, lane run q.
  float vb[K], vc[K];
  {
    const int n = L.tid >> 4, q = L.tid & 15;
    const int64_t t = t0 + q * K;
    load_run<T, K, kVec>(Bb + n * p.L, t, tend, vb);
    load_run<T, K, kVec>(Cb + n * p.L, t, tend, vc);
  }
  // This lane's tokens: discretisation step, dt*u and the D skip.
  const int64_t tl = t0 + L.li * K;
  float dt[K], du[K], y[K];
  float sdt = 0.0f;
  {
    float uu[K], dr[K];
    load_run<T, K, kVec>(urow, tl, tend, uu);
    load_run<T, K, kVec>(drow, tl, tend, dr);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float x = dr[j] + bias;
      float v = p.softplus ? softplus_f(x) : x;
      if (!kFull) v = (tl + j < tend) ? v : 0.0f;  // identity step
      dt[j] = v;
      du[j] = v * uu[j];
      y[j] = Dd * uu[j];
      sdt += v;
    }
  }

  __syncthreads();  // the previous block's tile is no longer read
  {
    const int n = L.tid >> 4, q = L.tid & 15;
    float4 *pb = reinterpret_cast<float4 *>(&sB[(n * kRowLanes + q) * KP]);
    float4 *pc = reinterpret_cast<float4 *>(&sC[(n * kRowLanes + q) * KP]);
#pragma unroll
    for (int j = 0; j < K / 4; ++j) {
      pb[j] = make_float4(vb[4 * j], vb[4 * j + 1], vb[4 * j + 2], vb[4 * j + 3]);
      pc[j] = make_float4(vc[4 * j], vc[4 * j + 1], vc[4 * j + 2], vc[4 * j + 3]);
    }
  }
  __syncthreads();

#pragma unroll
  for (int n = 0; n < kStates; ++n) {
    const float Aq = sA[L.ch * kStates + n];
    const float *pb = &sB[(n * kRowLanes + L.li) * KP];
    const float *pc = &sC[(n * kRowLanes + L.li) * KP];
    float a[K], bb[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a[j] = fast_exp2(dt[j] * Aq);
      bb[j] = du[j] * pb[j];
    }
    // Fold the lane's tokens into one affine map h -> P*h + H.
    float H = bb[0];
#pragma unroll
    for (int j = 1; j < K; ++j) H = fmaf(a[j], H, bb[j]);
    float P = fast_exp2(sdt * Aq);
    // The carried state (lane 15's, from the previous block) enters lane 0;
    // X is zero in the other lanes.
    const float X = row_last_to_first(hlast[n]);
    H = fmaf(P, X, H);
    // Inclusive scan of the affine maps over the 16 lanes of the row:
    // (P, H) <- (P * P', P * H' + H) with (P', H') from lane i - s.  Where
    // lane i - s does not exist H is unchanged (H' reads 0); P then becomes
    // 0, but a lane whose composition already starts at lane 0 never has
    // its P read again (the carry has entered before the scan).
    H = fmaf(P, row_shift_zero<kRowShr1>(H), H);
    P *= row_shift_zero<kRowShr1>(P);
    H = fmaf(P, row_shift_zero<kRowShr2>(H), H);
    P *= row_shift_zero<kRowShr2>(P);
    H = fmaf(P, row_shift_zero<kRowShr4>(H), H);
    P *= row_shift_zero<kRowShr4>(P);
    H = fmaf(P, row_shift_zero<kRowShr8>(H), H);
    // H is now the true state after this lane's last token; the lane's
    // incoming state is its left neighbour's (lane 0: the carried X).
    float h = row_shift_zero<kRowShr1>(H) + X;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      h = fmaf(a[j], h, bb[j]);
      y[j] = fmaf(pc[j], h, y[j]);
    }
    hlast[n] = h;
  }

  if (zrow) {
    float zz[K];
    load_run<T, K, kVec>(zrow, tl, tend, zz);
#pragma unroll
    for (int j = 0; j < K; ++j) y[j] *= silu_f(zz[j]);
  }
  if (row_ok) store_run<T, K, kVec && kFull>(yrow, tl, tend, y);
  sdt_total += sdt;
}

template <typename T, bool kVec>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void scan_kernel(ScanArgs p) {
  constexpr int K = kTokensPerLane;
  constexpr int KP = K + 4;  // padded LDS stride per lane run (bank spread)
  __shared__ float sB[kStates * kRowLanes * KP];
  __shared__ float sC[kStates * kRowLanes * KP];
  __shared__ float sA[kChannelsPerGroup * kStates];

  ScanLane L;
  L.tid = threadIdx.x;
  L.wave = L.tid >> 6;
  L.lane = L.tid & 63;
  L.row = L.lane >> 4;
  L.li = L.lane & 15;
  L.ch = L.wave * kRowsPerWave + L.row;  // channel slot in the group
  const int64_t b = blockIdx.y;
  const int64_t d0 = static_cast<int64_t>(blockIdx.x) * kChannelsPerGroup;
  const bool row_ok = d0 + L.ch < p.dim;
  const int64_t d = row_ok ? d0 + L.ch : p.dim - 1;  // clamped for reads
  const int chunk = blockIdx.z;
  const int64_t ct0 = static_cast<int64_t>(chunk) * p.chunk_len;
  const int64_t ct1 = ct0 + p.chunk_len < p.L ? ct0 + p.chunk_len : p.L;

  {
    const int c = L.tid >> 4, n = L.tid & 15;
    const int64_t dd = d0 + c < p.dim ? d0 + c : p.dim - 1;
    sA[L.tid] = p.A[dd * kStates + n] * kLog2e;  // 256 threads = 16 x 16
  }
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const int64_t bd = b * p.dim + d;

  // hlast[n]: this lane's state after its last token of the previous block;
  // lane 15 of the row holds the row's true carried state.
  float hlast[kStates];
#pragma unroll
  for (int n = 0; n < kStates; ++n)
    hlast[n] = (chunk == 0 && p.h0) ? p.h0[bd * kStates + n] : 0.0f;

  const T *urow = static_cast<const T *>(p.u) + bd * p.L;
  const T *drow = static_cast<const T *>(p.delta) + bd * p.L;
  const T *zrow = p.z ? static_cast<const T *>(p.z) + bd * p.L : nullptr;
  T *yrow = static_cast<T *>(p.y) + bd * p.L;
  const T *Bb = static_cast<const T *>(p.B) + b * kStates * p.L;
  const T *Cb = static_cast<const T *>(p.C) + b * kStates * p.L;
  float sdt_total = 0.0f;

  int64_t t0 = ct0;
  for (; t0 + kBlockTokens <= ct1; t0 += kBlockTokens)
    scan_block<T, kVec, true>(p, L, t0, ct1, Bb, Cb, urow, drow, zrow, yrow,
                              row_ok, bias, Dd, sB, sC, sA, hlast, sdt_total);
  if (t0 < ct1)
    scan_block<T, kVec, false>(p, L, t0, ct1, Bb, Cb, urow, drow, zrow, yrow,
                               row_ok, bias, Dd, sB, sC, sA, hlast, sdt_total);

  if (!row_ok) return;
  if (p.n_chunks == 1) {
    if (p.h_final && L.li == 15) {
#pragma unroll
      for (int n = 0; n < kStates; ++n) p.h_final[bd * kStates + n] = hlast[n];
    }
  } else {
    float s = sdt_total;  // sum of dt over the chunk, reduced over the row
    s += dpp<kRowRor8>(s, s);
    s += dpp<kRowRor4>(s, s);
    s += dpp<kRowRor2>(s, s);
    s += dpp<kRowRor1>(s, s);
    if (L.li == 15) {
      const int64_t base = bd * p.n_chunks + chunk;
#pragma unroll
      for (int n = 0; n < kStates; ++n) p.ws_H[base * kStates + n] = hlast[n];
      p.ws_S[base] = s;
    }
  }
}

// ------------------------------------------------------ chunk carry -----
// One thread per (batch, channel, state): chains the chunks' end states in
// order, h_in[c+1] = exp(A * sum_dt[c]) * h_in[c] + H[c], and records each
// chunk's incoming state; the last one is the sequence's final state.
__global__ __launch_bounds__(256) void carry_kernel(ScanArgs p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= p.batch * p.dim * kStates) return;
  const int64_t bd = gid >> 4;
  const int n = static_cast<int>(gid & 15);
  const int64_t d = bd % p.dim;
  const float Aq = p.A[d * kStates + n] * kLog2e;
  const int nc = p.n_chunks;
  float h = p.ws_H[(bd * nc) * kStates + n];
  for (int c = 1; c < nc; ++c) {
    p.ws_hin[(bd * nc + c) * kStates + n] = h;
    h = fmaf(fast_exp2(Aq * p.ws_S[bd * nc + c]), h,
             p.ws_H[(bd * nc + c) * kStates + n]);
  }
  if (p.h_final) p.h_final[bd * kStates + n] = h;
}

// --------------------------------------------------- chunk fix-up -------
// For chunk c >= 1 (scanned from a zero state), adds the part of y that its
// true incoming state contributes: y_t += silu(z_t) * sum_n C_t,n *
// exp(A_n * S_t) * h_in,n, S_t = running sum of dt inside the chunk.  One
// wave per (batch, channel, chunk), 64 tokens per step.  Stops once every
// decay factor is below 2^-40 when the factors cannot grow again (all A < 0
// and dt >= 0); otherwise covers the whole chunk.
template <typename T>
__global__ __launch_bounds__(64) void fixup_kernel(ScanArgs p) {
  const int lane = threadIdx.x;
  const int64_t d = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int c = blockIdx.z + 1;
  const int64_t bd = b * p.dim + d;
  const int64_t ct0 = static_cast<int64_t>(c) * p.chunk_len;
  const int64_t ct1 = ct0 + p.chunk_len < p.L ? ct0 + p.chunk_len : p.L;
  float Aq[kStates], hin[kStates];
  float amax = -INFINITY;
#pragma unroll
  for (int n = 0; n < kStates; ++n) {
    Aq[n] = p.A[d * kStates + n] * kLog2e;
    hin[n] = p.ws_hin[(bd * p.n_chunks + c) * kStates + n];
    amax = fmaxf(amax, Aq[n]);
  }
  const bool may_stop = p.softplus && amax < 0.0f;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const T *drow = static_cast<const T *>(p.delta) + bd * p.L;
  const T *zrow = p.z ? static_cast<const T *>(p.z) + bd * p.L : nullptr;
  const T *Cb = static_cast<const T *>(p.C) + b * kStates * p.L;
  T *yrow = static_cast<T *>(p.y) + bd * p.L;
  float S = 0.0f;
  for (int64_t t0 = ct0; t0 < ct1; t0 += 64) {
    const int64_t t = t0 + lane;
    const bool in = t < ct1;
    float dt = 0.0f;
    if (in) {
      const float x = to_f32<T>(drow[t]) + bias;
      dt = p.softplus ? softplus_f(x) : x;
    }
    const float St = S + wave_inclusive_sum(dt);
    float corr = 0.0f;
#pragma unroll
    for (int n = 0; n < kStates; ++n) {
      const float cn = in ? to_f32<T>(Cb[n * p.L + t]) : 0.0f;
      corr = fmaf(cn, fast_exp2(Aq[n] * St) * hin[n], corr);
    }
    if (in) {
      const float g = zrow ? silu_f(to_f32<T>(zrow[t])) : 1.0f;
      yrow[t] = from_f32<T>(fmaf(g, corr, to_f32<T>(yrow[t])));
    }
    S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(St), 63));
    if (may_stop && fast_exp2(amax * S) <= 0x1p-40f) break;
  }
}

// ------------------------------------------------------ decode step -----
// Four lanes per (batch, channel), four states each: the fp32 state is read
// and written with 16-byte accesses, fully coalesced; the 4-lane readout is
// a two-step DPP reduction inside each quad.
template <typename T, bool kVec>
__global__ __launch_bounds__(256) void step_kernel(StepArgs p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t nch = p.batch * p.dim;
  const int64_t ch_raw = gid >> 2;
  const bool ok = ch_raw < nch;
  const int64_t ch = ok ? ch_raw : nch - 1;
  const int q = static_cast<int>(gid & 3);
  const int64_t b = ch / p.dim;
  const int64_t d = ch - b * p.dim;

  const float x = to_f32<T>(static_cast<const T *>(p.x)[ch]);
  const float xr = to_f32<T>(static_cast<const T *>(p.delta)[ch]) +
                   (p.bias ? p.bias[d] : 0.0f);
  const float dt = p.softplus ? softplus_f(xr) : xr;
  const float dx = dt * x;

  float h[4], a4[4], b4[4], c4[4];
  float *st = p.state + ch * kStates + 4 * q;
  const float *Ap = p.A + d * kStates + 4 * q;
  const T *Bp = static_cast<const T *>(p.B) + b * kStates + 4 * q;
  const T *Cp = static_cast<const T *>(p.C) + b * kStates + 4 * q;
  if (kVec) {
    const float4 s4 = *reinterpret_cast<const float4 *>(st);
    const float4 av = *reinterpret_cast<const float4 *>(Ap);
    h[0] = s4.x; h[1] = s4.y; h[2] = s4.z; h[3] = s4.w;
    a4[0] = av.x; a4[1] = av.y; a4[2] = av.z; a4[3] = av.w;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) { h[i] = st[i]; a4[i] = Ap[i]; }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b4[i] = to_f32<T>(Bp[i]);
    c4[i] = to_f32<T>(Cp[i]);
  }
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = fmaf(fast_exp2(dt * a4[i] * kLog2e), h[i], dx * b4[i]);
    part = fmaf(c4[i], h[i], part);
  }
  part += dpp<kQuadXor1>(part, part);
  part += dpp<kQuadXor2>(part, part);
  if (!ok) return;
  if (kVec) {
    *reinterpret_cast<float4 *>(st) = make_float4(h[0], h[1], h[2], h[3]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) st[i] = h[i];
  }
  if (q == 0) {
    float yv = part + (p.D ? p.D[d] * x : 0.0f);
    if (p.z) yv *= silu_f(to_f32<T>(static_cast<const T *>(p.z)[ch]));
    static_cast<T *>(p.y)[ch] = from_f32<T>(yv);
  }
}

template <typename T, bool kVec>
hipError_t launch_scan_t(const ScanArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.dim + kChannelsPerGroup - 1) /
                                        kChannelsPerGroup),
                  static_cast<unsigned>(a.batch),
                  static_cast<unsigned>(a.n_chunks));
  hipLaunchKernelGGL((scan_kernel<T, kVec>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks == 1) return e;
  const int64_t nthreads = a.batch * a.dim * kStates;
  hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>((nthreads + 255) / 256)),
                     dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fgrid(static_cast<unsigned>(a.dim), static_cast<unsigned>(a.batch),
                   static_cast<unsigned>(a.n_chunks - 1));
  hipLaunchKernelGGL((fixup_kernel<T>), fgrid, dim3(64), 0, s, a);
  return hipGetLastError();
}

template <typename T, bool kVec>
hipError_t launch_step_t(const StepArgs &a, hipStream_t s) {
  const int64_t nthreads = a.batch * a.dim * 4;
  hipLaunchKernelGGL((step_kernel<T, kVec>),
                     dim3(static_cast<unsigned>((nthreads + 255) / 256)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int launch_scan(const ScanArgs &a, bool bf16, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch_scan_t<uint16_t, true>(a, s) : launch_scan_t<uint16_t, false>(a, s);
  return vec ? launch_scan_t<float, true>(a, s) : launch_scan_t<float, false>(a, s);
}

int launch_step(const StepArgs &a, bool bf16, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch_step_t<uint16_t, true>(a, s) : launch_step_t<uint16_t, false>(a, s);
  return vec ? launch_step_t<float, true>(a, s) : launch_step_t<float, false>(a, s);
}

const char *hip_error_string(int err) {
  return hipGetErrorString(static_cast<hipError_t>(err));
}

}  // namespace ssm
