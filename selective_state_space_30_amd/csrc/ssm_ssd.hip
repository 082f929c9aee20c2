// ssm_ssd.hip -- gfx950 (CDNA4) kernels of the Mamba-2 "SSD" (state space
// dual) forward: one scalar decay per head, d_state 64-256, bf16
// activations, fp32 accumulation on the matrix cores.
//
// "Mamba & State Space Models - Guide Complet", section 5: the SSM as a
// product with a structured matrix, y = (L o S) u, L the causal mask and S
// semiseparable.  With one scalar decay A per head the masked matrix of a
// chunk of T tokens factors into small dense products; between chunks a
// P x N state carries the past (the recurrent form):
//   cum_t   = sum_{r <= t in the chunk} dt_r,  dt = softplus(dt_raw + bias)
//   G       = C^T B                     (T x T, shared by a group's heads)
//   M[t,s]  = G[t,s] exp(A (cum_t - cum_s)) dt_s   for s <= t, else 0
//   y       = exp(A cum_t) (S C)[:, t] + (X M^T)[:, t] + D x,  then silu(z)
//   S      <- exp(A cum_T) S + (X diag(exp(A (cum_T - cum_s)) dt_s)) B^T
// All four products run on v_mfma_f32_16x16x32_bf16 (A operand: lane l,
// element e = A[l%16][8*(l/16)+e]; B: B[8*(l/16)+e][l%16]; result: lane l,
// element e = D[4*(l/16)+e][l%16], checked on the hardware).
//
// Work layout: ssd_prep_kernel forms G and C^T per (batch, group, chunk);
// ssd_kernel runs one workgroup per (batch, head) over the chunks in order,
// its 4 waves owning 16 head rows each; a wave's share of the state S (16 x
// N fp32) stays in matrix-core accumulators for the whole sequence.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int T = kSsdChunk;     // 64 tokens per chunk
constexpr int P = kSsdHeadDim;   // 64 rows per head
constexpr int kPad = 8;          // bf16 padding of LDS rows
constexpr int kRowT = T + kPad;  // row stride of [row][token] tiles

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const __bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// Loads 8 consecutive bf16 of a row (positions t .. t+7; those >= tend read
// as 0) and writes them to LDS.  kVec: the 8 lie in range and are 16-byte
// aligned.
template <bool kVec>
__device__ __forceinline__ void stage8(__bf16 *dst, const uint16_t *row, int64_t t,
                                       int64_t tend) {
  if (kVec && t + 8 <= tend) {
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(row + t);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dst[i] = __builtin_bit_cast(__bf16, t + i < tend ? row[t + i] : uint16_t(0));
  }
}

// 8 consecutive bf16 of a row (positions t .. t+7, those >= tend as 0) as
// one 16-byte word; kVec: 16-byte load when all 8 are in range.
template <bool kVec>
__device__ __forceinline__ uint4 load8(const uint16_t *row, int64_t t, int64_t tend) {
  if (kVec && t + 8 <= tend) return *reinterpret_cast<const uint4 *>(row + t);
  uint16_t v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = t + i < tend ? row[t + i] : uint16_t(0);
  return make_uint4(v[0] | (uint32_t(v[1]) << 16), v[2] | (uint32_t(v[3]) << 16),
                    v[4] | (uint32_t(v[5]) << 16), v[6] | (uint32_t(v[7]) << 16));
}

// ----------------------------------------------------------- chunk prep ---
// Per (batch, group, chunk): G = C^T B (64 x 64 fp32) and C transposed to
// [token][state] (the layout the y product reads).  Positions past L are 0.
template <int N, bool kVec>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdArgs p) {
  constexpr int kRowN = N + kPad;
  __shared__ __bf16 CtL[T * kRowN];  // [t][n]
  __shared__ __bf16 BtL[T * kRowN];  // [s][n]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int64_t t0 = c * T;
  const int64_t bg = b * p.ngroups + g;
  const uint16_t *Cg = static_cast<const uint16_t *>(p.C) + bg * N * p.L;
  const uint16_t *Bg = static_cast<const uint16_t *>(p.B) + bg * N * p.L;

  // transpose into LDS: thread -> (state n, 8 tokens)
  for (int q = tid; q < N * (T / 8); q += 256) {
    const int n = q / (T / 8), t8 = (q % (T / 8)) * 8;
    __bf16 cv[8], bv[8];
    stage8<kVec>(cv, Cg + n * p.L, t0 + t8, p.L);
    stage8<kVec>(bv, Bg + n * p.L, t0 + t8, p.L);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      CtL[(t8 + i) * kRowN + n] = cv[i];
      BtL[(t8 + i) * kRowN + n] = bv[i];
    }
  }
  __syncthreads();

  // G rows 16*wave .. +16 (t), all 64 columns (s); K = N
  float *Gc = p.G + (bg * p.nchunks + c) * T * T;
#pragma unroll
  for (int sj = 0; sj < T / 16; ++sj) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) {
      const bf16x8 a = lds8(&CtL[(16 * wave + (lane & 15)) * kRowN + 32 * ks + 8 * (lane >> 4)]);
      const bf16x8 bb = lds8(&BtL[(16 * sj + (lane & 15)) * kRowN + 32 * ks + 8 * (lane >> 4)]);
      acc = mfma(a, bb, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Gc[(16 * wave + 4 * (lane >> 4) + e) * T + 16 * sj + (lane & 15)] = acc[e];
  }
  // C^T of this chunk, [t][n] contiguous
  uint16_t *Ctw = static_cast<uint16_t *>(p.Ct) + (bg * p.nchunks + c) * T * N;
  for (int q = tid; q < T * (N / 8); q += 256) {
    const int t = q / (N / 8), n8 = (q % (N / 8)) * 8;
    *reinterpret_cast<uint4 *>(Ctw + t * N + n8) =
        *reinterpret_cast<const uint4 *>(&CtL[t * kRowN + n8]);
  }
}

// ------------------------------------------------------------- the scan ---
template <int N, bool kVec>
__global__ __launch_bounds__(256) void ssd_kernel(SsdArgs p) {
  constexpr int kRowN = N + kPad;
  constexpr int kNT = N / 16;  // state tiles per wave
  __shared__ __bf16 Xs[P * kRowT];   // [p][t]
  __shared__ __bf16 Zs[P * kRowT];   // [p][t]: z, then y
  __shared__ __bf16 Bs[N * kRowT];   // [n][t]
  __shared__ __bf16 Cs[T * kRowN];   // [t][n]
  __shared__ __bf16 Ms[T * kRowT];   // [t][s]
  __shared__ __bf16 Ss[P * kRowN];   // [p][n]: the state entering the chunk
  __shared__ float cums[T], dts[T], ets[T], wts[T];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t h = blockIdx.x, b = blockIdx.y;
  const int64_t g = h / (p.nheads / p.ngroups);
  const int64_t bh = b * p.nheads + h;
  const int64_t bg = b * p.ngroups + g;
  const float Aq = p.A[h] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const float Dh = p.D ? p.D[h] : 0.0f;
  const uint16_t *xh = static_cast<const uint16_t *>(p.x) + bh * P * p.L;
  const uint16_t *zh = p.z ? static_cast<const uint16_t *>(p.z) + bh * P * p.L : nullptr;
  const uint16_t *dth = static_cast<const uint16_t *>(p.dt) + bh * p.L;
  const uint16_t *Bg = static_cast<const uint16_t *>(p.B) + bg * N * p.L;
  uint16_t *yh = static_cast<uint16_t *>(p.y) + bh * P * p.L;

  // this wave's rows of the state, in accumulator layout: S[k][e] =
  // S[row 16*wave + 4*(lane/16) + e][state 16*k + lane%16]
  f32x4 S[kNT];
  const int prow = 16 * wave + 4 * (lane >> 4);
#pragma unroll
  for (int k = 0; k < kNT; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      S[k][e] = p.h0 ? p.h0[(bh * P + prow + e) * N + 16 * k + (lane & 15)] : 0.0f;

  // One thread's share of a chunk's inputs, loaded a chunk ahead into
  // registers (x, z: 2 x 8 tokens of a row; B: N/32 x 8 tokens of a state;
  // C^T: N/32 x 8 states of a token; G: 16 entries of row tid/4; dt: one
  // token, wave 0) and written to LDS once the previous chunk is done.
  constexpr int kXQ = P * (T / 8) / 256;   // 2
  constexpr int kBQ = N * (T / 8) / 256;   // N/32
  uint4 rx[kXQ], rz[kXQ], rb[kBQ], rc[kBQ];
  float4 rg[4];
  uint16_t rdt = 0;
  const int gt = tid >> 2, gs0 = (tid & 3) * 16;  // this thread's G entries
  auto fetch = [&](int c) {
    const int64_t t0 = static_cast<int64_t>(c) * T;
#pragma unroll
    for (int i = 0; i < kXQ; ++i) {
      const int q = tid + 256 * i, r = q / (T / 8), t8 = (q % (T / 8)) * 8;
      rx[i] = load8<kVec>(xh + r * p.L, t0 + t8, p.L);
      if (zh) rz[i] = load8<kVec>(zh + r * p.L, t0 + t8, p.L);
    }
#pragma unroll
    for (int i = 0; i < kBQ; ++i) {
      const int q = tid + 256 * i, n = q / (T / 8), t8 = (q % (T / 8)) * 8;
      rb[i] = load8<kVec>(Bg + n * p.L, t0 + t8, p.L);
    }
    const uint16_t *Cw = static_cast<const uint16_t *>(p.Ct) + (bg * p.nchunks + c) * T * N;
#pragma unroll
    for (int i = 0; i < kBQ; ++i) {
      const int q = tid + 256 * i, t = q / (N / 8), n8 = (q % (N / 8)) * 8;
      rc[i] = *reinterpret_cast<const uint4 *>(Cw + t * N + n8);
    }
    const float4 *Gr = reinterpret_cast<const float4 *>(
        p.G + ((bg * p.nchunks + c) * T + gt) * T + gs0);
#pragma unroll
    for (int i = 0; i < 4; ++i) rg[i] = Gr[i];
    if (wave == 0) rdt = t0 + lane < p.L ? dth[t0 + lane] : uint16_t(0);
  };
  auto deposit = [&]() {
#pragma unroll
    for (int i = 0; i < kXQ; ++i) {
      const int q = tid + 256 * i, r = q / (T / 8), t8 = (q % (T / 8)) * 8;
      *reinterpret_cast<uint4 *>(&Xs[r * kRowT + t8]) = rx[i];
      if (zh) *reinterpret_cast<uint4 *>(&Zs[r * kRowT + t8]) = rz[i];
    }
#pragma unroll
    for (int i = 0; i < kBQ; ++i) {
      const int q = tid + 256 * i, n = q / (T / 8), t8 = (q % (T / 8)) * 8;
      *reinterpret_cast<uint4 *>(&Bs[n * kRowT + t8]) = rb[i];
    }
#pragma unroll
    for (int i = 0; i < kBQ; ++i) {
      const int q = tid + 256 * i, t = q / (N / 8), n8 = (q % (N / 8)) * 8;
      *reinterpret_cast<uint4 *>(&Cs[t * kRowN + n8]) = rc[i];
    }
  };
  fetch(0);
  deposit();
  float gcur[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gcur[4 * i] = rg[i].x; gcur[4 * i + 1] = rg[i].y;
    gcur[4 * i + 2] = rg[i].z; gcur[4 * i + 3] = rg[i].w;
  }
  uint16_t dtcur = rdt;

#pragma unroll 1
  for (int c = 0; c < p.nchunks; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * T;
    // 1. steps, running sums and weights of the chunk (wave 0)
    if (wave == 0) {
      float v = 0.0f;
      if (t0 + lane < p.L) {
        const float raw = __uint_as_float(static_cast<uint32_t>(dtcur) << 16) + bias;
        v = p.softplus ? softplus_f(raw) : raw;
      }
      float cum = wave_inclusive_sum(v);
      float cend = lane_broadcast(cum, kWaveLanes - 1);
      asm volatile("" : "+s"(cend));  // formed by the whole wave first
      dts[lane] = v;
      cums[lane] = cum;
      ets[lane] = fast_exp2(Aq * cum);               // decay of the incoming state
      wts[lane] = fast_exp2(Aq * (cend - cum)) * v;  // weight of token s in the new state
    }
    // 2. the state entering the chunk, as bf16 rows [p][n]
#pragma unroll
    for (int k = 0; k < kNT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        Ss[(prow + e) * kRowN + 16 * k + (lane & 15)] = static_cast<__bf16>(S[k][e]);
    __syncthreads();
    if (c + 1 < p.nchunks) fetch(c + 1);  // in flight during this chunk's work

    // 3. M = G o decay mask o dt_s, bf16 [t][s]; thread -> row gt, 16 columns
    {
      const float ct = cums[gt];
      __bf16 mv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int sidx = gs0 + i;
        const float m = gcur[i] * fast_exp2(Aq * (ct - cums[sidx])) * dts[sidx];
        mv[i] = static_cast<__bf16>(sidx <= gt ? m : 0.0f);
      }
      *reinterpret_cast<bf16x8 *>(&Ms[gt * kRowT + gs0]) =
          bf16x8{mv[0], mv[1], mv[2], mv[3], mv[4], mv[5], mv[6], mv[7]};
      *reinterpret_cast<bf16x8 *>(&Ms[gt * kRowT + gs0 + 8]) =
          bf16x8{mv[8], mv[9], mv[10], mv[11], mv[12], mv[13], mv[14], mv[15]};
    }
    __syncthreads();
    // 4. y tiles of this wave's 16 rows: the incoming state's share
    //    exp(A cum_t) (S C)[p, t], then the chunk's own X M^T
    const int arow = 16 * wave + (lane & 15);  // A-operand row
    const int kq = 8 * (lane >> 4);            // A/B-operand k offset
    f32x4 acc[T / 16];
#pragma unroll
    for (int tj = 0; tj < T / 16; ++tj) {
      f32x4 a4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < N / 32; ++ks)
        a4 = mfma(lds8(&Ss[arow * kRowN + 32 * ks + kq]),
                  lds8(&Cs[(16 * tj + (lane & 15)) * kRowN + 32 * ks + kq]), a4);
      const float et = ets[16 * tj + (lane & 15)];
#pragma unroll
      for (int e = 0; e < 4; ++e) a4[e] *= et;
#pragma unroll
      for (int ks = 0; ks < T / 32; ++ks)
        a4 = mfma(lds8(&Xs[arow * kRowT + 32 * ks + kq]),
                  lds8(&Ms[(16 * tj + (lane & 15)) * kRowT + 32 * ks + kq]), a4);
      acc[tj] = a4;
    }

    // 5. the state after the chunk: exp(A cum_T) S + (X w) B^T
    {
      const float dend = fast_exp2(Aq * cums[T - 1]);
#pragma unroll
      for (int k = 0; k < kNT; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[k][e] *= dend;
#pragma unroll
      for (int ks = 0; ks < T / 32; ++ks) {
        const bf16x8 xa = lds8(&Xs[arow * kRowT + 32 * ks + kq]);
        bf16x8 xw;
#pragma unroll
        for (int i = 0; i < 8; ++i)
          xw[i] = static_cast<__bf16>(static_cast<float>(xa[i]) * wts[32 * ks + kq + i]);
#pragma unroll
        for (int k = 0; k < kNT; ++k)
          S[k] = mfma(xw, lds8(&Bs[(16 * k + (lane & 15)) * kRowT + 32 * ks + kq]), S[k]);
      }
    }

    // 6. skip and gate; y of this lane's elements goes into Zs (each element
    //    has one owner), then a coalesced store
#pragma unroll
    for (int tj = 0; tj < T / 16; ++tj) {
      const int t = 16 * tj + (lane & 15);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = prow + e;
        float yv = acc[tj][e] + Dh * static_cast<float>(Xs[r * kRowT + t]);
        if (zh) yv *= silu_f(static_cast<float>(Zs[r * kRowT + t]));
        Zs[r * kRowT + t] = static_cast<__bf16>(yv);
      }
    }
    __syncthreads();
    for (int q = tid; q < P * (T / 8); q += 256) {
      const int r = q / (T / 8), t8 = (q % (T / 8)) * 8;
      const int64_t t = t0 + t8;
      if (kVec && t + 8 <= p.L) {
        *reinterpret_cast<uint4 *>(yh + r * p.L + t) =
            *reinterpret_cast<const uint4 *>(&Zs[r * kRowT + t8]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (t + i < p.L)
            yh[r * p.L + t + i] = __builtin_bit_cast(uint16_t, Zs[r * kRowT + t8 + i]);
      }
    }
    __syncthreads();  // the chunk's tiles are free for the next one
    if (c + 1 < p.nchunks) {
      deposit();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gcur[4 * i] = rg[i].x; gcur[4 * i + 1] = rg[i].y;
        gcur[4 * i + 2] = rg[i].z; gcur[4 * i + 3] = rg[i].w;
      }
      dtcur = rdt;
    }
  }

  if (p.h_final) {
#pragma unroll
    for (int k = 0; k < kNT; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        p.h_final[(bh * P + prow + e) * N + 16 * k + (lane & 15)] = S[k][e];
  }
}

template <int N, bool kVec>
hipError_t launch_ssd_t(const SsdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((ssd_prep_kernel<N, kVec>),
                     dim3(static_cast<unsigned>(a.nchunks), static_cast<unsigned>(a.ngroups),
                          static_cast<unsigned>(a.batch)),
                     dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_kernel<N, kVec>),
                     dim3(static_cast<unsigned>(a.nheads), static_cast<unsigned>(a.batch)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int launch_ssd(const SsdArgs &a, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.dstate) {
    case 64:
      return vec ? launch_ssd_t<64, true>(a, s) : launch_ssd_t<64, false>(a, s);
    case 128:
      return vec ? launch_ssd_t<128, true>(a, s) : launch_ssd_t<128, false>(a, s);
    case 256:
      return vec ? launch_ssd_t<256, true>(a, s) : launch_ssd_t<256, false>(a, s);
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace ssm
