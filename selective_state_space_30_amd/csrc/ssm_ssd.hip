// ssm_ssd.hip -- gfx950 (CDNA4) kernels of the Mamba-2 "SSD" (state space
// dual) forward: one scalar decay per head, d_state 64-256, bf16
// activations, fp32 accumulation on the matrix cores.
//
// "Mamba & State Space Models - Guide Complet", section 5: the SSM as a
// product with a structured matrix, y = (L o S) u, L the causal mask and S
// semiseparable.  With one scalar decay A per head the masked matrix of a
// chunk of T tokens factors into small dense products; between chunks a
// P x N state carries the past (the recurrent form).  With a_t = A cum_t,
// cum_t = sum_{r <= t in the chunk} dt_r and dt = softplus(dt_raw + bias):
//   G       = C^T B, causal (G[t,s] = 0 for s > t; shared by a group's heads)
//   y_t     = exp(a_t) (C^T S^T)[t] + sum_{s<=t} G[t,s] exp(a_t - a_s) dt_s x_s
//             + D x_t,  then times silu(z_t)
//   S      <- exp(a_T) S + (X diag(exp(a_T - a_s) dt_s)) B^T
// The decay inside the chunk splits at a reference token m:
// exp(a_t - a_s) = u_t v_s / dt_s with u_t = exp(a_t - a_m) and v_s =
// exp(a_m - a_s) dt_s, so the chunk's own term is u_t (G (X diag v)^T)[t]: a
// plain product with the group's G.  While every |a_t - a_m| stays below
// kFactorLimit (base 2) the factors cannot overflow fp32 or bf16; a chunk
// with a steeper decay forms M = G o exp(a_t - a_s) dt_s element by element.
// The carried state and G's columns scaled by v_s (or M) enter the
// products as a pair of bf16 values (the value and its rounding error), so
// that none of them is rounded to bf16 alone; x is taken as it is stored,
// and G itself is kept in fp32.
// All products run on v_mfma_f32_16x16x32_bf16 (A operand: lane l, element
// e = A[l%16][8*(l/16)+e]; B: B[8*(l/16)+e][l%16]; result: lane l, element
// e = D[4*(l/16)+e][l%16], checked on the hardware).
//
// Work layout: ssd_prep_kernel forms the causal G (fp32) and C^T per
// (batch, group, chunk); ssd_kernel runs one workgroup per (batch, head,
// slice of the head's rows) over the chunks in order, the state staying in
// matrix-core accumulators for the whole sequence.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using namespace dev;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int T = kSsdChunk;     // 64 tokens per chunk
constexpr int P = kSsdHeadDim;   // 64 rows per head
constexpr int kPad = 8;          // bf16 padding of LDS rows
constexpr int kRowT = T + kPad;  // row stride of [row][token] tiles
constexpr int kRowG = T + 4;     // row stride of the prep kernel's fp32 G tile
// largest |a_t - a_m| (base-2 exponent) of the factored chunk term
constexpr float kFactorLimit = 96.0f;
constexpr int kRef = 31;         // reference token m of the factored decay

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

// 8 consecutive bf16 of a row of length tend, positions t .. t+7, as one
// 16-byte word, read unconditionally: positions past the row read some
// element of the row instead (callers give them zero weight), so the load
// has one path and no select on its result.  kVec: 16-byte aligned rows and
// tend % 8 == 0, so a group of 8 is wholly in or wholly past the row.
template <bool kVec>
__device__ __forceinline__ u32x4 load8_clamped(const uint16_t *row, int64_t t, int64_t tend) {
  if (kVec) return *reinterpret_cast<const u32x4 *>(row + (t + 8 <= tend ? t : tend - 8));
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = row[t + 2 * i < tend ? t + 2 * i : tend - 1];
    const uint32_t hi = row[t + 2 * i + 1 < tend ? t + 2 * i + 1 : tend - 1];
    w[i] = lo | (hi << 16);
  }
  return w;
}

// Byte view of n consecutive bf16 elements from `base` (wave-uniform) for
// buffer loads: reads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bf16_view(const uint16_t *base, int64_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), 0,
                                           static_cast<int>(n * 2), kBufferWord3);
}

// 16 bytes at byte offset voff + soff of a view (voff per lane, soff
// wave-uniform).
__device__ __forceinline__ u32x4 buf_load8(__amdgpu_buffer_rsrc_t v, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(v, voff, soff, 0));
}

// ----------------------------------------------------------- chunk prep ---
// Per (batch, group, chunk): the causal G = C^T B (64 x 64, [t][s], zero
// for s > t) in fp32, and C transposed to
// [token][state] (the layout the y product reads).  Positions past L are 0.
template <int N, bool kVec>
__global__ __launch_bounds__(256) void ssd_prep_kernel(SsdArgs p) {
  constexpr int kRowN = N + kPad;
  __shared__ __align__(16) __bf16 CtL[T * kRowN];  // [t][n]
  __shared__ __align__(16) __bf16 BtL[T * kRowN];  // [s][n]
  __shared__ __align__(16) float GL[T * kRowG];      // [t][s]
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
#pragma unroll
  for (int sj = 0; sj < T / 16; ++sj) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) {
      const bf16x8 a = lds8(&CtL[(16 * wave + (lane & 15)) * kRowN + 32 * ks + 8 * (lane >> 4)]);
      const bf16x8 bb = lds8(&BtL[(16 * sj + (lane & 15)) * kRowN + 32 * ks + 8 * (lane >> 4)]);
      acc = mfma(a, bb, acc);
    }
    const int s = 16 * sj + (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * wave + 4 * (lane >> 4) + e;
      GL[t * kRowG + s] = s <= t ? acc[e] : 0.0f;
    }
  }
  __syncthreads();
  float *Gw = static_cast<float *>(p.G) + (bg * p.nchunks + c) * T * T;
  for (int q = tid; q < T * (T / 4); q += 256) {
    const int t = q / (T / 4), s4 = (q % (T / 4)) * 4;
    *reinterpret_cast<f32x4 *>(Gw + t * T + s4) = *reinterpret_cast<const f32x4 *>(&GL[t * kRowG + s4]);
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
// One workgroup = one (batch, head) and R = 16*RP of the head's 64 rows (the
// rows of the state are independent; splitting them across workgroups buys
// parallelism at the price of re-reading the group's B, C^T and G).  kW = 4
// or 8 waves: wave w takes token tile tt = w % 4 and row group w / 4 (the
// row tiles split over kW/4 groups); per chunk it computes the y tiles of
// tokens 16 tt .. 16 tt + 15 of its row tiles and owns their state tiles of
// states [tt N/4, (tt+1) N/4).  The products are set up transposed (token
// or state as the matrix-core row index) so that a lane holds 4 consecutive
// tokens or states of one row.
//
// Each wave reads its own rows of C^T and G (the y products) and of B (the
// state update), so those go from memory straight into operand registers;
// the next chunk's are requested right after the last use.  LDS holds what
// the waves share, double-buffered by chunk parity: x and x w, z then
// y, the state entering the chunk (a bf16 pair); and the step quantities of
// three chunks (chunk c+2's are formed during chunk c by wave (c+2) mod 4).
//
// One barrier per chunk c: before it, the state entering c into LDS; after
// it, the y stores of chunk c-1, the step quantities of chunk c+2 (one
// wave), the x, z deposit of chunk c+1, then chunk c's products, new state
// and y (into LDS).  A buffer
// of parity c is written again only in iteration c+1 (deposit of c+2) or
// c+2 (state), after every wave has passed the barrier that ends its reads.
template <int N, bool kVec, int RP, int kW>
__global__ __launch_bounds__(64 * kW) void ssd_kernel(SsdArgs p) {
  constexpr int R = 16 * RP;          // rows of the head in this workgroup
  constexpr int kNTW = N / 64;        // state tiles per wave (per row tile)
  constexpr int kThreads = 64 * kW;
  constexpr int RPW = RP / (kW / 4);  // row tiles per wave
  static_assert((kW == 4 || kW == 8) && RPW >= 1 && RP % (kW / 4) == 0, "wave layout");
  // Tiles are unpadded; the 16-byte groups of a row are permuted by the row
  // (group g of row r at g ^ (r % 8)) so that 8 rows read at one group hit
  // 8 different bank sets.
  __shared__ __align__(16) __bf16 Xs[2][R * T];         // [p][t]: x_t
  __shared__ __align__(16) __bf16 XWs[2][2][R * T];     // [p][t]: x_t w_t, hi, lo
  __shared__ __align__(16) __bf16 Zs[2][R * T];         // [p][t]: z, then y
  __shared__ __align__(16) __bf16 Ss[2][2][R * N];      // [p][n]: entering state, hi, lo
  // dt, cum, exp(a_t), u_t, v_t, w_t of a chunk and whether its decay may
  // be factored; formed two chunks ahead by one wave (in turn), so three
  // sets are live
  __shared__ __align__(16) float Wq[3][6][T];
  __shared__ int Wf[3];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  const int tt = wave & 3;                       // token tile and state slice
  const int pr = 16 * (wave >> 2) * RPW;         // first row (in the workgroup) of this wave
  constexpr int kSplit = P / R;
  const int64_t h = blockIdx.x / kSplit, b = blockIdx.y;
  const int row0 = (blockIdx.x % kSplit) * R;
  const int64_t g = h / (p.nheads / p.ngroups);
  const int64_t bh = b * p.nheads + h;
  const int64_t bg = b * p.ngroups + g;
  const float Aq = p.A[h] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
  const float Dh = p.D ? p.D[h] : 0.0f;
  const int64_t L = p.L;
  const int nch = p.nchunks;
  const uint16_t *xh = static_cast<const uint16_t *>(p.x) + (bh * P + row0) * L;
  const uint16_t *zh = p.z ? static_cast<const uint16_t *>(p.z) + (bh * P + row0) * L : nullptr;
  const uint16_t *dth = static_cast<const uint16_t *>(p.dt) + bh * L;
  const uint16_t *Bg = static_cast<const uint16_t *>(p.B) + bg * N * L;
  const uint16_t *Ctg = static_cast<const uint16_t *>(p.Ct) + bg * nch * T * N;
  const float *Gg = static_cast<const float *>(p.G) + bg * nch * T * T;
  uint16_t *yh = static_cast<uint16_t *>(p.y) + (bh * P + row0) * L;
  const int kq = 8 * lq;                         // operand k offset of this lane
  const int ta = 16 * tt + li;                   // token row of this lane's A operands
  const int tq = 16 * tt + 4 * lq;               // first token of this lane's outputs
  // element (row r, column j) of a [row][T] or [row][N] tile, j in a
  // 16-byte group (8 elements) that is permuted by the row
  auto at = [](int r, int j) { return r * T + ((((j >> 3) ^ r) & 7) | (j >> 3 & ~7)) * 8 + (j & 7); };
  auto an = [](int r, int j) { return r * N + ((((j >> 3) ^ r) & 7) | (j >> 3 & ~7)) * 8 + (j & 7); };

  // State tiles in accumulator layout, transposed: S[pt][k][e] is the state
  // of row pr + 16*pt + li, state n = 16*(kNTW*tt + k) + 4*lq + e.
  f32x4 S[RPW][kNTW];
#pragma unroll
  for (int pt = 0; pt < RPW; ++pt)
#pragma unroll
    for (int k = 0; k < kNTW; ++k) {
      const int n = 16 * (kNTW * tt + k) + 4 * lq;
      if (p.h0) {  // 4-byte aligned rows: copied, not cast
        __builtin_memcpy(&S[pt][k], p.h0 + (bh * P + row0 + pr + 16 * pt + li) * N + n, 16);
      } else {
        S[pt][k] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }

  // operand registers of the chunk being computed: C^T row ta (states
  // 32 ks + kq ..), G row ta (tokens 32 ks + kq .., fp32), B rows of
  // this wave's state tiles (tokens 32 ks + kq ..)
  bf16x8 ca[N / 32], ba[2][kNTW];
  f32x4 ga[2][2];  // [ks][half]
  // (a chunk's C^T and G are small: a wave-uniform base and a 32-bit lane
  // offset address them)
  const int ct_off = ta * N + kq, g_off = ta * T + kq;
  auto load_ct = [&](int c) __attribute__((always_inline)) {
    const uint16_t *base = Ctg + static_cast<int64_t>(c) * T * N;
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
      ca[ks] = __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const u32x4 *>(base + (ct_off + 32 * ks)));
  };
  auto load_g = [&](int c) __attribute__((always_inline)) {
    const float *base = Gg + static_cast<int64_t>(c) * T * T;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        ga[ks][hf] = *reinterpret_cast<const f32x4 *>(base + (g_off + 32 * ks + 4 * hf));
  };
  // Aligned rows (kVec) are read through buffer views of whole matrices: a
  // loop-invariant 32-bit lane offset, the chunk's start as the scalar
  // offset, no address arithmetic per chunk; an 8-token piece never
  // straddles a row end, and pieces past L read the next row (weight 0: dt
  // = 0 there) or, past the view, 0.  Unaligned rows clamp per element.
  const __amdgpu_buffer_rsrc_t vB = bf16_view(Bg, N * L);
  int bo[2][kNTW];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int k = 0; k < kNTW; ++k)
      bo[ks][k] = static_cast<int>(((16 * (kNTW * tt + k) + li) * L + 32 * ks + kq) * 2);
  auto load_b = [&](int c) __attribute__((always_inline)) {
    const int64_t t0 = static_cast<int64_t>(c) * T;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int k = 0; k < kNTW; ++k)
        ba[ks][k] = __builtin_bit_cast(
            bf16x8, kVec ? buf_load8(vB, bo[ks][k], static_cast<int>(t0 * 2))
                         : load8_clamped<kVec>(Bg + (16 * (kNTW * tt + k) + li) * L,
                                               t0 + 32 * ks + kq, L));
  };
  // x and z as 16-byte pieces of rows (for LDS; with fewer pieces than
  // threads the upper threads repeat the lower ones' loads), dt one token a
  // lane.  Every load is unconditional (z repeats x when there is no gate),
  // so no register ever waits on a load just to be merged with another path.
  constexpr int kXP = R * (T / 8);
  constexpr int kXQ = (kXP + kThreads - 1) / kThreads;
  const uint16_t *zsrc = zh ? zh : xh;
  const __amdgpu_buffer_rsrc_t vX = bf16_view(xh, R * L), vZ = bf16_view(zsrc, R * L);
  const __amdgpu_buffer_rsrc_t vDt = bf16_view(dth, L);
  int xo[kXQ];
#pragma unroll
  for (int i = 0; i < kXQ; ++i) {
    const int q = (tid + kThreads * i) % kXP, r = q / (T / 8), t8 = (q % (T / 8)) * 8;
    xo[i] = static_cast<int>((r * L + t8) * 2);
  }
  u32x4 rx[kXQ], rz[kXQ];
  auto load_xz = [&](int c) __attribute__((always_inline)) {
    const int64_t t0 = static_cast<int64_t>(c) * T;
#pragma unroll
    for (int i = 0; i < kXQ; ++i) {
      if (kVec) {
        rx[i] = buf_load8(vX, xo[i], static_cast<int>(t0 * 2));
        rz[i] = buf_load8(vZ, xo[i], static_cast<int>(t0 * 2));
      } else {
        const int q = (tid + kThreads * i) % kXP, r = q / (T / 8), t8 = (q % (T / 8)) * 8;
        rx[i] = load8_clamped<kVec>(xh + r * L, t0 + t8, L);
        rz[i] = load8_clamped<kVec>(zsrc + r * L, t0 + t8, L);
      }
    }
  };
  auto load_dt = [&](int c) __attribute__((always_inline)) {
    // past L: 0 from the view (steps() gives those tokens dt = 0 anyway)
    return __builtin_amdgcn_raw_buffer_load_b16(vDt, lane * 2, c * T * 2, 0);
  };

  // The chunk's step quantities from its raw steps (one token a lane) into
  // q[0..5]; returns whether the factored form is safe (wave-uniform: every
  // lane of every wave sees the same values).
  auto steps = [&](uint16_t raw16, int64_t t0, float (*q)[T]) __attribute__((always_inline)) {
    float v = 0.0f;
    if (t0 + lane < L) {
      const float raw = __uint_as_float(static_cast<uint32_t>(raw16) << 16) + bias;
      v = p.softplus ? softplus_f(raw) : raw;
    }
    const float cum = wave_inclusive_sum(v);
    const float a = Aq * cum;
    float aend = lane_broadcast(a, kWaveLanes - 1);
    float aref = lane_broadcast(a, kRef);
    asm volatile("" : "+s"(aend), "+s"(aref));  // formed by the whole wave first
    q[0][lane] = v;
    q[1][lane] = cum;
    q[2][lane] = fast_exp2(a);                   // decay of the incoming state
    q[3][lane] = fast_exp2(a - aref);
    q[4][lane] = fast_exp2(aref - a) * v;
    q[5][lane] = fast_exp2(aend - a) * v;        // weight of token s in the new state
    return !__any(!(fabsf(a - aref) <= kFactorLimit));
  };
  // x, x w and z of a chunk into the LDS buffers of parity `buf` (the
  // step quantities q were just written by this wave, in order)
  auto deposit = [&](int buf, float (*q)[T]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kXQ; ++i) {
      const int pc = tid + kThreads * i, r = pc / (T / 8), t8 = (pc % (T / 8)) * 8;
      if (kXP % kThreads == 0 || pc < kXP) {
        *reinterpret_cast<u32x4 *>(&Xs[buf][at(r, t8)]) = rx[i];
        if (zh) *reinterpret_cast<u32x4 *>(&Zs[buf][at(r, t8)]) = rz[i];
        const bf16x8 xv = __builtin_bit_cast(bf16x8, rx[i]);
        const f32x4 w0 = *reinterpret_cast<const f32x4 *>(&q[5][t8]);
        const f32x4 w1 = *reinterpret_cast<const f32x4 *>(&q[5][t8 + 4]);
        bf16x8 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = static_cast<__bf16>(static_cast<float>(xv[e]) * w0[e]);
          o[e + 4] = static_cast<__bf16>(static_cast<float>(xv[e + 4]) * w1[e]);
        }
        bf16x8 lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = static_cast<__bf16>(static_cast<float>(xv[e]) * w0[e] - static_cast<float>(o[e]));
          lo[e + 4] = static_cast<__bf16>(static_cast<float>(xv[e + 4]) * w1[e] -
                                          static_cast<float>(o[e + 4]));
        }
        *reinterpret_cast<bf16x8 *>(&XWs[buf][0][at(r, t8)]) = o;
        *reinterpret_cast<bf16x8 *>(&XWs[buf][1][at(r, t8)]) = lo;
      }
    }
  };
  // coalesced y stores of chunk c: this thread's pieces of the y in
  // Zs[buf] are read into registers first (the deposit of chunk c+2 reuses
  // the buffer), and the stores go out after the deposit, so that its wait
  // for x and z does not also wait for them
  u32x4 ry[kXQ];
  auto read_y = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kXQ; ++i) {
      const int pc = tid + kThreads * i, r = pc / (T / 8), t8 = (pc % (T / 8)) * 8;
      if (kXP % kThreads == 0 || pc < kXP)
        ry[i] = *reinterpret_cast<const u32x4 *>(&Zs[buf][at(r, t8)]);
    }
  };
  // (a wave-uniform chunk base and 32-bit lane offsets: no 64-bit address
  // arithmetic per store; `rem` = the chunk's tokens inside L)
  auto store_y = [&](int c) __attribute__((always_inline)) {
    const int64_t t0 = static_cast<int64_t>(c) * T;
    uint16_t *yc = yh + t0;
    const int rem = L - t0 < T ? static_cast<int>(L - t0) : T;
#pragma unroll
    for (int i = 0; i < kXQ; ++i) {
      const int pc = tid + kThreads * i, t8 = (pc % (T / 8)) * 8;
      if (kXP % kThreads == 0 || pc < kXP) {
        uint16_t *yr = yc + (xo[i] / 2);  // row pc / 8, token t8 of the chunk
        if (kVec && t8 + 8 <= rem) {
          *reinterpret_cast<u32x4 *>(yr) = ry[i];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t w = ry[i][e >> 1];
            if (t8 + e < rem) yr[e] = static_cast<uint16_t>((e & 1) ? w >> 16 : w);
          }
        }
      }
    }
  };

  // The loads are issued in the order the loop issues them (x and z of the
  // next chunk, then this chunk's operand rows): the wait counters retire
  // in order, and a different order at the loop entry makes the compiler
  // wait for every load in flight before the deposit.
  load_xz(0);
  {
    // chunks 0 and 1: every wave forms them (the same values); chunk 0's
    // deposit reads what this wave wrote
    const bool f0 = steps(load_dt(0), 0, Wq[0]);
    const bool f1 = steps(load_dt(1), T, Wq[1]);
    if (tid == 0) {
      Wf[0] = f0;
      Wf[1] = f1;
    }
    deposit(0, Wq[0]);
  }
  uint16_t dtn = load_dt(2);
  load_xz(nch > 1 ? 1 : 0);
  __builtin_amdgcn_sched_barrier(0);  // keep that order through scheduling
  load_ct(0);
  __builtin_amdgcn_sched_barrier(0);
  load_g(0);
  __builtin_amdgcn_sched_barrier(0);
  load_b(0);

  int q0 = 0, q1 = 1, q2 = 2;  // step-quantity sets of chunks c, c+1, c+2
#pragma unroll 1
  for (int c = 0; c < nch; ++c) {
    const int64_t t0 = static_cast<int64_t>(c) * T;
    const int cur = c & 1, nxt = cur ^ 1;
    const bool more = c + 1 < nch;
    const int cn = more ? c + 1 : c;  // the chunk whose operands load next
    float (*q)[T] = Wq[q0];
    // 1. the state entering the chunk as bf16 pairs, rows [p][n] (4 states
    //    a lane)
#pragma unroll
    for (int pt = 0; pt < RPW; ++pt)
#pragma unroll
      for (int k = 0; k < kNTW; ++k) {
        const int n = 16 * (kNTW * tt + k) + 4 * lq;
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = static_cast<__bf16>(S[pt][k][e]);
          lo[e] = static_cast<__bf16>(S[pt][k][e] - static_cast<float>(hi[e]));
        }
        *reinterpret_cast<bf16x4 *>(&Ss[cur][0][an(pr + 16 * pt + li, n)]) = hi;
        *reinterpret_cast<bf16x4 *>(&Ss[cur][1][an(pr + 16 * pt + li, n)]) = lo;
      }
    __syncthreads();
    const bool factored = __builtin_amdgcn_readfirstlane(Wf[q0]) != 0;
    // 2. the previous chunk's y out; chunk c+2's step quantities (one
    //    wave); the next chunk's x w and z in (x and z were requested
    //    a chunk ago)
    if (c > 0) read_y(nxt);
    if (wave == ((c + 2) & 3) && c + 2 < nch) {
      const bool f = steps(dtn, t0 + 2 * T, Wq[q2]);
      if (lane == 0) Wf[q2] = f;
    }
    if (more) deposit(nxt, Wq[q1]);
    if (c > 0) store_y(c - 1);
    if (more) {
      dtn = load_dt(c + 3);
      load_xz(c + 2 < nch ? c + 2 : c + 1);
    }

    // 3. y^T tiles of tokens 16*tt.. : (C^T S^T)[t, p] (scaled by exp(a_t)
    //    in the epilogue), then the chunk's own term; G is zero above the
    //    diagonal, so the second 32 tokens of s only reach token tiles 2, 3
    //    (independent accumulators for the two halves of each pair keep the
    //    matrix-core chains short)
    f32x4 ao[RPW], ad[RPW], ao2[RPW], ad2[RPW];
#pragma unroll
    for (int pt = 0; pt < RPW; ++pt) {
      ao[pt] = ao2[pt] = ad[pt] = ad2[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
#pragma unroll
      for (int pt = 0; pt < RPW; ++pt) {
        ao[pt] = mfma(ca[ks], lds8(&Ss[cur][0][an(pr + 16 * pt + li, 32 * ks + kq)]), ao[pt]);
        ao2[pt] = mfma(ca[ks], lds8(&Ss[cur][1][an(pr + 16 * pt + li, 32 * ks + kq)]), ao2[pt]);
      }
    load_ct(cn);
    const int nks = tt < 2 ? 1 : 2;
    if (factored) {
      // u_t ((G diag v) X^T)[t, p]: the columns of G (this lane's row ta,
      // tokens s) scaled by v_s in fp32 and split into a bf16 pair, so that
      // x enters the product exactly and nothing is rounded to one bf16
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks < nks) {
          const int s0 = 32 * ks + kq;
          const f32x4 v0 = *reinterpret_cast<const f32x4 *>(&q[4][s0]);
          const f32x4 v1 = *reinterpret_cast<const f32x4 *>(&q[4][s0 + 4]);
          bf16x8 gh, gl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float gv = (e < 4 ? ga[ks][0][e] : ga[ks][1][e - 4]) * (e < 4 ? v0[e] : v1[e - 4]);
            gh[e] = static_cast<__bf16>(gv);
            gl[e] = static_cast<__bf16>(gv - static_cast<float>(gh[e]));
          }
#pragma unroll
          for (int pt = 0; pt < RPW; ++pt) {
            const bf16x8 xs = lds8(&Xs[cur][at(pr + 16 * pt + li, s0)]);
            ad[pt] = mfma(gh, xs, ad[pt]);
            ad2[pt] = mfma(gl, xs, ad2[pt]);
          }
        }
    } else {
      // M[t, s] = G[t, s] exp(a_t - a_s) dt_s formed in the operand
      // registers
      const float ct = q[1][ta];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        if (ks < nks) {
          const int s0 = 32 * ks + kq;
          bf16x8 m, ml;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float ex = s0 + e <= ta ? Aq * (ct - q[1][s0 + e]) : -INFINITY;
            const float gv = e < 4 ? ga[ks][0][e] : ga[ks][1][e - 4];
            const float mv = gv * fast_exp2(ex) * q[0][s0 + e];
            m[e] = static_cast<__bf16>(mv);
            ml[e] = static_cast<__bf16>(mv - static_cast<float>(m[e]));
          }
#pragma unroll
          for (int pt = 0; pt < RPW; ++pt) {
            const bf16x8 xs = lds8(&Xs[cur][at(pr + 16 * pt + li, s0)]);
            ad[pt] = mfma(m, xs, ad[pt]);
            ad2[pt] = mfma(ml, xs, ad2[pt]);
          }
        }
    }
    load_g(cn);

    // 4. the state after the chunk: S^T <- exp(a_T) S^T + B (X w)^T
    {
      const float dend = q[2][T - 1];
#pragma unroll
      for (int pt = 0; pt < RPW; ++pt)
#pragma unroll
        for (int k = 0; k < kNTW; ++k) S[pt][k] *= dend;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int pt = 0; pt < RPW; ++pt) {
          const bf16x8 xw = lds8(&XWs[cur][0][at(pr + 16 * pt + li, 32 * ks + kq)]);
          const bf16x8 xl = lds8(&XWs[cur][1][at(pr + 16 * pt + li, 32 * ks + kq)]);
#pragma unroll
          for (int k = 0; k < kNTW; ++k) {
            S[pt][k] = mfma(ba[ks][k], xw, S[pt][k]);
            S[pt][k] = mfma(ba[ks][k], xl, S[pt][k]);
          }
        }
      load_b(cn);
    }

    // 5. y = exp(a_t) (C^T S^T) + u_t (own term) + D x, times silu(z); this
    //    lane's 4 tokens replace z in Zs (each element has one owner)
    {
      const f32x4 et = *reinterpret_cast<const f32x4 *>(&q[2][tq]);
      const f32x4 ut = factored ? *reinterpret_cast<const f32x4 *>(&q[3][tq])
                                : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int pt = 0; pt < RPW; ++pt) {
        const int r = pr + 16 * pt + li;
        const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(&Xs[cur][at(r, tq)]);
        float yv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          yv[e] = et[e] * (ao[pt][e] + ao2[pt][e]) + ut[e] * (ad[pt][e] + ad2[pt][e]) +
                  Dh * static_cast<float>(xv[e]);
        if (zh) {
          const bf16x4 zv = *reinterpret_cast<const bf16x4 *>(&Zs[cur][at(r, tq)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) yv[e] *= silu_f(static_cast<float>(zv[e]));
        }
        *reinterpret_cast<bf16x4 *>(&Zs[cur][at(r, tq)]) =
            bf16x4{static_cast<__bf16>(yv[0]), static_cast<__bf16>(yv[1]),
                   static_cast<__bf16>(yv[2]), static_cast<__bf16>(yv[3])};
      }
    }
    const int qn = q0;
    q0 = q1;
    q1 = q2;
    q2 = qn;
  }
  __syncthreads();
  read_y((nch - 1) & 1);
  store_y(nch - 1);

  if (p.h_final) {
#pragma unroll
    for (int pt = 0; pt < RPW; ++pt)
#pragma unroll
      for (int k = 0; k < kNTW; ++k) {
        const int n = 16 * (kNTW * tt + k) + 4 * lq;
        __builtin_memcpy(p.h_final + (bh * P + row0 + pr + 16 * pt + li) * N + n, &S[pt][k], 16);
      }
  }
}

template <int N, bool kVec, int RP, int kW>
hipError_t launch_ssd_t(const SsdArgs &a, hipStream_t s) {
  hipLaunchKernelGGL((ssd_prep_kernel<N, kVec>),
                     dim3(static_cast<unsigned>(a.nchunks), static_cast<unsigned>(a.ngroups),
                          static_cast<unsigned>(a.batch)),
                     dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_kernel<N, kVec, RP, kW>),
                     dim3(static_cast<unsigned>(a.nheads * (P / (16 * RP))),
                          static_cast<unsigned>(a.batch)),
                     dim3(64 * kW), 0, s, a);
  return hipGetLastError();
}

// Waves per workgroup (4 or 8; 8 measured slower on the 80-head layer: the
// extra waves repeat the loads of C^T, G and B and the step quantities).
#ifndef SSM_SSD_WAVES
#define SSM_SSD_WAVES 4
#endif

// Rows of a head per workgroup: the fewest splits that still give one
// workgroup per compute unit (256), since each split re-reads the group's B,
// C^T and G and repeats the step quantities.  SSM_SSD_RP fixes the choice
// (row tiles of 16 per workgroup) for measurements.
template <int N, bool kVec>
hipError_t launch_ssd_n(const SsdArgs &a, hipStream_t s) {
  constexpr int kW = SSM_SSD_WAVES;
  const int64_t seqs = a.batch * a.nheads;
  constexpr int64_t kCUs = 256;
#ifdef SSM_SSD_RP
  const int rp = SSM_SSD_RP;
#else
  const int rp = seqs >= kCUs ? 4 : 2 * seqs >= kCUs ? 2 : 1;
#endif
  // 64 rows of a 256-state head would need more than the CU's 160 KB of LDS
  if constexpr (N < 256)
    if (rp == 4) return launch_ssd_t<N, kVec, 4, kW>(a, s);
  if (rp >= 2 || kW == 8) return launch_ssd_t<N, kVec, 2, kW>(a, s);
  return launch_ssd_t<N, kVec, 1, 4>(a, s);
}

}  // namespace

int launch_ssd(const SsdArgs &a, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (a.dstate) {
    case 64:
      return vec ? launch_ssd_n<64, true>(a, s) : launch_ssd_n<64, false>(a, s);
    case 128:
      return vec ? launch_ssd_n<128, true>(a, s) : launch_ssd_n<128, false>(a, s);
    case 256:
      return vec ? launch_ssd_n<256, true>(a, s) : launch_ssd_n<256, false>(a, s);
    default:
      return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace ssm
