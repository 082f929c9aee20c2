// ssm_bwd.hip -- gfx950 (CDNA4) kernels of the selective scan's backward
// pass (Euler input term).
//
// Gradients of a loss with respect to u, delta (before softplus), A, B, C,
// D, z, the delta bias and the initial state, given its gradients dy and
// dh_final, by the chain rule through the recurrence h_t = a_t h_{t-1} + b_t
// (a_t = exp(dt_t A), b_t = dt_t B_t u_t) of "Mamba & State Space Models -
// Guide Complet", section 4.  As the inferownia.pl page says of the
// selective scan ("Cena selekcji"), the backward pass recomputes the states
// instead of reading them from HBM: a checkpoint pass (the forward kernel)
// keeps only the state entering each 1024-token block, and each block is
// recomputed on chip before its gradients are formed.
//
// With lambda_t = dL/dh_t and mu_t = a_t lambda_t (what flows from token t
// to token t-1), the reverse recurrence is
//   lambda_t = gc_t C_t + mu_{t+1},   gc_t = dy_t silu(z_t),
// itself a scan of affine maps mu_{t+1} -> a_t (gc_t C_t + mu_{t+1}), run in
// reverse token order (the associativity of the Guide Complet's "Parallel
// Associative Scan" holds in either direction).  Per (t, n):
//   ddt_t += lambda (B u + A a h_{t-1}),  dA_n += lambda a h_{t-1} dt_t,
//   dB_{t,n} += lambda dt u,  du_t += lambda dt B,  dC_{t,n} += gc_t h_t.
//
// Work layout: one wave = one channel, a workgroup = 8 channels of one
// batch entry (2 waves per SIMD), a lane = 16 consecutive tokens;
// blocks are visited from the last to the first.  For each state the lane
// recomputes its 16 states (fold, 64-lane scan, replay from the block's
// checkpoint), folds the reverse maps of its tokens, and a reverse 64-lane
// scan (lanes reversed with ds_bpermute, then the forward DPP scan) gives
// each lane the mu entering from its right.  dB and dC are sums over all
// channels of a batch entry: after each state the 8 channels of a workgroup
// write their contributions to LDS, the workgroup sums them in a fixed order
// (no atomics: deterministic) into a per-workgroup partial sum, and a
// reduction kernel sums the partials.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using namespace dev;

// Lane i receives lane 63 - i's value (LDS crossbar, no memory access).
__device__ __forceinline__ float wave_reverse(float v, int lane) {
  return __int_as_float(
      __builtin_amdgcn_ds_bpermute((kWaveLanes - 1 - lane) << 2, __float_as_int(v)));
}

constexpr int kBwdThreads = kBwdWaves * kWaveLanes;

// Contributions of one state to dB and dC, one region per wave (channel):
// sR[wave][B|C][token j of a lane run][lane'], so a wave writing token j of
// its 64 runs touches 64 consecutive words.  lane' = lane ^ 8 (j / 4): the
// reduction's 4 threads that share a run read tokens 4 apart; LDS serves a
// wave's 32-bit accesses 32 lanes at a time, where this puts the 8 runs x 4
// token groups of each half-wave on 32 different banks.
constexpr int kRegionFloats = kBwdWaves * 2 * kTokensPerLane * kWaveLanes;  // 64 KB
// One state's B and C for the block: [B|C][lane run][token], runs padded to
// 20 floats (a lane's 16-byte reads of 8 consecutive runs hit 32 banks).
constexpr int kBwdTileFloats = 2 * kWaveLanes * (kTokensPerLane + 4);  // 10 KB
__device__ __forceinline__ int region_index(int wave, int mat, int j, int lane) {
  return ((wave * 2 + mat) * kTokensPerLane + j) * kWaveLanes + (lane ^ ((j >> 2) << 3));
}

// After every wave has written its region for state n: thread tid sums the
// channels' contributions (in channel order) for 4 consecutive tokens of one
// matrix and writes them to the workgroup's partial-sum row (a 16-byte
// store when kVec; the partial block through the buffer view).  Runs of K
// tokens (fewer than 16 in a short partial block): threads whose 4 tokens
// lie past the run have nothing to write.
template <bool kVec, bool kFull, int K = kTokensPerLane>
__device__ __forceinline__ void flush_state(const float *sR, int tid, float *pB_row,
                                            float *pC_row, int64_t t0, int64_t tend) {
  constexpr int kPer = 2 * kTokensPerLane * kWaveLanes / kBwdThreads;  // 4
  constexpr int kParts = kTokensPerLane / kPer;                        // per run
  const int mat = tid / (kBwdThreads / 2);  // first half: dB, second: dC (wave-uniform)
  const int r = tid % (kBwdThreads / 2);
  const int run = r / kParts;               // the lane run ...
  const int j0 = (r % kParts) * kPer;       // ... and which part of it
  if (K < kTokensPerLane && j0 >= K) return;
  float v[kPer];
#pragma unroll
  for (int jj = 0; jj < kPer; ++jj) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kBwdWaves; ++w) acc += sR[region_index(w, mat, j0 + jj, run)];
    v[jj] = acc;
  }
  float *row = mat ? pC_row : pB_row;
  store_run<float, kPer, kVec, kFull>(row, t0, t0 + run * K + j0, tend, v);
}

// Per-state values of one channel kept one state per lane (lane n holds
// state n) in a single register instead of 16 scalar registers.
__device__ __forceinline__ float state_of(float v, int n) { return lane_broadcast(v, n); }
__device__ __forceinline__ float set_state(float v, int lane, int n, float x) {
  return lane == n ? x : v;
}

// One block of one channel, in reverse.  hfv: the forward states entering
// the block (checkpoint; lane n = state n); muv: dL/dh flowing in from the
// right of the block (replaced by what flows out of its first token); dAv:
// running dA sums of the channel (lane n = state n, already times 1/ln2).
// K: tokens per lane.  Full blocks use kTokensPerLane; the partial last
// block uses the fewest of 4, 8, 16 that cover it, so its loops cost about
// its share of a block.
template <typename T, bool kVec, bool kFull, bool kSoftplus, int K = kTokensPerLane>
__device__ __forceinline__ void bwd_block(
    const BwdArgs &p, int wave, int lane, int64_t t0, int64_t tend, int64_t b,
    int64_t bd, int64_t g, const T *__restrict__ Bb, const T *__restrict__ Cb,
    bool ch_ok, float bias, float Dd, float Av, float hfv, float &muv, float &dAv,
    float &dDl, float &dbl, float *sT, float *sR, int tid) {
  static_assert(!kFull || K == kTokensPerLane, "full blocks: 16 tokens a lane");
  static_assert(K == 4 || K == 8 || K == 16, "runs of 4, 8 or 16 tokens");
  constexpr int KP = K == 4 ? 12 : K + 4;  // a multiple of 4 floats: 16-byte runs
  const int64_t tl = t0 + static_cast<int64_t>(lane) * K;
  const T *urow = static_cast<const T *>(p.u) + bd * p.L;
  const T *drow = static_cast<const T *>(p.delta) + bd * p.L;
  const T *zrow = p.z ? static_cast<const T *>(p.z) + bd * p.L : nullptr;
  const T *gyrow = static_cast<const T *>(p.dy) + bd * p.L;

  // staging role of this wave: matrix mat (B or C) of the next state,
  // 4-token piece `qr` of every lane run (runs shorter than 16 tokens have
  // fewer pieces; the waves past them stage nothing)
  constexpr int kQuarterRun = 4;
  constexpr int kPieces = K / kQuarterRun;
  const int mat = wave & 1, qr = wave >> 1;
  const bool stager = K == kTokensPerLane || qr < kPieces;
  const T *src = mat ? Cb : Bb;
  const int toff = (mat * kWaveLanes + lane) * KP + qr * kQuarterRun;
  const int64_t tq = tl + qr * kQuarterRun;
  float *pBg = p.pB + (b * p.groups + g) * kStates * p.L;  // this group's partial rows
  float *pCg = p.pC + (b * p.groups + g) * kStates * p.L;
  TileRun<T, kQuarterRun, kVec, kFull> run;
  if (stager) run.load(src, t0, tq, tend);  // state 0

  // per token: dt (as dt*log2 e), dt*u, the gated output gradient gc and
  // the sums over states s1 = sum lambda B, s2 = sum lambda a h_prev A
  float dtl[K], du[K], gc[K], s1[K], s2[K];
  float sdt = 0.0f;
  {
    float uu[K], dr[K];
    load_run<T, K, kVec, kFull>(urow, t0, tl, tend, uu);
    load_run<T, K, kVec, kFull>(drow, t0, tl, tend, dr);
    load_run<T, K, kVec, kFull>(gyrow, t0, tl, tend, gc);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float x = dr[j] + bias;
      float v = kSoftplus ? softplus_f(x) : x;
      if (!kFull) v = (tl + j < tend) ? v : 0.0f;  // identity step
      dtl[j] = v * kLog2e;
      du[j] = v * uu[j];
      sdt += v;
      s1[j] = 0.0f;
      s2[j] = 0.0f;
    }
  }
  if (zrow) {
    float zz[K];
    load_run<T, K, kVec, kFull>(zrow, t0, tl, tend, zz);
#pragma unroll
    for (int j = 0; j < K; ++j) gc[j] *= silu_f(zz[j]);
  }
  if (!ch_ok) {
    // a wave past the last channel: with gc = dt*u = 0 its dB and dC
    // contributions (lambda dt u and gc h) vanish; nothing else of it is
    // stored
#pragma unroll
    for (int j = 0; j < K; ++j) gc[j] = du[j] = 0.0f;
  }
  if (stager) run.store(sT, toff);
  const float sdtl = sdt * kLog2e;
  // One barrier per state: state n reads tile buffer n & 1 and writes
  // region buffer n & 1; before its barrier each wave stores its share of
  // state n+1's tile into the other tile buffer (last read by state n-1,
  // before the previous barrier); after it, the workgroup sums state n's
  // region, which is written again by state n+2, after the next barrier.
  __syncthreads();  // the tile of state 0 (and the previous block's last sums read)

#pragma unroll 1
  for (int n = 0; n < kStates; ++n) {
    if (stager && n + 1 < kStates) run.load(src + (n + 1) * p.L, t0, tq, tend);
    const float *tile = sT + (n & 1) * kBwdTileFloats;
    float *reg = sR + (n & 1) * kRegionFloats;
    float An = state_of(Av, n);
    asm volatile("" : "+s"(An));  // keep this state's work after the previous state's
    const float hfn = state_of(hfv, n);
    const float mun = state_of(muv, n);
    // this state's B and C for the lane's 16 tokens, read from the tile once
    float bv[K], cv[K];
    {
      const float4 *pb = reinterpret_cast<const float4 *>(&tile[lane * KP]);
      const float4 *pc = reinterpret_cast<const float4 *>(&tile[(kWaveLanes + lane) * KP]);
#pragma unroll
      for (int q = 0; q < K / 4; ++q) {
        const float4 x = pb[q], y4 = pc[q];
        bv[4 * q + 0] = x.x; bv[4 * q + 1] = x.y; bv[4 * q + 2] = x.z; bv[4 * q + 3] = x.w;
        cv[4 * q + 0] = y4.x; cv[4 * q + 1] = y4.y; cv[4 * q + 2] = y4.z; cv[4 * q + 3] = y4.w;
      }
    }
    // forward recomputation of this lane's 16 states:
    // hin = the state before the lane's first token, hs[j] = after token j
    float a[K], hs[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a[j] = fast_exp2(dtl[j] * An);
      hs[j] = du[j] * bv[j];  // dt B u, replaced by the state below
    }
    float H = hs[0];
#pragma unroll
    for (int j = 1; j < K; ++j) H = fmaf(a[j], H, hs[j]);
    const float Pl = fast_exp2(sdtl * An);  // product of the lane's a
    float P = Pl;
    H = fmaf(P, lane == 0 ? hfn : 0.0f, H);
    wave_affine_scan(P, H);
    const float hin = wave_shift_in(H, hfn);
    {
      float h = hin;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        h = fmaf(a[j], h, hs[j]);
        hs[j] = h;
      }
    }
    // reverse: the lane's map mu_in -> mu_out (tokens 15 .. 0), then the
    // 64 lanes composed from the right (reversed lane order, forward scan)
    float M = 0.0f;
#pragma unroll
    for (int j = K - 1; j >= 0; --j) M = fmaf(gc[j], cv[j], M) * a[j];
    float Pr = wave_reverse(Pl, lane);
    float Mr = wave_reverse(M, lane);
    Mr = fmaf(Pr, lane == 0 ? mun : 0.0f, Mr);
    wave_affine_scan(Pr, Mr);
    // cross-lane results are formed by the whole wave and pinned in a
    // scalar register before one lane takes them: otherwise the compiler
    // may move the DPP / readlane under the lane == n mask
    float mu_out = lane_broadcast(Mr, kWaveLanes - 1);
    asm volatile("" : "+s"(mu_out));
    muv = set_state(muv, lane, n, mu_out);
    float m = wave_reverse(wave_shift_in(Mr, mun), lane);
    // reverse replay: lambda_j = dL/dh_j, then the gradients of token j
    float dA_acc = 0.0f;
#pragma unroll
    for (int j = K - 1; j >= 0; --j) {
      const float lam = fmaf(gc[j], cv[j], m);
      s1[j] = fmaf(lam, bv[j], s1[j]);
      m = a[j] * lam;                                  // lambda a
      const float q = m * (j > 0 ? hs[j - 1] : hin);   // lambda a h_{j-1}
      s2[j] = fmaf(q, An, s2[j]);
      dA_acc = fmaf(q, dtl[j], dA_acc);
      reg[region_index(wave, 0, j, lane)] = lam * du[j];
      reg[region_index(wave, 1, j, lane)] = gc[j] * hs[j];
    }
    float dA_sum = lane_broadcast(wave_inclusive_sum(dA_acc), kWaveLanes - 1);
    asm volatile("" : "+s"(dA_sum));
    dAv += lane == n ? dA_sum : 0.0f;
    if (stager && n + 1 < kStates) run.store(sT + ((n + 1) & 1) * kBwdTileFloats, toff);
    __syncthreads();  // state n's contributions and state n+1's tile are in LDS
    flush_state<kVec, kFull, K>(reg, tid, pBg + n * p.L, pCg + n * p.L, t0, tend);
  }

  // per-token gradients
  float uu[K], dr[K];
  load_run<T, K, kVec, kFull>(urow, t0, tl, tend, uu);
  load_run<T, K, kVec, kFull>(drow, t0, tl, tend, dr);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const float x = dr[j] + bias;
    const float dt = kSoftplus ? softplus_f(x) : x;
    const float ddt = fmaf(uu[j], s1[j], s2[j]);
    const float dx = kSoftplus ? ddt * sigmoid_f(x) : ddt;
    dbl += (kFull || tl + j < tend) ? dx : 0.0f;
    dDl = fmaf(gc[j], uu[j], dDl);
    s1[j] = fmaf(dt, s1[j], gc[j] * Dd);  // du
    s2[j] = dx;                            // ddelta
  }
  if (ch_ok) {
    store_run<T, K, kVec, kFull>(static_cast<T *>(p.du) + bd * p.L, t0, tl, tend, s1);
    store_run<T, K, kVec, kFull>(static_cast<T *>(p.ddelta) + bd * p.L, t0, tl, tend, s2);
  }
  if (zrow && p.dz) {
    // the gate: dz = dy * yc * silu'(z), yc the pre-gate output the
    // checkpoint pass stored
    float zz[K], gy[K], yv[K];
    load_run<T, K, kVec, kFull>(zrow, t0, tl, tend, zz);
    load_run<T, K, kVec, kFull>(gyrow, t0, tl, tend, gy);
    load_run<T, K, kVec, kFull>(static_cast<const T *>(p.yc) + bd * p.L, t0, tl, tend, yv);
#pragma unroll
    for (int j = 0; j < K; ++j) yv[j] = gy[j] * yv[j] * dsilu_f(zz[j]);
    if (ch_ok)
      store_run<T, K, kVec, kFull>(static_cast<T *>(p.dz) + bd * p.L, t0, tl, tend, yv);
  }
}

template <typename T, bool kVec, bool kSoftplus>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_kernel(BwdArgs p) {
  __shared__ float sT[2 * kBwdTileFloats];  // one state's B, C (fp32), double-buffered
  __shared__ float sR[2 * kRegionFloats];   // dB, dC contributions of the 8 channels, double-buffered

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b = blockIdx.y;
  const int64_t g = blockIdx.x;
  const int64_t d_raw = g * kBwdWaves + wave;
  const bool ch_ok = d_raw < p.dim;
  const int64_t d = ch_ok ? d_raw : p.dim - 1;  // clamped for reads
  const int64_t bd = b * p.dim + d;
  const int ls = lane < kStates ? lane : 0;  // lane n <-> state n

  const float Av = p.A[d * kStates + ls];
  float muv = p.dh_final ? p.dh_final[bd * kStates + ls] : 0.0f;
  float dAv = 0.0f;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const T *Bb = static_cast<const T *>(p.B) + b * kStates * p.L;
  const T *Cb = static_cast<const T *>(p.C) + b * kStates * p.L;
  float dDl = 0.0f, dbl = 0.0f;

  const float *ck = p.ckpt + bd * p.nblk * kStates;
  const int64_t nfull = p.L / kBlockTokens;
  const int64_t rem = p.L - nfull * kBlockTokens;
  if (rem > 0) {  // the partial last block comes first
    const float hf = ck[nfull * kStates + ls];
    if (rem <= 4 * kWaveLanes)
      bwd_block<T, false, false, kSoftplus, 4>(p, wave, lane, nfull * kBlockTokens, p.L, b,
                                               bd, g, Bb, Cb, ch_ok, bias, Dd, Av, hf, muv,
                                               dAv, dDl, dbl, sT, sR, tid);
    else if (rem <= 8 * kWaveLanes)
      bwd_block<T, false, false, kSoftplus, 8>(p, wave, lane, nfull * kBlockTokens, p.L, b,
                                               bd, g, Bb, Cb, ch_ok, bias, Dd, Av, hf, muv,
                                               dAv, dDl, dbl, sT, sR, tid);
    else
      bwd_block<T, false, false, kSoftplus>(p, wave, lane, nfull * kBlockTokens, p.L, b, bd,
                                            g, Bb, Cb, ch_ok, bias, Dd, Av, hf, muv, dAv,
                                            dDl, dbl, sT, sR, tid);
  }
#pragma unroll 1
  for (int64_t k = nfull - 1; k >= 0; --k)
    bwd_block<T, kVec, true, kSoftplus>(p, wave, lane, k * kBlockTokens,
                                        (k + 1) * kBlockTokens, b, bd, g, Bb, Cb, ch_ok, bias,
                                        Dd, Av, ck[k * kStates + ls], muv, dAv, dDl, dbl, sT,
                                        sR, tid);

  if (!ch_ok) return;
  if (lane < kStates) {
    p.pA[bd * kStates + lane] = dAv * kLn2;  // sum of q * dt = q * dtl * ln2
    if (p.dh0) p.dh0[bd * kStates + lane] = muv;
  }
  float sD = lane_broadcast(wave_inclusive_sum(dDl), kWaveLanes - 1);
  float sb = lane_broadcast(wave_inclusive_sum(dbl), kWaveLanes - 1);
  asm volatile("" : "+s"(sD), "+s"(sb));  // formed by the whole wave first
  if (lane == 0) {
    p.pD[bd] = sD;
    p.pbias[bd] = sb;
  }
}

// dB[b, n, t] (blockIdx.y = 0) or dC (1): the sum over channel groups of
// the partial rows.  A workgroup takes 256 consecutive tokens (64 lanes x 4)
// of one (b, n) row; its 4 waves take every 4th group (16-byte loads, 1 KB
// per wave and group) and add up in LDS at the end.
constexpr int kReduceWaves = 4;
constexpr int kReduceTokens = 4 * kWaveLanes;  // per workgroup
__global__ __launch_bounds__(kReduceWaves * kWaveLanes) void bwd_reduce_bc_kernel(BwdArgs p) {
  __shared__ float4 red[kReduceWaves - 1][kWaveLanes];
  const int lane = threadIdx.x & 63;
  const int slice = threadIdx.x >> 6;
  const int64_t ntb = (p.L + kReduceTokens - 1) / kReduceTokens;
  const int64_t row = blockIdx.x / ntb;  // b * 16 + n
  const int64_t t = (blockIdx.x - row * ntb) * kReduceTokens + lane * 4;
  const int64_t b = row / kStates, n = row - b * kStates;
  const float *part = (blockIdx.y ? p.pC : p.pB) + (b * p.groups * kStates + n) * p.L;
  const int64_t gstride = kStates * p.L;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if ((p.L & 3) == 0 && t < p.L) {
    // This wave's groups slice, slice + 4, ... summed in order through a
    // ring of kRing loads in flight: group g's value is added, then group
    // g + kRing is requested into its register (the order of additions is
    // that of one group at a time).  The scheduling barriers keep each load
    // right after the add that frees its register; left to itself the
    // scheduler groups the loads and waits for all of them at once.
    constexpr int kRing = 8;
    const int64_t step = kReduceWaves * gstride;
    const int64_t ng = (p.groups - slice + kReduceWaves - 1) / kReduceWaves;
    const float *q = part + t + slice * gstride;
    int64_t g = 0;
    if (ng >= kRing) {
      float4 v[kRing];
#pragma unroll
      for (int k = 0; k < kRing; ++k)
        v[k] = *reinterpret_cast<const float4 *>(q + k * step);
      for (; g + 2 * kRing <= ng; g += kRing) {
        const float *qn = q + (g + kRing) * step;
#pragma unroll
        for (int k = 0; k < kRing; ++k) {
          acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
          v[k] = *reinterpret_cast<const float4 *>(qn + k * step);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int k = 0; k < kRing; ++k) {
        acc.x += v[k].x; acc.y += v[k].y; acc.z += v[k].z; acc.w += v[k].w;
      }
      g += kRing;
    }
    for (; g < ng; ++g) {
      const float4 v = *reinterpret_cast<const float4 *>(q + g * step);
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  } else if (t < p.L) {
    const int cnt = p.L - t < 4 ? static_cast<int>(p.L - t) : 4;
    for (int64_t gi = slice; gi < p.groups; gi += kReduceWaves) {
      const float *q = part + gi * gstride + t;
      acc.x += q[0];
      if (cnt > 1) acc.y += q[1];
      if (cnt > 2) acc.z += q[2];
      if (cnt > 3) acc.w += q[3];
    }
  }
  if (slice > 0) red[slice - 1][lane] = acc;
  __syncthreads();
  if (slice != 0 || t >= p.L) return;
#pragma unroll
  for (int i = 0; i < kReduceWaves - 1; ++i) {
    acc.x += red[i][lane].x; acc.y += red[i][lane].y;
    acc.z += red[i][lane].z; acc.w += red[i][lane].w;
  }
  float *out = (blockIdx.y ? p.dC : p.dB) + row * p.L + t;
  if ((p.L & 3) == 0) {
    *reinterpret_cast<float4 *>(out) = acc;
  } else {
    const int cnt = p.L - t < 4 ? static_cast<int>(p.L - t) : 4;
    out[0] = acc.x;
    if (cnt > 1) out[1] = acc.y;
    if (cnt > 2) out[2] = acc.z;
    if (cnt > 3) out[3] = acc.w;
  }
}

// dA[d, n], dD[d], dbias[d]: sums over the batch of the per-(b, d) partials.
__global__ __launch_bounds__(256) void bwd_reduce_param_kernel(BwdArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= p.dim * kStates) return;
  const int64_t d = i / kStates;
  float sa = 0.0f;
  for (int64_t b = 0; b < p.batch; ++b) sa += p.pA[(b * p.dim) * kStates + i];
  p.dA[i] = sa;
  if ((i % kStates) == 0) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t b = 0; b < p.batch; ++b) {
      sd += p.pD[b * p.dim + d];
      sb += p.pbias[b * p.dim + d];
    }
    if (p.dD) p.dD[d] = sd;
    if (p.dbias) p.dbias[d] = sb;
  }
}

template <typename T, bool kVec>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.groups), static_cast<unsigned>(a.batch));
  if (a.softplus)
    hipLaunchKernelGGL((bwd_kernel<T, kVec, true>), grid, dim3(kBwdThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_kernel<T, kVec, false>), grid, dim3(kBwdThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nwg = a.batch * kStates * ((a.L + kReduceTokens - 1) / kReduceTokens);
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(static_cast<unsigned>(nwg), 2), dim3(256), 0,
                     s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_param_kernel,
                     dim3(static_cast<unsigned>((a.dim * kStates + 255) / 256)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace

int launch_bwd(const BwdArgs &a, bool bf16, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch_bwd_t<uint16_t, true>(a, s) : launch_bwd_t<uint16_t, false>(a, s);
  return vec ? launch_bwd_t<float, true>(a, s) : launch_bwd_t<float, false>(a, s);
}

}  // namespace ssm
