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
// Work layout of the scan kernel (one wave = one channel; one workgroup = 4
// channels of one batch entry; one lane = 16 consecutive tokens; a block =
// 64 lanes x 16 = 1024 tokens):
//   * B and C of the block are read from HBM once per workgroup, two states
//     at a time into a double-buffered LDS tile (the next pair is fetched
//     while the current one is used), widened to fp32 and shared by the
//     workgroup's 4 channels;
//   * per lane and state n: dA and dB*u of its 16 tokens stay in registers;
//     the lane folds them into one affine pair (P, H); a 6-step DPP scan over
//     the 64 lanes composes the pairs (the state carried in from the previous
//     block enters lane 0 first); each lane then replays its 16 tokens from
//     its true incoming state and accumulates C_t,n * h into y;
//   * the channel's A, D, bias and carried state are wave-uniform (scalar
//     registers);
//   * the epilogue applies the gate and writes y; the state after the last
//     token goes to h_final.
// All arithmetic is fp32.  No MFMA: the work is a recurrence, not a dense
// contraction.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

using namespace dev;

// One block of 1024 tokens of one channel per wave (4 channels of one batch
// entry per workgroup).  kFull: the block lies wholly inside [t0, ct1), so
// nothing is masked; otherwise positions from ct1 on are identity steps
// (dt = 0, u = 0) and are not stored.  hc[n]: the channel's state carried in
// (wave-uniform), replaced by the state after the block.
// Instances that carry the next block's u and delta in registers across
// the block loop: aligned fp32 rows with the Euler term and no conv
// prologue (their register budget, sized for 3 waves per SIMD, has the 32
// registers free; the bf16 instance runs at its 128-register cap).
template <typename T, bool kVec, bool kConv, bool kZoh, bool kCkpt>
constexpr bool kPrefetch = sizeof(T) == 4 && kVec && !kConv && !kZoh && !kCkpt;

// K: tokens per lane.  Full blocks use kTokensPerLane; the last, partial
// block of a chunk uses the fewest of 4, 8, 16 that cover it, so its state
// loop costs about its share of a block rather than a whole one.
template <typename T, bool kVec, bool kFull, bool kSoftplus, bool kConv,
          bool kZoh, bool kCkpt, int K = kTokensPerLane>
__device__ __forceinline__ void scan_block(
    const ScanArgs &p, int wave, int lane, int64_t t0, int64_t ct1,
    const T *__restrict__ Bb, const T *__restrict__ Cb,
    const T *__restrict__ urow, const T *__restrict__ drow,
    const T *__restrict__ zrow, T *__restrict__ yrow, T *__restrict__ ycrow,
    bool ch_ok, float bias, float Dd, const float (&Ach)[kStates], float *sT,
    float (&hc)[kStates], float &sdt_total, const float (&wc)[kMaxConv], float cb,
    float (&xc)[kMaxConv - 1], float (&upf)[kTokensPerLane],
    float (&dpf)[kTokensPerLane], bool use_pf, int64_t pf_t0) {
  static_assert(!kFull || K == kTokensPerLane, "full blocks: 16 tokens a lane");
  static_assert(K == 4 || K == 8 || K == 16, "runs of 4, 8 or 16 tokens");
  // padded LDS stride of one lane's run: a lane's 16-byte reads of 8
  // consecutive runs fall on 32 different banks
  constexpr int KP = K == 4 ? 12 : K + 4;
  const int64_t tend = kFull ? t0 + kBlockTokens : ct1;
  const int64_t tl = t0 + static_cast<int64_t>(lane) * K;
  constexpr int kPhases = kStates / 2;
  constexpr int kTileFloats = 2 * 2 * kWaveLanes * KP;

  // Staging role of this wave: state (2*ph + st) of matrix B or C (both
  // wave-uniform, so the row is a valid buffer base in the partial block);
  // this lane: run `lane` of that row.
  const int st = wave >> 1, mat = wave & 1;
  const T *src = mat ? Cb : Bb;
  const int64_t tq = tl;
  const int toff = staging_offset<KP>(wave, lane);
  TileRun<T, K, kVec, kFull> run;
  run.load(src + st * p.L, t0, tq, tend);

  // This lane's tokens: the step dt (kept as dt*log2(e) for exp2), dt*u
  // and the D skip.
  float dtl[K], du[K], y[K];
  float sdt = 0.0f;
  {
    float uu[K], dr[K];
    if (kPrefetch<T, kVec, kConv, kZoh, kCkpt> && kFull && use_pf) {
#pragma unroll
      for (int j = 0; j < K; ++j) uu[j] = upf[j];
    } else {
      load_run<T, K, kVec, kFull>(urow, t0, tl, tend, uu);
    }
    if constexpr (kConv) {
      // urow holds the pre-conv input x: u = silu(cb + sum_k wc[k] *
      // x[t-3+k]).  The three values before the lane's first token come
      // from the left neighbour (lane 0: from the previous block / chunk).
      float xm[kMaxConv - 1];
#pragma unroll
      for (int k = 0; k < kMaxConv - 1; ++k)
        xm[k] = wave_shift_in(uu[K - (kMaxConv - 1) + k], xc[k]);
#pragma unroll
      for (int k = 0; k < kMaxConv - 1; ++k)
        xc[k] = lane_broadcast(uu[K - (kMaxConv - 1) + k], kWaveLanes - 1);
      float xs[K];
#pragma unroll
      for (int j = 0; j < K; ++j) xs[j] = uu[j];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float acc = cb;
#pragma unroll
        for (int k = 0; k < kMaxConv; ++k) {
          const int s = j - (kMaxConv - 1) + k;  // token of tap k
          acc = fmaf(wc[k], s >= 0 ? xs[s] : xm[s + kMaxConv - 1], acc);
        }
        uu[j] = silu_f(acc);
      }
    }
    if (kPrefetch<T, kVec, kConv, kZoh, kCkpt> && kFull && use_pf) {
#pragma unroll
      for (int j = 0; j < K; ++j) dr[j] = dpf[j];
    } else {
      load_run<T, K, kVec, kFull>(drow, t0, tl, tend, dr);
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float x = dr[j] + bias;
      float v = kSoftplus ? softplus_f(x) : x;
      if (!kFull) v = (tl + j < tend) ? v : 0.0f;  // identity step
      dtl[j] = v * kLog2e;
      du[j] = kZoh ? uu[j] : v * uu[j];  // ZOH: the coefficient carries dt
      y[j] = Dd * uu[j];
      sdt += v;
    }
  }
  // Phase 0's tile: its buffer was last read two phases ago, by every wave.
  run.store(sT, toff);
  const float sdtl = sdt * kLog2e;
  // u and delta of the full block at pf_t0 (the next one, or this one
  // again when none follows), in flight during this block's state loop
  if constexpr (kPrefetch<T, kVec, kConv, kZoh, kCkpt> && kFull) {
    const int64_t tlp = pf_t0 + static_cast<int64_t>(lane) * K;
    load_run<T, K, kVec, true>(urow, pf_t0, tlp, pf_t0 + kBlockTokens, upf);
    load_run<T, K, kVec, true>(drow, pf_t0, tlp, pf_t0 + kBlockTokens, dpf);
  }

  // B and C are staged two states at a time in a double-buffered LDS tile
  // (tile[buffer][state][B|C][lane run][KP]); while the 4 waves compute
  // phase ph, each thread already holds phase ph+1's run in registers.
#pragma unroll
  for (int ph = 0; ph < kPhases; ++ph) {
    if (ph + 1 < kPhases)
      run.load(src + (2 * (ph + 1) + st) * p.L, t0, tq, tend);
    __syncthreads();  // phase ph's tile is complete and visible
    const float *tile = sT + (ph & 1) * kTileFloats;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int n = 2 * ph + s2;
      float An = Ach[n];
      asm volatile("" : "+s"(An));  // keep this state's work after the previous state's
      const float *pb = &tile[((s2 * 2 + 0) * kWaveLanes + lane) * KP];
      const float *pc = &tile[((s2 * 2 + 1) * kWaveLanes + lane) * KP];
      float a[K], bb[K];
      if constexpr (kZoh) {
        // A = 0 needs no branch: its argument is 0, the series is selected
        // and gives dt (the 1/A = inf of the other operand is not used).
        const float inv_a = 1.0f / An;
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float arg = dtl[j] * An;
          a[j] = fast_exp2(arg);
          bb[j] = zoh_coeff(arg, a[j], dtl[j], inv_a) * (du[j] * pb[j]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j) {
          a[j] = fast_exp2(dtl[j] * An);
          bb[j] = du[j] * pb[j];
        }
      }
      // Fold the lane's tokens into one affine map h -> P*h + H.
      float H = bb[0];
#pragma unroll
      for (int j = 1; j < K; ++j) H = fmaf(a[j], H, bb[j]);
      float P = fast_exp2(sdtl * An);
      // The carried state enters through lane 0, then the maps compose.
      H = fmaf(P, lane == 0 ? hc[n] : 0.0f, H);
      wave_affine_scan(P, H);
      // H_i is the true state after lane i's last token; lane i starts from
      // lane i-1's (lane 0 from the carried state) and replays its tokens.
      float h = wave_shift_in(H, hc[n]);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        h = fmaf(a[j], h, bb[j]);
        y[j] = fmaf(pc[j], h, y[j]);
      }
      hc[n] = lane_broadcast(h, kWaveLanes - 1);
    }
    // Every wave has passed this phase's barrier, so the other buffer (read
    // in phase ph-1) is free: fill it with phase ph+1.
    if (ph + 1 < kPhases) run.store(sT + ((ph + 1) & 1) * kTileFloats, toff);
  }

  // checkpoint instance: the pre-gate output, for the backward's dz
  if (kCkpt && ycrow && ch_ok) store_run<T, K, kVec, kFull>(ycrow, t0, tl, tend, y);
  if (zrow) {
    float zz[K];
    load_run<T, K, kVec, kFull>(zrow, t0, tl, tend, zz);
#pragma unroll
    for (int j = 0; j < K; ++j) y[j] *= silu_f(zz[j]);
  }
  if (ch_ok) store_run<T, K, kVec, kFull>(yrow, t0, tl, tend, y);
  sdt_total += sdt;
}

// Waves per SIMD the register budget is sized for: 4 (128 VGPRs; 4
// workgroups x 40 KB fill a CU's 160 KB of LDS) for aligned bf16 rows with
// the Euler input term; 3 (168 VGPRs) otherwise, where the longer ZOH state
// loop, the wider fp32 loads or the element-wise loads of unaligned rows
// would spill or stall at 128 (measured: fp32 and unaligned bf16 run faster
// at 3).
template <typename T, bool kVec, bool kZoh>
constexpr int kOccupancy = (sizeof(T) == 2 && kVec && !kZoh) ? 4 : 3;

template <typename T, bool kVec, bool kSoftplus, bool kConv, bool kZoh, bool kCkpt = false>
__global__ __launch_bounds__(kWaveLanes * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(kOccupancy<T, kVec, kZoh>)))
void scan_kernel(ScanArgs p) {
  constexpr int KP = kTokensPerLane + 4;
  __shared__ float sT[2 * 2 * 2 * kWaveLanes * KP];  // 2 buffers x 2 states x B, C

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b = blockIdx.y;
  const int64_t d_raw = static_cast<int64_t>(blockIdx.x) * kChannelsPerGroup + wave;
  const bool ch_ok = d_raw < p.dim;
  const int64_t d = ch_ok ? d_raw : p.dim - 1;  // clamped for reads
  const int chunk = blockIdx.z;
  const int64_t ct0 = static_cast<int64_t>(chunk) * p.chunk_len;
  const int64_t ct1 = ct0 + p.chunk_len < p.L ? ct0 + p.chunk_len : p.L;
  const int64_t bd = b * p.dim + d;

  float Ach[kStates];  // the channel's A (wave-uniform)
#pragma unroll
  for (int n = 0; n < kStates; ++n) Ach[n] = p.A[d * kStates + n];
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  float hc[kStates];  // the channel's carried state (wave-uniform)
#pragma unroll
  for (int n = 0; n < kStates; ++n)
    hc[n] = (chunk == 0 && p.h0) ? p.h0[bd * kStates + n] : 0.0f;

  const T *urow = static_cast<const T *>(kConv ? p.x : p.u) + bd * p.L;
  const T *drow = static_cast<const T *>(p.delta) + bd * p.L;
  const T *zrow = p.z ? static_cast<const T *>(p.z) + bd * p.L : nullptr;
  T *yrow = static_cast<T *>(p.y) + bd * p.L;
  T *ycrow = (kCkpt && p.yc) ? static_cast<T *>(p.yc) + bd * p.L : nullptr;
  const T *Bb = static_cast<const T *>(p.B) + b * kStates * p.L;
  const T *Cb = static_cast<const T *>(p.C) + b * kStates * p.L;
  float sdt_total = 0.0f;

  // Conv prologue (wave-uniform): taps aligned to the last kMaxConv tokens
  // (fewer taps: leading zeros), bias, and the kMaxConv-1 inputs before the
  // chunk (zero before t = 0).
  float wc[kMaxConv], cb = 0.0f, xc[kMaxConv - 1];
#pragma unroll
  for (int k = 0; k < kMaxConv; ++k) {
    const int i = k - (kMaxConv - p.d_conv);
    wc[k] = (kConv && i >= 0) ? p.conv_w[d * p.d_conv + i] : 0.0f;
  }
  if (kConv && p.conv_b) cb = p.conv_b[d];
#pragma unroll
  for (int k = 0; k < kMaxConv - 1; ++k) {
    const int64_t t = ct0 - (kMaxConv - 1) + k;
    xc[k] = (kConv && t >= 0) ? to_f32<T>(urow[t]) : 0.0f;
  }

  // checkpoint instance (kCkpt; unsplit sequences): the state entering
  // block k goes to ckpt[b, d, k, :]; with p.yc the pre-gate output goes
  // there as well (the backward's own checkpoint pass runs without a gate
  // and takes y itself as the pre-gate output)
  const int64_t nblk = (p.L + kBlockTokens - 1) / kBlockTokens;
  float *ck = (kCkpt && ch_ok) ? p.ckpt + bd * nblk * kStates : nullptr;

  float upf[kTokensPerLane], dpf[kTokensPerLane];  // prefetched u, delta
  const int64_t last_full = ct0 + ((ct1 - ct0) / kBlockTokens - 1) * kBlockTokens;
  int64_t t0 = ct0;
#pragma unroll 1
  for (; t0 + kBlockTokens <= ct1; t0 += kBlockTokens) {
    if (kCkpt && ck && lane == 0) {
#pragma unroll
      for (int n = 0; n < kStates; ++n)
        ck[(t0 / kBlockTokens) * kStates + n] = hc[n];
    }
    scan_block<T, kVec, true, kSoftplus, kConv, kZoh, kCkpt>(
        p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd, Ach,
        sT, hc, sdt_total, wc, cb, xc,
        upf, dpf, t0 > ct0,
        t0 + 2 * kBlockTokens <= ct1 ? t0 + kBlockTokens : last_full);
  }
  if (kCkpt && t0 < ct1 && ck && lane == 0) {
#pragma unroll
    for (int n = 0; n < kStates; ++n) ck[(t0 / kBlockTokens) * kStates + n] = hc[n];
  }
  if (t0 < ct1) {
    // the last, partial block: branch-free scalar loads (keeps the register
    // budget of the full-block loop), as few tokens per lane as cover it
    const int64_t rem = ct1 - t0;
    if (rem <= 4 * kWaveLanes)
      scan_block<T, false, false, kSoftplus, kConv, kZoh, kCkpt, 4>(
          p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd,
          Ach, sT, hc, sdt_total, wc, cb, xc, upf, dpf, false, t0);
    else if (rem <= 8 * kWaveLanes)
      scan_block<T, false, false, kSoftplus, kConv, kZoh, kCkpt, 8>(
          p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd,
          Ach, sT, hc, sdt_total, wc, cb, xc, upf, dpf, false, t0);
    else
      scan_block<T, false, false, kSoftplus, kConv, kZoh, kCkpt>(
          p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd,
          Ach, sT, hc, sdt_total, wc, cb, xc, upf, dpf, false, t0);
  }

  if (!ch_ok) return;
  if (p.n_chunks == 1) {
    if (p.h_final && lane == 0) {
#pragma unroll
      for (int n = 0; n < kStates; ++n) p.h_final[bd * kStates + n] = hc[n];
    }
  } else {
    // sum of dt over the chunk (all lanes), for the chunk carry
    float s = lane_broadcast(wave_inclusive_sum(sdt_total), kWaveLanes - 1);
    asm volatile("" : "+s"(s));  // formed by the whole wave, then stored by lane 0
    if (lane == 0) {
      const int64_t base = bd * p.n_chunks + chunk;
#pragma unroll
      for (int n = 0; n < kStates; ++n) p.ws_H[base * kStates + n] = hc[n];
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

template <typename T, bool kVec>
hipError_t launch_scan_t(const ScanArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.dim + kChannelsPerGroup - 1) /
                                        kChannelsPerGroup),
                  static_cast<unsigned>(a.batch),
                  static_cast<unsigned>(a.n_chunks));
  // (conv prologue, softplus, ZOH) -> kernel instance
  using KernelFn = void (*)(ScanArgs);
  static constexpr KernelFn kernels[8] = {
      scan_kernel<T, kVec, false, false, false>, scan_kernel<T, kVec, true, false, false>,
      scan_kernel<T, kVec, false, true, false>,  scan_kernel<T, kVec, true, true, false>,
      scan_kernel<T, kVec, false, false, true>,  scan_kernel<T, kVec, true, false, true>,
      scan_kernel<T, kVec, false, true, true>,   scan_kernel<T, kVec, true, true, true>};
  const int which = (a.softplus ? 1 : 0) | (a.x ? 2 : 0) | (a.zoh ? 4 : 0);
  // the backward's checkpoint pass (Euler, no conv prologue, unsplit) has
  // instances of its own, so the forward instances carry none of its code
  static constexpr KernelFn ckpt_kernels[2] = {scan_kernel<T, kVec, false, false, false, true>,
                                               scan_kernel<T, kVec, true, false, false, true>};
  hipLaunchKernelGGL(a.ckpt ? ckpt_kernels[a.softplus ? 1 : 0] : kernels[which], grid,
                     dim3(kWaveLanes * kWavesPerGroup), 0, s, a);
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

}  // namespace

int launch_scan(const ScanArgs &a, bool bf16, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch_scan_t<uint16_t, true>(a, s) : launch_scan_t<uint16_t, false>(a, s);
  return vec ? launch_scan_t<float, true>(a, s) : launch_scan_t<float, false>(a, s);
}

const char *hip_error_string(int err) {
  return hipGetErrorString(static_cast<hipError_t>(err));
}

}  // namespace ssm
