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
//     while the current one is used), as fp32, shared by the workgroup's 4
//     channels: bf16 rows through registers (widened there), aligned fp32
//     rows of full blocks straight into LDS;
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
#include <mutex>
#include <type_traits>

#include "ssm_device.h"
#include "ssm_internal.h"

// Fixed device scratch of the allocation-free scan entry point: the split
// (chunked) scan's chunk end states, chunk dt sums and incoming states.  Each
// GPU holds its own copy for the life of the process.  In host code this
// name is only a handle for hipGetSymbolAddress: the device address comes
// from scan_scratch() below and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[ssm::kScanScratchBytes];

namespace ssm {
namespace {

using namespace dev;

// Full blocks of fp32 rows whose starts are 16-byte aligned stage B and C
// straight from memory into LDS (buffer loads with an LDS destination): no
// staging registers, no LDS stores.  One staging row of the phase tile (64
// runs of kTokensPerLane floats at the padded stride of kTokensPerLane + 4)
// is 5 such loads of 1 KB (64 lanes x 16 bytes, written to consecutive LDS
// addresses); slot s = 64 i + lane of the row holds quad s % 5 of run s / 5,
// the fifth quad being the stride's padding, filled with a copy of the
// fourth.  bf16 rows keep register staging: the tile is fp32, and widening
// once per workgroup in registers is cheaper than any conversion in LDS.
template <typename T, bool kVec>
constexpr bool kDirectStage = sizeof(T) == 4 && kVec;
constexpr int kDirectLoads = 5;
static_assert(kWaveLanes * (kTokensPerLane + 4) * 4 == kDirectLoads * kWaveLanes * 16,
              "a staging row is kDirectLoads loads of 16 bytes a lane");

// This lane's byte offsets into a block's row for each of the 5 loads.
__device__ __forceinline__ void direct_offsets(int lane, int (&off)[kDirectLoads]) {
#pragma unroll
  for (int i = 0; i < kDirectLoads; ++i) {
    const int s = kWaveLanes * i + lane, q = s % 5;
    off[i] = (s / 5) * kTokensPerLane * 4 + (q < 4 ? q : 3) * 16;
  }
}

// Stages the 1024 floats row[0 .. 1024) into a staging row at `dst` (LDS,
// 16-byte aligned).  `row` and `dst` are wave-uniform.  The loads complete
// in LDS by the next wait for all vector memory operations (every barrier
// of the phase loop waits for them).
__device__ __forceinline__ void stage_row_direct(float *dst, const float *row,
                                                 const int (&off)[kDirectLoads]) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(row), 0, kBlockTokens * 4, kBufferWord3);
#pragma unroll
  for (int i = 0; i < kDirectLoads; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void *)(dst + i * 4 * kWaveLanes), 16,
        off[i], 0, 0, 0);
}

// One block of 1024 tokens of one channel per wave (4 channels of one batch
// entry per workgroup).  kFull: the block lies wholly inside [t0, ct1), so
// nothing is masked; otherwise positions from ct1 on are identity steps
// (dt = 0, u = 0) and are not stored.  hc[n]: the channel's state carried in
// (wave-uniform), replaced by the state after the block.
// The channel's A and carried state (both wave-uniform).  StaticStates:
// the tuned 16 states in scalar registers, indexed by a fully unrolled
// state loop.  LaneStates<kR>: any count up to 64 * kR, state n in lane
// n % 64 of vector register n / 64, read with v_readlane in a state loop
// that is not unrolled (the register is picked by the wave-uniform n).
struct StaticStates {
  static constexpr bool kStatic = true;
  float A[kStates], h[kStates];
  __device__ __forceinline__ float a(int n) const { return A[n]; }
  __device__ __forceinline__ float get(int n) const { return h[n]; }
  __device__ __forceinline__ void set(int n, float v) { h[n] = v; }
};
template <int kR>
struct LaneStates {
  static constexpr bool kStatic = false;
  float Av[kR], hv[kR];
  int lane;
  __device__ __forceinline__ static float pick(const float (&v)[kR], int n) {
    if constexpr (kR == 1) {
      return lane_broadcast(v[0], n);
    } else {
      const int k = n >> 6, l = n & 63;
      float r = lane_broadcast(v[0], l);
#pragma unroll
      for (int i = 1; i < kR; ++i) r = k == i ? lane_broadcast(v[i], l) : r;
      return r;
    }
  }
  __device__ __forceinline__ float a(int n) const { return pick(Av, n); }
  __device__ __forceinline__ float get(int n) const { return pick(hv, n); }
  __device__ __forceinline__ void set(int n, float v) {
    asm volatile("" : "+s"(v));  // a wave-uniform value, formed before the select
    if constexpr (kR == 1) {
      hv[0] = lane == n ? v : hv[0];
    } else {
      const int k = n >> 6, l = n & 63;
#pragma unroll
      for (int i = 0; i < kR; ++i) hv[i] = (k == i && lane == l) ? v : hv[i];
    }
  }
};
// kN: kStates (the tuned instances), kMaxLaneStates (up to 64 states) or
// kMaxStates (up to 256)
constexpr int kMaxLaneStates = kWaveLanes;
template <int kN>
using StatesFor = typename std::conditional<
    kN == kStates, StaticStates, LaneStates<(kN + kWaveLanes - 1) / kWaveLanes>>::type;

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
          bool kZoh, bool kCkpt, int K = kTokensPerLane, typename SS>
__device__ __forceinline__ void scan_block(
    const ScanArgs &p, int wave, int lane, int64_t t0, int64_t ct1,
    const T *__restrict__ Bb, const T *__restrict__ Cb,
    const T *__restrict__ urow, const T *__restrict__ drow,
    const T *__restrict__ zrow, T *__restrict__ yrow, T *__restrict__ ycrow,
    bool ch_ok, float bias, float Dd, SS &S, float *sT,
    float &sdt_total, const float (&wc)[kMaxConv], float cb,
    float (&xc)[kMaxConv - 1], float (&upf)[kTokensPerLane],
    float (&dpf)[kTokensPerLane], bool use_pf, int64_t pf_t0,
    const int (&doff)[kDirectLoads], int64_t next_t0) {
  static_assert(!kFull || K == kTokensPerLane, "full blocks: 16 tokens a lane");
  static_assert(K == 4 || K == 8 || K == 16, "runs of 4, 8 or 16 tokens");
  // padded LDS stride of one lane's run: a lane's 16-byte reads of 8
  // consecutive runs fall on 32 different banks
  constexpr int KP = K == 4 ? 12 : K + 4;
  const int64_t tend = kFull ? t0 + kBlockTokens : ct1;
  const int64_t tl = t0 + static_cast<int64_t>(lane) * K;
  constexpr bool kPf = kPrefetch<T, kVec, kConv, kZoh, kCkpt> && SS::kStatic;
  const int nst = SS::kStatic ? kStates : p.N;  // states
  const int nph = (nst + 1) / 2;                // phases of two states
  constexpr int kTileFloats = 2 * 2 * kWaveLanes * KP;
  // B/C row of state r (an odd count's last phase stages its last row twice)
  auto row = [&](int r) { return SS::kStatic ? r : (r < nst ? r : nst - 1); };

  // Staging role of this wave: state (2*ph + st) of matrix B or C (both
  // wave-uniform, so the row is a valid buffer base in the partial block);
  // this lane: run `lane` of that row.
  const int st = wave >> 1, mat = wave & 1;
  const T *src = mat ? Cb : Bb;
  const int64_t tq = tl;
  const int toff = staging_offset<KP>(wave, lane);
  TileRun<T, K, kVec, kFull> run;
  // Direct staging (full blocks of aligned fp32 rows): the tuned instances
  // request the next block's phase-0 tile during this block's last phase
  // (their phase count is even, so buffer 0 is free then); the others
  // request it here.  Register staging loads phase 0's run here.
  // Either way, when the phase count is odd the previous block's last phase
  // read buffer 0, so a barrier comes first.
  constexpr bool kDirect = kFull && kDirectStage<T, kVec>;
  const float *srcf = reinterpret_cast<const float *>(src);
  float *const sdst = sT + wave * kWaveLanes * KP;  // this wave's staging row
  if constexpr (kDirect && !SS::kStatic) {
    if (nph & 1) __syncthreads();
    stage_row_direct(sdst, srcf + row(st) * p.L + t0, doff);
  } else if constexpr (!kDirect) {
    run.load(src + row(st) * p.L, t0, tq, tend);
  }

  // This lane's tokens: the step dt (kept as dt*log2(e) for exp2), dt*u
  // and the D skip.
  float dtl[K], du[K], y[K];
  float sdt = 0.0f;
  {
    float uu[K], dr[K];
    if (kPf && kFull && use_pf) {
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
    if (kPf && kFull && use_pf) {
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
  // Phase 0's tile: its buffer was last read two phases ago, by every wave
  // (by the previous block's last phase when the phase count is odd).
  if constexpr (!kDirect) {
    if (!SS::kStatic && (nph & 1)) __syncthreads();
    run.store(sT, toff);
  }
  const float sdtl = sdt * kLog2e;
  // u and delta of the full block at pf_t0 (the next one, or this one
  // again when none follows), in flight during this block's state loop
  if constexpr (kPf && kFull) {
    const int64_t tlp = pf_t0 + static_cast<int64_t>(lane) * K;
    load_run<T, K, kVec, true>(urow, pf_t0, tlp, pf_t0 + kBlockTokens, upf);
    load_run<T, K, kVec, true>(drow, pf_t0, tlp, pf_t0 + kBlockTokens, dpf);
  }

  // B and C are staged two states at a time in a double-buffered LDS tile
  // (tile[buffer][state][B|C][lane run][KP]); while the 4 waves compute
  // phase ph, each thread already holds phase ph+1's run in registers.
  // (the tuned instances unroll all 8 phases; the others loop)
  constexpr int kPhaseUnroll = SS::kStatic ? kStates / 2 : 1;
#pragma unroll kPhaseUnroll
  for (int ph = 0; ph < nph; ++ph) {
    if (!kDirect && ph + 1 < nph)
      run.load(src + row(2 * (ph + 1) + st) * p.L, t0, tq, tend);
    __syncthreads();  // phase ph's tile is complete and visible
    if constexpr (kDirect) {
      // the other buffer was last read in phase ph-1, before this barrier
      if (ph + 1 < nph)
        stage_row_direct(sdst + ((ph + 1) & 1) * kTileFloats,
                         srcf + row(2 * (ph + 1) + st) * p.L + t0, doff);
      else if (SS::kStatic)
        stage_row_direct(sdst, srcf + row(st) * p.L + next_t0, doff);
    }
    const float *tile = sT + (ph & 1) * kTileFloats;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const int n = 2 * ph + s2;
      if (!SS::kStatic && n >= nst) break;  // an odd count's last phase
      float An = S.a(n);
      asm volatile("" : "+s"(An));  // keep this state's work after the previous state's
      // ... and schedule it on its own: overlapped with the previous state's
      // replay, the 16 exp arguments found no free registers and shared one
      // temporary (measured ~2 % slower on the Mamba layers)
      __builtin_amdgcn_sched_barrier(0);
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
      const float hcn = S.get(n);
      H = fmaf(P, lane == 0 ? hcn : 0.0f, H);
      wave_affine_scan(P, H);
      // H_i is the true state after lane i's last token; lane i starts from
      // lane i-1's (lane 0 from the carried state) and replays its tokens.
      float h = wave_shift_in(H, hcn);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        h = fmaf(a[j], h, bb[j]);
        y[j] = fmaf(pc[j], h, y[j]);
      }
      S.set(n, lane_broadcast(h, kWaveLanes - 1));
    }
    // Every wave has passed this phase's barrier, so the other buffer (read
    // in phase ph-1) is free: fill it with phase ph+1.
    if (!kDirect && ph + 1 < nph) run.store(sT + ((ph + 1) & 1) * kTileFloats, toff);
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
// workgroups x 40 KB fill a CU's 160 KB of LDS) for bf16 rows, aligned or
// not, with the Euler or the ZOH input term (with each state scheduled on
// its own these fit 128 with at most a few spilled registers, measured on
// the 2.8B layer at 4 against 3: ZOH 264 vs 277 us, unaligned rows 313 vs
// 330 us); 3 (168 VGPRs) for fp32 rows, whose wider loads and the next
// block's u and delta carried in registers need the room (4 without that
// prefetch measured slower).
template <typename T, bool kVec, bool kZoh>
constexpr int kOccupancy = sizeof(T) == 2 ? 4 : 3;

// kN: kStates (the tuned 16-state instances), kMaxLaneStates (any d_state
// up to 64) or kMaxStates (up to 256).
template <typename T, bool kVec, bool kSoftplus, bool kConv, bool kZoh, bool kCkpt = false,
          int kN = kStates>
__global__ __launch_bounds__(kWaveLanes * kWavesPerGroup)
__attribute__((amdgpu_waves_per_eu(kOccupancy<T, kVec, kZoh>)))
void scan_kernel(ScanArgs p) {
  constexpr int KP = kTokensPerLane + 4;
  __shared__ __attribute__((aligned(16))) float sT[2 * 2 * 2 * kWaveLanes * KP];  // 2 buffers x 2 states x B, C

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

  // the channel's A and carried state (wave-uniform)
  using SS = StatesFor<kN>;
  constexpr bool kStatic = SS::kStatic;
  const int N = kStatic ? kStates : p.N;
  SS S;
  if constexpr (kStatic) {
#pragma unroll
    for (int n = 0; n < kStates; ++n) S.A[n] = p.A[d * kStates + n];
#pragma unroll
    for (int n = 0; n < kStates; ++n)
      S.h[n] = (chunk == 0 && p.h0) ? p.h0[bd * kStates + n] : 0.0f;
  } else {
    S.lane = lane;
#pragma unroll
    for (int i = 0; i < int(sizeof(S.hv) / sizeof(float)); ++i) {
      const int n = kWaveLanes * i + lane;
      S.Av[i] = p.A[d * N + (n < N ? n : 0)];  // clamped for reads
      S.hv[i] = (chunk == 0 && p.h0 && n < N) ? p.h0[bd * N + n] : 0.0f;
    }
  }
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;

  const T *urow = static_cast<const T *>(kConv ? p.x : p.u) + bd * p.L;
  const T *drow = static_cast<const T *>(p.delta) + bd * p.L;
  const T *zrow = p.z ? static_cast<const T *>(p.z) + bd * p.L : nullptr;
  T *yrow = static_cast<T *>(p.y) + bd * p.L;
  T *ycrow = (kCkpt && p.yc) ? static_cast<T *>(p.yc) + bd * p.L : nullptr;
  const T *Bb = static_cast<const T *>(p.B) + b * N * p.L;
  const T *Cb = static_cast<const T *>(p.C) + b * N * p.L;
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

  // checkpoint instance (kCkpt): the state entering block k goes to
  // ckpt[b, d, k, :]; with p.yc the pre-gate output goes there as well (the
  // backward's own checkpoint pass runs without a gate and takes y itself
  // as the pre-gate output).  Split into chunks (block-aligned), a chunk >= 1
  // starts from a zero state; its blocks' sums of dt since the chunk start
  // go to ckpt_s, from which ckpt_fix_kernel adds the true incoming state.
  const int64_t nblk = (p.L + kBlockTokens - 1) / kBlockTokens;
  float *ck = (kCkpt && ch_ok) ? p.ckpt + bd * nblk * N : nullptr;
  auto store_ckpt = [&](int64_t t0) {
    if (kCkpt && ck) {
      if (p.ckpt_s) {
        float s = lane_broadcast(wave_inclusive_sum(sdt_total), kWaveLanes - 1);
        asm volatile("" : "+s"(s));  // formed by the whole wave, then stored by lane 0
        if (lane == 0) p.ckpt_s[bd * nblk + t0 / kBlockTokens] = s;
      }
      if constexpr (kStatic) {
        if (lane == 0) {
#pragma unroll
          for (int n = 0; n < kStates; ++n) ck[(t0 / kBlockTokens) * kStates + n] = S.h[n];
        }
      } else {
#pragma unroll
        for (int i = 0; i < int(sizeof(S.hv) / sizeof(float)); ++i) {
          const int n = kWaveLanes * i + lane;
          if (n < N) ck[(t0 / kBlockTokens) * N + n] = S.hv[i];
        }
      }
    }
  };

  int doff[kDirectLoads];  // direct staging: this lane's load offsets
  direct_offsets(lane, doff);
  float upf[kTokensPerLane], dpf[kTokensPerLane];  // prefetched u, delta
  const int64_t last_full = ct0 + ((ct1 - ct0) / kBlockTokens - 1) * kBlockTokens;
  int64_t t0 = ct0;
  // direct staging in the tuned instances: the first full block's phase-0
  // tile is requested here, every later one by the block before it
  constexpr bool kDirectNext = kDirectStage<T, kVec> && kStatic;
  const bool any_full = ct0 + kBlockTokens <= ct1;  // the same in every wave
  if (kDirectNext && any_full)
    stage_row_direct(sT + wave * kWaveLanes * KP,
                     reinterpret_cast<const float *>((wave & 1) ? Cb : Bb) +
                         (wave >> 1) * p.L + ct0,
                     doff);
#pragma unroll 1
  for (; t0 + kBlockTokens <= ct1; t0 += kBlockTokens) {
    store_ckpt(t0);
    // the block whose phase-0 tile this block's last phase requests: the
    // next one, or (a valid source that nothing reads) this one again
    const int64_t next_t0 = t0 + 2 * kBlockTokens <= ct1 ? t0 + kBlockTokens : t0;
    scan_block<T, kVec, true, kSoftplus, kConv, kZoh, kCkpt>(
        p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd, S,
        sT, sdt_total, wc, cb, xc,
        upf, dpf, t0 > ct0,
        t0 + 2 * kBlockTokens <= ct1 ? t0 + kBlockTokens : last_full, doff, next_t0);
  }
  // the last full block's extra request lands before LDS is written again
  // or released
  if (kDirectNext && any_full) __syncthreads();
  if (t0 < ct1) store_ckpt(t0);
  if (t0 < ct1) {
    // the last, partial block: branch-free scalar loads (keeps the register
    // budget of the full-block loop), as few tokens per lane as cover it
    const int64_t rem = ct1 - t0;
    if (rem <= 4 * kWaveLanes)
      scan_block<T, false, false, kSoftplus, kConv, kZoh, kCkpt, 4>(
          p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd,
          S, sT, sdt_total, wc, cb, xc, upf, dpf, false, t0, doff, t0);
    else if (rem <= 8 * kWaveLanes)
      scan_block<T, false, false, kSoftplus, kConv, kZoh, kCkpt, 8>(
          p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd,
          S, sT, sdt_total, wc, cb, xc, upf, dpf, false, t0, doff, t0);
    else
      scan_block<T, false, false, kSoftplus, kConv, kZoh, kCkpt>(
          p, wave, lane, t0, ct1, Bb, Cb, urow, drow, zrow, yrow, ycrow, ch_ok, bias, Dd,
          S, sT, sdt_total, wc, cb, xc, upf, dpf, false, t0, doff, t0);
  }

  if (!ch_ok) return;
  // the state after the chunk: the final state, or the chunk's end state
  // (from its own start) and dt sum for the chunk carry
  float *hout = p.n_chunks == 1 ? p.h_final
                                : p.ws_H + (bd * p.n_chunks + chunk) * N;
  if (p.n_chunks > 1) {
    float s = lane_broadcast(wave_inclusive_sum(sdt_total), kWaveLanes - 1);
    asm volatile("" : "+s"(s));  // formed by the whole wave, then stored by lane 0
    if (lane == 0) p.ws_S[bd * p.n_chunks + chunk] = s;
  } else if (hout) {
    hout += bd * N;
  }
  if (hout) {
    if constexpr (kStatic) {
      if (lane == 0) {
#pragma unroll
        for (int n = 0; n < kStates; ++n) hout[n] = S.h[n];
      }
    } else {
#pragma unroll
      for (int i = 0; i < int(sizeof(S.hv) / sizeof(float)); ++i) {
        const int n = kWaveLanes * i + lane;
        if (n < N) hout[n] = S.hv[i];
      }
    }
  }
}

// ------------------------------------------------------ chunk carry -----
// One thread per (batch, channel, state): chains the chunks' end states in
// order, h_in[c+1] = exp(A * sum_dt[c]) * h_in[c] + H[c], and records each
// chunk's incoming state; the last one is the sequence's final state.
__global__ __launch_bounds__(256) void carry_kernel(ScanArgs p) {
  const int N = p.N;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= p.batch * p.dim * N) return;
  const int64_t bd = gid / N;
  const int n = static_cast<int>(gid - bd * N);
  const int64_t d = bd % p.dim;
  const float Aq = p.A[d * N + n] * kLog2e;
  const int nc = p.n_chunks;
  float h = p.ws_H[(bd * nc) * N + n];
  for (int c = 1; c < nc; ++c) {
    p.ws_hin[(bd * nc + c) * N + n] = h;
    h = fmaf(fast_exp2(Aq * p.ws_S[bd * nc + c]), h, p.ws_H[(bd * nc + c) * N + n]);
  }
  if (p.h_final) p.h_final[bd * N + n] = h;
}

// --------------------------------------------------- chunk fix-up -------
// For chunk c >= 1 (scanned from a zero state), adds the part of y that its
// true incoming state contributes: y_t += silu(z_t) * sum_n C_t,n *
// exp(A_n * S_t) * h_in,n, S_t = running sum of dt inside the chunk.  One
// wave per (batch, channel, chunk), 64 tokens per step.  Stops once every
// decay factor is below 2^-40 when the factors cannot grow again (all A < 0
// and dt >= 0); otherwise covers the whole chunk.  kN = kStates keeps the
// 16 states' A and h_in in registers; kN = 0 (any other count) reads them
// per state from memory (wave-uniform scalar loads).
template <typename T, int kN>
__global__ __launch_bounds__(64) void fixup_kernel(ScanArgs p) {
  constexpr bool kStatic = kN == kStates;
  const int N = kStatic ? kStates : p.N;
  const int lane = threadIdx.x;
  const int64_t d = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int c = blockIdx.z + 1;
  const int64_t bd = b * p.dim + d;
  const int64_t ct0 = static_cast<int64_t>(c) * p.chunk_len;
  const int64_t ct1 = ct0 + p.chunk_len < p.L ? ct0 + p.chunk_len : p.L;
  float Aq[kStatic ? kStates : 1], hin[kStatic ? kStates : 1];
  float amax = -INFINITY;
  const float *Arow = p.A + d * N;
  const float *hrow = p.ws_hin + (bd * p.n_chunks + c) * N;
  if constexpr (kStatic) {
#pragma unroll
    for (int n = 0; n < kStates; ++n) {
      Aq[n] = Arow[n] * kLog2e;
      hin[n] = hrow[n];
      amax = fmaxf(amax, Aq[n]);
    }
  } else {
    for (int n = 0; n < N; ++n) amax = fmaxf(amax, Arow[n] * kLog2e);
  }
  const bool may_stop = p.softplus && amax < 0.0f;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const T *drow = static_cast<const T *>(p.delta) + bd * p.L;
  const T *zrow = p.z ? static_cast<const T *>(p.z) + bd * p.L : nullptr;
  const T *Cb = static_cast<const T *>(p.C) + b * N * p.L;
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
    if constexpr (kStatic) {
#pragma unroll
      for (int n = 0; n < kStates; ++n) {
        const float cn = in ? to_f32<T>(Cb[n * p.L + t]) : 0.0f;
        corr = fmaf(cn, fast_exp2(Aq[n] * St) * hin[n], corr);
      }
    } else {
      for (int n = 0; n < N; ++n) {
        const float cn = in ? to_f32<T>(Cb[n * p.L + t]) : 0.0f;
        corr = fmaf(cn, fast_exp2(Arow[n] * kLog2e * St) * hrow[n], corr);
      }
    }
    if (in) {
      const float g = zrow ? silu_f(to_f32<T>(zrow[t])) : 1.0f;
      yrow[t] = from_f32<T>(fmaf(g, corr, to_f32<T>(yrow[t])));
    }
    S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(St), 63));
    if (may_stop && fast_exp2(amax * S) <= 0x1p-40f) break;
  }
}

// ------------------------------------------- checkpoint fix-up ------
// Checkpoint pass in split mode: a block of chunk c >= 1 stored the state
// reached from a zero state at the chunk start; the true one adds the
// chunk's incoming state carried over the block's dt sum S since the chunk
// start: ckpt += exp(A_n * S) * h_in(c)_n (the first block: S = 0, so the
// incoming state itself).  One thread per (batch, channel, block, state)
// over the blocks of chunks >= 1.
__global__ __launch_bounds__(256) void ckpt_fix_kernel(ScanArgs p) {
  const int N = p.N;
  const int64_t nblk = (p.L + kBlockTokens - 1) / kBlockTokens;
  const int64_t bpc = p.chunk_len / kBlockTokens;  // blocks per chunk
  const int64_t nfix = nblk - bpc;                 // blocks of chunks >= 1
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (gid >= p.batch * p.dim * nfix * N) return;
  const int64_t r = gid / N;
  const int n = static_cast<int>(gid - r * N);
  const int64_t k = bpc + r % nfix;
  const int64_t bd = r / nfix;
  const int64_t c = k / bpc;
  const float Aq = p.A[(bd % p.dim) * N + n] * kLog2e;
  const float hin = p.ws_hin[(bd * p.n_chunks + c) * N + n];
  float *q = p.ckpt + (bd * nblk + k) * N + n;
  *q = fmaf(fast_exp2(Aq * p.ckpt_s[bd * nblk + k]), hin, *q);
}

template <typename T, bool kVec, int kN>
hipError_t launch_scan_t(const ScanArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.dim + kChannelsPerGroup - 1) /
                                        kChannelsPerGroup),
                  static_cast<unsigned>(a.batch),
                  static_cast<unsigned>(a.n_chunks));
  // (conv prologue, softplus, ZOH) -> kernel instance
  using KernelFn = void (*)(ScanArgs);
  static constexpr KernelFn kernels[8] = {
      scan_kernel<T, kVec, false, false, false, false, kN>,
      scan_kernel<T, kVec, true, false, false, false, kN>,
      scan_kernel<T, kVec, false, true, false, false, kN>,
      scan_kernel<T, kVec, true, true, false, false, kN>,
      scan_kernel<T, kVec, false, false, true, false, kN>,
      scan_kernel<T, kVec, true, false, true, false, kN>,
      scan_kernel<T, kVec, false, true, true, false, kN>,
      scan_kernel<T, kVec, true, true, true, false, kN>};
  const int which = (a.softplus ? 1 : 0) | (a.x ? 2 : 0) | (a.zoh ? 4 : 0);
  // the backward's checkpoint pass (no conv prologue) has instances of its
  // own, so the forward instances carry none of its code
  static constexpr KernelFn ckpt_kernels[4] = {
      scan_kernel<T, kVec, false, false, false, true, kN>,
      scan_kernel<T, kVec, true, false, false, true, kN>,
      scan_kernel<T, kVec, false, false, true, true, kN>,
      scan_kernel<T, kVec, true, false, true, true, kN>};
  hipLaunchKernelGGL(a.ckpt ? ckpt_kernels[(a.softplus ? 1 : 0) | (a.zoh ? 2 : 0)]
                            : kernels[which], grid,
                     dim3(kWaveLanes * kWavesPerGroup), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_chunks == 1) return e;
  const int64_t nthreads = a.batch * a.dim * a.N;
  hipLaunchKernelGGL(carry_kernel, dim3(static_cast<unsigned>((nthreads + 255) / 256)),
                     dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fgrid(static_cast<unsigned>(a.dim), static_cast<unsigned>(a.batch),
                   static_cast<unsigned>(a.n_chunks - 1));
  constexpr int kFixN = kN == kStates ? kStates : 0;
  hipLaunchKernelGGL((fixup_kernel<T, kFixN>), fgrid, dim3(64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || !a.ckpt) return e;
  if (a.yc) {
    // the saving forward's pre-gate output, fixed up the same way
    ScanArgs ac = a;
    ac.y = a.yc;
    ac.z = nullptr;
    hipLaunchKernelGGL((fixup_kernel<T, kFixN>), fgrid, dim3(64), 0, s, ac);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nblk = (a.L + kBlockTokens - 1) / kBlockTokens;
  const int64_t nfix = a.batch * a.dim * (nblk - a.chunk_len / kBlockTokens) * a.N;
  hipLaunchKernelGGL(ckpt_fix_kernel, dim3(static_cast<unsigned>((nfix + 255) / 256)),
                     dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, bool kVec>
hipError_t launch_scan_n(const ScanArgs &a, hipStream_t s) {
  if (a.N == kStates) return launch_scan_t<T, kVec, kStates>(a, s);
  if (a.N <= kMaxLaneStates) return launch_scan_t<T, kVec, kMaxLaneStates>(a, s);
  return launch_scan_t<T, kVec, kMaxStates>(a, s);
}

}  // namespace

int launch_scan(const ScanArgs &a, bool bf16, bool vec, void *stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (bf16)
    return vec ? launch_scan_n<uint16_t, true>(a, s) : launch_scan_n<uint16_t, false>(a, s);
  return vec ? launch_scan_n<float, true>(a, s) : launch_scan_n<float, false>(a, s);
}

// Device address of `scratch` on the device that `stream` belongs to (the
// current device for the null stream), looked up once per device with that
// device current and kept.
int scan_scratch(void *stream, void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex m;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                        : hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(m);
  if (!addr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return static_cast<int>(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return static_cast<int>(e);
    void *p = nullptr;
    const hipError_t eg = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return static_cast<int>(e);
    if (eg != hipSuccess) return static_cast<int>(eg);
    if (!p) return static_cast<int>(hipErrorInvalidSymbol);
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

const char *hip_error_string(int err) {
  return hipGetErrorString(static_cast<hipError_t>(err));
}

}  // namespace ssm
