// ssm_bwd.hip -- gfx950 (CDNA4) kernels of the selective scan's backward
// pass (Euler or exact zero-order-hold input term).
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
// (no atomics: deterministic) and adds them into its slot's partial-sum row
// (the sweep runs as several launches in a row, each giving every slot its
// next channel group), and a reduction kernel sums the slots' rows.
//
// Sequence split (few channels, long sequences): the tokens are cut into
// block-aligned chunks swept in parallel.  The reverse recurrence is linear
// in what enters a chunk from its right, so bwd_adj_kernel first finds, for
// each chunk after the first, what it passes to its left from a zero right
// input and its decay product (over its decay horizon only), and
// bwd_adj_carry_kernel chains those from the last chunk to the first; each
// chunk's sweep then starts from its true incoming dL/dh.  The checkpoints
// come from the checkpoint pass, split the same way as the forward.
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

// The flush's share of thread tid (after every wave has written its region
// for a state): 4 consecutive tokens of one matrix (the first half of the
// threads dB, the second dC: wave-uniform) in one lane run.  Runs of K
// tokens (fewer than 16 in a short partial block): threads whose 4 tokens
// lie past the run have nothing to write.
constexpr int kFlushPer = 2 * kTokensPerLane * kWaveLanes / kBwdThreads;  // 4
struct FlushPos {
  int mat, run, j0;
  bool active;
};
template <int K>
__device__ __forceinline__ FlushPos flush_pos(int tid) {
  constexpr int kParts = kTokensPerLane / kFlushPer;  // per run
  FlushPos f;
  f.mat = tid / (kBwdThreads / 2);
  const int r = tid % (kBwdThreads / 2);
  f.run = r / kParts;
  f.j0 = (r % kParts) * kFlushPer;
  f.active = K == kTokensPerLane || f.j0 < K;
  return f;
}

// Sums the channels' contributions (in channel order) to its 4 tokens,
// adds them to what the slot's earlier channel groups left in its
// partial-sum row (prev, zeros for the slot's first group) and writes the
// row (a 16-byte store when kVec; the partial block through the buffer
// view).
template <bool kVec, bool kFull, int K = kTokensPerLane>
__device__ __forceinline__ void flush_state(const float *sR, const FlushPos &f,
                                            const float (&prev)[kFlushPer], float *pB_row,
                                            float *pC_row, int64_t t0, int64_t tend) {
  if (!f.active) return;
  float v[kFlushPer];
#pragma unroll
  for (int jj = 0; jj < kFlushPer; ++jj) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kBwdWaves; ++w) acc += sR[region_index(w, f.mat, f.j0 + jj, f.run)];
    v[jj] = prev[jj] + acc;
  }
  float *row = f.mat ? pC_row : pB_row;
  store_run<float, kFlushPer, kVec, kFull>(row, t0, t0 + f.run * K + f.j0, tend, v);
}

// Per-state values of one channel (wave-uniform), state n in lane n % 64
// of register n / 64 of kR vector registers (up to 64 kR states) rather
// than N scalar registers; the register of a state is picked by the
// wave-uniform n.
template <int kR>
struct PerState {
  float v[kR];
};
template <int kR>
__device__ __forceinline__ float state_of(const PerState<kR> &s, int n) {
  if constexpr (kR == 1) {
    return lane_broadcast(s.v[0], n);
  } else {
    const int k = n >> 6, l = n & 63;
    float r = lane_broadcast(s.v[0], l);
#pragma unroll
    for (int i = 1; i < kR; ++i) r = k == i ? lane_broadcast(s.v[i], l) : r;
    return r;
  }
}
// x must be wave-uniform and already formed by the whole wave
template <int kR>
__device__ __forceinline__ void set_state(PerState<kR> &s, int lane, int n, float x) {
  if constexpr (kR == 1) {
    s.v[0] = lane == n ? x : s.v[0];
  } else {
    const int k = n >> 6, l = n & 63;
#pragma unroll
    for (int i = 0; i < kR; ++i) s.v[i] = (k == i && lane == l) ? x : s.v[i];
  }
}
template <int kR>
__device__ __forceinline__ void add_state(PerState<kR> &s, int lane, int n, float x) {
  if constexpr (kR == 1) {
    s.v[0] += lane == n ? x : 0.0f;
  } else {
    const int k = n >> 6, l = n & 63;
#pragma unroll
    for (int i = 0; i < kR; ++i) s.v[i] += (k == i && lane == l) ? x : 0.0f;
  }
}

// One block of one channel, in reverse.  hfv: the forward states entering
// the block (checkpoint); muv: dL/dh flowing in from the right of the block
// (replaced by what flows out of its first token); dAv: running dA sums of
// the channel (already times 1/ln2); all per state as PerState<kR>.
// K: tokens per lane.  Full blocks use kTokensPerLane; the partial last
// block uses the fewest of 4, 8, 16 that cover it, so its loops cost about
// its share of a block.
template <typename T, bool kVec, bool kFull, bool kSoftplus, bool kZoh, int kR,
          int K = kTokensPerLane>
__device__ __forceinline__ void bwd_block(
    const BwdArgs &p, int wave, int lane, int64_t t0, int64_t tend, int64_t b,
    int64_t bd, int64_t slot, bool accum, const T *__restrict__ Bb, const T *__restrict__ Cb,
    bool ch_ok, float bias, float Dd, const PerState<kR> &Av, const PerState<kR> &hfv,
    PerState<kR> &muv, PerState<kR> &dAv, float &dDl, float &dbl, float *sT, float *sR,
    int tid) {
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
  float *pBg = p.pB + (b * p.slots + slot) * p.N * p.L;  // this slot's partial rows
  float *pCg = p.pC + (b * p.slots + slot) * p.N * p.L;
  const FlushPos fp = flush_pos<K>(tid);
  const int64_t tf = t0 + fp.run * K + fp.j0;  // the flush's first token
  TileRun<T, kQuarterRun, kVec, kFull> run;
  if (stager) run.load(src, t0, tq, tend);  // state 0

  // per token: dt (as dt*log2 e), dt*u, the gated output gradient gc and
  // the sums over states s1 = sum lambda B, s2 = sum lambda a h_prev A;
  // kept for the end of the block: us = u * sigmoid(delta + bias) and sg =
  // sigmoid(delta + bias) (the derivative of softplus; u and 1 without
  // softplus).  The gate's gradient dz needs nothing from the state loop
  // and is formed and stored here.
  float dtl[K], du[K], gc[K], s1[K], s2[K], us[K], sg[K];
  float sdt = 0.0f;
  {
    float uu[K], dr[K];
    load_run<T, K, kVec, kFull>(urow, t0, tl, tend, uu);
    load_run<T, K, kVec, kFull>(drow, t0, tl, tend, dr);
    load_run<T, K, kVec, kFull>(gyrow, t0, tl, tend, gc);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float x = dr[j] + bias;
      float v = x, sgm = 1.0f;
      if constexpr (kSoftplus) {
        // softplus_f with its terms kept: e = exp(-|x|), w = 1 + e;
        // sigmoid(x) = 1/w for x >= 0 and e/w below
        const float e = fast_exp2(-fabsf(x) * kLog2e);
        const float w = 1.0f + e;
        const float r = e - (w - 1.0f);
        v = fmaxf(x, 0.0f) + fmaf(__builtin_amdgcn_logf(w), kLn2, r);
        sgm = (x >= 0.0f ? 1.0f : e) * __builtin_amdgcn_rcpf(w);
      }
      if (!kFull) v = (tl + j < tend) ? v : 0.0f;  // identity step
      dtl[j] = v * kLog2e;
      du[j] = kZoh ? uu[j] : v * uu[j];  // ZOH: the coefficient carries dt
      sdt += v;
      us[j] = uu[j] * sgm;
      sg[j] = sgm;
      s1[j] = 0.0f;
      s2[j] = 0.0f;
    }
    if (zrow) {
      float zz[K];
      load_run<T, K, kVec, kFull>(zrow, t0, tl, tend, zz);
      if (p.dz) {
        // dz = dy * yc * silu'(z), yc the pre-gate output the checkpoint
        // pass stored; silu'(z) = sigmoid(z) (1 + z (1 - sigmoid(z)))
        float yv[K];
        load_run<T, K, kVec, kFull>(static_cast<const T *>(p.yc) + bd * p.L, t0, tl, tend, yv);
#pragma unroll
        for (int j = 0; j < K; ++j) {
          const float sz = sigmoid_f(zz[j]);
          yv[j] = gc[j] * yv[j] * (sz * fmaf(zz[j], 1.0f - sz, 1.0f));
          gc[j] *= zz[j] * sz;  // dy * silu(z)
        }
        if (ch_ok)
          store_run<T, K, kVec, kFull>(static_cast<T *>(p.dz) + bd * p.L, t0, tl, tend, yv);
      } else {
#pragma unroll
        for (int j = 0; j < K; ++j) gc[j] *= silu_f(zz[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < K; ++j) dDl = fmaf(gc[j], uu[j], dDl);
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
  for (int n = 0; n < p.N; ++n) {
    if (stager && n + 1 < p.N) run.load(src + (n + 1) * p.L, t0, tq, tend);
    // what the slot's earlier channel groups summed for this state's tokens,
    // requested now and added at the flush, after the state's work
    float prev[kFlushPer] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (accum && fp.active)
      load_run<float, kFlushPer, kVec, kFull>((fp.mat ? pCg : pBg) + n * p.L, t0, tf, tend, prev);
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
    const float inv_a = kZoh ? 1.0f / An : 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float arg = dtl[j] * An;
      a[j] = fast_exp2(arg);
      // the input term (dt B u, or the ZOH coefficient times B u), replaced
      // by the state below
      hs[j] = kZoh ? zoh_coeff(arg, a[j], dtl[j], inv_a) * (du[j] * bv[j]) : du[j] * bv[j];
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
    set_state(muv, lane, n, mu_out);
    float m = wave_reverse(wave_shift_in(Mr, mun), lane);
    // reverse replay: lambda_j = dL/dh_j, then the gradients of token j
    float dA_acc = 0.0f;
#pragma unroll
    for (int j = K - 1; j >= 0; --j) {
      const float lam = fmaf(gc[j], cv[j], m);
      const float hprev = j > 0 ? hs[j - 1] : hin;
      m = a[j] * lam;                                  // lambda a
      const float q = m * hprev;                       // lambda a h_{j-1}
      dA_acc = fmaf(q, dtl[j], dA_acc);
      if constexpr (kZoh) {
        // c = (exp(dt A) - 1)/A recomputed; dc/ddt = a, dc/dA = (dt a -
        // c)/A, or dt^2 (1/2 + x/3 + x^2/8 + x^3/30), x = dt A, where |dt
        // A| < 2^-5 ln2 (the series branch of zoh_coeff); here du = u
        const float arg = dtl[j] * An;
        const float c = zoh_coeff(arg, a[j], dtl[j], inv_a);
        const float bu = bv[j] * du[j];
        s1[j] = fmaf(lam, c * bv[j], s1[j]);            // sum lambda c B
        s2[j] = fmaf(m, fmaf(An, hprev, bu), s2[j]);    // sum lambda a (A h + B u)
        const float dt = dtl[j] * kLn2;
        const float x = arg * kLn2;
        const float ser = dt * dt * fmaf(x, fmaf(x, fmaf(x, 1.0f / 30.0f, 0.125f), 1.0f / 3.0f), 0.5f);
        const float dcda = fabsf(arg) < 0x1p-5f ? ser : (fmaf(dt, a[j], -c) * inv_a);
        dA_acc = fmaf(lam * bu, dcda * kLog2e, dA_acc);  // accumulated in log2 units
        reg[region_index(wave, 0, j, lane)] = lam * (c * du[j]);
      } else {
        s1[j] = fmaf(lam, bv[j], s1[j]);
        s2[j] = fmaf(q, An, s2[j]);
        reg[region_index(wave, 0, j, lane)] = lam * du[j];
      }
      reg[region_index(wave, 1, j, lane)] = gc[j] * hs[j];
    }
    float dA_sum = lane_broadcast(wave_inclusive_sum(dA_acc), kWaveLanes - 1);
    asm volatile("" : "+s"(dA_sum));
    add_state(dAv, lane, n, dA_sum);
    if (stager && n + 1 < p.N) run.store(sT + ((n + 1) & 1) * kBwdTileFloats, toff);
    __syncthreads();  // state n's contributions and state n+1's tile are in LDS
    flush_state<kVec, kFull, K>(reg, fp, prev, pBg + n * p.L, pCg + n * p.L, t0, tend);
  }

  // per-token gradients: du = dt * sum lambda B + gc D, ddelta = (u *
  // sum lambda B + sum lambda a h_prev A) * sigmoid(delta + bias)
#pragma unroll
  for (int j = 0; j < K; ++j) {
    // Euler: ddt = u * sum lambda B + sum lambda a A h_prev, du = dt * sum
    // lambda B; ZOH: ddt = sum lambda a (A h_prev + B u), du = sum lambda c B
    const float dx = kZoh ? s2[j] * sg[j] : fmaf(us[j], s1[j], s2[j] * sg[j]);
    dbl += (kFull || tl + j < tend) ? dx : 0.0f;
    s1[j] = kZoh ? fmaf(gc[j], Dd, s1[j]) : fmaf(dtl[j] * kLn2, s1[j], gc[j] * Dd);  // du
    s2[j] = dx;                                                                        // ddelta
  }
  if (ch_ok) {
    store_run<T, K, kVec, kFull>(static_cast<T *>(p.du) + bd * p.L, t0, tl, tend, s1);
    store_run<T, K, kVec, kFull>(static_cast<T *>(p.ddelta) + bd * p.L, t0, tl, tend, s2);
  }
}

// One channel group g (kBwdWaves channels of batch entry blockIdx.y) over
// chunk blockIdx.z, its dB/dC channel sums added into partial-sum row
// `slot` (accum: an earlier group of the slot has written it).
// kR: vector registers per per-state value (1: up to 64 states; 4: up to 256)
template <typename T, bool kVec, bool kSoftplus, bool kZoh, int kR>
__device__ __forceinline__ void bwd_group(const BwdArgs &p, int64_t g, int64_t slot, bool accum,
                                          float *sT, float *sR) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t b = blockIdx.y;
  const int c = blockIdx.z;  // chunk
  const int64_t d_raw = g * kBwdWaves + wave;
  const bool ch_ok = d_raw < p.dim;
  const int64_t d = ch_ok ? d_raw : p.dim - 1;  // clamped for reads
  const int64_t bd = b * p.dim + d;
  const int64_t bdc = bd * p.n_chunks + c;
  const int N = p.N;
  const int64_t ct0 = static_cast<int64_t>(c) * p.chunk_len;
  const int64_t ct1 = ct0 + p.chunk_len < p.L ? ct0 + p.chunk_len : p.L;

  // per state: A, dL/dh entering the chunk's last token from the right,
  // the dA sums (state n in lane n % 64 of register n / 64; reads clamped)
  PerState<kR> Av, muv, dAv;
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const int n = kWaveLanes * i + lane;
    const int ns = n < N ? n : 0;
    Av.v[i] = p.A[d * N + ns];
    muv.v[i] = p.n_chunks > 1 ? p.mu_in[bdc * N + ns]
                              : (p.dh_final ? p.dh_final[bd * N + ns] : 0.0f);
    dAv.v[i] = 0.0f;
  }
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const float Dd = p.D ? p.D[d] : 0.0f;
  const T *Bb = static_cast<const T *>(p.B) + b * N * p.L;
  const T *Cb = static_cast<const T *>(p.C) + b * N * p.L;
  float dDl = 0.0f, dbl = 0.0f;

  // the chunk's blocks (chunks start on block boundaries; only the last
  // chunk can end in a partial block), last to first
  const float *ck = p.ckpt + (bd * p.nblk + ct0 / kBlockTokens) * N;
  auto ckpt_of = [&](int64_t k) {  // the forward states entering block k
    PerState<kR> h;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int n = kWaveLanes * i + lane;
      h.v[i] = ck[k * N + (n < N ? n : 0)];
    }
    return h;
  };
  const int64_t nfull = (ct1 - ct0) / kBlockTokens;
  const int64_t rem = (ct1 - ct0) - nfull * kBlockTokens;
  if (rem > 0) {  // the partial last block comes first
    const PerState<kR> hf = ckpt_of(nfull);
    const int64_t t0 = ct0 + nfull * kBlockTokens;
    if (rem <= 4 * kWaveLanes)
      bwd_block<T, false, false, kSoftplus, kZoh, kR, 4>(p, wave, lane, t0, ct1, b, bd, slot, accum, Bb, Cb,
                                                     ch_ok, bias, Dd, Av, hf, muv, dAv, dDl,
                                                     dbl, sT, sR, tid);
    else if (rem <= 8 * kWaveLanes)
      bwd_block<T, false, false, kSoftplus, kZoh, kR, 8>(p, wave, lane, t0, ct1, b, bd, slot, accum, Bb, Cb,
                                                     ch_ok, bias, Dd, Av, hf, muv, dAv, dDl,
                                                     dbl, sT, sR, tid);
    else
      bwd_block<T, false, false, kSoftplus, kZoh, kR>(p, wave, lane, t0, ct1, b, bd, slot, accum, Bb, Cb,
                                                  ch_ok, bias, Dd, Av, hf, muv, dAv, dDl, dbl,
                                                  sT, sR, tid);
  }
#pragma unroll 1
  for (int64_t k = nfull - 1; k >= 0; --k)
    bwd_block<T, kVec, true, kSoftplus, kZoh, kR>(p, wave, lane, ct0 + k * kBlockTokens,
                                            ct0 + (k + 1) * kBlockTokens, b, bd, slot, accum, Bb, Cb,
                                            ch_ok, bias, Dd, Av, ckpt_of(k), muv, dAv, dDl,
                                            dbl, sT, sR, tid);

  if (!ch_ok) return;  // (only in the last group: nothing follows it)
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const int n = kWaveLanes * i + lane;
    if (n < N) {
      p.pA[bdc * N + n] = dAv.v[i] * kLn2;  // sum of q * dt = q * dtl * ln2
      if (p.dh0 && c == 0) p.dh0[bd * N + n] = muv.v[i];
    }
  }
  float sD = lane_broadcast(wave_inclusive_sum(dDl), kWaveLanes - 1);
  float sb = lane_broadcast(wave_inclusive_sum(dbl), kWaveLanes - 1);
  asm volatile("" : "+s"(sD), "+s"(sb));  // formed by the whole wave first
  if (lane == 0) {
    p.pD[bdc] = sD;
    p.pbias[bdc] = sb;
  }
}

// Launch `unit` of the sweep: workgroup (slot, b, c) takes channel group
// slot + unit * slots.  The launches run in unit order on one stream, so
// each partial-sum row is a fixed-order sum.
template <typename T, bool kVec, bool kSoftplus, bool kZoh, int kR>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_kernel(BwdArgs p) {
  __shared__ float sT[2 * kBwdTileFloats];  // one state's B, C (fp32), double-buffered
  __shared__ float sR[2 * kRegionFloats];   // dB, dC contributions of the 8 channels, double-buffered
  const int64_t slot = blockIdx.x;
  const int64_t g = slot + p.unit * p.slots;
  if (g >= p.groups) return;  // the whole workgroup
  bwd_group<T, kVec, kSoftplus, kZoh, kR>(p, g, slot, p.unit > 0, sT, sR);
}

// ------------------------------------------- sequence split: adjoints ---
// Chunk c >= 1 swept with nothing entering from its right passes to its
// left neighbour mu0 = sum_t D_t gc_t C_t, D_t = prod_{r = start..t} a_r =
// exp(A S_t) with S_t the chunk's sum of dt up to and including t, and any
// dL/dh mu entering from its right arrives decayed by the chunk's product
// Pc = exp(A S): mu_left = mu0 + Pc mu (the reverse recurrence is linear).
// One wave per (batch, channel, chunk >= 1), 64 tokens per step from the
// chunk start; like the forward's fix-up, it stops once every D_t is below
// 2^-40 when they cannot grow again (all A < 0, dt >= 0 under softplus),
// leaving Pc at that (negligible) value.
template <typename T>
__global__ __launch_bounds__(64) void bwd_adj_kernel(BwdArgs p) {
  constexpr int kG = 16;  // states per pass over the horizon
  const int lane = threadIdx.x;
  const int64_t d = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int c = blockIdx.z + 1;
  const int64_t bd = b * p.dim + d;
  const int N = p.N;
  const int64_t ct0 = static_cast<int64_t>(c) * p.chunk_len;
  const int64_t ct1 = ct0 + p.chunk_len < p.L ? ct0 + p.chunk_len : p.L;
  float amax = -INFINITY;
  for (int n = 0; n < N; ++n) amax = fmaxf(amax, p.A[d * N + n] * kLog2e);
  const bool may_stop = p.softplus && amax < 0.0f;
  const float bias = p.bias ? p.bias[d] : 0.0f;
  const T *drow = static_cast<const T *>(p.delta) + bd * p.L;
  const T *gyrow = static_cast<const T *>(p.dy) + bd * p.L;
  const T *zrow = p.z ? static_cast<const T *>(p.z) + bd * p.L : nullptr;
  const T *Cb = static_cast<const T *>(p.C) + b * N * p.L;
  const int64_t base = (bd * p.n_chunks + c) * N;
  for (int n0 = 0; n0 < N; n0 += kG) {
    float Aq[kG], acc[kG];
#pragma unroll
    for (int n = 0; n < kG; ++n) {
      Aq[n] = n0 + n < N ? p.A[d * N + n0 + n] * kLog2e : 0.0f;
      acc[n] = 0.0f;
    }
    float S = 0.0f;
    for (int64_t t0 = ct0; t0 < ct1; t0 += 64) {
      const int64_t t = t0 + lane;
      const bool in = t < ct1;
      float dt = 0.0f, gc = 0.0f;
      if (in) {
        const float x = to_f32<T>(drow[t]) + bias;
        dt = p.softplus ? softplus_f(x) : x;
        gc = to_f32<T>(gyrow[t]);
        if (zrow) gc *= silu_f(to_f32<T>(zrow[t]));
      }
      const float St = S + wave_inclusive_sum(dt);
#pragma unroll
      for (int n = 0; n < kG; ++n) {
        const float cn = (in && n0 + n < N) ? to_f32<T>(Cb[(n0 + n) * p.L + t]) : 0.0f;
        acc[n] = fmaf(fast_exp2(Aq[n] * St) * gc, cn, acc[n]);
      }
      S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(St), 63));
      if (may_stop && fast_exp2(amax * S) <= 0x1p-40f) break;
    }
#pragma unroll
    for (int n = 0; n < kG; ++n) {
      float m = lane_broadcast(wave_inclusive_sum(acc[n]), kWaveLanes - 1);
      asm volatile("" : "+s"(m));  // formed by the whole wave, then stored by lane 0
      if (lane == 0 && n0 + n < N) {
        p.mu0[base + n0 + n] = m;
        p.Pc[base + n0 + n] = fast_exp2(Aq[n] * S);
      }
    }
  }
}

// One thread per (batch, channel, state): the dL/dh entering each chunk
// from its right, from the last chunk (dh_final) to the first.
__global__ __launch_bounds__(256) void bwd_adj_carry_kernel(BwdArgs p) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int N = p.N;
  if (gid >= p.batch * p.dim * N) return;
  const int64_t bd = gid / N;
  const int n = static_cast<int>(gid - bd * N);
  const int nc = p.n_chunks;
  float mu = p.dh_final ? p.dh_final[gid] : 0.0f;
  for (int c = nc - 1; c >= 1; --c) {
    const int64_t i = (bd * nc + c) * N + n;
    p.mu_in[i] = mu;
    mu = fmaf(p.Pc[i], mu, p.mu0[i]);
  }
  p.mu_in[(bd * nc) * N + n] = mu;
}

// dB[b, n, t] (blockIdx.y = 0) or dC (1): the sum over slots of the
// partial rows.  A workgroup takes 256 consecutive tokens (64 lanes x 4)
// of one (b, n) row; its 4 waves take every 4th slot (16-byte loads, 1 KB
// per wave and slot) and add up in LDS at the end.
constexpr int kReduceWaves = 4;
constexpr int kReduceTokens = 4 * kWaveLanes;  // per workgroup
__global__ __launch_bounds__(kReduceWaves * kWaveLanes) void bwd_reduce_bc_kernel(BwdArgs p) {
  __shared__ float4 red[kReduceWaves - 1][kWaveLanes];
  const int lane = threadIdx.x & 63;
  const int slice = threadIdx.x >> 6;
  const int64_t ntb = (p.L + kReduceTokens - 1) / kReduceTokens;
  const int64_t row = blockIdx.x / ntb;  // b * N + n
  const int64_t t = (blockIdx.x - row * ntb) * kReduceTokens + lane * 4;
  const int64_t b = row / p.N, n = row - b * p.N;
  const float *part = (blockIdx.y ? p.pC : p.pB) + (b * p.slots * p.N + n) * p.L;
  const int64_t gstride = p.N * p.L;
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
    const int64_t ng = (p.slots - slice + kReduceWaves - 1) / kReduceWaves;
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
    for (int64_t gi = slice; gi < p.slots; gi += kReduceWaves) {
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

// dA[d, n], dD[d], dbias[d]: sums over the batch and the chunks of the
// per-(b, d, chunk) partials, in that order.
__global__ __launch_bounds__(256) void bwd_reduce_param_kernel(BwdArgs p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int N = p.N;
  if (i >= p.dim * N) return;
  const int64_t d = i / N;
  const int n = static_cast<int>(i % N);
  const int nc = p.n_chunks;
  float sa = 0.0f;
  for (int64_t b = 0; b < p.batch; ++b)
    for (int c = 0; c < nc; ++c) sa += p.pA[((b * p.dim + d) * nc + c) * N + n];
  p.dA[i] = sa;
  if (n == 0) {
    float sd = 0.0f, sb = 0.0f;
    for (int64_t b = 0; b < p.batch; ++b)
      for (int c = 0; c < nc; ++c) {
        sd += p.pD[(b * p.dim + d) * nc + c];
        sb += p.pbias[(b * p.dim + d) * nc + c];
      }
    if (p.dD) p.dD[d] = sd;
    if (p.dbias) p.dbias[d] = sb;
  }
}

template <typename T, bool kVec>
hipError_t launch_bwd_t(const BwdArgs &a, hipStream_t s) {
  if (a.n_chunks > 1) {
    hipLaunchKernelGGL((bwd_adj_kernel<T>),
                       dim3(static_cast<unsigned>(a.dim), static_cast<unsigned>(a.batch),
                            static_cast<unsigned>(a.n_chunks - 1)),
                       dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nthreads = a.batch * a.dim * a.N;
    hipLaunchKernelGGL(bwd_adj_carry_kernel,
                       dim3(static_cast<unsigned>((nthreads + 255) / 256)), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const dim3 grid(static_cast<unsigned>(a.slots), static_cast<unsigned>(a.batch),
                  static_cast<unsigned>(a.n_chunks));
  using Fn = void (*)(BwdArgs);
  // [more than 64 states][softplus | zoh]
  static constexpr Fn kernels[2][4] = {
      {bwd_kernel<T, kVec, false, false, 1>, bwd_kernel<T, kVec, true, false, 1>,
       bwd_kernel<T, kVec, false, true, 1>, bwd_kernel<T, kVec, true, true, 1>},
      {bwd_kernel<T, kVec, false, false, 4>, bwd_kernel<T, kVec, true, false, 4>,
       bwd_kernel<T, kVec, false, true, 4>, bwd_kernel<T, kVec, true, true, 4>}};
  const Fn sweep = kernels[a.N > kWaveLanes ? 1 : 0][(a.softplus ? 1 : 0) | (a.zoh ? 2 : 0)];
  const int64_t units = (a.groups + a.slots - 1) / a.slots;
  hipError_t e = hipSuccess;
  for (int64_t k = 0; k < units; ++k) {
    BwdArgs ak = a;
    ak.unit = k;
    hipLaunchKernelGGL(sweep, grid, dim3(kBwdThreads), 0, s, ak);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t nwg = a.batch * a.N * ((a.L + kReduceTokens - 1) / kReduceTokens);
  hipLaunchKernelGGL(bwd_reduce_bc_kernel, dim3(static_cast<unsigned>(nwg), 2),
                     dim3(kReduceWaves * kWaveLanes), 0,
                     s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_param_kernel,
                     dim3(static_cast<unsigned>((a.dim * a.N + 255) / 256)), dim3(256), 0,
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
