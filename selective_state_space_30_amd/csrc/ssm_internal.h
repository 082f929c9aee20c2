// ssm_internal.h -- launch interface between the C-ABI layer (ssm_api.cpp)
// and the gfx950 kernels (ssm_kernels.hip).  Not installed; not part of the
// public ABI in include/ssm_scan.h.
#pragma once

#include <cstddef>
#include <cstdint>

namespace ssm {

constexpr int kStates = 16;          // d_state supported by this build
constexpr int kWaveLanes = 64;       // one channel per 64-lane wave
constexpr int kWavesPerGroup = 4;    // waves (channels) per workgroup
constexpr int kChannelsPerGroup = kWavesPerGroup;                  // 4
constexpr int kTokensPerLane = 16;   // consecutive tokens owned by one lane
constexpr int kBlockTokens = kWaveLanes * kTokensPerLane;         // 1024
constexpr int kPhaseStates = 2;      // states per double-buffered B/C LDS tile
constexpr int kMaxConv = 4;          // taps of the fused causal conv1d prologue
constexpr int kBwdWaves = 8;         // waves (channels) per backward workgroup

struct ScanArgs {
  const void *u, *delta, *B, *C, *z;  // activations (dtype); u null with conv
  const void *x;                      // conv prologue: pre-conv input (dtype)
  const float *conv_w, *conv_b;       // conv prologue: (dim, d_conv), (dim)
  int d_conv;                         // conv prologue taps (1..4), 0 = none
  const float *A, *D, *bias, *h0;     // fp32 parameters / initial state
  void *y;                            // output (dtype)
  float *h_final;                     // fp32 (batch, dim, 16) or null
  float *ws_H;                        // split mode: chunk end states (b,d,c,n)
  float *ws_S;                        // split mode: chunk sums of dt (b,d,c)
  float *ws_hin;                      // split mode: chunk incoming states (b,d,c,n)
  int64_t batch, dim, L;
  int64_t chunk_len;                  // tokens per chunk (== L when not split)
  int n_chunks;
  int softplus;                       // 1: dt = softplus(delta + bias)
  int zoh;                            // 1: exact ZOH input term
  float *ckpt;                        // backward's checkpoint pass: the state
                                      // at every block start, (batch, dim,
                                      // ceil(L/1024), 16)
  void *yc;                           // with ckpt: the pre-gate output (dtype),
                                      // or null
};

// Backward pass.  Per-workgroup partial sums (a workgroup = kBwdWaves
// channels of one batch entry) are reduced by a second kernel.
struct BwdArgs {
  const void *u, *delta, *B, *C, *z, *dy;  // activation dtype
  const float *A, *D, *bias, *h0, *dh_final;
  const float *ckpt;                  // (batch, dim, nblk, 16) forward states
  const void *yc;                     // (batch, dim, L) pre-gate output, dtype
  void *dz;                           // activation dtype output, or null
  void *du, *ddelta;                  // activation dtype outputs
  float *dh0;                         // (batch, dim, 16) or null
  float *pB, *pC;                     // (batch, groups, 16, L) partial dB, dC
  float *pA;                          // (batch, dim, 16) partial dA
  float *pD, *pbias;                  // (batch, dim) partial dD, dbias
  float *dA, *dB, *dC, *dD, *dbias;   // reduced outputs (dD, dbias: or null)
  int64_t batch, dim, L;
  int64_t groups;                     // ceil(dim / kBwdWaves)
  int nblk;                           // ceil(L / 1024)
  int softplus;
};

// Mamba-2 SSD forward (one scalar decay per head; bf16 activations).
constexpr int kSsdChunk = 64;        // tokens per chunk
constexpr int kSsdHeadDim = 64;      // rows (headdim) per head
struct SsdArgs {
  const void *x, *dt, *B, *C, *z;     // bf16: (b,h,P,L), (b,h,L), (b,g,N,L) x2, (b,h,P,L)
  const float *A, *D, *dt_bias, *h0;  // (h), (h), (h), (b,h,P,N)
  void *y;                            // bf16 (b,h,P,L)
  float *h_final;                     // (b,h,P,N) or null
  void *G;                            // workspace: bf16 (b,g,chunk,2,64,64) causal C^T B, hi and lo
  void *Ct;                           // workspace: bf16 (b,g,chunk,64,N) C transposed
  int64_t batch, nheads, ngroups, L;
  int nchunks, dstate;
  int softplus;
};

struct StepArgs {
  float *state;
  const void *x, *delta, *B, *C, *z;
  const float *A, *D, *bias;
  void *y;
  int64_t batch, dim;
  int softplus;
  int zoh;
  // conv prologue (d_conv > 0): u = silu(conv_b + sum_k conv_w[d, k] *
  // window_k) over the d_conv - 1 inputs kept in conv_state and x; the
  // state's window is shifted in place
  void *conv_state;                   // (batch, dim, d_conv - 1), dtype
  const float *conv_w, *conv_b;       // (dim, d_conv), (dim)
  int d_conv;                         // 1..4, 0 = no prologue
};

// Workspace layout of the split (chunked) scan, in floats, each part
// starting on a 256-byte boundary.
struct SplitLayout {
  size_t off_H, off_S, off_hin, total_bytes;
};
SplitLayout split_layout(int64_t batch, int64_t dim, int64_t n_chunks);

// Kernel launchers.  Return a hipError_t value as int (0 = success).
// `vec` selects 16-byte vector loads (the caller has checked alignment).
int launch_scan(const ScanArgs &a, bool bf16, bool vec, void *stream);
int launch_step(const StepArgs &a, bool bf16, bool vec, void *stream);
int launch_bwd(const BwdArgs &a, bool bf16, bool vec, void *stream);
int launch_ssd(const SsdArgs &a, bool vec, void *stream);

// Workspace layout of the backward pass, in bytes, each part 256-aligned.
struct BwdLayout {
  size_t off_ckpt, off_yc, off_pB, off_pC, off_pA, off_pD, off_pbias, total_bytes;
};
BwdLayout bwd_layout(int64_t batch, int64_t dim, int64_t seqlen, int64_t elem_bytes);
const char *hip_error_string(int err);

}  // namespace ssm
