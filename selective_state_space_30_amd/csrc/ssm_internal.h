// ssm_internal.h -- launch interface between the C-ABI layer (ssm_api.cpp)
// and the gfx950 kernels (ssm_kernels.hip).  Not installed; not part of the
// public ABI in include/ssm_scan.h.
#pragma once

#include <cstddef>
#include <cstdint>

namespace ssm {

constexpr int kStates = 16;          // d_state of the tuned instances
constexpr int kMaxStates = 256;      // any d_state up to this (state n in lane n % 64)
constexpr int kWaveLanes = 64;       // one channel per 64-lane wave
constexpr int kWavesPerGroup = 4;    // waves (channels) per workgroup
constexpr int kChannelsPerGroup = kWavesPerGroup;                  // 4
constexpr int kTokensPerLane = 16;   // consecutive tokens owned by one lane
constexpr int kBlockTokens = kWaveLanes * kTokensPerLane;         // 1024
constexpr int kPhaseStates = 2;      // states per double-buffered B/C LDS tile
constexpr int kMaxConv = 4;          // taps of the fused causal conv1d prologue
constexpr int kBwdWaves = 8;         // waves (channels) per backward workgroup
// Backward sweep workgroups resident at once on the chip: one per compute
// unit (the sweep's LDS tiles take 148 KB of a CU's 160 KB), 256 CUs.  A
// fixed count, not a queried one, so that the order of the dB/dC sums (and
// so their bits) is the same on every device.
constexpr int kBwdResident = 256;

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
  int N;                              // d_state (kStates: the tuned instances)
  int64_t chunk_len;                  // tokens per chunk (== L when not split)
  int n_chunks;
  int softplus;                       // 1: dt = softplus(delta + bias)
  int zoh;                            // 1: exact ZOH input term
  float *ckpt;                        // backward's checkpoint pass: the state
                                      // at every block start, (batch, dim,
                                      // ceil(L/1024), 16)
  void *yc;                           // with ckpt: the pre-gate output (dtype),
                                      // or null
  float *ckpt_s;                      // with ckpt in split mode: the chunk's
                                      // sum of dt before every block start
                                      // (batch, dim, ceil(L/1024)); else null
};

// Backward pass.  A workgroup sweeps kBwdWaves channels of one batch entry;
// the sweep is launched ceil(groups / slots) times in a row, launch k taking
// channel groups k * slots .. (k + 1) * slots - 1, and each adds its dB/dC
// channel sums into partial-sum row `slot` (fixed order); a second kernel
// sums the slots' rows.
struct BwdArgs {
  const void *u, *delta, *B, *C, *z, *dy;  // activation dtype
  const float *A, *D, *bias, *h0, *dh_final;
  const float *ckpt;                  // (batch, dim, nblk, 16) forward states
  const void *yc;                     // (batch, dim, L) pre-gate output, dtype
  void *dz;                           // activation dtype output, or null
  void *du, *ddelta;                  // activation dtype outputs
  float *dh0;                         // (batch, dim, 16) or null
  float *pB, *pC;                     // (batch, slots, N, L) partial dB, dC
  float *pA;                          // (batch, dim, n_chunks, 16) partial dA
  float *pD, *pbias;                  // (batch, dim, n_chunks) partial dD, dbias
  float *dA, *dB, *dC, *dD, *dbias;   // reduced outputs (dD, dbias: or null)
  int64_t batch, dim, L;
  int N;                              // d_state (<= kMaxStates: lane n % 64, register n / 64)
  int64_t groups;                     // ceil(dim / kBwdWaves)
  int64_t slots;                      // partial-sum rows per batch entry (<= groups)
  int64_t unit;                       // sweep launch: channel group slot + unit * slots
  int nblk;                           // ceil(L / 1024)
  int softplus;
  int zoh;                            // 1: exact ZOH input term
  // sequence split (n_chunks > 1; chunk_len a multiple of 1024, the last
  // chunk may be shorter): each chunk is swept from the dL/dh entering it
  // from the right, mu_in; chunks >= 1 first get, from a zero right input,
  // the dL/dh leaving their first token (mu0) and their decay product (Pc)
  int n_chunks;
  int64_t chunk_len;
  float *mu0, *Pc, *mu_in;            // (batch, dim, n_chunks, 16)
};

// Backward of the conv prologue (ssm_conv_bwd.hip): u formed into the
// workspace for the scan's backward, then dx and the taps' and bias's
// gradients from its du.
struct ConvBwdArgs {
  const void *x;                      // (batch, dim, L) activation dtype
  const float *conv_w, *conv_b;       // (dim, d_conv), (dim) or null
  int d_conv;                         // 1..4
  void *u;                            // workspace: (batch, dim, L) activation dtype
  const void *du;                     // the scan's gradient of u (activation dtype)
  void *dx;                           // output (batch, dim, L) activation dtype
  float *part;                        // workspace: (batch, dim, 5) per-row sums
  float *dconv_w, *dconv_b;           // outputs (dim, d_conv), (dim) or null
  int64_t batch, dim, L;
};

// Mamba-2 SSD forward (one scalar decay per head; bf16 activations).
constexpr int kSsdChunk = 64;        // tokens per chunk
constexpr int kSsdHeadDim = 64;      // rows (headdim) per head
struct SsdArgs {
  const void *x, *dt, *B, *C, *z;     // bf16: (b,h,P,L), (b,h,L), (b,g,N,L) x2, (b,h,P,L)
  const float *A, *D, *dt_bias, *h0;  // (h), (h), (h), (b,h,P,N)
  void *y;                            // bf16 (b,h,P,L)
  float *h_final;                     // (b,h,P,N) or null
  void *G;                            // workspace: fp32 (b,g,chunk,64,64) causal C^T B
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
  int N;                              // d_state
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
SplitLayout split_layout(int64_t batch, int64_t dim, int64_t N, int64_t n_chunks);

// Size of the fixed device scratch of ssm_scan_fwd_noalloc (a split layout
// must fit in it) and its device address for the device of `stream`
// (returns a hipError_t value as int, 0 = success).
constexpr size_t kScanScratchBytes = size_t(16) << 20;
int scan_scratch(void *stream, void **ptr);

// Kernel launchers.  Return a hipError_t value as int (0 = success).
// `vec` selects 16-byte vector loads (the caller has checked alignment).
int launch_scan(const ScanArgs &a, bool bf16, bool vec, void *stream);
int launch_step(const StepArgs &a, bool bf16, bool vec, void *stream);
int launch_bwd(const BwdArgs &a, bool bf16, bool vec, void *stream);
int launch_ssd(const SsdArgs &a, bool vec, void *stream);
int launch_conv_fwd(const ConvBwdArgs &a, bool bf16, void *stream);
int launch_conv_bwd(const ConvBwdArgs &a, bool bf16, void *stream);
// Roofline microbenchmarks (ssm_roofline.hip): n16 16-byte pieces per pass.
int launch_roofline_hbm(int kind, void *a, void *b, int64_t n16, int repeats,
                        void *stream);
int launch_roofline_valu(int kind, float *out, int64_t threads, int iters,
                         void *stream);

// Workspace layout of the backward pass, in bytes, each part 256-aligned.
// Workspace of the backward.  The checkpoint pass and the sweep each split
// long sequences with few channels into chunks of their own (ckpt_chunk,
// chunk: multiples of 1024 tokens, or the whole sequence).
struct BwdLayout {
  int64_t ckpt_chunk, ckpt_chunks;    // checkpoint pass (a forward scan)
  int64_t chunk, n_chunks;            // sweep
  int64_t slots;                      // dB/dC partial-sum rows per batch entry
  size_t off_ckpt, off_yc, off_pB, off_pC, off_pA, off_pD, off_pbias;
  size_t off_cks, off_H, off_S, off_hin;  // checkpoint pass split
  size_t off_mu0, off_Pc, off_muin;       // sweep split
  size_t total_bytes;
};
BwdLayout bwd_layout(int64_t batch, int64_t dim, int64_t N, int64_t seqlen,
                     int64_t elem_bytes);
const char *hip_error_string(int err);

}  // namespace ssm
