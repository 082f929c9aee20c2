// ssm_api.cpp -- the C ABI declared in include/ssm_scan.h: argument checks,
// the sequence-chunking plan and dispatch to the gfx950 kernels.  Every check
// runs before the first HIP call, so an invalid request never touches the
// device.
#include "ssm_scan.h"
#include "ssm_roofline.h"

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "ssm_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SSM_OK;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) {
  return !__builtin_mul_overflow(a, b, out);
}

// [p, p + n) and [q, q + m) intersect (both non-null, non-empty).
bool overlaps(const void *p, int64_t n, const void *q, int64_t m) {
  if (!p || !q || n <= 0 || m <= 0) return false;
  const char *a = static_cast<const char *>(p);
  const char *b = static_cast<const char *>(q);
  return a < b + m && b < a + n;
}

bool aligned(const void *p, size_t k) {
  return (reinterpret_cast<uintptr_t>(p) % k) == 0;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int64_t kMaxGridYZ = 65535;
// Waves the scan needs to keep all 1024 SIMDs of an MI355X busy: 8 per SIMD,
// two or more rounds at 3-4 resident waves; below half of this (one wave
// per channel) long sequences are split into chunks.  (Measured on 1536
// channels x 2^20 tokens: 8 chunks per channel ran 3-5 % faster than 4.)
constexpr int64_t kTargetWaves = 8192;
constexpr int64_t kMinAutoChunk = 8192;
constexpr int64_t kSimds = 1024;  // 256 CUs x 4 SIMDs
constexpr unsigned kKnownFlags = SSM_FLAG_DELTA_SOFTPLUS | SSM_FLAG_ZOH_B;

int check_sizes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  if (batch <= 0 || dim <= 0 || seqlen <= 0 || dstate <= 0)
    return fail(SSM_ERR_INVALID_ARG,
                "sizes must be positive (batch=%lld dim=%lld dstate=%lld seqlen=%lld)",
                (long long)batch, (long long)dim, (long long)dstate, (long long)seqlen);
  if (dstate > ssm::kMaxStates)
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld: this build supports dstate 1..%d",
                (long long)dstate, ssm::kMaxStates);
  int64_t e, e2;
  if (!mul_ok(batch, dim, &e) || !mul_ok(e, seqlen, &e2) || !mul_ok(e2, 8, &e2))
    return fail(SSM_ERR_INVALID_ARG, "batch*dim*seqlen overflows");
  if (batch > kMaxGridYZ)
    return fail(SSM_ERR_UNSUPPORTED, "batch=%lld exceeds %lld", (long long)batch,
                (long long)kMaxGridYZ);
  return SSM_OK;
}

int64_t choose_chunk(int64_t batch, int64_t dim, int64_t seqlen, int64_t requested) {
  int64_t chunk;
  if (requested > 0) {
    chunk = round_up(requested, ssm::kBlockTokens);
  } else {
    // one wave per (batch, channel)
    const int64_t waves = batch * dim;
    if (waves >= kTargetWaves / 2) return seqlen;
    const int64_t n_min = (kTargetWaves + waves - 1) / waves;
    // prefer, within twice the fewest chunks, a count that gives every SIMD
    // whole rounds at both 3 and 4 resident waves (12 waves per SIMD), else
    // a whole number of waves per SIMD
    int64_t n_c = n_min;
    for (const int64_t per : {12 * kSimds, kSimds}) {
      int64_t k = n_min;
      while (k <= 2 * n_min && (waves * k) % per != 0) ++k;
      if (k <= 2 * n_min) {
        n_c = k;
        break;
      }
    }
    chunk = round_up((seqlen + n_c - 1) / n_c, ssm::kBlockTokens);
    if (chunk < kMinAutoChunk) chunk = kMinAutoChunk;
  }
  return chunk >= seqlen ? seqlen : chunk;
}

// Tokens per chunk of the backward's sweep: the whole sequence while the
// channels alone give every SIMD two rounds of its 2 resident waves;
// otherwise the count of block-aligned chunks (of at least kMinBwdChunk
// tokens, at most kMaxBwdChunks) that minimises rounds x chunk length, the
// fewest within 5 % of that minimum (each chunk after the first costs an
// adjoint pre-pass over its decay horizon).
constexpr int64_t kMinBwdChunk = 8192;
constexpr int64_t kMaxBwdChunks = 16;
int64_t bwd_chunk(int64_t batch, int64_t dim, int64_t seqlen) {
  const int64_t slots = 2 * kSimds;
  const int64_t waves = batch * ((dim + ssm::kBwdWaves - 1) / ssm::kBwdWaves) * ssm::kBwdWaves;
  if (waves >= 2 * slots || seqlen < 2 * kMinBwdChunk) return seqlen;
  struct Pick { int64_t chunk; double cost; };
  Pick best{seqlen, static_cast<double>((waves + slots - 1) / slots)};  // unsplit
  Pick picks[kMaxBwdChunks];
  int np = 0;
  for (int64_t n = 2; n <= kMaxBwdChunks; ++n) {
    const int64_t chunk = round_up((seqlen + n - 1) / n, ssm::kBlockTokens);
    if (chunk < kMinBwdChunk) break;
    const int64_t nc = (seqlen + chunk - 1) / chunk;
    const double cost = static_cast<double>((waves * nc + slots - 1) / slots) *
                        static_cast<double>(chunk) / static_cast<double>(seqlen);
    picks[np++] = Pick{chunk, cost};
    if (cost < best.cost) best = Pick{chunk, cost};
  }
  const double unsplit = static_cast<double>((waves + slots - 1) / slots);
  if (unsplit <= 1.05 * best.cost) return seqlen;
  for (int i = 0; i < np; ++i)  // fewest chunks (longest chunk) first
    if (picks[i].cost <= 1.05 * best.cost) return picks[i].chunk;
  return best.chunk;
}

// dB/dC partial-sum rows per batch entry.  The sweep is launched u times,
// each launch taking `slots` channel groups per batch entry and adding
// group slot + k * slots into row `slot`, so the reduction reads
// ceil(groups / u) rows instead of groups.  u is the largest count whose u
// launches need no more rounds of kBwdResident workgroups than a single
// launch of every group does (the 2.8B layer: 2 x 640 groups, 5 rounds ->
// 5 launches of 2 x 128 workgroups).
int64_t bwd_slots(int64_t batch, int64_t dim, int64_t n_chunks) {
  const int64_t groups = (dim + ssm::kBwdWaves - 1) / ssm::kBwdWaves;
  const int64_t per_slot = batch * n_chunks;  // workgroups of one slot index
  auto rounds = [&](int64_t slots) {
    return (per_slot * slots + ssm::kBwdResident - 1) / ssm::kBwdResident;
  };
  const int64_t r1 = rounds(groups);
  int64_t best = groups;
  for (int64_t u = 2; u <= groups && u <= r1; ++u) {
    const int64_t slots = (groups + u - 1) / u;
    if (rounds(slots) * u <= r1) best = slots;
  }
  return best;
}

}  // namespace

namespace ssm {
BwdLayout bwd_layout(int64_t batch, int64_t dim, int64_t N, int64_t seqlen,
                     int64_t elem_bytes) {
  const size_t ns = static_cast<size_t>(N);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bd = static_cast<size_t>(batch) * dim;
  const size_t nblk = static_cast<size_t>((seqlen + kBlockTokens - 1) / kBlockTokens);
  BwdLayout l;
  l.ckpt_chunk = choose_chunk(batch, dim, seqlen, 0);
  l.ckpt_chunks = (seqlen + l.ckpt_chunk - 1) / l.ckpt_chunk;
  l.chunk = bwd_chunk(batch, dim, seqlen);
  l.n_chunks = (seqlen + l.chunk - 1) / l.chunk;
  l.slots = bwd_slots(batch, dim, l.n_chunks);
  const size_t part =
      static_cast<size_t>(batch) * static_cast<size_t>(l.slots) * ns * seqlen * sizeof(float);
  const size_t nc = static_cast<size_t>(l.n_chunks);
  const size_t ncc = static_cast<size_t>(l.ckpt_chunks);
  l.off_ckpt = 0;
  l.off_yc = up(l.off_ckpt + bd * nblk * ns * sizeof(float));
  l.off_pB = up(l.off_yc + bd * static_cast<size_t>(seqlen) * elem_bytes);
  l.off_pC = up(l.off_pB + part);
  l.off_pA = up(l.off_pC + part);
  l.off_pD = up(l.off_pA + bd * nc * ns * sizeof(float));
  l.off_pbias = up(l.off_pD + bd * nc * sizeof(float));
  size_t end = up(l.off_pbias + bd * nc * sizeof(float));
  // the split checkpoint pass: block dt sums, chunk end states, dt sums and
  // incoming states
  l.off_cks = l.off_H = l.off_S = l.off_hin = 0;
  if (ncc > 1) {
    l.off_cks = end;
    l.off_H = up(l.off_cks + bd * nblk * sizeof(float));
    l.off_S = up(l.off_H + bd * ncc * ns * sizeof(float));
    l.off_hin = up(l.off_S + bd * ncc * sizeof(float));
    end = up(l.off_hin + bd * ncc * ns * sizeof(float));
  }
  // the split sweep: the chunks' adjoints from a zero right input, their
  // decay products, and the adjoints entering them
  l.off_mu0 = l.off_Pc = l.off_muin = 0;
  if (nc > 1) {
    l.off_mu0 = end;
    l.off_Pc = up(l.off_mu0 + bd * nc * ns * sizeof(float));
    l.off_muin = up(l.off_Pc + bd * nc * ns * sizeof(float));
    end = up(l.off_muin + bd * nc * ns * sizeof(float));
  }
  l.total_bytes = end;
  return l;
}

SplitLayout split_layout(int64_t batch, int64_t dim, int64_t N, int64_t n_chunks) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t bdc = static_cast<size_t>(batch) * dim * n_chunks;
  SplitLayout l;
  l.off_H = 0;
  l.off_S = up(l.off_H + bdc * N * sizeof(float));
  l.off_hin = up(l.off_S + bdc * sizeof(float));
  l.total_bytes = up(l.off_hin + bdc * N * sizeof(float));
  return l;
}
}  // namespace ssm

extern "C" {

int ssm_abi_version(void) { return SSM_SCAN_ABI_VERSION; }

const char *ssm_last_error(void) { return g_last_error.c_str(); }

int ssm_scan_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                  int64_t requested_chunk, int64_t *chunk_len_out) {
  if (!chunk_len_out) return fail(SSM_ERR_INVALID_ARG, "chunk_len_out is NULL");
  int st = check_sizes(batch, dim, dstate, seqlen);
  if (st != SSM_OK) return st;
  if (requested_chunk < 0)
    return fail(SSM_ERR_INVALID_ARG, "requested_chunk must be >= 0");
  const int64_t chunk = choose_chunk(batch, dim, seqlen, requested_chunk);
  if ((seqlen + chunk - 1) / chunk > kMaxGridYZ)
    return fail(SSM_ERR_UNSUPPORTED, "more than %lld chunks requested",
                (long long)kMaxGridYZ);
  *chunk_len_out = chunk;
  return ok();
}

int ssm_scan_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                            int64_t seqlen, int64_t requested_chunk,
                            size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_INVALID_ARG, "bytes is NULL");
  int64_t chunk = 0;
  int st = ssm_scan_plan(batch, dim, dstate, seqlen, requested_chunk, &chunk);
  if (st != SSM_OK) return st;
  const int64_t n_chunks = (seqlen + chunk - 1) / chunk;
  *bytes = n_chunks > 1 ? ssm::split_layout(batch, dim, dstate, n_chunks).total_bytes : 0;
  return ok();
}

}  // extern "C"

namespace {

// Shared by ssm_state_update and ssm_conv_state_update (d_conv > 0: the
// conv prologue with its window in conv_state).
int step_impl(float *state, void *conv_state, const void *x, const float *conv_w,
              const float *conv_b, int d_conv, const void *delta, const float *A,
              const void *B, const void *C, const float *D, const void *z,
              const float *delta_bias, unsigned flags, void *y, int64_t batch,
              int64_t dim, int64_t dstate, int dtype, void *stream) {
  if (!state || !x || !delta || !A || !B || !C || !y)
    return fail(SSM_ERR_INVALID_ARG, "required pointer is NULL");
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~kKnownFlags)
    return fail(SSM_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  int st = check_sizes(batch, dim, dstate, 1);
  if (st != SSM_OK) return st;
  // grid: (ceil(dim / 64), ceil(batch / 2)), the second extent at most 65535
  int64_t e;
  if ((batch + 1) / 2 > kMaxGridYZ || !mul_ok(batch * dim, dstate * 4, &e) ||
      batch * dim >= (int64_t(1) << 32))
    return fail(SSM_ERR_UNSUPPORTED, "batch=%lld dim=%lld: too large for the decode grid",
                (long long)batch, (long long)dim);

  const bool bf16 = dtype == SSM_DTYPE_BF16;
  const int64_t es = bf16 ? 2 : 4;
  const void *acts[] = {x, delta, B, C, z, y, conv_state};
  for (const void *p : acts)
    if (p && !aligned(p, es))
      return fail(SSM_ERR_INVALID_ARG, "activation pointer %p not %lld-byte aligned", p,
                  (long long)es);
  const void *f32s[] = {state, A, D, delta_bias, conv_w, conv_b};
  for (const void *p : f32s)
    if (p && !aligned(p, 4))
      return fail(SSM_ERR_INVALID_ARG, "fp32 pointer %p not 4-byte aligned", p);

  const int64_t bdn = batch * dim * dstate * 4;
  const int64_t bd = batch * dim * es;
  const int64_t bn = batch * dstate * es;
  const int64_t csb = d_conv > 1 ? batch * dim * (d_conv - 1) * es : 0;
  const struct { const void *p; int64_t n; const char *name; } ins[] = {
      {x, bd, "x"}, {delta, bd, "delta"}, {z, bd, "z"}, {B, bn, "B"}, {C, bn, "C"},
      {A, dim * dstate * 4, "A"}, {D, dim * 4, "D"}, {delta_bias, dim * 4, "delta_bias"},
      {conv_w, d_conv > 0 ? dim * d_conv * 4 : 0, "conv_w"},
      {conv_b, d_conv > 0 ? dim * 4 : 0, "conv_b"}};
  for (const auto &in : ins) {
    if (overlaps(state, bdn, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "state overlaps input %s", in.name);
    if (overlaps(y, bd, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "y overlaps input %s", in.name);
    if (overlaps(conv_state, csb, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "conv_state overlaps input %s", in.name);
  }
  if (overlaps(y, bd, state, bdn))
    return fail(SSM_ERR_INVALID_ARG, "y overlaps state");
  if (overlaps(conv_state, csb, state, bdn) || overlaps(conv_state, csb, y, bd))
    return fail(SSM_ERR_INVALID_ARG, "conv_state overlaps state or y");

  const bool vec = aligned(state, 16) && aligned(A, 16) && aligned(B, 4 * es) &&
                   aligned(C, 4 * es);
  ssm::StepArgs a{};
  a.state = state; a.x = x; a.delta = delta; a.B = B; a.C = C; a.z = z;
  a.A = A; a.D = D; a.bias = delta_bias; a.y = y;
  a.batch = batch; a.dim = dim; a.N = static_cast<int>(dstate);
  a.softplus = (flags & SSM_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
  a.zoh = (flags & SSM_FLAG_ZOH_B) ? 1 : 0;
  a.conv_state = d_conv > 1 ? conv_state : nullptr;
  a.conv_w = conv_w; a.conv_b = conv_b; a.d_conv = d_conv;
  const int err = ssm::launch_step(a, bf16, vec, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  return ok();
}

// Sizes of the backward pass that fit its grid and its workspace arithmetic.
int check_bwd_sizes(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen) {
  int st = check_sizes(batch, dim, dstate, seqlen);
  if (st != SSM_OK) return st;
  const int64_t groups = (dim + ssm::kBwdWaves - 1) / ssm::kBwdWaves;
  int64_t e;
  if (groups >= (int64_t(1) << 31) || !mul_ok(batch * groups, dstate * seqlen, &e) ||
      !mul_ok(e, 8, &e))
    return fail(SSM_ERR_UNSUPPORTED, "backward workspace of this shape overflows");
  // the checkpoint pass's chunks are a grid dimension
  const int64_t cc = choose_chunk(batch, dim, seqlen, 0);
  if ((seqlen + cc - 1) / cc > kMaxGridYZ)
    return fail(SSM_ERR_UNSUPPORTED, "seqlen too long for the backward's checkpoint pass");
  // the channel-sum reduction launches one workgroup per 256 tokens of each
  // (batch, state) row
  if (batch * dstate * ((seqlen + 255) / 256) >= (int64_t(1) << 31))
    return fail(SSM_ERR_UNSUPPORTED, "batch*seqlen too large for the backward reduction");
  return SSM_OK;
}

// Shared by ssm_scan_fwd (u given), ssm_conv_scan_fwd (x, conv_w given;
// u = silu(conv1d(x)) is formed inside the kernel) and ssm_scan_fwd_save
// (saved = a backward workspace that receives the block checkpoints and the
// pre-gate output; whole sequences, no split).
int scan_impl(const void *u, const void *x, const float *conv_w,
              const float *conv_b, int d_conv, const void *delta,
              const float *A, const void *B, const void *C, const float *D,
              const void *z, const float *delta_bias, unsigned flags,
              const float *h0, void *y, float *h_final, int64_t batch,
              int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
              int64_t requested_chunk, void *workspace, size_t workspace_bytes,
              void *saved, size_t saved_bytes, void *stream, bool use_scratch = false) {
  if (x) {
    if (!conv_w) return fail(SSM_ERR_INVALID_ARG, "conv_w is NULL");
    if (d_conv < 1 || d_conv > ssm::kMaxConv)
      return fail(d_conv < 1 ? SSM_ERR_INVALID_ARG : SSM_ERR_UNSUPPORTED,
                  "d_conv=%d: supported 1..%d", d_conv, ssm::kMaxConv);
    if (!aligned(conv_w, 4) || (conv_b && !aligned(conv_b, 4)))
      return fail(SSM_ERR_INVALID_ARG, "conv weights not 4-byte aligned");
    u = x;  // the checks below apply to x in u's place
  }
  if (!u || !delta || !A || !B || !C || !y)
    return fail(SSM_ERR_INVALID_ARG,
                "required pointer is NULL (u/x=%p delta=%p A=%p B=%p C=%p y=%p)", u,
                delta, (const void *)A, B, C, y);
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~kKnownFlags)
    return fail(SSM_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  int st = check_sizes(batch, dim, dstate, seqlen);
  if (st != SSM_OK) return st;
  if (requested_chunk < 0)
    return fail(SSM_ERR_INVALID_ARG, "requested_chunk must be >= 0");

  const bool bf16 = dtype == SSM_DTYPE_BF16;
  const int64_t es = bf16 ? 2 : 4;
  const void *acts[] = {u, delta, B, C, z, y};
  for (const void *p : acts)
    if (p && !aligned(p, es))
      return fail(SSM_ERR_INVALID_ARG, "activation pointer %p not %lld-byte aligned", p,
                  (long long)es);
  const void *f32s[] = {A, D, delta_bias, h0, h_final};
  for (const void *p : f32s)
    if (p && !aligned(p, 4))
      return fail(SSM_ERR_INVALID_ARG, "fp32 pointer %p not 4-byte aligned", p);

  const int64_t big = batch * dim * seqlen * es;
  const int64_t bc = batch * dstate * seqlen * es;
  const int64_t sts = batch * dim * dstate * 4;
  const struct { const void *p; int64_t n; const char *name; } ins[] = {
      {u, big, x ? "x" : "u"}, {delta, big, "delta"}, {z, big, "z"}, {B, bc, "B"},
      {C, bc, "C"}, {A, dim * dstate * 4, "A"}, {D, dim * 4, "D"},
      {delta_bias, dim * 4, "delta_bias"}, {h0, sts, "h0"},
      {conv_w, x ? dim * d_conv * 4 : 0, "conv_w"},
      {conv_b, x ? dim * 4 : 0, "conv_b"}};
  for (const auto &in : ins) {
    if (overlaps(y, big, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "y overlaps input %s", in.name);
    if (overlaps(h_final, sts, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "h_final overlaps input %s", in.name);
  }
  if (overlaps(y, big, h_final, sts))
    return fail(SSM_ERR_INVALID_ARG, "y overlaps h_final");

  if (saved) {
    if (requested_chunk != 0)
      return fail(SSM_ERR_INVALID_ARG, "saving for the backward chooses its own split "
                                       "(requested_chunk must be 0)");
    st = check_bwd_sizes(batch, dim, dstate, seqlen);
    if (st != SSM_OK) return st;
    const ssm::BwdLayout l = ssm::bwd_layout(batch, dim, dstate, seqlen, es);
    if (saved_bytes < l.total_bytes)
      return fail(SSM_ERR_WORKSPACE, "backward workspace of %zu bytes needed (got %zu bytes at %p)",
                  l.total_bytes, saved_bytes, saved);
    if (!aligned(saved, 256))
      return fail(SSM_ERR_INVALID_ARG, "backward workspace %p not 256-byte aligned", saved);
    const void *all[] = {u, delta, z, B, C, A, D, delta_bias, h0, y, h_final};
    const int64_t sizes[] = {big, big, big, bc, bc, dim * dstate * 4, dim * 4, dim * 4,
                             sts, big, sts};
    for (int i = 0; i < 11; ++i)
      if (overlaps(saved, static_cast<int64_t>(l.total_bytes), all[i], sizes[i]))
        return fail(SSM_ERR_INVALID_ARG, "backward workspace overlaps an argument array");
  }
  // (saving for the backward: the split of the backward's own checkpoint
  // pass, whose buffers its workspace holds)
  const int64_t chunk = choose_chunk(batch, dim, seqlen, requested_chunk);
  const int64_t n_chunks = (seqlen + chunk - 1) / chunk;
  if (n_chunks > kMaxGridYZ)
    return fail(SSM_ERR_UNSUPPORTED, "more than %lld chunks requested",
                (long long)kMaxGridYZ);

  ssm::ScanArgs a{};
  if (n_chunks > 1 && use_scratch) {
    // the library's fixed device scratch; the size check is arithmetic
    // only, the address lookup is the first HIP call
    const ssm::SplitLayout l = ssm::split_layout(batch, dim, dstate, n_chunks);
    if (l.total_bytes > ssm::kScanScratchBytes)
      return fail(SSM_ERR_WORKSPACE,
                  "this shape splits into %lld chunks and needs %zu bytes of scratch; "
                  "the fixed scratch holds %zu (use ssm_scan_fwd with a workspace)",
                  (long long)n_chunks, l.total_bytes, ssm::kScanScratchBytes);
    void *p = nullptr;
    const int err = ssm::scan_scratch(stream, &p);
    if (err != 0)
      return fail(SSM_ERR_HIP, "device scratch lookup failed: %s",
                  ssm::hip_error_string(err));
    char *w = static_cast<char *>(p);
    a.ws_H = reinterpret_cast<float *>(w + l.off_H);
    a.ws_S = reinterpret_cast<float *>(w + l.off_S);
    a.ws_hin = reinterpret_cast<float *>(w + l.off_hin);
  } else if (n_chunks > 1 && saved) {
    const ssm::BwdLayout l = ssm::bwd_layout(batch, dim, dstate, seqlen, es);
    char *w = static_cast<char *>(saved);
    a.ckpt_s = reinterpret_cast<float *>(w + l.off_cks);
    a.ws_H = reinterpret_cast<float *>(w + l.off_H);
    a.ws_S = reinterpret_cast<float *>(w + l.off_S);
    a.ws_hin = reinterpret_cast<float *>(w + l.off_hin);
  } else if (n_chunks > 1) {
    const ssm::SplitLayout l = ssm::split_layout(batch, dim, dstate, n_chunks);
    if (!workspace || workspace_bytes < l.total_bytes)
      return fail(SSM_ERR_WORKSPACE,
                  "workspace of %zu bytes needed (got %zu bytes at %p)", l.total_bytes,
                  workspace_bytes, workspace);
    if (!aligned(workspace, 256))
      return fail(SSM_ERR_INVALID_ARG, "workspace %p not 256-byte aligned", workspace);
    const void *all[] = {u, delta, z, B, C, A, D, delta_bias, h0, y, h_final};
    const int64_t sizes[] = {big, big, big, bc, bc, dim * dstate * 4, dim * 4, dim * 4,
                             sts, big, sts};
    for (int i = 0; i < 11; ++i)
      if (overlaps(workspace, static_cast<int64_t>(l.total_bytes), all[i], sizes[i]))
        return fail(SSM_ERR_INVALID_ARG, "workspace overlaps an argument array");
    char *w = static_cast<char *>(workspace);
    a.ws_H = reinterpret_cast<float *>(w + l.off_H);
    a.ws_S = reinterpret_cast<float *>(w + l.off_S);
    a.ws_hin = reinterpret_cast<float *>(w + l.off_hin);
  }

  // 16-byte vector loads need every activation row to start 16-byte aligned.
  bool vec = (seqlen * es) % 16 == 0;
  for (const void *p : acts)
    if (p && !aligned(p, 16)) vec = false;

  a.u = x ? nullptr : u; a.delta = delta; a.B = B; a.C = C; a.z = z;
  a.x = x; a.conv_w = conv_w; a.conv_b = conv_b; a.d_conv = x ? d_conv : 0;
  a.A = A; a.D = D; a.bias = delta_bias; a.h0 = h0;
  a.y = y; a.h_final = h_final;
  a.batch = batch; a.dim = dim; a.L = seqlen; a.N = static_cast<int>(dstate);
  a.chunk_len = chunk;
  a.n_chunks = static_cast<int>(n_chunks);
  a.softplus = (flags & SSM_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
  a.zoh = (flags & SSM_FLAG_ZOH_B) ? 1 : 0;
  if (saved) {
    const ssm::BwdLayout l = ssm::bwd_layout(batch, dim, dstate, seqlen, es);
    a.ckpt = reinterpret_cast<float *>(static_cast<char *>(saved) + l.off_ckpt);
    a.yc = static_cast<char *>(saved) + l.off_yc;
  }
  const int err = ssm::launch_scan(a, bf16, vec, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  return ok();
}

}  // namespace

extern "C" {

int ssm_scan_fwd(const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *z,
                 const float *delta_bias, unsigned flags, const float *h0,
                 void *y, float *h_final, int64_t batch, int64_t dim,
                 int64_t dstate, int64_t seqlen, int dtype,
                 int64_t requested_chunk, void *workspace,
                 size_t workspace_bytes, void *stream) {
  if (!u) return fail(SSM_ERR_INVALID_ARG, "u is NULL");
  return scan_impl(u, nullptr, nullptr, nullptr, 0, delta, A, B, C, D, z,
                   delta_bias, flags, h0, y, h_final, batch, dim, dstate,
                   seqlen, dtype, requested_chunk, workspace, workspace_bytes,
                   nullptr, 0, stream);
}

int ssm_scan_fwd_noalloc(const void *u, const void *delta, const float *A,
                         const void *B, const void *C, const float *D, const void *z,
                         const float *delta_bias, unsigned flags, const float *h0,
                         void *y, float *h_final, int64_t batch, int64_t dim,
                         int64_t dstate, int64_t seqlen, int dtype,
                         int64_t requested_chunk, void *stream) {
  if (!u) return fail(SSM_ERR_INVALID_ARG, "u is NULL");
  return scan_impl(u, nullptr, nullptr, nullptr, 0, delta, A, B, C, D, z,
                   delta_bias, flags, h0, y, h_final, batch, dim, dstate,
                   seqlen, dtype, requested_chunk, nullptr, 0, nullptr, 0, stream,
                   /*use_scratch=*/true);
}

int ssm_scan_fwd_save(const void *u, const void *delta, const float *A,
                      const void *B, const void *C, const float *D, const void *z,
                      const float *delta_bias, unsigned flags, const float *h0,
                      void *y, float *h_final, int64_t batch, int64_t dim,
                      int64_t dstate, int64_t seqlen, int dtype, void *bwd_workspace,
                      size_t bwd_workspace_bytes, void *stream) {
  if (!u) return fail(SSM_ERR_INVALID_ARG, "u is NULL");
  if (!bwd_workspace) return fail(SSM_ERR_WORKSPACE, "bwd_workspace is NULL");
  return scan_impl(u, nullptr, nullptr, nullptr, 0, delta, A, B, C, D, z,
                   delta_bias, flags, h0, y, h_final, batch, dim, dstate,
                   seqlen, dtype, 0, nullptr, 0, bwd_workspace, bwd_workspace_bytes,
                   stream);
}

int ssm_conv_scan_fwd(const void *x, const float *conv_w, const float *conv_b,
                      int d_conv, const void *delta, const float *A,
                      const void *B, const void *C, const float *D,
                      const void *z, const float *delta_bias, unsigned flags,
                      const float *h0, void *y, float *h_final, int64_t batch,
                      int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                      int64_t requested_chunk, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!x) return fail(SSM_ERR_INVALID_ARG, "x is NULL");
  // The conv prologue over more than 64 lane-held states gave intermittent
  // wrong outputs near the start of the sequence (cause not found); refused
  // until it is.
  if (dstate > 64)
    return fail(SSM_ERR_UNSUPPORTED, "the conv prologue supports dstate <= 64 (got %lld)",
                (long long)dstate);
  return scan_impl(nullptr, x, conv_w, conv_b, d_conv, delta, A, B, C, D, z,
                   delta_bias, flags, h0, y, h_final, batch, dim, dstate,
                   seqlen, dtype, requested_chunk, workspace, workspace_bytes,
                   nullptr, 0, stream);
}

int ssm_state_update(float *state, const void *x, const void *delta,
                     const float *A, const void *B, const void *C,
                     const float *D, const void *z, const float *delta_bias,
                     unsigned flags, void *y, int64_t batch, int64_t dim,
                     int64_t dstate, int dtype, void *stream) {
  return step_impl(state, nullptr, x, nullptr, nullptr, 0, delta, A, B, C, D, z,
                   delta_bias, flags, y, batch, dim, dstate, dtype, stream);
}

int ssm_conv_state_update(float *state, void *conv_state, const void *x,
                          const float *conv_w, const float *conv_b, int d_conv,
                          const void *delta, const float *A, const void *B,
                          const void *C, const float *D, const void *z,
                          const float *delta_bias, unsigned flags, void *y,
                          int64_t batch, int64_t dim, int64_t dstate, int dtype,
                          void *stream) {
  if (!conv_w) return fail(SSM_ERR_INVALID_ARG, "conv_w is NULL");
  if (d_conv < 1 || d_conv > ssm::kMaxConv)
    return fail(d_conv < 1 ? SSM_ERR_INVALID_ARG : SSM_ERR_UNSUPPORTED,
                "d_conv=%d: supported 1..%d", d_conv, ssm::kMaxConv);
  if (d_conv > 1 && !conv_state)
    return fail(SSM_ERR_INVALID_ARG, "conv_state is NULL (d_conv=%d)", d_conv);
  return step_impl(state, conv_state, x, conv_w, conv_b, d_conv, delta, A, B, C, D,
                   z, delta_bias, flags, y, batch, dim, dstate, dtype, stream);
}

}  // extern "C"

extern "C" {

int ssm_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                int64_t seqlen, int dtype, size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_INVALID_ARG, "bytes is NULL");
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  int st = check_bwd_sizes(batch, dim, dstate, seqlen);
  if (st != SSM_OK) return st;
  *bytes = ssm::bwd_layout(batch, dim, dstate, seqlen, dtype == SSM_DTYPE_BF16 ? 2 : 4)
               .total_bytes;
  return ok();
}

int ssm_scan_bwd_plan(int64_t batch, int64_t dim, int64_t dstate, int64_t seqlen,
                      int64_t *plan_out) {
  if (!plan_out) return fail(SSM_ERR_INVALID_ARG, "plan_out is NULL");
  int st = check_bwd_sizes(batch, dim, dstate, seqlen);
  if (st != SSM_OK) return st;
  const ssm::BwdLayout l = ssm::bwd_layout(batch, dim, dstate, seqlen, 4);
  const int64_t groups = (dim + ssm::kBwdWaves - 1) / ssm::kBwdWaves;
  plan_out[0] = l.chunk;
  plan_out[1] = l.ckpt_chunk;
  plan_out[2] = l.slots;
  plan_out[3] = (groups + l.slots - 1) / l.slots;
  return ok();
}

}  // extern "C"

namespace {

// ssm_scan_bwd's checks and launches; check_only: the checks alone (no HIP
// call), so a caller that runs other kernels first can validate everything
// before its first launch.
int scan_bwd_impl(const void *u, const void *delta, const float *A,
                  const void *B, const void *C, const float *D, const void *z,
                  const float *delta_bias, unsigned flags, const float *h0,
                  const void *dy, const float *dh_final, void *du, void *ddelta,
                  float *dA, float *dB, float *dC, float *dD,
                  float *ddelta_bias, void *dz, float *dh0, int64_t batch,
                  int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                  void *workspace, size_t workspace_bytes, void *stream,
                  bool check_only) {
  if (!u || !delta || !A || !B || !C || !dy || !du || !ddelta || !dA || !dB || !dC)
    return fail(SSM_ERR_INVALID_ARG, "required pointer is NULL");
  if (dz && !z) return fail(SSM_ERR_INVALID_ARG, "dz given without z");
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~(kKnownFlags | SSM_FLAG_BWD_SAVED))
    return fail(SSM_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  int st = check_bwd_sizes(batch, dim, dstate, seqlen);
  if (st != SSM_OK) return st;

  const bool bf16 = dtype == SSM_DTYPE_BF16;
  const int64_t es = bf16 ? 2 : 4;
  const void *acts[] = {u, delta, B, C, z, dy, du, ddelta, dz};
  for (const void *p : acts)
    if (p && !aligned(p, es))
      return fail(SSM_ERR_INVALID_ARG, "activation pointer %p not %lld-byte aligned", p,
                  (long long)es);
  const void *f32s[] = {A, D, delta_bias, h0, dh_final, dA, dB, dC, dD, ddelta_bias, dh0};
  for (const void *p : f32s)
    if (p && !aligned(p, 4))
      return fail(SSM_ERR_INVALID_ARG, "fp32 pointer %p not 4-byte aligned", p);

  const int64_t big = batch * dim * seqlen * es;
  const int64_t bc = batch * dstate * seqlen * es;
  const int64_t bcf = batch * dstate * seqlen * 4;
  const int64_t sts = batch * dim * dstate * 4;
  const struct { const void *p; int64_t n; const char *name; } ins[] = {
      {u, big, "u"}, {delta, big, "delta"}, {z, big, "z"}, {dy, big, "dy"},
      {B, bc, "B"}, {C, bc, "C"}, {A, dim * dstate * 4, "A"}, {D, dim * 4, "D"},
      {delta_bias, dim * 4, "delta_bias"}, {h0, sts, "h0"}, {dh_final, sts, "dh_final"}};
  const struct { const void *p; int64_t n; const char *name; } outs[] = {
      {du, big, "du"}, {ddelta, big, "ddelta"}, {dz, big, "dz"}, {dA, dim * dstate * 4, "dA"},
      {dB, bcf, "dB"}, {dC, bcf, "dC"}, {dD, dim * 4, "dD"},
      {ddelta_bias, dim * 4, "ddelta_bias"}, {dh0, sts, "dh0"}};
  for (const auto &o : outs) {
    for (const auto &in : ins)
      if (overlaps(o.p, o.n, in.p, in.n))
        return fail(SSM_ERR_INVALID_ARG, "%s overlaps input %s", o.name, in.name);
    for (const auto &o2 : outs)
      if (&o2 != &o && overlaps(o.p, o.n, o2.p, o2.n))
        return fail(SSM_ERR_INVALID_ARG, "%s overlaps %s", o.name, o2.name);
  }

  const ssm::BwdLayout l = ssm::bwd_layout(batch, dim, dstate, seqlen, es);
  if (!workspace || workspace_bytes < l.total_bytes)
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu bytes at %p)",
                l.total_bytes, workspace_bytes, workspace);
  if (!aligned(workspace, 256))
    return fail(SSM_ERR_INVALID_ARG, "workspace %p not 256-byte aligned", workspace);
  for (const auto &in : ins)
    if (overlaps(workspace, static_cast<int64_t>(l.total_bytes), in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "workspace overlaps input %s", in.name);
  for (const auto &o : outs)
    if (overlaps(workspace, static_cast<int64_t>(l.total_bytes), o.p, o.n))
      return fail(SSM_ERR_INVALID_ARG, "workspace overlaps output %s", o.name);

  if (check_only) return SSM_OK;
  bool vec = (seqlen * es) % 16 == 0;
  for (const void *p : acts)
    if (p && !aligned(p, 16)) vec = false;

  char *w = static_cast<char *>(workspace);
  float *ckpt = reinterpret_cast<float *>(w + l.off_ckpt);

  void *yc = w + l.off_yc;

  // 1. checkpoint pass: the forward scan without the gate, keeping the
  //    block-start states and the pre-gate output (for dz); skipped when
  //    ssm_scan_fwd_save already left them in this workspace.  Split like
  //    the forward when the channels are few (chunks scanned from a zero
  //    state, chained, the pre-gate output and the checkpoints fixed up).
  const bool saved = (flags & SSM_FLAG_BWD_SAVED) != 0;
  ssm::ScanArgs fa{};
  fa.u = u; fa.delta = delta; fa.B = B; fa.C = C; fa.z = nullptr;
  fa.A = A; fa.D = D; fa.bias = delta_bias; fa.h0 = h0;
  fa.y = yc; fa.h_final = nullptr;
  fa.batch = batch; fa.dim = dim; fa.L = seqlen; fa.N = static_cast<int>(dstate);
  fa.chunk_len = l.ckpt_chunk; fa.n_chunks = static_cast<int>(l.ckpt_chunks);
  fa.softplus = (flags & SSM_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
  fa.zoh = (flags & SSM_FLAG_ZOH_B) ? 1 : 0;
  fa.ckpt = ckpt;
  if (l.ckpt_chunks > 1) {
    fa.ckpt_s = reinterpret_cast<float *>(w + l.off_cks);
    fa.ws_H = reinterpret_cast<float *>(w + l.off_H);
    fa.ws_S = reinterpret_cast<float *>(w + l.off_S);
    fa.ws_hin = reinterpret_cast<float *>(w + l.off_hin);
  }
  int err = saved ? 0 : ssm::launch_scan(fa, bf16, vec, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));

  // 2. reverse sweep and 3. reductions
  ssm::BwdArgs a{};
  a.u = u; a.delta = delta; a.B = B; a.C = C; a.z = z; a.dy = dy;
  a.A = A; a.D = D; a.bias = delta_bias; a.h0 = h0; a.dh_final = dh_final;
  a.ckpt = ckpt; a.yc = yc; a.dz = dz;
  a.du = du; a.ddelta = ddelta; a.dh0 = dh0;
  a.pB = reinterpret_cast<float *>(w + l.off_pB);
  a.pC = reinterpret_cast<float *>(w + l.off_pC);
  a.pA = reinterpret_cast<float *>(w + l.off_pA);
  a.pD = reinterpret_cast<float *>(w + l.off_pD);
  a.pbias = reinterpret_cast<float *>(w + l.off_pbias);
  a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD; a.dbias = ddelta_bias;
  a.batch = batch; a.dim = dim; a.L = seqlen; a.N = static_cast<int>(dstate);
  a.groups = (dim + ssm::kBwdWaves - 1) / ssm::kBwdWaves;
  a.slots = l.slots;
  a.nblk = static_cast<int>((seqlen + ssm::kBlockTokens - 1) / ssm::kBlockTokens);
  a.softplus = fa.softplus;
  a.zoh = fa.zoh;
  a.n_chunks = static_cast<int>(l.n_chunks);
  a.chunk_len = l.chunk;
  if (l.n_chunks > 1) {
    a.mu0 = reinterpret_cast<float *>(w + l.off_mu0);
    a.Pc = reinterpret_cast<float *>(w + l.off_Pc);
    a.mu_in = reinterpret_cast<float *>(w + l.off_muin);
  }
  err = ssm::launch_bwd(a, bf16, vec, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  return ok();
}

}  // namespace

extern "C" {

int ssm_scan_bwd(const void *u, const void *delta, const float *A,
                 const void *B, const void *C, const float *D, const void *z,
                 const float *delta_bias, unsigned flags, const float *h0,
                 const void *dy, const float *dh_final, void *du, void *ddelta,
                 float *dA, float *dB, float *dC, float *dD,
                 float *ddelta_bias, void *dz, float *dh0, int64_t batch,
                 int64_t dim, int64_t dstate, int64_t seqlen, int dtype,
                 void *workspace, size_t workspace_bytes, void *stream) {
  return scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, flags, h0, dy, dh_final, du,
                       ddelta, dA, dB, dC, dD, ddelta_bias, dz, dh0, batch, dim, dstate,
                       seqlen, dtype, workspace, workspace_bytes, stream, false);
}

// Workspace of ssm_conv_scan_bwd: the scan backward's, then u and its
// gradient (activation dtype) and the per-row conv sums, 256-byte aligned.
struct ConvBwdLayout {
  size_t off_u, off_du, off_part, total_bytes;
};

static ConvBwdLayout conv_bwd_layout(int64_t batch, int64_t dim, int64_t N, int64_t seqlen,
                                     int64_t es) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t big = static_cast<size_t>(batch) * dim * seqlen * es;
  ConvBwdLayout l;
  l.off_u = up(ssm::bwd_layout(batch, dim, N, seqlen, es).total_bytes);
  l.off_du = up(l.off_u + big);
  l.off_part = up(l.off_du + big);
  l.total_bytes = up(l.off_part + static_cast<size_t>(batch) * dim * (ssm::kMaxConv + 1) *
                                      sizeof(float));
  return l;
}

int ssm_conv_scan_bwd_workspace_size(int64_t batch, int64_t dim, int64_t dstate,
                                     int64_t seqlen, int dtype, size_t *bytes) {
  size_t b0 = 0;
  const int st = ssm_scan_bwd_workspace_size(batch, dim, dstate, seqlen, dtype, &b0);
  if (st != SSM_OK) return st;
  if (!bytes) return fail(SSM_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = conv_bwd_layout(batch, dim, dstate, seqlen, dtype == SSM_DTYPE_BF16 ? 2 : 4)
               .total_bytes;
  return ok();
}

int ssm_conv_scan_bwd(const void *x, const float *conv_w, const float *conv_b,
                      int d_conv, const void *delta, const float *A, const void *B,
                      const void *C, const float *D, const void *z,
                      const float *delta_bias, unsigned flags, const float *h0,
                      const void *dy, const float *dh_final, void *dx,
                      float *dconv_w, float *dconv_b, void *ddelta, float *dA,
                      float *dB, float *dC, float *dD, float *ddelta_bias, void *dz,
                      float *dh0, int64_t batch, int64_t dim, int64_t dstate,
                      int64_t seqlen, int dtype, void *workspace,
                      size_t workspace_bytes, void *stream) {
  if (!x || !conv_w || !dx || !dconv_w)
    return fail(SSM_ERR_INVALID_ARG, "required pointer is NULL (x, conv_w, dx, dconv_w)");
  if (d_conv < 1 || d_conv > ssm::kMaxConv)
    return fail(d_conv < 1 ? SSM_ERR_INVALID_ARG : SSM_ERR_UNSUPPORTED,
                "d_conv=%d: supported 1..%d", d_conv, ssm::kMaxConv);
  if (dtype != SSM_DTYPE_F32 && dtype != SSM_DTYPE_BF16)
    return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & SSM_FLAG_BWD_SAVED)
    return fail(SSM_ERR_INVALID_ARG, "SSM_FLAG_BWD_SAVED: the conv backward has no saving forward");
  int st = check_bwd_sizes(batch, dim, dstate, seqlen);
  if (st != SSM_OK) return st;
  const int64_t es = dtype == SSM_DTYPE_BF16 ? 2 : 4;
  if (!aligned(x, es) || !aligned(dx, es))
    return fail(SSM_ERR_INVALID_ARG, "x or dx not %lld-byte aligned", (long long)es);
  const void *f32s[] = {conv_w, conv_b, dconv_w, dconv_b};
  for (const void *p : f32s)
    if (p && !aligned(p, 4))
      return fail(SSM_ERR_INVALID_ARG, "fp32 pointer %p not 4-byte aligned", p);
  const ConvBwdLayout l = conv_bwd_layout(batch, dim, dstate, seqlen, es);
  if (!workspace || workspace_bytes < l.total_bytes)
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu bytes at %p)",
                l.total_bytes, workspace_bytes, workspace);
  if (!aligned(workspace, 256))
    return fail(SSM_ERR_INVALID_ARG, "workspace %p not 256-byte aligned", workspace);
  const int64_t big = batch * dim * seqlen * es;
  const int64_t bc = batch * dstate * seqlen * es;
  const int64_t sts = batch * dim * dstate * 4;
  const int64_t ws = static_cast<int64_t>(l.total_bytes);
  // the conv's own arrays against each other and the workspace (the scan
  // backward's checks below cover the rest, with u and du in the workspace)
  const struct { const void *p; int64_t n; const char *name; } ins[] = {
      {x, big, "x"}, {conv_w, dim * d_conv * 4, "conv_w"}, {conv_b, conv_b ? dim * 4 : 0, "conv_b"},
      {delta, big, "delta"}, {z, big, "z"}, {dy, big, "dy"}, {B, bc, "B"}, {C, bc, "C"},
      {A, dim * dstate * 4, "A"}, {D, dim * 4, "D"}, {delta_bias, dim * 4, "delta_bias"},
      {h0, sts, "h0"}, {dh_final, sts, "dh_final"}};
  const struct { const void *p; int64_t n; const char *name; } outs[] = {
      {dx, big, "dx"}, {dconv_w, dim * d_conv * 4, "dconv_w"},
      {dconv_b, dconv_b ? dim * 4 : 0, "dconv_b"}};
  for (const auto &o : outs) {
    for (const auto &in : ins)
      if (overlaps(o.p, o.n, in.p, in.n))
        return fail(SSM_ERR_INVALID_ARG, "%s overlaps input %s", o.name, in.name);
    if (overlaps(o.p, o.n, workspace, ws))
      return fail(SSM_ERR_INVALID_ARG, "%s overlaps the workspace", o.name);
    const void *sc[] = {ddelta, dA, dB, dC, dD, ddelta_bias, dz, dh0};
    const int64_t scn[] = {big, dim * dstate * 4, batch * dstate * seqlen * 4,
                           batch * dstate * seqlen * 4, dim * 4, dim * 4, big, sts};
    for (int i = 0; i < 8; ++i)
      if (overlaps(o.p, o.n, sc[i], scn[i]))
        return fail(SSM_ERR_INVALID_ARG, "%s overlaps another gradient", o.name);
  }
  if (overlaps(dx, big, dconv_w, dim * d_conv * 4) ||
      overlaps(dx, big, dconv_b, conv_b ? dim * 4 : 0) ||
      overlaps(dconv_w, dim * d_conv * 4, dconv_b, dconv_b ? dim * 4 : 0))
    return fail(SSM_ERR_INVALID_ARG, "dx, dconv_w and dconv_b overlap");
  for (const auto &in : ins)
    if (overlaps(workspace, ws, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "workspace overlaps input %s", in.name);
  char *w = static_cast<char *>(workspace);
  void *u = w + l.off_u;
  void *du = w + l.off_du;
  const size_t bwd_bytes = l.off_u;  // the scan backward's part comes first
  st = scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, flags, h0, dy, dh_final, du, ddelta,
                     dA, dB, dC, dD, ddelta_bias, dz, dh0, batch, dim, dstate, seqlen, dtype,
                     workspace, bwd_bytes, stream, true);
  if (st != SSM_OK) return st;

  ssm::ConvBwdArgs c{};
  c.x = x; c.conv_w = conv_w; c.conv_b = conv_b; c.d_conv = d_conv;
  c.u = u; c.du = du; c.dx = dx;
  c.part = reinterpret_cast<float *>(w + l.off_part);
  c.dconv_w = dconv_w; c.dconv_b = dconv_b;
  c.batch = batch; c.dim = dim; c.L = seqlen;
  const bool bf16 = dtype == SSM_DTYPE_BF16;
  int err = ssm::launch_conv_fwd(c, bf16, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  st = scan_bwd_impl(u, delta, A, B, C, D, z, delta_bias, flags, h0, dy, dh_final, du, ddelta,
                     dA, dB, dC, dD, ddelta_bias, dz, dh0, batch, dim, dstate, seqlen, dtype,
                     workspace, bwd_bytes, stream, false);
  if (st != SSM_OK) return st;
  err = ssm::launch_conv_bwd(c, bf16, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  return ok();
}

}  // extern "C"

namespace {

// Workspace of the SSD forward: G = C^T B per chunk (fp32 64 x 64) and C
// transposed per chunk (bf16 64 x N), each part 256-byte aligned.
struct SsdLayout {
  size_t off_G, off_Ct, total_bytes;
};
SsdLayout ssd_layout(int64_t batch, int64_t ngroups, int64_t dstate, int64_t seqlen) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t chunks = static_cast<size_t>(batch) * ngroups *
                        static_cast<size_t>((seqlen + ssm::kSsdChunk - 1) / ssm::kSsdChunk);
  SsdLayout l;
  l.off_G = 0;
  l.off_Ct = up(chunks * ssm::kSsdChunk * ssm::kSsdChunk * 2 * 2);
  l.total_bytes = up(l.off_Ct + chunks * ssm::kSsdChunk * static_cast<size_t>(dstate) * 2);
  return l;
}

int check_ssd_sizes(int64_t batch, int64_t nheads, int64_t headdim, int64_t ngroups,
                    int64_t dstate, int64_t seqlen) {
  if (batch <= 0 || nheads <= 0 || headdim <= 0 || ngroups <= 0 || dstate <= 0 ||
      seqlen <= 0)
    return fail(SSM_ERR_INVALID_ARG, "sizes must be positive");
  if (nheads % ngroups != 0)
    return fail(SSM_ERR_INVALID_ARG, "nheads=%lld is not a multiple of ngroups=%lld",
                (long long)nheads, (long long)ngroups);
  if (headdim != ssm::kSsdHeadDim)
    return fail(SSM_ERR_UNSUPPORTED, "headdim=%lld: this build supports %d",
                (long long)headdim, ssm::kSsdHeadDim);
  if (dstate != 64 && dstate != 128 && dstate != 256)
    return fail(SSM_ERR_UNSUPPORTED, "dstate=%lld: this build supports 64, 128, 256",
                (long long)dstate);
  int64_t e;
  if (!mul_ok(batch * nheads, headdim * seqlen, &e) || !mul_ok(e, 8, &e) ||
      !mul_ok(batch * ngroups, dstate * seqlen, &e) || !mul_ok(e, 8, &e))
    return fail(SSM_ERR_INVALID_ARG, "sizes overflow");
  if (batch > kMaxGridYZ || nheads >= (int64_t(1) << 31) ||
      (seqlen + ssm::kSsdChunk - 1) / ssm::kSsdChunk > (int64_t(1) << 30))
    return fail(SSM_ERR_UNSUPPORTED, "grid too large");
  // the kernel reads a group's B and a head's rows through 32-bit byte views
  if (dstate * seqlen * 2 >= (int64_t(1) << 31))
    return fail(SSM_ERR_UNSUPPORTED, "dstate*seqlen=%lld: at most 2^30 - 1 in this build",
                (long long)(dstate * seqlen));
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_ssd_workspace_size(int64_t batch, int64_t ngroups, int64_t dstate,
                           int64_t seqlen, size_t *bytes) {
  if (!bytes) return fail(SSM_ERR_INVALID_ARG, "bytes is NULL");
  int st = check_ssd_sizes(batch, ngroups, ssm::kSsdHeadDim, ngroups, dstate, seqlen);
  if (st != SSM_OK) return st;
  *bytes = ssd_layout(batch, ngroups, dstate, seqlen).total_bytes;
  return ok();
}

int ssm_ssd_fwd(const void *x, const void *dt, const float *A, const void *B,
                const void *C, const float *D, const void *z,
                const float *dt_bias, unsigned flags, const float *h0, void *y,
                float *h_final, int64_t batch, int64_t nheads, int64_t headdim,
                int64_t ngroups, int64_t dstate, int64_t seqlen, int dtype,
                void *workspace, size_t workspace_bytes, void *stream) {
  if (!x || !dt || !A || !B || !C || !y)
    return fail(SSM_ERR_INVALID_ARG, "required pointer is NULL");
  if (dtype == SSM_DTYPE_F32)
    return fail(SSM_ERR_UNSUPPORTED, "the SSD form runs on bf16 activations only");
  if (dtype != SSM_DTYPE_BF16) return fail(SSM_ERR_INVALID_ARG, "unknown dtype %d", dtype);
  if (flags & ~kKnownFlags) return fail(SSM_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (flags & SSM_FLAG_ZOH_B)
    return fail(SSM_ERR_UNSUPPORTED, "the SSD form implements the Euler input term only");
  int st = check_ssd_sizes(batch, nheads, headdim, ngroups, dstate, seqlen);
  if (st != SSM_OK) return st;

  const void *acts[] = {x, dt, B, C, z, y};
  for (const void *p : acts)
    if (p && !aligned(p, 2))
      return fail(SSM_ERR_INVALID_ARG, "bf16 pointer %p not 2-byte aligned", p);
  const void *f32s[] = {A, D, dt_bias, h0, h_final};
  for (const void *p : f32s)
    if (p && !aligned(p, 4))
      return fail(SSM_ERR_INVALID_ARG, "fp32 pointer %p not 4-byte aligned", p);
  const int64_t big = batch * nheads * headdim * seqlen * 2;
  const int64_t bc = batch * ngroups * dstate * seqlen * 2;
  const int64_t sts = batch * nheads * headdim * dstate * 4;
  const struct { const void *p; int64_t n; const char *name; } ins[] = {
      {x, big, "x"}, {z, big, "z"}, {dt, batch * nheads * seqlen * 2, "dt"},
      {B, bc, "B"}, {C, bc, "C"}, {A, nheads * 4, "A"}, {D, nheads * 4, "D"},
      {dt_bias, nheads * 4, "dt_bias"}, {h0, sts, "h0"}};
  for (const auto &in : ins) {
    if (overlaps(y, big, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "y overlaps input %s", in.name);
    if (overlaps(h_final, sts, in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "h_final overlaps input %s", in.name);
  }
  if (overlaps(y, big, h_final, sts)) return fail(SSM_ERR_INVALID_ARG, "y overlaps h_final");
  const SsdLayout l = ssd_layout(batch, ngroups, dstate, seqlen);
  if (!workspace || workspace_bytes < l.total_bytes)
    return fail(SSM_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu bytes at %p)",
                l.total_bytes, workspace_bytes, workspace);
  if (!aligned(workspace, 256))
    return fail(SSM_ERR_INVALID_ARG, "workspace %p not 256-byte aligned", workspace);
  for (const auto &in : ins)
    if (overlaps(workspace, static_cast<int64_t>(l.total_bytes), in.p, in.n))
      return fail(SSM_ERR_INVALID_ARG, "workspace overlaps input %s", in.name);
  if (overlaps(workspace, static_cast<int64_t>(l.total_bytes), y, big) ||
      overlaps(workspace, static_cast<int64_t>(l.total_bytes), h_final, sts))
    return fail(SSM_ERR_INVALID_ARG, "workspace overlaps an output");

  // 16-byte loads and stores need every row to start 16-byte aligned
  bool vec = (seqlen % 8) == 0;
  const void *rows[] = {x, z, y, B, C};
  for (const void *p : rows)
    if (p && !aligned(p, 16)) vec = false;

  char *w = static_cast<char *>(workspace);
  ssm::SsdArgs a{};
  a.x = x; a.dt = dt; a.B = B; a.C = C; a.z = z;
  a.A = A; a.D = D; a.dt_bias = dt_bias; a.h0 = h0;
  a.y = y; a.h_final = h_final;
  a.G = w + l.off_G;
  a.Ct = w + l.off_Ct;
  a.batch = batch; a.nheads = nheads; a.ngroups = ngroups; a.L = seqlen;
  a.nchunks = static_cast<int>((seqlen + ssm::kSsdChunk - 1) / ssm::kSsdChunk);
  a.dstate = static_cast<int>(dstate);
  a.softplus = (flags & SSM_FLAG_DELTA_SOFTPLUS) ? 1 : 0;
  const int err = ssm::launch_ssd(a, vec, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  return ok();
}

}  // extern "C"

// ------------------------------------------------ roofline microbenchmarks
extern "C" {

int ssm_roofline_hbm(int kind, void *a, void *b, size_t bytes, int repeats,
                     void *stream) {
  if (kind < SSM_ROOFLINE_COPY || kind > SSM_ROOFLINE_READ)
    return fail(SSM_ERR_INVALID_ARG, "unknown HBM kind %d", kind);
  if (bytes == 0 || bytes % SSM_ROOFLINE_HBM_QUANTUM != 0 || bytes >= (size_t(1) << 46))
    return fail(SSM_ERR_INVALID_ARG, "bytes=%zu: must be a positive multiple of %d below 2^46",
                bytes, SSM_ROOFLINE_HBM_QUANTUM);
  if (repeats < 1 || repeats > 1000)
    return fail(SSM_ERR_INVALID_ARG, "repeats=%d: must be 1..1000", repeats);
  if (!a || !aligned(a, 16)) return fail(SSM_ERR_INVALID_ARG, "a: NULL or not 16-byte aligned");
  if (kind == SSM_ROOFLINE_COPY) {
    if (!b || !aligned(b, 16))
      return fail(SSM_ERR_INVALID_ARG, "b: NULL or not 16-byte aligned");
    if (overlaps(a, static_cast<int64_t>(bytes), b, static_cast<int64_t>(bytes)))
      return fail(SSM_ERR_INVALID_ARG, "a and b overlap");
  } else if (kind == SSM_ROOFLINE_READ) {
    if (!b || !aligned(b, 4)) return fail(SSM_ERR_INVALID_ARG, "b: NULL or not 4-byte aligned");
    if (overlaps(a, static_cast<int64_t>(bytes), b, 4))
      return fail(SSM_ERR_INVALID_ARG, "a and b overlap");
  }
  const int err = ssm::launch_roofline_hbm(kind, a, b, static_cast<int64_t>(bytes / 16),
                                           repeats, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  return ok();
}

int ssm_roofline_valu(int kind, float *out, int64_t threads, int iters, void *stream) {
  if (kind < SSM_ROOFLINE_EXP || kind > SSM_ROOFLINE_MIXED)
    return fail(SSM_ERR_INVALID_ARG, "unknown VALU kind %d", kind);
  if (threads <= 0 || threads % SSM_ROOFLINE_VALU_QUANTUM != 0 || threads > (int64_t(1) << 26))
    return fail(SSM_ERR_INVALID_ARG,
                "threads=%lld: must be a positive multiple of %d, at most 2^26",
                (long long)threads, SSM_ROOFLINE_VALU_QUANTUM);
  if (iters < 1 || iters > (1 << 20))
    return fail(SSM_ERR_INVALID_ARG, "iters=%d: must be 1..2^20", iters);
  if (!out || !aligned(out, 4)) return fail(SSM_ERR_INVALID_ARG, "out: NULL or misaligned");
  const int err = ssm::launch_roofline_valu(kind, out, threads, iters, stream);
  if (err != 0)
    return fail(SSM_ERR_HIP, "kernel launch failed: %s", ssm::hip_error_string(err));
  return ok();
}

}  // extern "C"
