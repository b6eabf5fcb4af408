// C ABI of libssd.so: host-side validation, launch planning and dispatch.
// Every argument is checked before anything is enqueued, so an error status
// means no device memory was touched.  No C++ exception crosses the ABI.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "ssd_common.h"

namespace ssd {
namespace {

thread_local std::string g_last_error;

constexpr int kP = 64;
constexpr int kN = 128;
// the chunk length the block runs its layer with ("Mamba2(..., chunk_size=128)")
constexpr int kBf16Chunk = 128;
// MI355X: 256 compute units; one matrix-core walker fits per CU (its LDS
// footprint is 67 to 115 KiB of 160 KiB, by chunk length).  The sequence-split plan below is sized
// for this count so that the workspace size is a pure function of the shape.
constexpr int kWalkerSlots = 256;
constexpr int kMaxSegments = 64;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(SSD_ERR_HIP, "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

bool valid_dtype(int d) { return d == SSD_F32 || d == SSD_BF16; }
size_t esize(ssd_dtype_t d) { return d == SSD_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte range [lo, hi) of a token-major tensor: rows = B*L, each `width`
// elements wide, `stride` elements apart.  Empty when rows == 0.
struct Range {
  uintptr_t lo = 0, hi = 0;
  bool empty() const { return hi <= lo; }
};
Range tok_range(const void* p, int64_t rows, int64_t stride, int64_t width, size_t es) {
  Range r;
  if (p == nullptr || rows <= 0 || width <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + (uintptr_t)(((rows - 1) * stride + width) * (int64_t)es);
  return r;
}
Range dense_range(const void* p, int64_t n, size_t es) {
  Range r;
  if (p == nullptr || n <= 0) return r;
  r.lo = reinterpret_cast<uintptr_t>(p);
  r.hi = r.lo + (uintptr_t)(n * (int64_t)es);
  return r;
}
bool overlap(const Range& a, const Range& b) {
  return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

// Number of sequence segments for the matrix-core scan: the smallest S that
// minimises the estimated time of the two passes (below).
int plan_segments(int batch, int seqlen, int nheads, int chunk) {
  const int64_t bh = (int64_t)batch * nheads * scan_bf16_walkers_per_head(chunk);
  const int nc = (seqlen + chunk - 1) / chunk;
  if (bh <= 0 || nc <= 1) return 1;
  // Cost in units of a fifth of a full walker's chunk step: pass 2 runs
  // bh * s walkers, one per CU at a time, each over `per` chunks; pass 1 runs
  // the bh * (s - 1) state-only walkers two per CU at a time, a round of them
  // costing four fifths of a full round per chunk; each round of walkers also
  // pays about one chunk step of start-up (first loads, state in and out).
  // (Fitted to the long-context workload, 80 heads x 1024 chunks: measured
  // best at 19 segments, 3.39 ms per call, against 3.50 ms at 64.)
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int s = 1; s <= std::min(nc, kMaxSegments); ++s) {
    const int64_t per = (nc + s - 1) / s;
    const int64_t rounds2 = (bh * s + kWalkerSlots - 1) / kWalkerSlots;
    const int64_t rounds1 = s > 1 ? (bh * (s - 1) + 2 * kWalkerSlots - 1) / (2 * kWalkerSlots) : 0;
    const int64_t cost = rounds2 * (per + 1) * 5 + rounds1 * (per + 1) * 4;
    if (cost < best_cost) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace of the matrix-core scan: per-segment states and log decays when
// the sequence is split, and the B|C pack (B and C of every chunk and group,
// post-conv, in the bf16 layouts the matrix-core products read).
struct WsLayout {
  size_t seg_state = 0, seg_ld = 0, bc = 0, total = 0;
};
WsLayout ws_layout(int batch, int seqlen, int nheads, int ngroups, int chunk, int nseg) {
  WsLayout w;
  const size_t bh = (size_t)batch * nheads;
  size_t off = 0;
  w.seg_state = off;
  if (nseg > 1) off += round_up(bh * nseg * kP * kN * sizeof(float), 256);
  w.seg_ld = off;
  if (nseg > 1) off += round_up(bh * nseg * sizeof(float), 256);
  w.bc = off;
  off += round_up(scan_bf16_pack_bytes(batch, seqlen, ngroups, chunk), 256);
  w.total = off;
  return w;
}

}  // namespace

hipError_t launch_copy_or_zero(void* dst, const void* src, size_t bytes, hipStream_t stream);

}  // namespace ssd

using namespace ssd;

extern "C" {

const char* ssd_version(void) { return "ssd-mi355x 0.1 (gfx950)"; }

const char* ssd_status_string(int status) {
  switch (status) {
    case SSD_OK: return "ok";
    case SSD_ERR_INVALID_ARG: return "invalid argument";
    case SSD_ERR_UNSUPPORTED: return "unsupported shape or option";
    case SSD_ERR_WORKSPACE: return "workspace missing or too small";
    case SSD_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* ssd_last_error(void) { return g_last_error.c_str(); }

int ssd_calibrate_stream(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  g_last_error.clear();
  if (dst == nullptr || src == nullptr)
    return fail(SSD_ERR_INVALID_ARG, "calibrate_stream: dst or src is NULL");
  if (bytes % 16 != 0 || !aligned(dst, 16) || !aligned(src, 16))
    return fail(SSD_ERR_INVALID_ARG, "calibrate_stream: bytes and pointers must be 16-byte multiples");
  if (dst != src && overlap(dense_range(dst, (int64_t)bytes, 1), dense_range(src, (int64_t)bytes, 1)))
    return fail(SSD_ERR_INVALID_ARG, "calibrate_stream: dst partly overlaps src");
  if (bytes / 16 / 512 > (size_t)INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "calibrate_stream: %zu bytes is too large", bytes);
  const hipError_t e = launch_stream(dst, src, bytes, 1.0f, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "calibrate_stream launch");
}

int ssd_calibrate_mfma_bf16(float* out, int blocks, int iters, hipStream_t stream) {
  g_last_error.clear();
  if (out == nullptr || blocks <= 0 || iters <= 0)
    return fail(SSD_ERR_INVALID_ARG, "calibrate_mfma_bf16: bad argument");
  const hipError_t e = launch_mfma_loop(out, blocks, iters, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "calibrate_mfma_bf16 launch");
}

size_t ssd_decode_cache_bytes(int nheads, int headdim, int ngroups, int dstate, int width,
                              ssd_dtype_t conv_dtype) {
  if (nheads <= 0 || headdim <= 0 || ngroups <= 0 || dstate <= 0 || width < 1 ||
      !valid_dtype(conv_dtype) || nheads % ngroups != 0)
    return 0;
  const size_t cdim = (size_t)nheads * headdim + 2 * (size_t)ngroups * dstate;
  return 4 * (size_t)nheads * headdim * dstate + (size_t)(width - 1) * cdim * esize(conv_dtype);
}

int ssd_causal_conv1d_fwd(const void* x, int64_t x_tok_stride, ssd_dtype_t x_dtype,
                          const float* weight, const float* bias, const void* conv_state_in,
                          void* conv_state_out, void* out, int64_t out_tok_stride,
                          ssd_dtype_t out_dtype, int batch, int seqlen, int cdim, int width,
                          int apply_silu, hipStream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(x_dtype) || !valid_dtype(out_dtype))
    return fail(SSD_ERR_INVALID_ARG, "conv1d: bad dtype");
  if (batch < 0 || seqlen < 0 || cdim <= 0)
    return fail(SSD_ERR_INVALID_ARG, "conv1d: bad size batch=%d seqlen=%d cdim=%d", batch,
                seqlen, cdim);
  if (batch > 65535)  // the batch is the third grid dimension of the launch
    return fail(SSD_ERR_UNSUPPORTED, "conv1d: batch %d > 65535", batch);
  if (width < 1) return fail(SSD_ERR_INVALID_ARG, "conv1d: width %d < 1", width);
  if (width > 4) return fail(SSD_ERR_UNSUPPORTED, "conv1d: width %d > 4", width);
  if (apply_silu != 0 && apply_silu != 1)
    return fail(SSD_ERR_INVALID_ARG, "conv1d: apply_silu must be 0 or 1");
  const int64_t rows = (int64_t)batch * seqlen;
  if (weight == nullptr) return fail(SSD_ERR_INVALID_ARG, "conv1d: weight is NULL");
  if (rows > 0 && (x == nullptr || out == nullptr))
    return fail(SSD_ERR_INVALID_ARG, "conv1d: x or out is NULL");
  if (x_tok_stride < cdim || out_tok_stride < cdim)
    return fail(SSD_ERR_INVALID_ARG, "conv1d: token stride below cdim");
  const Range rx = tok_range(x, rows, x_tok_stride, cdim, esize(x_dtype));
  const Range ro = tok_range(out, rows, out_tok_stride, cdim, esize(out_dtype));
  const int64_t hist_n = (int64_t)batch * (width - 1) * cdim;
  const Range rhi = dense_range(conv_state_in, hist_n, esize(x_dtype));
  const Range rho = dense_range(conv_state_out, hist_n, esize(x_dtype));
  if (overlap(ro, rx) || overlap(ro, rhi) || overlap(ro, rho))
    return fail(SSD_ERR_INVALID_ARG, "conv1d: out overlaps an input");
  if (overlap(rho, rhi) || overlap(rho, rx))
    return fail(SSD_ERR_INVALID_ARG, "conv1d: conv_state_out overlaps an input");
  if (batch == 0) return SSD_OK;
  if (rows == 0 && conv_state_out == nullptr) return SSD_OK;
  hipError_t e = launch_causal_conv1d(x, x_tok_stride, x_dtype, weight, bias, conv_state_in,
                                      conv_state_out, cdim, out, out_tok_stride, out_dtype, batch,
                                      seqlen, cdim, width, apply_silu, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "conv1d launch");
}

size_t ssd_chunk_scan_workspace_bytes(int batch, int seqlen, int nheads, int headdim,
                                      int ngroups, int dstate, int chunk, ssd_math_t math,
                                      int fused_conv) {
  (void)headdim; (void)dstate; (void)fused_conv;
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || ngroups <= 0) return 0;
  if (math != SSD_MATH_BF16 || !scan_bf16_supports_chunk(chunk)) return 0;
  return ws_layout(batch, seqlen, nheads, ngroups, chunk,
                   plan_segments(batch, seqlen, nheads, chunk))
      .total;
}

int ssd_chunk_scan_fwd(const void* x, int64_t x_tok_stride, const void* Bm,
                       int64_t b_tok_stride, const void* Cm, int64_t c_tok_stride,
                       ssd_dtype_t xbc_dtype, const float* conv_w, const float* conv_b,
                       int conv_width, const void* conv_state_in, void* conv_state_out,
                       const void* dt, int64_t dt_tok_stride, const void* z,
                       int64_t z_tok_stride, ssd_dtype_t act_dtype, const float* A,
                       const float* D, const float* dt_bias, int dt_softplus,
                       const float* initial_state, float* final_state, void* y,
                       int64_t y_tok_stride, ssd_dtype_t y_dtype, int batch, int seqlen,
                       int nheads, int headdim, int ngroups, int dstate, int chunk,
                       ssd_math_t math, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  g_last_error.clear();
  // ---- enums and sizes
  if (!valid_dtype(xbc_dtype) || !valid_dtype(act_dtype) || !valid_dtype(y_dtype))
    return fail(SSD_ERR_INVALID_ARG, "scan: bad dtype");
  if (math != SSD_MATH_F32 && math != SSD_MATH_BF16)
    return fail(SSD_ERR_INVALID_ARG, "scan: bad math mode %d", (int)math);
  if (batch < 0 || seqlen < 0 || nheads <= 0 || ngroups <= 0 || headdim <= 0 || dstate <= 0 ||
      chunk <= 0)
    return fail(SSD_ERR_INVALID_ARG, "scan: bad size");
  if (nheads % ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "scan: nheads %d not a multiple of ngroups %d", nheads,
                ngroups);
  if (batch > 65535)  // the batch is the third grid dimension of the pack and conv launches
    return fail(SSD_ERR_UNSUPPORTED, "scan: batch %d > 65535", batch);
  if (dt_softplus != 0 && dt_softplus != 1)
    return fail(SSD_ERR_INVALID_ARG, "scan: dt_softplus must be 0 or 1");
  if (headdim != kP || dstate != kN)
    return fail(SSD_ERR_UNSUPPORTED, "scan: headdim %d / dstate %d (supported: 64 / 128)",
                headdim, dstate);
  if (math == SSD_MATH_BF16 && !scan_bf16_supports_chunk(chunk))
    return fail(SSD_ERR_UNSUPPORTED, "scan: chunk %d (matrix-core path supports 64/128/256)",
                chunk);
  if (math == SSD_MATH_F32 && chunk != 32 && chunk != 64 && chunk != 128 && chunk != 256)
    return fail(SSD_ERR_UNSUPPORTED, "scan: chunk %d (fp32 path supports 32/64/128/256)", chunk);
  // ---- conv options
  if (conv_w == nullptr) {
    if (conv_b != nullptr || conv_state_in != nullptr || conv_state_out != nullptr)
      return fail(SSD_ERR_INVALID_ARG, "scan: conv_b/conv_state given without conv_w");
  } else {
    if (conv_width < 1) return fail(SSD_ERR_INVALID_ARG, "scan: conv_width %d < 1", conv_width);
    if (conv_width > 4) return fail(SSD_ERR_UNSUPPORTED, "scan: conv_width %d > 4", conv_width);
  }
  // ---- pointers, strides, alignment
  if (A == nullptr) return fail(SSD_ERR_INVALID_ARG, "scan: A is NULL");
  const int64_t rows = (int64_t)batch * seqlen;
  const int64_t HP = (int64_t)nheads * kP, GN = (int64_t)ngroups * kN;
  const int64_t cdim = HP + 2 * GN;
  if (rows > 0 && (x == nullptr || Bm == nullptr || Cm == nullptr || dt == nullptr ||
                   y == nullptr))
    return fail(SSD_ERR_INVALID_ARG, "scan: x, Bm, Cm, dt or y is NULL");
  if (x_tok_stride < HP || b_tok_stride < GN || c_tok_stride < GN || dt_tok_stride < nheads ||
      y_tok_stride < HP || (z != nullptr && z_tok_stride < HP))
    return fail(SSD_ERR_INVALID_ARG, "scan: a token stride is below its row width");
  const size_t xe = esize(xbc_dtype), ae = esize(act_dtype), ye = esize(y_dtype);
  const void* ptrs16[] = {x, Bm, Cm, z, y, initial_state, final_state, conv_state_in,
                          conv_state_out};
  for (const void* p : ptrs16)
    if (p != nullptr && !aligned(p, 16))
      return fail(SSD_ERR_INVALID_ARG, "scan: a tensor base pointer is not 16-byte aligned");
  if ((x_tok_stride * (int64_t)xe) % 16 || (b_tok_stride * (int64_t)xe) % 16 ||
      (c_tok_stride * (int64_t)xe) % 16 || (y_tok_stride * (int64_t)ye) % 16 ||
      (z != nullptr && (z_tok_stride * (int64_t)ae) % 16))
    return fail(SSD_ERR_INVALID_ARG, "scan: a token stride is not a multiple of 16 bytes");
  // the matrix-core walker addresses a chunk's rows (up to 256 + 3 of them)
  // by 32-bit byte offsets from the chunk's first row
  if (math == SSD_MATH_BF16 && x_tok_stride * (int64_t)xe * 260 >= (INT64_C(1) << 32))
    return fail(SSD_ERR_UNSUPPORTED, "scan: x token stride %lld too large for the matrix-core path",
                (long long)x_tok_stride);
  // ---- aliasing: y may not overlap any input; the conv states may not overlap
  const Range ry = tok_range(y, rows, y_tok_stride, HP, ye);
  const int64_t nstate = (int64_t)batch * nheads * kP * kN;
  const int64_t nhist = conv_w ? (int64_t)batch * (conv_width - 1) * cdim : 0;
  const Range ins[] = {tok_range(x, rows, x_tok_stride, HP, xe),
                       tok_range(Bm, rows, b_tok_stride, GN, xe),
                       tok_range(Cm, rows, c_tok_stride, GN, xe),
                       tok_range(dt, rows, dt_tok_stride, nheads, ae),
                       tok_range(z, rows, z_tok_stride, HP, ae),
                       dense_range(initial_state, nstate, 4),
                       dense_range(final_state, nstate, 4),
                       dense_range(conv_state_in, nhist, xe),
                       dense_range(conv_state_out, nhist, xe)};
  for (const Range& r : ins)
    if (overlap(ry, r)) return fail(SSD_ERR_INVALID_ARG, "scan: y overlaps another tensor");
  const Range rso = dense_range(conv_state_out, nhist, xe);
  for (int i = 0; i < 8; ++i)
    if (overlap(rso, ins[i]))
      return fail(SSD_ERR_INVALID_ARG, "scan: conv_state_out overlaps another tensor");
  const Range rfs = dense_range(final_state, nstate, 4);
  for (int i = 0; i < 5; ++i)
    if (overlap(rfs, ins[i]))
      return fail(SSD_ERR_INVALID_ARG, "scan: final_state overlaps an activation");
  // the state of (b, h) is read whole before it is written, but by the
  // workgroup of (b, h) only: final_state may be initial_state itself, and
  // no other overlap of the two is allowed
  if (final_state != initial_state && overlap(rfs, ins[5]))
    return fail(SSD_ERR_INVALID_ARG,
                "scan: final_state partly overlaps initial_state (only exact aliasing is allowed)");
  // ---- workspace
  const bool mc = math == SSD_MATH_BF16 && rows > 0;
  const int nseg = mc ? plan_segments(batch, seqlen, nheads, chunk) : 1;
  const WsLayout wl = mc ? ws_layout(batch, seqlen, nheads, ngroups, chunk, nseg) : WsLayout{};
  const size_t ws_need = wl.total;
  if (ws_need > 0) {
    if (workspace == nullptr || workspace_bytes < ws_need)
      return fail(SSD_ERR_WORKSPACE, "scan: workspace needs %zu bytes, got %zu", ws_need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(SSD_ERR_INVALID_ARG, "scan: workspace is not 256-byte aligned");
    const Range rws = dense_range(workspace, (int64_t)ws_need, 1);
    if (overlap(rws, ry) || overlap(rws, rso) || overlap(rws, rfs))
      return fail(SSD_ERR_INVALID_ARG, "scan: workspace overlaps a tensor");
    for (const Range& r : ins)
      if (overlap(rws, r)) return fail(SSD_ERR_INVALID_ARG, "scan: workspace overlaps a tensor");
  }

  if (batch == 0) return SSD_OK;
  hipError_t e = hipSuccess;
  if (seqlen == 0) {
    // nothing to scan: hand the states through
    if (final_state != nullptr && final_state != initial_state)
      e = launch_copy_or_zero(final_state, initial_state, (size_t)nstate * 4, stream);
    if (e == hipSuccess && conv_state_out != nullptr)
      e = launch_copy_or_zero(conv_state_out, conv_state_in, (size_t)nhist * xe, stream);
    return e == hipSuccess ? SSD_OK : hip_fail(e, "scan: state hand-through");
  }

  ScanArgs a{};
  a.x = x; a.x_stride = x_tok_stride;
  a.Bm = Bm; a.b_stride = b_tok_stride;
  a.Cm = Cm; a.c_stride = c_tok_stride;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_k = conv_w ? conv_width : 0;
  a.conv_state_in = conv_state_in; a.conv_state_out = conv_state_out;
  a.dt = dt; a.dt_stride = dt_tok_stride;
  a.z = z; a.z_stride = z_tok_stride;
  a.A = A; a.D = D; a.dt_bias = dt_bias; a.dt_softplus = dt_softplus;
  a.initial_state = initial_state; a.final_state = final_state;
  a.y = y; a.y_stride = y_tok_stride;
  a.batch = batch; a.seqlen = seqlen; a.nheads = nheads; a.ngroups = ngroups; a.chunk = chunk;
  const int nc = (seqlen + chunk - 1) / chunk;
  a.nseg = nseg;
  a.seg_chunks = (nc + nseg - 1) / nseg;
  a.nseg = (nc + a.seg_chunks - 1) / a.seg_chunks;  // no empty trailing segment
  char* ws = static_cast<char*>(workspace);
  if (nseg > 1) {
    a.seg_state = reinterpret_cast<float*>(ws + wl.seg_state);
    a.seg_logdecay = reinterpret_cast<float*>(ws + wl.seg_ld);
  }
  if (math == SSD_MATH_BF16) a.bc_pack = ws + wl.bc;
  e = math == SSD_MATH_BF16 ? launch_scan_bf16(a, xbc_dtype, act_dtype, y_dtype, stream)
                            : launch_scan_f32(a, xbc_dtype, act_dtype, y_dtype, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "scan launch");
}

}  // extern "C"

namespace {

// Argument checks shared by both decode entry points; fills the byte ranges
// of y and of the inputs (state, xbc, conv_state, dt, z) for the workspace
// check.  `who` prefixes the message.
int check_state_update(const char* who, float* state, const void* xbc, ssd_dtype_t xbc_dtype,
                       void* conv_state, const float* conv_w, const float* conv_b,
                       int conv_width, const void* dt, const void* z, ssd_dtype_t act_dtype,
                       const float* A, int dt_softplus, void* y, ssd_dtype_t y_dtype, int batch,
                       int nheads, int headdim, int ngroups, int dstate, Range* ry, Range ins[5]) {
  if (!valid_dtype(xbc_dtype) || !valid_dtype(act_dtype) || !valid_dtype(y_dtype))
    return fail(SSD_ERR_INVALID_ARG, "%s: bad dtype", who);
  if (batch < 0 || nheads <= 0 || ngroups <= 0 || headdim <= 0 || dstate <= 0)
    return fail(SSD_ERR_INVALID_ARG, "%s: bad size", who);
  if (nheads % ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "%s: nheads %d not a multiple of ngroups %d", who,
                nheads, ngroups);
  if (dt_softplus != 0 && dt_softplus != 1)
    return fail(SSD_ERR_INVALID_ARG, "%s: dt_softplus must be 0 or 1", who);
  if (batch > 65535)  // the batch is the second grid dimension of every launch
    return fail(SSD_ERR_UNSUPPORTED, "%s: batch %d > 65535", who, batch);
  if (headdim != kP || dstate != kN)
    return fail(SSD_ERR_UNSUPPORTED, "%s: headdim %d / dstate %d (supported: 64 / 128)", who,
                headdim, dstate);
  if (conv_w == nullptr) {
    if (conv_state != nullptr || conv_b != nullptr)
      return fail(SSD_ERR_INVALID_ARG, "%s: conv_state/conv_b given without conv_w", who);
  } else {
    if (conv_width < 1) return fail(SSD_ERR_INVALID_ARG, "%s: conv_width < 1", who);
    if (conv_width > 4) return fail(SSD_ERR_UNSUPPORTED, "%s: conv_width > 4", who);
    if (conv_width > 1 && conv_state == nullptr)
      return fail(SSD_ERR_INVALID_ARG, "%s: conv_w given without conv_state", who);
  }
  if (batch > 0 && (state == nullptr || xbc == nullptr || dt == nullptr || A == nullptr ||
                    y == nullptr))
    return fail(SSD_ERR_INVALID_ARG, "%s: state, xbc, dt, A or y is NULL", who);
  if (state != nullptr && !aligned(state, 16))
    return fail(SSD_ERR_INVALID_ARG, "%s: state is not 16-byte aligned", who);
  const int64_t HP = (int64_t)nheads * kP, cdim = HP + 2 * (int64_t)ngroups * kN;
  const size_t xe = esize(xbc_dtype), ae = esize(act_dtype), ye = esize(y_dtype);
  *ry = dense_range(y, (int64_t)batch * HP, ye);
  ins[0] = dense_range(state, (int64_t)batch * nheads * kP * kN, 4);
  ins[1] = dense_range(xbc, (int64_t)batch * cdim, xe);
  ins[2] = dense_range(conv_state, conv_w ? (int64_t)batch * (conv_width - 1) * cdim : 0, xe);
  ins[3] = dense_range(dt, (int64_t)batch * nheads, ae);
  ins[4] = dense_range(z, (int64_t)batch * HP, ae);
  for (int i = 0; i < 5; ++i) {
    const Range& r = ins[i];
    if (overlap(*ry, r)) return fail(SSD_ERR_INVALID_ARG, "%s: y overlaps an input", who);
  }
  for (int i = 1; i < 5; ++i)
    if (overlap(ins[0], ins[i]))
      return fail(SSD_ERR_INVALID_ARG, "%s: state overlaps another tensor", who);
  for (int i = 0; i < 5; ++i)
    if (i != 2 && overlap(ins[2], ins[i]))
      return fail(SSD_ERR_INVALID_ARG, "%s: conv_state overlaps another tensor", who);
  return SSD_OK;
}

}  // namespace

extern "C" {

int ssd_state_update(float* state, const void* xbc, ssd_dtype_t xbc_dtype, void* conv_state,
                     const float* conv_w, const float* conv_b, int conv_width, const void* dt,
                     const void* z, ssd_dtype_t act_dtype, const float* A, const float* D,
                     const float* dt_bias, int dt_softplus, void* y, ssd_dtype_t y_dtype,
                     int batch, int nheads, int headdim, int ngroups, int dstate,
                     hipStream_t stream) {
  g_last_error.clear();
  Range ry, ins[5];
  const int st = check_state_update("state_update", state, xbc, xbc_dtype, conv_state, conv_w,
                                    conv_b, conv_width, dt, z, act_dtype, A, dt_softplus, y,
                                    y_dtype, batch, nheads, headdim, ngroups, dstate, &ry, ins);
  if (st != SSD_OK) return st;
  if (batch == 0) return SSD_OK;
  hipError_t e = launch_state_update(state, xbc, xbc_dtype, conv_state, conv_w, conv_b,
                                     conv_w ? conv_width : 1, dt, z, act_dtype, A, D, dt_bias,
                                     dt_softplus, y, y_dtype, batch, nheads, ngroups, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "state_update launch");
}

size_t ssd_state_update_workspace_bytes(int batch, int nheads, int headdim, int ngroups,
                                        int dstate) {
  if (batch < 0 || nheads <= 0 || ngroups <= 0 || headdim != kP || dstate != kN ||
      nheads % ngroups != 0)
    return 0;
  return 4 * (size_t)batch * ((size_t)nheads * kP + 2 * (size_t)ngroups * kN);
}

int ssd_state_update_ws(float* state, const void* xbc, ssd_dtype_t xbc_dtype, void* conv_state,
                        const float* conv_w, const float* conv_b, int conv_width,
                        const void* dt, const void* z, ssd_dtype_t act_dtype, const float* A,
                        const float* D, const float* dt_bias, int dt_softplus, void* y,
                        ssd_dtype_t y_dtype, int batch, int nheads, int headdim, int ngroups,
                        int dstate, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  g_last_error.clear();
  Range ry, ins[5];
  const int st = check_state_update("state_update_ws", state, xbc, xbc_dtype, conv_state,
                                    conv_w, conv_b, conv_width, dt, z, act_dtype, A, dt_softplus,
                                    y, y_dtype, batch, nheads, headdim, ngroups, dstate, &ry, ins);
  if (st != SSD_OK) return st;
  const int64_t cdim = (int64_t)nheads * kP + 2 * (int64_t)ngroups * kN;
  if ((int64_t)batch * cdim > ((int64_t)1 << 31) - 256)
    return fail(SSD_ERR_UNSUPPORTED, "state_update_ws: batch x channels exceeds 2^31");
  if (batch == 0) return SSD_OK;
  const size_t need = ssd_state_update_workspace_bytes(batch, nheads, headdim, ngroups, dstate);
  if (workspace == nullptr || workspace_bytes < need)
    return fail(SSD_ERR_WORKSPACE, "state_update_ws: workspace needs %zu bytes, got %zu", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned(workspace, 256))
    return fail(SSD_ERR_INVALID_ARG, "state_update_ws: workspace is not 256-byte aligned");
  const Range rws = dense_range(workspace, (int64_t)need, 1);
  if (overlap(rws, ry))
    return fail(SSD_ERR_INVALID_ARG, "state_update_ws: workspace overlaps a tensor");
  for (int i = 0; i < 5; ++i)
    if (overlap(rws, ins[i]))
      return fail(SSD_ERR_INVALID_ARG, "state_update_ws: workspace overlaps a tensor");
  hipError_t e = launch_state_update_ws(
      state, xbc, xbc_dtype, conv_state, conv_w, conv_b, conv_w ? conv_width : 1, dt, z,
      act_dtype, A, D, dt_bias, dt_softplus, y, y_dtype, batch, nheads, ngroups,
      static_cast<float*>(workspace), stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "state_update_ws launch");
}

int ssd_state_update_noalloc(float* state, const void* xbc, ssd_dtype_t xbc_dtype,
                             void* conv_state, const float* conv_w, const float* conv_b,
                             int conv_width, const void* dt, const void* z,
                             ssd_dtype_t act_dtype, const float* A, const float* D,
                             const float* dt_bias, int dt_softplus, void* y, ssd_dtype_t y_dtype,
                             int batch, int nheads, int headdim, int ngroups, int dstate,
                             hipStream_t stream) {
  g_last_error.clear();
  Range ry, ins[5];
  const int st = check_state_update("state_update_noalloc", state, xbc, xbc_dtype, conv_state,
                                    conv_w, conv_b, conv_width, dt, z, act_dtype, A, dt_softplus,
                                    y, y_dtype, batch, nheads, headdim, ngroups, dstate, &ry, ins);
  if (st != SSD_OK) return st;
  const int64_t cdim = (int64_t)nheads * kP + 2 * (int64_t)ngroups * kN;
  if ((int64_t)batch * cdim > kNoAllocScratchFloats)
    return fail(SSD_ERR_UNSUPPORTED,
                "state_update_noalloc: batch x channels = %lld exceeds its static scratch of "
                "%lld floats (16 MiB); use ssd_state_update_ws with a workspace",
                (long long)((int64_t)batch * cdim), (long long)kNoAllocScratchFloats);
  if (batch == 0) return SSD_OK;
  float* post = nullptr;
  hipError_t e = no_alloc_scratch(&post);
  if (e != hipSuccess) return hip_fail(e, "state_update_noalloc: scratch address");
  e = launch_state_update_ws(state, xbc, xbc_dtype, conv_state, conv_w, conv_b,
                             conv_w ? conv_width : 1, dt, z, act_dtype, A, D, dt_bias,
                             dt_softplus, y, y_dtype, batch, nheads, ngroups, post, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "state_update_noalloc launch");
}

// ------------------------------------------------------------------ backward

size_t ssd_chunk_scan_bwd_workspace_bytes(int batch, int seqlen, int nheads, int headdim,
                                          int ngroups, int dstate, int conv_width) {
  if (batch <= 0 || seqlen < 0 || nheads <= 0 || ngroups <= 0 || headdim != kP ||
      dstate != kN || nheads % ngroups != 0 || conv_width < 0 || conv_width > 4)
    return 0;
  size_t o[7];
  return scan_bwd_workspace_layout(batch, seqlen, nheads, ngroups, conv_width, &o[0], &o[1],
                                   &o[2], &o[3], &o[4], &o[5], &o[6]);
}

int ssd_chunk_scan_bwd(const void* x, int64_t x_tok_stride, const void* Bm,
                       int64_t b_tok_stride, const void* Cm, int64_t c_tok_stride,
                       ssd_dtype_t xbc_dtype, const float* conv_w, const float* conv_b,
                       int conv_width, const void* conv_state_in, const void* dt,
                       int64_t dt_tok_stride, const void* z, int64_t z_tok_stride,
                       ssd_dtype_t act_dtype, const float* A, const float* D,
                       const float* dt_bias, int dt_softplus, const float* initial_state,
                       const void* dout, int64_t dout_tok_stride, ssd_dtype_t dout_dtype,
                       const float* d_final_state, float* dxbc, float* ddt, float* dz,
                       float* dA, float* dD, float* ddt_bias, float* d_initial_state,
                       float* dconv_w, float* dconv_b, float* d_conv_state_in, int batch,
                       int seqlen, int nheads, int headdim, int ngroups, int dstate,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(xbc_dtype) || !valid_dtype(act_dtype) || !valid_dtype(dout_dtype))
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: bad dtype");
  if (batch < 0 || seqlen < 0 || nheads <= 0 || ngroups <= 0 || headdim <= 0 || dstate <= 0)
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: bad size");
  if (nheads % ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: nheads %d not a multiple of ngroups %d", nheads,
                ngroups);
  if (dt_softplus != 0 && dt_softplus != 1)
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: dt_softplus must be 0 or 1");
  if (batch > 65535)  // the batch is the third grid dimension of the conv launches
    return fail(SSD_ERR_UNSUPPORTED, "scan_bwd: batch %d > 65535", batch);
  if (headdim != kP || dstate != kN)
    return fail(SSD_ERR_UNSUPPORTED, "scan_bwd: headdim %d / dstate %d (supported: 64 / 128)",
                headdim, dstate);
  if (conv_w == nullptr) {
    if (conv_b || conv_state_in || dconv_w || dconv_b || d_conv_state_in)
      return fail(SSD_ERR_INVALID_ARG, "scan_bwd: conv arguments given without conv_w");
  } else {
    if (conv_width < 1) return fail(SSD_ERR_INVALID_ARG, "scan_bwd: conv_width %d < 1", conv_width);
    if (conv_width > 4) return fail(SSD_ERR_UNSUPPORTED, "scan_bwd: conv_width %d > 4", conv_width);
  }
  if (A == nullptr || dA == nullptr) return fail(SSD_ERR_INVALID_ARG, "scan_bwd: A or dA is NULL");
  if (z == nullptr && dz != nullptr)
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: dz given without z");
  const int64_t rows = (int64_t)batch * seqlen;
  const int64_t HP = (int64_t)nheads * kP, GN = (int64_t)ngroups * kN, cdim = HP + 2 * GN;
  if (rows > 0 && (x == nullptr || Bm == nullptr || Cm == nullptr || dt == nullptr ||
                   dout == nullptr || dxbc == nullptr || ddt == nullptr))
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: x, Bm, Cm, dt, dout, dxbc or ddt is NULL");
  if (x_tok_stride < HP || b_tok_stride < GN || c_tok_stride < GN || dt_tok_stride < nheads ||
      dout_tok_stride < HP || (z != nullptr && z_tok_stride < HP))
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: a token stride is below its row width");
  const size_t xe = esize(xbc_dtype), ae = esize(act_dtype), de = esize(dout_dtype);
  const void* ptrs16[] = {x, Bm, Cm, z, dout, initial_state, d_final_state, conv_state_in,
                          dxbc, d_initial_state};
  for (const void* p : ptrs16)
    if (p != nullptr && !aligned(p, 16))
      return fail(SSD_ERR_INVALID_ARG, "scan_bwd: a tensor base pointer is not 16-byte aligned");
  if ((x_tok_stride * (int64_t)xe) % 16 || (b_tok_stride * (int64_t)xe) % 16 ||
      (c_tok_stride * (int64_t)xe) % 16 || (dout_tok_stride * (int64_t)de) % 16 ||
      (z != nullptr && (z_tok_stride * (int64_t)ae) % 16))
    return fail(SSD_ERR_INVALID_ARG, "scan_bwd: a token stride is not a multiple of 16 bytes");
  // every output is dense fp32; none may overlap an input or another output
  const int64_t nstate = (int64_t)batch * nheads * kP * kN;
  const int K = conv_w ? conv_width : 0;
  const int64_t nhist = conv_w ? (int64_t)batch * (K - 1) * cdim : 0;
  const Range ins[] = {tok_range(x, rows, x_tok_stride, HP, xe),
                       tok_range(Bm, rows, b_tok_stride, GN, xe),
                       tok_range(Cm, rows, c_tok_stride, GN, xe),
                       tok_range(dt, rows, dt_tok_stride, nheads, ae),
                       tok_range(z, rows, z_tok_stride, HP, ae),
                       tok_range(dout, rows, dout_tok_stride, HP, de),
                       dense_range(initial_state, nstate, 4), dense_range(d_final_state, nstate, 4),
                       dense_range(conv_state_in, nhist, xe), dense_range(A, nheads, 4),
                       dense_range(D, nheads, 4), dense_range(dt_bias, nheads, 4),
                       dense_range(conv_w, cdim * K, 4), dense_range(conv_b, cdim, 4)};
  const Range outs[] = {dense_range(dxbc, rows * cdim, 4), dense_range(ddt, rows * nheads, 4),
                        dense_range(dz, rows * HP, 4), dense_range(dA, nheads, 4),
                        dense_range(dD, nheads, 4), dense_range(ddt_bias, nheads, 4),
                        dense_range(d_initial_state, nstate, 4),
                        dense_range(dconv_w, cdim * K, 4), dense_range(dconv_b, cdim, 4),
                        dense_range(d_conv_state_in, nhist, 4)};
  const int nouts = (int)(sizeof outs / sizeof outs[0]);
  for (int i = 0; i < nouts; ++i) {
    for (const Range& r : ins)
      if (overlap(outs[i], r)) return fail(SSD_ERR_INVALID_ARG, "scan_bwd: an output overlaps an input");
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return fail(SSD_ERR_INVALID_ARG, "scan_bwd: two outputs overlap");
  }
  size_t o[7];
  const size_t need = batch > 0 ? scan_bwd_workspace_layout(batch, seqlen, nheads, ngroups, K,
                                                            &o[0], &o[1], &o[2], &o[3], &o[4],
                                                            &o[5], &o[6])
                                : 0;
  if (batch > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(SSD_ERR_WORKSPACE, "scan_bwd: workspace needs %zu bytes, got %zu", need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(SSD_ERR_INVALID_ARG, "scan_bwd: workspace is not 256-byte aligned");
    const Range rws = dense_range(workspace, (int64_t)need, 1);
    for (const Range& r : ins)
      if (overlap(rws, r)) return fail(SSD_ERR_INVALID_ARG, "scan_bwd: workspace overlaps a tensor");
    for (const Range& r : outs)
      if (overlap(rws, r)) return fail(SSD_ERR_INVALID_ARG, "scan_bwd: workspace overlaps a tensor");
  }
  if (batch == 0) return SSD_OK;
  if (seqlen == 0) {
    // nothing to differentiate through: the initial state's gradient is the
    // final state's, every other gradient is zero
    hipError_t e = hipSuccess;
    float* zeros[] = {dA, dD, ddt_bias, dconv_w, dconv_b, d_conv_state_in};
    const int64_t zn[] = {nheads, nheads, nheads, cdim * K, cdim, nhist};
    for (int i = 0; i < 6 && e == hipSuccess; ++i)
      if (zeros[i] != nullptr && zn[i] > 0)
        e = launch_copy_or_zero(zeros[i], nullptr, (size_t)zn[i] * 4, stream);
    if (e == hipSuccess && d_initial_state != nullptr)
      e = launch_copy_or_zero(d_initial_state, d_final_state, (size_t)nstate * 4, stream);
    return e == hipSuccess ? SSD_OK : hip_fail(e, "scan_bwd: empty sequence");
  }
  ScanBwdLaunch l{};
  l.x = x; l.x_stride = x_tok_stride;
  l.Bm = Bm; l.b_stride = b_tok_stride;
  l.Cm = Cm; l.c_stride = c_tok_stride;
  l.xbc_dtype = xbc_dtype;
  l.conv_w = conv_w; l.conv_b = conv_b; l.conv_k = K; l.conv_state_in = conv_state_in;
  l.dt = dt; l.dt_stride = dt_tok_stride;
  l.z = z; l.z_stride = z_tok_stride;
  l.act_dtype = act_dtype;
  l.A = A; l.D = D; l.dt_bias = dt_bias; l.dt_softplus = dt_softplus;
  l.h0 = initial_state;
  l.dout = dout; l.dout_stride = dout_tok_stride; l.dout_dtype = dout_dtype;
  l.dhT = d_final_state;
  l.dxbc = dxbc; l.ddt = ddt; l.dz = dz; l.dA = dA; l.dD = dD; l.ddt_bias = ddt_bias;
  l.dh0 = d_initial_state;
  l.dconv_w = dconv_w; l.dconv_b = dconv_b; l.dconv_state_in = d_conv_state_in;
  l.batch = batch; l.seqlen = seqlen; l.nheads = nheads; l.ngroups = ngroups;
  l.workspace = workspace;
  hipError_t e = launch_scan_bwd(l, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "scan_bwd launch");
}

// ------------------------------------------------------------------ the block

int ssd_rmsnorm_fwd(const void* x, int64_t x_tok_stride, ssd_dtype_t x_dtype,
                    const float* weight, float eps, void* out, int64_t out_tok_stride,
                    ssd_dtype_t out_dtype, int64_t ntok, int dim, hipStream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(x_dtype) || !valid_dtype(out_dtype))
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: bad dtype");
  if (ntok < 0 || dim <= 0)
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: bad size ntok=%lld dim=%d", (long long)ntok, dim);
  if (dim % 8 != 0) return fail(SSD_ERR_UNSUPPORTED, "rmsnorm: dim %d not a multiple of 8", dim);
  if (!(eps >= 0.f) || !(eps < 1e30f))
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: eps must be finite and >= 0");
  if (ntok > INT32_MAX) return fail(SSD_ERR_UNSUPPORTED, "rmsnorm: more than 2^31-1 rows");
  if (x_tok_stride < dim || out_tok_stride < dim)
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: token stride below dim");
  if (ntok > 0 && (x == nullptr || out == nullptr))
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: x or out is NULL");
  const size_t xe = esize(x_dtype), oe = esize(out_dtype);
  if ((x && !aligned(x, 16)) || (out && !aligned(out, 16)) || (weight && !aligned(weight, 16)) ||
      (x_tok_stride * (int64_t)xe) % 16 || (out_tok_stride * (int64_t)oe) % 16)
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: rows and weight must be 16-byte aligned");
  const Range rx = tok_range(x, ntok, x_tok_stride, dim, xe);
  const Range ro = tok_range(out, ntok, out_tok_stride, dim, oe);
  const bool same = x == out && x_dtype == out_dtype && x_tok_stride == out_tok_stride;
  if (!same && overlap(rx, ro))
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: out overlaps x (only exact in-place is allowed)");
  if (overlap(ro, dense_range(weight, dim, 4)))
    return fail(SSD_ERR_INVALID_ARG, "rmsnorm: out overlaps weight");
  hipError_t e = launch_rmsnorm(x, x_tok_stride, x_dtype, weight, eps, out, out_tok_stride,
                                out_dtype, ntok, dim, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "rmsnorm launch");
}

int ssd_linear_fwd(const void* a, int64_t lda, const void* w, int64_t ldw, const void* residual,
                   int64_t ldr, ssd_dtype_t res_dtype, void* out, int64_t ldo,
                   ssd_dtype_t out_dtype, int64_t M, int N, int K, hipStream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(out_dtype) || (residual != nullptr && !valid_dtype(res_dtype)))
    return fail(SSD_ERR_INVALID_ARG, "linear: bad dtype");
  if (M < 0 || N <= 0 || K <= 0)
    return fail(SSD_ERR_INVALID_ARG, "linear: bad size M=%lld N=%d K=%d", (long long)M, N, K);
  if (K % 8 != 0) return fail(SSD_ERR_UNSUPPORTED, "linear: K %d not a multiple of 8", K);
  if ((M + 255) / 256 * (int64_t)((N + 255) / 256) > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "linear: too many output tiles");
  if (lda < K || ldw < K || ldo < N || (residual != nullptr && ldr < N))
    return fail(SSD_ERR_INVALID_ARG, "linear: a leading dimension is below its row width");
  if (w == nullptr || (M > 0 && (a == nullptr || out == nullptr)))
    return fail(SSD_ERR_INVALID_ARG, "linear: a, w or out is NULL");
  const size_t oe = esize(out_dtype), re = residual ? esize(res_dtype) : 2;
  const void* ptrs16[] = {a, w, out, residual};
  for (const void* p : ptrs16)
    if (p != nullptr && !aligned(p, 16))
      return fail(SSD_ERR_INVALID_ARG, "linear: a base pointer is not 16-byte aligned");
  if ((lda * 2) % 16 || (ldw * 2) % 16 || (ldo * (int64_t)oe) % 16 ||
      (residual != nullptr && (ldr * (int64_t)re) % 16))
    return fail(SSD_ERR_INVALID_ARG, "linear: a row stride is not a multiple of 16 bytes");
  const Range ra = tok_range(a, M, lda, K, 2), rw = tok_range(w, N, ldw, K, 2);
  const Range ro = tok_range(out, M, ldo, N, oe), rr = tok_range(residual, M, ldr, N, re);
  if (overlap(ro, ra) || overlap(ro, rw))
    return fail(SSD_ERR_INVALID_ARG, "linear: out overlaps a or w");
  const bool same = residual == out && res_dtype == out_dtype && ldr == ldo;
  if (!same && overlap(ro, rr))
    return fail(SSD_ERR_INVALID_ARG, "linear: out overlaps residual (only exact in-place is allowed)");
  hipError_t e = launch_gemm_bf16(a, lda, w, ldw, residual, ldr, res_dtype, out, ldo, out_dtype,
                                  M, N, K, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "linear launch");
}

}  // extern "C"

namespace {
// Workspace of the block: normed input | in_proj output (z | x B C | dt, rows
// padded to 8 elements) | layer output y, all bf16, then the layer's own.
struct BlockWs {
  int64_t ld_in = 0;
  size_t u = 0, zx = 0, y = 0, scan = 0, scan_bytes = 0, total = 0;
};
BlockWs block_ws(int batch, int seqlen, int d_model, int nheads, int ngroups) {
  BlockWs w;
  const int64_t T = (int64_t)batch * seqlen;
  const int64_t HP = (int64_t)nheads * kP, GN = (int64_t)ngroups * kN;
  w.ld_in = (2 * HP + 2 * GN + nheads + 7) / 8 * 8;
  size_t off = 0;
  w.u = off; off += round_up((size_t)T * d_model * 2, 256);
  w.zx = off; off += round_up((size_t)T * w.ld_in * 2, 256);
  w.y = off; off += round_up((size_t)T * HP * 2, 256);
  w.scan = off;
  w.scan_bytes = ssd_chunk_scan_workspace_bytes(batch, seqlen, nheads, kP, ngroups, kN,
                                                kBf16Chunk, SSD_MATH_BF16, 1);
  off += round_up(w.scan_bytes, 256);
  w.total = off;
  return w;
}
}  // namespace

extern "C" {

size_t ssd_block_workspace_bytes(int batch, int seqlen, int d_model, int nheads, int headdim,
                                 int ngroups, int dstate) {
  if (batch <= 0 || seqlen <= 0 || d_model <= 0 || nheads <= 0 || ngroups <= 0 ||
      headdim != kP || dstate != kN || nheads % ngroups != 0)
    return 0;
  return block_ws(batch, seqlen, d_model, nheads, ngroups).total;
}

int ssd_block_fwd(const void* h, ssd_dtype_t h_dtype, const float* norm_w, float norm_eps,
                  const void* in_proj_w, const float* conv_w, const float* conv_b,
                  int conv_width, const float* A, const float* D, const float* dt_bias,
                  int dt_softplus, const void* out_proj_w, const void* conv_state_in,
                  void* conv_state_out, const float* initial_state, float* final_state,
                  void* out, ssd_dtype_t out_dtype, int batch, int seqlen, int d_model,
                  int nheads, int headdim, int ngroups, int dstate, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(h_dtype) || !valid_dtype(out_dtype))
    return fail(SSD_ERR_INVALID_ARG, "block: bad dtype");
  if (batch < 0 || seqlen < 0 || d_model <= 0 || nheads <= 0 || ngroups <= 0 ||
      headdim <= 0 || dstate <= 0)
    return fail(SSD_ERR_INVALID_ARG, "block: bad size");
  if (nheads % ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "block: nheads %d not a multiple of ngroups %d", nheads,
                ngroups);
  if (headdim != kP || dstate != kN)
    return fail(SSD_ERR_UNSUPPORTED, "block: headdim %d / dstate %d (supported: 64 / 128)",
                headdim, dstate);
  if (d_model % 8 != 0)
    return fail(SSD_ERR_UNSUPPORTED, "block: d_model %d not a multiple of 8", d_model);
  if (conv_w == nullptr || in_proj_w == nullptr || out_proj_w == nullptr || A == nullptr)
    return fail(SSD_ERR_INVALID_ARG, "block: conv_w, in_proj_w, out_proj_w or A is NULL");
  if (conv_width < 1) return fail(SSD_ERR_INVALID_ARG, "block: conv_width %d < 1", conv_width);
  if (conv_width > 4) return fail(SSD_ERR_UNSUPPORTED, "block: conv_width %d > 4", conv_width);
  if (!(norm_eps >= 0.f) || !(norm_eps < 1e30f))
    return fail(SSD_ERR_INVALID_ARG, "block: norm_eps must be finite and >= 0");
  if (dt_softplus != 0 && dt_softplus != 1)
    return fail(SSD_ERR_INVALID_ARG, "block: dt_softplus must be 0 or 1");
  const int64_t T = (int64_t)batch * seqlen;
  if (T > INT32_MAX) return fail(SSD_ERR_UNSUPPORTED, "block: more than 2^31-1 tokens");
  if (T > 0 && (h == nullptr || out == nullptr))
    return fail(SSD_ERR_INVALID_ARG, "block: h or out is NULL");
  // everything the layer call below would reject is rejected here, before
  // the first launch
  const void* ptrs16[] = {h, out, norm_w, in_proj_w, out_proj_w, conv_state_in,
                          conv_state_out, initial_state, final_state};
  for (const void* p : ptrs16)
    if (p != nullptr && !aligned(p, 16))
      return fail(SSD_ERR_INVALID_ARG, "block: a tensor base pointer is not 16-byte aligned");
  const int64_t HP = (int64_t)nheads * kP, GN = (int64_t)ngroups * kN;
  const int64_t d_in = 2 * HP + 2 * GN + nheads, cdim = HP + 2 * GN;
  if (d_in > INT32_MAX || HP > INT32_MAX)
    return fail(SSD_ERR_UNSUPPORTED, "block: projection too wide");
  const size_t he = esize(h_dtype), oe = esize(out_dtype);
  // out: exact in-place update of h is allowed, any other overlap is not
  const Range rh = dense_range(h, T * d_model, he), ro = dense_range(out, T * d_model, oe);
  const bool same = out == h && out_dtype == h_dtype;
  if (!same && overlap(ro, rh)) return fail(SSD_ERR_INVALID_ARG, "block: out overlaps h");
  const int64_t nstate = (int64_t)batch * nheads * kP * kN;
  const int64_t nhist = (int64_t)batch * (conv_width - 1) * cdim;
  const Range params[] = {dense_range(norm_w, d_model, 4), dense_range(in_proj_w, d_in * d_model, 2),
                          dense_range(out_proj_w, (int64_t)d_model * HP, 2),
                          dense_range(conv_w, cdim * conv_width, 4), dense_range(conv_b, cdim, 4),
                          dense_range(A, nheads, 4), dense_range(D, nheads, 4),
                          dense_range(dt_bias, nheads, 4), dense_range(conv_state_in, nhist, 2),
                          dense_range(initial_state, nstate, 4),
                          dense_range(conv_state_out, nhist, 2),
                          dense_range(final_state, nstate, 4)};
  for (const Range& r : params)
    if (overlap(ro, r)) return fail(SSD_ERR_INVALID_ARG, "block: out overlaps a parameter or state");
  {
    const Range rso = dense_range(conv_state_out, nhist, 2);
    if (overlap(rso, dense_range(conv_state_in, nhist, 2)) ||
        overlap(rso, dense_range(initial_state, nstate, 4)) ||
        overlap(rso, dense_range(final_state, nstate, 4)) || overlap(rso, rh))
      return fail(SSD_ERR_INVALID_ARG, "block: conv_state_out overlaps another tensor");
    const Range rfs = dense_range(final_state, nstate, 4);
    if (overlap(rfs, rh) || overlap(rfs, dense_range(conv_state_in, nhist, 2)))
      return fail(SSD_ERR_INVALID_ARG, "block: final_state overlaps another tensor");
  }
  const BlockWs wl = block_ws(batch, seqlen, d_model, nheads, ngroups);
  if (T > 0) {
    if (workspace == nullptr || workspace_bytes < wl.total)
      return fail(SSD_ERR_WORKSPACE, "block: workspace needs %zu bytes, got %zu", wl.total,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (!aligned(workspace, 256))
      return fail(SSD_ERR_INVALID_ARG, "block: workspace is not 256-byte aligned");
    const Range rws = dense_range(workspace, (int64_t)wl.total, 1);
    if (overlap(rws, rh) || overlap(rws, ro))
      return fail(SSD_ERR_INVALID_ARG, "block: workspace overlaps h or out");
    for (const Range& r : params)
      if (overlap(rws, r))
        return fail(SSD_ERR_INVALID_ARG, "block: workspace overlaps a parameter or state");
  }
  if (batch == 0) return SSD_OK;
  char* ws = static_cast<char*>(workspace);
  bf16* u = T > 0 ? reinterpret_cast<bf16*>(ws + wl.u) : nullptr;
  bf16* zx = T > 0 ? reinterpret_cast<bf16*>(ws + wl.zx) : nullptr;
  bf16* y = T > 0 ? reinterpret_cast<bf16*>(ws + wl.y) : nullptr;
  hipError_t e = hipSuccess;
  if (T > 0) {
    e = launch_rmsnorm(h, d_model, h_dtype, norm_w, norm_eps, u, d_model, SSD_BF16, T, d_model,
                       stream);
    if (e != hipSuccess) return hip_fail(e, "block: rmsnorm launch");
    e = launch_gemm_bf16(u, d_model, in_proj_w, d_model, nullptr, 0, SSD_BF16, zx, wl.ld_in,
                         SSD_BF16, T, (int)d_in, d_model, stream);
    if (e != hipSuccess) return hip_fail(e, "block: in_proj launch");
  }
  // the layer on the in_proj output: z | x B C | dt, one row per token
  const int rc = ssd_chunk_scan_fwd(
      zx ? zx + HP : nullptr, wl.ld_in, zx ? zx + 2 * HP : nullptr, wl.ld_in,
      zx ? zx + 2 * HP + GN : nullptr, wl.ld_in, SSD_BF16, conv_w, conv_b, conv_width,
      conv_state_in, conv_state_out, zx ? zx + 2 * HP + 2 * GN : nullptr, wl.ld_in, zx, wl.ld_in,
      SSD_BF16, A, D, dt_bias, dt_softplus, initial_state, final_state, y, HP, SSD_BF16, batch,
      seqlen, nheads, kP, ngroups, kN, kBf16Chunk, SSD_MATH_BF16, T > 0 ? ws + wl.scan : nullptr,
      wl.scan_bytes, stream);
  if (rc != SSD_OK) {
    g_last_error = "block: " + g_last_error;
    return rc;
  }
  if (T == 0) return SSD_OK;
  e = launch_gemm_bf16(y, HP, out_proj_w, HP, h, d_model, h_dtype, out, d_model, out_dtype, T,
                       d_model, (int)HP, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "block: out_proj launch");
}

}  // extern "C"
