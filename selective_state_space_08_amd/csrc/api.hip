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
constexpr int kBf16Chunk = 128;
// MI355X: 256 compute units; one matrix-core walker fits per CU (its LDS
// footprint is ~120 KiB of 160 KiB).  The sequence-split plan below is sized
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
// minimises (rounds of walkers over the CU slots) x (chunks per segment).
int plan_segments(int batch, int seqlen, int nheads) {
  const int64_t bh = (int64_t)batch * nheads;
  const int nc = (seqlen + kBf16Chunk - 1) / kBf16Chunk;
  if (bh <= 0 || nc <= 1) return 1;
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int s = 1; s <= std::min(nc, kMaxSegments); ++s) {
    const int64_t rounds = (bh * s + kWalkerSlots - 1) / kWalkerSlots;
    const int64_t per = (nc + s - 1) / s;
    // pass 1 walks S-1 segments state-only: charge it half a walk
    const int64_t cost = rounds * per * 2 + (s > 1 ? per : 0);
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
WsLayout ws_layout(int batch, int seqlen, int nheads, int ngroups, int nseg) {
  WsLayout w;
  const size_t bh = (size_t)batch * nheads;
  size_t off = 0;
  w.seg_state = off;
  if (nseg > 1) off += round_up(bh * nseg * kP * kN * sizeof(float), 256);
  w.seg_ld = off;
  if (nseg > 1) off += round_up(bh * nseg * sizeof(float), 256);
  w.bc = off;
  off += round_up(scan_bf16_pack_bytes(batch, seqlen, ngroups), 256);
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
  (void)headdim; (void)dstate; (void)chunk; (void)fused_conv;
  if (batch <= 0 || seqlen <= 0 || nheads <= 0 || ngroups <= 0) return 0;
  if (math != SSD_MATH_BF16) return 0;
  return ws_layout(batch, seqlen, nheads, ngroups, plan_segments(batch, seqlen, nheads)).total;
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
  if (dt_softplus != 0 && dt_softplus != 1)
    return fail(SSD_ERR_INVALID_ARG, "scan: dt_softplus must be 0 or 1");
  if (headdim != kP || dstate != kN)
    return fail(SSD_ERR_UNSUPPORTED, "scan: headdim %d / dstate %d (supported: 64 / 128)",
                headdim, dstate);
  if (math == SSD_MATH_BF16 && chunk != kBf16Chunk)
    return fail(SSD_ERR_UNSUPPORTED, "scan: chunk %d (matrix-core path supports 128)", chunk);
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
  // ---- workspace
  const bool mc = math == SSD_MATH_BF16 && rows > 0;
  const int nseg = mc ? plan_segments(batch, seqlen, nheads) : 1;
  const WsLayout wl = mc ? ws_layout(batch, seqlen, nheads, ngroups, nseg) : WsLayout{};
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

int ssd_state_update(float* state, const void* xbc, ssd_dtype_t xbc_dtype, void* conv_state,
                     const float* conv_w, const float* conv_b, int conv_width, const void* dt,
                     const void* z, ssd_dtype_t act_dtype, const float* A, const float* D,
                     const float* dt_bias, int dt_softplus, void* y, ssd_dtype_t y_dtype,
                     int batch, int nheads, int headdim, int ngroups, int dstate,
                     hipStream_t stream) {
  g_last_error.clear();
  if (!valid_dtype(xbc_dtype) || !valid_dtype(act_dtype) || !valid_dtype(y_dtype))
    return fail(SSD_ERR_INVALID_ARG, "state_update: bad dtype");
  if (batch < 0 || nheads <= 0 || ngroups <= 0 || headdim <= 0 || dstate <= 0)
    return fail(SSD_ERR_INVALID_ARG, "state_update: bad size");
  if (nheads % ngroups != 0)
    return fail(SSD_ERR_INVALID_ARG, "state_update: nheads %d not a multiple of ngroups %d",
                nheads, ngroups);
  if (dt_softplus != 0 && dt_softplus != 1)
    return fail(SSD_ERR_INVALID_ARG, "state_update: dt_softplus must be 0 or 1");
  if (headdim != kP || dstate != kN)
    return fail(SSD_ERR_UNSUPPORTED, "state_update: headdim %d / dstate %d (supported: 64 / 128)",
                headdim, dstate);
  if (conv_w == nullptr) {
    if (conv_state != nullptr || conv_b != nullptr)
      return fail(SSD_ERR_INVALID_ARG, "state_update: conv_state/conv_b given without conv_w");
  } else {
    if (conv_width < 1) return fail(SSD_ERR_INVALID_ARG, "state_update: conv_width < 1");
    if (conv_width > 4) return fail(SSD_ERR_UNSUPPORTED, "state_update: conv_width > 4");
    if (conv_width > 1 && conv_state == nullptr)
      return fail(SSD_ERR_INVALID_ARG, "state_update: conv_w given without conv_state");
  }
  if (batch > 0 && (state == nullptr || xbc == nullptr || dt == nullptr || A == nullptr ||
                    y == nullptr))
    return fail(SSD_ERR_INVALID_ARG, "state_update: state, xbc, dt, A or y is NULL");
  if (state != nullptr && !aligned(state, 16))
    return fail(SSD_ERR_INVALID_ARG, "state_update: state is not 16-byte aligned");
  const int64_t HP = (int64_t)nheads * kP, cdim = HP + 2 * (int64_t)ngroups * kN;
  const size_t xe = esize(xbc_dtype), ae = esize(act_dtype), ye = esize(y_dtype);
  const Range ry = dense_range(y, (int64_t)batch * HP, ye);
  const Range ins[] = {dense_range(state, (int64_t)batch * nheads * kP * kN, 4),
                       dense_range(xbc, (int64_t)batch * cdim, xe),
                       dense_range(conv_state, conv_w ? (int64_t)batch * (conv_width - 1) * cdim : 0, xe),
                       dense_range(dt, (int64_t)batch * nheads, ae),
                       dense_range(z, (int64_t)batch * HP, ae)};
  for (const Range& r : ins)
    if (overlap(ry, r)) return fail(SSD_ERR_INVALID_ARG, "state_update: y overlaps an input");
  for (int i = 1; i < 5; ++i)
    if (overlap(ins[0], ins[i]))
      return fail(SSD_ERR_INVALID_ARG, "state_update: state overlaps another tensor");
  for (int i = 0; i < 5; ++i)
    if (i != 2 && overlap(ins[2], ins[i]))
      return fail(SSD_ERR_INVALID_ARG, "state_update: conv_state overlaps another tensor");
  if (batch == 0) return SSD_OK;
  hipError_t e = launch_state_update(state, xbc, xbc_dtype, conv_state, conv_w, conv_b,
                                     conv_w ? conv_width : 1, dt, z, act_dtype, A, D, dt_bias,
                                     dt_softplus, y, y_dtype, batch, nheads, ngroups, stream);
  return e == hipSuccess ? SSD_OK : hip_fail(e, "state_update launch");
}

}  // extern "C"
