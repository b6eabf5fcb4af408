// Chunked selective scan on the gfx950 matrix cores (SSD_MATH_BF16).
//
// The recurrence h_t = exp(delta_t A) h_{t-1} + delta_t x_t B_t^T,
// y_t = C_t h_t + D x_t ("Hybrid Architectures for Language Models" summary,
// section 2 Background) is evaluated in its chunked matrix form (the same
// section: SSD recasts the state-space computation as matrix multiplies).
// For a chunk of Q = 128 tokens with cumulative log decay Lam_t:
//   Y      = (C B^T o exp(Lam_t - Lam_s) delta_s [s <= t]) X + diag(exp Lam) C H^T
//   H_next = exp(Lam_last) H + (X o w)^T B,  w_s = exp(Lam_last - Lam_s) delta_s
//   out    = (Y + D x) * silu(z)
// All products are 16x16x32 bf16 MFMAs with fp32 accumulation.  The chunk
// state product, whose result is carried across the whole sequence, splits
// both operands into bf16 hi + lo parts and sums hi*hi + hi*lo + lo*hi, so
// the carried state keeps ~16 mantissa bits instead of 8.
//
// One workgroup ("walker", 8 waves, two per SIMD so that each hides the
// other's LDS, matrix-core and memory latency) owns one (sequence, head) --
// or one segment of it, see below -- and walks its chunks in order, carrying
// the fp32 state H [64 x 128] in MFMA accumulator registers, so no state goes
// to HBM between chunks.  Wave w owns the 16 output rows of row tile
// rt(w) = w < 4 ? w : 11 - w (the two waves of a SIMD together own tiles
// i and 7 - i, which balances the causal triangle of C B^T) and the 16 state
// columns n in [16 w, 16 w + 16).
//
// LDS per walker (~151 KiB of gfx950's 160 KiB): B and x of the chunk in
// fp32 (the bf16 operands and their hi/lo parts are formed on the fly), C and
// the bf16 copy of H for the read-out, and the per-token decays.
//
// The decayed C B^T tile never touches LDS: it is produced as the transpose
// (B C^T, rows s, columns t) so that each lane's accumulator column is one
// output row t; after masking and decay, the 4 values a lane holds from each
// of two neighbouring 16-token tiles are exactly its 8 A-operand values for
// one K=32 step of M X, with the K index permuted the same way on the X side.
//
// Low (batch x heads) counts are split along the sequence: pass 1 runs the
// state-only walker on segments 0..S-2 from a zero state, a small combine
// kernel chains the segment states (H_in[k] = exp(sum of log decay of
// segment k-1) H_in[k-1] + H_loc[k-1]), and pass 2 walks every segment from
// its own incoming state.
//
// Walker order is XCD-aware: workgroups are dealt to the 8 XCDs round-robin,
// so consecutive walker indices are remapped to put the heads that read the
// same group's B and C (same sequence, group and segment) on one XCD, where
// they share its L2.
#include "ssd_common.h"

namespace ssd {
namespace {

constexpr int Q = 128;
constexpr int P = 64;
constexpr int N = 128;
constexpr int THREADS = 512;  // 8 waves
constexpr int NXCD = 8;
constexpr int LDB = N + 8;     // bf16 row stride of sC, sH (272 B: 16-B row reads conflict-free)
constexpr int LDB32 = N + 4;   // fp32 row stride of sB32 (528 B)
constexpr int LDX32 = Q + 4;   // fp32 row stride of sX32 [p][t] (528 B)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// D = A B + C for a 16x16 tile, K = 32.  Lane l = i + 16 q holds A[i][8q..8q+7],
// B[8q..8q+7][j = l % 16] and D[4q..4q+3][j = l % 16].
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 to_bf16x8(float4 a, float4 b) {
  bf16x8 r;
  r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
  r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
  return r;
}

// v = hi + lo with hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = (bf16)v[e];
    hi[e] = h;
    lo[e] = (bf16)(v[e] - (float)h);
  }
}

// 8 raw elements of one token row, kept packed between load and use
template <typename T> struct Raw8;
template <> struct Raw8<bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float* v) const {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <typename T>
__device__ __forceinline__ float ld1(const void* p, int64_t i) {
  return to_f32(static_cast<const T*>(p)[i]);
}

// 8 values -> LDS row, as fp32 or bf16
__device__ __forceinline__ void put8(float* dst, const float* v) {
  reinterpret_cast<float4*>(dst)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(dst)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void put8(bf16* dst, const float* v) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
  *reinterpret_cast<bf16x8*>(dst) = r;
}

// The rows of one 8-channel column piece a thread stages: positions
// tstart + i, i < R + HALO (HALO = 3 rows of conv history in front when the
// conv is fused).  Every load is unconditional: its address is chosen first
// -- positions before the sequence read the conv history, positions past
// its end re-read the last row -- and values outside the sequence and its
// history are zeroed when read back, so all loads of a chunk are in flight
// together.
template <typename Tx, int NR>
struct RowLoad {
  Raw8<Tx> v[NR];
  __device__ __forceinline__ void load(const ScanArgs& a, const Tx* src, int64_t stride, int col,
                                       int c0, int cdim, int b, int tstart) {
    const int L = a.seqlen, K = a.conv_k;
    const Tx* hist = static_cast<const Tx*>(a.conv_state_in);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int tau = tstart + i;
      const Tx* p;
      if (tau < 0 && hist != nullptr && tau >= -(K - 1))
        p = hist + ((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + c0;
      else
        p = src + ((int64_t)b * L + min(max(tau, 0), L - 1)) * stride + col;
      v[i].load(p);
    }
  }
  __device__ __forceinline__ void get(const ScanArgs& a, int tstart, int i, float* out) const {
    const int tau = tstart + i;
    const bool ok = tau < a.seqlen &&
                    (tau >= 0 || (a.conv_state_in != nullptr && tau >= -(a.conv_k - 1)));
    v[i].get(out);
    if (!ok) {
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] = 0.f;
    }
  }
};

// Depthwise conv + SiLU of R consecutive rows of 8 channels from R + 3 raw
// rows (the first 3 are the history in front); row i goes to dst + i * ld,
// zero for rows >= nvalid.  cw is the conv of the workgroup's channels in
// LDS: tap j of local channel c at cw[j * P + c] (taps right-aligned, zero in
// front when the width is below 4), the bias at cw[4 * P + c]; cl is the
// local channel of the first of the 8.
template <typename Tx, int R, typename Td>
__device__ __forceinline__ void conv_rows_to(const ScanArgs& a, const RowLoad<Tx, R + 3>& rl,
                                             int tstart, const float* cw, int cl, int rfirst,
                                             int nvalid, Td* dst, int ld) {
  float w4[4][8], bv[8];
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    const float4 lo = *reinterpret_cast<const float4*>(cw + j * P + cl);
    const float4 hi = *reinterpret_cast<const float4*>(cw + j * P + cl + 4);
    float* d = j < 4 ? w4[j] : bv;
    d[0] = lo.x; d[1] = lo.y; d[2] = lo.z; d[3] = lo.w;
    d[4] = hi.x; d[5] = hi.y; d[6] = hi.z; d[7] = hi.w;
  }
  float win[3][8];
  rl.get(a, tstart, 0, win[0]);
  rl.get(a, tstart, 1, win[1]);
  rl.get(a, tstart, 2, win[2]);
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float cur[8], o[8];
    rl.get(a, tstart, i + 3, cur);
    const bool ok = rfirst + i < nvalid;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = bv[e] + w4[0][e] * win[0][e] + w4[1][e] * win[1][e] +
                      w4[2][e] * win[2][e] + w4[3][e] * cur[e];
      o[e] = ok ? silu_f32(u) : 0.f;
      win[0][e] = win[1][e];
      win[1][e] = win[2][e];
      win[2][e] = cur[e];
    }
    put8(dst + i * ld, o);
  }
}

// Rows as they are (post-conv input), zero for rows >= nvalid.
template <typename Tx, int R, typename Td>
__device__ __forceinline__ void copy_rows_to(const ScanArgs& a, const RowLoad<Tx, R>& rl,
                                             int tstart, int rfirst, int nvalid, Td* dst, int ld) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float o[8];
    rl.get(a, tstart, i, o);
    if (rfirst + i >= nvalid)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = 0.f;
    put8(dst + i * ld, o);
  }
}

// One chunk's B and C for the whole workgroup: thread (cv = tid % 16,
// rg = tid / 16) owns rows [4 rg, 4 rg + 4) x channels [8 cv, 8 cv + 8) of B
// and of C (post-conv values of type Tbc).
template <typename Tbc, bool WITH_C>
struct StageBC {
  RowLoad<Tbc, 4> rb;
  RowLoad<Tbc, WITH_C ? 4 : 1> rc;

  __device__ __forceinline__ void load(const ScanArgs& a, int b, int g, int t0) {
    const int tid = threadIdx.x;
    const int cv = tid & 15, rg = tid >> 4;
    const int cdim = a.nheads * P + 2 * a.ngroups * N;
    rb.load(a, static_cast<const Tbc*>(a.Bm), a.b_stride, g * N + 8 * cv, 0, cdim, b,
            t0 + 4 * rg);
    if constexpr (WITH_C)
      rc.load(a, static_cast<const Tbc*>(a.Cm), a.c_stride, g * N + 8 * cv, 0, cdim, b,
              t0 + 4 * rg);
  }

  __device__ __forceinline__ void store(const ScanArgs& a, int t0, int Lc, float* sB32,
                                        bf16* sC) const {
    const int tid = threadIdx.x;
    const int cv = tid & 15, rg = tid >> 4;
    copy_rows_to<Tbc, 4>(a, rb, t0 + 4 * rg, 4 * rg, Lc, sB32 + (4 * rg) * LDB32 + 8 * cv, LDB32);
    if constexpr (WITH_C)
      copy_rows_to<Tbc, 4>(a, rc, t0 + 4 * rg, 4 * rg, Lc, sC + (4 * rg) * LDB + 8 * cv, LDB);
  }
};

// One chunk's x for the whole workgroup: thread (xv = tid % 8, xr = tid / 8)
// owns rows [2 xr, 2 xr + 2) x channels [8 xv, 8 xv + 8) (raw values of type
// Tx with 3 rows of history in front when XCONV, post-conv otherwise).
template <typename Tx, bool XCONV>
struct StageX {
  static constexpr int HX = XCONV ? 3 : 0;
  RowLoad<Tx, 2 + HX> rx;

  __device__ __forceinline__ void load(const ScanArgs& a, int b, int h, int t0) {
    const int tid = threadIdx.x;
    const int xv = tid & 7, xr = tid >> 3;
    const int cdim = a.nheads * P + 2 * a.ngroups * N;
    rx.load(a, static_cast<const Tx*>(a.x), a.x_stride, h * P + 8 * xv, h * P + 8 * xv, cdim, b,
            t0 + 2 * xr - HX);
  }

  // 2 rows x 8 channels, transposed into sX32[p][t]
  __device__ __forceinline__ void store(const ScanArgs& a, const float* cw, int t0, int Lc,
                                        float* sX32) const {
    const int tid = threadIdx.x;
    const int xv = tid & 7, xr = tid >> 3;
    float tmp[2 * 8];
    if constexpr (XCONV)
      conv_rows_to<Tx, 2>(a, rx, t0 + 2 * xr - 3, cw, 8 * xv, 2 * xr, Lc, tmp, 8);
    else
      copy_rows_to<Tx, 2>(a, rx, t0 + 2 * xr, 2 * xr, Lc, tmp, 8);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      *reinterpret_cast<float2*>(sX32 + (8 * xv + e) * LDX32 + 2 * xr) =
          make_float2(tmp[e], tmp[8 + e]);
  }
};

// In-place inclusive prefix sum of s[0..Q) by waves 0 and 1 (fixed order).
__device__ __forceinline__ void scan_lam(float* s, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float v = 0.f;
  if (tid < Q) {
    v = s[tid];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float o = __shfl_up(v, d, 64);
      if (lane >= d) v += o;
    }
    if (lane == 63) red[w] = v;
  }
  __syncthreads();
  if (tid >= 64 && tid < Q) s[tid] = v + red[0];
  if (tid < 64) s[tid] = v;
  __syncthreads();
}

// Walker index of this workgroup: (sequence b, head h, segment seg), with
// the heads of one (b, group, segment) contiguous and dealt to one XCD.
struct Walker {
  int b, h, seg;
};
__device__ __forceinline__ Walker walker_of(int lin, int total, int H, int G, int nsegs) {
  // item order: ((b * nsegs + seg) * G + g) * hpg + hh; lin -> item puts
  // item ranges of length total/8 on one XCD (lin % 8)
  const int per = total / NXCD;
  int item = lin;
  if (lin < per * NXCD) item = (lin % NXCD) * per + lin / NXCD;
  const int hpg = H / G;
  const int hh = item % hpg;
  int rest = item / hpg;
  const int g = rest % G;
  rest /= G;
  const int seg = rest % nsegs;
  const int b = rest / nsegs;
  return Walker{b, g * hpg + hh, seg};
}

template <typename Tx, typename Tbc, typename Ta, typename Ty, bool XCONV, bool STATE_ONLY>
__global__ __launch_bounds__(THREADS) void scan_bf16_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) float sB32[Q * LDB32];
  __shared__ __attribute__((aligned(16))) float sX32[P * LDX32];
  __shared__ __attribute__((aligned(16))) bf16 sC[STATE_ONLY ? 8 : Q * LDB];
  __shared__ __attribute__((aligned(16))) bf16 sH[STATE_ONLY ? 8 : P * LDB];
  __shared__ __attribute__((aligned(16))) float sLam[Q];
  __shared__ __attribute__((aligned(16))) float sDel[Q];
  __shared__ __attribute__((aligned(16))) float sW[Q];
  __shared__ float sRed[4];
  __shared__ __attribute__((aligned(16))) float sCw[XCONV ? 5 * P : 4];  // x-channel conv

  const int H = a.nheads, G = a.ngroups, L = a.seqlen;
  // pass 1 (state-only) walks segments 0..nseg-2, pass 2 all segments
  const int nsegs = STATE_ONLY ? a.nseg - 1 : a.nseg;
  const Walker wk = walker_of(blockIdx.x, gridDim.x, H, G, nsegs);
  const int b = wk.b, h = wk.h, seg = wk.seg;
  const int bh = b * H + h;
  const int hpg = H / G, g = h / hpg;
  const int HP = H * P, GN = G * N, cdim = HP + 2 * GN;
  const int nc = (L + Q - 1) / Q;
  const int cbeg = seg * a.seg_chunks;
  const int cend = min(nc, cbeg + a.seg_chunks);

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  const int rt = w < 4 ? w : 11 - w;  // output row tile: rows [16 rt, 16 rt + 16)
  const int ncol = 16 * w + l16;      // state column n of this lane
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.f;
  const Tx* xg = static_cast<const Tx*>(a.x);

  // ---- incoming state: element r of hacc[pt] is (p = 16 pt + 4 q + r, n = ncol)
  const float* h_in = nullptr;
  if (!STATE_ONLY) {
    if (a.nseg > 1)
      h_in = a.seg_state + ((int64_t)bh * a.nseg + seg) * P * N;
    else
      h_in = a.initial_state ? a.initial_state + (int64_t)bh * P * N : nullptr;
  }
  f32x4 hacc[4];
#pragma unroll
  for (int pt = 0; pt < 4; ++pt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * pt + 4 * q + r;
      hacc[pt][r] = h_in ? h_in[p * N + ncol] : 0.f;
      if (!STATE_ONLY) sH[p * LDB + ncol] = (bf16)hacc[pt][r];
    }
  float log_decay = 0.f;  // sum of delta*A over the segment (state-only pass)
  if (XCONV && tid < P) {
    // the conv of this head's x channels: read at every chunk from LDS (the
    // first read follows the barrier at the top of the chunk loop)
    const int K = a.conv_k;
    const int64_t ch = (int64_t)h * P + tid;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = j - (4 - K);
      sCw[j * P + tid] = k >= 0 ? a.conv_w[ch * K + k] : 0.f;
    }
    sCw[4 * P + tid] = a.conv_b ? a.conv_b[ch] : 0.f;
  }

  // Chunk c+1's x and dt are loaded as soon as chunk c is in LDS, so they are
  // in flight while chunk c is computed.  B and C, which the heads of a group
  // share through L2, are loaded at the top of their own chunk, and z after
  // the staging, ahead of its use in the epilogue.
  StageX<Tx, XCONV> sx;
  float dtv = 0.f;
  auto prefetch = [&](int cc) {
    const int tt0 = cc * Q;
    sx.load(a, b, h, tt0);
    if (tid < Q)
      dtv = ld1<Ta>(a.dt, ((int64_t)b * L + min(tt0 + tid, L - 1)) * a.dt_stride + h);
  };
  if (cbeg < cend) prefetch(cbeg);

  for (int c = cbeg; c < cend; ++c) {
    const int t0 = c * Q;
    const int Lc = min(Q, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;
    StageBC<Tbc, !STATE_ONLY> sbc;
    sbc.load(a, b, g, t0);
    __syncthreads();  // the previous chunk is done with every LDS buffer
    if (tid < Q) {
      const float d = tid < Lc ? make_delta(dtv, a.dt_bias, h, a.dt_softplus) : 0.f;
      sDel[tid] = d;
      sLam[tid] = d * Ah;
    }
    sx.store(a, sCw, t0, Lc, sX32);
    sbc.store(a, t0, Lc, sB32, sC);
    if (c + 1 < cend) prefetch(c + 1);
    // z in the accumulator layout: zr[pj][r] is (t = 16 rt + 4 q + r,
    // p = 16 pj + l16); rows past the end re-read the last row, never stored
    float zr[4][4];
#pragma unroll
    for (int pj = 0; pj < 4; ++pj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = min(16 * rt + 4 * q + r, Lc - 1);
        zr[pj][r] = (!STATE_ONLY && a.z != nullptr)
                        ? ld1<Ta>(a.z, (row0 + t) * a.z_stride + h * P + 16 * pj + l16)
                        : 0.f;
      }
    __syncthreads();
    scan_lam(sLam, sRed);
    const float lam_last = sLam[Q - 1];
    if (STATE_ONLY) log_decay += lam_last;
    if (tid < Q) sW[tid] = __expf(lam_last - sLam[tid]) * sDel[tid];
    __syncthreads();

    if (!STATE_ONLY) {
      // ---- inter-chunk read-out: Y = diag(exp Lam) C H^T;
      //      element r of yacc[pj] is (t = 16 rt + 4 q + r, p = 16 pj + l16)
      f32x4 yacc[4] = {};
      const bf16* crow = sC + (16 * rt + l16) * LDB + 8 * q;
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk) {
        const bf16x8 af = lds8(crow + 32 * kk);
#pragma unroll
        for (int pj = 0; pj < 4; ++pj)
          yacc[pj] = mfma(af, lds8(sH + (16 * pj + l16) * LDB + 32 * kk + 8 * q), yacc[pj]);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __expf(sLam[16 * rt + 4 * q + r]);
#pragma unroll
        for (int pj = 0; pj < 4; ++pj) yacc[pj][r] *= e;
      }

      // ---- intra-chunk: Y += (C B^T o decay mask) X over the source tiles
      //      u <= rt, two 16-token tiles per K=32 step
      const int tcol = 16 * rt + l16;
      const float lam_t = sLam[tcol];
      for (int u0 = 0; u0 <= rt; u0 += 2) {
        bf16x8 mf;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int u = u0 + half;
          f32x4 cb = {};
          if (u <= rt) {
            const float* brow = sB32 + (16 * u + l16) * LDB32 + 8 * q;
#pragma unroll
            for (int kk = 0; kk < N / 32; ++kk) {
              const float4* bp = reinterpret_cast<const float4*>(brow + 32 * kk);
              cb = mfma(to_bf16x8(bp[0], bp[1]), lds8(crow + 32 * kk), cb);
            }
          }
          // cb[r] = (B C^T)[s = 16 u + 4 q + r][t = tcol]
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = 16 * u + 4 * q + r;
            const float m = (u <= rt && s <= tcol) ? cb[r] * __expf(lam_t - sLam[s]) * sDel[s] : 0.f;
            mf[4 * half + r] = (bf16)m;
          }
        }
#pragma unroll
        for (int pj = 0; pj < 4; ++pj) {
          const float* xp = sX32 + (16 * pj + l16) * LDX32 + 4 * q;
          const bf16x8 xf = to_bf16x8(*reinterpret_cast<const float4*>(xp + 16 * u0),
                                      *reinterpret_cast<const float4*>(xp + 16 * u0 + 16));
          yacc[pj] = mfma(mf, xf, yacc[pj]);
        }
      }

      // ---- epilogue: skip, gate, store
      Ty* yg = static_cast<Ty*>(a.y);
      const int tb = 16 * rt + 4 * q;
#pragma unroll
      for (int pj = 0; pj < 4; ++pj) {
        const float4 xq = *reinterpret_cast<const float4*>(sX32 + (16 * pj + l16) * LDX32 + tb);
        const float xs[4] = {xq.x, xq.y, xq.z, xq.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (tb + r < Lc) {
            float yv = yacc[pj][r] + Dh * xs[r];
            if (a.z != nullptr) yv *= silu_f32(zr[pj][r]);
            yg[(row0 + tb + r) * a.y_stride + h * P + 16 * pj + l16] = from_f32<Ty>(yv);
          }
        }
      }
      __syncthreads();  // every wave is done reading sH
    }

    // ---- state: H <- exp(Lam_last) H + (X o w)^T B, operands split hi + lo;
    //      this wave's columns n = 16 w + l16, all 64 rows p
    const float gamma = __expf(lam_last);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) hacc[pt] *= gamma;
#pragma unroll
    for (int kk = 0; kk < Q / 32; ++kk) {
      const int s0 = 32 * kk + 8 * q;
      float bv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) bv[e] = sB32[(s0 + e) * LDB32 + ncol];
      bf16x8 bhi, blo;
      split8(bv, bhi, blo);
      const float4 w0 = *reinterpret_cast<const float4*>(sW + s0);
      const float4 w1 = *reinterpret_cast<const float4*>(sW + s0 + 4);
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const float* xr = sX32 + (16 * pt + l16) * LDX32 + s0;
        const float4 x0 = *reinterpret_cast<const float4*>(xr);
        const float4 x1 = *reinterpret_cast<const float4*>(xr + 4);
        const float xw[8] = {x0.x * w0.x, x0.y * w0.y, x0.z * w0.z, x0.w * w0.w,
                             x1.x * w1.x, x1.y * w1.y, x1.z * w1.z, x1.w * w1.w};
        bf16x8 ahi, alo;
        split8(xw, ahi, alo);
        hacc[pt] = mfma(ahi, bhi, hacc[pt]);
        hacc[pt] = mfma(ahi, blo, hacc[pt]);
        hacc[pt] = mfma(alo, bhi, hacc[pt]);
      }
    }
    if (!STATE_ONLY) {
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sH[(16 * pt + 4 * q + r) * LDB + ncol] = (bf16)hacc[pt][r];
    }
  }

  // ---- outgoing state
  float* h_out = nullptr;
  if (STATE_ONLY)
    h_out = a.seg_state + ((int64_t)bh * a.nseg + seg + 1) * P * N;
  else if (seg == a.nseg - 1)
    h_out = a.final_state ? a.final_state + (int64_t)bh * P * N : nullptr;
  if (h_out != nullptr) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int r = 0; r < 4; ++r) h_out[(16 * pt + 4 * q + r) * N + ncol] = hacc[pt][r];
  }
  if (STATE_ONLY && tid == 0) a.seg_logdecay[(int64_t)bh * a.nseg + seg] = log_decay;

  // ---- conv history hand-over of this head's x channels (last segment; the
  //      B and C channels are handed over by their conv pass)
  if (XCONV && !STATE_ONLY && seg == a.nseg - 1 && a.conv_state_out != nullptr) {
    const int K = a.conv_k;
    Tx* out = static_cast<Tx*>(a.conv_state_out);
    const Tx* hin = static_cast<const Tx*>(a.conv_state_in);
    for (int i = tid; i < (K - 1) * P; i += THREADS) {
      const int j = i / P, c = h * P + i % P;
      const int tau = L - (K - 1) + j;  // < L
      Tx v = from_f32<Tx>(0.f);
      if (tau >= 0)
        v = xg[((int64_t)b * L + tau) * a.x_stride + c];
      else if (hin != nullptr)
        v = hin[((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + c];
      out[((int64_t)b * (K - 1) + j) * cdim + c] = v;
    }
  }
}

// H_in[0] = h0; H_in[k] = exp(log_decay[k-1]) H_in[k-1] + H_loc[k-1], in place:
// slot k holds H_loc[k-1] on entry and H_in[k] on exit.
__global__ __launch_bounds__(THREADS) void combine_segments_kernel(ScanArgs a) {
  const int bh = blockIdx.x;
  float* slots = a.seg_state + (int64_t)bh * a.nseg * P * N;
  const float* ld = a.seg_logdecay + (int64_t)bh * a.nseg;
  for (int i = threadIdx.x; i < P * N; i += THREADS) {
    float carry = a.initial_state ? a.initial_state[(int64_t)bh * P * N + i] : 0.f;
    slots[i] = carry;
    for (int k = 1; k < a.nseg; ++k) {
      carry = __expf(ld[k - 1]) * carry + slots[(int64_t)k * P * N + i];
      slots[(int64_t)k * P * N + i] = carry;
    }
  }
}

template <typename Tx, typename Tbc, typename Ta, typename Ty, bool XCONV>
hipError_t launch_walkers(const ScanArgs& a, hipStream_t stream) {
  const int BH = a.batch * a.nheads;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((scan_bf16_kernel<Tx, Tbc, Ta, Ty, XCONV, true>), dim3(BH * (a.nseg - 1)),
                       dim3(THREADS), 0, stream, a);
    hipLaunchKernelGGL(combine_segments_kernel, dim3(BH), dim3(THREADS), 0, stream, a);
  }
  hipLaunchKernelGGL((scan_bf16_kernel<Tx, Tbc, Ta, Ty, XCONV, false>), dim3(BH * a.nseg),
                     dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename Ta, typename Ty>
hipError_t pick_x(const ScanArgs& a, ssd_dtype_t xd, hipStream_t s) {
  if (a.conv_w != nullptr)  // raw x, post-conv fp32 B and C from the conv pass
    return xd == SSD_BF16 ? launch_walkers<bf16, float, Ta, Ty, true>(a, s)
                          : launch_walkers<float, float, Ta, Ty, true>(a, s);
  return xd == SSD_BF16 ? launch_walkers<bf16, bf16, Ta, Ty, false>(a, s)
                        : launch_walkers<float, float, Ta, Ty, false>(a, s);
}

}  // namespace

hipError_t launch_scan_bf16(const ScanArgs& a, ssd_dtype_t xd, ssd_dtype_t ad, ssd_dtype_t yd,
                            hipStream_t s) {
  if (ad == SSD_BF16)
    return yd == SSD_F32 ? pick_x<bf16, float>(a, xd, s) : pick_x<bf16, bf16>(a, xd, s);
  return yd == SSD_F32 ? pick_x<float, float>(a, xd, s) : pick_x<float, bf16>(a, xd, s);
}

}  // namespace ssd
