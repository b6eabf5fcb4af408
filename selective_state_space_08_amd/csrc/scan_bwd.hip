// The layer's backward pass: the gradients of a loss with respect to every
// input of ssd_chunk_scan_fwd, given the gradient of its output (and of its
// final state).  Reverse-mode differentiation of the recurrence of "Hybrid
// Architectures for Language Models: Systematic Analysis and Design
// Insights" (Korean summary), section 2 Background, in the chunked form the
// forward pass uses, fp32 throughout: the products of size P x N on the
// fp32 matrix cores, the rest on the vector ALUs.
//
// Kernels, in launch order:
//   1. the post-conv x|B|C in fp32 (the conv kernel, or a conversion);
//   2. fwd_states_kernel: the state entering every chunk, per (b, h);
//   3. bwd_chunk_kernel: per (b, h), the chunks in reverse order with the
//      state's gradient carried in registers; per chunk it forms the
//      gradients of x (this head), of B and C (this head's share), of dt and
//      z, and the per-(b, h) sums for A, D and dt_bias;
//   4. reduce_bc_kernel: the heads of a group add up their B and C shares;
//   5. (conv) conv_bwd_kernel: the gradients of the raw inputs, of the conv
//      history, and per-block sums for the conv weights and bias;
//   6. reduce_params_kernel: those per-block and per-(b, h) sums, in a fixed
//      order (no atomics: the result is bitwise reproducible).
#include "ssd_common.h"

namespace ssd {
namespace {

constexpr int BQ = 32;    // tokens per chunk
constexpr int BP = 64;    // head dim
constexpr int BN = 128;   // state dim
constexpr int BT = 256;   // threads
// LDS pitches of the [.][n], [.][p] and [.][s] tiles: 12 mod 64 floats, so
// that 16 lanes reading 16 rows at one column, or 16 columns of one row,
// hit distinct banks
constexpr int QN = BN + 12;
constexpr int QP = BP + 12;
constexpr int QQ = BQ + 12;

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ float ld(const T* p) { return to_f32(*p); }

__device__ __forceinline__ float silu_grad_f32(float u) {
  const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-u));
  return sg * (1.f + u * (1.f - sg));
}

struct BwdArgs {
  const float* post;          // [B, L, Cdim] post-conv x|B|C, fp32
  const void* dt; int64_t dt_stride;
  const void* z; int64_t z_stride;
  const void* dout; int64_t dout_stride;
  const float* A; const float* D; const float* dt_bias; int dt_softplus;
  const float* h0; const float* dhT;
  float* states;              // [B, H, nc, P, N]
  float* dpost;               // [B, L, Cdim]: x part written here
  float* dBh; float* dCh;     // [B, L, H, N]: a token's heads side by side
  float* ddt;                 // [B, L, H]
  float* dz;                  // [B, L, H, P] or null
  float* dh0;                 // [B, H, P, N] or null
  float* part;                // [B, H, 3]: dA, dD, dt_bias sums
  int batch, seqlen, nheads, ngroups, nc, cdim;
};

// delta of token t (0 past the end); v is dt + dt_bias (for softplus')
template <typename Ta>
__device__ __forceinline__ float delta_of(const BwdArgs& a, int64_t row, int h, bool valid,
                                          float& v) {
  v = 0.f;
  if (!valid) return 0.f;
  v = ld(static_cast<const Ta*>(a.dt) + row * a.dt_stride + h) + (a.dt_bias ? a.dt_bias[h] : 0.f);
  return a.dt_softplus ? softplus_f32(v) : v;
}

// D = A B + D for one 16x16 fp32 tile and K = 4 on the matrix cores.  Lane
// l = i + 16 q holds A[i][q] and B[q][i] and ends with D[4 q + r][i], r < 4.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The products of one group of 16 k.  Lane (i, q) holds the 4 consecutive
// k = 4 q .. 4 q + 3 of the group: for operands stored with k contiguous
// they are one float4 read; step e takes k = 4 q + e on both sides, which
// is a permutation of the group's 16 k.
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 mfma_k16(f32x4 a4, f32x4 b4, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 4; ++e) acc = mfma4(a4[e], b4[e], acc);
  return acc;
}

// One activation element, kept raw between its load and its use, so that a
// load issued ahead of time is not waited for at the load.
template <typename T> struct RawS;
template <> struct RawS<bf16> {
  unsigned short u = 0;
  __device__ __forceinline__ void load(const bf16* p) {
    u = *reinterpret_cast<const unsigned short*>(p);
  }
  __device__ __forceinline__ float get() const { return __uint_as_float((uint32_t)u << 16); }
};
template <> struct RawS<float> {
  float f = 0.f;
  __device__ __forceinline__ void load(const float* p) { f = *p; }
  __device__ __forceinline__ float get() const { return f; }
};

// ---------------------------------------------------------------- states

// The state entering each chunk, for every (b, h): states[b][h][c] = H before
// chunk c, with H <- e^lam_last H + (x o w)^T B per chunk on the fp32 matrix
// cores.  4 waves; wave w holds the [p][n] tiles (w, 0..7) of the state in
// accumulator registers (lane l = i + 16 q: p = 16 w + 4 q + r,
// n = 16 nt + i).  x and B are staged transposed ([p][s], [n][s]) so that
// each lane reads 4 consecutive s as one float4.  The next chunk's x, B and
// dt are loaded into registers (unconditionally; rows past the end of the
// sequence are zeroed when staged) while this chunk is applied.
template <typename Ta>
__global__ __launch_bounds__(BT) void fwd_states_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float sXT[BP][QQ];
  __shared__ __attribute__((aligned(16))) float sBT[BN][QQ];
  __shared__ __attribute__((aligned(16))) float sW[BQ];
  __shared__ float sGam;
  const int H = a.nheads, G = a.ngroups, L = a.seqlen;
  const int b = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);
  const int HP = H * BP;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;
  f32x4 hs[8];
  {
    const float* h0 = a.h0 ? a.h0 + ((int64_t)b * H + h) * BP * BN : nullptr;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        hs[nt][e] = h0 ? h0[(16 * w + 4 * lq + e) * BN + 16 * nt + li] : 0.f;
  }
  const float Ah = a.A[h];
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.f;
  // staging: x as 2 float4s per thread (t = tid / 16 + 16 k, p4 = 4 (tid % 16)),
  // B as 4 float4s (t = tid / 32 + 8 k, n4 = 4 (tid % 32)), dt (lane t % 32)
  const int xt = tid >> 4, p4 = 4 * (tid & 15), bt = tid >> 5, n4 = 4 * (tid & 31);
  f32x4 px0, px1, pb0, pb1, pb2, pb3;
  RawS<Ta> pdt;
  auto fetch = [&](int c) {
    const int t0 = c * BQ, Lc = min(BQ, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;
    auto row = [&](int t) { return a.post + (row0 + min(t, Lc - 1)) * a.cdim; };
    px0 = *reinterpret_cast<const f32x4*>(row(xt) + h * BP + p4);
    px1 = *reinterpret_cast<const f32x4*>(row(xt + 16) + h * BP + p4);
    pb0 = *reinterpret_cast<const f32x4*>(row(bt) + HP + g * BN + n4);
    pb1 = *reinterpret_cast<const f32x4*>(row(bt + 8) + HP + g * BN + n4);
    pb2 = *reinterpret_cast<const f32x4*>(row(bt + 16) + HP + g * BN + n4);
    pb3 = *reinterpret_cast<const f32x4*>(row(bt + 24) + HP + g * BN + n4);
    pdt.load(static_cast<const Ta*>(a.dt) + (row0 + min(tid & 31, Lc - 1)) * a.dt_stride + h);
  };
  if (a.nc > 0) fetch(0);
  for (int c = 0; c < a.nc; ++c) {
    const int t0 = c * BQ, Lc = min(BQ, L - t0);
    {
      auto put = [&](float (*dst)[QQ], int r0, int t, f32x4 v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[r0 + e][t] = t < Lc ? v[e] : 0.f;
      };
      put(sXT, p4, xt, px0);
      put(sXT, p4, xt + 16, px1);
      put(sBT, n4, bt, pb0);
      put(sBT, n4, bt + 8, pb1);
      put(sBT, n4, bt + 16, pb2);
      put(sBT, n4, bt + 24, pb3);
    }
    if (w == 0) {
      const int t = lane & 31;
      const bool real = lane < BQ && t < Lc;
      const float v = pdt.get() + dtb;
      float d = a.dt_softplus ? softplus_f32(v) : v;
      if (!real) d = 0.f;
      float lam = d * Ah;
      for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_up(lam, o, 64);
        if (t >= o) lam += u;
      }
      const float last = __shfl(lam, Lc - 1, 64);
      if (lane < BQ) sW[t] = __expf(last - lam) * d;
      if (lane == 0) sGam = __expf(last);
    }
    __syncthreads();
    if (c + 1 < a.nc) fetch(c + 1);
    float* st = a.states + (((int64_t)b * H + h) * a.nc + c) * BP * BN;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) st[(16 * w + 4 * lq + e) * BN + 16 * nt + li] = hs[nt][e];
    const float gam = sGam;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) hs[nt] *= gam;
#pragma unroll
    for (int gq = 0; gq < BQ / 16; ++gq) {
      const int s0 = 16 * gq + 4 * lq;
      const f32x4 a4 = lds4(&sXT[16 * w + li][s0]) * lds4(&sW[s0]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) hs[nt] = mfma_k16(a4, lds4(&sBT[16 * nt + li][s0]), hs[nt]);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- backward

// Block sum of one value per thread (fixed order), returned to every thread.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* sred) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sred[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += sred[i];
  return s;
}

constexpr int WT = 512;  // threads of the reverse walker: 8 waves, two per SIMD

// v moved across lanes by the DPP control CTRL within each row of 16 lanes
// (lanes whose source is outside the row read 0)
template <int CTRL>
__device__ __forceinline__ float dpp_row_or0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a row (lanes 16 k .. 16 k + 15) by DPP row shifts
// (1, 2, 4, 8: an inclusive prefix sum), in registers; complete in the row's
// last lane (16 k + 15), in a fixed order.
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_row_or0<0x111>(v);
  v += dpp_row_or0<0x112>(v);
  v += dpp_row_or0<0x114>(v);
  v += dpp_row_or0<0x118>(v);
  return v;
}

// One chunk's x, B, C (post-conv rows), the state entering it and dt, in
// registers: thread tid holds the float4 tid of x [t][p], the float4s
// tid + WT k of B and C [t][n] and of the state [p][n], and (threads of
// wave 0) dt of token tid % 32.  Every load is unconditional (rows past the
// end of the sequence re-read its last row), so that none waits for another
// and no address is selected per lane; the rows past the end are zeroed
// when stored (store()).
template <typename Ta>
struct ChunkRegs {
  f32x4 x, b0, b1, c0, c1, h0, h1, h2, h3;
  RawS<Ta> dt;

  __device__ __forceinline__ void load(const BwdArgs& a, const float* st, int64_t row0, int Lc,
                                       int h, int g) {
    const int tid = threadIdx.x;
    const int HP = a.nheads * BP, GN = a.ngroups * BN;
    auto row = [&](int t) { return a.post + (row0 + min(t, Lc - 1)) * a.cdim; };
    {
      const int t = tid >> 4, p4 = 4 * (tid & 15);
      x = *reinterpret_cast<const f32x4*>(row(t) + h * BP + p4);
    }
    {
      const int t = tid >> 5, n4 = 4 * (tid & 31);
      b0 = *reinterpret_cast<const f32x4*>(row(t) + HP + g * BN + n4);
      c0 = *reinterpret_cast<const f32x4*>(row(t) + HP + GN + g * BN + n4);
      b1 = *reinterpret_cast<const f32x4*>(row(t + 16) + HP + g * BN + n4);
      c1 = *reinterpret_cast<const f32x4*>(row(t + 16) + HP + GN + g * BN + n4);
    }
    {
      const f32x4* s4 = reinterpret_cast<const f32x4*>(st) + tid;
      h0 = s4[0];
      h1 = s4[WT];
      h2 = s4[2 * WT];
      h3 = s4[3 * WT];
    }
    // (every lane loads; lanes past the chunk re-read its first token)
    const int t = tid & 31;
    dt.load(static_cast<const Ta*>(a.dt) + (row0 + min(t, Lc - 1)) * a.dt_stride + h);
  }

  // x, B, C and the state into LDS, rows t >= Lc of x, B, C as zeros
  __device__ __forceinline__ void store(float (*sX)[QP], float (*sB)[QN], float (*sC)[QN],
                                        float (*sH)[QN], int Lc) const {
    const int tid = threadIdx.x;
    const f32x4 zero4 = {};
    {
      const int t = tid >> 4;
      *reinterpret_cast<f32x4*>(&sX[t][4 * (tid & 15)]) = t < Lc ? x : zero4;
    }
    const int t = tid >> 5, n4 = 4 * (tid & 31);
    *reinterpret_cast<f32x4*>(&sB[t][n4]) = t < Lc ? b0 : zero4;
    *reinterpret_cast<f32x4*>(&sC[t][n4]) = t < Lc ? c0 : zero4;
    *reinterpret_cast<f32x4*>(&sB[t + 16][n4]) = t + 16 < Lc ? b1 : zero4;
    *reinterpret_cast<f32x4*>(&sC[t + 16][n4]) = t + 16 < Lc ? c1 : zero4;
    *reinterpret_cast<f32x4*>(&sH[t][n4]) = h0;
    *reinterpret_cast<f32x4*>(&sH[t + 16][n4]) = h1;
    *reinterpret_cast<f32x4*>(&sH[t + 32][n4]) = h2;
    *reinterpret_cast<f32x4*>(&sH[t + 48][n4]) = h3;
  }
};

// The reverse walk over one (b, h), 8 waves, five barriers per chunk.  All
// products run on the fp32 matrix cores in 16x16 tiles (lane l = i + 16 q
// of a tile holds rows 4 q .. 4 q + 3 of column i):
//   - S = C B^T and dM = dY X^T: the three causal [t][s] tiles (S in two K
//     halves on waves 0..5, dM on waves 5..7);
//   - Yoff = e^lam C H_in^T + M X, and HB = B dH_out^T + ... for dx: the
//     [t][p] tile (w / 4, w % 4) of each wave, where the gate and the
//     gradient of x are then formed element by element;
//   - dC = e^lam dY H_in + dS B and dB = w X dH_out + dS^T C: the [t][n]
//     tiles (w / 4, 2 (w % 4) + 0/1);
//   - dH <- e^lam_last dH + (e^lam dY)^T C: the [p][n] tiles (w / 2,
//     4 (w % 2) + 0..3), kept in accumulator registers across the chunks.
// The next chunk's x, B, C, entering state and dt are loaded into
// registers while the current chunk is computed (dout and z one phase
// later).  LDS pitches are 12 mod 64 floats, so that 16 lanes reading 16
// rows at one column, or 16 columns of one row, hit distinct banks.
template <typename Ta, typename Td>
__global__ __launch_bounds__(WT) void bwd_chunk_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) float sX[BQ][QP];
  __shared__ __attribute__((aligned(16))) float sDY[BQ][QP];
  __shared__ __attribute__((aligned(16))) float sB[BQ][QN];
  __shared__ __attribute__((aligned(16))) float sC[BQ][QN];
  __shared__ __attribute__((aligned(16))) float sH[BP][QN];    // state entering the chunk
  __shared__ __attribute__((aligned(16))) float sDH[BP][QN];   // gradient of the state leaving it
  __shared__ __attribute__((aligned(16))) float sSX[BQ][QQ];  // (C_t . B_s) exp(lam_t - lam_s), s <= t; M_ts = sSX delta_s
  // dM_ts exp(lam_t - lam_s) delta_s, and dM_ts S_ts exp(lam_t - lam_s);
  // before that, the two K halves of S
  __shared__ __attribute__((aligned(16))) float sDS[BQ][QQ];
  __shared__ __attribute__((aligned(16))) float sE[BQ][QQ];
  __shared__ __attribute__((aligned(16))) float sDel[BQ];
  __shared__ __attribute__((aligned(16))) float sLam[BQ];
  __shared__ __attribute__((aligned(16))) float sEl[BQ];
  __shared__ float sV[BQ];
  // per-tile partial sums over p (4 p tiles) and over s or t (2 tiles)
  __shared__ float sDLp[4][BQ], sDWp[4][BQ], sRowP[2][BQ], sColP[2][BQ];
  __shared__ float sRed[WT / 64];

  const int H = a.nheads, G = a.ngroups, L = a.seqlen;
  const int b = blockIdx.x / H, h = blockIdx.x % H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lq = lane >> 4;  // matrix-core lane coordinates
  const float Ah = a.A[h], Dh = a.D ? a.D[h] : 0.f;
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.f;
  // this wave's tiles: [t][p] tile (ty, py); [t][n] tiles (ty, nb + 0/1);
  // dH tiles (hp, hn + 0..3)
  const int ty = w >> 2, py = w & 3, nb = 2 * (w & 3);
  const int hp = w >> 1, hn = 4 * (w & 1);
  const int pcol = 16 * py + li;  // the lane's column p in its [t][p] tile
  const float* states_bh = a.states + ((int64_t)b * H + h) * a.nc * BP * BN;

  f32x4 dh[4];
  {
    const float* src = a.dhT ? a.dhT + ((int64_t)b * H + h) * BP * BN : nullptr;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dh[j][e] = src ? src[(16 * hp + 4 * lq + e) * BN + 16 * (hn + j) + li] : 0.f;
  }
  float dD_part = 0.f, dA_part = 0.f, dbias_part = 0.f;

  // ---- the next chunk's operands, in registers
  ChunkRegs<Ta> nx;
  auto fetch_main = [&](int c) {
    const int t0 = c * BQ;
    nx.load(a, states_bh + (int64_t)c * BP * BN, (int64_t)b * L + t0, min(BQ, L - t0), h, g);
  };
  // dout and z of the lane's 4 elements (t = 16 ty + 4 lq + e, p = pcol)
  RawS<Td> pdo[4];
  RawS<Ta> pz[4];
  auto fetch_gate = [&](int c) {
    const int t0 = c * BQ, Lc = min(BQ, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;
    const Td* dob = static_cast<const Td*>(a.dout) + row0 * a.dout_stride + h * BP + pcol;
    const Ta* zb = a.z ? static_cast<const Ta*>(a.z) + row0 * a.z_stride + h * BP + pcol : nullptr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = min(16 * ty + 4 * lq + e, Lc - 1);  // (rows past the end: never used)
      pdo[e].load(dob + (int64_t)t * a.dout_stride);
      if (a.z) pz[e].load(zb + (int64_t)t * a.z_stride);
    }
  };
  if (a.nc > 0) {
    fetch_main(a.nc - 1);
    fetch_gate(a.nc - 1);
  }

  for (int c = a.nc - 1; c >= 0; --c) {
    const int t0 = c * BQ, Lc = min(BQ, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;

    // ---- P0: the chunk into LDS; the next chunk's loads; delta and lam
    nx.store(sX, sB, sC, sH, Lc);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sDH[16 * hp + 4 * lq + e][16 * (hn + j) + li] = dh[j][e];
    if (w == 0) {
      const int t = lane & 31;
      const bool real = lane < BQ && t < Lc;
      const float v = real ? nx.dt.get() + dtb : 0.f;
      float d = a.dt_softplus ? softplus_f32(v) : v;
      if (!real) d = 0.f;
      float lam = d * Ah;
      for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_up(lam, o, 64);
        if (t >= o) lam += u;
      }
      if (lane < BQ) {
        sDel[t] = d;
        sLam[t] = lam;
        sEl[t] = __expf(lam);
        sV[t] = v;
      }
    }
    if (c > 0) fetch_main(c - 1);
    __syncthreads();  // B1
    const float lam_last = sLam[Lc - 1];
    const float gam = __expf(lam_last);

    // ---- P1: S (two K halves, waves 0..5), Yoff and HB tiles, <dH, H_in>
    if (w < 6) {
      const int tsel = w >> 1, kh = w & 1;
      const int tt = tsel == 0 ? 0 : 1, ts = tsel == 2 ? 1 : 0;
      f32x4 sp = {};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k0 = 64 * kh + 16 * j + 4 * lq;
        sp = mfma_k16(lds4(&sC[16 * tt + li][k0]), lds4(&sB[16 * ts + li][k0]), sp);
      }
      float(*dst)[QQ] = kh == 0 ? sDS : sE;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[16 * tt + 4 * lq + e][16 * ts + li] = sp[e];
    }
    f32x4 yo = {}, hb = {};
#pragma unroll 2
    for (int j = 0; j < BN / 16; ++j) {
      const int k0 = 16 * j + 4 * lq;
      const f32x4 c4 = lds4(&sC[16 * ty + li][k0]), h4 = lds4(&sH[pcol][k0]);
      const f32x4 b4 = lds4(&sB[16 * ty + li][k0]), d4 = lds4(&sDH[pcol][k0]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        yo = mfma4(c4[e], h4[e], yo);
        hb = mfma4(b4[e], d4[e], hb);
      }
    }
    {
      float hh = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          hh = fmaf(dh[j][e], sH[16 * hp + 4 * lq + e][16 * (hn + j) + li], hh);
      for (int o = 32; o > 0; o >>= 1) hh += __shfl_xor(hh, o, 64);
      if (lane == 0) sRed[w] = hh;
    }
    __syncthreads();  // B2

    // ---- P2: M = (S o exp) delta (this wave's rows, written once to sSX),
    //      y = Yoff + M X + D x, the gate and its gradient; dw partials
    {
      // dz of this lane's column p at token t: dzrow[t * H * P]
      float* dzrow = a.dz ? a.dz + (row0 * H + h) * BP + pcol : nullptr;
      // e^lam_t Yoff, the inter-chunk part of y (also for the gradient of lam)
#pragma unroll
      for (int e = 0; e < 4; ++e) yo[e] *= sEl[16 * ty + 4 * lq + e];
      f32x4 yv = yo;
      const int ta = 16 * ty + li;   // the A operand's row t
      const float lam_a = sLam[ta];
#pragma unroll
      for (int j = 0; j < BQ / 16; ++j) {
        const int s0 = 16 * j + 4 * lq;
        const f32x4 p0 = lds4(&sDS[ta][s0]), p1 = lds4(&sE[ta][s0]);
        const f32x4 l4 = lds4(&sLam[s0]), d4 = lds4(&sDel[s0]);
        float xb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) xb[e] = sX[s0 + e][pcol];
        f32x4 sx;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sx[e] = s0 + e <= ta ? (p0[e] + p1[e]) * __expf(lam_a - l4[e]) : 0.f;
        if (py == 0) *reinterpret_cast<f32x4*>(&sSX[ta][s0]) = sx;
#pragma unroll
        for (int e = 0; e < 4; ++e) yv = mfma4(sx[e] * d4[e], xb[e], yv);
      }
      float dl[4], dw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ty + 4 * lq + e;
        const bool ok = t < Lc;
        const float xv = sX[t][pcol];
        const float y = yv[e] + Dh * xv;
        float dyv = 0.f;
        if (ok) {
          const float dout = pdo[e].get();
          if (a.z) {
            const float zz = pz[e].get();
            dyv = dout * silu_f32(zz);
            if (a.dz) dzrow[(int64_t)t * (H * BP)] = dout * y * silu_grad_f32(zz);
          } else {
            dyv = dout;
          }
        }
        sDY[t][pcol] = dyv;
        dD_part = fmaf(dyv, xv, dD_part);
        dl[e] = row_sum16(dyv * yo[e]);
        dw[e] = row_sum16(xv * hb[e]);
      }
      if (li == 15) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sDLp[py][16 * ty + 4 * lq + e] = dl[e];
          sDWp[py][16 * ty + 4 * lq + e] = dw[e];
        }
      }
    }
    if (c > 0) fetch_gate(c - 1);
    __syncthreads();  // B3

    // ---- P3: dM, dS, E and their row / column sums (waves 5..7); the first
    //      parts of dC and dB; dx; the update of dH
    if (w >= 5) {
      const int tsel = w - 5;
      const int tt = tsel == 0 ? 0 : 1, ts = tsel == 2 ? 1 : 0;
      f32x4 dm = {};
#pragma unroll
      for (int j = 0; j < BP / 16; ++j) {
        const int k0 = 16 * j + 4 * lq;
        dm = mfma_k16(lds4(&sDY[16 * tt + li][k0]), lds4(&sX[16 * ts + li][k0]), dm);
      }
      const int s = 16 * ts + li;
      const float lam_s = sLam[s], del_s = sDel[s];
      float rowp[4], colp = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * tt + 4 * lq + e;
        const bool ok = s <= t;
        const float ds = dm[e] * __expf(sLam[t] - lam_s) * del_s;
        const float ee = dm[e] * sSX[t][s];  // (0 above the diagonal)
        sDS[t][s] = ok ? ds : 0.f;
        sE[t][s] = ee;
        rowp[e] = row_sum16(ee * del_s);
        colp += ee;
      }
      colp += __shfl_xor(colp, 16, 64);
      colp += __shfl_xor(colp, 32, 64);
      if (li == 15) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sRowP[ts][16 * tt + 4 * lq + e] = rowp[e];
      }
      if (lq == 0) sColP[tt][s] = colp;
    } else if (w == 4) {
      // the [t][s] tile above the diagonal (t < 16 <= s) is zero
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sDS[4 * lq + e][16 + li] = 0.f;
        sE[4 * lq + e][16 + li] = 0.f;
      }
      if (lane < 16) {
        sRowP[1][lane] = 0.f;
        sColP[0][16 + lane] = 0.f;
      }
    }
    f32x4 dc[2] = {}, db[2] = {};
#pragma unroll 2
    for (int j = 0; j < BP / 16; ++j) {
      const int k0 = 16 * j + 4 * lq;
      const f32x4 ay = lds4(&sDY[16 * ty + li][k0]);   // dC += dY H_in
      const f32x4 ax = lds4(&sX[16 * ty + li][k0]);    // dB += X dH_out
      float bh[4][2], bd[4][2];
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          bh[e][k] = sH[k0 + e][16 * (nb + k) + li];
          bd[e][k] = sDH[k0 + e][16 * (nb + k) + li];
        }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          dc[k] = mfma4(ay[e], bh[e][k], dc[k]);
          db[k] = mfma4(ax[e], bd[e][k], db[k]);
        }
    }
    {
      // dx_t = D dy_t + w_t HB_t + sum_u M_ut dy_u, in the [t][p] tile
      f32x4 dx;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ty + 4 * lq + e;
        dx[e] = hb[e] * (__expf(lam_last - sLam[t]) * sDel[t]);
      }
      const int ta = 16 * ty + li;
      const float del_a = sDel[ta];
#pragma unroll
      for (int j = 0; j < BQ / 16; ++j) {
        const int u0 = 16 * j + 4 * lq;
        float am[4], by[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          am[e] = sSX[u0 + e][ta];
          by[e] = sDY[u0 + e][pcol];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) dx = mfma4(am[e] * del_a, by[e], dx);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ty + 4 * lq + e;
        if (t < Lc) a.dpost[(row0 + t) * a.cdim + h * BP + pcol] = dx[e] + Dh * sDY[t][pcol];
      }
    }
    // dH_in = e^lam_last dH_out + sum_t e^lam_t dy_t C_t^T
#pragma unroll
    for (int j = 0; j < 4; ++j) dh[j] *= gam;
#pragma unroll
    for (int jg = 0; jg < BQ / 16; ++jg) {
      const int t0g = 16 * jg + 4 * lq;
      const f32x4 el4 = lds4(&sEl[t0g]);
      float ay[4], bc[4][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ay[e] = sDY[t0g + e][16 * hp + li] * el4[e];
#pragma unroll
        for (int j = 0; j < 4; ++j) bc[e][j] = sC[t0g + e][16 * (hn + j) + li];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j) dh[j] = mfma4(ay[e], bc[e][j], dh[j]);
    }
    __syncthreads();  // B4

    // ---- P4: the second parts of dC and dB, written to HBM; the decays and
    //      delta (wave 0, one lane per token)
    {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ty + 4 * lq + e;
        const float el = sEl[t];
        const float ws = __expf(lam_last - sLam[t]) * sDel[t];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          dc[k][e] *= el;
          db[k][e] *= ws;
        }
      }
#pragma unroll
      for (int j = 0; j < BQ / 16; ++j) {
        const int s0 = 16 * j + 4 * lq;
        const f32x4 as = lds4(&sDS[16 * ty + li][s0]);   // dC_t += dS_ts B_s
        float at[4], bb[4][2], bc[4][2];                 // dB_t += dS_st C_s
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          at[e] = sDS[s0 + e][16 * ty + li];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            bb[e][k] = sB[s0 + e][16 * (nb + k) + li];
            bc[e][k] = sC[s0 + e][16 * (nb + k) + li];
          }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            dc[k] = mfma4(as[e], bb[e][k], dc[k]);
            db[k] = mfma4(at[e], bc[e][k], db[k]);
          }
      }
      float* dcp = a.dCh + (((int64_t)b * L + t0) * H + h) * BN;
      float* dbp = a.dBh + (((int64_t)b * L + t0) * H + h) * BN;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ty + 4 * lq + e;
        if (t < Lc) {
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            dcp[(int64_t)t * H * BN + 16 * (nb + k) + li] = dc[k][e];
            dbp[(int64_t)t * H * BN + 16 * (nb + k) + li] = db[k][e];
          }
        }
      }
    }
    if (w == 0) {
      const int t = lane & 31;
      const bool real = lane < BQ;
      const float del = real ? sDel[t] : 0.f, lam = sLam[t];
      const float wt = __expf(lam_last - lam) * del;
      const float dw = sDWp[0][t] + sDWp[1][t] + sDWp[2][t] + sDWp[3][t];
      const float dlo = sDLp[0][t] + sDLp[1][t] + sDLp[2][t] + sDLp[3][t];
      const float rowg = sRowP[0][t] + sRowP[1][t];
      const float cole = sColP[0][t] + sColP[1][t];
      const float colg = cole * del;
      float dot_hh = 0.f;
#pragma unroll
      for (int i = 0; i < WT / 64; ++i) dot_hh += sRed[i];
      // gradient of the chunk's total log-decay (through w and the carry)
      float dwl = real ? dw * wt : 0.f;
      for (int o = 16; o > 0; o >>= 1) dwl += __shfl_xor(dwl, o, 32);
      const float dlam_last = dwl + gam * dot_hh;
      float dlam = real ? rowg - colg + dlo - dw * wt : 0.f;
      if (real && t == Lc - 1) dlam += dlam_last;
      // suffix sums over the chunk: lam_t = A sum_{r <= t} delta_r
      float suf = dlam;
      for (int o = 1; o < 32; o <<= 1) {
        const float u = __shfl_down(suf, o, 32);
        if (t + o < 32) suf += u;
      }
      const float ddel = cole + (real ? dw * __expf(lam_last - lam) : 0.f) + Ah * suf;
      if (real) {
        dA_part = fmaf(del, suf, dA_part);
        const float sg = a.dt_softplus ? __builtin_amdgcn_rcpf(1.f + __expf(-sV[t])) : 1.f;
        const float dd = ddel * sg;
        if (t < Lc) {
          a.ddt[(row0 + t) * H + h] = dd;
          dbias_part += dd;
        }
      }
    }
    __syncthreads();  // B5
  }

  if (a.dh0) {
    float* dst = a.dh0 + ((int64_t)b * H + h) * BP * BN;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(16 * hp + 4 * lq + e) * BN + 16 * (hn + j) + li] = dh[j][e];
  }
  const float sA = block_sum<WT / 64>(dA_part, sRed);
  const float sD = block_sum<WT / 64>(dD_part, sRed);
  const float sb = block_sum<WT / 64>(dbias_part, sRed);
  if (tid == 0) {
    float* pp = a.part + ((int64_t)b * H + h) * 3;
    pp[0] = sA;
    pp[1] = sD;
    pp[2] = sb;
  }
}

// The B and C gradients of a group: the sum of its heads' shares, in head
// order.  One thread per (b, t, 4 consecutive n of B or C); the shares of a
// token's heads are side by side, so a group's are one contiguous piece.
__global__ void reduce_bc_kernel(const float* __restrict__ dBh, const float* __restrict__ dCh,
                                 float* __restrict__ dpost, int batch, int seqlen, int nheads,
                                 int ngroups, int cdim) {
  const int GN4 = ngroups * BN / 4;
  const int64_t total = (int64_t)batch * seqlen * 2 * GN4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int k = (int)(i % (2 * GN4));
  const int64_t bt = i / (2 * GN4);  // b * seqlen + t
  const bool isC = k >= GN4;
  const int gn = (isC ? k - GN4 : k) * 4;
  const int g = gn / BN, n = gn % BN;
  const int hpg = nheads / ngroups;
  const float* src = isC ? dCh : dBh;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // (unrolled so that the loads of several heads are in flight together;
  // the sum is still taken over j in order)
#pragma unroll 8
  for (int j = 0; j < hpg; ++j) {
    const int h = g * hpg + j;
    const float4 v = *reinterpret_cast<const float4*>(src + (bt * nheads + h) * BN + n);
    acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
  }
  const int HP = nheads * BP;
  *reinterpret_cast<float4*>(dpost + bt * cdim + HP + (isC ? ngroups * BN : 0) + gn) = acc;
}

// ---------------------------------------------------------------- conv

constexpr int CT = 64;   // tokens per conv block

// One thread per (b, channel, block of CT tokens).  The block owns the raw
// positions [t0, t1); they receive w[k] du[t] from the tokens t in
// [t0, t1 + K - 1).  Walking t upwards with the last four raw inputs and the
// four open positions' sums in registers (weights zero-padded to four taps),
// each position is written once all its taps are in.  The first block also
// writes the conv history's gradient; every block writes its sums for the
// conv weights and bias over its own tokens.
template <typename Tx>
__global__ void conv_bwd_kernel(const void* x, int64_t xs, const void* Bm, int64_t bs,
                                const void* Cm, int64_t cs, const float* __restrict__ w,
                                const float* __restrict__ bias, const void* hist,
                                const float* __restrict__ dpost, float* __restrict__ dxbc,
                                float* __restrict__ dhist, float* __restrict__ wpart,
                                int batch, int seqlen, int cdim, int HP, int GN, int K) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const int blk = blockIdx.y, b = blockIdx.z;
  if (c >= cdim) return;
  const Tx* src;
  int64_t st;
  int cc;
  if (c < HP) { src = static_cast<const Tx*>(x); st = xs; cc = c; }
  else if (c < HP + GN) { src = static_cast<const Tx*>(Bm); st = bs; cc = c - HP; }
  else { src = static_cast<const Tx*>(Cm); st = cs; cc = c - HP - GN; }
  const Tx* hs = static_cast<const Tx*>(hist);
  auto raw = [&](int tau) -> float {  // raw input at position tau (history below 0)
    if (tau >= 0) return to_f32(src[((int64_t)b * seqlen + tau) * st + cc]);
    if (hs == nullptr || tau < -(K - 1)) return 0.f;
    return to_f32(hs[((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + c]);
  };
  // taps right-aligned in four slots: slot j meets raw position t - 3 + j
  float wp[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) wp[j] = j >= 4 - K ? w[c * K + (j - (4 - K))] : 0.f;
  const float bc = bias ? bias[c] : 0.f;
  const int t0 = blk * CT, t1 = min(seqlen, t0 + CT);
  const int tend = min(seqlen, t1 + K - 1);
  float win[4];   // raw inputs at t - 3 .. t (after the shift at the top of step t)
  float acc[4];   // open sums of raw positions t - 3 .. t
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    win[j] = j > 0 ? raw(t0 - 4 + j) : 0.f;
    acc[j] = 0.f;
  }
  float gw[4] = {0.f, 0.f, 0.f, 0.f}, gb = 0.f;
  auto emit = [&](int pos, float v) {
    if (pos >= t0 && pos < t1) dxbc[((int64_t)b * seqlen + pos) * cdim + c] = v;
    else if (pos < 0 && blk == 0 && dhist != nullptr && pos >= -(K - 1))
      dhist[((int64_t)b * (K - 1) + (K - 1) + pos) * cdim + c] = v;
  };
  // UNR tokens per step: their raw inputs and output gradients are loaded
  // together (positions past tend re-read the last one and are not used),
  // so that each thread keeps 2 UNR loads in flight; t >= t0 >= 0 here
  constexpr int UNR = 4;
  for (int tb = t0; tb < tend; tb += UNR) {
    float rv[UNR], dv[UNR];
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int t = min(tb + r, tend - 1);
      rv[r] = to_f32(src[((int64_t)b * seqlen + t) * st + cc]);
      dv[r] = dpost[((int64_t)b * seqlen + t) * cdim + c];
    }
#pragma unroll
    for (int r = 0; r < UNR; ++r) {
      const int t = tb + r;
      if (t >= tend) break;
      win[0] = win[1]; win[1] = win[2]; win[2] = win[3];
      win[3] = rv[r];
      float u = bc;
#pragma unroll
      for (int j = 0; j < 4; ++j) u = fmaf(wp[j], win[j], u);
      const float d = dv[r] * silu_grad_f32(u);
      if (t < t1) {
        gb += d;
#pragma unroll
        for (int j = 0; j < 4; ++j) gw[j] = fmaf(d, win[j], gw[j]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(wp[j], d, acc[j]);
      emit(t - 3, acc[0]);  // position t - 3 has all its taps
      acc[0] = acc[1]; acc[1] = acc[2]; acc[2] = acc[3]; acc[3] = 0.f;
    }
  }
  // the positions still open (their later taps lie past the sequence)
  emit(tend - 3, acc[0]);
  emit(tend - 2, acc[1]);
  emit(tend - 1, acc[2]);
  const int nblk = gridDim.y;
  float* wq = wpart + (((int64_t)b * nblk + blk) * cdim + c) * 5;
#pragma unroll
  for (int k = 0; k < 4; ++k) wq[k] = k < K ? gw[k + (4 - K)] : 0.f;
  wq[4] = gb;
}

// Fixed-order sums: dA, dD, dt_bias over the batch; the conv weights and bias
// over (b, block).
constexpr int RP_CH = 32;      // conv channels per workgroup
constexpr int RP_GROUPS = 8;   // partial-sum groups per channel
constexpr int RP_THREADS = RP_CH * RP_GROUPS;
__global__ __launch_bounds__(RP_THREADS) void reduce_params_kernel(
    const float* __restrict__ part, int batch, int nheads, float* dA, float* dD, float* dbias,
    const float* __restrict__ wpart, int nparts, int cdim, int K, float* dw, float* db) {
  __shared__ float sred[RP_GROUPS][RP_CH][5];
  const int tid = threadIdx.x;
  const int i = blockIdx.x * RP_THREADS + tid;
  if (i < nheads) {
    float sa = 0.f, sd = 0.f, sb = 0.f;
    for (int b = 0; b < batch; ++b) {
      const float* p = part + ((int64_t)b * nheads + i) * 3;
      sa += p[0]; sd += p[1]; sb += p[2];
    }
    dA[i] = sa;
    if (dD) dD[i] = sd;
    if (dbias) dbias[i] = sb;
  }
  if (wpart != nullptr) {  // (uniform)
    // channel c of this workgroup's RP_CH: group grp sums parts grp,
    // grp + RP_GROUPS, ... in order, then the groups are added in order
    const int cl = tid % RP_CH, grp = tid / RP_CH;
    const int c = blockIdx.x * RP_CH + cl;
    float s[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
    if (c < cdim)
      for (int j = grp; j < nparts; j += RP_GROUPS)
#pragma unroll
        for (int k = 0; k < 5; ++k) s[k] += wpart[((int64_t)j * cdim + c) * 5 + k];
#pragma unroll
    for (int k = 0; k < 5; ++k) sred[grp][cl][k] = s[k];
    __syncthreads();
    if (grp == 0 && c < cdim) {
      float t[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
      for (int gg = 0; gg < RP_GROUPS; ++gg)
#pragma unroll
        for (int k = 0; k < 5; ++k) t[k] += sred[gg][cl][k];
      if (dw)
        for (int k = 0; k < K; ++k) dw[c * K + k] = t[k];
      if (db) db[c] = t[4];
    }
  }
}

// x|B|C (post-conv inputs) to fp32 [B, L, Cdim]
template <typename Tx>
__global__ void gather_post_kernel(const void* x, int64_t xs, const void* Bm, int64_t bs,
                                   const void* Cm, int64_t cs, float* __restrict__ post,
                                   int64_t rows, int cdim, int HP, int GN) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * cdim) return;
  const int64_t r = i / cdim;
  const int c = (int)(i % cdim);
  float v;
  if (c < HP) v = to_f32(static_cast<const Tx*>(x)[r * xs + c]);
  else if (c < HP + GN) v = to_f32(static_cast<const Tx*>(Bm)[r * bs + c - HP]);
  else v = to_f32(static_cast<const Tx*>(Cm)[r * cs + c - HP - GN]);
  post[i] = v;
}

}  // namespace

size_t scan_bwd_workspace_layout(int batch, int seqlen, int nheads, int ngroups, int conv_width,
                                 size_t* off_post, size_t* off_states, size_t* off_dbh,
                                 size_t* off_dch, size_t* off_dpost, size_t* off_part,
                                 size_t* off_wpart) {
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  const size_t T = (size_t)batch * seqlen;
  const size_t cdim = (size_t)nheads * BP + 2 * (size_t)ngroups * BN;
  const size_t nc = (size_t)(seqlen + BQ - 1) / BQ;
  const size_t nblk = (size_t)(seqlen + CT - 1) / CT;
  size_t o = 0;
  *off_post = o; o += up(T * cdim * 4);
  *off_states = o; o += up((size_t)batch * nheads * nc * BP * BN * 4);
  *off_dbh = o; o += up((size_t)batch * nheads * seqlen * BN * 4);
  *off_dch = o; o += up((size_t)batch * nheads * seqlen * BN * 4);
  *off_dpost = o; o += up(conv_width > 0 ? T * cdim * 4 : 0);
  *off_part = o; o += up((size_t)batch * nheads * 3 * 4);
  *off_wpart = o; o += up(conv_width > 0 ? (size_t)batch * nblk * cdim * 5 * 4 : 0);
  return o;
}

hipError_t launch_scan_bwd(const ScanBwdLaunch& l, hipStream_t stream) {
  const int B = l.batch, L = l.seqlen, H = l.nheads, G = l.ngroups;
  const int HP = H * BP, GN = G * BN, cdim = HP + 2 * GN;
  const int64_t T = (int64_t)B * L;
  size_t o_post, o_st, o_db, o_dc, o_dp, o_part, o_wp;
  scan_bwd_workspace_layout(B, L, H, G, l.conv_w ? l.conv_k : 0, &o_post, &o_st, &o_db, &o_dc,
                            &o_dp, &o_part, &o_wp);
  char* ws = static_cast<char*>(l.workspace);
  float* post = reinterpret_cast<float*>(ws + o_post);
  const bool bf = l.xbc_dtype == SSD_BF16;
  hipError_t e;
  // 1. post-conv x|B|C in fp32
  if (l.conv_w) {
    // x, B and C are separate tensors: the conv runs on each channel range
    const void* srcs[3] = {l.x, l.Bm, l.Cm};
    const int64_t strides[3] = {l.x_stride, l.b_stride, l.c_stride};
    const int widths[3] = {HP, GN, GN};
    int c0 = 0;
    for (int k = 0; k < 3; ++k) {
      const size_t es = bf ? 2 : 4;
      const void* hist = l.conv_state_in
                             ? static_cast<const char*>(l.conv_state_in) + (size_t)c0 * es
                             : nullptr;
      e = launch_causal_conv1d(srcs[k], strides[k], l.xbc_dtype, l.conv_w + (size_t)c0 * l.conv_k,
                               l.conv_b ? l.conv_b + c0 : nullptr, hist, nullptr, cdim, post + c0,
                               cdim, SSD_F32, B, L, widths[k], l.conv_k, 1, stream);
      if (e != hipSuccess) return e;
      c0 += widths[k];
    }
  } else {
    const int64_t n = T * cdim;
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (bf)
      gather_post_kernel<bf16><<<grid, 256, 0, stream>>>(l.x, l.x_stride, l.Bm, l.b_stride, l.Cm,
                                                          l.c_stride, post, T, cdim, HP, GN);
    else
      gather_post_kernel<float><<<grid, 256, 0, stream>>>(l.x, l.x_stride, l.Bm, l.b_stride, l.Cm,
                                                           l.c_stride, post, T, cdim, HP, GN);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  BwdArgs a{};
  a.post = post;
  a.dt = l.dt; a.dt_stride = l.dt_stride;
  a.z = l.z; a.z_stride = l.z_stride;
  a.dout = l.dout; a.dout_stride = l.dout_stride;
  a.A = l.A; a.D = l.D; a.dt_bias = l.dt_bias; a.dt_softplus = l.dt_softplus;
  a.h0 = l.h0; a.dhT = l.dhT;
  a.states = reinterpret_cast<float*>(ws + o_st);
  // without a conv the post-conv gradient is the answer
  a.dpost = l.conv_w ? reinterpret_cast<float*>(ws + o_dp) : l.dxbc;
  a.dBh = reinterpret_cast<float*>(ws + o_db);
  a.dCh = reinterpret_cast<float*>(ws + o_dc);
  a.ddt = l.ddt; a.dz = l.dz; a.dh0 = l.dh0;
  a.part = reinterpret_cast<float*>(ws + o_part);
  a.batch = B; a.seqlen = L; a.nheads = H; a.ngroups = G; a.nc = (L + BQ - 1) / BQ;
  a.cdim = cdim;
  const dim3 grid_bh((unsigned)(B * H));
  const bool abf = l.act_dtype == SSD_BF16, dbf = l.dout_dtype == SSD_BF16;
  // 2. the state entering each chunk
  if (abf) fwd_states_kernel<bf16><<<grid_bh, BT, 0, stream>>>(a);
  else fwd_states_kernel<float><<<grid_bh, BT, 0, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 3. the chunks in reverse
  if (abf && dbf) bwd_chunk_kernel<bf16, bf16><<<grid_bh, WT, 0, stream>>>(a);
  else if (abf) bwd_chunk_kernel<bf16, float><<<grid_bh, WT, 0, stream>>>(a);
  else if (dbf) bwd_chunk_kernel<float, bf16><<<grid_bh, WT, 0, stream>>>(a);
  else bwd_chunk_kernel<float, float><<<grid_bh, WT, 0, stream>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // 4. B and C of each group
  {
    const int64_t n = T * 2 * (GN / 4);
    reduce_bc_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a.dBh, a.dCh, a.dpost, B, L,
                                                                      H, G, cdim);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 5. the conv
  const int nblk = (L + CT - 1) / CT;
  float* wpart = reinterpret_cast<float*>(ws + o_wp);
  if (l.conv_w) {
    const dim3 grid((unsigned)((cdim + 255) / 256), (unsigned)nblk, (unsigned)B);
    if (bf)
      conv_bwd_kernel<bf16><<<grid, 256, 0, stream>>>(
          l.x, l.x_stride, l.Bm, l.b_stride, l.Cm, l.c_stride, l.conv_w, l.conv_b,
          l.conv_state_in, a.dpost, l.dxbc, l.dconv_state_in, wpart, B, L, cdim, HP, GN, l.conv_k);
    else
      conv_bwd_kernel<float><<<grid, 256, 0, stream>>>(
          l.x, l.x_stride, l.Bm, l.b_stride, l.Cm, l.c_stride, l.conv_w, l.conv_b,
          l.conv_state_in, a.dpost, l.dxbc, l.dconv_state_in, wpart, B, L, cdim, HP, GN, l.conv_k);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 6. parameter sums
  {
    const int gh = (H + RP_THREADS - 1) / RP_THREADS;
    const int gc = l.conv_w ? (cdim + RP_CH - 1) / RP_CH : 0;
    reduce_params_kernel<<<(unsigned)(gh > gc ? gh : gc), RP_THREADS, 0, stream>>>(
        a.part, B, H, l.dA, l.dD, l.ddt_bias, l.conv_w ? wpart : nullptr, B * nblk, cdim,
        l.conv_k, l.dconv_w, l.dconv_b);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ssd
