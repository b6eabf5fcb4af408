// Chunked selective scan, every product in fp32 on the vector ALU.
//
// This is the fp32 path (SSD_MATH_F32).  It computes the same chunked form as
// the matrix-core kernel -- within a chunk the outputs are the lower-
// triangular (C B^T o decay) matrix applied to x plus the carried state read
// out through C; between chunks the state is decayed and the chunk's
// contribution added -- which is an exact re-association of the recurrence
// h_t = exp(delta_t A) h_{t-1} + delta_t x_t B_t^T, y_t = C_t h_t + D x_t
// ("Hybrid Architectures for Language Models" summary, section 2 Background:
// SSD recasts the state-space computation as matrix multiplies).
//
// One workgroup walks one (sequence, head) chunk by chunk with the fp32 state
// [64 x 128] in LDS; within a chunk it works on 32-token tiles.
#include "ssd_common.h"

namespace ssd {
namespace {

constexpr int P = 64;
constexpr int N = 128;
// Threads per walker: 512 (8 waves) when the walkers do not fill the chip,
// each alone on its CU; 256 otherwise, so that two share a CU (LDS allows two
// and 256 threads fit their registers).
constexpr int NUM_CUS = 256;
constexpr int TT = 32;  // token tile
// Row pitches of the LDS tiles: multiples of 4 floats, so that the inner
// loops read 4 consecutive k as one 16-byte read (sums still taken one k
// at a time, in order); 132 = 4 mod 32, so that 8 lanes reading 8 rows at
// one column (one 16-byte read each) fall on distinct banks.  The x tile is
// read one value per lane (consecutive p in consecutive lanes) and keeps an
// odd pitch.  At chunk 128 the walker takes under 80 KiB of LDS: two
// workgroups share a CU.
constexpr int LDN = N + 4;
// the C tile is only read a row per wave (or two) at a time: no padding
constexpr int LDC = N;
constexpr int LDP = P + 1;
constexpr int LDT = TT;

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
// s + a . b over 4 consecutive k, added one k at a time in order
__device__ __forceinline__ float dot4(float s, float4 a, float4 b) {
  s += a.x * b.x;
  s += a.y * b.y;
  s += a.z * b.z;
  s += a.w * b.w;
  return s;
}

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
  return to_f32(static_cast<const T*>(p)[i]);
}

// Raw conv input at tau (possibly negative) for the hand-over of the history.
template <typename Tx>
__device__ __forceinline__ float load_raw(const ScanArgs& a, const void* base, int64_t stride,
                                          int b, int tau, int j, int c, int cdim) {
  const int K = a.conv_k;
  if (tau >= 0) return ldf<Tx>(base, ((int64_t)b * a.seqlen + tau) * stride + j);
  if (a.conv_state_in != nullptr && tau >= -(K - 1))
    return ldf<Tx>(a.conv_state_in, ((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + c);
  return 0.f;
}

// A [TT][NC] tile of post-conv values into LDS (row r at dst + r * ld): the
// rows are tokens tok0 .. tok0 + TT - 1 of sequence b, the columns elements
// j0 .. j0 + NC - 1 of the tensor's row (conv channels c0 .. c0 + NC - 1).
// Rows from nvalid on are zero.  Thread t owns column t % NC and a run of
// TT / (NT / NC) consecutive rows: it issues every raw load of the run
// (with the conv, the run and its 3-token halo) before any arithmetic, and
// slides the conv window along the run.  Conv: u = bias + the taps' products
// added oldest input first (the first tap meets the token K - 1 before the
// output), then SiLU; before the first token the inputs come from the conv
// state (oldest row first) or are zero.
template <typename Tx, bool CONV, int NC, int NT>
__device__ __forceinline__ void fill_tile(const ScanArgs& a, const void* base, int64_t stride,
                                          int b, int tok0, int nvalid, int j0, int c0, int cdim,
                                          float* dst, int ld) {
  constexpr int RPT = TT / (NT / NC);
  const int col = threadIdx.x % NC, r0 = (threadIdx.x / NC) * RPT;
  const int L = a.seqlen, j = j0 + col, c = c0 + col;
  constexpr int HALO = CONV ? 3 : 0;
  float raw[RPT + HALO];
#pragma unroll
  for (int i = 0; i < RPT + HALO; ++i) {
    // (rows past the sequence re-read its last token; their results are zeroed)
    const int tau = min(max(tok0 + r0 - HALO + i, 0), L - 1);
    raw[i] = ldf<Tx>(base, ((int64_t)b * L + tau) * stride + j);
  }
  if (CONV && tok0 + r0 - HALO < 0) {  // the history before the first token
    const int K = a.conv_k;
#pragma unroll
    for (int i = 0; i < HALO; ++i) {
      const int tau = tok0 + r0 - HALO + i;
      if (tau < 0)
        raw[i] = a.conv_state_in != nullptr && tau >= -(K - 1)
                     ? ldf<Tx>(a.conv_state_in, ((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + c)
                     : 0.f;
    }
  }
  float out[RPT];
  if constexpr (CONV) {
    // taps right-aligned: tap k of 4 meets the token 3 - k before the output
    const int K = a.conv_k;
    float w4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w4[k] = k >= 4 - K ? a.conv_w[(int64_t)c * K + k - (4 - K)] : 0.f;
    const float bias = a.conv_b ? a.conv_b[c] : 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      float u = bias;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (k >= 4 - K) u += w4[k] * raw[r + k];
      out[r] = silu_f32(u);
    }
  } else {
#pragma unroll
    for (int r = 0; r < RPT; ++r) out[r] = raw[r];
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) dst[(r0 + r) * ld + col] = r0 + r < nvalid ? out[r] : 0.f;
}

// In-place inclusive prefix sum of s[0..n), n <= the block size; fixed order.
__device__ void block_inclusive_scan(float* s, int n, float* red) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float v = tid < n ? s[tid] : 0.f;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) red[w] = v;
  __syncthreads();
  float add = 0.f;
  for (int i = 0; i < w; ++i) add += red[i];
  if (tid < n) s[tid] = v + add;
  __syncthreads();
}

template <typename Tx, typename Ta, typename Ty, bool CONV, int NT>
__global__ __launch_bounds__(NT) void scan_f32_kernel(ScanArgs a) {
  constexpr int THREADS = NT;
  constexpr int RG = NT / 64;  // output rows: a wave per row group, RPW rows per thread
  constexpr int SC = NT / 64;  // state update: SC threads per state row p
  extern __shared__ float smem[];
  const int Q = a.chunk;
  float* sH = smem;                 // [P][LDN]  state
  float* sLam = sH + P * LDN;       // [Q]       cumulative log decay in the chunk
  float* sDel = sLam + Q;           // [Q]       delta; then exp(Lam_last - Lam_s) delta_s
  float* sCt = sDel + Q;            // [TT][LDC] C tile (output rows)
  float* sBt = sCt + TT * LDC;      // [TT][LDN] B tile (source rows)
  float* sX = sBt + TT * LDN;       // [TT][LDP] x tile (source rows)
  float* sM = sX + TT * LDP;        // [TT][LDT] masked, decayed C B^T tile
  float* sRed = sM + TT * LDT;      // [NT / 64]

  const int H = a.nheads, G = a.ngroups, L = a.seqlen;
  const int b = blockIdx.x / H, h = blockIdx.x % H;
  const int hpg = H / G, g = h / hpg;
  const int HP = H * P, GN = G * N, cdim = HP + 2 * GN;
  const int tid = threadIdx.x;
  const float Ah = a.A[h], Dh = a.D ? a.D[h] : 0.f;

  for (int i = tid; i < P * N; i += THREADS) {
    const int p = i / N, n = i % N;
    sH[p * LDN + n] =
        a.initial_state ? a.initial_state[((int64_t)b * H + h) * P * N + i] : 0.f;
  }

  // output-tile mapping: column p, rows tr + RG i
  constexpr int RPW = TT / RG;
  const int yp = tid & 63, tr = tid >> 6;
  // state-update mapping: row sp, columns sn0 .. sn0 + SW - 1
  constexpr int SW = N / SC;
  const int sp = tid / SC, sn0 = (tid % SC) * SW;

  for (int c0 = 0; c0 < L; c0 += Q) {
    const int Lc = min(Q, L - c0);
    __syncthreads();
    for (int t = tid; t < Q; t += THREADS) {
      const float d =
          t < Lc ? make_delta(ldf<Ta>(a.dt, ((int64_t)b * L + c0 + t) * a.dt_stride + h),
                              a.dt_bias, h, a.dt_softplus)
                 : 0.f;
      sDel[t] = d;
      sLam[t] = d * Ah;
    }
    __syncthreads();
    block_inclusive_scan(sLam, Q, sRed);
    // the decay to the chunk's last token: slot Lc - 1, not Q - 1 -- past the
    // end the increments are 0, but the scan adds them in another order, so
    // the two slots can differ by an ulp, which is large when |Lam| is
    const float lam_last = sLam[Lc - 1];

    for (int tt0 = 0; tt0 < Lc; tt0 += TT) {
      fill_tile<Tx, CONV, N, NT>(a, a.Cm, a.c_stride, b, c0 + tt0, Lc - tt0, g * N, HP + GN + g * N,
                             cdim, sCt, LDC);
      __syncthreads();
      // the read-out of the thread's RPW rows: each 4 n of the state row
      // read once for all of them (every row's sum still runs over n in order)
      float yacc[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) yacc[i] = 0.f;
#pragma unroll 2
      for (int n = 0; n < N; n += 4) {
        const float4 h4 = ld4(&sH[yp * LDN + n]);
#pragma unroll
        for (int i = 0; i < RPW; ++i) yacc[i] = dot4(yacc[i], ld4(&sCt[(tr + RG * i) * LDC + n]), h4);
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) yacc[i] *= expf(sLam[tt0 + tr + RG * i]);
      for (int st0 = 0; st0 <= tt0; st0 += TT) {
        __syncthreads();
        fill_tile<Tx, CONV, N, NT>(a, a.Bm, a.b_stride, b, c0 + st0, Lc - st0, g * N, HP + g * N, cdim,
                               sBt, LDN);
        fill_tile<Tx, CONV, P, NT>(a, a.x, a.x_stride, b, c0 + st0, Lc - st0, h * P, h * P, cdim, sX,
                               LDP);
        __syncthreads();
        {
          // the thread's TT * TT / THREADS elements share their column q: each
          // 4 n of row q of B read once for all of them
          constexpr int NE = TT * TT / THREADS;
          const int q = tid % TT, r0 = tid / TT, s = st0 + q;
          float dot[NE];
#pragma unroll
          for (int k = 0; k < NE; ++k) dot[k] = 0.f;
#pragma unroll 2
          for (int n = 0; n < N; n += 4) {
            const float4 b4 = ld4(&sBt[q * LDN + n]);
#pragma unroll
            for (int k = 0; k < NE; ++k)
              dot[k] = dot4(dot[k], ld4(&sCt[(r0 + k * (THREADS / TT)) * LDC + n]), b4);
          }
#pragma unroll
          for (int k = 0; k < NE; ++k) {
            const int r = r0 + k * (THREADS / TT), t = tt0 + r;
            sM[r * LDT + q] = s <= t ? dot[k] * expf(sLam[t] - sLam[s]) * sDel[s] : 0.f;
          }
        }
        __syncthreads();
        // each x value read once for the thread's RPW rows; every row's
        // sum still runs over q in order
        float sacc[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) sacc[i] = 0.f;
#pragma unroll 2
        for (int q = 0; q < TT; q += 4) {
          const float4 x4 = make_float4(sX[q * LDP + yp], sX[(q + 1) * LDP + yp],
                                        sX[(q + 2) * LDP + yp], sX[(q + 3) * LDP + yp]);
#pragma unroll
          for (int i = 0; i < RPW; ++i)
            sacc[i] = dot4(sacc[i], ld4(&sM[(tr + RG * i) * LDT + q]), x4);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) yacc[i] += sacc[i];
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int t = tt0 + tr + RG * i;
        if (t < Lc) {
          // sX holds the diagonal source tile, i.e. this output tile's x
          const float xv = sX[(tr + RG * i) * LDP + yp];
          float yv = yacc[i] + Dh * xv;
          if (a.z != nullptr)
            yv *= silu_f32(ldf<Ta>(a.z, ((int64_t)b * L + c0 + t) * a.z_stride + h * P + yp));
          static_cast<Ty*>(a.y)[((int64_t)b * L + c0 + t) * a.y_stride + h * P + yp] =
              from_f32<Ty>(yv);
        }
      }
      __syncthreads();
    }

    // state: H <- exp(lam_last) H + sum_s exp(lam_last - lam_s) delta_s x_s B_s^T.
    // Each token's weight exp(lam_last - lam_s) delta_s once per chunk, in
    // place of its delta (the output tiles are done with it; read past the
    // barrier at the top of the tile loop below)
    for (int t = tid; t < Q; t += THREADS) sDel[t] = expf(lam_last - sLam[t]) * sDel[t];
    float hacc[SW];
    const float gamma = expf(lam_last);
#pragma unroll
    for (int k = 0; k < SW; k += 4) {
      const float4 h4 = ld4(&sH[sp * LDN + sn0 + k]);
      hacc[k] = gamma * h4.x;
      hacc[k + 1] = gamma * h4.y;
      hacc[k + 2] = gamma * h4.z;
      hacc[k + 3] = gamma * h4.w;
    }
    for (int st0 = 0; st0 < Lc; st0 += TT) {
      __syncthreads();
      fill_tile<Tx, CONV, N, NT>(a, a.Bm, a.b_stride, b, c0 + st0, Lc - st0, g * N, HP + g * N, cdim,
                             sBt, LDN);
      fill_tile<Tx, CONV, P, NT>(a, a.x, a.x_stride, b, c0 + st0, Lc - st0, h * P, h * P, cdim, sX,
                             LDP);
      __syncthreads();
      for (int q = 0; q < TT && st0 + q < Lc; ++q) {
        const int s = st0 + q;
        const float ws = sDel[s] * sX[q * LDP + sp];
#pragma unroll
        for (int k = 0; k < SW; k += 4) {
          const float4 b4 = ld4(&sBt[q * LDN + sn0 + k]);
          hacc[k] += ws * b4.x;
          hacc[k + 1] += ws * b4.y;
          hacc[k + 2] += ws * b4.z;
          hacc[k + 3] += ws * b4.w;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SW; k += 4)
      *reinterpret_cast<float4*>(&sH[sp * LDN + sn0 + k]) =
          make_float4(hacc[k], hacc[k + 1], hacc[k + 2], hacc[k + 3]);
  }
  __syncthreads();

  if (a.final_state != nullptr)
    for (int i = tid; i < P * N; i += THREADS)
      a.final_state[((int64_t)b * H + h) * P * N + i] = sH[(i / N) * LDN + i % N];

  if (CONV && a.conv_state_out != nullptr) {
    const int K = a.conv_k;
    Tx* out = static_cast<Tx*>(a.conv_state_out);
    for (int i = tid; i < (K - 1) * P; i += THREADS) {
      const int j = i / P, p = i % P, c = h * P + p;
      out[((int64_t)b * (K - 1) + j) * cdim + c] =
          from_f32<Tx>(load_raw<Tx>(a, a.x, a.x_stride, b, L - (K - 1) + j, c, c, cdim));
    }
    if (h % hpg == 0)
      for (int i = tid; i < (K - 1) * 2 * N; i += THREADS) {
        const int j = i / (2 * N), e = i % (2 * N);
        const bool isB = e < N;
        const int n = isB ? e : e - N;
        const int c = (isB ? HP : HP + GN) + g * N + n;
        const float v = isB ? load_raw<Tx>(a, a.Bm, a.b_stride, b, L - (K - 1) + j, g * N + n, c, cdim)
                            : load_raw<Tx>(a, a.Cm, a.c_stride, b, L - (K - 1) + j, g * N + n, c, cdim);
        out[((int64_t)b * (K - 1) + j) * cdim + c] = from_f32<Tx>(v);
      }
  }
}

template <typename Tx, typename Ta, typename Ty, int NT>
hipError_t launch_nt(const ScanArgs& a, hipStream_t stream) {
  const size_t lds = sizeof(float) * ((size_t)P * LDN + 2 * a.chunk + TT * LDC + TT * LDN +
                                      TT * LDP + TT * LDT + NT / 64);
  const dim3 grid(a.batch * a.nheads);
  if (a.conv_w != nullptr) {
    auto k = scan_f32_kernel<Tx, Ta, Ty, true, NT>;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k, grid, dim3(NT), lds, stream, a);
  } else {
    auto k = scan_f32_kernel<Tx, Ta, Ty, false, NT>;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k, grid, dim3(NT), lds, stream, a);
  }
  return hipGetLastError();
}

template <typename Tx, typename Ta, typename Ty>
hipError_t launch_typed(const ScanArgs& a, hipStream_t stream) {
  return (int64_t)a.batch * a.nheads <= NUM_CUS ? launch_nt<Tx, Ta, Ty, 512>(a, stream)
                                                : launch_nt<Tx, Ta, Ty, 256>(a, stream);
}

template <typename Tx, typename Ta>
hipError_t pick_y(const ScanArgs& a, ssd_dtype_t yd, hipStream_t s) {
  return yd == SSD_F32 ? launch_typed<Tx, Ta, float>(a, s) : launch_typed<Tx, Ta, bf16>(a, s);
}

}  // namespace

hipError_t launch_scan_f32(const ScanArgs& a, ssd_dtype_t xd, ssd_dtype_t ad, ssd_dtype_t yd,
                           hipStream_t s) {
  if (xd == SSD_F32 && ad == SSD_F32) return pick_y<float, float>(a, yd, s);
  if (xd == SSD_F32) return pick_y<float, bf16>(a, yd, s);
  if (ad == SSD_F32) return pick_y<bf16, float>(a, yd, s);
  return pick_y<bf16, bf16>(a, yd, s);
}

}  // namespace ssd
