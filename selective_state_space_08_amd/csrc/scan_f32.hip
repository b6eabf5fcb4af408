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
constexpr int THREADS = 256;
constexpr int TT = 32;  // token tile
constexpr int LDN = N + 1;
constexpr int LDP = P + 1;
constexpr int LDT = TT + 1;

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
  return to_f32(static_cast<const T*>(p)[i]);
}

// Post-conv value of element j (index within its own tensor's row) of token t
// of sequence b; c is the element's conv channel (row of conv_w).
template <typename Tx, bool CONV>
__device__ __forceinline__ float load_post(const ScanArgs& a, const void* base, int64_t stride,
                                           int b, int t, int j, int c, int cdim) {
  if (!CONV) return ldf<Tx>(base, ((int64_t)b * a.seqlen + t) * stride + j);
  const int K = a.conv_k;
  float u = a.conv_b ? a.conv_b[c] : 0.f;
  for (int k = 0; k < K; ++k) {
    const int tau = t - (K - 1) + k;
    float v = 0.f;
    if (tau >= 0)
      v = ldf<Tx>(base, ((int64_t)b * a.seqlen + tau) * stride + j);
    else if (a.conv_state_in != nullptr)
      v = ldf<Tx>(a.conv_state_in, ((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + c);
    u += a.conv_w[(int64_t)c * K + k] * v;
  }
  return silu_f32(u);
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

// In-place inclusive prefix sum of s[0..n), n <= THREADS; fixed order.
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

template <typename Tx, typename Ta, typename Ty, bool CONV>
__global__ __launch_bounds__(THREADS) void scan_f32_kernel(ScanArgs a) {
  extern __shared__ float smem[];
  const int Q = a.chunk;
  float* sH = smem;                 // [P][LDN]  state
  float* sLam = sH + P * LDN;       // [Q]       cumulative log decay in the chunk
  float* sDel = sLam + Q;           // [Q]       delta
  float* sCt = sDel + Q;            // [TT][LDN] C tile (output rows)
  float* sBt = sCt + TT * LDN;      // [TT][LDN] B tile (source rows)
  float* sX = sBt + TT * LDN;       // [TT][LDP] x tile (source rows)
  float* sM = sX + TT * LDP;        // [TT][LDT] masked, decayed C B^T tile
  float* sRed = sM + TT * LDT;      // [4]

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

  // output-tile mapping: column p, rows tr + 4 i
  const int yp = tid & 63, tr = tid >> 6;
  // state-update mapping: row sp, columns sn0 .. sn0 + 31
  const int sp = tid >> 2, sn0 = (tid & 3) * 32;

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
      for (int i = tid; i < TT * N; i += THREADS) {
        const int r = i / N, n = i % N, t = tt0 + r;
        sCt[r * LDN + n] = t < Lc ? load_post<Tx, CONV>(a, a.Cm, a.c_stride, b, c0 + t, g * N + n,
                                                        HP + GN + g * N + n, cdim)
                                  : 0.f;
      }
      __syncthreads();
      float yacc[TT / 4];
#pragma unroll
      for (int i = 0; i < TT / 4; ++i) {
        const int r = tr + 4 * i;
        float s = 0.f;
        for (int n = 0; n < N; ++n) s += sCt[r * LDN + n] * sH[yp * LDN + n];
        yacc[i] = expf(sLam[tt0 + r]) * s;
      }
      for (int st0 = 0; st0 <= tt0; st0 += TT) {
        __syncthreads();
        for (int i = tid; i < TT * N; i += THREADS) {
          const int r = i / N, n = i % N, s = st0 + r;
          sBt[r * LDN + n] = s < Lc ? load_post<Tx, CONV>(a, a.Bm, a.b_stride, b, c0 + s, g * N + n,
                                                          HP + g * N + n, cdim)
                                    : 0.f;
        }
        for (int i = tid; i < TT * P; i += THREADS) {
          const int r = i / P, p = i % P, s = st0 + r;
          sX[r * LDP + p] = s < Lc ? load_post<Tx, CONV>(a, a.x, a.x_stride, b, c0 + s, h * P + p,
                                                         h * P + p, cdim)
                                   : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < TT * TT; e += THREADS) {
          const int r = e / TT, q = e % TT, t = tt0 + r, s = st0 + q;
          float v = 0.f;
          if (s <= t) {
            float dot = 0.f;
            for (int n = 0; n < N; ++n) dot += sCt[r * LDN + n] * sBt[q * LDN + n];
            v = dot * expf(sLam[t] - sLam[s]) * sDel[s];
          }
          sM[r * LDT + q] = v;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < TT / 4; ++i) {
          const int r = tr + 4 * i;
          float s = 0.f;
          for (int q = 0; q < TT; ++q) s += sM[r * LDT + q] * sX[q * LDP + yp];
          yacc[i] += s;
        }
      }
#pragma unroll
      for (int i = 0; i < TT / 4; ++i) {
        const int t = tt0 + tr + 4 * i;
        if (t < Lc) {
          const float xv =
              load_post<Tx, CONV>(a, a.x, a.x_stride, b, c0 + t, h * P + yp, h * P + yp, cdim);
          float yv = yacc[i] + Dh * xv;
          if (a.z != nullptr)
            yv *= silu_f32(ldf<Ta>(a.z, ((int64_t)b * L + c0 + t) * a.z_stride + h * P + yp));
          static_cast<Ty*>(a.y)[((int64_t)b * L + c0 + t) * a.y_stride + h * P + yp] =
              from_f32<Ty>(yv);
        }
      }
      __syncthreads();
    }

    // state: H <- exp(lam_last) H + sum_s exp(lam_last - lam_s) delta_s x_s B_s^T
    float hacc[32];
    const float gamma = expf(lam_last);
#pragma unroll
    for (int k = 0; k < 32; ++k) hacc[k] = gamma * sH[sp * LDN + sn0 + k];
    for (int st0 = 0; st0 < Lc; st0 += TT) {
      __syncthreads();
      for (int i = tid; i < TT * N; i += THREADS) {
        const int r = i / N, n = i % N, s = st0 + r;
        sBt[r * LDN + n] = s < Lc ? load_post<Tx, CONV>(a, a.Bm, a.b_stride, b, c0 + s, g * N + n,
                                                        HP + g * N + n, cdim)
                                  : 0.f;
      }
      for (int i = tid; i < TT * P; i += THREADS) {
        const int r = i / P, p = i % P, s = st0 + r;
        sX[r * LDP + p] = s < Lc ? load_post<Tx, CONV>(a, a.x, a.x_stride, b, c0 + s, h * P + p,
                                                       h * P + p, cdim)
                                 : 0.f;
      }
      __syncthreads();
      for (int q = 0; q < TT && st0 + q < Lc; ++q) {
        const int s = st0 + q;
        const float ws = expf(lam_last - sLam[s]) * sDel[s] * sX[q * LDP + sp];
#pragma unroll
        for (int k = 0; k < 32; ++k) hacc[k] += ws * sBt[q * LDN + sn0 + k];
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32; ++k) sH[sp * LDN + sn0 + k] = hacc[k];
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

template <typename Tx, typename Ta, typename Ty>
hipError_t launch_typed(const ScanArgs& a, hipStream_t stream) {
  const size_t lds = sizeof(float) * ((size_t)P * LDN + 2 * a.chunk + 2 * TT * LDN + TT * LDP +
                                      TT * LDT + 4);
  const dim3 grid(a.batch * a.nheads);
  if (a.conv_w != nullptr) {
    auto k = scan_f32_kernel<Tx, Ta, Ty, true>;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k, grid, dim3(THREADS), lds, stream, a);
  } else {
    auto k = scan_f32_kernel<Tx, Ta, Ty, false>;
    (void)hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k, grid, dim3(THREADS), lds, stream, a);
  }
  return hipGetLastError();
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
