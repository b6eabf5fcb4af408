// Depthwise causal conv1d + SiLU over [B, L, Cdim] (the conv in front of the
// Mamba-2 scan: kernel 4, SiLU; "Nemotron-H style Hybrid Mamba-Transformer 3B
// feasibility study", table 1.4).
//
// HBM-bound: each input element is read once and each output written once.
// A thread owns VEC adjacent channels and walks TOK consecutive tokens,
// keeping the last three inputs in registers, so neighbouring threads read
// neighbouring pieces of one token row (fully coalesced) and the 3-token halo
// is re-read only once per TOK tokens.  VEC is 4 for bf16 in and fp32 out
// (8-byte loads, one 16-byte store per lane and token: a wave's store is one
// 1 KiB piece), 8 for bf16 in and out, 4 for fp32 in.  The loads of 4 tokens
// are issued together, and large problems take windows of 128 or 256 tokens,
// which spread each thread's tap loads and halo over more outputs (bf16 in,
// fp32 out at 4 x 8192 tokens x 10240 channels: 0.645 ms with 8 channels,
// 32-token windows and one load at a time, 0.578 with 4 loads in flight,
// 0.466 with 128-token windows, 0.417 with 4 channels and 256-token windows;
// 8 loads in flight or non-temporal output stores were no faster).
#include "ssd_common.h"

namespace ssd {
namespace {

// tokens per thread (window lengths; the launch picks one, below)
constexpr int TOK_SHORT = 32, TOK_LONG = 128, TOK_WIDE = 256;
constexpr int NUM_CUS = 256;
constexpr int THREADS = 256;

template <typename T, int VEC> struct Vec;
template <> struct Vec<bf16, 8> {
  static __device__ __forceinline__ void load(const bf16* p, float* v) {
    uint4 r = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct Vec<bf16, 4> {
  static __device__ __forceinline__ void load(const bf16* p, float* v) {
    const uint2 r = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xffff0000u);
  }
};
template <> struct Vec<float, 4> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
};
template <typename T> struct Vec<T, 1> {
  static __device__ __forceinline__ void load(const T* p, float* v) { v[0] = to_f32(*p); }
};

template <typename T, int VEC>
__device__ __forceinline__ void store_vec(T* p, const float* v) {
#pragma unroll
  for (int i = 0; i < VEC; ++i) p[i] = from_f32<T>(v[i]);
}
template <>
__device__ __forceinline__ void store_vec<float, 8>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store_vec<float, 4>(float* p, const float* v) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16 a = (bf16)lo, b = (bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
template <>
__device__ __forceinline__ void store_vec<bf16, 8>(bf16* p, const float* v) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

// raw input of channels [c, c+VEC) at position tau of sequence b (tau may be
// negative: then the history row (K-1)+tau, or zero)
template <typename Tin, int VEC>
__device__ __forceinline__ void load_raw(const Tin* x, int64_t x_stride, const Tin* hist,
                                         int64_t hs, int b, int L, int K, int tau, int c,
                                         float* v) {
  if (tau >= 0) {
    Vec<Tin, VEC>::load(x + ((int64_t)b * L + tau) * x_stride + c, v);
  } else if (hist != nullptr && tau >= -(K - 1)) {
    Vec<Tin, VEC>::load(hist + ((int64_t)b * (K - 1) + (K - 1) + tau) * hs + c, v);
  } else {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] = 0.f;
  }
}

template <typename Tin, typename Tout, int VEC, int TOK>
__global__ __launch_bounds__(THREADS) void causal_conv1d_kernel(
    const Tin* __restrict__ x, int64_t x_stride, const float* __restrict__ w,
    const float* __restrict__ bias, const Tin* __restrict__ hist_in,
    Tin* __restrict__ hist_out, int64_t hs, Tout* __restrict__ out, int64_t out_stride, int L,
    int C, int K, int apply_silu) {
  const int nv = C / VEC;
  const int cv = blockIdx.x * THREADS + threadIdx.x;
  if (cv >= nv) return;
  const int c = cv * VEC;
  const int b = blockIdx.z;
  const int t0 = blockIdx.y * TOK;

  // taps right-aligned to the current token: w4[3] meets x[t], w4[3-j] meets x[t-j]
  float w4[4][VEC], bv[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    bv[i] = bias ? bias[c + i] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = j - (4 - K);
      w4[j][i] = k >= 0 ? w[(int64_t)(c + i) * K + k] : 0.f;
    }
  }

  if (t0 < L) {
    float win[3][VEC];  // x[t-3], x[t-2], x[t-1]
#pragma unroll
    for (int j = 0; j < 3; ++j)
      load_raw<Tin, VEC>(x, x_stride, hist_in, hs, b, L, K, t0 - 3 + j, c, win[j]);
    const int t1 = min(L, t0 + TOK);
    // UNR tokens per step: their loads are issued together (rows past the end
    // re-read the last row and are not stored), so that each thread keeps
    // UNR loads in flight
    constexpr int UNR = 4;
    for (int tb = t0; tb < t1; tb += UNR) {
      float cur[UNR][VEC];
#pragma unroll
      for (int r = 0; r < UNR; ++r)
        Vec<Tin, VEC>::load(x + ((int64_t)b * L + min(tb + r, t1 - 1)) * x_stride + c, cur[r]);
#pragma unroll
      for (int r = 0; r < UNR; ++r) {
        float o[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          float u = bv[i] + w4[0][i] * win[0][i] + w4[1][i] * win[1][i] +
                    w4[2][i] * win[2][i] + w4[3][i] * cur[r][i];
          o[i] = apply_silu ? silu_f32(u) : u;
          win[0][i] = win[1][i];
          win[1][i] = win[2][i];
          win[2][i] = cur[r][i];
        }
        if (tb + r < t1) store_vec<Tout, VEC>(out + ((int64_t)b * L + tb + r) * out_stride + c, o);
      }
    }
  }

  // the last token tile hands the last K-1 raw inputs on
  if (hist_out != nullptr && blockIdx.y == gridDim.y - 1) {
    for (int j = 0; j < K - 1; ++j) {
      float v[VEC];
      load_raw<Tin, VEC>(x, x_stride, hist_in, hs, b, L, K, L - (K - 1) + j, c, v);
      store_vec<Tin, VEC>(hist_out + ((int64_t)b * (K - 1) + j) * hs + c, v);
    }
  }
}

template <typename Tin, typename Tout, int VEC, int TL>
hipError_t launch_tl(const void* x, int64_t x_stride, const float* w, const float* bias,
                     const void* hist_in, void* hist_out, int64_t hs, void* out,
                     int64_t out_stride, int B, int L, int C, int K, int apply_silu,
                     int64_t gx, hipStream_t stream) {
  dim3 grid((unsigned)gx, L > 0 ? (L + TL - 1) / TL : 1, B);
  hipLaunchKernelGGL((causal_conv1d_kernel<Tin, Tout, VEC, TL>), grid, dim3(THREADS), 0, stream,
                     static_cast<const Tin*>(x), x_stride, w, bias,
                     static_cast<const Tin*>(hist_in), static_cast<Tin*>(hist_out), hs,
                     static_cast<Tout*>(out), out_stride, L, C, K, apply_silu);
  return hipGetLastError();
}

// The window length: TOK_WIDE tokens (WIDE instances only) when that still
// gives every CU at least 4 workgroups, else TOK_LONG when every CU gets one,
// else TOK_SHORT.
template <typename Tin, typename Tout, int VEC, bool WIDE>
hipError_t launch_typed(const void* x, int64_t x_stride, const float* w, const float* bias,
                        const void* hist_in, void* hist_out, int64_t hs, void* out,
                        int64_t out_stride, int B, int L, int C, int K, int apply_silu,
                        hipStream_t stream) {
  const int nv = C / VEC;
  const int64_t gx = (nv + THREADS - 1) / THREADS;
  auto wgs = [&](int tl) { return gx * ((L + tl - 1) / tl) * B; };
  if (WIDE && wgs(TOK_WIDE) >= 4 * NUM_CUS)
    return launch_tl<Tin, Tout, VEC, TOK_WIDE>(x, x_stride, w, bias, hist_in, hist_out, hs, out,
                                               out_stride, B, L, C, K, apply_silu, gx, stream);
  if (wgs(TOK_LONG) >= NUM_CUS)
    return launch_tl<Tin, Tout, VEC, TOK_LONG>(x, x_stride, w, bias, hist_in, hist_out, hs, out,
                                               out_stride, B, L, C, K, apply_silu, gx, stream);
  return launch_tl<Tin, Tout, VEC, TOK_SHORT>(x, x_stride, w, bias, hist_in, hist_out, hs, out,
                                              out_stride, B, L, C, K, apply_silu, gx, stream);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename Tin, typename Tout>
hipError_t dispatch_vec(const void* x, int64_t x_stride, const float* w, const float* bias,
                        const void* hist_in, void* hist_out, int64_t hs, void* out,
                        int64_t out_stride, int B, int L, int C, int K, int apply_silu,
                        hipStream_t stream) {
  // bf16 in and fp32 out: 4 channels per thread, so that each lane's output
  // row is one 16-byte store and a wave's store is 1 KiB in one piece; its
  // registers then leave room for 256-token windows
  constexpr bool BF_TO_F32 = sizeof(Tin) == 2 && sizeof(Tout) == 4;
  constexpr int V = sizeof(Tin) == 2 ? (BF_TO_F32 ? 4 : 8) : 4;
  const bool vec_ok = C % V == 0 && x_stride % V == 0 && out_stride % V == 0 && hs % V == 0 &&
                      aligned16(x) &&
                      (hist_in == nullptr || aligned16(hist_in)) &&
                      (hist_out == nullptr || aligned16(hist_out)) &&
                      (sizeof(Tout) == 2 ? aligned16(out) && out_stride % 8 == 0
                                         : aligned16(out));
  if (vec_ok)
    return launch_typed<Tin, Tout, V, BF_TO_F32>(x, x_stride, w, bias, hist_in, hist_out, hs, out,
                                      out_stride, B, L, C, K, apply_silu, stream);
  return launch_typed<Tin, Tout, 1, false>(x, x_stride, w, bias, hist_in, hist_out, hs, out,
                                    out_stride, B, L, C, K, apply_silu, stream);
}

}  // namespace

hipError_t launch_causal_conv1d(const void* x, int64_t x_stride, ssd_dtype_t x_dtype,
                                const float* w, const float* bias, const void* hist_in,
                                void* hist_out, int64_t hs, void* out, int64_t out_stride,
                                ssd_dtype_t out_dtype, int B, int L, int C, int K,
                                int apply_silu, hipStream_t stream) {
  if (x_dtype == SSD_BF16 && out_dtype == SSD_F32)
    return dispatch_vec<bf16, float>(x, x_stride, w, bias, hist_in, hist_out, hs, out, out_stride,
                                     B, L, C, K, apply_silu, stream);
  if (x_dtype == SSD_BF16 && out_dtype == SSD_BF16)
    return dispatch_vec<bf16, bf16>(x, x_stride, w, bias, hist_in, hist_out, hs, out, out_stride,
                                    B, L, C, K, apply_silu, stream);
  if (x_dtype == SSD_F32 && out_dtype == SSD_F32)
    return dispatch_vec<float, float>(x, x_stride, w, bias, hist_in, hist_out, hs, out, out_stride,
                                      B, L, C, K, apply_silu, stream);
  return dispatch_vec<float, bf16>(x, x_stride, w, bias, hist_in, hist_out, hs, out, out_stride, B,
                                   L, C, K, apply_silu, stream);
}

}  // namespace ssd
