// One-token decode step of the Mamba-2 layer: conv step on the ring of the
// last K-1 raw inputs, then h <- exp(delta A) h + delta x B^T, y = h C + D x,
// gated by SiLU(z).  The state is of fixed size per sequence (the
// O(1)-per-token decode of the "Nemotron-H paper explainer", Transformer-vs-
// Mamba table; the fixed Mamba cache of "Hybrid Architectures ..." summary,
// Appendix C).
//
// HBM-bound: the fp32 state (32 KiB per head) is read and written once per
// step and is ~98% of the bytes.  Short-lived workgroups that each sweep a
// short contiguous range stream HBM faster on this GPU than a few that walk
// many heads one after the other.  Two implementations, which differ in
// where the conv step happens:
//
// conv_step_kernel + state_stream_kernel (with a workspace): the conv step
// and ring shift of every channel first, one thread per (sequence, channel),
// writing the post-conv x|B|C in fp32 to the workspace; then one workgroup of
// 256 threads per (sequence, head, block of 16 state rows), two float4 of the
// state per thread, which reads it from there (the 64 workgroups of a
// sequence and group share B and C through L2).
//
// state_conv_stream_kernel + ring_shift_bc_kernel (no workspace): one
// workgroup of 256 threads per (sequence, head), eight float4 of the state
// per thread, all loaded after the conv's small inputs.  It convolves what it
// needs from the unshifted ring itself (the group's B and C, the head's x)
// and shifts the ring columns of the head's x channels; B and C columns,
// which every workgroup of the group reads, are shifted by a second small
// launch.
#include <mutex>

#include "ssd_common.h"

namespace ssd {
namespace {

constexpr int P = 64;
constexpr int N = 128;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ with a workspace

// v moved across lanes by the DPP control CTRL (lanes whose source lies
// outside the pattern, or outside ROW_MASK's rows, read 0)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or0(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Sum over each half wave (lanes 0..31 and 32..63), complete in lanes 31 and
// 63: prefix sums within each row of 16 lanes (row_shr 1, 2, 4, 8), then the
// last lane of rows 0 and 2 added into rows 1 and 3 (row_bcast:15).  The
// order of the additions is fixed, so the sum is deterministic.
__device__ __forceinline__ float half_wave_sum(float v) {
  v += dpp_or0<0x111, 0xf>(v);
  v += dpp_or0<0x112, 0xf>(v);
  v += dpp_or0<0x114, 0xf>(v);
  v += dpp_or0<0x118, 0xf>(v);
  v += dpp_or0<0x142, 0xa>(v);
  return v;
}

constexpr int SS_THREADS = 256;
constexpr int SS_JJ = 2;                          // float4 of the state per thread
constexpr int SS_ROWS = SS_THREADS / (N / 4) * SS_JJ;  // 16 state rows per workgroup
constexpr int CONV_THREADS = 256;

// Conv step of every channel: post[b, c] = SiLU(conv_b[c] + sum_k w[c, k]
// u_k) over the ring's K-1 raw inputs (oldest first) and the new one, and the
// ring shifted by one token; without a conv post[b, c] is the input itself.
// One thread per (sequence, channel): it reads and writes only that
// channel's ring column, so no ordering between threads is needed.
template <typename Tx>
__global__ __launch_bounds__(CONV_THREADS) void conv_step_kernel(
    const Tx* __restrict__ xbc, Tx* __restrict__ ring, const float* __restrict__ conv_w,
    const float* __restrict__ conv_b, int K, int64_t C, int64_t total, float* __restrict__ post) {
  const int64_t i = (int64_t)blockIdx.x * CONV_THREADS + threadIdx.x;
  if (i >= total) return;
  const Tx raw = xbc[i];
  float out = to_f32(raw);
  if (conv_w != nullptr) {
    const int64_t b = i / C, c = i - b * C;
    float u = conv_b ? conv_b[c] : 0.f;
    if (K > 1) {
      Tx* r = ring + b * (K - 1) * C + c;  // r[k*C]: row k, oldest first
      for (int k = 0; k < K - 1; ++k) u += conv_w[c * K + k] * to_f32(r[(int64_t)k * C]);
      for (int k = 0; k + 1 < K - 1; ++k) r[(int64_t)k * C] = r[(int64_t)(k + 1) * C];
      r[(int64_t)(K - 2) * C] = raw;
    }
    u += conv_w[c * K + K - 1] * out;
    out = silu_f32(u);
  }
  post[i] = out;
}

// State update and readout from the post-conv values.  Workgroup (h, rb) of
// sequence b owns state rows 16 rb .. 16 rb + 15 of head h; thread t holds
// columns 4 (t % 32) .. +3 of rows 16 rb + t / 32 and 16 rb + t / 32 + 8.
// Each row's readout h C is summed over the half wave that holds it.
template <typename Ta, typename Ty>
__global__ __launch_bounds__(SS_THREADS) void state_stream_kernel(
    float* __restrict__ state, const float* __restrict__ post, const Ta* __restrict__ dt,
    const Ta* __restrict__ z, const float* __restrict__ A, const float* __restrict__ D,
    const float* __restrict__ dt_bias, int softplus, Ty* __restrict__ y, int H, int G) {
  constexpr int RB = P / SS_ROWS;
  const int h = blockIdx.x / RB, rb = blockIdx.x - h * RB, b = blockIdx.y;
  const int g = h / (H / G);
  const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N, C = HP + 2 * GN;
  const int tid = threadIdx.x;
  const int p0 = SS_ROWS * rb + (tid >> 5), n4 = 4 * (tid & 31);
  f32x4* sp = reinterpret_cast<f32x4*>(state + (((int64_t)b * H + h) * P + p0) * N + n4);
  f32x4 s[SS_JJ];
#pragma unroll
  for (int j = 0; j < SS_JJ; ++j) s[j] = __builtin_nontemporal_load(sp + j * 8 * (N / 4));
  const float* pb = post + (int64_t)b * C;
  const f32x4 Bv = *reinterpret_cast<const f32x4*>(pb + HP + (int64_t)g * N + n4);
  const f32x4 Cv = *reinterpret_cast<const f32x4*>(pb + HP + GN + (int64_t)g * N + n4);
  const float delta = make_delta(to_f32(dt[(int64_t)b * H + h]), dt_bias, h, softplus);
  const float a = __expf(delta * A[h]);
  const float Dh = D ? D[h] : 0.f;
#pragma unroll
  for (int j = 0; j < SS_JJ; ++j) {
    const int p = p0 + 8 * j;
    const int64_t hp = (int64_t)h * P + p;
    const float xp = pb[hp];
    const float gate = z != nullptr ? silu_f32(to_f32(z[(int64_t)b * HP + hp])) : 1.f;
    s[j] = a * s[j] + (delta * xp) * Bv;
    __builtin_nontemporal_store(s[j], sp + j * 8 * (N / 4));
    const float acc =
        half_wave_sum(s[j].x * Cv.x + s[j].y * Cv.y + s[j].z * Cv.z + s[j].w * Cv.w);
    if ((tid & 31) == 31) y[(int64_t)b * HP + hp] = from_f32<Ty>((acc + Dh * xp) * gate);
  }
}

// ------------------------------------------------------------ without a workspace

// Post-conv value of channel c of sequence b: SiLU(conv_b[c] + sum_k w[c, k]
// u_k) over the ring's K-1 raw inputs (oldest first) and the new one, summed
// in the order conv_step_kernel uses; without a conv, the input itself.  With
// SHIFT the channel's ring column is also shifted by one token (the caller
// owns that column).
template <bool SHIFT, typename Tx>
__device__ __forceinline__ float conv_channel(const Tx* __restrict__ xbc, Tx* __restrict__ ring,
                                              const float* __restrict__ conv_w,
                                              const float* __restrict__ conv_b, int K, int64_t b,
                                              int64_t C, int64_t c) {
  const Tx raw = xbc[b * C + c];
  float out = to_f32(raw);
  if (conv_w == nullptr) return out;
  float u = conv_b ? conv_b[c] : 0.f;
  if (K > 1) {
    Tx* r = ring + b * (K - 1) * C + c;  // r[k*C]: row k, oldest first
    for (int k = 0; k < K - 1; ++k) u += conv_w[c * K + k] * to_f32(r[(int64_t)k * C]);
    if (SHIFT) {
      for (int k = 0; k + 1 < K - 1; ++k) r[(int64_t)k * C] = r[(int64_t)(k + 1) * C];
      r[(int64_t)(K - 2) * C] = raw;
    }
  }
  u += conv_w[c * K + K - 1] * out;
  return silu_f32(u);
}

// delta, exp(delta A) and D of head h into out[0..2]
__device__ __forceinline__ void sdelta_of(float dtv, const float* __restrict__ dt_bias, int h,
                                          int softplus, const float* __restrict__ A,
                                          const float* __restrict__ D, float (&out)[3]) {
  const float delta = make_delta(dtv, dt_bias, h, softplus);
  out[0] = delta;
  out[1] = __expf(delta * A[h]);
  out[2] = D ? D[h] : 0.f;
}

// One workgroup per head: every workgroup convolves the group's B and C, so
// the fewer the workgroups, the less of that (measured at B = 256, H = 128:
// 0.354 ms per step with the head's 64 rows per workgroup, 0.368 with 32,
// 0.377 with 16).
constexpr int CS_JJ = 8;                          // float4 of the state per thread
constexpr int CS_ROWS = SS_THREADS / (N / 4) * CS_JJ;  // state rows per workgroup: 64

// The raw inputs of one channel's conv step at width 4, loaded together so
// that they are in flight with the state's loads; summed in the order
// conv_step_kernel uses.
template <typename Tx>
struct Conv4 {
  float w0, w1, w2, w3, bias, r0, r1, r2, raw;
  Tx traw, t1, t2;
  __device__ __forceinline__ void load(const Tx* __restrict__ xbc, const Tx* __restrict__ ring,
                                       const float* __restrict__ conv_w,
                                       const float* __restrict__ conv_b, int64_t b, int64_t C,
                                       int64_t c) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(conv_w + c * 4);
    w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    bias = conv_b ? conv_b[c] : 0.f;
    const Tx* r = ring + b * 3 * C + c;
    const Tx t0 = r[0];
    t1 = r[C], t2 = r[2 * C];
    traw = xbc[b * C + c];
    r0 = to_f32(t0);
  }
  __device__ __forceinline__ float value() {
    r1 = to_f32(t1), r2 = to_f32(t2), raw = to_f32(traw);
    float u = bias;
    u += w0 * r0;
    u += w1 * r1;
    u += w2 * r2;
    u += w3 * raw;
    return silu_f32(u);
  }
  // the channel's ring column shifted by one token
  __device__ __forceinline__ void shift(Tx* __restrict__ ring, int64_t b, int64_t C, int64_t c) {
    Tx* r = ring + b * 3 * C + c;
    r[0] = t1, r[C] = t2, r[2 * C] = traw;
  }
};

// The decode step with no workspace, first launch.  Workgroup (h, rb) of
// sequence b owns state rows CS_ROWS rb .. CS_ROWS rb + CS_ROWS - 1 of head h
// (with CS_ROWS = 64, the whole head): thread t holds columns 4 (t % 32) ..
// +3 of rows CS_ROWS rb + t / 32 + 8 j.  It takes the conv step of what those
// rows need straight from the (unshifted) ring: B and C of the head's group
// (one channel per thread) and x of its rows, into LDS.  The ring columns of
// those x channels belong to this workgroup alone, so it shifts them;
// the group's B and C columns are read by every workgroup of the group, so
// ring_shift_bc_kernel shifts them afterwards.  W4 (conv width 4, the
// layer's): the conv's inputs are loaded before the state, so that the conv
// is computed while the state is in flight; otherwise (other widths, no
// conv) the conv follows the state's loads.  GATED (width 4 only): z is given.
template <bool W4, bool GATED, typename Tx, typename Ta, typename Ty>
__global__ __launch_bounds__(SS_THREADS) void state_conv_stream_kernel(
    float* __restrict__ state, const Tx* __restrict__ xbc, Tx* __restrict__ ring,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, int K,
    const Ta* __restrict__ dt, const Ta* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ D, const float* __restrict__ dt_bias, int softplus,
    Ty* __restrict__ y, int H, int G) {
  static_assert(2 * N == SS_THREADS, "one thread per B and C channel of a group");
  __shared__ f32x4 sbc[2 * N / 4];  // post-conv B | C of the group
  __shared__ float sx[SS_THREADS];  // post-conv x of the workgroup's rows (slots 0 .. CS_ROWS - 1)
  constexpr int RB = P / CS_ROWS;
  const int h = blockIdx.x / RB, rb = blockIdx.x - h * RB, b = blockIdx.y;
  const int g = h / (H / G);
  const int64_t HP = (int64_t)H * P, GN = (int64_t)G * N, C = HP + 2 * GN;
  const int tid = threadIdx.x;
  const int p0 = CS_ROWS * rb + (tid >> 5), n4 = 4 * (tid & 31);
  const int64_t cbc = HP + (int64_t)g * N + (tid < N ? tid : GN + (tid - N));
  const int64_t cx = (int64_t)h * P + CS_ROWS * rb + (tid & (CS_ROWS - 1));
  f32x4* sp = reinterpret_cast<f32x4*>(state + (((int64_t)b * H + h) * P + p0) * N + n4);
  f32x4 s[CS_JJ];
  float gate[CS_JJ];
  float sdel[3];  // delta, exp(delta A), D of the head
  if constexpr (W4) {
    // every small load first (dt, z, the conv's inputs; the x channel's by all
    // threads, so no branch splits them), then the state: waiting for the
    // small ones then leaves the state in flight
    const Ta dtv = dt[(int64_t)b * H + h];
    Ta zr[CS_JJ];
    if constexpr (GATED) {
#pragma unroll
      for (int j = 0; j < CS_JJ; ++j) zr[j] = z[(int64_t)b * HP + (int64_t)h * P + p0 + 8 * j];
    }
    Conv4<Tx> vbc, vx;
    vbc.load(xbc, ring, conv_w, conv_b, b, C, cbc);
    vx.load(xbc, ring, conv_w, conv_b, b, C, cx);
#pragma unroll
    for (int j = 0; j < CS_JJ; ++j) s[j] = __builtin_nontemporal_load(sp + j * 8 * (N / 4));
    reinterpret_cast<float*>(sbc)[tid] = vbc.value();
    // every thread keeps its x channel's value (threads 0 .. CS_ROWS - 1
    // hold the distinct ones), so that the loads above are not moved into
    // the branch
    sx[tid] = vx.value();
    if (tid < CS_ROWS) vx.shift(ring, b, C, cx);
#pragma unroll
    for (int j = 0; j < CS_JJ; ++j) gate[j] = GATED ? silu_f32(to_f32(zr[j])) : 1.f;
    sdelta_of(to_f32(dtv), dt_bias, h, softplus, A, D, sdel);
  } else {
#pragma unroll
    for (int j = 0; j < CS_JJ; ++j) s[j] = __builtin_nontemporal_load(sp + j * 8 * (N / 4));
    reinterpret_cast<float*>(sbc)[tid] = conv_channel<false>(xbc, ring, conv_w, conv_b, K, b, C, cbc);
    if (tid < CS_ROWS) sx[tid] = conv_channel<true>(xbc, ring, conv_w, conv_b, K, b, C, cx);
#pragma unroll
    for (int j = 0; j < CS_JJ; ++j)
      gate[j] = z != nullptr ? silu_f32(to_f32(z[(int64_t)b * HP + (int64_t)h * P + p0 + 8 * j])) : 1.f;
    sdelta_of(to_f32(dt[(int64_t)b * H + h]), dt_bias, h, softplus, A, D, sdel);
  }
  const float delta = sdel[0], a = sdel[1], Dh = sdel[2];
  __syncthreads();
  const f32x4 Bv = sbc[tid & 31];
  const f32x4 Cv = sbc[N / 4 + (tid & 31)];
#pragma unroll
  for (int j = 0; j < CS_JJ; ++j) {
    const int p = p0 + 8 * j;
    const int64_t hp = (int64_t)h * P + p;
    const float xp = sx[p - CS_ROWS * rb];
    s[j] = a * s[j] + (delta * xp) * Bv;
    __builtin_nontemporal_store(s[j], sp + j * 8 * (N / 4));
    const float acc =
        half_wave_sum(s[j].x * Cv.x + s[j].y * Cv.y + s[j].z * Cv.z + s[j].w * Cv.w);
    if ((tid & 31) == 31) y[(int64_t)b * HP + hp] = from_f32<Ty>((acc + Dh * xp) * gate[j]);
  }
}

// Second launch: the ring columns of every B and C channel shifted by one
// token, the new raw input appended.  One thread per (sequence, channel).
template <typename Tx>
__global__ __launch_bounds__(CONV_THREADS) void ring_shift_bc_kernel(
    const Tx* __restrict__ xbc, Tx* __restrict__ ring, int K, int64_t HP, int64_t C,
    int64_t nbc, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * CONV_THREADS + threadIdx.x;
  if (i >= total) return;
  const int64_t b = i / nbc, c = HP + (i - b * nbc);
  Tx* r = ring + b * (K - 1) * C + c;
  for (int k = 0; k + 1 < K - 1; ++k) r[(int64_t)k * C] = r[(int64_t)(k + 1) * C];
  r[(int64_t)(K - 2) * C] = xbc[b * C + c];
}

template <typename Tx, typename Ta, typename Ty>
hipError_t launch_typed(float* state, const void* xbc, void* ring, const float* conv_w,
                        const float* conv_b, int K, const void* dt, const void* z,
                        const float* A, const float* D, const float* dt_bias, int softplus,
                        void* y, int B, int H, int G, hipStream_t stream) {
  // width 4 with 16-byte aligned taps: the conv's loads go out before the state's
  const bool w4 = conv_w != nullptr && K == 4 && (reinterpret_cast<uintptr_t>(conv_w) & 15) == 0;
  auto kern = !w4              ? state_conv_stream_kernel<false, true, Tx, Ta, Ty>
              : z != nullptr ? state_conv_stream_kernel<true, true, Tx, Ta, Ty>
                             : state_conv_stream_kernel<true, false, Tx, Ta, Ty>;
  hipLaunchKernelGGL(kern, dim3(H * (P / CS_ROWS), B), dim3(SS_THREADS), 0, stream, state,
                     static_cast<const Tx*>(xbc), static_cast<Tx*>(ring), conv_w, conv_b, K,
                     static_cast<const Ta*>(dt), static_cast<const Ta*>(z), A, D, dt_bias,
                     softplus, static_cast<Ty*>(y), H, G);
  if (conv_w != nullptr && K > 1) {
    const int64_t HP = (int64_t)H * P, nbc = 2 * (int64_t)G * N, C = HP + nbc;
    const int64_t total = (int64_t)B * nbc;
    hipLaunchKernelGGL(ring_shift_bc_kernel<Tx>,
                       dim3((unsigned)((total + CONV_THREADS - 1) / CONV_THREADS)),
                       dim3(CONV_THREADS), 0, stream, static_cast<const Tx*>(xbc),
                       static_cast<Tx*>(ring), K, HP, C, nbc, total);
  }
  return hipGetLastError();
}

template <typename Tx, typename Ta>
hipError_t pick_y(ssd_dtype_t yd, float* state, const void* xbc, void* ring, const float* w,
                  const float* cb, int K, const void* dt, const void* z, const float* A,
                  const float* D, const float* dtb, int sp, void* y, int B, int H, int G,
                  hipStream_t s) {
  if (yd == SSD_F32)
    return launch_typed<Tx, Ta, float>(state, xbc, ring, w, cb, K, dt, z, A, D, dtb, sp, y, B, H,
                                       G, s);
  return launch_typed<Tx, Ta, bf16>(state, xbc, ring, w, cb, K, dt, z, A, D, dtb, sp, y, B, H, G,
                                    s);
}

template <typename Tx, typename Ta, typename Ty>
hipError_t launch_ws_typed(float* state, const void* xbc, void* ring, const float* conv_w,
                           const float* conv_b, int K, const void* dt, const void* z,
                           const float* A, const float* D, const float* dt_bias, int softplus,
                           void* y, int B, int H, int G, float* post, hipStream_t stream) {
  const int64_t C = (int64_t)H * P + 2 * (int64_t)G * N, total = (int64_t)B * C;
  hipLaunchKernelGGL(conv_step_kernel<Tx>, dim3((unsigned)((total + CONV_THREADS - 1) / CONV_THREADS)),
                     dim3(CONV_THREADS), 0, stream, static_cast<const Tx*>(xbc),
                     static_cast<Tx*>(ring), conv_w, conv_b, K, C, total, post);
  hipLaunchKernelGGL((state_stream_kernel<Ta, Ty>), dim3(H * (P / SS_ROWS), B), dim3(SS_THREADS),
                     0, stream, state, post, static_cast<const Ta*>(dt),
                     static_cast<const Ta*>(z), A, D, dt_bias, softplus, static_cast<Ty*>(y), H,
                     G);
  return hipGetLastError();
}

template <typename Tx, typename Ta>
hipError_t pick_y_ws(ssd_dtype_t yd, float* state, const void* xbc, void* ring, const float* w,
                     const float* cb, int K, const void* dt, const void* z, const float* A,
                     const float* D, const float* dtb, int sp, void* y, int B, int H, int G,
                     float* post, hipStream_t s) {
  if (yd == SSD_F32)
    return launch_ws_typed<Tx, Ta, float>(state, xbc, ring, w, cb, K, dt, z, A, D, dtb, sp, y, B,
                                          H, G, post, s);
  return launch_ws_typed<Tx, Ta, bf16>(state, xbc, ring, w, cb, K, dt, z, A, D, dtb, sp, y, B, H,
                                       G, post, s);
}

}  // namespace

// ------------------------------------------------------------ without any allocation

// Scratch of the allocation-free decode step: the post-conv x|B|C of the
// step (one float per sequence and channel), in a file-scope device array
// instead of a caller's workspace.  Every device the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// uses the array's name as an address (on the host it is only a stand-in
// for the symbol); it uses the device address looked up per device below.
static __device__ __align__(256) float scratch[kNoAllocScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// The current device's address of the scratch array: looked up once per
// device, with that device current, on its first call, and kept.
hipError_t no_alloc_scratch(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_state_update(float* state, const void* xbc, ssd_dtype_t xd, void* ring,
                               const float* conv_w, const float* conv_b, int K, const void* dt,
                               const void* z, ssd_dtype_t ad, const float* A, const float* D,
                               const float* dt_bias, int softplus, void* y, ssd_dtype_t yd,
                               int B, int H, int G, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (xd == SSD_BF16 && ad == SSD_BF16)
    return pick_y<bf16, bf16>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                              softplus, y, B, H, G, s);
  if (xd == SSD_BF16)
    return pick_y<bf16, float>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                               softplus, y, B, H, G, s);
  if (ad == SSD_BF16)
    return pick_y<float, bf16>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                               softplus, y, B, H, G, s);
  return pick_y<float, float>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                              softplus, y, B, H, G, s);
}

hipError_t launch_state_update_ws(float* state, const void* xbc, ssd_dtype_t xd, void* ring,
                                  const float* conv_w, const float* conv_b, int K, const void* dt,
                                  const void* z, ssd_dtype_t ad, const float* A, const float* D,
                                  const float* dt_bias, int softplus, void* y, ssd_dtype_t yd,
                                  int B, int H, int G, float* post, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (xd == SSD_BF16 && ad == SSD_BF16)
    return pick_y_ws<bf16, bf16>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                                 softplus, y, B, H, G, post, s);
  if (xd == SSD_BF16)
    return pick_y_ws<bf16, float>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                                  softplus, y, B, H, G, post, s);
  if (ad == SSD_BF16)
    return pick_y_ws<float, bf16>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                                  softplus, y, B, H, G, post, s);
  return pick_y_ws<float, float>(yd, state, xbc, ring, conv_w, conv_b, K, dt, z, A, D, dt_bias,
                                 softplus, y, B, H, G, post, s);
}

}  // namespace ssd
