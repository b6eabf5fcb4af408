// One-token decode step of the Mamba-2 layer: conv step on the ring of the
// last K-1 raw inputs, then h <- exp(delta A) h + delta x B^T, y = h C + D x,
// gated by SiLU(z).  The state is of fixed size per sequence (the
// O(1)-per-token decode of the "Nemotron-H paper explainer", Transformer-vs-
// Mamba table; the fixed Mamba cache of "Hybrid Architectures ..." summary,
// Appendix C).
//
// HBM-bound: the fp32 state (32 KiB per head) is read and written once per
// step and is ~98% of the bytes.  Two implementations:
//
// state_update_kernel (no workspace): one workgroup owns one (sequence,
// group): it convolves the group's channels once (x of its H/G heads, B and
// C of the group), so the ring rows it shifts are touched by no other
// workgroup, then streams the heads' states with 16-byte coalesced,
// non-temporal accesses (512 threads, 4 float4 per thread per head),
// prefetching the next head's state while it updates the current one.
//
// conv_step_kernel + state_stream_kernel (with a workspace): the conv step
// and ring shift of every channel first, one thread per (sequence, channel),
// writing the post-conv x|B|C in fp32 to the workspace; then one workgroup of
// 256 threads per (sequence, head, block of 16 state rows), two float4 of the
// state per thread, both loaded before anything else.  Narrow workgroups that
// each sweep a short contiguous range stream HBM faster on this GPU than a
// few wide workgroups that walk many heads one after the other (measured at
// B = 256, H = 128: 0.355 ms against 0.404 ms per step), and the 40 KiB of
// post-conv values per sequence are read from L2 by the 32 workgroups that
// share them instead of being recomputed.
#include <mutex>

#include "ssd_common.h"

namespace ssd {
namespace {

constexpr int P = 64;
constexpr int N = 128;
constexpr int THREADS = 512;
constexpr int ROWS_PER_PASS = THREADS / (N / 4);  // 16 state rows per pass
constexpr int PASSES = P / ROWS_PER_PASS;         // 4 float4 per thread per head

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The state is streamed once per step and not reused: non-temporal loads
// and stores keep it from displacing other data in the caches.
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_stream(float4* p, float4 v) {
  const f32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(p));
}
// base + off bytes, for a wave-uniform base and a per-lane offset below
// 4 GiB: a scalar base and a 32-bit vector offset instead of a 64-bit
// address per lane
template <typename T>
__device__ __forceinline__ T* at_bytes(T* base, uint32_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ const T* at_bytes(const T* base, uint32_t off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}

template <typename Tx, typename Ta, typename Ty>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(8))) void state_update_kernel(
    float* __restrict__ state, const Tx* __restrict__ xbc, Tx* __restrict__ ring,
    const float* __restrict__ conv_w, const float* __restrict__ conv_b, int K,
    const Ta* __restrict__ dt, const Ta* __restrict__ z, const float* __restrict__ A,
    const float* __restrict__ D, const float* __restrict__ dt_bias, int softplus,
    Ty* __restrict__ y, int H, int G) {
  // LDS: post-conv x of the group's heads | B | C, then the gate silu(z) of
  // the group's heads, then delta, exp(delta A) and D of each head
  extern __shared__ float sxc[];
  const int g = blockIdx.x, b = blockIdx.y;
  const int hpg = H / G;
  const int HP = H * P, GN = G * N, C = HP + 2 * GN;
  const int nx = hpg * P, nch = nx + 2 * N;
  const int tid = threadIdx.x;
  float* sgate = sxc + nch;
  float* sdel = sgate + nx;
  float* sdec = sdel + hpg;
  float* sskip = sdec + hpg;

  // The first head's state does not depend on the conv step: its loads are
  // issued first, so they are in flight during it.
  const int h0 = g * hpg;
  float4* st = reinterpret_cast<float4*>(state + ((int64_t)b * H + h0) * P * N);
  // the thread's byte offset within a head's state, pass j at + j * THREADS * 16
  const uint32_t toff = (uint32_t)tid * 16;
  float4 cur[PASSES];
#pragma unroll
  for (int j = 0; j < PASSES; ++j) cur[j] = ld_stream(at_bytes(st, toff + j * THREADS * 16));

  // Everything per head that the state loop needs is read here, ahead of it:
  // inside the loop the only loads are the state stream, so waiting for one
  // head's state never waits behind a small load issued after the prefetch.
  for (int i = tid; i < nx; i += THREADS)
    sgate[i] = z != nullptr ? silu_f32(to_f32(z[(int64_t)b * HP + h0 * P + i])) : 1.f;
  if (tid < hpg) {
    const int h = h0 + tid;
    const float delta = make_delta(to_f32(dt[(int64_t)b * H + h]), dt_bias, h, softplus);
    sdel[tid] = delta;
    sdec[tid] = __expf(delta * A[h]);
    sskip[tid] = D ? D[h] : 0.f;
  }

  // conv step for the group's channels; each channel's ring column is owned
  // by this workgroup alone
  for (int i = tid; i < nch; i += THREADS) {
    const int c = i < nx ? g * nx + i
                         : (i < nx + N ? HP + g * N + (i - nx) : HP + GN + g * N + (i - nx - N));
    const Tx raw = xbc[(int64_t)b * C + c];
    float v = to_f32(raw);
    if (conv_w != nullptr) {
      Tx* r = ring + (int64_t)b * (K - 1) * C + c;  // r[k*C]: row k, oldest first
      float u = conv_b ? conv_b[c] : 0.f;
      for (int k = 0; k < K - 1; ++k) u += conv_w[(int64_t)c * K + k] * to_f32(r[(int64_t)k * C]);
      u += conv_w[(int64_t)c * K + K - 1] * v;
      for (int k = 0; k + 1 < K - 1; ++k) r[(int64_t)k * C] = r[(int64_t)(k + 1) * C];
      if (K > 1) r[(int64_t)(K - 2) * C] = raw;
      v = silu_f32(u);
    }
    sxc[i] = v;
  }
  __syncthreads();

  // thread -> float4 column n4 = tid % 32 (fixed), rows p = tid / 32 + ROWS_PER_PASS j
  const int col = tid & 31;
  const int row0 = tid >> 5;


  // one head: update the state in v, store it and the outputs
  auto head = [&](int hh, float4 (&v)[PASSES]) {
    const int h = h0 + hh;
    const float delta = sdel[hh];
    const float a = sdec[hh];
    const float Dh = sskip[hh];
    const float4 Bv = reinterpret_cast<const float4*>(sxc + nx)[col];
    const float4 Cv = reinterpret_cast<const float4*>(sxc + nx + N)[col];
    float4* sh = st + (int64_t)hh * (P * N / 4);
    Ty* yh = y + (int64_t)b * HP + (int64_t)h * P;
#pragma unroll
    for (int j = 0; j < PASSES; ++j) {
      const int p = row0 + ROWS_PER_PASS * j;
      const float xp = sxc[hh * P + p];
      const float dx = delta * xp;
      float4 s = v[j];
      s.x = a * s.x + dx * Bv.x;
      s.y = a * s.y + dx * Bv.y;
      s.z = a * s.z + dx * Bv.z;
      s.w = a * s.w + dx * Bv.w;
      st_stream(at_bytes(sh, toff + j * THREADS * 16), s);
      float acc = s.x * Cv.x + s.y * Cv.y + s.z * Cv.z + s.w * Cv.w;
      // sum over the 32 lanes holding row p (fixed butterfly order: deterministic)
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 32);
      if (col == 0) {
        const float yv = (acc + Dh * xp) * sgate[hh * P + p];
        yh[p] = from_f32<Ty>(yv);
      }
    }
  };
  auto prefetch = [&](int hh, float4 (&v)[PASSES]) {
    const float4* sn = st + (int64_t)hh * (P * N / 4);
#pragma unroll
    for (int j = 0; j < PASSES; ++j) v[j] = ld_stream(at_bytes(sn, toff + j * THREADS * 16));
  };
  // two register sets in turn: head hh from one while head hh + 1 loads
  // into the other
  float4 alt[PASSES];
  for (int hh = 0; hh < hpg; hh += 2) {
    if (hh + 1 < hpg) prefetch(hh + 1, alt);
    head(hh, cur);
    if (hh + 1 < hpg) {
      if (hh + 2 < hpg) prefetch(hh + 2, cur);
      head(hh + 1, alt);
    }
  }
}

template <typename Tx, typename Ta, typename Ty>
hipError_t launch_typed(float* state, const void* xbc, void* ring, const float* conv_w,
                        const float* conv_b, int K, const void* dt, const void* z,
                        const float* A, const float* D, const float* dt_bias, int softplus,
                        void* y, int B, int H, int G, hipStream_t stream) {
  const int hpg = H / G;
  const size_t lds = sizeof(float) * (size_t)(2 * hpg * P + 2 * N + 3 * hpg);
  if (lds > 64 * 1024) {  // many heads per group: opt in to more than 64 KiB
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&state_update_kernel<Tx, Ta, Ty>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((state_update_kernel<Tx, Ta, Ty>), dim3(G, B), dim3(THREADS), lds, stream,
                     state, static_cast<const Tx*>(xbc), static_cast<Tx*>(ring), conv_w, conv_b,
                     K, static_cast<const Ta*>(dt), static_cast<const Ta*>(z), A, D, dt_bias,
                     softplus, static_cast<Ty*>(y), H, G);
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
