// Measurement aids: the rates this GPU actually reaches on plain streaming
// and on back-to-back bf16 matrix-core products.  They are not part of the
// layer; a benchmark divides its kernels' rates by these (beside the
// published peaks) and scales HBM byte counters by the copy's known size.
//
// gfx950 only.
#include "ssd_common.h"

namespace ssd {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int STREAM_THREADS = 256;
constexpr int STREAM_U = 2;  // 16-byte words per thread, all loaded before any store

// Streams n 16-byte words once: dst[i] = a * src[i].  In place (dst == src)
// every word is read and written back at the same address, as the decode
// step does with its state; otherwise it is a copy (a = 1).  Non-temporal
// loads and stores: the data is touched once.  One pass, no grid-stride loop.
__global__ __launch_bounds__(STREAM_THREADS) void stream_kernel(f32x4* dst, const f32x4* src,
                                                                size_t n, float a) {
  const size_t base = (size_t)blockIdx.x * STREAM_THREADS * STREAM_U + threadIdx.x;
  f32x4 v[STREAM_U];
#pragma unroll
  for (int u = 0; u < STREAM_U; ++u) {
    const size_t i = base + (size_t)u * STREAM_THREADS;
    if (i < n) v[u] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int u = 0; u < STREAM_U; ++u) {
    const size_t i = base + (size_t)u * STREAM_THREADS;
    if (i < n) __builtin_nontemporal_store(a * v[u], dst + i);
  }
}

constexpr int MFMA_THREADS = 256;  // 4 waves

// Each wave issues iters x 8 16x16x32 bf16 MFMAs on register
// operands, in 8 independent accumulator chains so that no product
// waits for the previous one (each accumulator is next read 7 products after
// it is written); the accumulators are summed and stored once, so the work
// cannot be dropped.  The eight products of an iteration are one asm
// statement: written with the builtin, the compiler rotates the accumulators
// through extra register moves each iteration, which halves the rate it
// measures.  No memory is accessed in the statement.
__global__ __launch_bounds__(MFMA_THREADS) void mfma_loop_kernel(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (float)((lane * 8 + e) % 97) - 0.05f);
    b[e] = (__bf16)(0.002f * (float)((lane * 5 + 3 * e) % 89) - 0.09f);
  }
  f32x4 c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
  for (int i = 0; i < iters; ++i) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %9, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %8, %9, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %8, %9, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %8, %9, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %9, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %8, %9, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %8, %9, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %8, %9, %7"
        : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3), "+a"(c4), "+a"(c5), "+a"(c6), "+a"(c7)
        : "v"(a), "v"(b));
  }
  // wait states before the accumulators are read by ordinary instructions
  // (the compiler cannot see that the statement above wrote them with MFMAs)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const f32x4 s = ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7));
  out[(size_t)blockIdx.x * MFMA_THREADS + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

}  // namespace

hipError_t launch_stream(void* dst, const void* src, size_t bytes, float a, hipStream_t stream) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  const size_t per = (size_t)STREAM_THREADS * STREAM_U;
  hipLaunchKernelGGL(stream_kernel, dim3((unsigned)((n + per - 1) / per)), dim3(STREAM_THREADS),
                     0, stream, static_cast<f32x4*>(dst), static_cast<const f32x4*>(src), n, a);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(float* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3((unsigned)blocks), dim3(MFMA_THREADS), 0, stream, out,
                     iters);
  return hipGetLastError();
}

}  // namespace ssd
