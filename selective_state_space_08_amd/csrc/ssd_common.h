// Shared device helpers and kernel-launch declarations for libssd.so.
// gfx950 (CDNA4) only: wave64, bf16 MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd.h"

namespace ssd {

using bf16 = __bf16;

// ------------------------------------------------------------------ numerics

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
// round to nearest even (gfx950 converts in hardware)
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// softplus(v) = log(1 + e^v) in the form that neither overflows nor cancels,
// max(v, 0) + log1p(e) with e = exp(-|v|) in (0, 1].  log1p(e) is taken as
// log(u) e / (u - 1), u = fl(1 + e): the quotient cancels the rounding of
// 1 + e (D. Goldberg, "What every computer scientist should know about
// floating-point arithmetic", 1991, theorem 4), a few ulps in all, with the
// hardware logarithm; where u rounds to 1, log1p(e) = e to within rounding.
__device__ __forceinline__ float softplus_f32(float v) {
  const float e = __expf(-fabsf(v));
  const float u = 1.f + e;
  const float d = u - 1.f;
  const float l = d == 0.f ? e : __logf(u) * (e * __builtin_amdgcn_rcpf(d));
  return fmaxf(v, 0.f) + l;
}

// SiLU(u) = u * sigmoid(u), with the hardware reciprocal (1 ulp) in place of
// an IEEE division
__device__ __forceinline__ float silu_f32(float u) {
  return u * __builtin_amdgcn_rcpf(1.f + __expf(-u));
}

// delta = softplus(dt + bias) | dt + bias
__device__ __forceinline__ float make_delta(float dt, const float* dt_bias, int h,
                                            int softplus) {
  float v = dt + (dt_bias ? dt_bias[h] : 0.f);
  return softplus ? softplus_f32(v) : v;
}

// ------------------------------------------------------------------ arguments

// Everything a scan kernel needs; passed by value as the kernel argument.
struct ScanArgs {
  const void* x;  int64_t x_stride;
  const void* Bm; int64_t b_stride;
  const void* Cm; int64_t c_stride;
  const float* conv_w; const float* conv_b; int conv_k;   // conv_w == nullptr: post-conv
  const void* conv_state_in; void* conv_state_out;
  const void* dt; int64_t dt_stride;
  const void* z;  int64_t z_stride;
  const float* A; const float* D; const float* dt_bias; int dt_softplus;
  const float* initial_state; float* final_state;
  void* y; int64_t y_stride;
  int batch, seqlen, nheads, ngroups, chunk;
  // sequence split: each (b, h) is walked as `nseg` segments of `seg_chunks` chunks
  int nseg, seg_chunks;
  float* seg_state;      // [B, H, nseg, P, N] workspace (nseg > 1)
  float* seg_logdecay;   // [B, H, nseg]       workspace (nseg > 1)
  // matrix-core path: per (sequence, group, chunk) B and C in the layouts its
  // products read, written by the pack pass (workspace)
  const void* bc_pack;
};

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error; shapes are validated by the caller.

// hist_stride: elements between consecutive history rows (cdim for a dense
// [B, K-1, cdim] history; larger when the channels are a slice of one)
hipError_t launch_causal_conv1d(const void* x, int64_t x_stride, ssd_dtype_t x_dtype,
                                const float* w, const float* bias, const void* hist_in,
                                void* hist_out, int64_t hist_stride, void* out,
                                int64_t out_stride, ssd_dtype_t out_dtype, int batch, int seqlen,
                                int cdim, int width, int apply_silu, hipStream_t stream);

hipError_t launch_scan_f32(const ScanArgs& a, ssd_dtype_t xbc_dtype, ssd_dtype_t act_dtype,
                           ssd_dtype_t y_dtype, hipStream_t stream);

// Runs the B|C pack pass and the walkers for a.chunk in {64, 128, 256};
// a.bc_pack must hold scan_bf16_pack_bytes(batch, seqlen, ngroups, chunk)
// bytes of workspace.
hipError_t launch_scan_bf16(const ScanArgs& a, ssd_dtype_t xbc_dtype, ssd_dtype_t act_dtype,
                            ssd_dtype_t y_dtype, hipStream_t stream);
bool scan_bf16_supports_chunk(int chunk);
size_t scan_bf16_pack_bytes(int batch, int seqlen, int ngroups, int chunk);
// walkers per (sequence, head, segment): the head's channels are split at chunk 256
int scan_bf16_walkers_per_head(int chunk);

hipError_t launch_state_update(float* state, const void* xbc, ssd_dtype_t xbc_dtype,
                               void* ring, const float* conv_w, const float* conv_b, int K,
                               const void* dt, const void* z, ssd_dtype_t act_dtype,
                               const float* A, const float* D, const float* dt_bias,
                               int softplus, void* y, ssd_dtype_t y_dtype, int batch,
                               int nheads, int ngroups, hipStream_t stream);
// The two-kernel decode step; post must hold batch * Cdim floats.
hipError_t launch_state_update_ws(float* state, const void* xbc, ssd_dtype_t xbc_dtype,
                                  void* ring, const float* conv_w, const float* conv_b, int K,
                                  const void* dt, const void* z, ssd_dtype_t act_dtype,
                                  const float* A, const float* D, const float* dt_bias,
                                  int softplus, void* y, ssd_dtype_t y_dtype, int batch,
                                  int nheads, int ngroups, float* post, hipStream_t stream);

// The allocation-free decode step keeps its post-conv x|B|C in a static
// device array of this many floats (16 MiB per device); no_alloc_scratch
// gives the current device's address of it.
constexpr int64_t kNoAllocScratchFloats = (int64_t)(16 << 20) / 4;
hipError_t no_alloc_scratch(float** out);

// Everything the backward pass needs (validated by the caller).
struct ScanBwdLaunch {
  const void* x; int64_t x_stride;
  const void* Bm; int64_t b_stride;
  const void* Cm; int64_t c_stride;
  ssd_dtype_t xbc_dtype;
  const float* conv_w; const float* conv_b; int conv_k; const void* conv_state_in;
  const void* dt; int64_t dt_stride;
  const void* z; int64_t z_stride;
  ssd_dtype_t act_dtype;
  const float* A; const float* D; const float* dt_bias; int dt_softplus;
  const float* h0;
  const void* dout; int64_t dout_stride; ssd_dtype_t dout_dtype;
  const float* dhT;
  float* dxbc; float* ddt; float* dz; float* dA; float* dD; float* ddt_bias; float* dh0;
  float* dconv_w; float* dconv_b; float* dconv_state_in;
  int batch, seqlen, nheads, ngroups;
  void* workspace;
};
hipError_t launch_scan_bwd(const ScanBwdLaunch& l, hipStream_t stream);
// Workspace of the backward pass (total bytes) and its parts' offsets.
size_t scan_bwd_workspace_layout(int batch, int seqlen, int nheads, int ngroups, int conv_width,
                                 size_t* off_post, size_t* off_states, size_t* off_dbh,
                                 size_t* off_dch, size_t* off_dpost, size_t* off_part,
                                 size_t* off_wpart);

// RMSNorm of ntok rows of dim elements (dim % 8 == 0, rows 16-byte aligned).
hipError_t launch_rmsnorm(const void* x, int64_t xs, ssd_dtype_t x_dtype, const float* w,
                          float eps, void* out, int64_t os, ssd_dtype_t out_dtype, int64_t ntok,
                          int dim, hipStream_t stream);

// out = A W^T (+ res) on the matrix cores: A [M, K] and W [N, K] bf16,
// K % 8 == 0, rows 16-byte aligned; res (res_dtype) and out (out_dtype) [M, N].
hipError_t launch_gemm_bf16(const void* a, int64_t lda, const void* w, int64_t ldw,
                            const void* res, int64_t ldr, ssd_dtype_t res_dtype, void* out,
                            int64_t ldo, ssd_dtype_t out_dtype, int64_t M, int N, int K,
                            hipStream_t stream);

// Measurement aids: one streaming pass dst = a * src over bytes / 16 words
// (in place when dst == src), and blocks x 4 waves of back-to-back bf16 MFMAs
// (iters x 8 per wave) writing blocks x 256 floats to out.
hipError_t launch_stream(void* dst, const void* src, size_t bytes, float a, hipStream_t stream);
hipError_t launch_mfma_loop(float* out, int blocks, int iters, hipStream_t stream);

// Copies (or zero-fills when src is null) n floats / n elements: used for the
// state hand-through of empty sequences.  A kernel, not hipMemsetAsync.
hipError_t launch_copy_or_zero(void* dst, const void* src, size_t bytes, hipStream_t stream);

}  // namespace ssd
