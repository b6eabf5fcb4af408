// The block around the layer: the pre-norm RMSNorm and the bf16 matrix-core
// projection out = A W^T (+ residual) that serves as in_proj and out_proj
// (the pre-norm residual block x + mamba(norm(x)) of "Nemotron-H style Hybrid
// Mamba-Transformer 3B feasibility study", section 3.2, approach A; the
// projections hold about 3 * expand * d_model^2 parameters per layer, its
// section 2.4).
//
// gfx950 only.  The projection is a dense contraction, so it runs on the
// matrix cores: 256 x 256 output tiles per workgroup of 8 waves (two per
// SIMD, so that one wave's MFMAs cover the other's LDS reads), each wave a
// 128 x 64 sub-tile of 16x16x32 bf16 MFMAs with fp32 accumulators, K staged
// through LDS in steps of 64 with double buffering (one barrier per step).
#include "ssd_common.h"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ RMSNorm

constexpr int RN_THREADS = 256;

__device__ __forceinline__ void load8(const bf16* p, float v[8]) {
  const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(r[i] << 16);
    v[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(bf16* p, const float v[8]) {
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// One workgroup per token row: out = x / sqrt(mean(x^2) + eps) * w.  The sum
// of squares is taken in a fixed order (per thread, then a fixed tree), so the
// result is bitwise reproducible.  dim % 8 == 0 (checked by the caller).
template <typename Tin, typename Tout>
__global__ __launch_bounds__(RN_THREADS) void rmsnorm_kernel(const Tin* __restrict__ x,
                                                             int64_t xs,
                                                             const float* __restrict__ w,
                                                             float eps, Tout* __restrict__ out,
                                                             int64_t os, int dim) {
  __shared__ float sred[RN_THREADS / 64];
  const Tin* xr = x + (int64_t)blockIdx.x * xs;
  Tout* orow = out + (int64_t)blockIdx.x * os;
  float ss = 0.f;
  for (int i = threadIdx.x * 8; i < dim; i += RN_THREADS * 8) {
    float v[8];
    load8(xr + i, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((threadIdx.x & 63) == 0) sred[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < RN_THREADS / 64; ++i) tot += sred[i];
  const float r = 1.f / sqrtf(tot / (float)dim + eps);
  for (int i = threadIdx.x * 8; i < dim; i += RN_THREADS * 8) {
    float v[8];
    load8(xr + i, v);
    if (w != nullptr) {
      float wv[8];
      load8(w + i, wv);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * r * wv[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= r;
    }
    store8(orow + i, v);
  }
}

// ------------------------------------------------------------------ GEMM

constexpr int TM = 256, TN = 256, TK = 64, GEMM_THREADS = 512;
// LDS tiles are [row][64] bf16 (128-byte rows, no padding).  The 16-byte
// slot that holds chunk c of row r is c ^ (r % 8): the fragment reads of
// eight consecutive rows then fall on distinct bank groups, and a wave's
// direct global-to-LDS load, which fills 1 KiB of LDS lane by lane, can
// place eight whole rows.
__host__ __device__ constexpr int slot(int row, int chunk) { return chunk ^ (row & 7); }
constexpr int GROUP_M = 8;  // tile rows per group of the tile order
constexpr int NXCD = 8;

struct GemmArgs {
  const bf16* a; int64_t lda;
  const bf16* w; int64_t ldw;
  const void* res; int64_t ldr;
  void* out; int64_t ldo;
  int64_t M;
  int N, K;
  int tiles_m, tiles_n;
};

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Tile of workgroup `lin`.  Workgroups are dealt to the 8 XCDs round-robin;
// each XCD is given a contiguous run of the tile order, and the tile order
// walks GROUP_M tile rows column by column, so the tiles resident on one XCD
// at a time share rows of A and of W in that XCD's L2.
__device__ __forceinline__ void tile_of(int lin, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  const int per = total / NXCD, rem = total % NXCD;
  const int x = lin % NXCD, i = lin / NXCD;
  const int t = x * per + min(x, rem) + i;
  const int group = GROUP_M * tiles_n;
  const int first_m = (t / group) * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in = t % group;
  tm = first_m + in % gsize;
  tn = in / gsize;
}

template <typename T> __device__ __forceinline__ void load4(const T* p, float v[4]);
template <> __device__ __forceinline__ void load4<float>(const float* p, float v[4]) {
  const float4 r = *reinterpret_cast<const float4*>(p);
  v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
}
template <> __device__ __forceinline__ void load4<bf16>(const bf16* p, float v[4]) {
  const u32x2 r = *reinterpret_cast<const u32x2*>(p);
  v[0] = __uint_as_float(r[0] << 16); v[1] = __uint_as_float(r[0] & 0xffff0000u);
  v[2] = __uint_as_float(r[1] << 16); v[3] = __uint_as_float(r[1] & 0xffff0000u);
}
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16* p, const float v[4]) {
  bf16x4 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<bf16x4*>(p) = o;
}

// out[m][n] = sum_k A[m][k] W[n][k] (+ R[m][n]); A, W bf16 with K contiguous,
// fp32 accumulation, R of type TRes, out of type TOut.  K % 8 == 0 and every
// row 16-byte aligned (checked by the caller); rows past M or N are read
// clamped and their products never stored; columns past K are zeroed in LDS.
template <typename TOut, typename TRes>
__global__ __launch_bounds__(GEMM_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) bf16 sA[2][TM * TK];
  __shared__ __attribute__((aligned(1024))) bf16 sW[2][TN * TK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int wm = wv >> 2, wn = wv & 3;  // this wave's 128 x 64 sub-tile
  int tm, tn;
  tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * TM;
  const int n0 = tn * TN;

  // Direct loads: step i of wave wv fills tile rows 32 wv + 8 i .. + 7; lane l
  // fills slot l % 8 of row 32 wv + 8 i + l / 8, i.e. that row's chunk
  // (l % 8) ^ (l / 8).  Rows past M or N re-read the last row; chunks past K
  // re-read the row's last chunk (and are zeroed below).
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ lrow;
  const bf16* ga = g.a + min(m0 + 32 * wv + lrow, g.M - 1) * g.lda + 8 * lchunk;
  const bf16* gw = g.w + (int64_t)min(n0 + 32 * wv + lrow, g.N - 1) * g.ldw + 8 * lchunk;
  auto dload = [&](int kt, int buf) {
    const int k = min(kt * TK, g.K - 8 * (lchunk + 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t ra = min(m0 + 32 * wv + 8 * i + lrow, g.M - 1) - min(m0 + 32 * wv + lrow, g.M - 1);
      const int64_t rw = min(n0 + 32 * wv + 8 * i + lrow, g.N - 1) - min(n0 + 32 * wv + lrow, g.N - 1);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(ga + ra * g.lda + k),
          (__attribute__((address_space(3))) void*)&sA[buf][(32 * wv + 8 * i) * TK], 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(gw + rw * g.ldw + k),
          (__attribute__((address_space(3))) void*)&sW[buf][(32 * wv + 8 * i) * TK], 16, 0, 0);
    }
  };
  // after this wave's loads of the last step have landed: zero the chunks
  // past K.  Each lane clears exactly the slots its own direct loads filled
  // (slot l % 8 of rows 32 wv + 8 i + l / 8, which holds chunk lchunk), so
  // the wave's own wait for its loads orders every clear after the load it
  // replaces; a slot filled by another wave is never cleared here.
  const int nk = (g.K + TK - 1) / TK;
  const int kvalid = (g.K - (nk - 1) * TK) / 8;  // valid chunks of the last step
  auto zero_tail = [&](int buf) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (lchunk >= kvalid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 32 * wv + 8 * i + lrow;
        *reinterpret_cast<u32x4*>(&sA[buf][row * TK + 8 * slot(row, lchunk)]) = zero;
        *reinterpret_cast<u32x4*>(&sW[buf][row * TK + 8 * slot(row, lchunk)]) = zero;
      }
    }
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  dload(0, 0);
  if (nk == 1 && kvalid < 8) {
    __builtin_amdgcn_s_waitcnt(0);  // the loaded chunks first, then the zeros
    zero_tail(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // every fragment of this step first: the next step's direct loads, into
    // the other buffer, are issued only after this step's LDS reads.  The
    // wait counter does not tell those loads from LDS reads, so the products
    // below wait for all of this step's reads; the other wave on the SIMD
    // runs its products meanwhile.
    bf16x8 fa[2][8], fw[2][4];
#pragma unroll
    for (int s = 0; s < TK / 32; ++s) {
      const int c = slot(r16, 4 * s + q);  // rows 16 i + r16: row % 8 == r16 % 8
      fa[s][0] = *reinterpret_cast<const bf16x8*>(&sA[buf][(wm * 128 + r16) * TK + 8 * c]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fw[s][j] = *reinterpret_cast<const bf16x8*>(&sW[buf][(wn * 64 + 16 * j + r16) * TK + 8 * c]);
#pragma unroll
      for (int i = 1; i < 8; ++i)
        fa[s][i] = *reinterpret_cast<const bf16x8*>(&sA[buf][(wm * 128 + 16 * i + r16) * TK + 8 * c]);
    }
    // unconditional (the last step re-reads a tile into the spent buffer), so
    // that no branch separates the reads above from the products below; the
    // fences keep the loads ahead of the products, so that they have the
    // whole step to land
    __builtin_amdgcn_sched_barrier(0);
    dload(min(kt + 1, nk - 1), buf ^ 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < TK / 32; ++s)
      // W as the A operand: the result lands transposed, element r of
      // acc[i][j] at n = 16 j + 4 q + r, m = 16 i + r16 of the sub-tile
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma(fw[s][j], fa[s][i], acc[i][j]);
    if (kt + 2 == nk && kvalid < 8) {
      __builtin_amdgcn_s_waitcnt(0);
      zero_tail(buf ^ 1);
    }
    __syncthreads();
  }

  // epilogue: 4 consecutive columns per lane and tile
  TOut* out = static_cast<TOut*>(g.out);
  const TRes* res = static_cast<const TRes*>(g.res);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + wm * 128 + 16 * i + r16;
    if (m >= g.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + 16 * j + 4 * q;
      if (n >= g.N) continue;
      float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
      if (n + 4 <= g.N) {
        if (res != nullptr) {
          float rv[4];
          load4(res + m * g.ldr + n, rv);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += rv[e];
        }
        store4(out + m * g.ldo + n, v);
      } else {  // the ragged last columns, one at a time
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < g.N) {
            if (res != nullptr) v[e] += to_f32(res[m * g.ldr + n + e]);
            out[m * g.ldo + n + e] = from_f32<TOut>(v[e]);
          }
      }
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(const void* x, int64_t xs, ssd_dtype_t x_dtype, const float* w,
                          float eps, void* out, int64_t os, ssd_dtype_t out_dtype, int64_t ntok,
                          int dim, hipStream_t stream) {
  if (ntok <= 0) return hipSuccess;
  const dim3 grid((unsigned)ntok), block(RN_THREADS);
  if (x_dtype == SSD_BF16 && out_dtype == SSD_BF16)
    rmsnorm_kernel<bf16, bf16><<<grid, block, 0, stream>>>(
        static_cast<const bf16*>(x), xs, w, eps, static_cast<bf16*>(out), os, dim);
  else if (x_dtype == SSD_BF16)
    rmsnorm_kernel<bf16, float><<<grid, block, 0, stream>>>(
        static_cast<const bf16*>(x), xs, w, eps, static_cast<float*>(out), os, dim);
  else if (out_dtype == SSD_BF16)
    rmsnorm_kernel<float, bf16><<<grid, block, 0, stream>>>(
        static_cast<const float*>(x), xs, w, eps, static_cast<bf16*>(out), os, dim);
  else
    rmsnorm_kernel<float, float><<<grid, block, 0, stream>>>(
        static_cast<const float*>(x), xs, w, eps, static_cast<float*>(out), os, dim);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(const void* a, int64_t lda, const void* w, int64_t ldw,
                            const void* res, int64_t ldr, ssd_dtype_t res_dtype, void* out,
                            int64_t ldo, ssd_dtype_t out_dtype, int64_t M, int N, int K,
                            hipStream_t stream) {
  if (M <= 0 || N <= 0) return hipSuccess;
  GemmArgs g{};
  g.a = static_cast<const bf16*>(a); g.lda = lda;
  g.w = static_cast<const bf16*>(w); g.ldw = ldw;
  g.res = res; g.ldr = ldr;
  g.out = out; g.ldo = ldo;
  g.M = M; g.N = N; g.K = K;
  g.tiles_m = (int)((M + TM - 1) / TM);
  g.tiles_n = (N + TN - 1) / TN;
  const dim3 grid((unsigned)((int64_t)g.tiles_m * g.tiles_n)), block(GEMM_THREADS);
  const bool rb = res != nullptr && res_dtype == SSD_BF16;
  if (out_dtype == SSD_BF16) {
    if (rb) gemm_bf16_kernel<bf16, bf16><<<grid, block, 0, stream>>>(g);
    else gemm_bf16_kernel<bf16, float><<<grid, block, 0, stream>>>(g);
  } else {
    if (rb) gemm_bf16_kernel<float, bf16><<<grid, block, 0, stream>>>(g);
    else gemm_bf16_kernel<float, float><<<grid, block, 0, stream>>>(g);
  }
  return hipGetLastError();
}

}  // namespace ssd
