// Chunked selective scan on the gfx950 matrix cores (SSD_MATH_BF16).
//
// The recurrence h_t = exp(delta_t A) h_{t-1} + delta_t x_t B_t^T,
// y_t = C_t h_t + D x_t ("Hybrid Architectures for Language Models" summary,
// section 2 Background) is evaluated in its chunked matrix form (the same
// section: SSD recasts the state-space computation as matrix multiplies).
// For a chunk of Q tokens (Q = 64, 128 or 256, one instance each) with
// cumulative log decay Lam_t:
//   Y      = (C B^T o exp(Lam_t - Lam_s) delta_s [s <= t]) X + diag(exp Lam) C H^T
//   H_next = exp(Lam_last) H + (X o w)^T B,  w_s = exp(Lam_last - Lam_s) delta_s
//   out    = (Y + D x) * silu(z)
// All products are 16x16x32 bf16 MFMAs with fp32 accumulation.  The chunk
// state product, whose result is carried across the whole sequence, splits
// both operands into bf16 hi + lo parts and sums hi*hi + hi*lo + lo*hi, so
// the carried state keeps ~16 mantissa bits instead of 8.
//
// Two kernels:
//
// bc_pack_kernel, one workgroup per (sequence, group, chunk), applies the
// conv + SiLU to B and C once per group (or takes them post-conv) and writes
// them in the forms the matrix cores read, per chunk: C and B as bf16 [t][n],
// and B as bf16 hi and lo parts transposed, [n][s].  The heads of a group
// then read their B and C from this pack (through L2) with 16-byte loads and
// no conversion work.
//
// scan_bf16_kernel ("walker", 8 waves, two per SIMD) owns one (sequence,
// head) -- or one segment of it, see below; at Q = 256 one half of the head's
// channels -- and walks its chunks in order, carrying its rows of the fp32
// state H [64 x 128] in MFMA accumulator registers, so no state goes to HBM
// between chunks.  Wave w owns the 16 state columns n in [16 w, 16 w + 16),
// held as rows of H^T, and the output tokens of one or two 16-token row
// tiles, chosen so that the two waves of a SIMD share the causal triangle of
// C B^T evenly (at Q = 128, tiles w < 4 ? w : 11 - w: a SIMD owns tiles i
// and 7 - i).  Each wave loads the C rows of its tokens and the B^T rows of
// its state columns straight into registers; x and the bf16 copy of H, which
// every wave reads whole, go through LDS.
//
// Outputs are produced transposed (Y^T = H C^T + X^T (M)^T, rows p, columns
// t), so that each lane ends with 4 consecutive channels p of one token: z is
// read and y written as 4-element vectors.  The masked C B^T tile never
// touches LDS: it is produced as B C^T (rows s, columns t), whose accumulator
// layout, after masking and decay, is the B-operand layout of the next
// product for a K index permuted the same way on the X^T side.
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

constexpr int P = 64;
constexpr int N = 128;
constexpr int THREADS = 512;     // walker: 8 waves
constexpr int NXCD = 8;
constexpr int LDB = N + 8;       // bf16 row stride of [.][n] tiles (272 B)
// Row p of a bf16 [p][s] tile is stored at row p + p / 8: with the row
// pitches below, the 8 rows 8 apart that one staging store writes then fall
// into distinct LDS banks, and 16 consecutive rows (an MFMA operand read)
// still do.
__host__ __device__ constexpr int prow(int p) { return p + (p >> 3); }

__host__ __device__ constexpr int tri(int rt) { return rt * (rt + 1) / 2; }

// Column of token s in the rows of the bf16 x tile read by the intra-chunk
// product: within each 32-token block, token 16 h + 4 j + r (h < 2, j < 4,
// r < 4) sits at 8 j + 4 h + r, so that the 8 tokens one lane needs for a
// K = 32 step (4 of each of two 16-token tiles) are one 16-byte read.
__host__ __device__ constexpr int xcol(int s) {
  return (s & ~31) | ((s & 12) << 1) | ((s & 16) >> 2) | (s & 3);
}

// element offset of M[r][k] in fragment order, for a matrix whose rows have
// KS steps of K = 32
template <int KS>
__host__ __device__ constexpr int frag_off(int r, int k) {
  return (((r >> 4) * KS + (k >> 5)) * 64 + (r & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
}

// The shape of one instance, for the chunk length Q in {64, 128, 256}.
//
// A walker owns PW of the head's P = 64 channels: all of them for Q <= 128,
// half for Q = 256 (two walkers per head), where the [p][s] tiles of a whole
// head would not fit in the CU's 160 KiB of LDS.  Each wave owns the 16
// state columns n in [16 w, 16 w + 16) of the walker's rows p, and NIT
// "items" of output: a 16-token row tile rt and NPJ of the walker's 16-channel
// tiles.  The two waves of a SIMD (w and w + 4) get row tiles whose causal
// work adds up to the same amount:
//   Q =  64: rt = w < 4 ? w : 7 - w, channel tiles {0, 1} (w < 4) or {2, 3}
//   Q = 128: rt = w < 4 ? w : 11 - w, all four channel tiles
//   Q = 256: two items, rt = w and rt = 15 - w, both channel tiles
//
// One (sequence, group, chunk) of the B|C pack, in bf16 elements.  C and the
// hi/lo parts of B^T are stored in MFMA fragment order, so that a wave reads
// the operand of one 16-row tile and one K=32 step as 1 KiB in one piece:
// fragment (tile i16, step kk) holds, for lane l, the 8 elements
// M[16 i16 + l % 16][32 kk + 8 (l / 16) + e], e < 8, at
// ((i16 * KS + kk) * 64 + l) * 8 + e, with M = C [t][n] (KS = N / 32) or
// B^T [n][s] (KS = Q / 32).
// The causal 16x16 tiles of B C^T (rows s, columns t, tile (rt, u) with
// u <= rt holding s in [16 u, 16 u + 16), t in [16 rt, 16 rt + 16)) follow
// as fp32 in accumulator order: lane l of tile k = rt (rt + 1) / 2 + u holds
// (B C^T)[16 u + 4 (l / 16) + r][16 rt + l % 16], r < 4, at floats
// (k * 64 + l) * 4 + r.  They depend on the group only, so they are formed
// there once instead of once per head.
template <int Q_>
struct Geo {
  static constexpr int Q = Q_;
  static_assert(Q == 64 || Q == 128 || Q == 256, "chunk length");
  static constexpr int PW = Q == 256 ? 32 : 64;  // channels p per walker
  static constexpr int NPS = P / PW;             // walkers per head
  static constexpr int NRT = Q / 16;             // 16-token row tiles per chunk
  static constexpr int KQ = Q / 32;              // K = 32 steps over the chunk's tokens
  static constexpr int NPT = PW / 16;            // 16-channel tiles per walker
  static constexpr int NIT = Q == 256 ? 2 : 1;   // output items per wave
  static constexpr int NPJ = Q == 64 ? 2 : NPT;  // channel tiles per item
  static constexpr int LDT = Q + 8;              // bf16 row stride of [p][s] tiles
  static constexpr int PROWS = PW + PW / 8;
  static constexpr int LDX = PW + 4;             // fp32 row stride of x [t][p]
  static constexpr int NTRI = NRT * (NRT + 1) / 2;  // causal tiles
  static constexpr int PK_C = 0;                 // C  [t][n], fragment order
  static constexpr int PK_BTH = Q * N;           // B^T [n][s] hi, fragment order
  static constexpr int PK_BTL = 2 * Q * N;       // B^T [n][s] lo, fragment order
  static constexpr int PK_CB = 3 * Q * N;        // B C^T causal tiles, fp32
  static constexpr int PACK = 3 * Q * N + 2 * NTRI * 256;
  static constexpr int PACK_TOK = 4;             // pack: tokens per thread
  static constexpr int PACK_THREADS = 16 * Q / PACK_TOK;  // PACK_TOK tokens x 8 channels each
  // x staging: thread (xv = tid % XV, xr = tid / XV) owns channels
  // [8 xv, 8 xv + 8) of tokens [RX xr, RX xr + RX)
  static constexpr int XV = PW / 8;
  static constexpr int RX = Q * PW / (THREADS * 8);
  static constexpr int DW = Q / 64;              // waves that scan the decay
  // the B^T rows of a wave are loaded at the top of the chunk when they fit
  // in registers beside the rest, else step by step in the state product
  static constexpr bool BT_EARLY = KQ <= 4;
  // likewise the C B^T tiles of an item: all at once after the staging, or
  // two per K step of the intra-chunk product
  static constexpr bool CB_EARLY = NRT <= 8;

  __device__ static int rt_of(int w, int it) {
    if (Q == 64) return w < 4 ? w : 7 - w;
    if (Q == 128) return w < 4 ? w : 11 - w;
    return it == 0 ? w : 15 - w;
  }
  __device__ static int pj_base(int w) { return Q == 64 ? 2 * (w >> 2) : 0; }
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// D = A B + C for a 16x16 tile, K = 32.  Lane l = i + 16 q holds A[i][8q..8q+7],
// B[8q..8q+7][j = l % 16] and D[4q..4q+3][j = l % 16].
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 v) {
  return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

__device__ __forceinline__ bf16x8 lds8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x8 ldg8(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// v moved across lanes by the DPP control CTRL (lanes whose source is
// outside the pattern, or outside ROW_MASK's rows, read 0)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: shifts by
// 1, 2, 4 and 8 lanes within each row of 16 (row_shr), then the last lane of
// rows 0 and 2 added to rows 1 and 3 (row_bcast:15), then the last lane of
// row 1 added to rows 2 and 3 (row_bcast:31).  The order of the additions
// is fixed for every lane.
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_or0<0x111, 0xf>(v);
  v += dpp_or0<0x112, 0xf>(v);
  v += dpp_or0<0x114, 0xf>(v);
  v += dpp_or0<0x118, 0xf>(v);
  v += dpp_or0<0x142, 0xa>(v);
  v += dpp_or0<0x143, 0xc>(v);
  return v;
}

// base + off bytes, for a wave-uniform base and a per-lane offset below
// 4 GiB: the address form of a global access with a scalar base and a 32-bit
// vector offset, in place of a 64-bit address computed per lane
template <typename T>
__device__ __forceinline__ const T* at_bytes(const T* base, uint32_t off) {
  return reinterpret_cast<const T*>(reinterpret_cast<const char*>(base) + off);
}
template <typename T>
__device__ __forceinline__ T* at_bytes(T* base, uint32_t off) {
  return reinterpret_cast<T*>(reinterpret_cast<char*>(base) + off);
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also waits for
// every outstanding global load and store of the wave (it is a fence on all
// memory); no thread here reads another thread's global writes, so waiting
// for this wave's LDS operations (lgkmcnt = 0; vmcnt and expcnt left at their
// maxima in the gfx9 s_waitcnt encoding) is enough, and global loads issued
// ahead of time stay in flight across the barrier.  The signal fences keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// hi = bf16(v), lo = bf16(v - hi)
__device__ __forceinline__ void split1(float v, bf16& hi, bf16& lo) {
  hi = (bf16)v;
  lo = (bf16)(v - (float)hi);
}
// the same for two values, the hi pair converted once and read back from
// its bits
__device__ __forceinline__ void split2(float v0, float v1, bf16x2& hi, bf16x2& lo) {
  hi = bf16x2{(bf16)v0, (bf16)v1};
  const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
  lo = bf16x2{(bf16)(v0 - __uint_as_float(hb << 16)),
              (bf16)(v1 - __uint_as_float(hb & 0xffff0000u))};
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
// HIST = false: the caller knows that no position precedes the sequence
// (tstart >= 0), so the conv history is never read.
template <typename Tx, int NR>
struct RowLoad {
  Raw8<Tx> v[NR];
  template <bool HIST = true>
  __device__ __forceinline__ void load(const ScanArgs& a, const Tx* src, int64_t stride, int col,
                                       int c0, int cdim, int b, int tstart) {
    const int L = a.seqlen, K = a.conv_k;
    const Tx* hist = static_cast<const Tx*>(a.conv_state_in);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int tau = tstart + i;
      const Tx* p = src + ((int64_t)b * L + min(max(tau, 0), L - 1)) * stride + col;
      if (HIST) {
        const bool h = (tau < 0) & (hist != nullptr) & (tau >= -(K - 1));
        p = h ? hist + ((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + c0 : p;
      }
      v[i].load(p);
    }
  }
  // The same without the history (positions before the sequence re-read
  // its first row): a wave-uniform base row rbase, at or below every
  // clamped row, and 32-bit offsets from it instead of a 64-bit address per
  // row and lane (the caller checks that Q + 3 rows of the tensor span less
  // than 4 GiB)
  __device__ __forceinline__ void load_rows(const ScanArgs& a, const Tx* src, int64_t stride,
                                            int col, int b, int tstart, int rbase) {
    const int L = a.seqlen;
    const Tx* base = src + ((int64_t)b * L + rbase) * stride;
    const uint32_t sb = (uint32_t)(stride * (int64_t)sizeof(Tx));
    const uint32_t cb = (uint32_t)(col * (int)sizeof(Tx));
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const uint32_t row = (uint32_t)(min(max(tstart + i, 0), L - 1) - rbase);
      v[i].load(at_bytes(base, row * sb + cb));
    }
  }
  // CHECK = false: the caller knows every row lies in the sequence, or feeds
  // only outputs that are discarded (a chunk that neither starts the
  // sequence nor is cut short by its end), and the per-element selects are
  // left out
  template <bool CHECK = true>
  __device__ __forceinline__ void get(const ScanArgs& a, int tstart, int i, float* out) const {
    v[i].get(out);
    if (CHECK) {
      const int tau = tstart + i;
      // bitwise, not short-circuit: a per-lane test without branches
      const bool ok = (tau < a.seqlen) &
                      ((tau >= 0) | ((a.conv_state_in != nullptr) & (tau >= -(a.conv_k - 1))));
      if (!ok) {
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = 0.f;
      }
    }
  }
};

// Depthwise conv + SiLU of R consecutive rows of 8 channels from R + 3 raw
// rows (the first 3 are the history in front); row i goes to dst + i * ld,
// zero for rows >= nvalid.  cw is the conv of the workgroup's channels in
// LDS: tap j of local channel c at cw[j * cws + c] (taps right-aligned, zero
// in front when the width is below 4), the bias at cw[4 * cws + c]; cl is the
// local channel of the first of the 8; cws is the stride between taps (the
// number of channels staged).
template <typename Tx, int R, typename Td, bool CHECK = true>
__device__ __forceinline__ void conv_rows_to(const ScanArgs& a, const RowLoad<Tx, R + 3>& rl,
                                             int tstart, const float* cw, int cws, int cl,
                                             int rfirst, int nvalid, Td* dst, int ld) {
  float o[R][8];
  // two halves of 4 channels, so that only 20 taps and a window of 12 values
  // are held at a time (each element's arithmetic is the same either way)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float w4[4][4], bv[4];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const float4 t = *reinterpret_cast<const float4*>(cw + j * cws + cl + 4 * hf);
      float* d = j < 4 ? w4[j] : bv;
      d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
    }
    float win[3][4];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      float v[8];
      rl.template get<CHECK>(a, tstart, i, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) win[i][e] = v[4 * hf + e];
    }
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float v[8];
      rl.template get<CHECK>(a, tstart, i + 3, v);
      const bool ok = !CHECK || rfirst + i < nvalid;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float cur = v[4 * hf + e];
        const float u = bv[e] + w4[0][e] * win[0][e] + w4[1][e] * win[1][e] +
                        w4[2][e] * win[2][e] + w4[3][e] * cur;
        const float sv = silu_f32(u);  // for every lane, then selected
        o[i][4 * hf + e] = ok ? sv : 0.f;
        win[0][e] = win[1][e];
        win[1][e] = win[2][e];
        win[2][e] = cur;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) put8(dst + i * ld, o[i]);
}

// Rows as they are (post-conv input), zero for rows >= nvalid.
template <typename Tx, int R, typename Td, bool CHECK = true>
__device__ __forceinline__ void copy_rows_to(const ScanArgs& a, const RowLoad<Tx, R>& rl,
                                             int tstart, int rfirst, int nvalid, Td* dst, int ld) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float o[8];
    rl.template get<CHECK>(a, tstart, i, o);
    if (CHECK && rfirst + i >= nvalid)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = 0.f;
    put8(dst + i * ld, o);
  }
}


// One activation element, kept raw between load and use
template <typename T> struct Raw1;
template <> struct Raw1<bf16> {
  unsigned short u = 0;
  __device__ __forceinline__ void load(const bf16* p) {
    u = *reinterpret_cast<const unsigned short*>(p);
  }
  __device__ __forceinline__ float get() const { return __uint_as_float((uint32_t)u << 16); }
};
template <> struct Raw1<float> {
  float f = 0.f;
  __device__ __forceinline__ void load(const float* p) { f = *p; }
  __device__ __forceinline__ float get() const { return f; }
};

// 4 consecutive elements of an activation row, kept packed between load and
// use (z in the epilogue)
template <typename T> struct Raw4;
template <> struct Raw4<bf16> {
  uint2 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xffff0000u);
  }
};
template <> struct Raw4<float> {
  float4 f;
  __device__ __forceinline__ void load(const float* p) { f = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ void get(float* v) const {
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
};

// 4 consecutive outputs of one token
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  bf16x4 r;
  r[0] = (bf16)v[0]; r[1] = (bf16)v[1]; r[2] = (bf16)v[2]; r[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = r;
}

// ------------------------------------------------------------ B|C pack

// Swizzle key of row n of the pack's [n][s] B^T staging tile (Q / 8 blocks
// of 16 bytes per row): distinct across the rows 8 apart that 16 lanes write
// at once, and across 16 consecutive rows, which 16 lanes read at once.
template <int Q>
__device__ __forceinline__ int bt_key(int n) {
  return ((n >> 3) ^ ((n & 7) << 1)) & (Q / 8 - 1);
}


// One workgroup of 4 Q threads per (chunk c, group g, sequence b).  Thread
// (cv = tid % 16, rg = tid / 16) owns channels [8 cv, 8 cv + 8) and tokens
// [4 rg, 4 rg + 4) of the chunk for B and for C.  Tokens past the end of the
// sequence are written as zeros.  With the conv, the workgroup of the last
// chunk also hands the last K-1 raw B and C rows of the group over to
// conv_state_out.
template <typename Tin, bool CONV, int Q>
__global__ __launch_bounds__(Geo<Q>::PACK_THREADS) void bc_pack_kernel(ScanArgs a, bf16* pack) {
  using G_ = Geo<Q>;
  constexpr int PACK_THREADS = G_::PACK_THREADS, PACK = G_::PACK, NTRI = G_::NTRI;
  constexpr int KQ = G_::KQ, PT = G_::PACK_TOK;
  __shared__ __attribute__((aligned(16))) float sCw[CONV ? 5 * 2 * N : 4];
  __shared__ __attribute__((aligned(16))) bf16 sPB[Q * LDB];  // B [s][n] bf16
  __shared__ __attribute__((aligned(16))) bf16 sPC[Q * LDB];  // C [t][n] bf16
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int L = a.seqlen, nc = (L + Q - 1) / Q, G = a.ngroups;
  const int t0 = c * Q, Lc = min(Q, L - t0);
  const int tid = threadIdx.x, cv = tid & 15, rg = tid >> 4;
  const int HP = a.nheads * P, GN = G * N, cdim = HP + 2 * GN;
  bf16* pk = pack + ((int64_t)(b * G + g) * nc + c) * PACK;
  constexpr int HALO = CONV ? 3 : 0;

  // bf16 inputs: the raw B and C rows first, so that their loads are in
  // flight while the taps are read and staged (about 0.5% of the prefill
  // call); fp32 rows are loaded one tensor at a time, since holding both
  // would cost the kernel half its occupancy
  constexpr bool EARLY = sizeof(Tin) == 2;
  const int tstart = t0 + PT * rg - HALO;
  RowLoad<Tin, PT + HALO> rlm[2];
  auto load_rows = [&](int m) {
    const Tin* src = static_cast<const Tin*>(m == 0 ? a.Bm : a.Cm);
    const int64_t stride = m == 0 ? a.b_stride : a.c_stride;
    const int hcol = HP + m * GN + g * N + 8 * cv;  // channel in the conv state rows
    rlm[m].load(a, src, stride, g * N + 8 * cv, hcol, cdim, b, tstart);
  };
  if constexpr (EARLY) {
    load_rows(0);
    load_rows(1);
  }

  if constexpr (CONV) {
    // taps of the group's B channels (local 0..N-1) and C channels (N..2N-1)
    const int K = a.conv_k;
    for (int i = tid; i < 2 * N; i += PACK_THREADS) {
      const int ch = i < N ? HP + g * N + i : HP + GN + g * N + (i - N);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = j - (4 - K);
        sCw[j * 2 * N + i] = k >= 0 ? a.conv_w[(int64_t)ch * K + k] : 0.f;
      }
      sCw[4 * 2 * N + i] = a.conv_b ? a.conv_b[ch] : 0.f;
    }
    lds_barrier();
  }

  // C first, then B, whose values stay in v for the B^T parts
  float v[PT][8];
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const int m = 1 - mm;  // m = 0: B, m = 1: C
    if constexpr (!EARLY) load_rows(m);
    const RowLoad<Tin, PT + HALO>& rl = rlm[m];
    if constexpr (CONV)
      conv_rows_to<Tin, PT>(a, rl, tstart, sCw, 2 * N, m * N + 8 * cv, PT * rg, Lc, &v[0][0], 8);
    else
      copy_rows_to<Tin, PT>(a, rl, tstart, PT * rg, Lc, &v[0][0], 8);
    // bf16 rows [t][n] into LDS (the 8 channels 8 cv .. 8 cv + 7 of a row
    // are 8 consecutive elements)
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      bf16x8 r;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (bf16)v[i][e];
      *reinterpret_cast<bf16x8*>((m == 0 ? sPB : sPC) + (PT * rg + i) * LDB + 8 * cv) = r;
    }
  }
  lds_barrier();

  // Every part of the pack leaves through LDS, so that each wave writes whole
  // 1 KiB fragments (16 bytes per lane, consecutive lanes consecutive in
  // memory) rather than 16-byte pieces scattered over many lines.
  const int pw = tid >> 6, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  constexpr int NW = PACK_THREADS / 64;
  // causal tiles of B C^T (rows s, columns t) with fp32 accumulation, in the
  // accumulator order the walkers use; NTRI / NW tiles per wave (5, 9 or 17)
  {
    float* cbo = reinterpret_cast<float*>(pk + G_::PK_CB);
    for (int k = pw; k < NTRI; k += NW) {
      int rt = 0;
      while (tri(rt + 1) <= k) ++rt;
      const int u = k - tri(rt);
      const bf16* brow = sPB + (16 * u + l16) * LDB + 8 * q;
      const bf16* crow = sPC + (16 * rt + l16) * LDB + 8 * q;
      f32x4 acc = {};
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk)
        acc = mfma(lds8(brow + 32 * kk), lds8(crow + 32 * kk), acc);
      *reinterpret_cast<f32x4*>(cbo + (k * 64 + lane) * 4) = acc;
    }
  }
  // C in fragment order: fragment f = (t tile i16, K step kk) takes lane l's
  // 8 channels 32 kk + 8 q .. of token 16 i16 + l % 16
  for (int f = pw; f < (Q / 16) * (N / 32); f += NW) {
    const int i16 = f / (N / 32), kk = f % (N / 32);
    *reinterpret_cast<bf16x8*>(pk + G_::PK_C + (f * 64 + lane) * 8) =
        lds8(sPC + (16 * i16 + l16) * LDB + 32 * kk + 8 * q);
  }
  lds_barrier();

  // B^T hi and lo, [n][s], into the two tiles just read: row n holds Q
  // tokens with no padding, its 16-byte block cb (tokens 8 cb .. 8 cb + 7)
  // at block cb ^ bt_key(n), which keeps both the writes below (rows 8 apart
  // across lanes) and the fragment reads after (16 consecutive rows) clear
  // of bank conflicts
  static_assert(N * Q <= Q * LDB, "the B^T staging tile fits in the [t][n] tiles");
  bf16* sBTh = sPB;
  bf16* sBTl = sPC;
  static_assert(PT == 4, "B^T staging writes 4 tokens (half a 16-byte block) per row");
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      bf16 hh, ll;
      split1(v[i][e], hh, ll);
      hi[i] = hh;
      lo[i] = ll;
    }
    // tokens 4 rg .. 4 rg + 3: half (rg % 2) of 16-byte block rg / 2
    const int n = 8 * cv + e;
    const int o = n * Q + 8 * ((rg >> 1) ^ bt_key<Q>(n)) + 4 * (rg & 1);
    *reinterpret_cast<bf16x4*>(sBTh + o) = hi;
    *reinterpret_cast<bf16x4*>(sBTl + o) = lo;
  }
  lds_barrier();
  // fragment f = (n tile i16, K step kk): lane l's 8 tokens 32 kk + 8 q .. of
  // channel 16 i16 + l % 16
  for (int f = pw; f < 8 * KQ; f += NW) {
    const int i16 = f / KQ, kk = f % KQ;
    const int n = 16 * i16 + l16;
    const int o = n * Q + 8 * ((4 * kk + q) ^ bt_key<Q>(n));
    *reinterpret_cast<bf16x8*>(pk + G_::PK_BTH + (f * 64 + lane) * 8) = lds8(sBTh + o);
    *reinterpret_cast<bf16x8*>(pk + G_::PK_BTL + (f * 64 + lane) * 8) = lds8(sBTl + o);
  }

  // conv history hand-over of the group's B and C channels
  if (CONV && c == nc - 1 && a.conv_state_out != nullptr) {
    const int K = a.conv_k;
    Tin* out = static_cast<Tin*>(a.conv_state_out);
    const Tin* hin = static_cast<const Tin*>(a.conv_state_in);
    for (int i = tid; i < (K - 1) * 2 * N; i += PACK_THREADS) {
      const int j = i / (2 * N), cl = i % (2 * N);
      const int m = cl / N, n = cl % N;
      const int ch = HP + m * GN + g * N + n;
      const int tau = L - (K - 1) + j;  // < L
      Tin v = from_f32<Tin>(0.f);
      if (tau >= 0) {
        const Tin* src = static_cast<const Tin*>(m == 0 ? a.Bm : a.Cm);
        v = src[((int64_t)b * L + tau) * (m == 0 ? a.b_stride : a.c_stride) + g * N + n];
      } else if (hin != nullptr) {
        v = hin[((int64_t)b * (K - 1) + (K - 1) + tau) * cdim + ch];
      }
      out[((int64_t)b * (K - 1) + j) * cdim + ch] = v;
    }
  }
}

// ------------------------------------------------------------ x staging

// One chunk's x for the whole workgroup: thread (xv = tid % XV,
// xr = tid / XV) owns tokens [RX xr, RX xr + RX) x channels [8 xv, 8 xv + 8)
// of the walker's channels from p0 (raw values of type Tx with 3 rows of
// history in front when XCONV, post-conv otherwise).
template <typename Tx, bool XCONV, int Q>
struct StageX {
  using G_ = Geo<Q>;
  static constexpr int HX = XCONV ? 3 : 0, RX = G_::RX, XV = G_::XV;
  RowLoad<Tx, RX + HX> rx;

  template <bool HIST>
  __device__ __forceinline__ void load(const ScanArgs& a, int b, int h, int p0, int t0) {
    const int tid = threadIdx.x;
    const int xv = tid % XV, xr = tid / XV;
    const int cdim = a.nheads * P + 2 * a.ngroups * N;
    const int ch = h * P + p0 + 8 * xv;
    if constexpr (HIST)
      rx.template load<true>(a, static_cast<const Tx*>(a.x), a.x_stride, ch, ch, cdim, b,
                             t0 + RX * xr - HX);
    else  // (the rows before the sequence of a repeated first chunk: row 0)
      rx.load_rows(a, static_cast<const Tx*>(a.x), a.x_stride, ch, b, t0 + RX * xr - HX,
                   max(t0 - HX, 0));
  }

  // the thread's RX x 8 post-conv values, tmp[8 i + e] = x[RX xr + i][8 xv + e]
  // (zero past the end of the sequence)
  template <bool CHECK>
  __device__ __forceinline__ void compute(const ScanArgs& a, const float* cw, int t0, int Lc,
                                          float* tmp) const {
    const int tid = threadIdx.x;
    const int xv = tid % XV, xr = tid / XV;
    if constexpr (XCONV)
      conv_rows_to<Tx, RX, float, CHECK>(a, rx, t0 + RX * xr - 3, cw, G_::PW, 8 * xv, RX * xr, Lc,
                                         tmp, 8);
    else
      copy_rows_to<Tx, RX, float, CHECK>(a, rx, t0 + RX * xr, RX * xr, Lc, tmp, 8);
  }
};

// Walker index of this workgroup: (sequence b, head h, segment seg, channel
// slice ps), with the walkers of one (b, group, segment) contiguous and dealt
// to one XCD.
struct Walker {
  int b, h, seg, ps;
};
__device__ __forceinline__ Walker walker_of(int lin, int total, int H, int G, int nsegs,
                                            int nps) {
  // item order: (((b * nsegs + seg) * G + g) * hpg + hh) * nps + ps; lin ->
  // item puts item ranges of length total/8 on one XCD (lin % 8)
  const int per = total / NXCD;
  int item = lin;
  if (lin < per * NXCD) item = (lin % NXCD) * per + lin / NXCD;
  const int ps = item % nps;
  item /= nps;
  const int hpg = H / G;
  const int hh = item % hpg;
  int rest = item / hpg;
  const int g = rest % G;
  rest /= G;
  const int seg = rest % nsegs;
  const int b = rest / nsegs;
  return Walker{b, g * hpg + hh, seg, ps};
}

template <typename Tx, typename Ta, typename Ty, bool XCONV, bool STATE_ONLY, int Q>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(STATE_ONLY ? 4 : 1))) void scan_bf16_kernel(ScanArgs a) {
  using G_ = Geo<Q>;
  constexpr int PW = G_::PW, NRT = G_::NRT, KQ = G_::KQ, NPT = G_::NPT, NIT = G_::NIT;
  constexpr int NPJ = G_::NPJ, LDT = G_::LDT, PROWS = G_::PROWS, LDX = G_::LDX;
  constexpr int RX = G_::RX, XV = G_::XV, DW = G_::DW;
  constexpr bool OUT = !STATE_ONLY;
  // (the state-only walker runs four waves per SIMD, in 128 registers, and
  // loads its B^T rows step by step)
  constexpr bool BT_EARLY = G_::BT_EARLY && OUT;
  __shared__ __attribute__((aligned(16))) bf16 sXh[OUT ? PROWS * LDT : 8];  // x hi [p][s]
  __shared__ __attribute__((aligned(16))) bf16 sXWh[PROWS * LDT];            // (x o w) hi
  __shared__ __attribute__((aligned(16))) bf16 sXWl[PROWS * LDT];            // (x o w) lo
  __shared__ __attribute__((aligned(16))) float sX32[OUT ? Q * LDX : 4];  // x [t][p]
  __shared__ __attribute__((aligned(16))) bf16 sH[OUT ? PW * LDB : 8];    // H [p][n]
  // the decay of a chunk, in two buffers (chunk c in buffer c % 2): the next
  // chunk's is computed while the current one is in use
  __shared__ __attribute__((aligned(16))) float sLam[2 * Q];
  __shared__ __attribute__((aligned(16))) float sDel[2 * Q];
  // exp(Lam_r - Lam_s) delta_s, r the last token of s's 16-token tile
  __shared__ __attribute__((aligned(16))) float sE[OUT ? 2 * Q : 4];
  __shared__ float sRed[2 * DW];  // each decay wave's total, per buffer
  __shared__ __attribute__((aligned(16))) float sCw[XCONV ? 5 * PW : 4];  // x-channel conv

  const int H = a.nheads, G = a.ngroups, L = a.seqlen;
  // pass 1 (state-only) walks segments 0..nseg-2, pass 2 all segments
  const int nsegs = STATE_ONLY ? a.nseg - 1 : a.nseg;
  const Walker wk = walker_of(blockIdx.x, gridDim.x, H, G, nsegs, G_::NPS);
  const int b = wk.b, h = wk.h, seg = wk.seg;
  const int p0 = wk.ps * PW;  // the walker's first channel of the head
  const int bh = b * H + h;
  const int hpg = H / G, g = h / hpg;
  const int HP = H * P, GN = G * N, cdim = HP + 2 * GN;
  const int nc = (L + Q - 1) / Q;
  const int cbeg = seg * a.seg_chunks;
  const int cend = min(nc, cbeg + a.seg_chunks);
  const bf16* pack = static_cast<const bf16*>(a.bc_pack) + (int64_t)(b * G + g) * nc * G_::PACK;

  const int tid = threadIdx.x;
  // the wave index is uniform over the wave: held in a scalar register, the
  // branches on it below are scalar branches, not lane masks
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l16 = lane & 15, q = lane >> 4;
  const int pjb = G_::pj_base(w);      // first channel tile of the wave's items
  const int xv = tid % XV, xr = tid / XV;  // x staging: channels 8 xv.., tokens RX xr..
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.f;
  const float dtb = a.dt_bias ? a.dt_bias[h] : 0.f;
  const Tx* xg = static_cast<const Tx*>(a.x);

  // ---- incoming state.  The state is accumulated transposed, as H^T [n][p]:
  //      element r of hacc[pt] is (n = 16 w + 4 q + r, p = p0 + 16 pt + l16),
  //      so that each lane holds 4 consecutive n of one row p of H [p][n].
  const float* h_in = nullptr;
  if (OUT) {
    if (a.nseg > 1)
      h_in = a.seg_state + ((int64_t)bh * a.nseg + seg) * P * N;
    else
      h_in = a.initial_state ? a.initial_state + (int64_t)bh * P * N : nullptr;
  }
  const int hoff = 16 * w + 4 * q;  // the lane's first n in a row of H
  f32x4 hacc[NPT];
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt) {
    const int p = 16 * pt + l16;
    hacc[pt] = h_in ? *reinterpret_cast<const f32x4*>(h_in + (p0 + p) * N + hoff) : f32x4{};
    if (OUT) *reinterpret_cast<bf16x4*>(sH + p * LDB + hoff) = to_bf16x4(hacc[pt]);
  }
  float log_decay = 0.f;  // sum of delta*A over the segment (state-only pass)
  if (XCONV && tid < PW) {
    // the conv of this walker's x channels: read at every chunk from LDS (the
    // first read follows the barrier at the top of the chunk loop)
    const int K = a.conv_k;
    const int64_t ch = (int64_t)h * P + p0 + tid;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = j - (4 - K);
      sCw[j * PW + tid] = k >= 0 ? a.conv_w[ch * K + k] : 0.f;
    }
    sCw[4 * PW + tid] = a.conv_b ? a.conv_b[ch] : 0.f;
  }

  // Two barriers per chunk.  After the first: the bf16 copy of the state,
  // the conv of x and its staging, and the split of x o w (the chunk's decay
  // is already in LDS).  After the second: the state product, the read-out,
  // the intra-chunk product and the epilogue, and then waves 0 .. DW-1
  // compute the next chunk's decay.  Chunk c+1's x and dt are loaded as soon
  // as chunk c is staged, so they are in flight while chunk c is computed.
  // The per-wave operands (B^T rows, C rows, C B^T tiles) and z are loaded
  // within their own chunk, ahead of their first use.
  StageX<Tx, XCONV, Q> sx;
  // the prefetched dt stays in its raw form until it is used, so that no
  // conversion waits for the load while the prefetch is in flight
  Raw1<Ta> dtv;
  // (HIST: whether the chunk may be the first, whose conv reads the history)
  auto prefetch = [&](int cc, auto hist) {
    const int tt0 = cc * Q;
    sx.template load<decltype(hist)::value>(a, b, h, p0, tt0);
    // every lane loads (threads tid >= Q all re-read the chunk's first token,
    // one cache line, and never use it), so no branch separates these loads
    // from the ones after
    dtv.load(static_cast<const Ta*>(a.dt) +
             ((int64_t)b * L + min(tt0 + (tid < Q ? tid : 0), L - 1)) * a.dt_stride + h);
  };
  // delta, the cumulative log decay and the tile decays of chunk cc into
  // buffer cc % 2, by waves 0 .. DW-1 (one token per lane) from the dt in dtv
  auto delta_step = [&](int cc) {
    const int Lcc = min(Q, L - cc * Q);
    const int buf = (cc & 1) * Q;
    float d = dtv.get() + dtb;
    if (a.dt_softplus) d = softplus_f32(d);
    if (tid >= Lcc) d = 0.f;
    sDel[buf + tid] = d;
    // inclusive prefix sum of delta A over the wave's 64 tokens (fixed
    // order); the values of a later wave lack the totals of the waves before
    // it, which the readers add (lam() below)
    const float v = wave_prefix_sum(d * Ah);
    sLam[buf + tid] = v;
    if (lane == 63) sRed[(cc & 1) * DW + w] = v;
    // the tile's last token is in the same wave, so the difference needs
    // no carry; it is <= 0 (the decay only shrinks)
    const float vr = __shfl(v, lane | 15, 64);
    if (OUT) sE[buf + tid] = __expf(vr - v) * d;
  };
  if (cbeg < cend) {
    prefetch(cbeg, std::true_type{});
    if (w < DW) delta_step(cbeg);  // visible past the first barrier of the loop
  }

  for (int c = cbeg; c < cend; ++c) {
    const int t0 = c * Q;
    const int Lc = min(Q, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;
    const bf16* pk = pack + (int64_t)c * G_::PACK;
    // the items' row tiles, re-read at every chunk through an empty asm
    // statement: the compiler then evaluates the scalar tests on them where
    // they are used instead of hoisting them out of the loop as lane masks,
    // which exhausts the scalar registers
    int rtc[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      rtc[it] = G_::rt_of(w, it);
      asm volatile("" : "+s"(rtc[it]));
    }

    // this wave's B^T rows of its state columns (bth/btl, A operand
    // [i = n][k = s]) now when they fit in registers; C rows of its tokens
    // (cf, [k = n][j = t]) and z after the staging
    bf16x8 cf[4], bth[BT_EARLY ? KQ : 1], btl[BT_EARLY ? KQ : 1];
    auto bt_off = [&](int kk) { return (uint32_t)(((w * KQ + kk) * 64 + lane) * 8) * 2; };
    if constexpr (BT_EARLY) {
#pragma unroll
      for (int kk = 0; kk < KQ; ++kk) {
        bth[kk] = ldg8(at_bytes(pk + G_::PK_BTH, bt_off(kk)));
        btl[kk] = ldg8(at_bytes(pk + G_::PK_BTL, bt_off(kk)));
      }
    }

    lds_barrier();  // the previous chunk is done with every LDS buffer
    if (OUT && c > cbeg) {
      // the bf16 copy of the state for this chunk's read-out (the previous
      // chunk's read-out of the older state is complete past the barrier)
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt)
        *reinterpret_cast<bf16x4*>(sH + (16 * pt + l16) * LDB + hoff) = to_bf16x4(hacc[pt]);
    }
    // this chunk's decay (computed during the previous chunk, or before the
    // loop): Lam_s, the cumulative log decay of the chunk up to token s,
    // is the scanning wave's value plus the totals of the waves before it
    // (added in a fixed order)
    const float* cLam = sLam + (c & 1) * Q;
    const float* cDel = sDel + (c & 1) * Q;
    const float* cE = sE + (OUT ? (c & 1) * Q : 0);
    float pre[DW];  // pre[k]: the carry into the tokens of wave k
    pre[0] = 0.f;
#pragma unroll
    for (int k = 1; k < DW; ++k) pre[k] = pre[k - 1] + sRed[(c & 1) * DW + k - 1];
    auto carry_at = [&](int s) {
      if constexpr (DW == 1) return 0.f;
      else if constexpr (DW == 2) return s >= 64 ? pre[1] : 0.f;
      else return s >= 128 ? (s >= 192 ? pre[3] : pre[2]) : (s >= 64 ? pre[1] : 0.f);
    };
    auto lam = [&](int s) { return cLam[s] + carry_at(s); };
    // the decay to the chunk's last token: token Lc - 1, not Q - 1 -- past
    // the end the increments are 0, but they are summed in another order, so
    // the two can differ by an ulp, which is large when |Lam| is
    const float lam_last = lam(Lc - 1);
    if (STATE_ONLY) log_decay += lam_last;

    float xt[8 * RX];  // xt[8 i + e] = x[RX xr + i][8 xv + e], post-conv fp32
    // the selects for rows outside the sequence and tokens past its end only
    // where they can occur: its first chunk and a last chunk cut short
    // (a uniform test)
    if (c == 0 || Lc < Q)
      sx.template compute<true>(a, sCw, t0, Lc, xt);
    else
      sx.template compute<false>(a, sCw, t0, Lc, xt);
    if (OUT) {
#pragma unroll
      for (int i = 0; i < RX; ++i) {
        float* d = sX32 + (RX * xr + i) * LDX + 8 * xv;
        *reinterpret_cast<float4*>(d) = make_float4(xt[8 * i], xt[8 * i + 1], xt[8 * i + 2],
                                                    xt[8 * i + 3]);
        *reinterpret_cast<float4*>(d + 4) = make_float4(xt[8 * i + 4], xt[8 * i + 5],
                                                        xt[8 * i + 6], xt[8 * i + 7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16* d = sXh + prow(8 * xv + e) * LDT + xcol(RX * xr);
        if constexpr (RX == 2) {
          bf16x2 v2;
          v2[0] = (bf16)xt[e];
          v2[1] = (bf16)xt[8 + e];
          *reinterpret_cast<bf16x2*>(d) = v2;
        } else {
          *d = (bf16)xt[e];
        }
      }
    }

    // ---- (x o w) split into bf16 hi + lo, [p][s], once per workgroup, with
    //      w_s = exp(Lam_last - Lam_s) delta_s of the thread's tokens
    {
      float wt[RX];
#pragma unroll
      for (int i = 0; i < RX; ++i)
        wt[i] = __expf(lam_last - lam(RX * xr + i)) * cDel[RX * xr + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int o = prow(8 * xv + e) * LDT + RX * xr;
        if constexpr (RX == 2) {
          bf16x2 hi, lo;
          split2(xt[e] * wt[0], xt[8 + e] * wt[1], hi, lo);
          *reinterpret_cast<bf16x2*>(sXWh + o) = hi;
          *reinterpret_cast<bf16x2*>(sXWl + o) = lo;
        } else {
          bf16 hh, ll;
          split1(xt[e] * wt[0], hh, ll);
          sXWh[o] = hh;
          sXWl[o] = ll;
        }
      }
    }

    // The loads of this chunk's per-wave operands are spread over the
    // chunk (all waves issue theirs at the same time, and they share the
    // CU's load path): the next chunk's x and dt now, the C rows and C B^T
    // tiles after the staging barrier, z after the state product.
    Raw4<Ta> zr[NPJ];
    // B C^T tiles u <= rt of the item's tokens (u > rt: unused)
    f32x4 cbt[G_::CB_EARLY ? NRT : 1];
    // this lane's part of tile u of row tile rt
    auto cb_src = [&](int rt, int u) {
      return at_bytes(reinterpret_cast<const float*>(pk + G_::PK_CB) + (tri(rt) + u) * 256,
                      (uint32_t)lane * 16);
    };
    // C rows of item it's tokens and its C B^T tiles
    auto load_item = [&](int it) {
      const int rt = rtc[it];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        cf[kk] = ldg8(at_bytes(pk + G_::PK_C, (uint32_t)(((rt * 4 + kk) * 64 + lane) * 8) * 2));
      // tiles past rt are not loaded (wave-uniform branches; the loads
      // after these still retire after them)
      if constexpr (G_::CB_EARLY) {
#pragma unroll
        for (int u = 0; u < NRT; ++u)
          if (u <= rt) cbt[u] = *reinterpret_cast<const f32x4*>(cb_src(rt, u));
      }
    };
    // unconditional (the last chunk re-reads itself), so that no branch
    // separates these loads from the ones after
    // (chunk c + 1 >= 1 reads no history; at the last chunk the loads repeat
    // it and go unused)
    prefetch(min(c + 1, cend - 1), std::false_type{});
    lds_barrier();  // x, its bf16 copy and (x o w) are complete
    if (OUT) load_item(0);
    // ---- state: H^T <- exp(Lam_last) H^T + B^T (X o w), operands split
    //      hi + lo; this wave's rows n of H^T, all the walker's columns p.
    //      The read-out below still uses the previous state through its
    //      bf16 copy in sH, which is replaced at the start of the next chunk.
    const float gamma = __expf(lam_last);
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) hacc[pt] *= gamma;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      bf16x8 bh_k, bl_k;
      if constexpr (BT_EARLY) {
        bh_k = bth[kk];
        bl_k = btl[kk];
      } else {
        bh_k = ldg8(at_bytes(pk + G_::PK_BTH, bt_off(kk)));
        bl_k = ldg8(at_bytes(pk + G_::PK_BTL, bt_off(kk)));
      }
      bf16x8 xhi[NPT], xlo[NPT];
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const int o = prow(16 * pt + l16) * LDT + 32 * kk + 8 * q;
        xhi[pt] = lds8(sXWh + o);
        xlo[pt] = lds8(sXWl + o);
      }
      // the accumulators in turn, so that no product waits for the one
      // before it
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) hacc[pt] = mfma(bh_k, xhi[pt], hacc[pt]);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) hacc[pt] = mfma(bl_k, xhi[pt], hacc[pt]);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) hacc[pt] = mfma(bh_k, xlo[pt], hacc[pt]);
      // keep the operand loads of the next K step below this one's products
      // (hoisting them all at once costs more registers than the wave has)
      __builtin_amdgcn_sched_barrier(0);
    }

#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (!OUT) break;
      const int rt = rtc[it];
      const int tcol = 16 * rt + l16;  // output token of this lane
      if (it > 0) load_item(it);
      // z of token tcol, channels p0 + 16 (pjb + pj) + 4 q .. (tokens past the
      // end re-read the last one and are never stored); without a gate the
      // loads read the start of the B|C pack instead (at least 58 KiB of
      // global memory; the values are not used): no branch, and both
      // pointers stay global so the loads are not flat
      const Ta* zrow = a.z != nullptr
                           ? static_cast<const Ta*>(a.z) +
                                 (row0 + min(tcol, Lc - 1)) * a.z_stride + h * P + p0 +
                                 16 * pjb + 4 * q
                           : static_cast<const Ta*>(a.bc_pack) + 4 * q;
#pragma unroll
      for (int pj = 0; pj < NPJ; ++pj) zr[pj].load(zrow + 16 * pj);

      // ---- inter-chunk read-out, transposed: Y^T = H C^T scaled by exp(Lam_t);
      //      element r of yacc[pj] is (p = p0 + 16 (pjb + pj) + 4 q + r, t = tcol)
      f32x4 yacc[NPJ] = {};
#pragma unroll
      for (int kk = 0; kk < N / 32; ++kk)
#pragma unroll
        for (int pj = 0; pj < NPJ; ++pj)
          yacc[pj] = mfma(lds8(sH + (16 * (pjb + pj) + l16) * LDB + 32 * kk + 8 * q), cf[kk],
                          yacc[pj]);
      const float lam_t = lam(tcol);
      {
        const float e = __expf(lam_t);
#pragma unroll
        for (int pj = 0; pj < NPJ; ++pj) yacc[pj] *= e;
      }

      // ---- intra-chunk: Y^T += X^T (C B^T o decay mask)^T over the source
      //      tiles u <= rt, two 16-token tiles per K=32 step
#pragma unroll
      for (int u0 = 0; u0 < NRT; u0 += 2) {
        if (u0 > rt) break;
        // the step's x operands first, so that their LDS latency is hidden
        // behind the mask arithmetic
        // (u0 is even: the step's 32 tokens are one block of the x tile)
        bf16x8 xf[NPJ];
#pragma unroll
        for (int pj = 0; pj < NPJ; ++pj)
          xf[pj] = lds8(sXh + prow(16 * (pjb + pj) + l16) * LDT + 16 * u0 + 8 * q);
        f32x4 cbp[2];  // the step's two tiles, when they are loaded step by step
        if constexpr (!G_::CB_EARLY) {
#pragma unroll
          for (int half = 0; half < 2; ++half)
            if (u0 + half <= rt) cbp[half] = *reinterpret_cast<const f32x4*>(cb_src(rt, u0 + half));
        }
        bf16x8 mf;  // element 4 half + r: M[t = tcol][s = 16 (u0 + half) + 4 q + r]
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int u = u0 + half;
          if (u > rt) {  // past the diagonal tile (rt even): a zero K half
#pragma unroll
            for (int r = 0; r < 4; ++r) mf[4 * half + r] = (bf16)0.f;
            continue;
          }
          const f32x4 cb = G_::CB_EARLY ? cbt[u] : cbp[half];
          // cb[r] = (B C^T)[s = 16 u + 4 q + r][t = tcol]
          const int s0 = 16 * u + 4 * q;
          if (u < rt) {
            // below the diagonal every s precedes every t: the decay
            // exp(Lam_t - Lam_s) factors through the tile's last token r as
            // exp(Lam_t - Lam_r) exp(Lam_r - Lam_s), both factors <= 1
            const float f = __expf(lam_t - lam(16 * u + 15));
            const float4 e4 = *reinterpret_cast<const float4*>(cE + s0);
            mf[4 * half + 0] = (bf16)(cb[0] * f * e4.x);
            mf[4 * half + 1] = (bf16)(cb[1] * f * e4.y);
            mf[4 * half + 2] = (bf16)(cb[2] * f * e4.z);
            mf[4 * half + 3] = (bf16)(cb[3] * f * e4.w);
          } else {
            const float4 l4 = *reinterpret_cast<const float4*>(cLam + s0);
            const float4 d4 = *reinterpret_cast<const float4*>(cDel + s0);
            const float cs = carry_at(16 * u);  // the 4 tokens share a wave
            const float ls[4] = {l4.x + cs, l4.y + cs, l4.z + cs, l4.w + cs};
            const float ds[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // computed for every lane and then selected (no lane branch);
              // above the diagonal the exponent is positive and discarded.
              // In the diagonal tile s <= t is 4 q + r <= l16.
              const float m = cb[r] * __expf(lam_t - ls[r]) * ds[r];
              mf[4 * half + r] = (bf16)(4 * q + r <= l16 ? m : 0.f);
            }
          }
        }
#pragma unroll
        for (int pj = 0; pj < NPJ; ++pj) yacc[pj] = mfma(xf[pj], mf, yacc[pj]);
      }

      // ---- epilogue: skip, gate, store 4 consecutive channels per pj
      if (tcol < Lc) {
        Ty* yrow = static_cast<Ty*>(a.y) + (row0 + tcol) * a.y_stride + h * P + p0 + 16 * pjb +
                   4 * q;
        const float* xrow = sX32 + tcol * LDX + 16 * pjb + 4 * q;
        // one straight-line copy per case of the (uniform) gate test, so
        // that the exponentials of all the outputs can be in flight together
        auto emit = [&](auto gated) {
#pragma unroll
          for (int pj = 0; pj < NPJ; ++pj) {
            const float4 x4 = *reinterpret_cast<const float4*>(xrow + 16 * pj);
            const float xs[4] = {x4.x, x4.y, x4.z, x4.w};
            float zs[4];
            if constexpr (decltype(gated)::value) zr[pj].get(zs);
            float yv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              yv[r] = yacc[pj][r] + Dh * xs[r];
              if constexpr (decltype(gated)::value) yv[r] *= silu_f32(zs[r]);
            }
            store4(yrow + 16 * pj, yv);
          }
        };
        if (a.z != nullptr)
          emit(std::true_type{});
        else
          emit(std::false_type{});
      }
    }

    // ---- the next chunk's decay, by waves 0 .. DW-1 (at Q = 128 the two
    //      with the least intra-chunk work), into the other buffer: read past
    //      the next chunk's first barrier, while this chunk's buffer is still
    //      in use
    if (w < DW && c + 1 < cend) delta_step(c + 1);
  }

  // ---- outgoing state
  float* h_out = nullptr;
  if (STATE_ONLY)
    h_out = a.seg_state + ((int64_t)bh * a.nseg + seg + 1) * P * N;
  else if (seg == a.nseg - 1)
    h_out = a.final_state ? a.final_state + (int64_t)bh * P * N : nullptr;
  if (h_out != nullptr) {
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
      *reinterpret_cast<f32x4*>(h_out + (p0 + 16 * pt + l16) * N + hoff) = hacc[pt];
  }
  // (the channel slices of a head compute the same log decay; the first writes it)
  if (STATE_ONLY && tid == 0 && p0 == 0) a.seg_logdecay[(int64_t)bh * a.nseg + seg] = log_decay;

  // ---- conv history hand-over of this walker's x channels (last segment;
  //      the B and C channels are handed over by the pack kernel)
  if (XCONV && OUT && seg == a.nseg - 1 && a.conv_state_out != nullptr) {
    const int K = a.conv_k;
    Tx* out = static_cast<Tx*>(a.conv_state_out);
    const Tx* hin = static_cast<const Tx*>(a.conv_state_in);
    for (int i = tid; i < (K - 1) * PW; i += THREADS) {
      const int j = i / PW, c = h * P + p0 + i % PW;
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
// slot k holds H_loc[k-1] on entry and H_in[k] on exit.  The recurrence is
// independent per state element: workgroup (bh, part) takes 4 consecutive
// elements per thread (COMBINE_THREADS * 4 of the head's P*N), and loads
// the slots of COMBINE_BATCH segments at a time, ahead of the dependent
// multiply-adds, so that their latencies overlap.
constexpr int COMBINE_THREADS = 256;
constexpr int COMBINE_PARTS = P * N / (COMBINE_THREADS * 4);
constexpr int COMBINE_BATCH = 8;
__global__ __launch_bounds__(COMBINE_THREADS) void combine_segments_kernel(ScanArgs a) {
  const int bh = blockIdx.x, part = blockIdx.y;
  const int64_t i = (int64_t)4 * (part * COMBINE_THREADS + threadIdx.x);
  f32x4* slots = reinterpret_cast<f32x4*>(a.seg_state + (int64_t)bh * a.nseg * P * N + i);
  constexpr int64_t SLOT = P * N / 4;  // slot stride in f32x4
  const float* ld = a.seg_logdecay + (int64_t)bh * a.nseg;
  f32x4 carry = {0.f, 0.f, 0.f, 0.f};
  if (a.initial_state)
    carry = *reinterpret_cast<const f32x4*>(a.initial_state + (int64_t)bh * P * N + i);
  slots[0] = carry;
  for (int k0 = 1; k0 < a.nseg; k0 += COMBINE_BATCH) {
    const int nb = min(COMBINE_BATCH, a.nseg - k0);
    f32x4 loc[COMBINE_BATCH];
#pragma unroll
    for (int j = 0; j < COMBINE_BATCH; ++j)
      if (j < nb) loc[j] = slots[(k0 + j) * SLOT];
#pragma unroll
    for (int j = 0; j < COMBINE_BATCH; ++j) {
      if (j < nb) {
        carry = __expf(ld[k0 + j - 1]) * carry + loc[j];
        slots[(k0 + j) * SLOT] = carry;
      }
    }
  }
}

template <typename Tx, typename Ta, typename Ty, bool XCONV, int Q>
hipError_t launch_walkers(const ScanArgs& a, hipStream_t stream) {
  using G_ = Geo<Q>;
  const int nc = (a.seqlen + Q - 1) / Q;
  hipLaunchKernelGGL((bc_pack_kernel<Tx, XCONV, Q>), dim3(nc, a.ngroups, a.batch),
                     dim3(G_::PACK_THREADS), 0, stream, a,
                     static_cast<bf16*>(const_cast<void*>(a.bc_pack)));
  // no walker runs on a pack that was never written
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int W = a.batch * a.nheads * G_::NPS;  // walkers per segment
  if (a.nseg > 1) {
    hipLaunchKernelGGL((scan_bf16_kernel<Tx, Ta, Ty, XCONV, true, Q>), dim3(W * (a.nseg - 1)),
                       dim3(THREADS), 0, stream, a);
    hipLaunchKernelGGL(combine_segments_kernel, dim3(a.batch * a.nheads, COMBINE_PARTS),
                       dim3(COMBINE_THREADS), 0, stream, a);
  }
  hipLaunchKernelGGL((scan_bf16_kernel<Tx, Ta, Ty, XCONV, false, Q>), dim3(W * a.nseg),
                     dim3(THREADS), 0, stream, a);
  return hipGetLastError();
}

template <typename Ta, typename Ty, int Q>
hipError_t pick_x(const ScanArgs& a, ssd_dtype_t xd, hipStream_t s) {
  if (a.conv_w != nullptr)  // raw x|B|C: conv in the pack kernel and the walker
    return xd == SSD_BF16 ? launch_walkers<bf16, Ta, Ty, true, Q>(a, s)
                          : launch_walkers<float, Ta, Ty, true, Q>(a, s);
  return xd == SSD_BF16 ? launch_walkers<bf16, Ta, Ty, false, Q>(a, s)
                        : launch_walkers<float, Ta, Ty, false, Q>(a, s);
}

template <int Q>
hipError_t pick_types(const ScanArgs& a, ssd_dtype_t xd, ssd_dtype_t ad, ssd_dtype_t yd,
                      hipStream_t s) {
  if (ad == SSD_BF16)
    return yd == SSD_F32 ? pick_x<bf16, float, Q>(a, xd, s) : pick_x<bf16, bf16, Q>(a, xd, s);
  return yd == SSD_F32 ? pick_x<float, float, Q>(a, xd, s) : pick_x<float, bf16, Q>(a, xd, s);
}

}  // namespace

bool scan_bf16_supports_chunk(int chunk) { return chunk == 64 || chunk == 128 || chunk == 256; }

hipError_t launch_scan_bf16(const ScanArgs& a, ssd_dtype_t xd, ssd_dtype_t ad, ssd_dtype_t yd,
                            hipStream_t s) {
  switch (a.chunk) {
    case 64: return pick_types<64>(a, xd, ad, yd, s);
    case 128: return pick_types<128>(a, xd, ad, yd, s);
    case 256: return pick_types<256>(a, xd, ad, yd, s);
    default: return hipErrorInvalidValue;
  }
}

size_t scan_bf16_pack_bytes(int batch, int seqlen, int ngroups, int chunk) {
  const size_t nc = ((size_t)seqlen + chunk - 1) / chunk;
  const size_t pack = chunk == 64    ? Geo<64>::PACK
                      : chunk == 256 ? Geo<256>::PACK
                                     : Geo<128>::PACK;
  return (size_t)batch * ngroups * nc * pack * sizeof(bf16);
}

int scan_bf16_walkers_per_head(int chunk) { return chunk == 256 ? Geo<256>::NPS : 1; }

}  // namespace ssd
