// Linear layers y = x W^T (W stored [N, K] row-major) with fused epilogues.
//
// 2-byte operands (bf16, or IEEE binary16 for the block linears under the binary16
// precision mode): gfx950 MFMA (v_mfma_f32_16x16x32_{bf16,f16} in the large-tile kernels,
// v_mfma_f32_32x32x16_{bf16,f16} in the generic one; the kernels keep their bf16 names),
// fp32 accumulation.  A workgroup computes a
// BM x BN tile; operands are staged through LDS in 64-wide K slices with an XOR swizzle of
// the 16-byte chunks so the MFMA fragment reads are bank-conflict free, and the loads of
// later slices are in flight during the MFMAs of the current one.
//
// Epilogues (the blocks' fused ops, "双流块 / 单流块 / 激活函数与 FFN" of the Diffusers
// walk-through):
//   store          y = acc
//   SwiGLU         W rows [gate | up]; y[:, j] = silu(gate_j) * up_j.  The B-tile loader
//                  interleaves 32-row groups of gate and up rows, so each wave holds a
//                  gate column and its up column in the same lane and register.
//   gated residual y = resid + gate[batch] * acc
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <atomic>
#include <climits>
#include <mutex>
#include <type_traits>

namespace flux {

// ------------------------------------------------------------------------------------
// Epilogue functors: called once per output element (m < M, n < N checked by caller)
// ------------------------------------------------------------------------------------
// Row-vector access (kRow4): vec4(m, n, v, N) handles columns n .. n+3 (n % 4 == 0, columns
// at or past N skipped) of row m.  `vec` says the rows start on 4-element boundaries so
// the columns move as one 8- or 16-byte access; it is set on the host by set_vec().
template <class T>
inline bool row4_aligned(const T* p, int64_t ld) {
  return (reinterpret_cast<uintptr_t>(p) % (4 * sizeof(T))) == 0 && ld % 4 == 0;
}
template <class T>
FLUX_DEV void store4(T* p, float4 v);
template <>
FLUX_DEV void store4<float>(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
template <>
FLUX_DEV void store4<bf16>(bf16* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack2(v.x, v.y), pack2(v.z, v.w));
}
template <class T>
FLUX_DEV float4 load4(const T* p);
template <>
FLUX_DEV float4 load4<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <>
FLUX_DEV float4 load4<bf16>(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

template <class TY>
struct EpiStore {
  TY* y;
  int64_t ldy;
  bool vec = false;
  static constexpr bool kPaired = false;
  static constexpr bool kQuad = false;
  static constexpr bool kRow4 = true;
  void set_vec() { vec = row4_aligned(y, ldy); }
  FLUX_DEV int col_major_from() const { return INT_MAX; }
  FLUX_DEV void operator()(int m, int n, float v) const { y[m * ldy + n] = from_f32<TY>(v); }
  FLUX_DEV void vec4(int m, int n, float4 v, int N) const {
    if (vec && n + 3 < N) {
      store4<TY>(y + m * ldy + n, v);
      return;
    }
    const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (n + c < N) (*this)(m, n + c, a[c]);
  }
};

template <class TY>
struct EpiSwiGLU {
  TY* y;
  int64_t ldy;
  int n_half;  // H
  bool lo = false;  // also store lo = v - hi at column H + j (bf16 hi / lo pair)
  static constexpr bool kPaired = true;
  static constexpr bool kQuad = false;
  static constexpr bool kRow4 = false;
  // logical column n of the interleaved [gate | up] tile -> physical W row
  FLUX_DEV static int phys_row(int n, int H) {
    const int j = ((n >> 6) << 5) + (n & 31);
    return ((n >> 5) & 1) ? H + j : j;
  }
  FLUX_DEV void pair(int m, int j, float g, float u) const {
    const float v = silu_f(g) * u;
    const TY h = from_f32<TY>(v);
    y[m * ldy + j] = h;
    if (lo) y[m * ldy + n_half + j] = from_f32<TY>(v - to_f32(h));
  }
};

template <class TY, class TR>
struct EpiGatedResid {
  TY* y;
  int64_t ldy;
  const TR* r;
  int64_t ldr;
  const float* gate;
  int64_t gate_bs;
  int rpb;
  bool vec = false;
  static constexpr bool kPaired = false;
  static constexpr bool kQuad = false;
  static constexpr bool kRow4 = true;
  void set_vec() { vec = row4_aligned(y, ldy) && row4_aligned(r, ldr) && row4_aligned(gate, gate_bs); }
  FLUX_DEV int col_major_from() const { return INT_MAX; }
  FLUX_DEV void operator()(int m, int n, float v) const {
    const int b = m / rpb;
    y[m * ldy + n] = from_f32<TY>(fmaf(gate[b * gate_bs + n], v, to_f32(r[m * ldr + n])));
  }
  FLUX_DEV void vec4(int m, int n, float4 v, int N) const {
    const int b = m / rpb;
    if (vec && n + 3 < N) {
      const float4 x = load4<TR>(r + m * ldr + n);
      const float4 g = *reinterpret_cast<const float4*>(gate + b * gate_bs + n);
      store4<TY>(y + m * ldy + n, make_float4(fmaf(g.x, v.x, x.x), fmaf(g.y, v.y, x.y),
                                              fmaf(g.z, v.z, x.z), fmaf(g.w, v.w, x.w)));
      return;
    }
    const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (n + c < N) (*this)(m, n + c, a[c]);
  }
};

// q | k row-major, v transposed (V^T feeds the attention's PV product directly)
template <class TY>
struct EpiQKV {
  TY* y;
  int64_t ldy;
  TY* vt;
  int64_t ldvt;
  int two_d, dim, rpb, vt_off;
  bool vec = false;
  static constexpr bool kPaired = false;
  static constexpr bool kQuad = true;
  static constexpr bool kRow4 = true;
  void set_vec() { vec = row4_aligned(y, ldy); }
  // first column of the transposed (V) part: tiles at or past it take the column path
  FLUX_DEV int col_major_from() const { return two_d; }
  FLUX_DEV void vec4(int m, int n, float4 v, int N) const {
    if (vec && n + 3 < two_d) {
      store4<TY>(y + m * ldy + n, v);
      return;
    }
    const float a[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (n + c < N) (*this)(m, n + c, a[c]);
  }
  FLUX_DEV void operator()(int m, int n, float v) const {
    if (n < two_d) {
      y[m * ldy + n] = from_f32<TY>(v);
    } else {
      const int b = m / rpb, i = m - b * rpb;
      vt[((int64_t)b * dim + (n - two_d)) * ldvt + vt_off + i] = from_f32<TY>(v);
    }
  }
  // rows m .. m+3 of column n (m % 4 == 0): the V^T part gets one 8-byte store when the
  // four tokens are consecutive in one batch row and 8-byte aligned
  FLUX_DEV void quad(int m, int n, float v0, float v1, float v2, float v3, int M) const {
    if (n < two_d) {
      TY* p = y + m * ldy + n;
      p[0] = from_f32<TY>(v0);
      if (m + 1 < M) p[ldy] = from_f32<TY>(v1);
      if (m + 2 < M) p[2 * ldy] = from_f32<TY>(v2);
      if (m + 3 < M) p[3 * ldy] = from_f32<TY>(v3);
      return;
    }
    const int b = m / rpb, i = m - b * rpb;
    TY* p = vt + ((int64_t)b * dim + (n - two_d)) * ldvt + vt_off + i;
    if (sizeof(TY) == 2 && m + 3 < M && i + 3 < rpb && ((vt_off + i) & 3) == 0) {
      *reinterpret_cast<uint2*>(p) = make_uint2(pack2(v0, v1), pack2(v2, v3));
      return;
    }
    // rows that cross a batch boundary or the end (not reached for 4-aligned shapes)
    (*this)(m, n, v0);
    if (m + 1 < M) (*this)(m + 1, n, v1);
    if (m + 2 < M) (*this)(m + 2, n, v2);
    if (m + 3 < M) (*this)(m + 3, n, v3);
  }
};

// ------------------------------------------------------------------------------------
// bf16 MFMA kernel
// ------------------------------------------------------------------------------------
constexpr int kBK = 64;  // K slice
constexpr int kThreads = 256;

// element offset of (row, 16-byte chunk c) in a [rows][64] bf16 LDS tile.  A row is
// 128 bytes, half of the 64 x 4-byte banks, so rows 2r and 2r+1 share a bank row; XOR-ing
// the chunk with (row >> 1) & 7 makes 16 consecutive rows at one logical chunk land on 16
// distinct 16-byte bank groups (a conflict-free ds_read_b128 for every 16 lanes).
FLUX_DEV int swz_slot(int row, int c) { return c ^ ((row >> 1) & 7); }
FLUX_DEV int swz(int row, int c) { return row * kBK + (swz_slot(row, c) << 3); }

// 8-element MFMA fragments and products of the 2-byte operand types (bf16, binary16)
template <class T>
struct Frag8;
template <>
struct Frag8<bf16> {
  using type = bf16x8;
};
template <>
struct Frag8<f16> {
  using type = f16x8;
};
FLUX_DEV f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
FLUX_DEV f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
FLUX_DEV f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
FLUX_DEV f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int BM, int BN, class Epi, class TIn>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(const TIn* __restrict__ A,
                                                             int64_t lda,
                                                             const TIn* __restrict__ W,
                                                             int64_t ldw, int M, int N, int K,
                                                             int kw, int kdup, int n_half,
                                                             int tiles_n, Epi epi) {
  using Frag = typename Frag8<TIn>::type;
  constexpr int WGM = 2, WGN = 2;                // 2 x 2 waves
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;    // 32x32 MFMA tiles per wave
  constexpr int LA = BM * 8 / kThreads;          // 16-byte chunks per thread (A)
  constexpr int LB = BN * 8 / kThreads;
  static_assert(LA >= 1 && LB >= 1, "tile too small");
  static_assert(!Epi::kPaired || (TN % 2 == 0), "SwiGLU needs gate/up tile pairs");

  extern __shared__ __align__(16) char gen_lds[];
  TIn* smem = reinterpret_cast<TIn*>(gen_lds);
  TIn* As = smem;                   // [2][BM][64]
  TIn* Bs = smem + 2 * BM * kBK;    // [2][BN][64]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // grouped tile order: consecutive workgroups walk down M inside a band of N tiles,
  // so a wave of resident workgroups shares W tiles in L2
  const int bid = blockIdx.x;
  constexpr int GROUP = 8;
  const int tiles_m = (M + BM - 1) / BM;
  const int group_size = GROUP * tiles_n;
  const int g = bid / group_size;
  const int first_m = g * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (bid % group_size) % gm;
  const int tn = (bid % group_size) / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  // per-thread global source pointers (row fixed over the K loop)
  const TIn* a_src[LA];
  bool a_ok[LA];
  int a_lds[LA];
  const TIn* b_src[LB];
  bool b_ok[LB];
  int b_lds[LB];
  const int c8 = tid & 7;
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int r = (tid >> 3) + i * (kThreads / 8);
    const int gr = m0 + r;
    a_ok[i] = gr < M;
    a_src[i] = A + (int64_t)(a_ok[i] ? gr : 0) * lda + c8 * 8;
    a_lds[i] = swz(r, c8);
  }
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (tid >> 3) + i * (kThreads / 8);
    int gn = n0 + r;
    bool ok;
    if constexpr (Epi::kPaired) {
      const int j = ((gn >> 6) << 5) + (gn & 31);
      ok = j < n_half;
      gn = Epi::phys_row(gn, n_half);
    } else {
      ok = gn < N;
    }
    b_ok[i] = ok;
    b_src[i] = W + (int64_t)(ok ? gn : 0) * ldw + c8 * 8;
    b_lds[i] = swz(r, c8);
  }

  uint4 ra[LA], rb[LB];
  auto load_slice = [&](int k0) {
    const bool kin = (k0 + c8 * 8) < K;
    const int kb = (k0 + c8 * 8 >= kw) ? k0 - kdup : k0;  // W column of the hi / lo repeat
#pragma unroll
    for (int i = 0; i < LA; ++i)
      ra[i] = (a_ok[i] && kin) ? ld16(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      rb[i] = (b_ok[i] && kin) ? ld16(b_src[i] + kb) : make_uint4(0, 0, 0, 0);
  };
  auto store_slice = [&](int buf) {
    TIn* as = As + buf * BM * kBK;
    TIn* bs = Bs + buf * BN * kBK;
#pragma unroll
    for (int i = 0; i < LA; ++i) st16(as + a_lds[i], ra[i]);
#pragma unroll
    for (int i = 0; i < LB; ++i) st16(bs + b_lds[i], rb[i]);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = (K + kBK - 1) / kBK;
  load_slice(0);
  store_slice(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int lk = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_slice((kt + 1) * kBK);
    const TIn* as = As + cur * BM * kBK;
    const TIn* bs = Bs + cur * BN * kBK;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      Frag af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * 32 + lrow;
        af[i] = *reinterpret_cast<const Frag*>(as + swz(r, kk * 2 + lk));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WTN + j * 32 + lrow;
        bfr[j] = *reinterpret_cast<const Frag*>(bs + swz(r, kk * 2 + lk));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = mfma32x32x16(af[i], bfr[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_slice(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * WTM + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
      if (m >= M) continue;
      if constexpr (Epi::kPaired) {
#pragma unroll
        for (int j = 0; j < TN; j += 2) {
          const int nl = n0 + wn * WTN + j * 32 + lrow;  // logical gate column
          const int jj = ((nl >> 6) << 5) + (nl & 31);
          if (jj < n_half) epi.pair(m, jj, acc[i][j][r], acc[i][j + 1][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn * WTN + j * 32 + lrow;
          if (n < N) epi(m, n, acc[i][j][r]);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// bf16 MFMA kernel, large tiles, direct global->LDS loads (K % BK == 0)
//
// NWM x NWN waves; each owns a (BM/NWM) x (BN/NWN) tile of MI x MI MFMA blocks.  256x256
// tiles use 8 waves (two per SIMD, so one wave's waits overlap the other's MFMAs).  ST LDS
// stages of BK-wide K slices are filled by global_load_lds_dwordx4: one wave instruction
// writes 1 KB of LDS contiguously (lane i at byte 16 i), so each lane fetches the global
// chunk that belongs at its slot of the swizzled layout.  The loads use the scalar-base
// form (SGPR pointer advanced per slice + a fixed 32-bit per-lane byte offset) so a load
// costs two instructions.
//
// Schedule of one slice (KK = BK/16 MFMA k-steps, fragments double buffered in registers):
//   k-steps 0 .. KK-2:  MFMAs of step kk, each followed by one fragment read of step kk+1
//   k-step  KK-1:       wait for slice kt+1 and barrier (every wave is then done reading
//                       this stage), then MFMAs of the last step interleaved with the
//                       fragment reads of the next slice's step 0 and half the loads of
//                       slice kt+ST into the stage just freed (the other half goes with
//                       step 0 of the next slice)
// so the barrier is the only point where the MFMA pipe can drain, and the first fragments
// of a slice are read under the MFMAs of the previous one.  The K loop is peeled so the
// steady state carries no branches.  Rows past M / N are clamped to valid rows (their
// results are never stored).
//
// 256x256 tiles run an asymmetric variant in the full 160 KB of LDS: two A stages and three
// W stages.  W slices are loaded two slices ahead, in the first k-step of a slice, and get
// seven k-steps to land; A slices are loaded in the last k-step, after the barrier, and get
// four.  Weights are streamed from HBM once per step, so their latency is the one to hide.
// ------------------------------------------------------------------------------------
template <int N>
FLUX_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tile order: the hardware dispatches workgroup i to XCD i % 8.  Give each XCD a
// contiguous run of the logical order, and walk the logical order in bands of GROUP
// M-tiles so concurrently running workgroups share A and W slices in their L2.
FLUX_DEV int xcd_remap(int bid, int total) {
  return ((total & 7) == 0) ? (bid & 7) * (total >> 3) + (bid >> 3) : bid;
}
FLUX_DEV void logical_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP = 8;
  const int group_size = GROUP * tiles_n;
  const int g = bid / group_size;
  const int first_m = g * GROUP;
  const int gm = min(tiles_m - first_m, GROUP);
  const int r = bid - g * group_size;
  tm = first_m + r % gm;
  tn = r / gm;
}
FLUX_DEV void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  logical_coords(xcd_remap(bid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

// LDS layout of one operand slice: rows of BK elements of ES bytes (CPR chunks of 16
// bytes).  With 64 banks x 4 bytes (256 bytes) per bank row, 256 / (16 CPR) consecutive
// rows share a bank row; XOR-ing the chunk index with (row / rows_per_bank_row) spreads the
// 16 rows read by 16 lanes of a ds_read_b128 over 16 distinct 16-byte bank groups.
template <int BK, int ES = 2>
struct Swz {
  static constexpr int CE = 16 / ES;  // elements per chunk
  static constexpr int CPR = BK / CE;
  static constexpr int RSH = (CPR == 8) ? 1 : 2;
  FLUX_DEV static int slot(int row, int c) { return c ^ ((row >> RSH) & (CPR - 1)); }
  FLUX_DEV static int off(int row, int c) { return row * BK + slot(row, c) * CE; }
};

typedef uint8_t fp8;  // OCP E4M3 byte
typedef int v8i __attribute__((ext_vector_type(8)));

// Body of the large-tile kernels.  TIn = bf16 / binary16 (MFMA 32x32x16 or 16x16x32,
// MI = 32 / 16) or
// fp8 (E4M3 bytes, MFMA 32x32x64 with unit block scales; the accumulators are multiplied by
// the per-row scale sa[m] and the per-weight-row scale sw[n] before the epilogue).  Rows of
// a K slice are 64 or 128 bytes either way, so the load plan, the LDS layout and the
// schedule are shared.  The 16x16x32 form does the same work with a quarter of the
// accumulator registers per MFMA and measured ~10% more sustained throughput with real
// (full-entropy) operands, where the chip is power-bound.
// One product of a launch: operands, rows (and their tile count) and epilogue.  A launch
// runs one product, or two with the same N and K and operand strides (the double block's
// image and text streams); segment 1's tiles follow segment 0's in the logical tile order,
// so a partial last round of tiles (and its split-K) falls on segment 1.
template <class TIn, class Epi>
struct GemmSeg {
  const TIn* A;
  const TIn* W;
  int M;
  int tiles_m;
  Epi epi;
};

template <class TIn, int BM, int BN, int BK, int ST, int STW, int MI, int NWM, int NWN, class Epi>
FLUX_DEV void gemm_lds_body(const GemmSeg<TIn, Epi>& s0, const GemmSeg<TIn, Epi>& s1, int tiles0,
                            int64_t lda, int64_t ldw, int N, int K, int kw, int kdup, int n_half,
                            int tiles_n, int full_tiles, int splits, float* __restrict__ partial,
                            const float* __restrict__ sa, const float* __restrict__ sw) {
  constexpr int ES = sizeof(TIn);
  constexpr bool F8 = ES == 1;
  static_assert(BK * ES == 64 || BK * ES == 128, "BK: 64- or 128-byte slice rows");
  static_assert(ST >= 2 && ST <= 4, "stages");
  // STW == ST: A and W slices share the schedule; STW == 3 with ST == 2: W runs one slice
  // further ahead (the asymmetric schedule below)
  static_assert(STW == ST || (ST == 2 && STW == 3), "W stages");
  constexpr bool ASYM = STW != ST;
  using S = Swz<BK, ES>;
  constexpr int NWV = NWM * NWN;        // waves per workgroup
  constexpr int CPR = S::CPR;           // chunks per row
  constexpr int RPI = 64 / CPR;         // rows per wave load instruction
  constexpr int AI = BM / (NWV * RPI);  // A load instructions per wave per slice
  constexpr int BI = BN / (NWV * RPI);
  constexpr int LOADS = AI + BI;
  constexpr int WTM = BM / NWM, WTN = BN / NWN;
  static_assert(MI == 32 || (MI == 16 && !F8), "MFMA shape");
  constexpr int TM = WTM / MI, TN = WTN / MI;
  constexpr int KK = BK / (F8 ? 64 : 512 / MI);  // MFMA k-steps per slice
  constexpr int NF = TM + TN;           // fragments per k-step
  constexpr int AR = MI == 32 ? 16 : 4;  // accumulator registers per lane and MFMA block
  // fragment reads of the next k-step: one after every RSTEP-th MFMA
  constexpr int RSTEP = TM * TN >= 2 * NF ? 2 : 1;
  constexpr uint32_t A_STAGE_B = BM * BK * ES, W_STAGE_B = BN * BK * ES;
  static_assert(AI >= 1 && BI >= 1, "tile too small for the load plan");
  static_assert(KK % 2 == 0, "fragment sets alternate with the k-step parity");
  // SwiGLU: gate and up rows interleave per 32 W rows, so a gate block's partner is the
  // next 32x32 block or the 16x16 block two further
  static_assert(!Epi::kPaired || (TN % (64 / MI) == 0), "SwiGLU needs gate/up tile pairs");

  extern __shared__ __align__(16) char lds_raw[];
  TIn* smem = reinterpret_cast<TIn*>(lds_raw);
  // A stage s at smem + s * BM * BK; W stage s at smem + ST * BM * BK + s * BN * BK

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / NWN, wn = wave % NWN;
  // workgroups [0, full_tiles) own whole tiles (XCD-aware order); the rest split the
  // remaining tiles along K into `splits` ranges and write fp32 partial tiles
  const int nk_all = K / BK;
  int logical, k_begin = 0, k_end = nk_all, unit = -1;
  if ((int)blockIdx.x < full_tiles) {
    logical = xcd_remap(blockIdx.x, full_tiles);
  } else {
    unit = blockIdx.x - full_tiles;
    const int split = unit % splits;
    logical = full_tiles + unit / splits;
    k_begin = split * nk_all / splits;
    k_end = (split + 1) * nk_all / splits;
  }
  // the tile's product (segment); the selection is uniform across the workgroup
  const bool seg1 = logical >= tiles0;
  const GemmSeg<TIn, Epi>& G = seg1 ? s1 : s0;
  const TIn* __restrict__ A = G.A;
  const TIn* __restrict__ W = G.W;
  const int M = G.M;
  const Epi epi = G.epi;
  int tm, tn;
  logical_coords(seg1 ? logical - tiles0 : logical, G.tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // load plan: instruction j of wave w covers rows (w*AI + j)*RPI + [0, RPI); lane ->
  // row lane / CPR, LDS slot lane % CPR, global chunk = the chunk of that slot.  Byte
  // offsets from the operand base fit 32 bits (checked by the launcher).
  uint32_t a_off[AI], b_off[BI];
#pragma unroll
  for (int j = 0; j < AI; ++j) {
    const int r = (wave * AI + j) * RPI + lane / CPR;
    const int gr = min(m0 + r, M - 1);
    a_off[j] = (uint32_t)(((int64_t)gr * lda + S::slot(r, lane % CPR) * S::CE) * ES);
  }
#pragma unroll
  for (int j = 0; j < BI; ++j) {
    const int r = (wave * BI + j) * RPI + lane / CPR;
    int gn = n0 + r;
    if constexpr (Epi::kPaired) {
      const int jj = min(((gn >> 6) << 5) + (gn & 31), n_half - 1);
      gn = ((gn >> 5) & 1) ? n_half + jj : jj;
    } else {
      gn = min(gn, N - 1);
    }
    b_off[j] = (uint32_t)(((int64_t)gn * ldw + S::slot(r, lane % CPR) * S::CE) * ES);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_u32(smem));
  const int nk = k_end - k_begin;
  const int kb = k_begin * BK;
  // q-th load instruction of this wave's share of slice sl (q < AI: A rows, else W rows)
  auto dma = [&](int q, int sl) {
    const int k0 = kb + sl * BK;
    if (q < AI) {
      const uint32_t sb = lds0 + (uint32_t)(sl % ST) * A_STAGE_B;
      dma16s(A + k0, a_off[q], sb + (uint32_t)((wave * AI + q) * RPI * BK * ES));
    } else {
      // slices past kw repeat W columns (the lo plane of a hi / lo operand)
      const int kw0 = k0 >= kw ? k0 - kdup : k0;
      const uint32_t sb = lds0 + ST * A_STAGE_B + (uint32_t)(sl % STW) * W_STAGE_B;
      dma16s(W + kw0, b_off[q - AI], sb + (uint32_t)((wave * BI + q - AI) * RPI * BK * ES));
    }
  };

  using Acc = typename std::conditional<MI == 32, f32x16, f32x4>::type;
  Acc acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < AR; ++r) acc[i][j][r] = 0.f;

  // MFMA lane layout.  32x32: lane holds column lane & 31 and rows 8 (r/4) + 4 (lane/32) +
  // r%4; its A / B fragment is row lane & 31, k 8 (lane/32) .. + 8 of a 16-deep k-step.
  // 16x16: lane holds column lane & 15 and rows 4 (lane/16) + r; its fragment is row
  // lane & 15, k 8 (lane/16) .. + 8 of a 32-deep k-step.
  const int lrow = lane & (MI - 1), lk = lane / MI;
  auto acc_row = [&](int i, int r) {  // row of register r of block i within the wave tile
    return MI == 32 ? i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3) : i * 16 + 4 * lk + r;
  };
  auto acc_col = [&](int j) { return j * MI + lrow; };
  using Frag = typename std::conditional<F8, v8i, typename Frag8<
      typename std::conditional<F8, bf16, TIn>::type>::type>::type;
  Frag fr[2][NF];  // [set][A fragments | B fragments]
  auto rd = [&](int set, int q, int sl, int kk) {  // fragment q of k-step kk of slice sl
    const TIn* ob = q < TM ? smem + (sl % ST) * BM * BK
                           : smem + ST * BM * BK + (sl % STW) * BN * BK;
    const int row = q < TM ? wm * WTM + q * MI + lrow : wn * WTN + (q - TM) * MI + lrow;
    if constexpr (F8) {
      // k-step kk covers chunks 4 kk .. 4 kk + 3 (64 k); lane group lk holds two of them
      const uint4 lo = *reinterpret_cast<const uint4*>(ob + S::off(row, kk * 4 + 2 * lk));
      const uint4 hi = *reinterpret_cast<const uint4*>(ob + S::off(row, kk * 4 + 2 * lk + 1));
      fr[set][q] = Frag{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                        (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    } else {
      fr[set][q] = *reinterpret_cast<const Frag*>(ob + S::off(row, kk * (64 / MI) + lk));
    }
  };

  auto mfma = [&](int set, int i, int j) {
    if constexpr (F8)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fr[set][i], fr[set][TM + j], acc[i][j], 0, 0, 0, 127, 0, 127);
    else if constexpr (MI == 32)
      acc[i][j] = mfma32x32x16(fr[set][i], fr[set][TM + j], acc[i][j]);
    else
      acc[i][j] = mfma16x16x32(fr[set][i], fr[set][TM + j], acc[i][j]);
  };

  // prologue: fill the stages, wait for slice 0, read its first fragments.  Symmetric: ST
  // whole slices.  Asymmetric: A and W of slices 0 and 1 (W of slice 2 goes with the first
  // k-step of slice 0).
  constexpr int PRE = ASYM ? 2 : ST;  // slices loaded by the prologue
#pragma unroll
  for (int p = 0; p < PRE; ++p)
    if (p < nk)
#pragma unroll
      for (int q = 0; q < LOADS; ++q) dma(q, p);
  if (nk >= PRE)
    wait_vmcnt<(PRE - 1) * LOADS>();
  else
    wait_vmcnt<0>();
  __syncthreads();
  if (nk > 0)
#pragma unroll
    for (int q = 0; q < NF; ++q) rd(0, q, 0, 0);

  // One slice, symmetric stages.  The loads of slice kt+ST go into stage kt%ST, which the
  // barrier of the last k-step of slice kt frees; they are split over that k-step and the
  // first k-step of slice kt+1 (fewer loads in flight at once), and land before the barrier
  // of slice kt+1.
  // DMA_ON: start loading slice kt+ST; CONT: finish the loads begun in slice kt-1;
  // RD_ON: read the next slice's first fragments.
  constexpr int PER = (LOADS + 1) / 2;  // loads per k-step
  auto slice = [&](int kt, auto dma_on, auto rd_on, auto cont_on) {
    constexpr bool DMA_ON = decltype(dma_on)::value, RD_ON = decltype(rd_on)::value;
    constexpr bool CONT = decltype(cont_on)::value;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      const bool last = kk == KK - 1;
      if (last) {
        // slice kt+1 landed (later slices may still be in flight) and, after the barrier,
        // every wave is done reading slice kt's stage
        if (DMA_ON)
          wait_vmcnt<(ST - 2) * LOADS>();
        else
          wait_vmcnt<0>();
        __syncthreads();
      }
      const bool do_rd = !last || RD_ON;
      const int rsl = last ? kt + 1 : kt, rkk = last ? 0 : kk + 1;
      // loads [q0, q1) of slice ds in this k-step
      int q0 = 0, q1 = 0, ds = 0;
      if (last && DMA_ON) {
        q1 = PER;
        ds = kt + ST;
      } else if (kk == 0 && CONT) {
        q0 = PER;
        q1 = LOADS;
        ds = kt + ST - 1;
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < TM * TN; ++q) {
        const int i = q / TN, j = q % TN;
        mfma(cur, i, j);
        __builtin_amdgcn_sched_barrier(0);
        if (do_rd && q % RSTEP == 0 && q / RSTEP < NF) rd(nxt, q / RSTEP, rsl, rkk);
        if (q0 + q < q1) dma(q0 + q, ds);
        __builtin_amdgcn_sched_barrier(0);
      }
      // leftovers when a k-step has fewer MFMAs than reads or loads
#pragma unroll
      for (int q = TM * TN; q < PER; ++q)
        if (q0 + q < q1) dma(q0 + q, ds);
      if (do_rd)
#pragma unroll
        for (int q = (TM * TN + RSTEP - 1) / RSTEP; q < NF; ++q) rd(nxt, q, rsl, rkk);
    }
  };

  // One slice, asymmetric stages (A: 2, W: 3).  The first k-step of slice kt loads W of
  // slice kt+2 (its stage, that of slice kt-1, was freed by slice kt-1's last barrier); the
  // last k-step, after its barrier, loads A of slice kt+2 into the A stage of slice kt.  At
  // that barrier the only loads allowed in flight are the W loads of slice kt+2, issued
  // last: W gets seven k-steps to land, A four.  ON: slice kt+2 exists (both loads);
  // RD_ON: read the next slice's first fragments.
  auto slice_aw = [&](int kt, auto on, auto rd_on) {
    constexpr bool ON = decltype(on)::value, RD_ON = decltype(rd_on)::value;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cur = kk & 1, nxt = cur ^ 1;
      const bool last = kk == KK - 1;
      if (last) {
        if (ON)
          wait_vmcnt<BI>();
        else
          wait_vmcnt<0>();
        __syncthreads();
      }
      const bool do_rd = !last || RD_ON;
      const int rsl = last ? kt + 1 : kt, rkk = last ? 0 : kk + 1;
      // loads [q0, q1) of slice kt+2 in this k-step: W rows first, A rows last
      const int q0 = (ON && kk == 0) ? AI : 0;
      const int q1 = !ON ? 0 : kk == 0 ? LOADS : last ? AI : 0;
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < TM * TN; ++q) {
        const int i = q / TN, j = q % TN;
        mfma(cur, i, j);
        __builtin_amdgcn_sched_barrier(0);
        if (do_rd && q % RSTEP == 0 && q / RSTEP < NF) rd(nxt, q / RSTEP, rsl, rkk);
        if (q0 + q < q1) dma(q0 + q, kt + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int q = TM * TN; q < LOADS; ++q)
        if (q0 + q < q1) dma(q0 + q, kt + 2);
      if (do_rd)
#pragma unroll
        for (int q = (TM * TN + RSTEP - 1) / RSTEP; q < NF; ++q) rd(nxt, q, rsl, rkk);
    }
  };

  using On = std::true_type;
  using Off = std::false_type;
  int kt = 0;
  if constexpr (ASYM) {
    for (; kt + 2 < nk; ++kt) slice_aw(kt, On{}, On{});
    if (kt + 1 < nk) slice_aw(kt++, Off{}, On{});
    if (kt < nk) slice_aw(kt, Off{}, Off{});
  } else {
    if (kt + ST < nk) slice(kt++, On{}, On{}, Off{});
    for (; kt + ST < nk; ++kt) slice(kt, On{}, On{}, On{});
    // kt >= 1 here only if slice kt-1 started loading slice kt+ST-1 (< nk)
    if (kt >= 1 && kt + 1 < nk) slice(kt++, Off{}, On{}, On{});
    for (; kt + 1 < nk; ++kt) slice(kt, Off{}, On{}, Off{});
    if (kt < nk) {
      if (kt >= 1 && kt - 1 + ST < nk)
        slice(kt, Off{}, Off{}, On{});
      else
        slice(kt, Off{}, Off{}, Off{});
    }
  }

  if constexpr (F8) {
    // dequantize: y = sa[m] sw[n] acc (W row of logical column n: the SwiGLU pairing)
    float swv[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * WTN + acc_col(j);
      int pn;
      if constexpr (Epi::kPaired) {
        const int jj = min(((n >> 6) << 5) + (n & 31), n_half - 1);
        pn = ((n >> 5) & 1) ? n_half + jj : jj;
      } else {
        pn = min(n, N - 1);
      }
      swv[j] = sw[pn];
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < AR; ++r) {
        const float av = sa[min(m0 + wm * WTM + acc_row(i, r), M - 1)];
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j][r] *= av * swv[j];
      }
  }
  if (unit >= 0) {
    // split-K unit: raw fp32 partial tile [BM][BN] (local coordinates)
    float* pt = partial + (size_t)unit * BM * BN;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < AR; ++r) {
        const int ml = wm * WTM + acc_row(i, r);
#pragma unroll
        for (int j = 0; j < TN; ++j) pt[ml * BN + wn * WTN + acc_col(j)] = acc[i][j][r];
      }
    return;
  }
  if constexpr (Epi::kRow4) {
    // Row-vector epilogue through the (now idle) LDS stages.  Pass p stages the 16 rows
    // 16p .. 16p + 15 of every wave's tile (registers RPP p' .. of block p / (MI / 16)):
    // PR = 16*NWM rows of BN fp32 (two buffers, alternating), then each wave moves whole
    // staged rows with 16-byte LDS reads and row-contiguous global accesses (the residual /
    // gate loads of a pass are all in flight together).  Staged row sr holds tile row
    // (sr/16)*WTM + 16p + sr%16.  Its columns are XOR-ed with swz(sr) so the lane groups of
    // a ds_write (rows 4 apart) hit different banks.
    constexpr int PR = 16 * NWM, NT = 64 * NWV, CPO = BN / 4;
    constexpr int PER_T = PR * CPO / NT;
    constexpr int RPP = MI == 32 ? 8 : 4;  // accumulator registers per pass
    static_assert(PR * CPO % NT == 0 && BN % 64 == 0, "staged epilogue shape");
    static_assert(2 * PR * BN * 4 <= ST * A_STAGE_B + STW * W_STAGE_B, "staging buffers fit in the LDS stages");
    auto swz = [](int sr) { return MI == 32 ? ((sr >> 2) & 1) << 5 : ((sr >> 2) & 3) << 4; };
    float* stg = reinterpret_cast<float*>(smem);
    __syncthreads();  // every wave is done reading the last slice
#pragma unroll
    for (int p = 0; p < WTM / 16; ++p) {
      const int i = p / (MI / 16), r0 = (p % (MI / 16)) * RPP;
      float* buf = stg + (p & 1) * PR * BN;
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr) {
        const int sr = wm * 16 + (acc_row(i, r0 + rr) & 15);
#pragma unroll
        for (int j = 0; j < TN; ++j)
          buf[sr * BN + ((wn * WTN + acc_col(j)) ^ swz(sr))] = acc[i][j][r0 + rr];
      }
      __syncthreads();
      if (n0 < epi.col_major_from()) {
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
          const int e = tid + u * NT;
          const int sr = e / CPO, c = e % CPO;
          const int m = m0 + (sr >> 4) * WTM + 16 * p + (sr & 15);
          const int n = n0 + 4 * c;
          const float4 v = *reinterpret_cast<const float4*>(buf + sr * BN + ((4 * c) ^ swz(sr)));
          if (m < M && n < N) epi.vec4(m, n, v, N);
        }
      } else if constexpr (Epi::kQuad) {
        // column-major output: item = 4 consecutive rows (staged rows 4q .. 4q+3 of a wave
        // block, one swizzle) of one column; 4 lanes in a row cover 16 contiguous rows
#pragma unroll 2
        for (int u = 0; u < PER_T; ++u) {
          const int e = tid + u * NT;
          const int q = e & 3, col = (e >> 2) % BN, wb = (e >> 2) / BN;
          const int sr = wb * 16 + 4 * q;
          const float* src = buf + sr * BN + (col ^ swz(sr));
          const int m = m0 + wb * WTM + 16 * p + 4 * q;
          const int n = n0 + col;
          if (m < M && n < N) epi.quad(m, n, src[0], src[BN], src[2 * BN], src[3 * BN], M);
        }
      }
    }
    return;
  }
  if constexpr (Epi::kQuad) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r4 = 0; r4 < AR / 4; ++r4) {
        const int m = m0 + wm * WTM + acc_row(i, 4 * r4);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn * WTN + acc_col(j);
          if (n < N)
            epi.quad(m, n, acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2],
                     acc[i][j][4 * r4 + 3], M);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < AR; ++r) {
      const int m = m0 + wm * WTM + acc_row(i, r);
      if (m >= M) continue;
      if constexpr (Epi::kPaired) {
        constexpr int PO = 32 / MI;  // up block of gate block j: j + PO
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (j & PO) continue;
          const int nl = n0 + wn * WTN + acc_col(j);
          const int jj = ((nl >> 6) << 5) + (nl & 31);
          if (jj < n_half) epi.pair(m, jj, acc[i][j][r], acc[i][j + PO][r]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn * WTN + acc_col(j);
          if (n < N) epi(m, n, acc[i][j][r]);
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int ST, int STW, int MI, int OCC, int NWM, int NWN, class Epi,
          class TIn>
__global__ __launch_bounds__(64 * NWM * NWN, OCC) void gemm_bf16_lds_kernel(
    GemmSeg<TIn, Epi> s0, GemmSeg<TIn, Epi> s1, int tiles0, int64_t lda, int64_t ldw, int N,
    int K, int kw, int kdup, int n_half, int tiles_n, int full_tiles, int splits,
    float* __restrict__ partial) {
  gemm_lds_body<TIn, BM, BN, BK, ST, STW, MI, NWM, NWN, Epi>(s0, s1, tiles0, lda, ldw, N, K, kw,
                                                              kdup, n_half, tiles_n, full_tiles,
                                                              splits, partial, nullptr, nullptr);
}

template <int BM, int BN, int BK, int ST, int OCC, int NWM, int NWN, class Epi>
__global__ __launch_bounds__(64 * NWM * NWN, OCC) void gemm_fp8_lds_kernel(
    GemmSeg<fp8, Epi> s0, int64_t lda, int64_t ldw, int N, int K, int n_half, int tiles_n,
    int full_tiles, int splits, float* __restrict__ partial, const float* __restrict__ sa,
    const float* __restrict__ sw) {
  gemm_lds_body<fp8, BM, BN, BK, ST, ST, 32, NWM, NWN, Epi>(s0, s0, INT_MAX, lda, ldw, N, K, K, 0,
                                                            n_half, tiles_n, full_tiles, splits,
                                                            partial, sa, sw);
}

// Split-K tail: sum the `splits` partial tiles of each tail tile in a fixed order (so the
// result is deterministic) and apply the fused epilogue.  grid = (tail tiles, chunks);
// each thread owns 4 consecutive columns of one row (16-byte loads per partial).
template <int BM, int BN, class Epi, class TIn>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int splits, int full_tiles,
                                                            GemmSeg<TIn, Epi> s0,
                                                            GemmSeg<TIn, Epi> s1, int tiles0,
                                                            int tiles_n, int N, int n_half) {
  const int t = blockIdx.x;
  const int logical = full_tiles + t;
  const bool seg1 = logical >= tiles0;
  const GemmSeg<TIn, Epi>& G = seg1 ? s1 : s0;
  const int M = G.M;
  const Epi epi = G.epi;
  int tm, tn;
  logical_coords(seg1 ? logical - tiles0 : logical, G.tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const float* p = partial + (size_t)t * splits * BM * BN;
  const size_t stride = (size_t)BM * BN;
  if constexpr (Epi::kQuad) {
    if (n0 >= epi.col_major_from()) {
      // column-major output (V^T): the workgroup sums a 64-row x 16-column block with
      // row-contiguous 16-byte reads, transposes it through LDS, and stores 4 consecutive
      // rows of one column per thread (16 lanes cover 64 contiguous rows of a column)
      static_assert(BM % 64 == 0 && BN % 16 == 0, "transposed reduce blocks");
      __shared__ float sT[16][65];
      const int mb = blockIdx.y / (BN / 16), nb = blockIdx.y % (BN / 16);
      const int r = threadIdx.x >> 2, c4 = (threadIdx.x & 3) * 4;
      const float* pp = p + (size_t)(mb * 64 + r) * BN + nb * 16 + c4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
      for (int sp = 0; sp < splits; ++sp) {
        const float4 a = *reinterpret_cast<const float4*>(pp + sp * stride);
        v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
      }
      sT[c4][r] = v.x;
      sT[c4 + 1][r] = v.y;
      sT[c4 + 2][r] = v.z;
      sT[c4 + 3][r] = v.w;
      __syncthreads();
      const int cl = threadIdx.x >> 4, q = threadIdx.x & 15;
      const int m = m0 + mb * 64 + 4 * q, n = n0 + nb * 16 + cl;
      if (m < M && n < N)
        epi.quad(m, n, sT[cl][4 * q], sT[cl][4 * q + 1], sT[cl][4 * q + 2], sT[cl][4 * q + 3], M);
      return;
    }
  }
  const int e = blockIdx.y * 256 + threadIdx.x;
  if constexpr (Epi::kPaired) {
    // logical columns come in 64-groups: 32 gate columns, then their 32 up columns
    if (e >= BM * BN / 8) return;
    const int ml = e / (BN / 8), q = e % (BN / 8);
    const int nl = (q >> 3) * 64 + (q & 7) * 4;
    const int m = m0 + ml;
    if (m >= M) return;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
    const float* pg = p + ml * BN + nl;
#pragma unroll 4
    for (int sp = 0; sp < splits; ++sp) {
      const float4 a = *reinterpret_cast<const float4*>(pg + sp * stride);
      const float4 b = *reinterpret_cast<const float4*>(pg + sp * stride + 32);
      g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
      u.x += b.x; u.y += b.y; u.z += b.z; u.w += b.w;
    }
    const float gv[4] = {g.x, g.y, g.z, g.w}, uv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int nn = n0 + nl + c;
      const int jj = ((nn >> 6) << 5) + (nn & 31);
      if (jj < n_half) epi.pair(m, jj, gv[c], uv[c]);
    }
  } else {
    if (e >= BM * BN / 4) return;
    const int ml = e / (BN / 4), nl = (e % (BN / 4)) * 4;
    const int m = m0 + ml;
    if (m >= M) return;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    const float* pp = p + ml * BN + nl;
#pragma unroll 4
    for (int sp = 0; sp < splits; ++sp) {
      const float4 a = *reinterpret_cast<const float4*>(pp + sp * stride);
      v.x += a.x; v.y += a.y; v.z += a.z; v.w += a.w;
    }
    if constexpr (Epi::kRow4) {
      if (n0 + nl < N) epi.vec4(m, n0 + nl, v, N);
    } else {
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (n0 + nl + c < N) epi(m, n0 + nl + c, vv[c]);
    }
  }
}

// Bytes of split-K scratch the large-tile path may use (tail tiles x splits x tile).
constexpr size_t kSplitkBytes = (size_t)256 * 256 * 256 * sizeof(float);

// Raise a kernel's dynamic-LDS limit once per device.  `done` (one per kernel instance)
// holds a bit per device whose limit is set; the first launches on a device may race from
// several threads, so setting is serialised and the bit is published after it.
struct LdsLimit {
  std::atomic<uint64_t> done{0};
  std::mutex mu;
};
static hipError_t ensure_lds_limit(LdsLimit& st, const void* fn, size_t bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64)
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  const uint64_t bit = uint64_t{1} << dev;
  if (st.done.load(std::memory_order_acquire) & bit) return hipSuccess;
  std::lock_guard<std::mutex> g(st.mu);
  if (st.done.load(std::memory_order_relaxed) & bit) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) st.done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Launch one large-tile configuration (sets the dynamic LDS limit once per instance) over
// the products seg[0 .. nseg) (nseg 1 or 2; segment 1 may have no rows).
template <int BM, int BN, int BK, int ST, int STW, int MI, int OCC, int NWM, int NWN, class Epi,
          class TIn>
static hipError_t launch_lds(const GemmSeg<TIn, Epi>* seg, int nseg, int64_t lda, int64_t ldw,
                             int N, int K, int kw, int kdup, int n_half, int splits,
                             float* partial, hipStream_t s) {
  GemmSeg<TIn, Epi> g0 = seg[0], g1 = nseg > 1 ? seg[1] : seg[0];
  const int tiles_n = (N + BN - 1) / BN;
  g0.tiles_m = (g0.M + BM - 1) / BM;
  g1.tiles_m = (g1.M + BM - 1) / BM;
  const int tiles0 = g0.tiles_m * tiles_n;
  const int tiles = tiles0 + (nseg > 1 ? g1.tiles_m * tiles_n : 0);
  const int slots = 256 * OCC;
  const int tail = splits > 1 ? tiles % slots : 0;
  const int full = tiles - tail;
  if (tail == 0) splits = 1;
  if ((size_t)tail * splits * BM * BN * sizeof(float) > kSplitkBytes) return hipErrorInvalidValue;
  const size_t lds = (size_t)(ST * BM + STW * BN) * BK * sizeof(TIn);
  static LdsLimit limit;
  hipError_t le = ensure_lds_limit(
      limit,
      reinterpret_cast<const void*>(
          &gemm_bf16_lds_kernel<BM, BN, BK, ST, STW, MI, OCC, NWM, NWN, Epi, TIn>),
      lds);
  if (le != hipSuccess) return le;
  hipLaunchKernelGGL((gemm_bf16_lds_kernel<BM, BN, BK, ST, STW, MI, OCC, NWM, NWN, Epi, TIn>),
                     dim3(full + tail * splits), dim3(64 * NWM * NWN), lds, s, g0, g1, tiles0, lda,
                     ldw, N, K, kw, kdup, n_half, tiles_n, full, splits, partial);
  if (tail > 0) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int chunks = Epi::kPaired ? BM * BN / 8 / 256 : BM * BN / 4 / 256;
    hipLaunchKernelGGL((splitk_reduce_kernel<BM, BN, Epi, TIn>), dim3(tail, chunks), dim3(256),
                       0, s, partial, splits, full, g0, g1, tiles0, tiles_n, N, n_half);
  }
  return hipGetLastError();
}

// Same for the fp8 kernel (K slices of 128 bytes = 128 elements; one product).
template <int BM, int BN, int ST, int OCC, int NWM, int NWN, class Epi>
static hipError_t launch_lds_fp8(const fp8* A, int64_t lda, const fp8* W, int64_t ldw, int M,
                                 int N, int K, int n_half, const Epi& epi, int splits,
                                 float* partial, const float* sa, const float* sw, hipStream_t s) {
  constexpr int BK = 128;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int slots = 256 * OCC;
  const int tail = splits > 1 ? tiles % slots : 0;
  const int full = tiles - tail;
  if (tail == 0) splits = 1;
  if ((size_t)tail * splits * BM * BN * sizeof(float) > kSplitkBytes) return hipErrorInvalidValue;
  const GemmSeg<fp8, Epi> g{A, W, M, tiles_m, epi};
  const size_t lds = (size_t)ST * (BM + BN) * BK;
  static LdsLimit limit;
  hipError_t le = ensure_lds_limit(
      limit,
      reinterpret_cast<const void*>(&gemm_fp8_lds_kernel<BM, BN, BK, ST, OCC, NWM, NWN, Epi>),
      lds);
  if (le != hipSuccess) return le;
  hipLaunchKernelGGL((gemm_fp8_lds_kernel<BM, BN, BK, ST, OCC, NWM, NWN, Epi>),
                     dim3(full + tail * splits), dim3(64 * NWM * NWN), lds, s, g, lda, ldw, N, K,
                     n_half, tiles_n, full, splits, partial, sa, sw);
  if (tail > 0) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int chunks = Epi::kPaired ? BM * BN / 8 / 256 : BM * BN / 4 / 256;
    hipLaunchKernelGGL((splitk_reduce_kernel<BM, BN, Epi, fp8>), dim3(tail, chunks), dim3(256), 0,
                       s, partial, splits, full, g, g, INT_MAX, tiles_n, N, n_half);
  }
  return hipGetLastError();
}


// Choose the tile configuration (and split-K of the last partial round) with the smallest
// estimated time (over the tiles of one product, or of two with the same N and K).  A
// round of resident workgroups costs its MACs at about 1 PFLOP/s over
// the chip (times `rate`: 2 for fp8), scaled by the configuration's relative efficiency; a
// tail round split s ways along K costs 1/s of a round plus the fp32 partial tiles' round
// trip through HBM and the reduce launch.  best: 0 = 256x256, 1 = 256x128, 2 = 128x128.
static void pick_tile(int M, int N, int K, int bk, double rate, bool can_split, int& best,
                      int& best_split, int M1 = 0) {
  const int cus = 256;
  constexpr double kFlopPerCu = 4.0e12, kHbm = 5.0e12, kReduceLaunch = 3e-6;
  struct Cand { int bm, bn, occ; double eff; };
  const Cand cands[3] = {{256, 256, 1, 1.0}, {256, 128, 1, 0.8}, {128, 128, 2, 0.85}};
  const int nk = K / bk;
  best = 0;
  best_split = 1;
  double best_t = 1e300;
  for (int c = 0; c < 3; ++c) {
    // M1: rows of a second product in the same launch (tiles of both)
    const long tiles = (long)((M + cands[c].bm - 1) / cands[c].bm +
                              (M1 + cands[c].bm - 1) / cands[c].bm) *
                       ((N + cands[c].bn - 1) / cands[c].bn);
    const long slots = (long)cus * cands[c].occ;
    const double round = 2.0 * cands[c].bm * cands[c].bn * cands[c].occ * (double)K /
                         cands[c].eff / (kFlopPerCu * rate);
    const long tail = tiles % slots;
    const size_t tile_bytes = (size_t)cands[c].bm * cands[c].bn * sizeof(float);
    double t = (double)((tiles + slots - 1) / slots) * round;
    int split = 1;
    // split the tail: s units per tail tile, at least 8 K-slices each
    if (tail > 0 && can_split && 2 * tail <= slots) {
      int sp = (int)(slots / tail);
      sp = sp < nk / 8 ? sp : nk / 8;
      while (sp > 1 && (size_t)tail * sp * tile_bytes > kSplitkBytes) --sp;
      if (sp >= 2) {
        const double ts = (double)(tiles / slots) * round + round / sp +
                          2.0 * tail * sp * tile_bytes / kHbm + kReduceLaunch;
        if (ts < t) { t = ts; split = sp; }
      }
    }
    if (t < best_t * 0.999) { best_t = t; best = c; best_split = split; }
  }
}

// ------------------------------------------------------------------------------------
// fp32 path (tiny fp32 workloads): LDS-tiled FMA, 64 x 64 tile, 4 x 4 per thread with
// strided columns (tx + 16 jj) so the SwiGLU pairs (jj, jj+2) sit in one thread.
// ------------------------------------------------------------------------------------
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t lda,
                                                       const float* __restrict__ W, int64_t ldw,
                                                       int M, int N, int K, int n_half, Epi epi) {
  constexpr int T = 64, BKf = 16;
  __shared__ float As[BKf][T + 1];
  __shared__ float Bs[BKf][T + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * T, n0 = blockIdx.x * T;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BKf) {
    for (int e = threadIdx.x; e < T * BKf; e += 256) {
      const int r = e / BKf, kk = e % BKf;
      const int gm = m0 + r, gk = k0 + kk;
      As[kk][r] = (gm < M && gk < K) ? A[(int64_t)gm * lda + gk] : 0.f;
      int gn = n0 + r;
      bool ok;
      if constexpr (Epi::kPaired) {
        const int j = ((gn >> 6) << 5) + (gn & 31);
        ok = j < n_half;
        gn = Epi::phys_row(gn, n_half);
      } else {
        ok = gn < N;
      }
      Bs[kk][r] = (ok && gk < K) ? W[(int64_t)gn * ldw + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKf; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty + 16 * i;
    if (m >= M) continue;
    if constexpr (Epi::kPaired) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int nl = n0 + tx + 16 * j;
        const int jj = ((nl >> 6) << 5) + (nl & 31);
        if (jj < n_half) epi.pair(m, jj, acc[i][j], acc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx + 16 * j;
        if (n < N) epi(m, n, acc[i][j]);
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------------------
// Products y = A W^T (+ epilogue): one, or two with the same N, K and operand strides
// (A1, W1, M1, epi1) in one launch when the large-tile kernel takes them both, else one
// launch each.
template <class T, class Epi>
static hipError_t launch(const void* A, int64_t lda, const void* W, int64_t ldw, int M, int N,
                         int K, int n_half, const Epi& epi, hipStream_t s,
                         float* split_ws = nullptr, int kdup = 0, const void* A1 = nullptr,
                         const void* W1 = nullptr, int M1 = 0, const Epi* epi1 = nullptr) {
  if (M1 > 0 && M <= 0) return launch<T>(A1, lda, W1, ldw, M1, N, K, n_half, *epi1, s, split_ws, kdup);
  if (M <= 0 || N <= 0) return hipSuccess;
  const int kw = K - kdup;  // W columns; A columns past kw repeat W columns [kw - kdup, kw)
  if constexpr (sizeof(T) == 2) {
    // the large-tile kernel addresses operands with 32-bit byte offsets from their base
    const bool off32 = (int64_t)std::max(M, M1) * lda * 2 < (int64_t{1} << 32) &&
                       (int64_t)N * ldw * 2 < (int64_t{1} << 32);
    if (K % kBK == 0 && off32) {
      int best, best_split;
      pick_tile(M, N, K, kBK, 1.0, split_ws != nullptr, best, best_split, M1 > 0 ? M1 : 0);
      const GemmSeg<T, Epi> seg[2] = {
          {static_cast<const T*>(A), static_cast<const T*>(W), M, 0, epi},
          {static_cast<const T*>(M1 > 0 ? A1 : A), static_cast<const T*>(M1 > 0 ? W1 : W),
           M1 > 0 ? M1 : M, 0, M1 > 0 ? *epi1 : epi}};
      const int nseg = M1 > 0 ? 2 : 1;
      if (best == 0)
        return launch_lds<256, 256, 64, 2, 3, 16, 1, 4, 2>(seg, nseg, lda, ldw, N, K, kw, kdup,
                                                          n_half, best_split, split_ws, s);
      if (best == 1)
        return launch_lds<256, 128, 64, 2, 2, 16, 1, 4, 2>(seg, nseg, lda, ldw, N, K, kw, kdup,
                                                          n_half, best_split, split_ws, s);
      return launch_lds<128, 128, 64, 2, 2, 16, 2, 2, 2>(seg, nseg, lda, ldw, N, K, kw, kdup,
                                                        n_half, best_split, split_ws, s);
    }
  }
  if (M1 > 0) {
    hipError_t e = launch<T>(A, lda, W, ldw, M, N, K, n_half, epi, s, split_ws, kdup);
    if (e != hipSuccess) return e;
    return launch<T>(A1, lda, W1, ldw, M1, N, K, n_half, *epi1, s, split_ws, kdup);
  }
  if constexpr (sizeof(T) == 2) {
    constexpr int BM = 128, BN = 128;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const size_t lds = 2 * (BM + BN) * kBK * sizeof(T);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, Epi, T>), dim3(tiles_m * tiles_n), dim3(kThreads),
                       lds, s, static_cast<const T*>(A), lda, static_cast<const T*>(W), ldw,
                       M, N, K, kw, kdup, n_half, tiles_n, epi);
  } else {
    if (kdup) return hipErrorInvalidValue;  // hi / lo operands are a bf16-path feature
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL((gemm_f32_kernel<Epi>), grid, dim3(256), 0, s,
                       static_cast<const float*>(A), lda, static_cast<const float*>(W), ldw, M,
                       N, K, n_half, epi);
  }
  return hipGetLastError();
}

// Launch a's product (and b's, when given, in the same launch) with the epilogue that
// make(args) builds for each.
template <class T, class Make>
static hipError_t launch_args(const LinearArgs& a, const LinearArgs* b, int n_half, Make make,
                              hipStream_t s) {
  const auto e0 = make(a);
  if (!b)
    return launch<T>(a.x, a.ldx, a.w, a.ldw, a.m, a.n, a.k, n_half, e0, s, a.split_ws, a.kdup);
  const auto e1 = make(*b);
  return launch<T>(a.x, a.ldx, a.w, a.ldw, a.m, a.n, a.k, n_half, e0, s, a.split_ws, a.kdup, b->x,
                   b->w, b->m, &e1);
}

template <class T, class TY, class TR>
static hipError_t gated2(const LinearArgs& a, const LinearArgs* b, hipStream_t s) {
  return launch_args<T>(a, b, 0, [](const LinearArgs& q) {
    EpiGatedResid<TY, TR> epi{static_cast<TY*>(q.y), q.ldy, static_cast<const TR*>(q.resid),
                              q.ldr, q.gate, q.gate_bs, q.rows_per_batch};
    epi.set_vec();
    return epi;
  }, s);
}

template <class T>
static hipError_t gated(const LinearArgs& a, const LinearArgs* b, hipStream_t s) {
  if (a.y_dtype == DT_F32)
    return a.r_dtype == DT_F32 ? gated2<T, float, float>(a, b, s) : gated2<T, float, bf16>(a, b, s);
  return a.r_dtype == DT_F32 ? gated2<T, bf16, float>(a, b, s) : gated2<T, bf16, bf16>(a, b, s);
}

template <class T>
static hipError_t linear_t(const LinearArgs& a, const LinearArgs* b, hipStream_t s) {
  switch (a.epilogue) {
    case EPI_STORE:
      if (a.y_dtype == DT_F32)
        return launch_args<T>(a, b, 0, [](const LinearArgs& q) {
          EpiStore<float> epi{static_cast<float*>(q.y), q.ldy};
          epi.set_vec();
          return epi;
        }, s);
      return launch_args<T>(a, b, 0, [](const LinearArgs& q) {
        EpiStore<bf16> epi{static_cast<bf16*>(q.y), q.ldy};
        epi.set_vec();
        return epi;
      }, s);
    case EPI_SWIGLU:
      return launch_args<T>(a, b, a.n / 2, [](const LinearArgs& q) {
        return EpiSwiGLU<T>{static_cast<T*>(q.y), q.ldy, q.n / 2, q.swiglu_lo};
      }, s);
    case EPI_GATED_RESIDUAL:
      return gated<T>(a, b, s);
    case EPI_QKV:
      // q | k and V^T feed the attention: fp32 for fp32 operands, else bf16
      return launch_args<T>(a, b, 0, [](const LinearArgs& q) {
        using TQ = typename std::conditional<sizeof(T) == 4, float, bf16>::type;
        EpiQKV<TQ> epi{static_cast<TQ*>(q.y), q.ldy, static_cast<TQ*>(q.vt), q.ldvt,
                       2 * q.dim, q.dim, q.rows_per_batch, q.vt_off};
        epi.set_vec();
        return epi;
      }, s);
  }
  return hipErrorInvalidValue;
}

// fp8 linear: operands E4M3 with per-row scales (checked by the caller: K % 128 == 0,
// 32-bit byte offsets)
template <class Epi>
static hipError_t launch_fp8(const LinearArgs& a, const float* sa, const float* sw, int n_half,
                             const Epi& epi, hipStream_t s) {
  if (a.m <= 0 || a.n <= 0) return hipSuccess;
  int best, split;
  pick_tile(a.m, a.n, a.k, 128, 2.0, a.split_ws != nullptr, best, split);
  auto* x = static_cast<const fp8*>(a.x);
  auto* w = static_cast<const fp8*>(a.w);
  if (best == 0)
    return launch_lds_fp8<256, 256, 2, 1, 4, 2>(x, a.ldx, w, a.ldw, a.m, a.n, a.k, n_half, epi,
                                                 split, a.split_ws, sa, sw, s);
  if (best == 1)
    return launch_lds_fp8<256, 128, 2, 1, 4, 2>(x, a.ldx, w, a.ldw, a.m, a.n, a.k, n_half, epi,
                                                 split, a.split_ws, sa, sw, s);
  return launch_lds_fp8<128, 128, 2, 2, 2, 2>(x, a.ldx, w, a.ldw, a.m, a.n, a.k, n_half, epi,
                                               split, a.split_ws, sa, sw, s);
}

template <class TY, class TR>
static hipError_t gated_fp8(const LinearArgs& a, const float* sa, const float* sw, hipStream_t s) {
  EpiGatedResid<TY, TR> epi{static_cast<TY*>(a.y), a.ldy, static_cast<const TR*>(a.resid),
                            a.ldr, a.gate, a.gate_bs, a.rows_per_batch};
  epi.set_vec();
  return launch_fp8(a, sa, sw, 0, epi, s);
}

hipError_t linear_fp8(const LinearArgs& a, const float* sa, const float* sw, hipStream_t s) {
  switch (a.epilogue) {
    case EPI_STORE:
      if (a.y_dtype == DT_F32) {
        EpiStore<float> epi{static_cast<float*>(a.y), a.ldy};
        epi.set_vec();
        return launch_fp8(a, sa, sw, 0, epi, s);
      } else {
        EpiStore<bf16> epi{static_cast<bf16*>(a.y), a.ldy};
        epi.set_vec();
        return launch_fp8(a, sa, sw, 0, epi, s);
      }
    case EPI_SWIGLU:
      return launch_fp8(a, sa, sw, a.n / 2, EpiSwiGLU<bf16>{static_cast<bf16*>(a.y), a.ldy, a.n / 2},
                        s);
    case EPI_GATED_RESIDUAL:
      if (a.y_dtype == DT_F32)
        return a.r_dtype == DT_F32 ? gated_fp8<float, float>(a, sa, sw, s)
                                   : gated_fp8<float, bf16>(a, sa, sw, s);
      return a.r_dtype == DT_F32 ? gated_fp8<bf16, float>(a, sa, sw, s)
                                 : gated_fp8<bf16, bf16>(a, sa, sw, s);
  }
  return hipErrorInvalidValue;
}

size_t linear_splitk_bytes() { return kSplitkBytes; }

// Split-K scratch of flux_linear_noalloc: a fixed device array (each device that loads the
// library holds its own copy until the process ends), for callers that cannot allocate.
// Its size is the most the tile planner ever uses (kSplitkBytes), so every shape flux_linear
// accepts fits.  In host code `scratch` names a host-side stand-in, not the device
// array: the device address is resolved once per device with hipGetSymbolAddress (with
// that device current) and only that address is handed to kernels.
static __device__ __align__(256) char scratch[kSplitkBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];
}  // namespace

hipError_t linear_static_scratch(float** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_dev[dev] = p;
  }
  *ptr = static_cast<float*>(g_scratch_dev[dev]);
  *bytes = kSplitkBytes;
  return hipSuccess;
}

hipError_t linear(int dtype, const LinearArgs& a, hipStream_t s) {
  if (dtype == DT_F16) return linear_t<f16>(a, nullptr, s);
  return dtype == DT_BF16 ? linear_t<bf16>(a, nullptr, s) : linear_t<float>(a, nullptr, s);
}

hipError_t linear_pair(int dtype, const LinearArgs& a, const LinearArgs& b, hipStream_t s) {
  // one launch needs the same output width, depth, operand strides and epilogue kind
  const bool same = a.epilogue == b.epilogue && a.n == b.n && a.k == b.k && a.ldx == b.ldx &&
                    a.ldw == b.ldw && a.kdup == b.kdup && a.y_dtype == b.y_dtype &&
                    a.r_dtype == b.r_dtype && a.swiglu_lo == b.swiglu_lo && a.dim == b.dim;
  if (!same || a.m <= 0 || b.m <= 0) {
    hipError_t e = linear(dtype, a, s);
    if (e != hipSuccess) return e;
    return linear(dtype, b, s);
  }
  if (dtype == DT_F16) return linear_t<f16>(a, &b, s);
  return dtype == DT_BF16 ? linear_t<bf16>(a, &b, s) : linear_t<float>(a, &b, s);
}

}  // namespace flux
