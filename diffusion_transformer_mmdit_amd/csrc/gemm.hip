// Linear layers y = x W^T (W stored [N, K] row-major) with fused epilogues.
//
// bf16 path: gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation.  Each workgroup
// (4 waves) computes a BM x BN tile; operands are staged through LDS in 64-wide K
// slices, double buffered, with an XOR swizzle of the 16-byte chunks so the MFMA
// fragment reads are bank-conflict free.  Global loads of the next slice are issued
// before the MFMAs of the current one.
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

namespace flux {

// ------------------------------------------------------------------------------------
// Epilogue functors: called once per output element (m < M, n < N checked by caller)
// ------------------------------------------------------------------------------------
template <class TY>
struct EpiStore {
  TY* y;
  int64_t ldy;
  static constexpr bool kPaired = false;
  FLUX_DEV void operator()(int m, int n, float v) const { y[m * ldy + n] = from_f32<TY>(v); }
};

template <class TY>
struct EpiSwiGLU {
  TY* y;
  int64_t ldy;
  int n_half;  // H
  static constexpr bool kPaired = true;
  // logical column n of the interleaved [gate | up] tile -> physical W row
  FLUX_DEV static int phys_row(int n, int H) {
    const int j = ((n >> 6) << 5) + (n & 31);
    return ((n >> 5) & 1) ? H + j : j;
  }
  FLUX_DEV void pair(int m, int j, float g, float u) const {
    y[m * ldy + j] = from_f32<TY>(silu_f(g) * u);
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
  static constexpr bool kPaired = false;
  FLUX_DEV void operator()(int m, int n, float v) const {
    const int b = m / rpb;
    y[m * ldy + n] = from_f32<TY>(to_f32(r[m * ldr + n]) + gate[b * gate_bs + n] * v);
  }
};

// ------------------------------------------------------------------------------------
// bf16 MFMA kernel
// ------------------------------------------------------------------------------------
constexpr int kBK = 64;  // K slice
constexpr int kThreads = 256;

// element offset of (row, 16-byte chunk c) in a [rows][64] bf16 LDS tile
FLUX_DEV int swz(int row, int c) { return row * kBK + ((c ^ (row & 7)) << 3); }

template <int BM, int BN, class Epi>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(const bf16* __restrict__ A,
                                                             int64_t lda,
                                                             const bf16* __restrict__ W,
                                                             int64_t ldw, int M, int N, int K,
                                                             int n_half, int tiles_n, Epi epi) {
  constexpr int WGM = 2, WGN = 2;                // 2 x 2 waves
  constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave tile
  constexpr int TM = WTM / 32, TN = WTN / 32;    // 32x32 MFMA tiles per wave
  constexpr int LA = BM * 8 / kThreads;          // 16-byte chunks per thread (A)
  constexpr int LB = BN * 8 / kThreads;
  static_assert(LA >= 1 && LB >= 1, "tile too small");
  static_assert(!Epi::kPaired || (TN % 2 == 0), "SwiGLU needs gate/up tile pairs");

  extern __shared__ __align__(16) bf16 smem[];
  bf16* As = smem;                   // [2][BM][64]
  bf16* Bs = smem + 2 * BM * kBK;    // [2][BN][64]

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
  const bf16* a_src[LA];
  bool a_ok[LA];
  int a_lds[LA];
  const bf16* b_src[LB];
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
#pragma unroll
    for (int i = 0; i < LA; ++i)
      ra[i] = (a_ok[i] && kin) ? ld16(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      rb[i] = (b_ok[i] && kin) ? ld16(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
  };
  auto store_slice = [&](int buf) {
    bf16* as = As + buf * BM * kBK;
    bf16* bs = Bs + buf * BN * kBK;
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
    const bf16* as = As + cur * BM * kBK;
    const bf16* bs = Bs + cur * BN * kBK;
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * WTM + i * 32 + lrow;
        af[i] = *reinterpret_cast<const bf16x8*>(as + swz(r, kk * 2 + lk));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wn * WTN + j * 32 + lrow;
        bfr[j] = *reinterpret_cast<const bf16x8*>(bs + swz(r, kk * 2 + lk));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
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
template <class T, class Epi>
static hipError_t launch(const void* A, int64_t lda, const void* W, int64_t ldw, int M, int N,
                         int K, int n_half, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if constexpr (sizeof(T) == 2) {
    constexpr int BM = 128, BN = 128;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const size_t lds = 2 * (BM + BN) * kBK * sizeof(bf16);
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, Epi>), dim3(tiles_m * tiles_n), dim3(kThreads),
                       lds, s, static_cast<const bf16*>(A), lda, static_cast<const bf16*>(W), ldw,
                       M, N, K, n_half, tiles_n, epi);
  } else {
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL((gemm_f32_kernel<Epi>), grid, dim3(256), 0, s,
                       static_cast<const float*>(A), lda, static_cast<const float*>(W), ldw, M,
                       N, K, n_half, epi);
  }
  return hipGetLastError();
}

template <class T, class TY, class TR>
static hipError_t gated2(const LinearArgs& a, hipStream_t s) {
  return launch<T>(a.x, a.ldx, a.w, a.ldw, a.m, a.n, a.k, 0,
                   EpiGatedResid<TY, TR>{static_cast<TY*>(a.y), a.ldy,
                                         static_cast<const TR*>(a.resid), a.ldr, a.gate,
                                         a.gate_bs, a.rows_per_batch},
                   s);
}

template <class T>
static hipError_t gated(const LinearArgs& a, hipStream_t s) {
  if (a.y_dtype == DT_F32)
    return a.r_dtype == DT_F32 ? gated2<T, float, float>(a, s) : gated2<T, float, bf16>(a, s);
  return a.r_dtype == DT_F32 ? gated2<T, bf16, float>(a, s) : gated2<T, bf16, bf16>(a, s);
}

template <class T>
static hipError_t linear_t(const LinearArgs& a, hipStream_t s) {
  switch (a.epilogue) {
    case EPI_STORE:
      if (a.y_dtype == DT_F32)
        return launch<T>(a.x, a.ldx, a.w, a.ldw, a.m, a.n, a.k, 0,
                         EpiStore<float>{static_cast<float*>(a.y), a.ldy}, s);
      return launch<T>(a.x, a.ldx, a.w, a.ldw, a.m, a.n, a.k, 0,
                       EpiStore<bf16>{static_cast<bf16*>(a.y), a.ldy}, s);
    case EPI_SWIGLU:
      return launch<T>(a.x, a.ldx, a.w, a.ldw, a.m, a.n, a.k, a.n / 2,
                       EpiSwiGLU<T>{static_cast<T*>(a.y), a.ldy, a.n / 2}, s);
    case EPI_GATED_RESIDUAL:
      return gated<T>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t linear(int dtype, const LinearArgs& a, hipStream_t s) {
  return dtype == DT_BF16 ? linear_t<bf16>(a, s) : linear_t<float>(a, s);
}

}  // namespace flux
