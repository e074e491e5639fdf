// Bandwidth-bound fused kernels: LayerNorm + modulate, per-head RMSNorm + RoPE, and the
// RoPE position / angle table.
//
// LayerNorm + modulate ("双流块" AdaLN pre-norm of the Diffusers walk-through, eps 1e-6):
//   y = (1 + scale) * (x - mean) / sqrt(var + eps) + shift   (biased variance, no affine)
// One wave per row (two for fp32 rows of 6144 or more values): the row is held in
// registers (each lane moves 16 bytes of the input per chunk, so a wave instruction reads
// 1 KB contiguously), mean and variance are two exact passes over the registers with
// wave64 shuffle reductions.
//
// QK RMSNorm + RoPE ("双流块" norm_q / norm_k; "位置 id 的维度" per-axis rotary embedding,
// theta 2000, axes 32/32/32/32): 16 lanes own one (token, head) vector of 128 values;
// x / sqrt(mean(x^2) + eps) * gamma, then adjacent pairs (2p, 2p+1) rotate by the angle
// read from the (cos, sin) table built once per call from the integer ids.
#include "common.h"
#include "kernels.h"

namespace flux {

// ---- 8-element chunk I/O for bf16 / fp32 --------------------------------------------
template <class T>
FLUX_DEV void load8(const T* p, float* f);
template <>
FLUX_DEV void load8<bf16>(const bf16* p, float* f) {
  unpack8(ld16(p), f);
}
template <>
FLUX_DEV void load8<float>(const float* p, float* f) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
template <class T>
FLUX_DEV void store8(T* p, const float* f);
template <>
FLUX_DEV void store8<bf16>(bf16* p, const float* f) {
  st16(p, pack8(f));
}
template <>
FLUX_DEV void store8<f16>(f16* p, const float* f) {
  st16(p, pack8_as<f16>(f));
}
template <>
FLUX_DEV void store8<float>(float* p, const float* f) {
  *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(f[4], f[5], f[6], f[7]);
}

// Streaming load of a residual-stream row (fp32, read once here; marked for early
// eviction).  Measured from HBM at 4608 x 4096: 26.0 -> 22.4 us; the step is unchanged.
// The outputs keep normal stores: the next GEMM reads them many times from L2 / MALL.
FLUX_DEV float4 ld_stream4(const float4* p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

// Streaming load of 8 bf16 / fp32 values that a kernel reads once (q and k rows before the
// in-place RMSNorm + RoPE).  Measured from HBM at 4608 tokens x 32 heads: 36.7 -> 34.1 us;
// at 48 heads (the per-(token, head) kernel) it was 3% slower, so that kernel keeps plain
// loads.
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
template <class T>
FLUX_DEV void load8_stream(const T* p, float* f);
template <>
FLUX_DEV void load8_stream<bf16>(const bf16* p, float* f) {
  const u32x4s v = __builtin_nontemporal_load(reinterpret_cast<const u32x4s*>(p));
  unpack8(make_uint4(v[0], v[1], v[2], v[3]), f);
}
template <>
FLUX_DEV void load8_stream<float>(const float* p, float* f) {
  const float4 a = ld_stream4(reinterpret_cast<const float4*>(p));
  const float4 b = ld_stream4(reinterpret_cast<const float4*>(p + 4));
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// ------------------------------------------------------------------------------------
// LayerNorm + modulate
// ------------------------------------------------------------------------------------
// CW-element chunk I/O: a lane moves 16 bytes of the input type per chunk (CW = 4 fp32 or
// 8 bf16), so each wave instruction reads 1 KB contiguously.
template <class T, int CW>
FLUX_DEV void load_cw(const T* p, float* f) {
  if constexpr (CW == 8) {
    load8(p, f);
  } else {
    static_assert(sizeof(T) == 4 && CW == 4, "fp32 chunks of 4");
    const float4 a = *reinterpret_cast<const float4*>(p);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  }
}
template <class T, int CW>
FLUX_DEV void store_cw(T* p, const float* f) {
  if constexpr (CW == 8) {
    store8(p, f);
  } else if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack2_as<T>(f[0], f[1]), pack2_as<T>(f[2], f[3]));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
}
FLUX_DEV void load_mod(const float* p, float* f, int n) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  if (n == 8) {
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
}

// HILO: the output is carried at twice bf16's precision as a pair of bf16 planes in one
// row, hi = bf16(y) at columns [0, dim) and lo = bf16(y - hi) at [dim, 2 dim), so that a
// bf16 product over K = 2 dim against [W | W] gives y W^T to fp32 accumulation (TY = bf16).
template <class TX, class TY, int MAXI, bool EXACT, bool HILO = false>
__global__ __launch_bounds__(256) void ln_modulate_kernel(const TX* __restrict__ x, int64_t ldx,
                                                          TY* __restrict__ y, int64_t ldy,
                                                          int rows, int dim, int rpb,
                                                          const float* __restrict__ shift,
                                                          const float* __restrict__ scale,
                                                          int64_t mod_bs, float eps) {
  constexpr int CW = 16 / sizeof(TX);  // elements per lane chunk
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nch = dim / CW;
  const TX* xr = x + (int64_t)row * ldx;
  float v[MAXI][CW];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + 64 * i;
    if (EXACT || c < nch) {
      load_cw<TX, CW>(xr + c * CW, v[i]);
#pragma unroll
      for (int e = 0; e < CW; ++e) s += v[i][e];
    }
  }
  const float mean = wave_sum(s) / dim;
  float q = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + 64 * i;
    if (EXACT || c < nch) {
#pragma unroll
      for (int e = 0; e < CW; ++e) {
        v[i][e] -= mean;
        q += v[i][e] * v[i][e];
      }
    }
  }
  const float rstd = rsqrtf(wave_sum(q) / dim + eps);
  const int b = row / rpb;
  const float* sh = shift + b * mod_bs;
  const float* sc = scale + b * mod_bs;
  TY* yr = y + (int64_t)row * ldy;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int c = lane + 64 * i;
    if (EXACT || c < nch) {
      float a[CW], m[CW], o[CW];
      load_mod(sh + c * CW, a, CW);
      load_mod(sc + c * CW, m, CW);
#pragma unroll
      for (int e = 0; e < CW; ++e) o[e] = (1.f + m[e]) * (v[i][e] * rstd) + a[e];
      if constexpr (HILO) {
        static_assert(sizeof(TY) == 2, "hi/lo planes are bf16");
        // hi is exactly representable, so its store does not round again; o - hi is exact
        // in fp32 and lo rounds it to bf16
        float hi[CW], lo[CW];
#pragma unroll
        for (int e = 0; e < CW; ++e) {
          hi[e] = to_f32(from_f32<bf16>(o[e]));
          lo[e] = o[e] - hi[e];
        }
        store_cw<TY, CW>(yr + c * CW, hi);
        store_cw<TY, CW>(yr + dim + c * CW, lo);
      } else {
        store_cw<TY, CW>(yr + c * CW, o);
      }
    }
  }
}

// fp32 rows of exactly 256 J values (the residual stream), wide rows (J >= 24): two waves
// per row, each holding half of it (lane l of half h holds the float4s
// 4 (h 32 J + l + 64 j), j < J / 2, so every load instruction reads 1 KB contiguously).
// The halves' sums meet in LDS and are added in a fixed order (half 0 + half 1), so both
// waves compute the same mean and rstd. A whole row per wave needs 208 VGPRs at J = 24
// (2 waves per SIMD); half a row needs 114 (4 waves per SIMD).
template <class TY, int J>
__global__ __launch_bounds__(256) void ln_modulate_f32_split_kernel(
    const float* __restrict__ x, int64_t ldx, TY* __restrict__ y, int64_t ldy, int rows, int rpb,
    const float* __restrict__ shift, const float* __restrict__ scale, int64_t mod_bs, float eps) {
  constexpr int D = 256 * J, JH = J / 2;
  __shared__ float part[2][4];  // [sum | centred sum of squares][wave]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, half = w & 1;
  const int row = blockIdx.x * 2 + (w >> 1);
  // a wave past the last row reads that row and stores nothing (it still meets the barriers)
  const float4* xr =
      reinterpret_cast<const float4*>(x + (int64_t)min(row, rows - 1) * ldx) + half * 64 * JH;
  float4 v[JH];
#pragma unroll
  for (int j = 0; j < JH; ++j) v[j] = ld_stream4(xr + lane + 64 * j);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < JH; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  s = wave_sum(s);
  if (lane == 0) part[0][w] = s;
  __syncthreads();
  const float mean = (part[0][w & 2] + part[0][w | 1]) * (1.f / D);
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < JH; ++j) {
    v[j].x -= mean;
    v[j].y -= mean;
    v[j].z -= mean;
    v[j].w -= mean;
    q += (v[j].x * v[j].x + v[j].y * v[j].y) + (v[j].z * v[j].z + v[j].w * v[j].w);
  }
  q = wave_sum(q);
  if (lane == 0) part[1][w] = q;
  __syncthreads();
  const float rstd = rsqrtf((part[1][w & 2] + part[1][w | 1]) * (1.f / D) + eps);
  if (row >= rows) return;
  const int b = row / rpb;
  const float4* sh = reinterpret_cast<const float4*>(shift + b * mod_bs) + half * 64 * JH;
  const float4* sc = reinterpret_cast<const float4*>(scale + b * mod_bs) + half * 64 * JH;
  TY* yr = y + (int64_t)row * ldy + half * 256 * JH;
#pragma unroll
  for (int j = 0; j < JH; ++j) {
    const int c = lane + 64 * j;
    const float4 a = sh[c], m = sc[c];
    float o[4] = {(1.f + m.x) * (v[j].x * rstd) + a.x, (1.f + m.y) * (v[j].y * rstd) + a.y,
                  (1.f + m.z) * (v[j].z * rstd) + a.z, (1.f + m.w) * (v[j].w * rstd) + a.w};
    store_cw<TY, 4>(yr + 4 * c, o);
    // the modulation vectors' loads are issued 4 chunks at a time, not all hoisted ahead
    // of the loop (that would cost the registers the split saves)
    if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
}

// The same rows for J <= 16 (the Klein widths), one wave per row: lane l holds the
// float4s 4 (l + 64 j), j < J. Here the row fits one wave at 5-6 waves per SIMD, and this
// form beats the two-wave split at the step's 4608 rows. The workgroups
// are laid out per batch item (rows_per_batch / 4 of them, rounded up, for each item), so
// the 4 rows of one workgroup share one shift / scale pair, which is staged in LDS while
// the rows' loads are in flight. Reading the modulation from LDS instead of holding it in
// registers leaves room for 5 waves per SIMD at J = 16 (4 with the vectors in registers).
template <class TY, int J>
__global__ __launch_bounds__(256) void ln_modulate_f32_kernel(const float* __restrict__ x,
                                                              int64_t ldx, TY* __restrict__ y,
                                                              int64_t ldy, int rows, int rpb,
                                                              int wg_per_item,
                                                              const float* __restrict__ shift,
                                                              const float* __restrict__ scale,
                                                              int64_t mod_bs, float eps) {
  constexpr int D = 256 * J;
  __shared__ float4 mod_shift[D / 4], mod_scale[D / 4];
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x / wg_per_item;
  const int r = (blockIdx.x % wg_per_item) * 4 + (threadIdx.x >> 6);  // row within the item
  const int row = item * rpb + r;
  const bool live = r < rpb && row < rows;  // wave-uniform; a dead wave reads the item's first row
  const float4* xr = reinterpret_cast<const float4*>(x + (int64_t)(live ? row : item * rpb) * ldx);
  float4 v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = ld_stream4(xr + lane + 64 * j);
  const float4* sh = reinterpret_cast<const float4*>(shift + item * mod_bs);
  const float4* sc = reinterpret_cast<const float4*>(scale + item * mod_bs);
  for (int c = threadIdx.x; c < D / 4; c += 256) {
    mod_shift[c] = sh[c];
    mod_scale[c] = sc[c];
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) s += (v[j].x + v[j].y) + (v[j].z + v[j].w);
  const float mean = wave_sum(s) * (1.f / D);
  float q = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    v[j].x -= mean;
    v[j].y -= mean;
    v[j].z -= mean;
    v[j].w -= mean;
    q += (v[j].x * v[j].x + v[j].y * v[j].y) + (v[j].z * v[j].z + v[j].w * v[j].w);
  }
  const float rstd = rsqrtf(wave_sum(q) * (1.f / D) + eps);
  __syncthreads();
  if (!live) return;
  TY* yr = y + (int64_t)row * ldy;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = lane + 64 * j;
    const float4 a = mod_shift[c], m = mod_scale[c];
    float o[4] = {(1.f + m.x) * (v[j].x * rstd) + a.x, (1.f + m.y) * (v[j].y * rstd) + a.y,
                  (1.f + m.z) * (v[j].z * rstd) + a.z, (1.f + m.w) * (v[j].w * rstd) + a.w};
    store_cw<TY, 4>(yr + 4 * c, o);
  }
}

template <class TX, class TY>
static hipError_t ln_dispatch(const void* x, int64_t ldx, void* y, int64_t ldy, int rows, int dim,
                              int rpb, const float* shift, const float* scale, int64_t mod_bs,
                              float eps, hipStream_t s) {
  constexpr int CW = 16 / sizeof(TX);
  const int per_lane = (dim / CW + 63) / 64;
  dim3 grid((rows + 3) / 4), block(256);
  auto* xp = static_cast<const TX*>(x);
  auto* yp = static_cast<TY*>(y);
  if constexpr (sizeof(TX) == 4) {
    // rows of one batch item: a row count past the last item's end only shortens that item
    const int per_item = rpb < rows ? rpb : rows;
    const int items = (rows + per_item - 1) / per_item, wg_per_item = (per_item + 3) / 4;
#define FLUX_LN32(J)                                                                         \
  if (dim == 256 * J) {                                                                     \
    hipLaunchKernelGGL((ln_modulate_f32_kernel<TY, J>), dim3(items * wg_per_item), block, 0, \
                       s, xp, ldx, yp, ldy, rows, per_item, wg_per_item, shift, scale,      \
                       mod_bs, eps);                                                        \
    return hipGetLastError();                                                              \
  }
#define FLUX_LN32S(J)                                                                       \
  if (dim == 256 * J) {                                                                     \
    hipLaunchKernelGGL((ln_modulate_f32_split_kernel<TY, J>), dim3((rows + 1) / 2), block, 0, \
                       s, xp, ldx, yp, ldy, rows, rpb, shift, scale, mod_bs, eps);          \
    return hipGetLastError();                                                              \
  }
    FLUX_LN32(12) FLUX_LN32(16) FLUX_LN32S(24) FLUX_LN32S(32)
#undef FLUX_LN32S
#undef FLUX_LN32
  }
  // rows that fill whole sets of 64 chunks (every traced width) take the unguarded kernel
  const bool exact = (dim / CW) % 64 == 0;
#define FLUX_LN(N)                                                                           \
  do {                                                                                      \
    if (exact && (dim / CW) == 64 * N)                                                      \
      hipLaunchKernelGGL((ln_modulate_kernel<TX, TY, N, true>), grid, block, 0, s, xp, ldx, \
                         yp, ldy, rows, dim, rpb, shift, scale, mod_bs, eps);               \
    else                                                                                    \
      hipLaunchKernelGGL((ln_modulate_kernel<TX, TY, N, false>), grid, block, 0, s, xp,     \
                         ldx, yp, ldy, rows, dim, rpb, shift, scale, mod_bs, eps);          \
  } while (0)
  if (per_lane <= 1) FLUX_LN(1);
  else if (per_lane <= 2) FLUX_LN(2);
  else if (per_lane <= 4) FLUX_LN(4);
  else if (per_lane <= 8) FLUX_LN(8);
  else if (per_lane <= 12) FLUX_LN(12);
  else if (per_lane <= 16) FLUX_LN(16);
  else if (per_lane <= 24) FLUX_LN(24);
  else if (per_lane <= 32) FLUX_LN(32);
  else return hipErrorInvalidValue;
#undef FLUX_LN
  return hipGetLastError();
}

hipError_t layernorm_modulate(int x_dtype, int y_dtype, const void* x, int64_t ldx, void* y,
                              int64_t ldy, int rows, int dim, int rpb, const float* shift,
                              const float* scale, int64_t mod_bs, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (y_dtype == DT_F16)  // binary16 outputs (the inputs of binary16 products)
    return x_dtype == DT_BF16
               ? ln_dispatch<bf16, f16>(x, ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps, s)
               : ln_dispatch<float, f16>(x, ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps, s);
  if (x_dtype == DT_BF16)
    return y_dtype == DT_BF16
               ? ln_dispatch<bf16, bf16>(x, ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps, s)
               : ln_dispatch<bf16, float>(x, ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps, s);
  return y_dtype == DT_BF16
             ? ln_dispatch<float, bf16>(x, ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps, s)
             : ln_dispatch<float, float>(x, ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps, s);
}

template <class TX>
static hipError_t ln_hilo_dispatch(const TX* x, int64_t ldx, bf16* y, int64_t ldy, int rows,
                                   int dim, int rpb, const float* shift, const float* scale,
                                   int64_t mod_bs, float eps, hipStream_t s) {
  constexpr int CW = 16 / sizeof(TX);
  const int per_lane = (dim / CW + 63) / 64;
  const bool exact = (dim / CW) % 64 == 0;
  dim3 grid((rows + 3) / 4), block(256);
#define FLUX_LNH(N)                                                                            \
  do {                                                                                        \
    if (exact && (dim / CW) == 64 * N)                                                        \
      hipLaunchKernelGGL((ln_modulate_kernel<TX, bf16, N, true, true>), grid, block, 0, s, x, \
                         ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps);             \
    else                                                                                      \
      hipLaunchKernelGGL((ln_modulate_kernel<TX, bf16, N, false, true>), grid, block, 0, s,   \
                         x, ldx, y, ldy, rows, dim, rpb, shift, scale, mod_bs, eps);          \
  } while (0)
  if (per_lane <= 2) FLUX_LNH(2);
  else if (per_lane <= 4) FLUX_LNH(4);
  else if (per_lane <= 8) FLUX_LNH(8);
  else if (per_lane <= 16) FLUX_LNH(16);
  else if (per_lane <= 24) FLUX_LNH(24);
  else if (per_lane <= 32) FLUX_LNH(32);
  else return hipErrorInvalidValue;
#undef FLUX_LNH
  return hipGetLastError();
}

hipError_t layernorm_modulate_hilo(int x_dtype, const void* x, int64_t ldx, void* y, int64_t ldy,
                                   int rows, int dim, int rpb, const float* shift,
                                   const float* scale, int64_t mod_bs, float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  bf16* yp = static_cast<bf16*>(y);
  if (x_dtype == DT_BF16)
    return ln_hilo_dispatch(static_cast<const bf16*>(x), ldx, yp, ldy, rows, dim, rpb, shift,
                            scale, mod_bs, eps, s);
  return ln_hilo_dispatch(static_cast<const float*>(x), ldx, yp, ldy, rows, dim, rpb, shift,
                          scale, mod_bs, eps, s);
}

// ------------------------------------------------------------------------------------
// RoPE table: integer positions and (cos, sin) of the angles, joint order [txt ; img]
// ------------------------------------------------------------------------------------
__global__ void rope_table_kernel(const int32_t* __restrict__ txt_ids,
                                  const int32_t* __restrict__ img_ids, int n_txt, int n_img,
                                  int4 axes, float theta, int32_t* __restrict__ pos,
                                  float2* __restrict__ cs) {
  constexpr int P = 64;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int L = n_txt + n_img;
  if (idx >= L * P) return;
  const int j = idx / P, p = idx % P;
  // axis a owns pairs [c_a, c_a + d_a / 2)
  const int d[4] = {axes.x, axes.y, axes.z, axes.w};
  int a = 0, first = 0;
  while (a < 3 && p >= first + d[a] / 2) {
    first += d[a] / 2;
    ++a;
  }
  const int jl = p - first;
  const int32_t* row = (j < n_txt) ? (txt_ids + (int64_t)j * 4) : (img_ids + (int64_t)(j - n_txt) * 4);
  const int32_t ps = row[a];
  pos[idx] = ps;
  if (!cs) return;  // positions only
  const double omega = pow((double)theta, -2.0 * jl / (double)d[a]);
  const double phi = (double)ps * omega;
  cs[idx] = make_float2((float)cos(phi), (float)sin(phi));
}

hipError_t rope_table(const int32_t* txt_ids, const int32_t* img_ids, int n_txt, int n_img,
                      const int32_t* axes_dim, float theta, int32_t* pos, float2* cs,
                      hipStream_t s) {
  const int total = (n_txt + n_img) * 64;
  if (total <= 0) return hipSuccess;
  int4 axes = make_int4(axes_dim[0], axes_dim[1], axes_dim[2], axes_dim[3]);
  hipLaunchKernelGGL(rope_table_kernel, dim3((total + 255) / 256), dim3(256), 0, s, txt_ids,
                     img_ids, n_txt, n_img, axes, theta, pos, cs);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// QK RMSNorm + RoPE, in place
// ------------------------------------------------------------------------------------
template <class T>
FLUX_DEV T* seq_ptr(const SeqView& v, int b, int j) {
  return (j < v.n0) ? static_cast<T*>(v.base0) + b * v.bs0 + (int64_t)j * v.ld
                    : static_cast<T*>(v.base1) + b * v.bs1 + (int64_t)(j - v.n0) * v.ld;
}

template <class T>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(SeqView q, SeqView k, int batch,
                                                           int seq, int heads,
                                                           const float* __restrict__ qg0,
                                                           const float* __restrict__ kg0,
                                                           const float* __restrict__ qg1,
                                                           const float* __restrict__ kg1,
                                                           const float2* __restrict__ cs,
                                                           float eps) {
  const int l16 = threadIdx.x & 15;
  const int64_t unit = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int64_t total = (int64_t)batch * seq * heads * 2;
  if (unit >= total) return;
  const int which = unit & 1;                 // 0 = q, 1 = k
  const int64_t th = unit >> 1;
  const int head = th % heads;
  const int64_t bj = th / heads;
  const int j = bj % seq;
  const int b = bj / seq;
  const SeqView& v = which ? k : q;
  const bool seg1 = j >= v.n0;
  const float* g = which ? (seg1 ? kg1 : kg0) : (seg1 ? qg1 : qg0);
  T* p = seq_ptr<T>(v, b, j) + head * 128 + l16 * 8;
  float x[8], gm[8];
  load8(p, x);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
  const float r = rsqrtf(group_sum16(ss) * (1.f / 128.f) + eps);
  load8(g + l16 * 8, gm);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = x[e] * r * gm[e];
  const float4* c4 = reinterpret_cast<const float4*>(cs + (int64_t)j * 64 + l16 * 4);
  const float4 c01 = c4[0], c23 = c4[1];
  const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
  const float sn[4] = {c01.y, c01.w, c23.y, c23.w};
  float o[8];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    o[2 * t] = x[2 * t] * cc[t] - x[2 * t + 1] * sn[t];
    o[2 * t + 1] = x[2 * t] * sn[t] + x[2 * t + 1] * cc[t];
  }
  store8(p, o);
}

// One workgroup per token: thread t owns chunks c = t + 256 i, i < NI, of the token's
// [q | k] (8 values each); c % 16 == t % 16, so the thread's (cos, sin) slice of the token
// and its position in every head are fixed, and the angle table row is read once per
// token. All NI chunks are loaded before the first is normalised, so NI loads per thread
// are in flight at once. Unless the chunks fill all NI rounds (EXACT: heads % 8 == 0), those
// past the token's 2 * heads * 16 (whole 32-lane groups) are computed on zeros, not stored.
template <class T, int NI, bool EXACT>
__global__ __launch_bounds__(256) void qk_norm_rope_token_kernel(
    SeqView q, SeqView k, int batch, int seq, int heads, const float* __restrict__ qg0,
    const float* __restrict__ kg0, const float* __restrict__ qg1, const float* __restrict__ kg1,
    const float2* __restrict__ cs, float eps) {
  const int l16 = threadIdx.x & 15;
  const int qchunks = heads * 16, nch = 2 * qchunks;
  const int64_t token = blockIdx.x;
  const int j = token % seq, b = token / seq;
  const float4* c4 = reinterpret_cast<const float4*>(cs + (int64_t)j * 64 + l16 * 4);
  const float4 c01 = c4[0], c23 = c4[1];
  const float cc[4] = {c01.x, c01.z, c23.x, c23.z};
  const float sn[4] = {c01.y, c01.w, c23.y, c23.w};
  float x[NI][8];
  T* ptr[NI];
  const float* gam[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = threadIdx.x + 256 * i;
    const int which = c >= qchunks;
    const int head = (c - which * qchunks) >> 4;
    const SeqView& v = which ? k : q;
    const bool seg1 = j >= v.n0;
    gam[i] = which ? (seg1 ? kg1 : kg0) : (seg1 ? qg1 : qg0);
    ptr[i] = seq_ptr<T>(v, b, j) + head * 128 + l16 * 8;
    if (EXACT || c < nch) {
      load8_stream(ptr[i], x[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
    }
  }
  float gm[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i) load8(gam[i] + l16 * 8, gm[i]);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[i][e] * x[i][e];
    const float r = rsqrtf(group_sum16(ss) * (1.f / 128.f) + eps);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[i][e] = x[i][e] * r * gm[i][e];
    float o[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      o[2 * t] = x[i][2 * t] * cc[t] - x[i][2 * t + 1] * sn[t];
      o[2 * t + 1] = x[i][2 * t] * sn[t] + x[i][2 * t + 1] * cc[t];
    }
    if (EXACT || threadIdx.x + 256 * i < nch) store8(ptr[i], o);
  }
}

hipError_t qk_norm_rope(int dtype, SeqView q, SeqView k, int batch, int seq, int heads,
                        const float* qg0, const float* kg0, const float* qg1, const float* kg1,
                        const float2* cs, float eps, hipStream_t s) {
  const int64_t units = (int64_t)batch * seq * heads * 2;
  if (units <= 0) return hipSuccess;
  // measured on MI355X: the per-token kernel is faster up to 32 heads (4 chunks per
  // thread), the per-(token, head) one above (at 48 heads and 16896 tokens by 8%)
  if (heads <= 32) {
    dim3 grid((unsigned)((int64_t)batch * seq)), block(256);
    const int ni = (heads + 7) / 8;  // chunks per thread: 2 * heads * 16 over 256 threads
    const bool exact = heads % 8 == 0;
#define FLUX_QKT(NI, EX)                                                                      \
  if (ni == NI && exact == EX) {                                                             \
    if (dtype == DT_BF16)                                                                    \
      hipLaunchKernelGGL((qk_norm_rope_token_kernel<bf16, NI, EX>), grid, block, 0, s, q, k,  \
                         batch, seq, heads, qg0, kg0, qg1, kg1, cs, eps);                   \
    else                                                                                     \
      hipLaunchKernelGGL((qk_norm_rope_token_kernel<float, NI, EX>), grid, block, 0, s, q, k, \
                         batch, seq, heads, qg0, kg0, qg1, kg1, cs, eps);                   \
    return hipGetLastError();                                                               \
  }
    FLUX_QKT(1, true) FLUX_QKT(2, true) FLUX_QKT(3, true) FLUX_QKT(4, true)
    FLUX_QKT(1, false) FLUX_QKT(2, false) FLUX_QKT(3, false) FLUX_QKT(4, false)
#undef FLUX_QKT
  }
  dim3 grid((units + 15) / 16), block(256);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(qk_norm_rope_kernel<bf16>, grid, block, 0, s, q, k, batch, seq, heads, qg0,
                       kg0, qg1, kg1, cs, eps);
  else
    hipLaunchKernelGGL(qk_norm_rope_kernel<float>, grid, block, 0, s, q, k, batch, seq, heads, qg0,
                       kg0, qg1, kg1, cs, eps);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------
// Row copies between joint-sequence views (merge / split of the streams)
// ------------------------------------------------------------------------------------
template <class TS, class TD>
__global__ void copy_rows_kernel(SeqView src, SeqView dst, int batch, int seq, int dim) {
  const int nch = dim >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)batch * seq * nch) return;
  const int c = idx % nch;
  const int64_t bj = idx / nch;
  const int j = bj % seq, b = bj / seq;
  float f[8];
  load8(seq_ptr<TS>(src, b, j) + c * 8, f);
  store8(seq_ptr<TD>(dst, b, j) + c * 8, f);
}

hipError_t copy_rows(int src_dtype, SeqView src, int dst_dtype, SeqView dst, int batch, int seq,
                     int dim, hipStream_t s) {
  const int64_t total = (int64_t)batch * seq * (dim / 8);
  if (total <= 0) return hipSuccess;
  dim3 grid((total + 255) / 256), block(256);
  if (src_dtype == DT_BF16 && dst_dtype == DT_BF16)
    hipLaunchKernelGGL((copy_rows_kernel<bf16, bf16>), grid, block, 0, s, src, dst, batch, seq, dim);
  else if (src_dtype == DT_BF16)
    hipLaunchKernelGGL((copy_rows_kernel<bf16, float>), grid, block, 0, s, src, dst, batch, seq, dim);
  else if (dst_dtype == DT_BF16)
    hipLaunchKernelGGL((copy_rows_kernel<float, bf16>), grid, block, 0, s, src, dst, batch, seq, dim);
  else
    hipLaunchKernelGGL((copy_rows_kernel<float, float>), grid, block, 0, s, src, dst, batch, seq, dim);
  return hipGetLastError();
}

}  // namespace flux
