// Conditioning path: timestep sinusoid and the HBM-bound matrix-vector products of the
// MLPEmbedder and the AdaLN modulation linears ("时间步缩放" and "双流块 / 单流块" of the
// Diffusers walk-through; "条件注入" of the FLUX.2 [klein] note: 256-channel sinusoid of
// 1000 t, then MLPEmbedder, then modulation = Linear(silu(temb))).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace flux {

// e[b, k] = cos(1000 t_b f_k), e[b, half + k] = sin(1000 t_b f_k), f_k = 10000^(-k/half);
// evaluated in double precision (arguments reach 1000 rad).
__global__ void sinusoid_kernel(const float* __restrict__ t, int batch, int half,
                                float* __restrict__ e) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= batch * half) return;
  const int b = idx / half, k = idx % half;
  const double tau = 1000.0 * (double)t[b];
  const double f = pow(10000.0, -(double)k / (double)half);
  const double a = tau * f;
  e[(int64_t)b * 2 * half + k] = (float)cos(a);
  e[(int64_t)b * 2 * half + half + k] = (float)sin(a);
}

hipError_t timestep_sinusoid(const float* t, int batch, int half, float* e, hipStream_t s) {
  const int total = batch * half;
  hipLaunchKernelGGL(sinusoid_kernel, dim3((total + 255) / 256), dim3(256), 0, s, t, batch, half,
                     e);
  return hipGetLastError();
}

// 8 weights of a row: bf16 with one 16-byte streaming load (every weight is read once per
// call, so it is marked for early eviction), fp32 with two plain 16-byte loads.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
FLUX_DEV void wload8(const bf16* p, float* f) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  unpack8(make_uint4(v[0], v[1], v[2], v[3]), f);
}
FLUX_DEV void wload8(const float* p, float* f) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}

// y[b, n] += W[n, 8c .. 8c + 8) . x[b, 8c .. 8c + 8) for b < nb: the per-lane partial dot
// products of one 8-element chunk, x read from xb (global or LDS, row stride K).
FLUX_DEV void gemv_chunk(const float* wf, const float* xb, int K, int c, int nb, float* acc) {
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    if (bb < nb) {
      const float* xp = xb + (int64_t)bb * K + c * 8;
      const float4 a = *reinterpret_cast<const float4*>(xp);
      const float4 bq = *reinterpret_cast<const float4*>(xp + 4);
      acc[bb] += wf[0] * a.x + wf[1] * a.y + wf[2] * a.z + wf[3] * a.w + wf[4] * bq.x +
                 wf[5] * bq.y + wf[6] * bq.z + wf[7] * bq.w;
    }
  }
}

// Wave sums of the partials, optional SiLU, one store per (batch row, n).
FLUX_DEV void gemv_finish(const float* acc, int nb, int silu_out, int lane, float* y, int64_t N,
                          int n) {
#pragma unroll
  for (int bb = 0; bb < 4; ++bb) {
    if (bb < nb) {
      float v = wave_sum(acc[bb]);
      if (silu_out) v = silu_f(v);
      if (lane == 0) y[bb * N + n] = v;
    }
  }
}

// x (batch <= 4 rows of K floats) staged in LDS once per workgroup; each wave then walks the
// output rows n, n + 4 * gridDim.x, ... and reads each W row once, 16 bytes per lane per
// chunk.  With the grid capped at the resident workgroups, x is fetched from L2 once per
// workgroup instead of once per 4 rows, and no workgroup launch is spent on 4 rows.
// Measured from HBM (rotating weight sets, the 6D x D modulation at D 4096): 40.5 -> 32.2 us,
// 6.26 TB/s; the conditioning chain with it 56.4 -> 48.0 us.
template <class TW>
__global__ __launch_bounds__(256) void gemv_rows_kernel(const TW* __restrict__ W, int N, int K,
                                                        const float* __restrict__ x, int batch,
                                                        int silu_out, float* __restrict__ y) {
  extern __shared__ float4 xs4[];
  const int nx4 = batch * K / 4;
  for (int i = threadIdx.x; i < nx4; i += 256) xs4[i] = reinterpret_cast<const float4*>(x)[i];
  __syncthreads();
  const float* xs = reinterpret_cast<const float*>(xs4);
  const int lane = threadIdx.x & 63;
  const int nch = K >> 3;
  for (int n = blockIdx.x * 4 + (threadIdx.x >> 6); n < N; n += gridDim.x * 4) {
    const TW* w = W + (int64_t)n * K;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < nch; c += 64) {
      float wf[8];
      wload8(w + c * 8, wf);
      gemv_chunk(wf, xs, K, c, batch, acc);
    }
    gemv_finish(acc, batch, silu_out, lane, y, N, n);
  }
}

// Any batch and K: one wave per output row, x read through L1 / L2, up to 4 batch rows per
// pass over the W row.
template <class TW>
__global__ __launch_bounds__(256) void gemv_kernel(const TW* __restrict__ W, int N, int K,
                                                   const float* __restrict__ x, int batch,
                                                   int silu_out, float* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const TW* w = W + (int64_t)n * K;
  const int nch = K >> 3;
  for (int b0 = 0; b0 < batch; b0 += 4) {
    const int nb = min(4, batch - b0);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < nch; c += 64) {
      float wf[8];
      wload8(w + c * 8, wf);
      gemv_chunk(wf, x + (int64_t)b0 * K, K, c, nb, acc);
    }
    gemv_finish(acc, nb, silu_out, lane, y + (int64_t)b0 * N, N, n);
  }
}

// x staged in LDS up to this many bytes (within the default dynamic-LDS limit)
constexpr size_t kGemvLdsBytes = 65536;

hipError_t gemv(int w_dtype, const void* W, int N, int K, const float* x, int batch,
                bool silu_in, bool silu_out, float* y, hipStream_t s) {
  if (silu_in) return hipErrorInvalidValue;  // producers apply silu on their outputs
  if (N <= 0 || batch <= 0) return hipSuccess;
  if (K % 8) return hipErrorInvalidValue;
  const dim3 block(256);
  const size_t xbytes = (size_t)batch * K * sizeof(float);
  if (batch <= 4 && xbytes <= kGemvLdsBytes) {
    // resident workgroups: 8 per CU by threads, fewer when x takes more than 20 KB of LDS
    const int per_cu = (int)std::min<size_t>(8, (160 * 1024) / xbytes);
    const dim3 grid((unsigned)std::min(((int64_t)N + 3) / 4, (int64_t)256 * per_cu));
    if (w_dtype == DT_BF16)
      hipLaunchKernelGGL(gemv_rows_kernel<bf16>, grid, block, xbytes, s,
                         static_cast<const bf16*>(W), N, K, x, batch, (int)silu_out, y);
    else
      hipLaunchKernelGGL(gemv_rows_kernel<float>, grid, block, xbytes, s,
                         static_cast<const float*>(W), N, K, x, batch, (int)silu_out, y);
    return hipGetLastError();
  }
  const dim3 grid((N + 3) / 4);
  if (w_dtype == DT_BF16)
    hipLaunchKernelGGL(gemv_kernel<bf16>, grid, block, 0, s, static_cast<const bf16*>(W), N, K, x,
                       batch, (int)silu_out, y);
  else
    hipLaunchKernelGGL(gemv_kernel<float>, grid, block, 0, s, static_cast<const float*>(W), N, K,
                       x, batch, (int)silu_out, y);
  return hipGetLastError();
}

}  // namespace flux
