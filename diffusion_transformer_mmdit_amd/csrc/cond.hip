// Conditioning path: timestep sinusoid and the HBM-bound matrix-vector products of the
// MLPEmbedder and the AdaLN modulation linears ("时间步缩放" and "双流块 / 单流块" of the
// Diffusers walk-through; "条件注入" of the FLUX.2 [klein] note: 256-channel sinusoid of
// 1000 t, then MLPEmbedder, then modulation = Linear(silu(temb))).
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

// One wave per output row n; W row read once with 16-byte loads (8 elements per lane per
// step), up to 4 batch rows per pass.  x stays in L1/L2 (it is K floats per batch row).
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
      if constexpr (sizeof(TW) == 2) {
        unpack8(ld16(w + c * 8), wf);
      } else {
        const float4 a = *reinterpret_cast<const float4*>(w + c * 8);
        const float4 bq = *reinterpret_cast<const float4*>(w + c * 8 + 4);
        wf[0] = a.x; wf[1] = a.y; wf[2] = a.z; wf[3] = a.w;
        wf[4] = bq.x; wf[5] = bq.y; wf[6] = bq.z; wf[7] = bq.w;
      }
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        if (bb < nb) {
          const float* xp = x + (int64_t)(b0 + bb) * K + c * 8;
          const float4 a = *reinterpret_cast<const float4*>(xp);
          const float4 bq = *reinterpret_cast<const float4*>(xp + 4);
          acc[bb] += wf[0] * a.x + wf[1] * a.y + wf[2] * a.z + wf[3] * a.w + wf[4] * bq.x +
                     wf[5] * bq.y + wf[6] * bq.z + wf[7] * bq.w;
        }
      }
    }
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) {
      if (bb < nb) {
        float v = wave_sum(acc[bb]);
        if (silu_out) v = silu_f(v);
        if (lane == 0) y[(int64_t)(b0 + bb) * N + n] = v;
      }
    }
  }
}

hipError_t gemv(int w_dtype, const void* W, int N, int K, const float* x, int batch,
                bool silu_in, bool silu_out, float* y, hipStream_t s) {
  if (silu_in) return hipErrorInvalidValue;  // producers apply silu on their outputs
  if (N <= 0 || batch <= 0) return hipSuccess;
  dim3 grid((N + 3) / 4), block(256);
  if (w_dtype == DT_BF16)
    hipLaunchKernelGGL(gemv_kernel<bf16>, grid, block, 0, s, static_cast<const bf16*>(W), N, K, x,
                       batch, (int)silu_out, y);
  else
    hipLaunchKernelGGL(gemv_kernel<float>, grid, block, 0, s, static_cast<const float*>(W), N, K,
                       x, batch, (int)silu_out, y);
  return hipGetLastError();
}

}  // namespace flux
