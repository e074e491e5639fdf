// FP8 (E4M3) per-row quantization for the fp8 linear layer.
//
// The FLUX.2 [klein] research note, Infra (量化), reports FP8 releases of the models and
// their speed-ups but no recipe.  Reading used here: OCP E4M3 (1 sign, 4 exponent bits with
// bias 7, 3 mantissa bits, largest finite 448, no infinities), scales per row (activation
// rows, weight rows = output channels) s = amax / 448, codes = E4M3(x / s) rounded to
// nearest even with saturation at 448.
//
// One wave per row: a first pass finds the row's absolute maximum with 16-byte loads, a
// second pass (the row is cache resident) divides by the scale and packs 8 codes per
// 8-byte store.  HBM traffic: the row once, the codes once, 4 bytes of scale.
#include "common.h"
#include "kernels.h"

namespace flux {

// E4M3 code of a float, round to nearest (ties to even), |v| >= 448 saturates to 448,
// NaN -> 0x7F.  Normal range: keep 3 of the 23 fp32 mantissa bits with RNE on the rest;
// below 2^-6 the spacing is 2^-9, so the code is rint(|v| * 2^9) (8 = smallest normal).
FLUX_DEV uint32_t e4m3_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fu;
  const float a = fminf(fabsf(v), 448.f);
  const uint32_t ab = __float_as_uint(a);
  const int e = (int)(ab >> 23) - 127;
  uint32_t code;
  if (e >= -6) {
    const uint32_t m = ab & 0x7fffffu;
    const uint32_t keep = m >> 20, rem = m & 0xfffffu;
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
    uint32_t ee = (uint32_t)(e + 7), kk = keep + up;
    if (kk == 8u) {
      kk = 0u;
      ee += 1u;
    }
    code = (ee << 3) | kk;
    if (code > 0x7eu) code = 0x7eu;
  } else {
    code = (uint32_t)__builtin_rintf(a * 512.f);
  }
  return sign | code;
}

template <class T>
FLUX_DEV void load8(const T* p, float (&v)[8]);
template <>
FLUX_DEV void load8<bf16>(const bf16* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
FLUX_DEV void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 c = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = c.x; v[5] = c.y; v[6] = c.z; v[7] = c.w;
}

// 4 rows per 256-thread workgroup, one wave per row; `vec`: rows 16-byte aligned and cols a
// multiple of 8 (else element by element)
template <class T>
__global__ __launch_bounds__(256) void quant_fp8_rows_kernel(const T* __restrict__ x, int64_t ldx,
                                                             int rows, int cols,
                                                             uint8_t* __restrict__ q, int64_t ldq,
                                                             float* __restrict__ s_out, int vec) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const T* xr = x + (int64_t)row * ldx;
  uint8_t* qr = q + (int64_t)row * ldq;
  float amax = 0.f;
  if (vec) {
    for (int c0 = lane * 8; c0 < cols; c0 += 512) {
      float v[8];
      load8<T>(xr + c0, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    }
  } else {
    for (int c = lane; c < cols; c += 64) amax = fmaxf(amax, fabsf(to_f32(xr[c])));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  const float sc = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
  if (lane == 0) s_out[row] = sc;
  if (vec) {
    for (int c0 = lane * 8; c0 < cols; c0 += 512) {
      float v[8];
      load8<T>(xr + c0, v);
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= e4m3_rne(__fdiv_rn(v[i], sc)) << (8 * i);
        hi |= e4m3_rne(__fdiv_rn(v[4 + i], sc)) << (8 * i);
      }
      *reinterpret_cast<uint2*>(qr + c0) = make_uint2(lo, hi);
    }
  } else {
    for (int c = lane; c < cols; c += 64) qr[c] = (uint8_t)e4m3_rne(__fdiv_rn(to_f32(xr[c]), sc));
  }
}

hipError_t quantize_fp8_rows(int x_dtype, const void* x, int64_t ldx, int rows, int cols,
                             uint8_t* q, int64_t ldq, float* s_out, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int es = x_dtype == DT_BF16 ? 2 : 4;
  const bool vec = cols % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
                   (ldx * es) % 16 == 0 && (reinterpret_cast<uintptr_t>(q) & 7) == 0 &&
                   ldq % 8 == 0;
  const dim3 grid((rows + 3) / 4);
  if (x_dtype == DT_BF16)
    hipLaunchKernelGGL(quant_fp8_rows_kernel<bf16>, grid, dim3(256), 0, s,
                       static_cast<const bf16*>(x), ldx, rows, cols, q, ldq, s_out, vec ? 1 : 0);
  else
    hipLaunchKernelGGL(quant_fp8_rows_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(x), ldx, rows, cols, q, ldq, s_out, vec ? 1 : 0);
  return hipGetLastError();
}

}  // namespace flux
