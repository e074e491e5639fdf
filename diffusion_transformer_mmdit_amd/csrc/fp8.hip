// FP8 (E4M3) per-row quantization for the fp8 linear layer.
//
// The FLUX.2 [klein] research note, Infra (量化), reports FP8 releases of the models and
// their speed-ups but no recipe.  Reading used here: OCP E4M3 (1 sign, 4 exponent bits with
// bias 7, 3 mantissa bits, largest finite 448, no infinities), scales per row (activation
// rows, weight rows = output channels) s = amax / 448 for dequantization, codes =
// E4M3(x * (448 / amax)) rounded to nearest even with saturation at 448.
//
// One wave per row.  Rows of up to 4096 elements are held in registers (8 16-byte loads per
// lane, all in flight together): amax, then the codes from the registers, 8 codes per
// 8-byte store.  Longer rows take two passes (amax, then the codes; the row is cache
// resident).  HBM traffic: the row once, the codes once, 4 bytes of scale.
#include "common.h"
#include "kernels.h"

namespace flux {

// Four E4M3 codes (low byte first) of v[0..3], round to nearest even, saturating at 448,
// NaN -> 0x7F.  v_cvt_pk_fp8_f32 rounds to nearest even; over every fp32 value with
// |v| <= 448 its codes equal those of the definition (an exhaustive comparison with a
// bit-level encoder), so inputs are clamped into that range first.
FLUX_DEV uint32_t e4m3x4(const float (&v)[4]) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_fmed3f(v[i], -448.f, 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  uint32_t u = (uint32_t)w;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (v[i] != v[i]) u = (u & ~(0xffu << (8 * i))) | (0x7fu << (8 * i));
  return u;
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
  constexpr int CH = 8;  // chunks of 8 elements per lane kept in registers
  if (vec && cols <= 512 * CH) {
    float v[CH][8];
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (lane * 8 + 512 * i < cols) load8<T>(xr + lane * 8 + 512 * i, v[i]);
#pragma unroll
    for (int i = 0; i < CH; ++i)
      if (lane * 8 + 512 * i < cols)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float sc = amax > 0.f ? __fdiv_rn(amax, 448.f) : 1.f;
    const float rc = amax > 0.f ? __fdiv_rn(448.f, amax) : 1.f;
    if (lane == 0) s_out[row] = sc;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c0 = lane * 8 + 512 * i;
      if (c0 < cols) {
        const float a[4] = {v[i][0] * rc, v[i][1] * rc, v[i][2] * rc, v[i][3] * rc};
        const float b[4] = {v[i][4] * rc, v[i][5] * rc, v[i][6] * rc, v[i][7] * rc};
        *reinterpret_cast<uint2*>(qr + c0) = make_uint2(e4m3x4(a), e4m3x4(b));
      }
    }
    return;
  }
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
  const float rc = amax > 0.f ? __fdiv_rn(448.f, amax) : 1.f;
  if (lane == 0) s_out[row] = sc;
  if (vec) {
    for (int c0 = lane * 8; c0 < cols; c0 += 512) {
      float v[8];
      load8<T>(xr + c0, v);
      const float a[4] = {v[0] * rc, v[1] * rc, v[2] * rc, v[3] * rc};
      const float b[4] = {v[4] * rc, v[5] * rc, v[6] * rc, v[7] * rc};
      *reinterpret_cast<uint2*>(qr + c0) = make_uint2(e4m3x4(a), e4m3x4(b));
    }
  } else {
    for (int c = lane; c < cols; c += 64) {
      const float a[4] = {to_f32(xr[c]) * rc, 0.f, 0.f, 0.f};
      qr[c] = (uint8_t)(e4m3x4(a) & 0xffu);
    }
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
