// Shared device helpers for the gfx950 kernels of libflux.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;  // IEEE binary16
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

#define FLUX_DEV __device__ __forceinline__

// ---- scalar conversions -------------------------------------------------------------
FLUX_DEV float to_f32(float x) { return x; }
FLUX_DEV float to_f32(bf16 x) { return static_cast<float>(x); }
FLUX_DEV float to_f32(f16 x) { return static_cast<float>(x); }

template <class T>
FLUX_DEV T from_f32(float x);
template <>
FLUX_DEV float from_f32<float>(float x) { return x; }
template <>
FLUX_DEV bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }  // RNE
template <>
FLUX_DEV f16 from_f32<f16>(float x) { return static_cast<f16>(x); }  // RNE

// ---- 16-byte vector loads / stores of 8 bf16 or 4 fp32 ------------------------------
FLUX_DEV uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
FLUX_DEV void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// 8 bf16 packed in a uint4 -> 8 floats
FLUX_DEV void unpack8(uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (one v_cvt_pk_bf16_f32, round to nearest even)
FLUX_DEV uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

FLUX_DEV uint4 pack8(const float* f) {
  return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

// two floats -> packed binary16 pair (round to nearest even)
FLUX_DEV uint32_t pack2h(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// the pair packing of a 2-byte storage type
template <class T>
FLUX_DEV uint32_t pack2_as(float a, float b);
template <>
FLUX_DEV uint32_t pack2_as<bf16>(float a, float b) { return pack2(a, b); }
template <>
FLUX_DEV uint32_t pack2_as<f16>(float a, float b) { return pack2h(a, b); }
template <class T>
FLUX_DEV uint4 pack8_as(const float* f) {
  return make_uint4(pack2_as<T>(f[0], f[1]), pack2_as<T>(f[2], f[3]), pack2_as<T>(f[4], f[5]),
                    pack2_as<T>(f[6], f[7]));
}

// ---- wave64 reductions ---------------------------------------------------------------
FLUX_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

FLUX_DEV float group_sum16(float v) {  // sum over aligned groups of 16 lanes
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// x * sigmoid(x) with the hardware reciprocal (1 ulp) instead of an IEEE division: within
// 2 ulp of the correctly rounded result, far below the bf16 rounding of the outputs
FLUX_DEV float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// ---- direct global->LDS loads ---------------------------------------------------------
// Byte address of an LDS object (wave-uniform when the object is).
FLUX_DEV uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte global->LDS loads issued through inline asm (M0 = wave-uniform LDS byte address;
// lane i writes LDS bytes [16 i, 16 i + 16)).  The compiler does not track these loads, so
// it adds no conservative vmcnt(0) before later LDS reads or barriers; callers wait
// explicitly (s_waitcnt vmcnt) before they read the data.  M0 is listed as clobbered, a
// reserved register clang warns it may not preserve: that is safe because no instruction
// the compiler generates for these kernels uses M0 (tests/test_asm_m0.py checks the
// gfx950 assembly of every source that includes these helpers).
//   dma16s: global address = scalar base + per-lane 32-bit byte offset
//   dma16v: per-lane 64-bit global address
FLUX_DEV void dma16s(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_addr), "v"(voff),
               "s"(base)
               : "memory", "m0");
}
FLUX_DEV void dma16v(const void* g, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr)
               : "memory", "m0");
}

// ---- dtype tags shared with the host -------------------------------------------------
enum { DT_BF16 = 0, DT_F32 = 1, DT_F16 = 2 };
