// Host-side launchers of the sampling-loop kernels (sampler.hip).  Same conventions as
// kernels.h: enqueue on `s`, arguments validated by the caller, return hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {
// z: latent [B, C, H, W] fp32 (H, W even); x: tokens [B, (H/2)(W/2), 4C] fp32 with token
// channel 4 ch + 2 ph + pw of patch (r, c) in row-major patch order.
hipError_t pack_latents(const float* z, float* x, int B, int C, int H, int W, hipStream_t s);
hipError_t unpack_latents(const float* x, float* z, int B, int C, int H, int W, hipStream_t s);
// img_ids [gh * gw, 4] = (t_axis, r, c, 0) row-major; txt_ids [n_txt, 4] = (0, 0, 0, i)
hipError_t generation_ids(int32_t* img_ids, int gh, int gw, int32_t* txt_ids, int n_txt,
                          hipStream_t s, int t_axis = 0);
// x[0 .. n) += dt * v_eff (n % 4 == 0, 16-byte aligned), v_eff = v or, guided,
// v[i] for the conditional half and v[n + i] for the unconditional: v_u + g (v_c - v_u).
// v == nullptr leaves x unchanged.  xin (optional, xin_dtype): model input = new x, written
// to xin[0 .. n) and, guided, also to xin[n .. 2n).  t_out (optional): t_out[0 .. nt) =
// t_val, the timestep of the next step.
hipError_t sampler_update(int xin_dtype, float* x, const float* v, int64_t n, float dt, float g,
                          bool guided, void* xin, float* t_out, int nt, float t_val,
                          hipStream_t s);
}  // namespace flux
