// Sampling-loop kernels around the denoiser step: latent packing, generation ids and the
// fused Euler / guidance update.
//
// FLUX.2 [klein] research note, 训练方法 (latent rectified flow; 4 distilled steps, or 50
// base steps with the two forwards of classifier-free guidance) and Visual tokenizer / VAE
// (32-channel latent, 2x2 patchify to the 128 input channels); Diffusers walk-through of
// Flux2Transformer2DModel, the pipeline call chain (packed latents with 4-D ids, a
// flow-matching Euler scheduler calling the transformer once per step).
//
// All of these move a few MB per call (the Klein-9B 1024^2 state is 4096 x 128 fp32), so
// they are simple element-per-thread kernels with vector accesses along the token rows.
#include "common.h"
#include "sampler.h"

namespace flux {

// tokens[b, r*gw + c, 4 ch + 2 ph + pw] = z[b, ch, 2r + ph, 2c + pw]; one thread per
// (b, ch, patch row r, patch column c), consecutive threads along c: two contiguous 8-byte
// reads (the patch's rows), one 16-byte write.
__global__ void pack_latents_kernel(const float* __restrict__ z, float* __restrict__ x, int B,
                                    int C, int H, int W) {
  const int gw = W / 2, gh = H / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)B * C * gh * gw) return;
  const int c = (int)(idx % gw);
  const int64_t q = idx / gw;
  const int r = (int)(q % gh);
  const int64_t bc = q / gh;
  const int ch = (int)(bc % C), b = (int)(bc / C);
  const float* src = z + (bc * H + 2 * r) * W + 2 * c;
  const float2 top = *reinterpret_cast<const float2*>(src);
  const float2 bot = *reinterpret_cast<const float2*>(src + W);
  *reinterpret_cast<float4*>(x + ((int64_t)b * gh * gw + (int64_t)r * gw + c) * 4 * C + 4 * ch) =
      make_float4(top.x, top.y, bot.x, bot.y);
}

// inverse of pack_latents_kernel, same thread mapping
__global__ void unpack_latents_kernel(const float* __restrict__ x, float* __restrict__ z, int B,
                                      int C, int H, int W) {
  const int gw = W / 2, gh = H / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)B * C * gh * gw) return;
  const int c = (int)(idx % gw);
  const int64_t q = idx / gw;
  const int r = (int)(q % gh);
  const int64_t bc = q / gh;
  const int ch = (int)(bc % C), b = (int)(bc / C);
  const float4 v = *reinterpret_cast<const float4*>(
      x + ((int64_t)b * gh * gw + (int64_t)r * gw + c) * 4 * C + 4 * ch);
  float* dst = z + (bc * H + 2 * r) * W + 2 * c;
  *reinterpret_cast<float2*>(dst) = make_float2(v.x, v.y);
  *reinterpret_cast<float2*>(dst + W) = make_float2(v.z, v.w);
}

// image token (r, c) -> (t_axis, r, c, 0) row-major; text token i -> (0, 0, 0, i)
__global__ void generation_ids_kernel(int32_t* __restrict__ img_ids, int gh, int gw,
                                      int32_t* __restrict__ txt_ids, int n_txt, int t_axis) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int n_img = gh * gw;
  if (idx < n_img) {
    *reinterpret_cast<int4*>(img_ids + 4 * idx) = make_int4(t_axis, idx / gw, idx % gw, 0);
  } else if (idx < n_img + n_txt) {
    const int i = idx - n_img;
    *reinterpret_cast<int4*>(txt_ids + 4 * i) = make_int4(0, 0, 0, i);
  }
}

template <class T>
FLUX_DEV void store4_as(T* p, float4 v);
template <>
FLUX_DEV void store4_as<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
FLUX_DEV void store4_as<bf16>(bf16* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack2(v.x, v.y), pack2(v.z, v.w));
}

// x += dt * v_eff over n4 groups of 4 elements; v_eff = v, or with guidance v_u + g (v_c -
// v_u) where group i of the conditional half is v[i] and of the unconditional half
// v[half4 + i].  Without v the state is left as is.  xin (optional) receives the model
// input: the new state in the model dtype, written to both halves with guidance.  The
// first nt threads also write the next level's timestep t_val to t_out.
template <class T>
__global__ void sampler_update_kernel(float* __restrict__ x, const float* __restrict__ v,
                                      int64_t n4, int64_t half4, float dt, float g, int guided,
                                      T* __restrict__ xin, float* __restrict__ t_out, int nt,
                                      float t_val) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nt) t_out[i] = t_val;
  if (i >= n4) return;
  float4 s = reinterpret_cast<float4*>(x)[i];
  if (v) {
    float4 ve = reinterpret_cast<const float4*>(v)[i];
    if (guided) {
      const float4 vu = reinterpret_cast<const float4*>(v)[half4 + i];
      ve = make_float4(fmaf(g, ve.x - vu.x, vu.x), fmaf(g, ve.y - vu.y, vu.y),
                       fmaf(g, ve.z - vu.z, vu.z), fmaf(g, ve.w - vu.w, vu.w));
    }
    s = make_float4(fmaf(dt, ve.x, s.x), fmaf(dt, ve.y, s.y), fmaf(dt, ve.z, s.z),
                    fmaf(dt, ve.w, s.w));
    reinterpret_cast<float4*>(x)[i] = s;
  }
  if (xin) {
    store4_as<T>(xin + 4 * i, s);
    if (guided) store4_as<T>(xin + 4 * (half4 + i), s);
  }
}

static unsigned blocks_for(int64_t n, int threads) {
  return (unsigned)((n + threads - 1) / threads);
}

hipError_t pack_latents(const float* z, float* x, int B, int C, int H, int W, hipStream_t s) {
  const int64_t n = (int64_t)B * (H / 2) * (W / 2) * C;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_latents_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, z, x, B, C,
                     H, W);
  return hipGetLastError();
}

hipError_t unpack_latents(const float* x, float* z, int B, int C, int H, int W, hipStream_t s) {
  const int64_t n = (int64_t)B * C * (H / 2) * (W / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(unpack_latents_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, x, z, B,
                     C, H, W);
  return hipGetLastError();
}

hipError_t generation_ids(int32_t* img_ids, int gh, int gw, int32_t* txt_ids, int n_txt,
                          hipStream_t s, int t_axis) {
  const int n = gh * gw + n_txt;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(generation_ids_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, s, img_ids,
                     gh, gw, txt_ids, n_txt, t_axis);
  return hipGetLastError();
}

hipError_t sampler_update(int xin_dtype, float* x, const float* v, int64_t n, float dt, float g,
                          bool guided, void* xin, float* t_out, int nt, float t_val,
                          hipStream_t s) {
  const int64_t n4 = n / 4;
  const int64_t threads = n4 > nt ? n4 : nt;
  if (threads == 0) return hipSuccess;
  if (xin_dtype == DT_BF16)
    hipLaunchKernelGGL(sampler_update_kernel<bf16>, dim3(blocks_for(threads, 256)), dim3(256), 0,
                       s, x, v, n4, n4, dt, g, guided ? 1 : 0, static_cast<bf16*>(xin), t_out,
                       t_out ? nt : 0, t_val);
  else
    hipLaunchKernelGGL(sampler_update_kernel<float>, dim3(blocks_for(threads, 256)), dim3(256), 0,
                       s, x, v, n4, n4, dt, g, guided ? 1 : 0, static_cast<float*>(xin), t_out,
                       t_out ? nt : 0, t_val);
  return hipGetLastError();
}

}  // namespace flux
