// Host-side launchers of the libflux kernels (internal interface between the C ABI
// orchestration and the .hip translation units).  Every launcher enqueues on `s`,
// assumes arguments were validated by the caller and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_GATED_RESIDUAL = 2 };

struct LinearArgs {
  int epilogue;
  int m, n, k;
  const void* x;
  int64_t ldx;
  const void* w;
  int64_t ldw;
  void* y;
  int64_t ldy;
  int y_dtype;            // DT_BF16 / DT_F32 (store and gated residual)
  const void* resid;      // gated residual input (may equal y)
  int64_t ldr;
  int r_dtype;
  const float* gate;      // [batch, gate_bs]
  int64_t gate_bs;
  int rows_per_batch;
};

// y = x W^T with epilogue; dtype = type of x and W (DT_BF16 -> MFMA path).
hipError_t linear(int dtype, const LinearArgs& a, hipStream_t s);

// e[b, :] = [cos(1000 t_b f) | sin(1000 t_b f)], f_k = 10000^(-k/half); e: [batch, 2*half]
hipError_t timestep_sinusoid(const float* t, int batch, int half, float* e, hipStream_t s);

// y[b, n] = (silu_out ? silu : id)(sum_k W[n, k] * (silu_in ? silu : id)(x[b, k]))
// W: [N, K] of w_dtype; x, y float.
hipError_t gemv(int w_dtype, const void* W, int N, int K, const float* x, int batch,
                bool silu_in, bool silu_out, float* y, hipStream_t s);

// y[r, :] = (1 + scale[b]) * LN(x[r, :]) + shift[b], b = r / rows_per_batch
hipError_t layernorm_modulate(int x_dtype, int y_dtype, const void* x, int64_t ldx, void* y,
                              int64_t ldy, int rows, int dim, int rows_per_batch,
                              const float* shift, const float* scale, int64_t mod_bs, float eps,
                              hipStream_t s);

// RoPE tables for the joint sequence [txt ; img]: pos [L, P] int32 and cs [L, P] (cos, sin)
// with P = head_dim / 2 pairs; axes_dim gives the per-axis widths (4 axes).
hipError_t rope_table(const int32_t* txt_ids, const int32_t* img_ids, int n_txt, int n_img,
                      const int32_t* axes_dim, float theta, int32_t* pos, float2* cs,
                      hipStream_t s);

// Joint-sequence view: token j of batch b lives at
//   j <  n0 : base0 + b * bs0 + j * ld
//   j >= n0 : base1 + b * bs1 + (j - n0) * ld      (elements)
struct SeqView {
  void* base0;
  void* base1;
  int64_t bs0, bs1, ld;
  int n0;
};

// In-place per-head RMSNorm (gamma per segment) + RoPE of q and k.
hipError_t qk_norm_rope(int dtype, SeqView q, SeqView k, int batch, int seq, int heads,
                        const float* qg0, const float* kg0, const float* qg1, const float* kg1,
                        const float2* cs, float eps, hipStream_t s);

// O = softmax(Q K^T / sqrt(128)) V per head; head_dim 128.
hipError_t attention(int dtype, SeqView q, SeqView k, SeqView v, SeqView o, int batch, int seq,
                     int heads, hipStream_t s);

// Copy rows between two joint-sequence views (dtype conversion allowed).
hipError_t copy_rows(int src_dtype, SeqView src, int dst_dtype, SeqView dst, int batch, int seq,
                     int dim, hipStream_t s);

}  // namespace flux
