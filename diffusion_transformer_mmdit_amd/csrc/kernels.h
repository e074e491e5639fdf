// Host-side launchers of the libflux kernels (internal interface between the C ABI
// orchestration and the .hip translation units).  Every launcher enqueues on `s`,
// assumes arguments were validated by the caller and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flux {

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_GATED_RESIDUAL = 2, EPI_QKV = 3 };

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
  // EPI_QKV: columns [0, 2*dim) go to y (q | k, row-major, ldy); columns [2*dim, 3*dim)
  // go transposed to vt[(b * dim + f) * ldvt + vt_off + i] for row m = b * rows_per_batch + i
  void* vt;
  int64_t ldvt;
  int vt_off;
  int dim;
  // optional scratch of linear_splitk_bytes() bytes: lets the large-tile path split the
  // last partial round of tiles along K (nullptr: never split)
  float* split_ws;
  // hi / lo operands: x has k = kw + kdup columns whose last kdup repeat the W columns
  // [kw - kdup, kw) (x column c >= kw reads W column c - kdup), so one product sums
  // x_hi W^T + x_lo W^T.  kdup = 0: plain (W has k columns).  kw and kdup are multiples of 64.
  int kdup;
  // EPI_SWIGLU: with swiglu_lo, the output is a bf16 hi / lo pair, hi at column j and
  // lo = bf16(v - hi) at column n / 2 + j of the same row
  bool swiglu_lo;
};

// scratch size that enables every split-K choice of linear()
size_t linear_splitk_bytes();
// Device address (for the current device) and size of the library's fixed split-K scratch
// array, the one flux_linear_noalloc uses; resolved once per device.
hipError_t linear_static_scratch(float** ptr, size_t* bytes);

// y = x W^T with epilogue; dtype = type of x and W (DT_BF16 / DT_F16 -> MFMA path; with
// DT_F16 the SwiGLU output is binary16 and the QKV outputs stay bf16).
hipError_t linear(int dtype, const LinearArgs& a, hipStream_t s);
// Two independent products with the same epilogue kind, n, k, operand strides and dtypes
// (the double block's image and text streams) in one launch: b's tiles follow a's, so a
// partial last round of tiles falls on b.  Otherwise (or when either has no rows) one launch
// each.  The split-K scratch is a's.
hipError_t linear_pair(int dtype, const LinearArgs& a, const LinearArgs& b, hipStream_t s);
// fp8 (E4M3) linear: x [m, ldx] and W [n, ldw] bytes, y = sa[m] sw[n] (x W^T) with the
// epilogue (EPI_STORE, EPI_SWIGLU, EPI_GATED_RESIDUAL); k % 128 == 0.
hipError_t linear_fp8(const LinearArgs& a, const float* sa, const float* sw, hipStream_t s);
// Per-row E4M3 quantization of x [rows, ldx] (x_dtype): s[r] = amax(|x[r, :cols]|) / 448
// (1 for an all-zero row), q[r, c] = E4M3(fp32(x * (448 / amax))) rounded to nearest even,
// saturating (the multiplier, not a division by s; both fp32, correctly rounded).
hipError_t quantize_fp8_rows(int x_dtype, const void* x, int64_t ldx, int rows, int cols,
                             uint8_t* q, int64_t ldq, float* s_out, hipStream_t s);

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
// The same with the output as bf16 hi / lo planes in one row of y (bf16): hi = bf16(out)
// at columns [0, dim), lo = bf16(out - hi) at [dim, 2 dim); ldy >= 2 dim.
hipError_t layernorm_modulate_hilo(int x_dtype, const void* x, int64_t ldx, void* y, int64_t ldy,
                                   int rows, int dim, int rpb, const float* shift,
                                   const float* scale, int64_t mod_bs, float eps, hipStream_t s);

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

// O = softmax(Q K^T / sqrt(128)) V per head; head_dim 128.  q, k, o are joint-sequence
// views (head h at columns [128 h, 128 h + 128)); V is given transposed:
// vt[(b * heads * 128 + f) * ld_vt + j] = V[b, j, f], with ld_vt a multiple of 64 and the
// columns [seq, ld_vt) finite (zero).  split_ws (attention_split_bytes() of device memory,
// or null to run every unit whole) holds the partial outputs of key-split units.
// Optional extra keys and values appended after the `seq` keys of the view (a reference
// K/V cache): key j (< n) of batch b is k + bb * bs + j * ld (head h at columns
// [128 h, 128 h + 128)), its values column j of the rows bb * dim + f of vt (ld_vt a
// multiple of 64, columns [n, ld_vt) finite), with bb = b % nb.
struct KvExtra {
  const void* k;
  int64_t bs, ld;
  const void* vt;
  int64_t ld_vt;
  int n, nb;
};
// o_dtype: storage type of O (-1: dtype; bf16 operands may write DT_F16 instead)
hipError_t attention(int dtype, SeqView q, SeqView k, const void* vt, int64_t ld_vt, SeqView o,
                     int batch, int seq, int heads, float* split_ws, hipStream_t s,
                     const KvExtra* extra = nullptr, int o_dtype = -1);
size_t attention_split_bytes();

// vt[(b * dim + f) * ld_vt + j] = v(b, j)[f] for j < seq
hipError_t transpose_v(int dtype, SeqView v, void* vt, int64_t ld_vt, int dim, int batch, int seq,
                       hipStream_t s);

// p[r * ld + c] = 0 for r < rows, c0 <= c < c1
hipError_t zero_cols(int dtype, void* p, int64_t ld, int64_t rows, int c0, int c1, hipStream_t s);

// Copy rows between two joint-sequence views (dtype conversion allowed).
hipError_t copy_rows(int src_dtype, SeqView src, int dst_dtype, SeqView dst, int batch, int seq,
                     int dim, hipStream_t s);

}  // namespace flux
