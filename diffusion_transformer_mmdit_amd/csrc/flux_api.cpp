// C ABI of libflux: argument validation, workspace carving and the launch sequences of the
// double-stream block, the single-stream block and the denoiser step.
//
// Block structure follows the Diffusers walk-through of Flux2Transformer2DModel (sections
// 双流块 Flux2TransformerBlock, 单流块 Flux2SingleTransformerBlock, 激活函数与 FFN,
// 前向传播输入输出约定) and the FLUX.2 Klein 9B shape trace (sections 3 and 4).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "flux.h"
#include "kernels.h"
#include "sampler.h"

using namespace flux;

// ------------------------------------------------------------------------------------
// errors
// ------------------------------------------------------------------------------------
static thread_local std::string g_err;

static int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define HIP_TRY(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(FLUX_EHIP, "%s failed: %s", #expr, hipGetErrorString(e_));            \
  } while (0)

extern "C" const char* flux_last_error(void) { return g_err.c_str(); }
extern "C" const char* flux_version(void) { return "libflux 0.1 (gfx950)"; }

// ------------------------------------------------------------------------------------
// measurement hook: event pairs around the launches of one site, created up front
// ------------------------------------------------------------------------------------
namespace {
struct Timing {
  std::mutex mu;
  std::atomic<int> site{0};
  std::vector<hipEvent_t> ev;  // start, end, start, end, ...
  int used = 0;                // pairs handed out
  int dropped = 0;             // launches past the armed capacity
};
Timing g_timing;

void timing_release() {
  for (hipEvent_t e : g_timing.ev) (void)hipEventDestroy(e);
  g_timing.ev.clear();
  g_timing.used = g_timing.dropped = 0;
}

// Records the start event on construction and the end event on destruction when `site` is
// the armed one; costs one relaxed atomic load otherwise.
class TimedSite {
 public:
  TimedSite(int site, hipStream_t s) : s_(s) {
    if (g_timing.site.load(std::memory_order_relaxed) != site) return;
    std::lock_guard<std::mutex> lk(g_timing.mu);
    if (g_timing.site.load(std::memory_order_relaxed) != site) return;
    if ((size_t)(2 * g_timing.used + 2) > g_timing.ev.size()) {
      ++g_timing.dropped;
      return;
    }
    const int i = g_timing.used++;
    if (hipEventRecord(g_timing.ev[2 * i], s) == hipSuccess) end_ = g_timing.ev[2 * i + 1];
  }
  ~TimedSite() {
    if (end_) (void)hipEventRecord(end_, s_);
  }
  TimedSite(const TimedSite&) = delete;
  TimedSite& operator=(const TimedSite&) = delete;

 private:
  hipStream_t s_;
  hipEvent_t end_ = nullptr;
};
}  // namespace

extern "C" int flux_timing_begin(int site, int max_launches) {
  if (site < FLUX_SITE_SINGLE_QKV || site > FLUX_SITE_DOUBLE_MLP_OUT)
    return fail(FLUX_EINVAL, "unknown timing site %d", site);
  if (max_launches <= 0 || max_launches > (1 << 16))
    return fail(FLUX_EINVAL, "max_launches must be in [1, 65536] (got %d)", max_launches);
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.site.store(0);
  timing_release();
  g_timing.ev.reserve(2 * (size_t)max_launches);
  for (int i = 0; i < 2 * max_launches; ++i) {
    hipEvent_t e;
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      timing_release();
      return fail(FLUX_EHIP, "hipEventCreate failed: %s", hipGetErrorString(r));
    }
    g_timing.ev.push_back(e);
  }
  g_timing.site.store(site);
  return FLUX_OK;
}

extern "C" int flux_timing_end(int* launches, double* mean_us) {
  if (!launches || !mean_us) return fail(FLUX_EINVAL, "launches and mean_us are required");
  std::lock_guard<std::mutex> lk(g_timing.mu);
  g_timing.site.store(0);
  *launches = 0;
  *mean_us = 0.0;
  if (g_timing.dropped > 0) {
    const int d = g_timing.dropped;
    timing_release();
    return fail(FLUX_EINVAL, "%d launches exceeded the armed capacity", d);
  }
  double sum = 0.0;
  for (int i = 0; i < g_timing.used; ++i) {
    hipError_t r = hipEventSynchronize(g_timing.ev[2 * i + 1]);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_timing.ev[2 * i], g_timing.ev[2 * i + 1]);
    if (r != hipSuccess) {
      timing_release();
      return fail(FLUX_EHIP, "timing event %d: %s", i, hipGetErrorString(r));
    }
    sum += ms;
  }
  *launches = g_timing.used;
  if (g_timing.used > 0) *mean_us = 1e3 * sum / g_timing.used;
  timing_release();
  return FLUX_OK;
}

// ------------------------------------------------------------------------------------
// validation helpers
// ------------------------------------------------------------------------------------
static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// the kernels take the public dtype codes as they are (DT_BF16, DT_F32, DT_F16 in common.h)
static_assert(FLUX_BF16 == 0 && FLUX_F32 == 1 && FLUX_F16 == 2, "dtype codes of the kernels");
static int esize(int dtype) { return dtype == FLUX_F32 ? 4 : 2; }

static int check_cfg(const flux_cfg* c) {
  if (!c) return fail(FLUX_EINVAL, "cfg is NULL");
  if (c->dtype != FLUX_BF16 && c->dtype != FLUX_F32)
    return fail(FLUX_EDTYPE, "unknown dtype %d", c->dtype);
  if (c->head_dim != 128) return fail(FLUX_ESHAPE, "head_dim must be 128 (got %d)", c->head_dim);
  if (c->heads <= 0 || c->dim != c->heads * c->head_dim)
    return fail(FLUX_ESHAPE, "dim (%d) must equal heads (%d) * head_dim", c->dim, c->heads);
  if (c->mlp_hidden <= 0 || c->mlp_hidden % 8)
    return fail(FLUX_ESHAPE, "mlp_hidden must be a positive multiple of 8 (got %d)", c->mlp_hidden);
  int sum = 0;
  for (int a = 0; a < 4; ++a) {
    if (c->axes_dim[a] < 0 || c->axes_dim[a] % 2)
      return fail(FLUX_ESHAPE, "axes_dim[%d] = %d must be even and >= 0", a, c->axes_dim[a]);
    sum += c->axes_dim[a];
  }
  if (sum != c->head_dim) return fail(FLUX_ESHAPE, "axes_dim must sum to head_dim (got %d)", sum);
  if (!(c->rope_theta > 0.f)) return fail(FLUX_EINVAL, "rope_theta must be > 0");
  if (!(c->eps > 0.f)) return fail(FLUX_EINVAL, "eps must be > 0");
  if (c->dim > 8192) return fail(FLUX_ESHAPE, "dim > 8192 is not supported");
  if (c->precision != FLUX_PRECISION_BF16 && c->precision != FLUX_PRECISION_SPLIT &&
      c->precision != FLUX_PRECISION_F16)
    return fail(FLUX_EINVAL, "unknown precision %d", c->precision);
  if (c->precision == FLUX_PRECISION_F16 && c->dtype != FLUX_BF16)
    return fail(FLUX_EDTYPE, "FLUX_PRECISION_F16 needs FLUX_BF16");
  if (c->precision == FLUX_PRECISION_SPLIT) {
    if (c->dtype != FLUX_BF16) return fail(FLUX_EDTYPE, "FLUX_PRECISION_SPLIT needs FLUX_BF16");
    if (c->mlp_hidden % 64)
      return fail(FLUX_ESHAPE, "FLUX_PRECISION_SPLIT needs mlp_hidden % 64 == 0 (got %d)",
                  c->mlp_hidden);
  }
  return FLUX_OK;
}

// hi / lo operands (FLUX_PRECISION_SPLIT): 2 planes, else 1
static int planes(const flux_cfg* c) { return c->precision == FLUX_PRECISION_SPLIT ? 2 : 1; }

// Storage type of the block linears' operands (their weights, the LayerNorm + modulate and
// SwiGLU outputs, the attention output): binary16 with FLUX_PRECISION_F16, else cfg->dtype
static int blk_dtype(const flux_cfg* c) {
  return c->precision == FLUX_PRECISION_F16 ? FLUX_F16 : c->dtype;
}

static int check_sizes(int batch, int n_img, int n_txt) {
  if (batch <= 0) return fail(FLUX_EINVAL, "batch must be > 0 (got %d)", batch);
  if (n_img <= 0) return fail(FLUX_EINVAL, "n_img must be > 0 (got %d)", n_img);
  if (n_txt < 0) return fail(FLUX_EINVAL, "n_txt must be >= 0 (got %d)", n_txt);
  return FLUX_OK;
}

#define CHECK(x)              \
  do {                        \
    int st_ = (x);            \
    if (st_ != FLUX_OK) return st_; \
  } while (0)

static int need(const void* p, const char* name) {
  if (!p) return fail(FLUX_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(FLUX_EALIGN, "%s is not 16-byte aligned", name);
  return FLUX_OK;
}

// ------------------------------------------------------------------------------------
// workspace carving (a dry run with base == nullptr gives the size)
// ------------------------------------------------------------------------------------
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = reinterpret_cast<T*>(base + off);
    off += n * sizeof(T);
    return p;
  }
};

static int check_ws(void* ws, size_t have, size_t want) {
  if (want == 0) return FLUX_OK;
  if (!ws) return fail(FLUX_EWORKSPACE, "workspace is NULL (need %zu bytes)", want);
  if (reinterpret_cast<uintptr_t>(ws) & 255u)
    return fail(FLUX_EWORKSPACE, "workspace is not 256-byte aligned");
  if (have < want) return fail(FLUX_EWORKSPACE, "workspace has %zu bytes, need %zu", have, want);
  return FLUX_OK;
}

// conditioning scratch: sinusoid, hidden, silu(temb)
struct CondBufs {
  float* e;
  float* h1;
  float* stemb;
};
static CondBufs carve_cond(Carver& cv, int B, int D) {
  CondBufs c;
  c.e = cv.take<float>((size_t)B * 256);
  c.h1 = cv.take<float>((size_t)B * D);
  c.stemb = cv.take<float>((size_t)B * D);
  return c;
}

// silu(temb) for every batch row: temb = W2 silu(W1 sinusoid(1000 t))
static int run_cond(const flux_cfg* c, const flux_temb_weights* tw, const float* t, int B,
                    const CondBufs& cb, hipStream_t s) {
  HIP_TRY(timestep_sinusoid(t, B, 128, cb.e, s));
  HIP_TRY(gemv(c->dtype, tw->w1, c->dim, 256, cb.e, B, false, true, cb.h1, s));
  HIP_TRY(gemv(c->dtype, tw->w2, c->dim, c->dim, cb.h1, B, false, true, cb.stemb, s));
  return FLUX_OK;
}

static int check_temb(const flux_temb_weights* tw) {
  CHECK(need(tw->w1, "temb.w1"));
  CHECK(need(tw->w2, "temb.w2"));
  return FLUX_OK;
}

// rope tables for the joint sequence
struct RopeBufs {
  int32_t* pos;
  float2* cs;
};
static RopeBufs carve_rope(Carver& cv, int L) {
  RopeBufs r;
  r.pos = cv.take<int32_t>((size_t)L * 64);
  r.cs = cv.take<float2>((size_t)L * 64);
  return r;
}

// ------------------------------------------------------------------------------------
// linear helper
// ------------------------------------------------------------------------------------
static LinearArgs lin_args(int epi, int m, int n, int k, const void* x, int64_t ldx,
                           const void* w, int64_t ldw, void* y, int64_t ldy, int y_dtype,
                           const void* resid = nullptr, int64_t ldr = 0,
                           int r_dtype = FLUX_F32, const float* gate = nullptr,
                           int64_t gate_bs = 0, int rpb = 1, float* split_ws = nullptr,
                           int kdup = 0, bool swiglu_lo = false) {
  LinearArgs a{};
  a.kdup = kdup;
  a.swiglu_lo = swiglu_lo;
  a.epilogue = epi;
  a.m = m;
  a.n = n;
  a.k = k;
  a.x = x;
  a.ldx = ldx;
  a.w = w;
  a.ldw = ldw;
  a.y = y;
  a.ldy = ldy;
  a.y_dtype = y_dtype;
  a.resid = resid;
  a.ldr = ldr;
  a.r_dtype = r_dtype;
  a.gate = gate;
  a.gate_bs = gate_bs;
  a.rows_per_batch = rpb;
  a.split_ws = split_ws;
  return a;
}

static int lin(const flux_cfg* c, int epi, int m, int n, int k, const void* x, int64_t ldx,
               const void* w, int64_t ldw, void* y, int64_t ldy, int y_dtype,
               const void* resid = nullptr, int64_t ldr = 0, int r_dtype = FLUX_F32,
               const float* gate = nullptr, int64_t gate_bs = 0, int rpb = 1, hipStream_t s = 0,
               float* split_ws = nullptr, int kdup = 0, bool swiglu_lo = false) {
  HIP_TRY(linear(c->dtype, lin_args(epi, m, n, k, x, ldx, w, ldw, y, ldy, y_dtype, resid, ldr,
                                    r_dtype, gate, gate_bs, rpb, split_ws, kdup, swiglu_lo),
                 s));
  return FLUX_OK;
}

// lin for the block linears: operands of blk_dtype(c)
static int lin_b(const flux_cfg* c, int epi, int m, int n, int k, const void* x, int64_t ldx,
                 const void* w, int64_t ldw, void* y, int64_t ldy, int y_dtype,
                 const void* resid = nullptr, int64_t ldr = 0, int r_dtype = FLUX_F32,
                 const float* gate = nullptr, int64_t gate_bs = 0, int rpb = 1,
                 hipStream_t s = 0, float* split_ws = nullptr, int kdup = 0,
                 bool swiglu_lo = false) {
  HIP_TRY(linear(blk_dtype(c), lin_args(epi, m, n, k, x, ldx, w, ldw, y, ldy, y_dtype, resid,
                                        ldr, r_dtype, gate, gate_bs, rpb, split_ws, kdup,
                                        swiglu_lo),
                 s));
  return FLUX_OK;
}

// q | k row-major into qk [m, 2D]; v transposed into vt [B*D, ldvt] at token offset vt_off.
// x: [m, D] or, with hi / lo operands, [m, 2D] (hi | lo planes).
static LinearArgs qkv_args(const flux_cfg* c, int m, const void* x, const void* w, void* qk,
                           void* vt, int64_t ldvt, int vt_off, int rpb, float* split_ws) {
  LinearArgs a{};
  const int P = planes(c);
  a.epilogue = EPI_QKV;
  a.m = m;
  a.n = 3 * c->dim;
  a.k = P * c->dim;
  a.kdup = (P - 1) * c->dim;
  a.x = x;
  a.ldx = P * c->dim;
  a.w = w;
  a.ldw = c->dim;
  a.y = qk;
  a.ldy = 2 * c->dim;
  a.y_dtype = c->dtype;
  a.rows_per_batch = rpb;
  a.vt = vt;
  a.ldvt = ldvt;
  a.vt_off = vt_off;
  a.dim = c->dim;
  a.split_ws = split_ws;
  return a;
}

static int lin_qkv(const flux_cfg* c, int m, const void* x, const void* w, void* qk, void* vt,
                   int64_t ldvt, int vt_off, int rpb, hipStream_t s, float* split_ws) {
  HIP_TRY(linear(blk_dtype(c), qkv_args(c, m, x, w, qk, vt, ldvt, vt_off, rpb, split_ws), s));
  return FLUX_OK;
}

// Scratch shared, one after the other on the stream, by the linear layers' split-K tails
// and the attention's key-split units.
static size_t split_scratch_bytes() {
  const size_t a = linear_splitk_bytes(), b = attention_split_bytes();
  return a > b ? a : b;
}

// V^T row pitch: the sequence rounded up to the attention's 64-key tiles
static int64_t vt_pitch(int L) { return ((int64_t)L + 63) / 64 * 64; }

// ------------------------------------------------------------------------------------
// double-stream block
// ------------------------------------------------------------------------------------
// One block's slot of the reference K/V cache: the reference tokens' q | k rows (k after
// RMSNorm + RoPE; q is only used while the cache is filled) and their V^T.
struct RefSlot {
  void* qk;       // [B * n, 2D]
  void* vt;       // [B * D, vt_pitch(n)]
  int n;          // reference tokens per batch item
};
// How a block call uses its slot: not at all; it computes the reference tokens themselves
// (writes the slot; the block's image stream / sequence IS the references); it attends to
// them as extra keys.
enum RefUse { REF_NONE = 0, REF_FILL = 1, REF_KEYS = 2 };

// With hi / lo operands (FLUX_PRECISION_SPLIT) ln and mlp hold two planes per row.
struct DoubleScratch {
  void* ln[2];    // [B*N_s, D] compute dtype       (0 = txt, 1 = img)
  void* qk[2];    // [B*N_s, 2D] q | k
  void* vt;       // [B*D, vt_pitch(L)] V^T of the joint sequence
  void* o[2];     // [B*N_s, D]
  float* mid[2];  // [B*N_s, D] residual after the attention branch
  void* mlp[2];   // [B*N_s, H]
  float* split;   // split-K scratch of the linear layers
};

static DoubleScratch carve_double(Carver& cv, const flux_cfg* c, int B, int Ni, int Nt) {
  DoubleScratch d;
  const int es = esize(c->dtype), P = planes(c);
  const int D = c->dim, H = c->mlp_hidden;
  const int n[2] = {Nt, Ni};
  for (int i = 0; i < 2; ++i) {
    const size_t rows = (size_t)B * n[i];
    d.ln[i] = cv.take<char>(rows * P * D * es);
    d.qk[i] = cv.take<char>(rows * 2 * D * es);
    d.o[i] = cv.take<char>(rows * D * es);
    d.mid[i] = cv.take<float>(rows * D);
    d.mlp[i] = cv.take<char>(rows * P * H * es);
  }
  d.vt = cv.take<char>((size_t)B * D * vt_pitch(Ni + Nt) * es);
  d.split = cv.take<float>(split_scratch_bytes() / sizeof(float));
  return d;
}

static int check_stream(const flux_stream_weights* w, const char* nm) {
  char buf[64];
  snprintf(buf, sizeof buf, "%s.qkv", nm);
  CHECK(need(w->qkv, buf));
  snprintf(buf, sizeof buf, "%s.out", nm);
  CHECK(need(w->out, buf));
  snprintf(buf, sizeof buf, "%s.mlp_in", nm);
  CHECK(need(w->mlp_in, buf));
  snprintf(buf, sizeof buf, "%s.mlp_out", nm);
  CHECK(need(w->mlp_out, buf));
  snprintf(buf, sizeof buf, "%s.q_norm", nm);
  CHECK(need(w->q_norm, buf));
  snprintf(buf, sizeof buf, "%s.k_norm", nm);
  CHECK(need(w->k_norm, buf));
  return FLUX_OK;
}

// in[s] / out[s]: stream residuals [B*N_s, D] of in_dt / out_dt; mods[s]: [B, 6D] f32
// Slot of the reference cache as extra attention keys
static KvExtra extra_keys(const flux_cfg* c, const RefSlot* ref, int B) {
  KvExtra x{};
  const int D = c->dim, es = esize(c->dtype);
  x.k = static_cast<const char*>(ref->qk) + (size_t)D * es;  // k columns of the q | k rows
  x.bs = (int64_t)ref->n * 2 * D;
  x.ld = 2 * D;
  x.vt = ref->vt;
  x.ld_vt = vt_pitch(ref->n);
  x.n = ref->n;
  x.nb = B;
  return x;
}

// ref_use == REF_FILL: Nt must be 0 and the image stream is the reference tokens; their
// q | k and V^T go to the slot.  REF_KEYS: the slot's tokens are extra keys of the
// attention.
static int run_double(const flux_cfg* c, const flux_stream_weights* sw[2], int B, int Ni, int Nt,
                      const void* in[2], int in_dt, void* out[2], int out_dt,
                      const float* mods[2], const float2* cs, const DoubleScratch& d,
                      hipStream_t s, const RefSlot* ref = nullptr, int ref_use = REF_NONE) {
  const int D = c->dim, H = c->mlp_hidden, T = c->dtype, TB = blk_dtype(c);
  const int n[2] = {Nt, Ni};
  const int64_t mbs = 6 * (int64_t)D;
  const int L = Nt + Ni;
  const int64_t ldvt = vt_pitch(L);
  const bool fill = ref_use == REF_FILL;
  void* qk[2] = {d.qk[0], fill ? ref->qk : d.qk[1]};
  void* vtb = fill ? ref->vt : d.vt;
  const int P = planes(c);
  // LayerNorm + modulate into ln (two planes: hi | lo with FLUX_PRECISION_SPLIT)
  auto ln_mod = [&](int dt, const void* x, void* y, int rows, int rpb, const float* sh,
                    const float* sc) -> hipError_t {
    if (P == 2)
      return layernorm_modulate_hilo(dt, x, D, y, 2 * D, rows, D, rpb, sh, sc, mbs, c->eps, s);
    return layernorm_modulate(dt, TB, x, D, y, D, rows, D, rpb, sh, sc, mbs, c->eps, s);
  };
  // timing-hook sites: the block's launches (both streams' products in one launch), unless
  // the block is filling the reference cache
  auto site = [&](int id) { return fill ? 0 : id; };
  // The two streams' products share N and K: each linear runs as one launch, the image
  // stream's tiles first (whole rounds at the common sizes) and the text stream's after them.
  for (int i = 0; i < 2; ++i)
    if (n[i] > 0) HIP_TRY(ln_mod(in_dt, in[i], d.ln[i], B * n[i], n[i], mods[i], mods[i] + D));
  {
    TimedSite ts(site(FLUX_SITE_DOUBLE_QKV), s);
    HIP_TRY(linear_pair(TB, qkv_args(c, B * Ni, d.ln[1], sw[1]->qkv, qk[1], vtb, ldvt, Nt, Ni,
                                    d.split),
                        qkv_args(c, B * Nt, d.ln[0], sw[0]->qkv, qk[0], vtb, ldvt, 0, Nt,
                                 d.split),
                        s));
  }
  if (ldvt > L) HIP_TRY(zero_cols(T, vtb, ldvt, (int64_t)B * D, L, (int)ldvt, s));
  // joint views: segment 0 = text rows, segment 1 = image rows
  const int es = esize(T);
  auto view = [&](int col, void* const* bufs, int64_t ld) {
    SeqView v;
    v.base0 = static_cast<char*>(bufs[0]) + (size_t)col * es;
    v.base1 = static_cast<char*>(bufs[1]) + (size_t)col * es;
    v.bs0 = (int64_t)Nt * ld;
    v.bs1 = (int64_t)Ni * ld;
    v.ld = ld;
    v.n0 = Nt;
    return v;
  };
  SeqView qv = view(0, qk, 2 * D), kv = view(D, qk, 2 * D);
  SeqView ov = view(0, d.o, D);
  HIP_TRY(qk_norm_rope(T, qv, kv, B, L, c->heads, sw[0]->q_norm, sw[0]->k_norm, sw[1]->q_norm,
                       sw[1]->k_norm, cs, c->eps, s));
  KvExtra xk{};
  if (ref_use == REF_KEYS) xk = extra_keys(c, ref, B);
  {
    TimedSite ts(site(FLUX_SITE_DOUBLE_ATTENTION), s);
    HIP_TRY(attention(T, qv, kv, vtb, ldvt, ov, B, L, c->heads, d.split, s,
                      ref_use == REF_KEYS ? &xk : nullptr, TB));
  }
  // x + gate1 * (O W_o^T)  -> mid (f32)
  auto out_args = [&](int i) {
    return lin_args(EPI_GATED_RESIDUAL, B * n[i], D, D, d.o[i], D, sw[i]->out, D, d.mid[i], D,
                    FLUX_F32, in[i], D, in_dt, mods[i] + 2 * D, mbs, n[i], d.split);
  };
  {
    TimedSite ts(site(FLUX_SITE_DOUBLE_OUT), s);
    HIP_TRY(linear_pair(TB, out_args(1), out_args(0), s));
  }
  for (int i = 0; i < 2; ++i)
    if (n[i] > 0)
      HIP_TRY(ln_mod(FLUX_F32, d.mid[i], d.ln[i], B * n[i], n[i], mods[i] + 3 * D,
                     mods[i] + 4 * D));
  auto mlp_in_args = [&](int i) {
    return lin_args(EPI_SWIGLU, B * n[i], 2 * H, P * D, d.ln[i], P * D, sw[i]->mlp_in, D,
                    d.mlp[i], P * H, TB, nullptr, 0, 0, nullptr, 0, 1, d.split, (P - 1) * D,
                    P == 2);
  };
  {
    TimedSite ts(site(FLUX_SITE_DOUBLE_MLP_IN), s);
    HIP_TRY(linear_pair(TB, mlp_in_args(1), mlp_in_args(0), s));
  }
  // mid + gate2 * (M W_out^T) -> out
  auto mlp_out_args = [&](int i) {
    return lin_args(EPI_GATED_RESIDUAL, B * n[i], D, P * H, d.mlp[i], P * H, sw[i]->mlp_out, H,
                    out[i], D, out_dt, d.mid[i], D, FLUX_F32, mods[i] + 5 * D, mbs, n[i],
                    d.split, (P - 1) * H);
  };
  TimedSite ts(site(FLUX_SITE_DOUBLE_MLP_OUT), s);
  HIP_TRY(linear_pair(TB, mlp_out_args(1), mlp_out_args(0), s));
  return FLUX_OK;
}

extern "C" size_t flux_double_block_workspace_size(const flux_cfg* c, int B, int Ni, int Nt) {
  if (check_cfg(c) != FLUX_OK || check_sizes(B, Ni, Nt) != FLUX_OK) return 0;
  Carver cv(nullptr);
  carve_cond(cv, B, c->dim);
  cv.take<float>((size_t)B * 12 * c->dim);
  carve_rope(cv, Ni + Nt);
  carve_double(cv, c, B, Ni, Nt);
  return cv.off;
}

extern "C" int flux_double_block_fwd(const flux_cfg* c, const flux_double_weights* w,
                                     const float* t, int B, int Ni, int Nt, const void* img,
                                     const void* txt, const int32_t* img_ids,
                                     const int32_t* txt_ids, void* img_out, void* txt_out,
                                     void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  CHECK(check_sizes(B, Ni, Nt));
  if (!w) return fail(FLUX_EINVAL, "weights is NULL");
  if (!t) return fail(FLUX_EINVAL, "t is NULL");
  CHECK(check_temb(&w->temb));
  CHECK(need(w->mod_img, "mod_img"));
  CHECK(need(w->mod_txt, "mod_txt"));
  CHECK(check_stream(&w->img, "img"));
  CHECK(check_stream(&w->txt, "txt"));
  CHECK(need(img, "img"));
  CHECK(need(img_out, "img_out"));
  if (!img_ids) return fail(FLUX_EINVAL, "img_ids is NULL");
  if (Nt > 0) {
    CHECK(need(txt, "txt"));
    CHECK(need(txt_out, "txt_out"));
    if (!txt_ids) return fail(FLUX_EINVAL, "txt_ids is NULL");
  }
  const size_t want = flux_double_block_workspace_size(c, B, Ni, Nt);
  CHECK(check_ws(ws, ws_bytes, want));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = c->dim;

  Carver cv(ws);
  CondBufs cb = carve_cond(cv, B, D);
  float* mods = cv.take<float>((size_t)B * 12 * D);
  RopeBufs rb = carve_rope(cv, Ni + Nt);
  DoubleScratch d = carve_double(cv, c, B, Ni, Nt);

  CHECK(run_cond(c, &w->temb, t, B, cb, s));
  float* mod_txt = mods;
  float* mod_img = mods + (size_t)B * 6 * D;
  HIP_TRY(gemv(c->dtype, w->mod_txt, 6 * D, D, cb.stemb, B, false, false, mod_txt, s));
  HIP_TRY(gemv(c->dtype, w->mod_img, 6 * D, D, cb.stemb, B, false, false, mod_img, s));
  HIP_TRY(rope_table(txt_ids, img_ids, Nt, Ni, c->axes_dim, c->rope_theta, rb.pos, rb.cs, s));

  const flux_stream_weights* sw[2] = {&w->txt, &w->img};
  const void* in[2] = {txt, img};
  void* out[2] = {txt_out, img_out};
  const float* md[2] = {mod_txt, mod_img};
  return run_double(c, sw, B, Ni, Nt, in, c->dtype, out, c->dtype, md, rb.cs, d, s);
}

// ------------------------------------------------------------------------------------
// single-stream block (on the merged [txt ; img] sequence)
// ------------------------------------------------------------------------------------
struct SingleScratch {
  void* ln;   // [B*L, D]  (hi | lo planes: [B*L, 2D])
  void* qk;   // [B*L, 2D] q | k
  void* vt;   // [B*D, vt_pitch(L)] V^T
  void* cat;  // [B*L, D + H]  = [attention output | SwiGLU output]
              // (hi / lo: [B*L, D + 2H] = [attention output | SwiGLU hi | SwiGLU lo])
  float* split;  // split-K scratch of the linear layers
};

static SingleScratch carve_single(Carver& cv, const flux_cfg* c, int B, int L) {
  SingleScratch d;
  const int es = esize(c->dtype), P = planes(c);
  const size_t rows = (size_t)B * L;
  d.ln = cv.take<char>(rows * P * c->dim * es);
  d.qk = cv.take<char>(rows * 2 * c->dim * es);
  d.vt = cv.take<char>((size_t)B * c->dim * vt_pitch(L) * es);
  d.cat = cv.take<char>(rows * (c->dim + P * c->mlp_hidden) * es);
  d.split = cv.take<float>(split_scratch_bytes() / sizeof(float));
  return d;
}

static int check_single_w(const flux_single_weights* w, bool with_mod) {
  if (with_mod) {
    CHECK(check_temb(&w->temb));
    CHECK(need(w->mod, "mod"));
  }
  CHECK(need(w->linear1, "linear1"));
  CHECK(need(w->linear2, "linear2"));
  CHECK(need(w->q_norm, "q_norm"));
  CHECK(need(w->k_norm, "k_norm"));
  return FLUX_OK;
}

// x: merged [B*L, D] of in_dt; out: [B*L, D] of out_dt (may alias x); mod [B, 3D]
// ref_use == REF_FILL: the sequence is the reference tokens; their q | k and V^T go to the
// slot, and with kv_only the block stops there (the last block: its output is not needed).
// REF_KEYS: the slot's tokens are extra keys of the attention.
static int run_single(const flux_cfg* c, const flux_single_weights* w, int B, int L, const void* x,
                      int in_dt, void* out, int out_dt, const float* mod, const float2* cs,
                      const SingleScratch& d, hipStream_t s, const RefSlot* ref = nullptr,
                      int ref_use = REF_NONE, bool kv_only = false) {
  const int D = c->dim, H = c->mlp_hidden, T = c->dtype, es = esize(T), P = planes(c);
  const int TB = blk_dtype(c);  // es is also its size: 2 bytes for bf16 and binary16
  const int rows = B * L;
  const int64_t mbs = 3 * (int64_t)D, ldc = D + P * H;
  const bool fill = ref_use == REF_FILL;
  void* qkb = fill ? ref->qk : d.qk;
  void* vtb = fill ? ref->vt : d.vt;
  if (P == 2)
    HIP_TRY(layernorm_modulate_hilo(in_dt, x, D, d.ln, 2 * D, rows, D, L, mod, mod + D, mbs,
                                    c->eps, s));
  else
    HIP_TRY(layernorm_modulate(in_dt, TB, x, D, d.ln, D, rows, D, L, mod, mod + D, mbs, c->eps, s));
  const int64_t ldvt = vt_pitch(L);
  {
    TimedSite ts(fill ? 0 : FLUX_SITE_SINGLE_QKV, s);
    CHECK(lin_qkv(c, rows, d.ln, w->linear1, qkb, vtb, ldvt, 0, L, s, d.split));
  }
  if (ldvt > L) HIP_TRY(zero_cols(T, vtb, ldvt, (int64_t)B * D, L, (int)ldvt, s));
  const char* w_mlp = static_cast<const char*>(w->linear1) + (size_t)3 * D * D * es;
  if (kv_only) {
    SeqView qv, kv;
    qv.base0 = qv.base1 = qkb;
    kv.base0 = kv.base1 = static_cast<char*>(qkb) + (size_t)D * es;
    qv.bs0 = qv.bs1 = kv.bs0 = kv.bs1 = (int64_t)L * 2 * D;
    qv.ld = kv.ld = 2 * D;
    qv.n0 = kv.n0 = L;
    HIP_TRY(qk_norm_rope(T, qv, kv, B, L, c->heads, w->q_norm, w->k_norm, w->q_norm, w->k_norm,
                         cs, c->eps, s));
    return FLUX_OK;
  }
  {
    TimedSite ts(fill ? 0 : FLUX_SITE_SINGLE_MLP_IN, s);
    CHECK(lin_b(c, EPI_SWIGLU, rows, 2 * H, P * D, d.ln, P * D, w_mlp, D,
              static_cast<char*>(d.cat) + (size_t)D * es, ldc, TB, nullptr, 0, 0, nullptr, 0, 1,
              s, d.split, (P - 1) * D, P == 2));
  }
  auto view = [&](void* base, int col, int64_t ld) {
    SeqView v;
    v.base0 = v.base1 = static_cast<char*>(base) + (size_t)col * es;
    v.bs0 = v.bs1 = (int64_t)L * ld;
    v.ld = ld;
    v.n0 = L;
    return v;
  };
  SeqView qv = view(qkb, 0, 2 * D), kv = view(qkb, D, 2 * D);
  SeqView ov = view(d.cat, 0, ldc);
  HIP_TRY(qk_norm_rope(T, qv, kv, B, L, c->heads, w->q_norm, w->k_norm, w->q_norm, w->k_norm, cs,
                       c->eps, s));
  {
    TimedSite ts(fill ? 0 : FLUX_SITE_SINGLE_ATTENTION, s);
    KvExtra xk{};
    if (ref_use == REF_KEYS) xk = extra_keys(c, ref, B);
    HIP_TRY(attention(T, qv, kv, vtb, ldvt, ov, B, L, c->heads, d.split, s,
                      ref_use == REF_KEYS ? &xk : nullptr, TB));
  }
  TimedSite ts(fill ? 0 : FLUX_SITE_SINGLE_LINEAR2, s);
  // [O | M] W2^T, or with hi / lo [O | M_hi | M_lo] whose M_lo columns repeat W2's M columns
  CHECK(lin_b(c, EPI_GATED_RESIDUAL, rows, D, (int)ldc, d.cat, ldc, w->linear2, D + H, out, D,
            out_dt, x, D, in_dt, mod + 2 * D, mbs, L, s, d.split, (P - 1) * H));
  return FLUX_OK;
}

static SeqView stream_view(const void* txt, const void* img, int Nt, int Ni, int D) {
  SeqView v;
  v.base0 = const_cast<void*>(txt);
  v.base1 = const_cast<void*>(img);
  v.bs0 = (int64_t)Nt * D;
  v.bs1 = (int64_t)Ni * D;
  v.ld = D;
  v.n0 = Nt;
  return v;
}

static SeqView merged_view(void* base, int L, int D) {
  SeqView v;
  v.base0 = v.base1 = base;
  v.bs0 = v.bs1 = (int64_t)L * D;
  v.ld = D;
  v.n0 = L;
  return v;
}

extern "C" size_t flux_single_block_workspace_size(const flux_cfg* c, int B, int Ni, int Nt) {
  if (check_cfg(c) != FLUX_OK || check_sizes(B, Ni, Nt) != FLUX_OK) return 0;
  const int L = Ni + Nt;
  Carver cv(nullptr);
  carve_cond(cv, B, c->dim);
  cv.take<float>((size_t)B * 3 * c->dim);
  carve_rope(cv, L);
  cv.take<char>((size_t)B * L * c->dim * esize(c->dtype));
  carve_single(cv, c, B, L);
  return cv.off;
}

extern "C" int flux_single_block_fwd(const flux_cfg* c, const flux_single_weights* w,
                                     const float* t, int B, int Ni, int Nt, const void* img,
                                     const void* txt, const int32_t* img_ids,
                                     const int32_t* txt_ids, void* img_out, void* txt_out,
                                     void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  CHECK(check_sizes(B, Ni, Nt));
  if (!w) return fail(FLUX_EINVAL, "weights is NULL");
  if (!t) return fail(FLUX_EINVAL, "t is NULL");
  CHECK(check_single_w(w, true));
  CHECK(need(img, "img"));
  CHECK(need(img_out, "img_out"));
  if (!img_ids) return fail(FLUX_EINVAL, "img_ids is NULL");
  if (Nt > 0) {
    CHECK(need(txt, "txt"));
    CHECK(need(txt_out, "txt_out"));
    if (!txt_ids) return fail(FLUX_EINVAL, "txt_ids is NULL");
  }
  const size_t want = flux_single_block_workspace_size(c, B, Ni, Nt);
  CHECK(check_ws(ws, ws_bytes, want));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int D = c->dim, L = Ni + Nt, T = c->dtype;

  Carver cv(ws);
  CondBufs cb = carve_cond(cv, B, D);
  float* mod = cv.take<float>((size_t)B * 3 * D);
  RopeBufs rb = carve_rope(cv, L);
  void* xm = cv.take<char>((size_t)B * L * D * esize(T));
  SingleScratch d = carve_single(cv, c, B, L);

  CHECK(run_cond(c, &w->temb, t, B, cb, s));
  HIP_TRY(gemv(T, w->mod, 3 * D, D, cb.stemb, B, false, false, mod, s));
  HIP_TRY(rope_table(txt_ids, img_ids, Nt, Ni, c->axes_dim, c->rope_theta, rb.pos, rb.cs, s));
  // merge [txt ; img] -> xm, run in place, split back
  HIP_TRY(copy_rows(T, stream_view(txt, img, Nt, Ni, D), T, merged_view(xm, L, D), B, L, D, s));
  CHECK(run_single(c, w, B, L, xm, T, xm, T, mod, rb.cs, d, s));
  HIP_TRY(copy_rows(T, merged_view(xm, L, D), T, stream_view(txt_out, img_out, Nt, Ni, D), B, L, D,
                    s));
  return FLUX_OK;
}

// ------------------------------------------------------------------------------------
// denoiser step
// ------------------------------------------------------------------------------------
struct StepBufs {
  CondBufs cb;
  float* mod_dimg;
  float* mod_dtxt;
  float* mod_single;
  float* mod_final;
  RopeBufs rb;
  float* res;      // merged residual [B, L, D] f32
  float* res_txt;  // double-phase stream residuals (alias into res when B == 1)
  float* res_img;
  void* ln_head;   // [B*Ni, D] compute dtype; bf16: [B*Ni, 2D] hi | lo planes
  DoubleScratch d;
  SingleScratch sg;
};

static StepBufs carve_step(Carver& cv, const flux_cfg* c, int B, int Ni, int Nt) {
  StepBufs sb;
  const int D = c->dim, L = Ni + Nt;
  sb.cb = carve_cond(cv, B, D);
  sb.mod_dimg = cv.take<float>((size_t)B * 6 * D);
  sb.mod_dtxt = cv.take<float>((size_t)B * 6 * D);
  sb.mod_single = cv.take<float>((size_t)B * 3 * D);
  sb.mod_final = cv.take<float>((size_t)B * 2 * D);
  sb.rb = carve_rope(cv, L);
  sb.res = cv.take<float>((size_t)B * L * D);
  if (B == 1) {
    sb.res_txt = sb.res;
    sb.res_img = sb.res + (size_t)Nt * D;
  } else {
    sb.res_txt = cv.take<float>((size_t)B * Nt * D);
    sb.res_img = cv.take<float>((size_t)B * Ni * D);
  }
  const bool hilo = c->dtype == FLUX_BF16;
  sb.ln_head = cv.take<char>((size_t)B * Ni * D * esize(c->dtype) * (hilo ? 2 : 1));
  // block scratch: the double and single phases never overlap, so they share memory
  Carver dc(cv.base ? cv.base + ((cv.off + 255) & ~size_t(255)) : nullptr);
  sb.d = carve_double(dc, c, B, Ni, Nt);
  Carver sc(cv.base ? cv.base + ((cv.off + 255) & ~size_t(255)) : nullptr);
  sb.sg = carve_single(sc, c, B, L);
  cv.off = ((cv.off + 255) & ~size_t(255)) + (dc.off > sc.off ? dc.off : sc.off);
  return sb;
}

extern "C" size_t flux_denoiser_step_workspace_size(const flux_cfg* c, int B, int Ni, int Nt) {
  if (check_cfg(c) != FLUX_OK || check_sizes(B, Ni, Nt) != FLUX_OK) return 0;
  Carver cv(nullptr);
  carve_step(cv, c, B, Ni, Nt);
  return cv.off;
}

// configuration and weights of a denoiser step (everything but the per-call buffers)
static int check_model(const flux_cfg* c, const flux_model_weights* w, int B, int Ni, int Nt) {
  CHECK(check_cfg(c));
  CHECK(check_sizes(B, Ni, Nt));
  if (!w) return fail(FLUX_EINVAL, "weights is NULL");
  if (c->in_channels <= 0 || c->in_channels % 8)
    return fail(FLUX_ESHAPE, "in_channels must be a positive multiple of 8");
  if (Nt > 0 && (c->context_dim <= 0 || c->context_dim % 8))
    return fail(FLUX_ESHAPE, "context_dim must be a positive multiple of 8");
  if (c->n_double < 0 || c->n_single < 0) return fail(FLUX_EINVAL, "negative block count");
  CHECK(need(w->img_in, "img_in"));
  CHECK(check_temb(&w->temb));
  CHECK(need(w->mod_double_img, "mod_double_img"));
  CHECK(need(w->mod_double_txt, "mod_double_txt"));
  CHECK(need(w->mod_single, "mod_single"));
  CHECK(need(w->mod_final, "mod_final"));
  CHECK(need(w->proj_out, "proj_out"));
  if (c->n_double > 0 && !w->double_blocks) return fail(FLUX_EINVAL, "double_blocks is NULL");
  if (c->n_single > 0 && !w->single_blocks) return fail(FLUX_EINVAL, "single_blocks is NULL");
  for (int i = 0; i < c->n_double; ++i) {
    CHECK(check_stream(&w->double_blocks[i].img, "double.img"));
    CHECK(check_stream(&w->double_blocks[i].txt, "double.txt"));
  }
  for (int i = 0; i < c->n_single; ++i) CHECK(check_single_w(&w->single_blocks[i], false));
  if (Nt > 0) CHECK(need(w->txt_in, "txt_in"));
  return FLUX_OK;
}

// launch sequence of one validated step; ws holds flux_denoiser_step_workspace_size bytes
static RefSlot ref_slot(const flux_cfg* c, const void* cache, int B, int Nr, int layer);

// launch sequence of one validated step; ws holds flux_denoiser_step_workspace_size bytes.
// With a reference cache (Nr > 0), every block also attends to its slot's reference keys.
static int run_step(const flux_cfg* c, const flux_model_weights* w, const float* t, int B,
                    int Ni, int Nt, const void* x, const void* ctx, const int32_t* img_ids,
                    const int32_t* txt_ids, float* out, void* ws, hipStream_t s,
                    const void* cache = nullptr, int Nr = 0) {
  const int use = (cache != nullptr && Nr > 0) ? REF_KEYS : REF_NONE;
  const int D = c->dim, L = Ni + Nt, T = c->dtype;
  Carver cv(ws);
  StepBufs sb = carve_step(cv, c, B, Ni, Nt);

  // conditioning, shared modulation, rope tables
  CHECK(run_cond(c, &w->temb, t, B, sb.cb, s));
  HIP_TRY(gemv(T, w->mod_double_img, 6 * D, D, sb.cb.stemb, B, false, false, sb.mod_dimg, s));
  HIP_TRY(gemv(T, w->mod_double_txt, 6 * D, D, sb.cb.stemb, B, false, false, sb.mod_dtxt, s));
  HIP_TRY(gemv(T, w->mod_single, 3 * D, D, sb.cb.stemb, B, false, false, sb.mod_single, s));
  HIP_TRY(gemv(T, w->mod_final, 2 * D, D, sb.cb.stemb, B, false, false, sb.mod_final, s));
  HIP_TRY(rope_table(txt_ids, img_ids, Nt, Ni, c->axes_dim, c->rope_theta, sb.rb.pos, sb.rb.cs, s));

  // stems (fp32 residual stream); the block scratch is idle until the first block, so its
  // split-K area serves their tails
  CHECK(lin(c, EPI_STORE, B * Ni, D, c->in_channels, x, c->in_channels, w->img_in, c->in_channels,
            sb.res_img, D, FLUX_F32, nullptr, 0, 0, nullptr, 0, 1, s, sb.d.split));
  if (Nt > 0)
    CHECK(lin(c, EPI_STORE, B * Nt, D, c->context_dim, ctx, c->context_dim, w->txt_in,
              c->context_dim, sb.res_txt, D, FLUX_F32, nullptr, 0, 0, nullptr, 0, 1, s, sb.d.split));

  // double-stream blocks
  const void* in[2] = {sb.res_txt, sb.res_img};
  void* io[2] = {sb.res_txt, sb.res_img};
  const float* md[2] = {sb.mod_dtxt, sb.mod_dimg};
  for (int i = 0; i < c->n_double; ++i) {
    const flux_stream_weights* sw[2] = {&w->double_blocks[i].txt, &w->double_blocks[i].img};
    const RefSlot slot = use ? ref_slot(c, cache, B, Nr, i) : RefSlot{};
    CHECK(run_double(c, sw, B, Ni, Nt, in, FLUX_F32, io, FLUX_F32, md, sb.rb.cs, sb.d, s, &slot,
                     use));
  }
  // merge [txt ; img] (already merged when B == 1)
  if (B > 1)
    HIP_TRY(copy_rows(FLUX_F32, stream_view(sb.res_txt, sb.res_img, Nt, Ni, D), FLUX_F32,
                      merged_view(sb.res, L, D), B, L, D, s));
  // single-stream blocks
  for (int i = 0; i < c->n_single; ++i) {
    const RefSlot slot = use ? ref_slot(c, cache, B, Nr, c->n_double + i) : RefSlot{};
    CHECK(run_single(c, &w->single_blocks[i], B, L, sb.res, FLUX_F32, sb.res, FLUX_F32,
                     sb.mod_single, sb.rb.cs, sb.sg, s, &slot, use));
  }
  // head: keep image tokens, final LayerNorm + modulate, proj_out
  if (T == FLUX_BF16) {
    // The projection's input is the one bf16 operand whose rounding reaches the output
    // without passing another block: it is carried as bf16 hi + lo planes, and one GEMM
    // over K = 2D reads proj_out for both (fp32 accumulation).
    for (int b = 0; b < B; ++b) {
      const float* rows = sb.res + ((size_t)b * L + Nt) * D;
      void* lnb = static_cast<char*>(sb.ln_head) + (size_t)b * Ni * 2 * D * 2;
      HIP_TRY(layernorm_modulate_hilo(FLUX_F32, rows, D, lnb, 2 * D, Ni, D, Ni,
                                      sb.mod_final + (size_t)b * 2 * D,
                                      sb.mod_final + (size_t)b * 2 * D + D, 2 * D, c->eps, s));
    }
    CHECK(lin(c, EPI_STORE, B * Ni, c->in_channels, 2 * D, sb.ln_head, 2 * D, w->proj_out, D,
              out, c->in_channels, FLUX_F32, nullptr, 0, 0, nullptr, 0, 1, s, sb.sg.split, D));
    return FLUX_OK;
  }
  for (int b = 0; b < B; ++b) {
    const float* rows = sb.res + ((size_t)b * L + Nt) * D;
    void* lnb = static_cast<char*>(sb.ln_head) + (size_t)b * Ni * D * esize(T);
    HIP_TRY(layernorm_modulate(FLUX_F32, T, rows, D, lnb, D, Ni, D, Ni,
                               sb.mod_final + (size_t)b * 2 * D, sb.mod_final + (size_t)b * 2 * D + D,
                               2 * D, c->eps, s));
  }
  CHECK(lin(c, EPI_STORE, B * Ni, c->in_channels, D, sb.ln_head, D, w->proj_out, D, out,
            c->in_channels, FLUX_F32, nullptr, 0, 0, nullptr, 0, 1, s, sb.sg.split));
  return FLUX_OK;
}

extern "C" int flux_denoiser_step(const flux_cfg* c, const flux_model_weights* w, const float* t,
                                  const float* guidance, int B, int Ni, int Nt, const void* x,
                                  const void* ctx, const int32_t* img_ids,
                                  const int32_t* txt_ids, float* out, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (guidance) return fail(FLUX_EINVAL, "guidance must be NULL (no guidance embedder)");
  CHECK(check_model(c, w, B, Ni, Nt));
  if (!t) return fail(FLUX_EINVAL, "t is NULL");
  CHECK(need(x, "x"));
  CHECK(need(out, "out"));
  if (!img_ids) return fail(FLUX_EINVAL, "img_ids is NULL");
  if (Nt > 0) {
    CHECK(need(ctx, "ctx"));
    if (!txt_ids) return fail(FLUX_EINVAL, "txt_ids is NULL");
  }
  CHECK(check_ws(ws, ws_bytes, flux_denoiser_step_workspace_size(c, B, Ni, Nt)));
  return run_step(c, w, t, B, Ni, Nt, x, ctx, img_ids, txt_ids, out, ws,
                  static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------------------------
// sampling loop ([KLEIN] 训练方法: rectified flow, 4 distilled steps or 50 base steps with
// classifier-free guidance; [DIFF] pipeline call chain: packed latents and ids, a
// flow-matching Euler scheduler calling the transformer once per step)
// ------------------------------------------------------------------------------------
struct SampleBufs {
  float* x;        // state [B, Ni, in_ch] fp32
  void* xin;       // model input [Bm, Ni, in_ch] (model dtype)
  float* v;        // velocity [Bm, Ni, in_ch] fp32
  void* ctx2;      // [cond ; uncond] condition [2B, Nt, ctx_dim] (guided only)
  float* t;        // [Bm]
  int32_t* img_ids;
  int32_t* txt_ids;
  void* step_ws;
};

static SampleBufs carve_sample(Carver& cv, const flux_cfg* c, int B, int Ni, int Nt, bool guided) {
  SampleBufs sb;
  const int Bm = guided ? 2 * B : B, es = esize(c->dtype);
  const size_t tok = (size_t)Ni * c->in_channels;
  sb.x = cv.take<float>((size_t)B * tok);
  sb.xin = cv.take<char>((size_t)Bm * tok * es);
  sb.v = cv.take<float>((size_t)Bm * tok);
  sb.ctx2 = guided ? cv.take<char>((size_t)Bm * Nt * c->context_dim * es) : nullptr;
  sb.t = cv.take<float>((size_t)Bm);
  sb.img_ids = cv.take<int32_t>((size_t)Ni * 4);
  sb.txt_ids = cv.take<int32_t>((size_t)(Nt > 0 ? Nt : 1) * 4);
  sb.step_ws = cv.take<char>(flux_denoiser_step_workspace_size(c, Bm, Ni, Nt));
  return sb;
}

static int check_latent(int B, int C, int H, int W) {
  if (B <= 0 || C <= 0 || H <= 0 || W <= 0) return fail(FLUX_EINVAL, "sizes must be > 0");
  if (H % 2 || W % 2) return fail(FLUX_ESHAPE, "latent height and width must be even");
  if ((int64_t)B * C * H * W >= (int64_t{1} << 31))
    return fail(FLUX_ESHAPE, "latent has 2^31 or more elements");
  return FLUX_OK;
}

extern "C" size_t flux_denoise_workspace_size(const flux_cfg* c, int B, int latent_h,
                                              int latent_w, int Nt, int guided) {
  if (check_cfg(c) != FLUX_OK || c->in_channels <= 0 || c->in_channels % 8) return 0;
  if (check_latent(B, c->in_channels / 4, latent_h, latent_w) != FLUX_OK) return 0;
  const int Ni = (latent_h / 2) * (latent_w / 2);
  if (check_sizes(guided ? 2 * B : B, Ni, Nt) != FLUX_OK) return 0;
  Carver cv(nullptr);
  carve_sample(cv, c, B, Ni, Nt, guided != 0);
  return cv.off;
}

extern "C" int flux_denoise(const flux_cfg* c, const flux_model_weights* w, int n_steps,
                            const float* sigmas, float guidance_scale, int B, int latent_h,
                            int latent_w, int Nt, const float* noise, const void* ctx,
                            const void* ctx_uncond, float* latents_out, void* ws,
                            size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  if (c->in_channels <= 0 || c->in_channels % 8)
    return fail(FLUX_ESHAPE, "in_channels must be a positive multiple of 8");
  const int C = c->in_channels / 4;
  CHECK(check_latent(B, C, latent_h, latent_w));
  if (n_steps <= 0 || n_steps > 10000) return fail(FLUX_EINVAL, "n_steps must be in [1, 10000]");
  std::vector<float> sig(n_steps + 1);
  for (int i = 0; i <= n_steps; ++i)
    sig[i] = sigmas ? sigmas[i] : (float)(1.0 - (double)i / n_steps);
  for (int i = 0; i <= n_steps; ++i) {
    if (!std::isfinite(sig[i])) return fail(FLUX_EINVAL, "sigmas[%d] is not finite", i);
    if (i > 0 && !(sig[i] < sig[i - 1]))
      return fail(FLUX_EINVAL, "sigmas must decrease strictly (sigmas[%d] >= sigmas[%d])", i,
                  i - 1);
  }
  const bool guided = ctx_uncond != nullptr;
  if (guided && !std::isfinite(guidance_scale))
    return fail(FLUX_EINVAL, "guidance_scale is not finite");
  const int Ni = (latent_h / 2) * (latent_w / 2), Bm = guided ? 2 * B : B;
  CHECK(check_model(c, w, Bm, Ni, Nt));
  CHECK(need(noise, "noise"));
  CHECK(need(latents_out, "latents_out"));
  if (Nt > 0) CHECK(need(ctx, "ctx"));
  if (guided && Nt == 0) return fail(FLUX_EINVAL, "guidance needs a text condition (n_txt > 0)");
  if (guided) CHECK(need(ctx_uncond, "ctx_uncond"));
  CHECK(check_ws(ws, ws_bytes, flux_denoise_workspace_size(c, B, latent_h, latent_w, Nt, guided)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = c->dtype;
  Carver cv(ws);
  SampleBufs sb = carve_sample(cv, c, B, Ni, Nt, guided);
  const int64_t n = (int64_t)B * Ni * c->in_channels;

  HIP_TRY(generation_ids(sb.img_ids, latent_h / 2, latent_w / 2, sb.txt_ids, Nt, s));
  const void* cond = ctx;
  if (guided) {
    const size_t bytes = (size_t)B * Nt * c->context_dim * esize(T);
    HIP_TRY(hipMemcpyAsync(sb.ctx2, ctx, bytes, hipMemcpyDeviceToDevice, s));
    HIP_TRY(hipMemcpyAsync(static_cast<char*>(sb.ctx2) + bytes, ctx_uncond, bytes,
                           hipMemcpyDeviceToDevice, s));
    cond = sb.ctx2;
  }
  HIP_TRY(pack_latents(noise, sb.x, B, C, latent_h, latent_w, s));
  for (int i = 0; i < n_steps; ++i) {
    // x_i = x_{i-1} + (sigma_i - sigma_{i-1}) v_{i-1}, then the model input in its dtype
    HIP_TRY(sampler_update(T, sb.x, i ? sb.v : nullptr, n, i ? sig[i] - sig[i - 1] : 0.f,
                           guidance_scale, guided, sb.xin, sb.t, Bm, sig[i], s));
    CHECK(run_step(c, w, sb.t, Bm, Ni, Nt, sb.xin, cond, sb.img_ids, sb.txt_ids, sb.v,
                   sb.step_ws, s));
  }
  HIP_TRY(sampler_update(T, sb.x, sb.v, n, sig[n_steps] - sig[n_steps - 1], guidance_scale,
                         guided, nullptr, nullptr, 0, 0.f, s));
  HIP_TRY(unpack_latents(sb.x, latents_out, B, C, latent_h, latent_w, s));
  return FLUX_OK;
}

extern "C" int flux_pack_latents(int B, int C, int H, int W, const float* z, float* tokens,
                                 void* stream) {
  CHECK(check_latent(B, C, H, W));
  CHECK(need(z, "z"));
  CHECK(need(tokens, "tokens"));
  HIP_TRY(pack_latents(z, tokens, B, C, H, W, static_cast<hipStream_t>(stream)));
  return FLUX_OK;
}

extern "C" int flux_unpack_latents(int B, int C, int H, int W, const float* tokens, float* z,
                                   void* stream) {
  CHECK(check_latent(B, C, H, W));
  CHECK(need(tokens, "tokens"));
  CHECK(need(z, "z"));
  HIP_TRY(unpack_latents(tokens, z, B, C, H, W, static_cast<hipStream_t>(stream)));
  return FLUX_OK;
}

extern "C" int flux_generation_ids(int grid_h, int grid_w, int n_txt, int32_t* img_ids,
                                   int32_t* txt_ids, void* stream) {
  if (grid_h <= 0 || grid_w <= 0 || n_txt < 0)
    return fail(FLUX_EINVAL, "need grid_h, grid_w > 0 and n_txt >= 0");
  if ((int64_t)grid_h * grid_w + n_txt >= (int64_t{1} << 30))
    return fail(FLUX_ESHAPE, "too many tokens");
  CHECK(need(img_ids, "img_ids"));
  if (n_txt > 0) CHECK(need(txt_ids, "txt_ids"));
  HIP_TRY(generation_ids(img_ids, grid_h, grid_w, txt_ids, n_txt, static_cast<hipStream_t>(stream)));
  return FLUX_OK;
}

// ------------------------------------------------------------------------------------
// reference-image K/V cache ([DIFF] 参考图 KV 缓存机制: Flux2KVLayerCache per block,
// extract / cached modes; [KLEIN] Infra, KV 缓存).  Reference tokens attend only to
// reference tokens and are modulated at the fixed timestep 0, so their K/V do not depend
// on the noisy image, the text or t: the extract step is the reference-only forward that
// fills the cache (flux_ref_cache_fill) followed by the cached step.
// ------------------------------------------------------------------------------------
static size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

static void ref_slot_bytes(const flux_cfg* c, int B, int Nr, size_t& qk, size_t& vt) {
  const int es = esize(c->dtype);
  qk = align256((size_t)B * Nr * 2 * c->dim * es);
  vt = align256((size_t)B * c->dim * vt_pitch(Nr) * es);
}

static RefSlot ref_slot(const flux_cfg* c, const void* cache, int B, int Nr, int layer) {
  size_t qk, vt;
  ref_slot_bytes(c, B, Nr, qk, vt);
  char* base = const_cast<char*>(static_cast<const char*>(cache)) + (size_t)layer * (qk + vt);
  return RefSlot{base, base + qk, Nr};
}

extern "C" size_t flux_ref_cache_size(const flux_cfg* c, int B, int Nr) {
  if (check_cfg(c) != FLUX_OK || B <= 0 || Nr <= 0 || c->n_double < 0 || c->n_single < 0)
    return 0;
  size_t qk, vt;
  ref_slot_bytes(c, B, Nr, qk, vt);
  return (size_t)(c->n_double + c->n_single) * (qk + vt);
}

static int check_cache(const flux_cfg* c, const void* cache, size_t bytes, int B, int Nr) {
  const size_t want = flux_ref_cache_size(c, B, Nr);
  if (!cache) return fail(FLUX_EINVAL, "cache is NULL");
  if (reinterpret_cast<uintptr_t>(cache) & 255u)
    return fail(FLUX_EALIGN, "cache is not 256-byte aligned");
  if (bytes < want) return fail(FLUX_EWORKSPACE, "cache has %zu bytes, need %zu", bytes, want);
  return FLUX_OK;
}

extern "C" size_t flux_ref_cache_fill_workspace_size(const flux_cfg* c, int B, int Nr) {
  if (check_cfg(c) != FLUX_OK || check_sizes(B, Nr, 0) != FLUX_OK) return 0;
  Carver cv(nullptr);
  carve_step(cv, c, B, Nr, 0);
  cv.take<float>((size_t)B);
  return cv.off;
}

static int run_ref_fill(const flux_cfg* c, const flux_model_weights* w, int B, int Nr,
                        const void* ref_x, const int32_t* ref_ids, void* cache, void* ws,
                        hipStream_t s) {
  const int D = c->dim, T = c->dtype;
  Carver cv(ws);
  StepBufs sb = carve_step(cv, c, B, Nr, 0);
  float* t0 = cv.take<float>((size_t)B);
  HIP_TRY(sampler_update(T, nullptr, nullptr, 0, 0.f, 0.f, false, nullptr, t0, B, 0.f, s));
  CHECK(run_cond(c, &w->temb, t0, B, sb.cb, s));
  HIP_TRY(gemv(T, w->mod_double_img, 6 * D, D, sb.cb.stemb, B, false, false, sb.mod_dimg, s));
  HIP_TRY(gemv(T, w->mod_single, 3 * D, D, sb.cb.stemb, B, false, false, sb.mod_single, s));
  HIP_TRY(rope_table(ref_ids, ref_ids, 0, Nr, c->axes_dim, c->rope_theta, sb.rb.pos, sb.rb.cs, s));
  CHECK(lin(c, EPI_STORE, B * Nr, D, c->in_channels, ref_x, c->in_channels, w->img_in,
            c->in_channels, sb.res_img, D, FLUX_F32, nullptr, 0, 0, nullptr, 0, 1, s, sb.d.split));
  const void* in[2] = {sb.res_txt, sb.res_img};
  void* io[2] = {sb.res_txt, sb.res_img};
  const float* md[2] = {sb.mod_dimg, sb.mod_dimg};
  for (int i = 0; i < c->n_double; ++i) {
    const flux_stream_weights* sw[2] = {&w->double_blocks[i].txt, &w->double_blocks[i].img};
    const RefSlot slot = ref_slot(c, cache, B, Nr, i);
    CHECK(run_double(c, sw, B, Nr, 0, in, FLUX_F32, io, FLUX_F32, md, sb.rb.cs, sb.d, s, &slot,
                     REF_FILL));
  }
  if (B > 1)
    HIP_TRY(copy_rows(FLUX_F32, stream_view(sb.res_txt, sb.res_img, 0, Nr, D), FLUX_F32,
                      merged_view(sb.res, Nr, D), B, Nr, D, s));
  for (int i = 0; i < c->n_single; ++i) {
    const RefSlot slot = ref_slot(c, cache, B, Nr, c->n_double + i);
    CHECK(run_single(c, &w->single_blocks[i], B, Nr, sb.res, FLUX_F32, sb.res, FLUX_F32,
                     sb.mod_single, sb.rb.cs, sb.sg, s, &slot, REF_FILL, i == c->n_single - 1));
  }
  return FLUX_OK;
}

extern "C" int flux_ref_cache_fill(const flux_cfg* c, const flux_model_weights* w, int B, int Nr,
                                   const void* ref_x, const int32_t* ref_ids, void* cache,
                                   size_t cache_bytes, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_model(c, w, B, Nr, 0));
  CHECK(need(ref_x, "ref_x"));
  CHECK(need(ref_ids, "ref_ids"));
  CHECK(check_cache(c, cache, cache_bytes, B, Nr));
  CHECK(check_ws(ws, ws_bytes, flux_ref_cache_fill_workspace_size(c, B, Nr)));
  return run_ref_fill(c, w, B, Nr, ref_x, ref_ids, cache, ws, static_cast<hipStream_t>(stream));
}

extern "C" int flux_denoiser_step_cached(const flux_cfg* c, const flux_model_weights* w,
                                         const float* t, int B, int Ni, int Nt, int Nr,
                                         const void* x, const void* ctx, const int32_t* img_ids,
                                         const int32_t* txt_ids, const void* cache,
                                         size_t cache_bytes, float* out, void* ws,
                                         size_t ws_bytes, void* stream) {
  CHECK(check_model(c, w, B, Ni, Nt));
  if (Nr <= 0) return fail(FLUX_EINVAL, "n_ref must be > 0 (got %d)", Nr);
  if (!t) return fail(FLUX_EINVAL, "t is NULL");
  CHECK(need(x, "x"));
  CHECK(need(out, "out"));
  if (!img_ids) return fail(FLUX_EINVAL, "img_ids is NULL");
  if (Nt > 0) {
    CHECK(need(ctx, "ctx"));
    if (!txt_ids) return fail(FLUX_EINVAL, "txt_ids is NULL");
  }
  CHECK(check_cache(c, cache, cache_bytes, B, Nr));
  CHECK(check_ws(ws, ws_bytes, flux_denoiser_step_workspace_size(c, B, Ni, Nt)));
  return run_step(c, w, t, B, Ni, Nt, x, ctx, img_ids, txt_ids, out, ws,
                  static_cast<hipStream_t>(stream), cache, Nr);
}

// sampling with reference latents [B, R, C, ref_h, ref_w]: packed references (ids
// (1 + j, r, c, 0)), the cache filled once (use_cache) or before every step
struct RefSampleBufs {
  float* ref_f;     // packed references [B, Nr, in_ch] fp32
  void* ref_in;     // the same in the model dtype
  int32_t* ref_ids;
  void* cache;
  void* run_ws;     // step / fill workspace (never used at the same time)
};

static RefSampleBufs carve_ref_sample(Carver& cv, const flux_cfg* c, int B, int Ni, int Nt,
                                      int Nr) {
  RefSampleBufs r;
  const size_t tok = (size_t)B * Nr * c->in_channels;
  r.ref_f = cv.take<float>(tok);
  r.ref_in = cv.take<char>(tok * esize(c->dtype));
  r.ref_ids = cv.take<int32_t>((size_t)Nr * 4);
  r.cache = cv.take<char>(flux_ref_cache_size(c, B, Nr));
  const size_t a = flux_denoiser_step_workspace_size(c, B, Ni, Nt);
  const size_t f = flux_ref_cache_fill_workspace_size(c, B, Nr);
  r.run_ws = cv.take<char>(a > f ? a : f);
  return r;
}

extern "C" size_t flux_denoise_refs_workspace_size(const flux_cfg* c, int B, int latent_h,
                                                   int latent_w, int Nt, int n_refs, int ref_h,
                                                   int ref_w) {
  if (check_cfg(c) != FLUX_OK || c->in_channels <= 0 || c->in_channels % 8) return 0;
  const int C = c->in_channels / 4;
  if (check_latent(B, C, latent_h, latent_w) != FLUX_OK || n_refs <= 0 ||
      check_latent(B * n_refs, C, ref_h, ref_w) != FLUX_OK)
    return 0;
  const int Ni = (latent_h / 2) * (latent_w / 2), Nr = n_refs * (ref_h / 2) * (ref_w / 2);
  if (check_sizes(B, Ni, Nt) != FLUX_OK) return 0;
  Carver cv(nullptr);
  SampleBufs sb = carve_sample(cv, c, B, Ni, Nt, false);
  (void)sb;
  carve_ref_sample(cv, c, B, Ni, Nt, Nr);
  return cv.off;
}

extern "C" int flux_denoise_refs(const flux_cfg* c, const flux_model_weights* w, int n_steps,
                                 const float* sigmas, int B, int latent_h, int latent_w, int Nt,
                                 const float* noise, const void* ctx, int n_refs, int ref_h,
                                 int ref_w, const float* refs, int use_cache, float* latents_out,
                                 void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  if (c->in_channels <= 0 || c->in_channels % 8)
    return fail(FLUX_ESHAPE, "in_channels must be a positive multiple of 8");
  const int C = c->in_channels / 4;
  CHECK(check_latent(B, C, latent_h, latent_w));
  if (n_refs <= 0) return fail(FLUX_EINVAL, "n_refs must be > 0 (use flux_denoise without)");
  CHECK(check_latent(B * n_refs, C, ref_h, ref_w));
  if (n_steps <= 0 || n_steps > 10000) return fail(FLUX_EINVAL, "n_steps must be in [1, 10000]");
  std::vector<float> sig(n_steps + 1);
  for (int i = 0; i <= n_steps; ++i)
    sig[i] = sigmas ? sigmas[i] : (float)(1.0 - (double)i / n_steps);
  for (int i = 0; i <= n_steps; ++i) {
    if (!std::isfinite(sig[i])) return fail(FLUX_EINVAL, "sigmas[%d] is not finite", i);
    if (i > 0 && !(sig[i] < sig[i - 1]))
      return fail(FLUX_EINVAL, "sigmas must decrease strictly (sigmas[%d] >= sigmas[%d])", i,
                  i - 1);
  }
  const int gh = ref_h / 2, gw = ref_w / 2;
  const int Ni = (latent_h / 2) * (latent_w / 2), Nr = n_refs * gh * gw;
  CHECK(check_model(c, w, B, Ni, Nt));
  CHECK(check_sizes(B, Nr, 0));
  CHECK(need(noise, "noise"));
  CHECK(need(refs, "refs"));
  CHECK(need(latents_out, "latents_out"));
  if (Nt > 0) CHECK(need(ctx, "ctx"));
  CHECK(check_ws(ws, ws_bytes, flux_denoise_refs_workspace_size(c, B, latent_h, latent_w, Nt,
                                                                 n_refs, ref_h, ref_w)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = c->dtype;
  Carver cv(ws);
  SampleBufs sb = carve_sample(cv, c, B, Ni, Nt, false);
  RefSampleBufs rb = carve_ref_sample(cv, c, B, Ni, Nt, Nr);
  const int64_t n = (int64_t)B * Ni * c->in_channels;

  HIP_TRY(generation_ids(sb.img_ids, latent_h / 2, latent_w / 2, sb.txt_ids, Nt, s));
  for (int j = 0; j < n_refs; ++j)
    HIP_TRY(generation_ids(rb.ref_ids + (size_t)j * gh * gw * 4, gh, gw, nullptr, 0, s, 1 + j));
  // references as [B * R] latents -> [B, R * gh * gw] tokens, then the model dtype
  HIP_TRY(pack_latents(refs, rb.ref_f, B * n_refs, C, ref_h, ref_w, s));
  HIP_TRY(sampler_update(T, rb.ref_f, nullptr, (int64_t)B * Nr * c->in_channels, 0.f, 0.f,
                         false, rb.ref_in, nullptr, 0, 0.f, s));
  HIP_TRY(pack_latents(noise, sb.x, B, C, latent_h, latent_w, s));
  for (int i = 0; i < n_steps; ++i) {
    if (i == 0 || !use_cache)
      CHECK(run_ref_fill(c, w, B, Nr, rb.ref_in, rb.ref_ids, rb.cache, rb.run_ws, s));
    HIP_TRY(sampler_update(T, sb.x, i ? sb.v : nullptr, n, i ? sig[i] - sig[i - 1] : 0.f, 1.f,
                           false, sb.xin, sb.t, B, sig[i], s));
    CHECK(run_step(c, w, sb.t, B, Ni, Nt, sb.xin, ctx, sb.img_ids, sb.txt_ids, sb.v, rb.run_ws,
                   s, rb.cache, Nr));
  }
  HIP_TRY(sampler_update(T, sb.x, sb.v, n, sig[n_steps] - sig[n_steps - 1], 1.f, false, nullptr,
                         nullptr, 0, 0.f, s));
  HIP_TRY(unpack_latents(sb.x, latents_out, B, C, latent_h, latent_w, s));
  return FLUX_OK;
}

// ------------------------------------------------------------------------------------
// single operations
// ------------------------------------------------------------------------------------
extern "C" int flux_rope_positions(const flux_cfg* c, const int32_t* txt_ids,
                                   const int32_t* img_ids, int n_txt, int n_img, int32_t* pos,
                                   void* stream) {
  CHECK(check_cfg(c));
  if (n_txt < 0 || n_img < 0 || n_txt + n_img <= 0)
    return fail(FLUX_EINVAL, "need n_txt >= 0, n_img >= 0 and at least one token");
  if ((n_txt && !txt_ids) || (n_img && !img_ids) || !pos)
    return fail(FLUX_EINVAL, "NULL pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  HIP_TRY(rope_table(txt_ids, img_ids, n_txt, n_img, c->axes_dim, c->rope_theta, pos, nullptr, s));
  return FLUX_OK;
}

extern "C" size_t flux_modulation_workspace_size(const flux_cfg* c, int B) {
  if (check_cfg(c) != FLUX_OK || B <= 0) return 0;
  Carver cv(nullptr);
  carve_cond(cv, B, c->dim);
  return cv.off;
}

extern "C" int flux_modulation(const flux_cfg* c, const flux_temb_weights* tw, const void* w_mod,
                               int n_out, const float* t, int B, float* out, void* ws,
                               size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  if (B <= 0 || n_out <= 0) return fail(FLUX_EINVAL, "batch and n_out must be > 0");
  if (!tw || !t || !out) return fail(FLUX_EINVAL, "NULL pointer");
  CHECK(check_temb(tw));
  CHECK(need(w_mod, "w_mod"));
  CHECK(check_ws(ws, ws_bytes, flux_modulation_workspace_size(c, B)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  CondBufs cb = carve_cond(cv, B, c->dim);
  CHECK(run_cond(c, tw, t, B, cb, s));
  HIP_TRY(gemv(c->dtype, w_mod, n_out, c->dim, cb.stemb, B, false, false, out, s));
  return FLUX_OK;
}

extern "C" int flux_layernorm_modulate(const flux_cfg* c, int rows, int rpb, const void* x,
                                       int x_dtype, const float* shift, const float* scale,
                                       void* y, void* stream) {
  CHECK(check_cfg(c));
  if (rows <= 0 || rpb <= 0) return fail(FLUX_EINVAL, "rows and rows_per_batch must be > 0");
  if (x_dtype != FLUX_BF16 && x_dtype != FLUX_F32) return fail(FLUX_EDTYPE, "bad x_dtype");
  CHECK(need(x, "x"));
  CHECK(need(y, "y"));
  CHECK(need(shift, "shift"));
  CHECK(need(scale, "scale"));
  HIP_TRY(layernorm_modulate(x_dtype, blk_dtype(c), x, c->dim, y, c->dim, rows, c->dim, rpb, shift,
                             scale, c->dim, c->eps, static_cast<hipStream_t>(stream)));
  return FLUX_OK;
}

extern "C" size_t flux_qk_norm_rope_workspace_size(const flux_cfg* c, int n_txt, int n_img) {
  if (check_cfg(c) != FLUX_OK || n_txt < 0 || n_img < 0) return 0;
  Carver cv(nullptr);
  carve_rope(cv, n_txt + n_img);
  return cv.off;
}

extern "C" int flux_qk_norm_rope(const flux_cfg* c, int B, int n_txt, int n_img, void* q, void* k,
                                 int64_t ld, const float* qg_txt, const float* kg_txt,
                                 const float* qg_img, const float* kg_img,
                                 const int32_t* txt_ids, const int32_t* img_ids, void* ws,
                                 size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  const int L = n_txt + n_img;
  if (B <= 0 || n_txt < 0 || n_img < 0 || L <= 0) return fail(FLUX_EINVAL, "bad sizes");
  if (ld < c->dim || (ld * esize(c->dtype)) % 16) return fail(FLUX_EALIGN, "bad ld %lld", (long long)ld);
  CHECK(need(q, "q"));
  CHECK(need(k, "k"));
  CHECK(need(qg_img, "q_norm_img"));
  CHECK(need(kg_img, "k_norm_img"));
  CHECK(need(qg_txt, "q_norm_txt"));
  CHECK(need(kg_txt, "k_norm_txt"));
  if ((n_txt && !txt_ids) || (n_img && !img_ids)) return fail(FLUX_EINVAL, "ids NULL");
  CHECK(check_ws(ws, ws_bytes, flux_qk_norm_rope_workspace_size(c, n_txt, n_img)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  RopeBufs rb = carve_rope(cv, L);
  HIP_TRY(rope_table(txt_ids, img_ids, n_txt, n_img, c->axes_dim, c->rope_theta, rb.pos, rb.cs, s));
  auto mk = [&](void* base) {
    SeqView v;
    v.base0 = base;
    v.base1 = static_cast<char*>(base) + (size_t)n_txt * ld * esize(c->dtype);
    v.bs0 = v.bs1 = (int64_t)L * ld;
    v.ld = ld;
    v.n0 = n_txt;
    return v;
  };
  HIP_TRY(qk_norm_rope(c->dtype, mk(q), mk(k), B, L, c->heads, qg_txt, kg_txt, qg_img, kg_img,
                       rb.cs, c->eps, s));
  return FLUX_OK;
}

// workspace: V^T [B*D, vt_pitch(seq)], then the partial outputs of key-split units
struct AttnScratch {
  void* vt;
  float* split;
};
static AttnScratch carve_attention(Carver& cv, const flux_cfg* c, int B, int seq) {
  AttnScratch a;
  a.vt = cv.take<char>((size_t)B * c->dim * vt_pitch(seq) * esize(c->dtype));
  a.split = cv.take<float>(attention_split_bytes() / sizeof(float));
  return a;
}

extern "C" size_t flux_attention_workspace_size(const flux_cfg* c, int B, int seq) {
  if (check_cfg(c) != FLUX_OK || B <= 0 || seq <= 0) return 0;
  Carver cv(nullptr);
  carve_attention(cv, c, B, seq);
  return cv.off;
}

extern "C" int flux_attention(const flux_cfg* c, int B, int seq, const void* q, const void* k,
                              const void* v, int64_t ld_in, void* o, int64_t ld_out, void* ws,
                              size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  if (B <= 0 || seq <= 0) return fail(FLUX_EINVAL, "batch and seq must be > 0");
  const int es = esize(c->dtype);
  if (ld_in < c->dim || ld_out < c->dim || (ld_in * es) % 16 || (ld_out * es) % 16)
    return fail(FLUX_EALIGN, "leading dimensions must be >= dim and 16-byte multiples");
  CHECK(need(q, "q"));
  CHECK(need(k, "k"));
  CHECK(need(v, "v"));
  CHECK(need(o, "o"));
  CHECK(check_ws(ws, ws_bytes, flux_attention_workspace_size(c, B, seq)));
  auto mk = [&](const void* base, int64_t ld) {
    SeqView sv;
    sv.base0 = sv.base1 = const_cast<void*>(base);
    sv.bs0 = sv.bs1 = (int64_t)seq * ld;
    sv.ld = ld;
    sv.n0 = seq;
    return sv;
  };
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  const AttnScratch a = carve_attention(cv, c, B, seq);
  const int64_t ldvt = vt_pitch(seq);
  HIP_TRY(transpose_v(c->dtype, mk(v, ld_in), a.vt, ldvt, c->dim, B, seq, s));
  if (ldvt > seq) HIP_TRY(zero_cols(c->dtype, a.vt, ldvt, (int64_t)B * c->dim, seq, (int)ldvt, s));
  HIP_TRY(attention(c->dtype, mk(q, ld_in), mk(k, ld_in), a.vt, ldvt, mk(o, ld_out), B, seq,
                    c->heads, a.split, s, nullptr, blk_dtype(c)));
  return FLUX_OK;
}

// ------------------------------------------------------------------------------------
// FP8 (E4M3) linear layer ([KLEIN] Infra, 量化: FP8 releases; recipe = reading: per-row
// amax / 448 scales, round to nearest even, saturating)
// ------------------------------------------------------------------------------------
extern "C" int flux_quantize_fp8_rows(int rows, int cols, const void* x, int x_dtype,
                                      int64_t ldx, void* q, int64_t ldq, float* scales,
                                      void* stream) {
  if (rows <= 0 || cols <= 0) return fail(FLUX_EINVAL, "rows and cols must be > 0");
  if (x_dtype != FLUX_BF16 && x_dtype != FLUX_F32) return fail(FLUX_EDTYPE, "bad x_dtype");
  if (ldx < cols || ldq < cols) return fail(FLUX_ESHAPE, "ldx and ldq must be >= cols");
  if (!x || !q || !scales) return fail(FLUX_EINVAL, "x, q and scales are required");
  HIP_TRY(quantize_fp8_rows(x_dtype, x, ldx, rows, cols, static_cast<uint8_t*>(q), ldq, scales,
                            static_cast<hipStream_t>(stream)));
  return FLUX_OK;
}

extern "C" int flux_linear_fp8(const flux_cfg* c, int epi, int m, int n, int k, const void* qa,
                               int64_t lda, const float* sa, const void* qw, int64_t ldw,
                               const float* sw, void* y, int64_t ldy, int y_dtype,
                               const void* resid, int64_t ldr, const float* gate, int rpb,
                               void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_cfg(c));
  if (m <= 0 || n <= 0 || k <= 0) return fail(FLUX_EINVAL, "m, n, k must be > 0");
  if (k % 128) return fail(FLUX_ESHAPE, "k must be a multiple of 128 for the fp8 linear");
  if (lda < k || ldw < k || lda % 16 || ldw % 16)
    return fail(FLUX_EALIGN, "lda/ldw must be >= k and multiples of 16 bytes");
  if ((int64_t)m * lda >= (int64_t{1} << 32) || (int64_t)n * ldw >= (int64_t{1} << 32))
    return fail(FLUX_ESHAPE, "operands of 4 GiB or more");
  CHECK(need(qa, "qa"));
  CHECK(need(qw, "qw"));
  if (!sa || !sw) return fail(FLUX_EINVAL, "sa and sw are required");
  if (!y) return fail(FLUX_EINVAL, "y is NULL");
  float* split = nullptr;
  if (ws) {
    if (reinterpret_cast<uintptr_t>(ws) & 255u)
      return fail(FLUX_EWORKSPACE, "workspace is not 256-byte aligned");
    if (ws_bytes < linear_splitk_bytes())
      return fail(FLUX_EWORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes,
                  linear_splitk_bytes());
    split = static_cast<float*>(ws);
  }
  LinearArgs a{};
  a.m = m;
  a.n = n;
  a.k = k;
  a.x = qa;
  a.ldx = lda;
  a.w = qw;
  a.ldw = ldw;
  a.y = y;
  a.ldy = ldy;
  a.y_dtype = y_dtype;
  a.rows_per_batch = 1;
  a.split_ws = split;
  if (epi == FLUX_EPI_SWIGLU) {
    if (n % 2) return fail(FLUX_ESHAPE, "SwiGLU needs an even n");
    if (ldy < n / 2) return fail(FLUX_ESHAPE, "ldy < n/2");
    a.epilogue = EPI_SWIGLU;
  } else {
    if (y_dtype != FLUX_BF16 && y_dtype != FLUX_F32) return fail(FLUX_EDTYPE, "bad y_dtype");
    if (ldy < n) return fail(FLUX_ESHAPE, "ldy < n");
    if (epi == FLUX_EPI_STORE) {
      a.epilogue = EPI_STORE;
    } else if (epi == FLUX_EPI_GATED_RESIDUAL) {
      if (!resid || !gate) return fail(FLUX_EINVAL, "resid and gate are required");
      if (rpb <= 0 || m % rpb) return fail(FLUX_ESHAPE, "m must be a multiple of rows_per_batch");
      if (ldr < n) return fail(FLUX_ESHAPE, "ldr < n");
      a.epilogue = EPI_GATED_RESIDUAL;
      a.resid = resid;
      a.ldr = ldr;
      a.r_dtype = y_dtype;
      a.gate = gate;
      a.gate_bs = n;
      a.rows_per_batch = rpb;
    } else {
      return fail(FLUX_EINVAL, "unknown epilogue %d", epi);
    }
  }
  HIP_TRY(linear_fp8(a, sa, sw, static_cast<hipStream_t>(stream)));
  return FLUX_OK;
}

extern "C" size_t flux_linear_workspace_size(void) { return linear_splitk_bytes(); }

// flux_linear / flux_linear_noalloc after the workspace is settled (split: split-K
// scratch of linear_splitk_bytes() bytes, or NULL)
static int linear_entry(const flux_cfg* c, int epi, int m, int n, int k, const void* x,
                        int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy,
                        int y_dtype, const void* resid, int64_t ldr, const float* gate, int rpb,
                        float* split, hipStream_t s) {
  if (epi == FLUX_EPI_SWIGLU) {
    if (n % 2) return fail(FLUX_ESHAPE, "SwiGLU needs an even n");
    if (ldy < n / 2) return fail(FLUX_ESHAPE, "ldy < n/2");
    return lin_b(c, EPI_SWIGLU, m, n, k, x, ldx, w, ldw, y, ldy, blk_dtype(c), nullptr, 0, 0, nullptr,
               0, 1, s, split);
  }
  if (y_dtype != FLUX_BF16 && y_dtype != FLUX_F32) return fail(FLUX_EDTYPE, "bad y_dtype");
  if (ldy < n) return fail(FLUX_ESHAPE, "ldy < n");
  if (epi == FLUX_EPI_STORE)
    return lin_b(c, EPI_STORE, m, n, k, x, ldx, w, ldw, y, ldy, y_dtype, nullptr, 0, 0, nullptr,
                 0, 1, s, split);
  if (epi == FLUX_EPI_GATED_RESIDUAL) {
    if (!resid || !gate) return fail(FLUX_EINVAL, "resid and gate are required");
    if (rpb <= 0 || m % rpb) return fail(FLUX_ESHAPE, "m must be a multiple of rows_per_batch");
    if (ldr < n) return fail(FLUX_ESHAPE, "ldr < n");
    return lin_b(c, EPI_GATED_RESIDUAL, m, n, k, x, ldx, w, ldw, y, ldy, y_dtype, resid, ldr,
                 y_dtype, gate, n, rpb, s, split);
  }
  return fail(FLUX_EINVAL, "unknown epilogue %d", epi);
}

static int check_linear_args(const flux_cfg* c, int epi, int m, int n, int k, const void* x,
                             int64_t ldx, const void* w, int64_t ldw, const void* y) {
  CHECK(check_cfg(c));
  if (m <= 0 || n <= 0 || k <= 0) return fail(FLUX_EINVAL, "m, n, k must be > 0");
  if (k % 8) return fail(FLUX_ESHAPE, "k must be a multiple of 8");
  const int es = esize(c->dtype);
  if (ldx < k || ldw < k || (ldx * es) % 16 || (ldw * es) % 16)
    return fail(FLUX_EALIGN, "ldx/ldw must be >= k and 16-byte multiples");
  CHECK(need(x, "x"));
  CHECK(need(w, "w"));
  if (!y) return fail(FLUX_EINVAL, "y is NULL");
  if (epi != FLUX_EPI_STORE && epi != FLUX_EPI_SWIGLU && epi != FLUX_EPI_GATED_RESIDUAL)
    return fail(FLUX_EINVAL, "unknown epilogue %d", epi);
  return FLUX_OK;
}

extern "C" int flux_linear(const flux_cfg* c, int epi, int m, int n, int k, const void* x,
                           int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy,
                           int y_dtype, const void* resid, int64_t ldr, const float* gate,
                           int rpb, void* ws, size_t ws_bytes, void* stream) {
  CHECK(check_linear_args(c, epi, m, n, k, x, ldx, w, ldw, y));
  float* split = nullptr;
  if (ws) {
    if (reinterpret_cast<uintptr_t>(ws) & 255u)
      return fail(FLUX_EWORKSPACE, "workspace is not 256-byte aligned");
    if (ws_bytes < linear_splitk_bytes())
      return fail(FLUX_EWORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes,
                  linear_splitk_bytes());
    split = static_cast<float*>(ws);
  }
  return linear_entry(c, epi, m, n, k, x, ldx, w, ldw, y, ldy, y_dtype, resid, ldr, gate, rpb,
                      split, static_cast<hipStream_t>(stream));
}

extern "C" int flux_linear_noalloc(const flux_cfg* c, int epi, int m, int n, int k, const void* x,
                                   int64_t ldx, const void* w, int64_t ldw, void* y, int64_t ldy,
                                   int y_dtype, const void* resid, int64_t ldr, const float* gate,
                                   int rpb, void* stream) {
  CHECK(check_linear_args(c, epi, m, n, k, x, ldx, w, ldw, y));
  float* split = nullptr;
  size_t bytes = 0;
  const hipError_t e = linear_static_scratch(&split, &bytes);
  if (e != hipSuccess)
    return fail(FLUX_EHIP, "flux_linear_noalloc: device scratch not available: %s",
                hipGetErrorString(e));
  // the tile planner never plans more split-K scratch than linear_splitk_bytes()
  if (bytes < linear_splitk_bytes())
    return fail(FLUX_EWORKSPACE, "static scratch has %zu bytes, the planner may use %zu", bytes,
                linear_splitk_bytes());
  return linear_entry(c, epi, m, n, k, x, ldx, w, ldw, y, ldy, y_dtype, resid, ldr, gate, rpb,
                      split, static_cast<hipStream_t>(stream));
}
