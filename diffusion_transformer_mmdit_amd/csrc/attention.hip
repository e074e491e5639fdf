// Joint multi-head attention O = softmax(Q K^T / sqrt(128)) V over the whole [txt ; img]
// sequence, no mask (the scaled dot-product attention formula of the kwkr.cn article,
// section 2; "Joint multi-head attention: separate QKV, shared attention" of the Klein 9B
// shape trace, section 4).
//
// bf16 path (gfx950 MFMA 32x32x16, fp32 softmax and accumulation), flash style:
//   * a workgroup of 4 waves owns 128 queries of one (batch, head); each wave 32 queries
//     whose Q fragments stay in registers for the whole key loop;
//   * K and V tiles of 64 keys are staged in LDS (double buffered, next tile's global
//     loads issued before the current tile's MFMAs).  K is stored row-major with an XOR
//     swizzle; V is transposed on its way into LDS (V^T[d][key]) so the PV product reads
//     contiguous keys;
//   * scores are computed transposed, S^T = K Q^T, so each lane owns one query and 32 of
//     the tile's 64 keys: the row max and row sum need one cross-lane exchange (lane ^ 32);
//     O^T = V^T P^T is accumulated the same way, so the online-softmax rescale is a
//     per-lane scalar;
//   * softmax uses exp2 with log2(e)/sqrt(d) folded into one FMA per score.
#include "common.h"
#include "kernels.h"

namespace flux {

template <class T>
FLUX_DEV const T* seq_cptr(const SeqView& v, int b, int j) {
  return (j < v.n0) ? static_cast<const T*>(v.base0) + b * v.bs0 + (int64_t)j * v.ld
                    : static_cast<const T*>(v.base1) + b * v.bs1 + (int64_t)(j - v.n0) * v.ld;
}
template <class T>
FLUX_DEV T* seq_mptr(const SeqView& v, int b, int j) {
  return (j < v.n0) ? static_cast<T*>(v.base0) + b * v.bs0 + (int64_t)j * v.ld
                    : static_cast<T*>(v.base1) + b * v.bs1 + (int64_t)(j - v.n0) * v.ld;
}

constexpr int kHD = 128;       // head dim
constexpr int kBQ = 128;       // queries per workgroup
constexpr int kBKV = 64;       // keys per tile
constexpr int kVTLD = kBKV + 4;  // V^T row pitch (elements): 34 words -> conflict-free reads

FLUX_DEV int kswz(int row, int c) { return row * kHD + ((c ^ (row & 15)) << 3); }

__global__ __launch_bounds__(256) void flash_attn_bf16_kernel(SeqView qv, SeqView kv, SeqView vv,
                                                              SeqView ov, int seq, int heads,
                                                              float scale_log2) {
  __shared__ __align__(16) bf16 Ks[2][kBKV * kHD];
  __shared__ __align__(16) bf16 VTs[2][kHD * kVTLD];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int head = blockIdx.y, b = blockIdx.z;
  const int q0 = blockIdx.x * kBQ + wave * 32;
  const int hoff = head * kHD;

  // ---- Q fragments (B operand of S^T = K Q^T): query l32, dims 16 kk + 8 g .. + 8
  bf16x8 qf[8];
  {
    const int qi = q0 + l32;
    if (qi < seq) {
      const bf16* qp = seq_cptr<bf16>(qv, b, qi) + hoff + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[kk][e] = static_cast<bf16>(0.f);
    }
  }

  // ---- tile loaders: K rows (t>>4)+16i, chunk t&15; V keys 4(t&15)+i, dims 8(t>>4)..+8
  const int kc = tid & 15, kr = tid >> 4;
  const int vkg = tid & 15, vdc = tid >> 4;
  uint4 kreg[4], vreg[4];
  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kv0 + kr + 16 * i;
      kreg[i] = key < seq ? ld16(seq_cptr<bf16>(kv, b, key) + hoff + kc * 8) : make_uint4(0, 0, 0, 0);
      const int vkey = kv0 + 4 * vkg + i;
      vreg[i] = vkey < seq ? ld16(seq_cptr<bf16>(vv, b, vkey) + hoff + vdc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st16(&Ks[buf][kswz(kr + 16 * i, kc)], kreg[i]);
    const uint32_t w[4][4] = {{vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w},
                              {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w},
                              {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w},
                              {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w}};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sh = (e & 1) * 16;
      const uint32_t a0 = (w[0][e >> 1] >> sh) & 0xffffu, a1 = (w[1][e >> 1] >> sh) & 0xffffu;
      const uint32_t a2 = (w[2][e >> 1] >> sh) & 0xffffu, a3 = (w[3][e >> 1] >> sh) & 0xffffu;
      uint2 pk = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
      *reinterpret_cast<uint2*>(&VTs[buf][(vdc * 8 + e) * kVTLD + 4 * vkg]) = pk;
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int ntiles = (seq + kBKV - 1) / kBKV;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int cur = it & 1;
    const int kv0 = it * kBKV;
    if (it + 1 < ntiles) load_tile(kv0 + kBKV);

    // S^T = K Q^T for keys [kv0, kv0 + 64): s[0] keys 0..31, s[1] keys 32..63
    f32x16 s[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[h][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[cur][kswz(l32, 2 * kk + g)]);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(&Ks[cur][kswz(32 + l32, 2 * kk + g)]);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[kk], s[1], 0, 0, 0);
    }

    // mask keys past the end (only the last tile can have them)
    if (kv0 + kBKV > seq) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + 32 * h + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= seq) s[h][r] = -INFINITY;
        }
    }

    // online softmax (raw-score units; exp2 argument scaled by log2(e)/sqrt(d))
    float mx = s[0][0];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[h][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f((m_run - m_new) * scale_log2);
    const float mb = m_new * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(s[h][r], scale_log2, -mb));
        s[h][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // O^T += V^T P^T over 4 chunks of 16 keys
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8 pf;
#pragma unroll
      for (int i = 0; i < 8; ++i) pf[i] = static_cast<bf16>(s[c >> 1][8 * (c & 1) + i]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const bf16* vrow = &VTs[cur][(32 * dt + l32) * kVTLD + 16 * c + 4 * g];
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
        bf16x8 vf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vf[i] = lo[i];
          vf[4 + i] = hi[i];
        }
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[dt], 0, 0, 0);
      }
    }

    if (it + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }

  // normalise and write O[query][d]: lane owns query l32, dims 32 dt + 8 (r/4) + 4 g + r%4
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.f / l_tot;
  const int qi = q0 + l32;
  if (qi < seq) {
    bf16* op = seq_mptr<bf16>(ov, b, qi) + hoff;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * dt + 8 * r4 + 4 * g;
        uint2 pk = make_uint2(pack2(o[dt][4 * r4] * inv, o[dt][4 * r4 + 1] * inv),
                              pack2(o[dt][4 * r4 + 2] * inv, o[dt][4 * r4 + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = pk;
      }
  }
}

// fp32 path (tiny fp32 workloads): one wave per (query, head); each lane owns 2 dims.
__global__ __launch_bounds__(64) void attn_f32_kernel(SeqView qv, SeqView kv, SeqView vv,
                                                      SeqView ov, int seq, int heads, float scale) {
  const int lane = threadIdx.x;
  const int qi = blockIdx.x, head = blockIdx.y, b = blockIdx.z;
  const int d = head * kHD + 2 * lane;
  const float* qp = seq_cptr<float>(qv, b, qi) + d;
  const float q0 = qp[0], q1 = qp[1];
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int j = 0; j < seq; ++j) {
    const float* kp = seq_cptr<float>(kv, b, j) + d;
    const float s = wave_sum(q0 * kp[0] + q1 * kp[1]) * scale;
    const float m_new = fmaxf(m, s);
    const float a = expf(m - m_new), p = expf(s - m_new);
    const float* vp = seq_cptr<float>(vv, b, j) + d;
    l = l * a + p;
    o0 = o0 * a + p * vp[0];
    o1 = o1 * a + p * vp[1];
    m = m_new;
  }
  float* op = seq_mptr<float>(ov, b, qi) + d;
  op[0] = o0 / l;
  op[1] = o1 / l;
}

hipError_t attention(int dtype, SeqView q, SeqView k, SeqView v, SeqView o, int batch, int seq,
                     int heads, hipStream_t s) {
  if (seq <= 0 || batch <= 0) return hipSuccess;
  if (dtype == DT_BF16) {
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)kHD);
    dim3 grid((seq + kBQ - 1) / kBQ, heads, batch);
    hipLaunchKernelGGL(flash_attn_bf16_kernel, grid, dim3(256), 0, s, q, k, v, o, seq, heads,
                       scale_log2);
  } else {
    dim3 grid(seq, heads, batch);
    hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(64), 0, s, q, k, v, o, seq, heads,
                       1.f / sqrtf((float)kHD));
  }
  return hipGetLastError();
}

}  // namespace flux
